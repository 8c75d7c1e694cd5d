// Batched "NT" matrix product engine used by every contraction of the layer.
//
//   C[b](m, n) = ((alpha * sum_k A[b](m, k) * B[b](n, k)) + R[b](m, n)) * s[n]
//                + beta * D[b](m, n)
//
// with optional terms. A and B come in several storage layouts (see the mode
// enums); the product always runs on MFMA matrix cores (bfloat16 inputs with
// float32 accumulation, or float32 inputs and accumulation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

enum AMode { A_KCONTIG = 0, A_MCONTIG = 1 };        // A[m*lda + k] or A[k*lda + m]
enum BMode { B_KCONTIG = 0, B_NCONTIG = 1, B_KCONTIG_I8 = 2 };  // B[n*ldb + k] or B[k*ldb + n]
enum CType { C_F32 = 0, C_BF16 = 1 };

struct GemmDesc {
  const void* A = nullptr; int64_t lda = 0; int64_t sA = 0;   // sA: batch stride (elements)
  const void* B = nullptr; int64_t ldb = 0; int64_t sB = 0;
  void* C = nullptr; int64_t ldc = 0; int64_t sC = 0;
  void* C2 = nullptr; int64_t ldc2 = 0; int64_t sC2 = 0;      // optional bf16 copy of C
  const void* R = nullptr; int64_t ldr = 0; int64_t sR = 0;   // residual, same type as A
  const float* scale = nullptr; int64_t sScale = 0;           // per-column multiplier
  const float* D = nullptr; int64_t ldd = 0; int64_t sD = 0;  // float addend
  float alpha = 1.f;
  float beta = 0.f;
  int M = 0, N = 0, K = 0;
  int batch = 1;
  int ksplit = 1;            // split s covers k in [s*kchunk, (s+1)*kchunk)
  int kchunk = 0;            // multiple of the tile depth
  int64_t sCsplit = 0;       // output stride between splits
  // Short last block: batch b limits the dims selected by ragged_mask
  // (1 = M, 2 = N, 4 = K) to min(nominal, ragged_dim - b * ragged_blk).
  int ragged_dim = 0;
  int ragged_blk = 0;
  int ragged_mask = 0;
  // 1: write the whole nominal M x N output (zeros outside the limits), as
  // split partial sums and zero-padded blocks need.
  int store_full = 0;
  // 1: the dense W0 product (its own kernel symbol, so profiles separate it)
  int dense = 0;
  // dense product with 1-byte B codes: 1 = OCP E4M3 fp8 bytes, 0 = int8
  int b_fp8 = 0;
};

// Launch on `stream`. a_mode/b_mode/c_type select the kernel; returns false if
// the combination is not built. bf16 inputs: A and (non-I8) B are bfloat16.
bool gemm_bf16(const GemmDesc& d, int a_mode, int b_mode, int c_type, hipStream_t stream);
bool gemm_f32(const GemmDesc& d, int a_mode, int b_mode, hipStream_t stream);

// Dense bfloat16 product for the W0 products (gemm_dense.hip): A [M][K]
// K-contiguous, B [N][K] K-contiguous (b_ncontig false) or [K][N]
// N-contiguous (b_ncontig true), bfloat16 or, with b_int8, int8 codes
// dequantised to bfloat16 inside the product (N and ldb multiples of 16);
// C bfloat16, optional per-column scale; uses A, lda, B, ldb, C, ldc, scale,
// M, N, K only. Returns false unless K % 64 == 0 and N % 8 == 0.
// split_ws: gemm_dense_split_bytes(M, N, K) bytes (256-byte aligned) for
// splitting the output tiles of a partial last round along K; with NULL, or
// 0 bytes needed, every tile runs whole.
size_t gemm_dense_split_bytes(int M, int N, int K);
bool gemm_dense_bf16(const GemmDesc& d, void* split_ws, hipStream_t stream, bool b_ncontig, bool b_int8);

}  // namespace poetx
