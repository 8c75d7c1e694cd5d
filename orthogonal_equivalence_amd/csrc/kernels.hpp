// Launchers of the non-GEMM kernels (aux.hip). All launch on `stream` and
// return false only for an argument combination they do not handle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace poetx {

// Small independent work a launch can carry for the launches after it,
// spread over all its threads: dst0 / dst1 = the inverses of the
// permutations src0 / src1 of [0, n0) / [0, n1) (dst[src[i]] = i, entries
// clamped to the range), and z0[0, nz0), z1[0, nz1) set to zero. Counts of 0
// leave a part out.
struct SideJob {
  const int32_t* src0 = nullptr;
  int32_t* dst0 = nullptr;
  int n0 = 0;
  const int32_t* src1 = nullptr;
  int32_t* dst1 = nullptr;
  int n1 = 0;
  float* z0 = nullptr;
  int64_t nz0 = 0;
  float* z1 = nullptr;
  int64_t nz1 = 0;
  bool empty() const { return n0 <= 0 && n1 <= 0 && nz0 <= 0 && nz1 <= 0; }
};

// The side job's share of the calling thread (grid-stride over the launch).
__device__ __forceinline__ void run_side_job(const SideJob& j) {
  const int64_t total = static_cast<int64_t>(j.n0) + j.n1 + j.nz0 + j.nz1;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    if (i < j.n0) {
      const int32_t v = j.src0[i];
      j.dst0[v < 0 ? 0 : (v >= j.n0 ? j.n0 - 1 : v)] = static_cast<int32_t>(i);
    } else if (i < j.n0 + j.n1) {
      const int32_t k = static_cast<int32_t>(i - j.n0);
      const int32_t v = j.src1[k];
      j.dst1[v < 0 ? 0 : (v >= j.n1 ? j.n1 - 1 : v)] = k;
    } else if (i < j.n0 + j.n1 + j.nz0) {
      j.z0[i - j.n0 - j.n1] = 0.f;
    } else {
      j.z1[i - j.n0 - j.n1 - j.nz0] = 0.f;
    }
  }
}

// The side job in a launch of its own (for paths whose kernels do not carry it).
void side_job(const SideJob& job, hipStream_t stream);

// out[ro][i] = in[ri][cidx[i]] for i < ncols, rows r < nrows, with
// ri = rmap_in ? rmap_in[r] : r and ro = rmap_out ? rmap_out[r] : r.
// esize = element bytes (1, 2 or 4); ncols % 8 == 0. Indices are clamped to
// [0, ncols) and [0, nrows).
bool gather_cols(const void* in, int64_t ld_in, const int32_t* rmap_in, void* out, int64_t ld_out,
                 const int32_t* rmap_out, const int32_t* cidx, int64_t ncols, int64_t nrows, int esize,
                 hipStream_t stream);

// inv[perm[i]] = i (perm entries clamped to [0, n)).
void inverse_perm(const int32_t* perm, int32_t* inv, int64_t n, hipStream_t stream);

// out0[i] = inv0[next0[i]] for i < n0 and out1[i] = inv1[next1[i]] for
// i < n1, in one launch (next entries clamped to [0, n)).
void compose_perm(const int32_t* inv0, const int32_t* next0, int32_t* out0, int64_t n0, const int32_t* inv1,
                  const int32_t* next1, int32_t* out1, int64_t n1, hipStream_t stream);

// out[r][c] = in[inv_r[next_r[r]]][inv_c[next_c[c]]] for a row-major
// nrows x ncols matrix (ncols % 8 == 0, element bytes esize): a matrix whose
// rows and columns are in the frame of one pair of permutations, rewritten in
// the frame of another (inv_*: inverses of the old permutations, next_*: the
// new ones). The composition happens inside the gather where rows fit its
// LDS pipeline; otherwise rmap / cmap (nrows / ncols int32 of scratch)
// receive the composed maps first. job runs in the gather's launch, or in a
// launch of its own before it; nothing runs when false is returned.
bool reframe_rows_cols(const void* in, const int32_t* inv_r, const int32_t* next_r, void* out,
                       const int32_t* inv_c, const int32_t* next_c, int32_t* rmap, int32_t* cmap, int64_t ncols,
                       int64_t nrows, int esize, hipStream_t stream, const SideJob& job = SideJob());

// out[i] = in[idx[i]] (float), idx clamped to [0, n).
void gather_f32(const float* in, const int32_t* idx, float* out, int64_t n, hipStream_t stream);

// out (cols x rows) = transpose of in (rows x cols), element bytes 1, 2 or 4.
bool transpose(const void* in, void* out, int64_t rows, int64_t cols, int esize, hipStream_t stream);

// Zero n floats (a fill kernel, safe inside captured graphs).
void fill_zero_f32(float* p, int64_t n, hipStream_t stream);
// p0[0, n0) and p1[0, n1) set to zero in one launch
void fill_zero2_f32(float* p0, int64_t n0, float* p1, int64_t n1, hipStream_t stream);

// Quantized base weight around a merge (per-output-column scales; the byte
// codes int8, or OCP E4M3 fp8 with fp8):
// out[r][c] = value(wq[r][c]) * scale[cmap ? cmap[c] : c] as float (cols % 8 == 0);
bool dequant_i8_cols(const int8_t* wq, const float* scale, const int32_t* cmap, float* out, int64_t rows,
                     int64_t cols, hipStream_t stream, bool fp8 = false);
// out[i] = in[i] widened from bfloat16;
void bf16_to_f32(const uint16_t* in, float* out, int64_t n, hipStream_t stream);
// out[i] = the int8 code in[i] as bfloat16 (exact), n % 8 == 0 (else false);
bool i8_to_bf16(const int8_t* in, uint16_t* out, int64_t n, hipStream_t stream);
// and the storage again: int8: scale[c] = max_r |w[r][c]| / 127 (1 for a
// zero column), wq = clamp(rint(w / scale), -127, 127); fp8: scale[c] =
// max_r |w[r][c]| / 448 (1 for a zero column), wq = the E4M3 byte of w /
// scale (nearest, ties to even, saturated at 448); amax: cols words of
// scratch (cols % 8 == 0).
bool requant_i8_cols(const float* w, unsigned int* amax, int8_t* wq, float* scale, int64_t rows, int64_t cols,
                     hipStream_t stream, bool fp8 = false);

// Skew blocks from packed parameters: Qf[z] (b x b, float) if Qf is not null
// and a bfloat16 copy if Qh is not null. Blocks [0, n0) come from (q0, dim0), blocks
// [n0, n0 + n1) from (q1, dim1). A side's block z has size
// r = min(b, dim - z*b) and packed offset z*b(b-1)/2; entries outside r x r
// are zero.
void unpack_skew2(const float* q0, int64_t dim0, int n0, const float* q1, int64_t dim1, int n1, int b, float* Qf,
                  uint16_t* Qh, hipStream_t stream);

// S = 2 Q + Q2, written as bfloat16 (Sh) or float (Sf), n elements.
void cnp_mid(const float* Qf, const float* Q2f, uint16_t* Sh, float* Sf, int64_t n, hipStream_t stream);

// G - I = 2Q + 2Q2 + T per block, written as plane 0 (row-major) and plane 1
// (transposed) of a CNP block buffer in bfloat16 (bf16 = true) or float:
// blocks [0, n0) into g0 (n0 blocks), the next n1 into g1.
void cnp_finish2(const float* Qf, const float* Q2f, const float* Tf, int b, int n0, void* g0, int n1, void* g1,
                 bool bf16, hipStream_t stream);

// dq[k(i,l)] = E[i][l] - E[l][i] (i < l < r): blocks [0, n0) into dq0 (side of
// width dim0), the next n1 into dq1.
void pack_asym2(const float* E, int b, int64_t dim0, int n0, float* dq0, int64_t dim1, int n1, float* dq1,
                hipStream_t stream);

// U = sum over the partials part[s][z] (fixed order s = 0, 1, ...) of the
// b x b blocks of two sides in one launch: nblk0 blocks with nsplit0 partials
// from part0, then nblk1 with nsplit1 from part1 (nblk1 = 0: one side).
// Written as Us = (U + U^T)/2 and Uk = (U - U^T)/2 for the nblk0 + nblk1
// blocks back to back (float; bfloat16 copies if Ush / Ukh are not null).
void reduce_symskew2(const float* part0, int nsplit0, int nblk0, const float* part1, int nsplit1, int nblk1, int b,
                     float* Us, float* Uk, uint16_t* Ush, uint16_t* Ukh, hipStream_t stream);

// H1 = 4 Uk - 2 (P1 - P1^T) per block (float and/or bfloat16 outputs).
void cnp_h1(const float* Uk, const float* P1, int b, int nblk, float* Hf, uint16_t* Hh, hipStream_t stream);

// Streaming block-diagonal product (block_apply.hip) on token-major bfloat16
// rows: out[t][j*b + c] = (in[t][j*b + c] + sum_k in[t][j*b + k] *
// plane[j][c][k]) * scale[j*b + c] (scale optional), for the ceil(dim/b)
// blocks of a row of width dim (row stride ld). plane holds b x b bfloat16
// blocks, zero outside a short last block. The same launch also does job.
// Returns false unless b is 64, 128, 256 or 512, or when job is not empty
// and T = 0 (no launch).
bool block_apply_bf16(const uint16_t* in, uint16_t* out, int64_t ld, const uint16_t* plane, const float* scale,
                      int64_t T, int64_t dim, int b, hipStream_t stream, const SideJob& job = SideJob());

// Batched b x b block products with fused epilogue (block_prod.hip), for
// bfloat16 blocks with b a multiple of 128 (up to 1024). Per block z:
//   acc = A1 B1^T + A2 B2^T   (A2 B2^T subtracted instead when neg2 != 0;
//                               the second pair is optional)
//   v1  = alpha acc + beta Ef + gamma Eh,   v2 = alpha2 acc + gamma2 Eh
// with all matrices row-major [nblk][b][b] (Ef float, Eh and the operands
// bfloat16, either addend optional). v1 goes to out1 (row-major) and/or
// out1t (transposed), as float if out1_f32 else bfloat16; v2 to out2
// (bfloat16, row-major). Outputs of blocks z >= z_split go to out1_hi /
// out1t_hi at block z - z_split (two sides batched in one launch). pk
// (optional, float) receives the strict upper triangle of v1 packed row by
// row: for block zl of its side (zl = z, or z - z_split into pk_hi), of size
// r = min(b, dim - zl b) with dim = pk_dim (pk_dim_hi), entry (i, l), i < l
// < r, goes to pk[zl b (b-1)/2 + i r - i (i+1)/2 + l - i - 1]; tiles wholly
// below the diagonal are then skipped. With pk the only output is the packed
// one and v1 takes no Eh term (gamma is ignored).
struct BlockProdDesc {
  const uint16_t* A1 = nullptr;
  const uint16_t* B1 = nullptr;
  const uint16_t* A2 = nullptr;
  const uint16_t* B2 = nullptr;
  int neg2 = 0;
  int b = 0;
  int nblk = 0;
  float alpha = 1.f, beta = 0.f, gamma = 0.f, alpha2 = 0.f, gamma2 = 0.f;
  const float* Ef = nullptr;
  const uint16_t* Eh = nullptr;
  void* out1 = nullptr;
  void* out1t = nullptr;
  int out1_f32 = 0;
  void* out2 = nullptr;
  int z_split = 1 << 30;
  void* out1_hi = nullptr;
  void* out1t_hi = nullptr;
  float* pk = nullptr;
  float* pk_hi = nullptr;
  int64_t pk_dim = 0, pk_dim_hi = 0;
};
bool block_prod_bf16(const BlockProdDesc& d, hipStream_t stream);

// The Cayley-Neumann build of 256 x 256 bfloat16 blocks from Q (cnp_fused.hip):
// Qh holds Q of blocks [0, n0 + n1) as bfloat16 [b][b] each (unpack_skew2's
// bfloat16 output); blocks [0, n0) go to the CNP buffer g0 ([2][n0][b][b]:
// G - I, then (G - I)^T), blocks [n0, n0 + n1) to g1. Four workgroups per
// block, Q kept in LDS, no scratch. Returns false unless b == 256.
bool cnp_build_fused(const uint16_t* Qh, int n0, int n1, int b, void* g0, void* g1, hipStream_t stream);

// Left block product (block_apply.hip) on a row-major rows x ncols bfloat16
// matrix (row stride ld): out[j*256 + i][c] = in[j*256 + i][c] + sum_k
// plane[j][i][k] in[j*256 + k][c] for the ceil(rows/256) row blocks; plane
// holds 256 x 256 bfloat16 blocks, zero outside a short last block. The same
// launch also does job. b = 256 and ncols a multiple of 8 only (returns false
// otherwise, and when job is not empty and there is nothing to launch).
bool block_apply_left_bf16(const uint16_t* in, uint16_t* out, int64_t ld, const uint16_t* plane, int64_t rows,
                           int64_t ncols, int b, hipStream_t stream, const SideJob& job = SideJob());

// Token sums of the block gradients (block_grad.hip) for bfloat16 blocks of
// 256 or 512: part[s][j][i][c] = sum over the tokens of split s of
// act[t][j*b + i] * dout[t][j*b + c], written for every (i, c) < b (zeros
// outside a short last block). block_grad_splits gives the split count the
// kernel uses for T tokens (0 if b is not 256 or 512), for dim features plus
// dim1 more of a second side in the same launch. block_grad2_bf16 runs two
// sides with the same b and split count in one launch (act1 null: one side).
int block_grad_splits(int64_t T, int64_t dim, int b, int64_t dim1 = 0);
bool block_grad_bf16(const uint16_t* act, const uint16_t* dout, float* part, int64_t ld, int64_t T, int64_t dim,
                     int b, int nsplit, hipStream_t stream);
bool block_grad2_bf16(const uint16_t* act0, const uint16_t* dout0, float* part0, int64_t dim0,
                      const uint16_t* act1, const uint16_t* dout1, float* part1, int64_t dim1, int64_t T, int b,
                      int nsplit, hipStream_t stream);

// Seeded uniformly random permutation of [0, n) (perm.hip): index i's key is
// the top 44 bits of word i mod 4 of Philox4x64-10 at counter
// (i div 4, draw, 0, 0) under key (seed, tag), and perm lists the indices by
// ascending (key, index). keys: n words of scratch. 1 <= n <= kMaxPermDim
// (returns false otherwise).
constexpr int64_t kMaxPermDim = int64_t(1) << 20;
// draws of at most this many indices run in one workgroup's LDS (no use of
// `keys`); 10 bytes per index plus 4 KB of bucket counters fit 160 KB
constexpr int64_t kLdsPermMax = 15360;
bool sample_perm(int64_t n, uint64_t seed, uint64_t tag, uint64_t draw, int32_t* perm, uint64_t* keys,
                 hipStream_t stream);

}  // namespace poetx
