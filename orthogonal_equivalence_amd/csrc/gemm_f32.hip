// float32 MFMA matrix-product engine (v_mfma_f32_32x32x2f32) for layers kept
// in float32. Same contract as the bfloat16 engine (gemm.hpp); A, B, R are
// float32, C is float32. 64 x 64 output tiles, 2 x 2 waves of 32 x 32, K
// staged 16 deep through LDS in a K-major layout, which serves the one-value
// MFMA fragments without bank conflicts whatever the operand's layout in
// memory.
#include "common.hpp"
#include "gemm.hpp"

namespace poetx {
namespace {

struct LimF {
  int M, N, K;
};

__device__ __forceinline__ LimF limits_f(const GemmDesc& d, int b) {
  LimF l{d.M, d.N, d.K};
  if (d.ragged_dim > 0) {
    const int lim = d.ragged_dim - b * d.ragged_blk;
    if (d.ragged_mask & 1) l.M = min(l.M, lim);
    if (d.ragged_mask & 2) l.N = min(l.N, lim);
    if (d.ragged_mask & 4) l.K = min(l.K, lim);
  }
  return l;
}

constexpr int BMf = 64, BNf = 64, BKf = 16, kPadF = 4;

// K-contiguous ([rows][K]) or row-contiguous ([K][rows]) operand into LDS[k][row].
template <bool KCONTIG>
__device__ __forceinline__ void stage_f32(float* lds, const float* base, int64_t ld, int row0, int rowlim,
                                          int k0, int kend, int tid) {
#pragma unroll
  for (int e = 0; e < (BMf * BKf) / 256; ++e) {
    const int idx = tid + e * 256;
    int row, k;
    if (KCONTIG) {
      row = idx / BKf;
      k = idx % BKf;
    } else {
      row = idx % BMf;
      k = idx / BMf;
    }
    const int gr = row0 + row, gk = k0 + k;
    float v = 0.f;
    if (gr < rowlim && gk < kend)
      v = KCONTIG ? base[static_cast<int64_t>(gr) * ld + gk] : base[static_cast<int64_t>(gk) * ld + gr];
    lds[k * (BMf + kPadF) + row] = v;
  }
}

template <int AM, int BMD>
__global__ void __launch_bounds__(256) k_gemm_f32(const GemmDesc d, int tiles_m, int tiles_n) {
  __shared__ float As[BKf * (BMf + kPadF)];
  __shared__ float Bs[BKf * (BNf + kPadF)];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int pid = static_cast<int>(blockIdx.x);
  const int tm = pid % tiles_m, tn = pid / tiles_m;
  const int m0 = tm * BMf, n0 = tn * BNf;
  const int z = blockIdx.z;
  const int bidx = z / d.ksplit, split = z % d.ksplit;
  const LimF lim = limits_f(d, bidx);
  const int kbeg = d.ksplit > 1 ? split * d.kchunk : 0;
  const int kend = d.ksplit > 1 ? min(lim.K, kbeg + d.kchunk) : lim.K;

  const float* A = static_cast<const float*>(d.A) + static_cast<int64_t>(bidx) * d.sA;
  const float* B = static_cast<const float*>(d.B) + static_cast<int64_t>(bidx) * d.sB;
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;

  for (int k0 = kbeg; k0 < kend; k0 += BKf) {
    stage_f32<AM == A_KCONTIG>(As, A, d.lda, m0, lim.M, k0, kend, tid);
    stage_f32<BMD == B_KCONTIG>(Bs, B, d.ldb, n0, lim.N, k0, kend, tid);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKf; kk += 2) {
      const int k = kk + (lane >> 5);
      const float a = As[k * (BMf + kPadF) + wm * 32 + (lane & 31)];
      const float b = Bs[k * (BNf + kPadF) + wn * 32 + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc, 0, 0, 0);
    }
    __syncthreads();
  }

  float* C = static_cast<float*>(d.C) + static_cast<int64_t>(bidx) * d.sC + static_cast<int64_t>(split) * d.sCsplit;
  const float* R = d.R ? static_cast<const float*>(d.R) + static_cast<int64_t>(bidx) * d.sR : nullptr;
  const float* S = d.scale ? d.scale + static_cast<int64_t>(bidx) * d.sScale : nullptr;
  const float* D = d.D ? d.D + static_cast<int64_t>(bidx) * d.sD : nullptr;
  const int sM = d.store_full ? d.M : lim.M;
  const int sN = d.store_full ? d.N : lim.N;
  const int n = n0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
    if (m < sM && n < sN) {
      float v = d.alpha * acc[r];
      if (m < lim.M && n < lim.N) {
        if (R) v += R[static_cast<int64_t>(m) * d.ldr + n];
        if (S) v *= S[n];
        if (D) v += d.beta * D[static_cast<int64_t>(m) * d.ldd + n];
      }
      C[static_cast<int64_t>(m) * d.ldc + n] = v;
    }
  }
}

template <int AM, int BMD>
void launch_f32(const GemmDesc& d, hipStream_t s) {
  const int tm = (d.M + BMf - 1) / BMf, tn = (d.N + BNf - 1) / BNf;
  hipLaunchKernelGGL((k_gemm_f32<AM, BMD>), dim3(tm * tn, 1, d.batch * d.ksplit), dim3(256), 0, s, d, tm, tn);
}

}  // namespace

bool gemm_f32(const GemmDesc& d, int a_mode, int b_mode, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return true;
  if (a_mode == A_KCONTIG && b_mode == B_KCONTIG) launch_f32<A_KCONTIG, B_KCONTIG>(d, s);
  else if (a_mode == A_KCONTIG && b_mode == B_NCONTIG) launch_f32<A_KCONTIG, B_NCONTIG>(d, s);
  else if (a_mode == A_MCONTIG && b_mode == B_NCONTIG) launch_f32<A_MCONTIG, B_NCONTIG>(d, s);
  else if (a_mode == A_MCONTIG && b_mode == B_KCONTIG) launch_f32<A_MCONTIG, B_KCONTIG>(d, s);
  else return false;
  return true;
}

}  // namespace poetx
