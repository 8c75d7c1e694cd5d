// Cayley-Neumann build in one launch for 256 x 256 bfloat16 blocks.
//
// G = (I+Q)(I+Q+Q^2+Q^3) for skew Q stored as its packed strict upper
// triangle (zhichai.net digest of arXiv:2603.05500, section "3.
// Cayley-Neumann 参数化优化"), written with every higher term formed from Q
// and Q^2 as the page's fused kernel arranges it:
//   G - I = 2Q + 2Q^2 + S Q^2,   S = 2Q + Q^2,
// and, so that every product needs only Q and rows of its own, the last term
// is taken as (S Q) Q. Q^2 is symmetric and Q skew, so with Q's rows in LDS
// every product is a "rows times rows" MFMA product:
//   Q^2[i][j]     = -(Q Q^T)[i][j]
//   (S Q)[i][j]   = -(S Q^T)[i][j]
//   (T Q)[i][j]   = -(T Q^T)[i][j],   T = S Q.
//
// Four workgroups share a block, one per 64-row panel p of G - I, and each
// keeps the whole Q on chip:
//   0. Q (bfloat16, unpacked from the packed parameters by the launch before
//      this one) goes global -> LDS with direct loads (128 KB);
//   1. C = Q Q_p^T (256 x 64): Q^2 of the panel, kept in registers.
//   2. S_p = 2 Q_p + Q^2_p into the panel buffer (64 rows, 32 KB);
//      C = Q S_p^T gives T_p = S_p Q, written over S_p.
//   3. C = Q T_p^T gives T_p Q = S_p Q^2.
//   4. G - I = 2 Q_p + 2 Q^2_p + S_p Q^2 into the panel buffer, then plane 0
//      (its rows) and plane 1 (its columns, the rows of (G - I)^T) with
//      16-byte stores.
// Every C is computed as 256 rows (j) x 64 columns (i of the panel), so a
// lane's accumulators hold four consecutive j of one i: the panel rows are
// written to LDS with 8-byte stores, every read of a pass issued before its
// writes. Q, S and T are rounded to bfloat16 for the products; Q^2 of the
// panel stays float32. The four workgroups of a block run on one XCD, so three
// of them read Q from L2.
// 512 threads: 8 waves, 4 (j) x 2 (i), each 64 x 32 outputs as two tiles of
// v_mfma_f32_32x32x16_bf16. A short last block (r < 256) unpacks to zeros
// outside r x r, so every plane entry outside it is zero.
#include "common.hpp"
#include "kernels.hpp"

namespace poetx {
namespace {

constexpr int B = 256;
constexpr int PR = 64;                    // panel rows
constexpr int NT = 512;
constexpr int QROW = B * 2;               // bytes of a bfloat16 row of Q or of the panel
constexpr int kQBytes = B * QROW;         // 128 KB
constexpr int kPanelBytes = PR * QROW;    // 32 KB
constexpr int TM = 2;                     // 32-row MFMA tiles of j per wave

// 16-byte chunk c of row r (of Q or of the panel) sits in slot c ^ (r % 16):
// the 16 rows of a fragment read (same chunk) land in 16 different slots of a
// 256-byte bank window.
__device__ __forceinline__ int slot_off(int r, int col) {
  return r * QROW + (((col >> 3) ^ (r & 15)) << 4) + (col & 7) * 2;
}

struct CnpFusedArgs {
  const bf16_t* Qh;  // [n0 + n1][B][B], Q of every block row-major
  int n0, n1;
  bf16_t* g0;  // CNP buffer of side 0: [2][n0][B][B]
  bf16_t* g1;  // side 1: [2][n1][B][B]
};

// four bfloat16 values at LDS byte offset o (8-byte aligned) as floats
__device__ __forceinline__ void lds_read4(const char* base, int o, float (&v)[4]) {
  const uint2 h = *reinterpret_cast<const uint2*>(base + o);
  v[0] = __uint_as_float(h.x << 16);
  v[1] = __uint_as_float(h.x & 0xffff0000u);
  v[2] = __uint_as_float(h.y << 16);
  v[3] = __uint_as_float(h.y & 0xffff0000u);
}

__device__ __forceinline__ void lds_write4(char* base, int o, const float (&v)[4]) {
  *reinterpret_cast<uint2*>(base + o) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

__device__ __forceinline__ uint4 pack8(const float* w) {
  return make_uint4(pack_bf16x2(w[0], w[1]), pack_bf16x2(w[2], w[3]), pack_bf16x2(w[4], w[5]),
                    pack_bf16x2(w[6], w[7]));
}

__device__ __forceinline__ float bf16_value(bf16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// C[j][i] += sum_k Q[j][k] X[i][k] over K = 256: A fragments from Q's rows j,
// B fragments from the panel operand's rows i (both in LDS, same swizzle).
__device__ __forceinline__ void rows_times_rows(const char* Qs, const char* X, int j0, int i0, int lane,
                                                f32x16_t (&acc)[TM]) {
  const int lrow = lane & 31, hi = lane >> 5;
  const int sw = lrow & 15;  // row % 16 of every fragment row of this lane
#pragma unroll 4
  for (int kk = 0; kk < B / 16; ++kk) {
    const int slot = ((2 * kk + hi) ^ sw) << 4;
    bf16x8_t af[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) af[t] = *reinterpret_cast<const bf16x8_t*>(Qs + (j0 + t * 32 + lrow) * QROW + slot);
    const bf16x8_t bf = *reinterpret_cast<const bf16x8_t*>(X + (i0 + lrow) * QROW + slot);
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[t], bf, acc[t], 0, 0, 0);
  }
}

__global__ void __launch_bounds__(NT, 1) k_cnp_build256(const CnpFusedArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[kQBytes + kPanelBytes];
  char* const Qs = smem;
  char* const Ps = smem + kQBytes;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the four panels of a block on one XCD
  const int pid = xcd_remap(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int z = pid >> 2, p = pid & 3;
  const bool hi = z >= a.n0;
  const int zl = hi ? z - a.n0 : z;
  bf16_t* g = hi ? a.g1 : a.g0;
  const int nside = hi ? a.n1 : a.n0;
  bf16_t* plane0 = g + static_cast<int64_t>(zl) * B * B;
  bf16_t* plane1 = g + static_cast<int64_t>(nside + zl) * B * B;

  // ---- 0. Q into LDS ---------------------------------------------------------
  // 128 instructions of 1 KB (two rows each), 16 per wave: lane l lands in
  // slot l % 32 of row 2 k + l / 32 and fetches the chunk that belongs there.
  {
    const bf16_t* src = a.Qh + static_cast<int64_t>(z) * B * B;
    const int sub = lane >> 5, sl = lane & 31;
#pragma unroll
    for (int k = 0; k < kQBytes / 1024 / (NT / 64); ++k) {
      const int inst = wave * (kQBytes / 1024 / (NT / 64)) + k;
      const int row = 2 * inst + sub;
      const int c = sl ^ (row & 15);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + row * B + c * 8),
                                       (__attribute__((address_space(3))) void*)(Qs + inst * 1024), 16, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }

  // wave tile: j in [jw, jw + 64), i (panel row) in [iw, iw + 32)
  const int jw = (wave & 3) * 64, iw = (wave >> 2) * 32;
  const int ip = iw + (lane & 31);   // the panel row of this lane's accumulators
  const int ig = p * PR + ip;        // ... as a row of the block
  // j of accumulator elements 4 grp .. 4 grp + 3 of tile t
  const int jlane = jw + 4 * (lane >> 5);

  f32x16_t q2[TM], acc[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) q2[t][e] = 0.f;

  // ---- 1. Q^2 of the panel: C = Q Q_p^T = -Q^2 (Q^2 symmetric) ---------------
  rows_times_rows(Qs, Qs + p * PR * QROW, jw, iw, lane, q2);

  // ---- 2. S_p = 2 Q_p + Q^2_p, then T_p = S_p Q -------------------------------
  {
    float qv[TM][4][4];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) lds_read4(Qs, slot_off(ig, jlane + 32 * t + 8 * grp), qv[t][grp]);
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        float s[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) s[e] = 2.f * qv[t][grp][e] - q2[t][4 * grp + e];
        lds_write4(Ps, slot_off(ip, jlane + 32 * t + 8 * grp), s);
      }
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  rows_times_rows(Qs, Ps, jw, iw, lane, acc);  // C = S_p Q^T = -T_p
  __syncthreads();                               // every wave is done reading S_p
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {
      float tv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) tv[e] = -acc[t][4 * grp + e];
      lds_write4(Ps, slot_off(ip, jlane + 32 * t + 8 * grp), tv);
    }
  __syncthreads();

  // ---- 3. T_p Q = S_p Q^2 -------------------------------------------------------
#pragma unroll
  for (int t = 0; t < TM; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  rows_times_rows(Qs, Ps, jw, iw, lane, acc);  // C = T_p Q^T = -(S_p Q^2)
  __syncthreads();                               // every wave is done reading T_p

  // ---- 4. G - I = 2 Q_p + 2 Q^2_p + S_p Q^2 -------------------------------------
  {
    float qv[TM][4][4];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) lds_read4(Qs, slot_off(ig, jlane + 32 * t + 8 * grp), qv[t][grp]);
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = 2.f * qv[t][grp][e] - 2.f * q2[t][4 * grp + e] - acc[t][4 * grp + e];
        lds_write4(Ps, slot_off(ip, jlane + 32 * t + 8 * grp), v);
      }
  }
  __syncthreads();
  // plane 0: the panel's 64 rows (512 bytes each), 16 bytes per thread and
  // step; plane 1: row j of (G - I)^T holds column j of G - I, and this panel
  // gives its entries p*64 .. p*64 + 63, 8 of them per thread and step
  constexpr int kSteps = kPanelBytes / 16 / NT;
  uint4 rows[kSteps];
  uint32_t cols[kSteps][8];
#pragma unroll
  for (int k = 0; k < kSteps; ++k) {
    const int ch = tid + k * NT;
    rows[k] = *reinterpret_cast<const uint4*>(Ps + slot_off(ch >> 5, (ch & 31) * 8));
    const int j = ch >> 3, i8 = (ch & 7) * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) cols[k][e] = *reinterpret_cast<const uint16_t*>(Ps + slot_off(i8 + e, j));
  }
#pragma unroll
  for (int k = 0; k < kSteps; ++k) {
    const int ch = tid + k * NT;
    *reinterpret_cast<uint4*>(plane0 + static_cast<int64_t>(p * PR + (ch >> 5)) * B + (ch & 31) * 8) = rows[k];
    const int j = ch >> 3, i8 = (ch & 7) * 8;
    *reinterpret_cast<uint4*>(plane1 + static_cast<int64_t>(j) * B + p * PR + i8) =
        make_uint4(cols[k][0] | (cols[k][1] << 16), cols[k][2] | (cols[k][3] << 16), cols[k][4] | (cols[k][5] << 16),
                   cols[k][6] | (cols[k][7] << 16));
  }
}

}  // namespace

bool cnp_build_fused(const uint16_t* Qh, int n0, int n1, int b, void* g0, void* g1, hipStream_t s) {
  if (b != B) return false;
  if (n0 + n1 <= 0) return true;
  CnpFusedArgs a;
  a.Qh = Qh;
  a.n0 = n0;
  a.n1 = n1;
  a.g0 = static_cast<bf16_t*>(g0);
  a.g1 = static_cast<bf16_t*>(g1);
  hipLaunchKernelGGL(k_cnp_build256, dim3(static_cast<unsigned>(4 * (n0 + n1))), dim3(NT), 0, s, a);
  return true;
}

}  // namespace poetx
