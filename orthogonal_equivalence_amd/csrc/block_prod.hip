// Batched b x b block products for the Cayley-Neumann map and its adjoint
// (bfloat16 operands, float32 accumulation), with the element-wise steps
// around each product fused into its epilogue:
//   acc = A1 B1^T (+ or -) A2 B2^T           per block z, K = b per pair
//   v1  = alpha * acc + beta * Ef + gamma * Eh     (Ef float, Eh bfloat16 addends)
//   v2  = alpha2 * acc + gamma2 * Eh
// written as out1 (row-major), out1t (transposed) and out2 (row-major), each
// optional. All operands are row-major [nblk][b][b] (rows K-contiguous), so a
// product with a symmetric or skew right factor needs no transposed copy: for
// skew Q, M Q = -M Q^T; for symmetric S, M S = M S^T.
//
// The Cayley-Neumann build (zhichai.net digest of arXiv:2603.05500, section
// "3. Cayley-Neumann 参数化优化") is two such products, Q^2 = -Q Q^T with
// S = 2Q + Q^2 in the epilogue, then G - I = 2Q + 2Q^2 + S Q^2 written as both
// planes of the block buffer; the adjoint is three (see poetx_abi.hip), the
// last of which writes the packed gradient straight from its epilogue.
//
// gfx950 design: 128 x 128 output tile per workgroup (the tiles of one block
// on one XCD), 8 waves of 64 x 32 (2 x 1 tiles of v_mfma_f32_32x32x16_bf16;
// two waves per SIMD, so that one wave's LDS and MFMA latencies run under
// the other's work), K in steps of 64 through two LDS stages filled with
// global_load_lds_dwordx4 (128-byte rows, XOR swizzle); the epilogue stages
// each wave's 32 x 32 band through LDS so that row-major and transposed
// outputs are both written with 16-byte stores.
#include "common.hpp"
#include "kernels.hpp"

namespace poetx {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_t;

constexpr int TB = 128;             // output tile
constexpr int BK = 64;              // K per stage
constexpr int NT = 512;             // 8 waves: 2 along M x 4 along N
constexpr int WTN = 32;             // wave tile width (columns)
constexpr int kRowBytes = BK * 2;   // 128
constexpr int kTileBytes = TB * kRowBytes;  // 16 KB per operand and stage
constexpr int kStageBytes = 2 * kTileBytes;
constexpr int kInst = kTileBytes / 1024 / (NT / 64);  // loads per wave per operand (2)
constexpr int kSlab = WTN + 4;      // epilogue slab row stride (floats)

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ void load_tile(const bf16_t* __restrict__ g, int b, int row0, int k0, char* lds, int wave,
                                          int lane) {
  const int sub = lane >> 3, slot = lane & 7;
#pragma unroll
  for (int i = 0; i < kInst; ++i) {
    const int rbase = (wave * kInst + i) * 8;
    const int r = rbase + sub;
    const int c = slot ^ swz(r);
    const bf16_t* src = g + static_cast<int64_t>(row0 + r) * b + k0 + c * 8;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t)(lds + rbase * kRowBytes), 16, 0, 0);
  }
}

__device__ __forceinline__ void store8(void* base, int64_t off, bool f32, const float (&v)[8]) {
  if (f32) {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    *reinterpret_cast<uint4*>(static_cast<bf16_t*>(base) + off) =
        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7]));
  }
}

__global__ void __launch_bounds__(NT, 2) k_block_prod(const BlockProdDesc d) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * kStageBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int tiles = d.b / TB;
  const int per_blk = tiles * tiles;
  // the tiles of a block run on one XCD, so its operand rows are re-read
  // from that XCD's L2
  const int pid = xcd_remap(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int z = pid / per_blk;
  const int t = pid % per_blk;
  const int i0 = (t / tiles) * TB, n0 = (t % tiles) * TB;
  const int64_t zoff = static_cast<int64_t>(z) * d.b * d.b;
  // outputs of the second side start at its own block 0
  const bool hi = z >= d.z_split;
  const int64_t zout = static_cast<int64_t>(hi ? z - d.z_split : z) * d.b * d.b;
  void* const out1 = hi ? d.out1_hi : d.out1;
  void* const out1t = hi ? d.out1t_hi : d.out1t;
  // packed strict upper triangle: nothing to do below the diagonal
  float* const pk = hi ? d.pk_hi : d.pk;
  if ((d.pk || d.pk_hi) && (pk == nullptr || i0 > n0)) return;
  const int zl = hi ? z - d.z_split : z;
  const int pk_r = static_cast<int>(min(static_cast<int64_t>(d.b), (hi ? d.pk_dim_hi : d.pk_dim) -
                                                                       static_cast<int64_t>(zl) * d.b));
  const int64_t pk_off = static_cast<int64_t>(zl) * d.b * (d.b - 1) / 2;
  const int ksteps = d.b / BK;
  const int nk = ksteps * (d.A2 ? 2 : 1);

  constexpr int TNw = WTN / 32;
  f32x16_t acc[2][TNw];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < TNw; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  auto issue = [&](int s, char* st) {
    const bool second = s >= ksteps;
    const bf16_t* A = (second ? d.A2 : d.A1) + zoff;
    const bf16_t* B = (second ? d.B2 : d.B1) + zoff;
    const int k0 = (second ? s - ksteps : s) * BK;
    load_tile(A, d.b, i0, k0, st, wave, lane);
    load_tile(B, d.b, n0, k0, st + kTileBytes, wave, lane);
  };

  const int lrow = lane & 31;
  const int sw = swz(lrow);
  int koff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) koff[kk] = lrow * kRowBytes + (((2 * kk + (lane >> 5)) ^ sw) << 4);
  const int abase = wm * 64 * kRowBytes;
  const int bbase = kTileBytes + wn * WTN * kRowBytes;

  issue(0, smem);
  for (int s = 0; s < nk; ++s) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (s + 1 < nk) issue(s + 1, smem + ((s + 1) & 1) * kStageBytes);
    if (s == ksteps && d.neg2) {
      // acc = -(A1 B1^T) before the second pair, so that the sum is the difference up to sign
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < TNw; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = -acc[i][j][r];
    }
    const char* st = smem + (s & 1) * kStageBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8_t af[2], bfr[TNw];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(st + abase + i * 32 * kRowBytes + koff[kk]);
#pragma unroll
      for (int j = 0; j < TNw; ++j) bfr[j] = *reinterpret_cast<const bf16x8_t*>(st + bbase + j * 32 * kRowBytes + koff[kk]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < TNw; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }
  // with neg2, acc = -(P1) + P2 = -(P1 - P2): fold the sign into the coefficients
  const float sgn = d.neg2 ? -1.f : 1.f;
  const float alpha = d.alpha * sgn, alpha2 = d.alpha2 * sgn;

  // epilogue: per wave and 32-row band, a 32 x WTN slab of v1 (and v2)
  __syncthreads();
  float* slab = reinterpret_cast<float*>(smem) + wave * 32 * kSlab;
  constexpr int kCpr = WTN / 8;              // 8-column chunks per slab row
  constexpr int kCpl = 32 * kCpr / 64;       // chunks per lane
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int j = 0; j < TNw; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        slab[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * kSlab + j * 32 + lrow] = acc[i][j][r];
    if (pk) {
      // packed upper triangle: lane -> column (64 / WTN rows at a time), one
      // row per step, so that each store instruction covers contiguous runs
      // of the rows' packed entries
      constexpr int kRowsAtOnce = 64 / WTN;
      const int lc = lane % WTN, lr = lane / WTN;
      const int gn = n0 + wn * WTN + lc;
      float ef[32 / kRowsAtOnce];
#pragma unroll
      for (int q = 0; q < 32 / kRowsAtOnce; ++q) {
        const int gi = i0 + wm * 64 + i * 32 + q * kRowsAtOnce + lr;
        ef[q] = d.Ef ? d.Ef[zoff + static_cast<int64_t>(gi) * d.b + gn] : 0.f;
      }
#pragma unroll
      for (int q = 0; q < 32 / kRowsAtOnce; ++q) {
        const int row = q * kRowsAtOnce + lr;
        const int gi = i0 + wm * 64 + i * 32 + row;
        const float v = alpha * slab[row * kSlab + lc] + d.beta * ef[q];
        if (gi < gn && gn < pk_r)
          pk[pk_off + static_cast<int64_t>(gi) * pk_r - static_cast<int64_t>(gi) * (gi + 1) / 2 + gn - gi - 1] = v;
      }
      continue;
    }
    // row pass: lane -> (row, 8 columns); 32 rows x kCpr chunks
#pragma unroll
    for (int c = 0; c < kCpl; ++c) {
      const int ch = lane + c * 64;
      const int row = ch / kCpr, col = (ch % kCpr) * 8;
      const int gi = i0 + wm * 64 + i * 32 + row, gn = n0 + wn * WTN + col;
      const int64_t roff = static_cast<int64_t>(gi) * d.b + gn;
      const int64_t off = zoff + roff;
      float a[8], v1[8];
      const float4 p0 = *reinterpret_cast<const float4*>(slab + row * kSlab + col);
      const float4 p1 = *reinterpret_cast<const float4*>(slab + row * kSlab + col + 4);
      a[0] = p0.x; a[1] = p0.y; a[2] = p0.z; a[3] = p0.w; a[4] = p1.x; a[5] = p1.y; a[6] = p1.z; a[7] = p1.w;
      float ef[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, eh[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (d.Ef) {
        const float4 q0 = *reinterpret_cast<const float4*>(d.Ef + off);
        const float4 q1 = *reinterpret_cast<const float4*>(d.Ef + off + 4);
        ef[0] = q0.x; ef[1] = q0.y; ef[2] = q0.z; ef[3] = q0.w; ef[4] = q1.x; ef[5] = q1.y; ef[6] = q1.z; ef[7] = q1.w;
      }
      if (d.Eh) {
        const uint4 h = *reinterpret_cast<const uint4*>(d.Eh + off);
        const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          eh[2 * e] = __uint_as_float(hw[e] << 16);
          eh[2 * e + 1] = __uint_as_float(hw[e] & 0xffff0000u);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) v1[e] = alpha * a[e] + d.beta * ef[e] + d.gamma * eh[e];
      if (out1) store8(out1, zout + roff, d.out1_f32, v1);
      if (d.out2) {
        float v2[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v2[e] = alpha2 * a[e] + d.gamma2 * eh[e];
        store8(d.out2, off, false, v2);
      }
      if (out1t) {
        // v1 back into the slab for the transposed pass
        *reinterpret_cast<float4*>(slab + row * kSlab + col) = make_float4(v1[0], v1[1], v1[2], v1[3]);
        *reinterpret_cast<float4*>(slab + row * kSlab + col + 4) = make_float4(v1[4], v1[5], v1[6], v1[7]);
      }
    }
    if (out1t) {
      // transposed pass: lane -> (column, 8 rows); WTN columns x 4 row groups
#pragma unroll
      for (int c = 0; c < WTN * 4 / 64; ++c) {
        const int ch = lane + c * 64;
        const int col = ch >> 2, rg = (ch & 3) * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = slab[(rg + e) * kSlab + col];
        const int gn = n0 + wn * WTN + col, gi = i0 + wm * 64 + i * 32 + rg;
        store8(out1t, zout + static_cast<int64_t>(gn) * d.b + gi, d.out1_f32, v);
      }
    }
  }
}

}  // namespace

bool block_prod_bf16(const BlockProdDesc& d, hipStream_t s) {
  if (d.nblk <= 0) return true;
  if (d.b % TB != 0 || d.b < TB || d.b > 1024 || !d.A1 || !d.B1 || (d.A2 && !d.B2)) return false;
  const int tiles = d.b / TB;
  hipLaunchKernelGGL(k_block_prod, dim3(static_cast<unsigned>(d.nblk * tiles * tiles)), dim3(NT), 0, s, d);
  return true;
}

}  // namespace poetx
