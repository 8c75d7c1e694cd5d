// bfloat16 MFMA matrix-product engine for gfx950 (see gemm.hpp for the
// contract). One workgroup computes a BM x BN output tile with 2 x 2 waves;
// each wave owns a (BM/2) x (BN/2) sub-tile made of 32 x 32 MFMA tiles
// (v_mfma_f32_32x32x16_bf16, float32 accumulators held for the whole K loop).
// Operand tiles pass through double-buffered LDS in a K-contiguous layout with
// a 16-byte row pad, so each MFMA fragment is one 16-byte LDS read. Operands
// stored M- or N-contiguous in memory are transposed in registers (8 x 8
// blocks of 16-bit values) on their way into LDS; int8 operands are widened
// to bfloat16 (exact for |v| <= 127) on the same path.
#include "common.hpp"
#include "gemm.hpp"

namespace poetx {
namespace {

constexpr int kPad = 8;  // bfloat16 elements of padding per LDS row

struct Lim {
  int M, N, K;
};

__device__ __forceinline__ Lim batch_limits(const GemmDesc& d, int b) {
  Lim l{d.M, d.N, d.K};
  if (d.ragged_dim > 0) {
    const int lim = d.ragged_dim - b * d.ragged_blk;
    if (d.ragged_mask & 1) l.M = min(l.M, lim);
    if (d.ragged_mask & 2) l.N = min(l.N, lim);
    if (d.ragged_mask & 4) l.K = min(l.K, lim);
  }
  return l;
}

// 8 x 8 transpose of 16-bit values: in[r] holds row r (8 values), out[c]
// receives column c. v_perm_b32 picks the low or high halves of two words.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
  uint32_t iw[32];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    iw[r * 4 + 0] = in[r].x;
    iw[r * 4 + 1] = in[r].y;
    iw[r * 4 + 2] = in[r].z;
    iw[r * 4 + 3] = in[r].w;
  }
  uint32_t ow[32];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      ow[c * 4 + p] = __builtin_amdgcn_perm(iw[(2 * p + 1) * 4 + w], iw[(2 * p) * 4 + w], sel);
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) out[c] = make_uint4(ow[c * 4], ow[c * 4 + 1], ow[c * 4 + 2], ow[c * 4 + 3]);
}

__device__ __forceinline__ uint32_t i8x2_to_bf16x2(uint32_t w, int byte) {
  const float lo = static_cast<float>(static_cast<int8_t>((w >> (8 * byte)) & 0xff));
  const float hi = static_cast<float>(static_cast<int8_t>((w >> (8 * byte + 8)) & 0xff));
  // small integers are exact in bfloat16: keep the upper halves
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

__device__ __forceinline__ void i8x16_to_bf16x16(uint4 v, uint4& lo, uint4& hi) {
  lo = make_uint4(i8x2_to_bf16x2(v.x, 0), i8x2_to_bf16x2(v.x, 2), i8x2_to_bf16x2(v.y, 0), i8x2_to_bf16x2(v.y, 2));
  hi = make_uint4(i8x2_to_bf16x2(v.z, 0), i8x2_to_bf16x2(v.z, 2), i8x2_to_bf16x2(v.w, 0), i8x2_to_bf16x2(v.w, 2));
}

// ---------------------------------------------------------------------------
// operand staging: global -> registers (gload) and registers -> LDS (lstore)
// ---------------------------------------------------------------------------

// Operand stored K-contiguous: row r of the tile is ROWS-dim index, 8 values a chunk.
template <int ROWS, int BK, int NT>
struct StageK {
  static constexpr int kChunks = ROWS * BK / 8;
  static constexpr int kPer = (kChunks + NT - 1) / NT;
  uint4 r[kPer];
  __device__ __forceinline__ void gload(const bf16_t* base, int64_t ld, int row0, int rowlim, int k0,
                                        int kend, int tid) {
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int ch = tid + c * NT;
      const int row = ch / (BK / 8), kc = ch % (BK / 8);
      const int gr = row0 + row, gk = k0 + kc * 8;
      if (ch < kChunks && gr < rowlim && gk < kend)
        r[c] = *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(gr) * ld + gk);
      else
        r[c] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void lstore(bf16_t* lds, int tid) const {
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int ch = tid + c * NT;
      const int row = ch / (BK / 8), kc = ch % (BK / 8);
      if (ch < kChunks) *reinterpret_cast<uint4*>(lds + row * (BK + kPad) + kc * 8) = r[c];
    }
  }
};

// Operand stored row-dim contiguous ([K][ROWS]): 8 x 8 blocks transposed.
template <int ROWS, int BK, int NT>
struct StageT {
  static constexpr int kBlocks = ROWS * BK / 64;
  static constexpr int kPer = (kBlocks + NT - 1) / NT;
  uint4 r[kPer][8];
  __device__ __forceinline__ void gload(const bf16_t* base, int64_t ld, int row0, int rowlim, int k0,
                                        int kend, int tid) {
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int blk = tid + c * NT;
      const int rb = blk % (ROWS / 8), kb = blk / (ROWS / 8);
      const int gr = row0 + rb * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int gk = k0 + kb * 8 + i;
        if (blk < kBlocks && gr < rowlim && gk < kend)
          r[c][i] = *reinterpret_cast<const uint4*>(base + static_cast<int64_t>(gk) * ld + gr);
        else
          r[c][i] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void lstore(bf16_t* lds, int tid) const {
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int blk = tid + c * NT;
      const int rb = blk % (ROWS / 8), kb = blk / (ROWS / 8);
      if (blk < kBlocks) {
        uint4 t[8];
        transpose8x8(r[c], t);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<uint4*>(lds + (rb * 8 + i) * (BK + kPad) + kb * 8) = t[i];
      }
    }
  }
};

// int8 operand stored K-contiguous, widened to bfloat16.
template <int ROWS, int BK, int NT>
struct StageI8 {
  static constexpr int kChunks = ROWS * BK / 16;
  static constexpr int kPer = (kChunks + NT - 1) / NT;
  uint4 r[kPer];
  __device__ __forceinline__ void gload(const int8_t* base, int64_t ld, int row0, int rowlim, int k0,
                                        int kend, int tid) {
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int ch = tid + c * NT;
      const int row = ch / (BK / 16), kc = ch % (BK / 16);
      const int gr = row0 + row, gk = k0 + kc * 16;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ch < kChunks && gr < rowlim) {
        const int8_t* p = base + static_cast<int64_t>(gr) * ld + gk;
        if (gk + 16 <= kend) {
          v = *reinterpret_cast<const uint4*>(p);
        } else if (gk + 8 <= kend) {
          const uint2 h = *reinterpret_cast<const uint2*>(p);
          v = make_uint4(h.x, h.y, 0, 0);
        }
      }
      r[c] = v;
    }
  }
  __device__ __forceinline__ void lstore(bf16_t* lds, int tid) const {
#pragma unroll
    for (int c = 0; c < kPer; ++c) {
      const int ch = tid + c * NT;
      const int row = ch / (BK / 16), kc = ch % (BK / 16);
      if (ch < kChunks) {
        uint4 lo, hi;
        i8x16_to_bf16x16(r[c], lo, hi);
        *reinterpret_cast<uint4*>(lds + row * (BK + kPad) + kc * 16) = lo;
        *reinterpret_cast<uint4*>(lds + row * (BK + kPad) + kc * 16 + 8) = hi;
      }
    }
  }
};

template <int AM, int ROWS, int BK, int NT> struct AStageSel;
template <int ROWS, int BK, int NT> struct AStageSel<A_KCONTIG, ROWS, BK, NT> { using type = StageK<ROWS, BK, NT>; };
template <int ROWS, int BK, int NT> struct AStageSel<A_MCONTIG, ROWS, BK, NT> { using type = StageT<ROWS, BK, NT>; };
template <int BMD, int ROWS, int BK, int NT> struct BStageSel;
template <int ROWS, int BK, int NT> struct BStageSel<B_KCONTIG, ROWS, BK, NT> { using type = StageK<ROWS, BK, NT>; };
template <int ROWS, int BK, int NT> struct BStageSel<B_NCONTIG, ROWS, BK, NT> { using type = StageT<ROWS, BK, NT>; };
template <int ROWS, int BK, int NT> struct BStageSel<B_KCONTIG_I8, ROWS, BK, NT> { using type = StageI8<ROWS, BK, NT>; };

template <int CT> struct CSel;
template <> struct CSel<C_F32> { using type = float; };
template <> struct CSel<C_BF16> { using type = bf16_t; };

template <int BM, int BN, int BK, int WM, int WN, int AM, int BMD, int CT, int DENSE>
__global__ void __launch_bounds__(64 * WM * WN)
k_gemm_bf16(const GemmDesc d, int tiles_m, int tiles_n) {
  constexpr int NT = 64 * WM * WN;
  constexpr int LS = BK + kPad;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  using TC = typename CSel<CT>::type;
  using AStage = typename AStageSel<AM, BM, BK, NT>::type;
  using BStage = typename BStageSel<BMD, BN, BK, NT>::type;

  constexpr int kOpBytes = 2 * (BM + BN) * LS * 2;
  constexpr int kSlabStride = WTN + 8;  // floats; 4 rows apart = 32 banks apart
  constexpr int kEpiBytes = WM * WN * 32 * kSlabStride * 4;
  __shared__ __attribute__((aligned(16))) char smem[kOpBytes > kEpiBytes ? kOpBytes : kEpiBytes];
  bf16_t (*As)[BM * LS] = reinterpret_cast<bf16_t (*)[BM * LS]>(smem);
  bf16_t (*Bs)[BN * LS] = reinterpret_cast<bf16_t (*)[BN * LS]>(smem + 2 * BM * LS * 2);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % WM, wn = wave / WM;

  // tile order: XCD-contiguous ranges, grouped by GM tile rows
  constexpr int GM = 8;
  const int pid = xcd_remap(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int group = GM * tiles_n;
  const int first_m = (pid / group) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  const int tm = first_m + (pid % group) % gsz;
  const int tn = (pid % group) / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  const int z = blockIdx.z;
  const int bidx = z / d.ksplit, split = z % d.ksplit;
  const Lim lim = batch_limits(d, bidx);
  const int kbeg = d.ksplit > 1 ? split * d.kchunk : 0;
  const int kend = d.ksplit > 1 ? min(lim.K, kbeg + d.kchunk) : lim.K;
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  const bf16_t* A = static_cast<const bf16_t*>(d.A) + static_cast<int64_t>(bidx) * d.sA;
  const int esizeB = (BMD == B_KCONTIG_I8) ? 1 : 2;
  const char* Bbase = static_cast<const char*>(d.B) + static_cast<int64_t>(bidx) * d.sB * esizeB;

  AStage sa;
  BStage sb;
  auto gload = [&](int k0) {
    sa.gload(A, d.lda, m0, lim.M, k0, kend, tid);
    if constexpr (BMD == B_KCONTIG_I8)
      sb.gload(reinterpret_cast<const int8_t*>(Bbase), d.ldb, n0, lim.N, k0, kend, tid);
    else
      sb.gload(reinterpret_cast<const bf16_t*>(Bbase), d.ldb, n0, lim.N, k0, kend, tid);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nk > 0) {
    gload(kbeg);
    sa.lstore(As[0], tid);
    sb.lstore(Bs[0], tid);
  }
  __syncthreads();

  const int arow = wm * WTM + (lane & 31);
  const int brow = wn * WTN + (lane & 31);
  const int kofs = (lane >> 5) * 8;
  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) gload(kbeg + (it + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[TM], bfg[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[cur][(arow + i * 32) * LS + kk * 16 + kofs]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfg[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[cur][(brow + j * 32) * LS + kk * 16 + kofs]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfg[j], acc[i][j], 0, 0, 0);
    }
    if (it + 1 < nk) {
      sa.lstore(As[cur ^ 1], tid);
      sb.lstore(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // Epilogue. An MFMA accumulator tile holds column n = lane % 32 and rows
  // 8*(r/4) + 4*(lane/32) + r%4. Each wave stages 32 rows of its sub-tile in
  // its own LDS slab, then writes them back 8 columns (16 bytes) per lane.
  TC* C = static_cast<TC*>(d.C) + static_cast<int64_t>(bidx) * d.sC + static_cast<int64_t>(split) * d.sCsplit;
  bf16_t* C2 = d.C2 ? static_cast<bf16_t*>(d.C2) + static_cast<int64_t>(bidx) * d.sC2 : nullptr;
  const bf16_t* R = d.R ? static_cast<const bf16_t*>(d.R) + static_cast<int64_t>(bidx) * d.sR : nullptr;
  const float* S = d.scale ? d.scale + static_cast<int64_t>(bidx) * d.sScale : nullptr;
  const float* D = d.D ? d.D + static_cast<int64_t>(bidx) * d.sD : nullptr;
  const int sM = d.store_full ? d.M : lim.M;
  const int sN = d.store_full ? d.N : lim.N;
  float* slab = reinterpret_cast<float*>(smem) + wave * 32 * kSlabStride;
  constexpr int kChunksPerRow = WTN / 8;
  constexpr int kChunksPerLane = 32 * kChunksPerRow / 64;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    __syncthreads();  // operand tiles (first pass) or previous slab reads are done
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        slab[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * kSlabStride + j * 32 + (lane & 31)] = acc[i][j][r];
    __syncthreads();
#pragma unroll 2
    for (int c = 0; c < kChunksPerLane; ++c) {
      const int ch = lane + c * 64;
      const int row = ch / kChunksPerRow, col = (ch % kChunksPerRow) * 8;
      const int m = m0 + wm * WTM + i * 32 + row;
      const int n = n0 + wn * WTN + col;
      if (m >= sM || n >= sN) continue;
      const float4 p0 = *reinterpret_cast<const float4*>(slab + row * kSlabStride + col);
      const float4 p1 = *reinterpret_cast<const float4*>(slab + row * kSlabStride + col + 4);
      float v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= d.alpha;
      if (m < lim.M && n < lim.N) {
        if (R) {
          const uint4 rv = *reinterpret_cast<const uint4*>(R + static_cast<int64_t>(m) * d.ldr + n);
          const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[2 * e] += __uint_as_float(rw[e] << 16);
            v[2 * e + 1] += __uint_as_float(rw[e] & 0xffff0000u);
          }
        }
        if (S) {
          const float4 s0 = *reinterpret_cast<const float4*>(S + n);
          const float4 s1 = *reinterpret_cast<const float4*>(S + n + 4);
          v[0] *= s0.x; v[1] *= s0.y; v[2] *= s0.z; v[3] *= s0.w;
          v[4] *= s1.x; v[5] *= s1.y; v[6] *= s1.z; v[7] *= s1.w;
        }
        if (D) {
          const float4 d0 = *reinterpret_cast<const float4*>(D + static_cast<int64_t>(m) * d.ldd + n);
          const float4 d1 = *reinterpret_cast<const float4*>(D + static_cast<int64_t>(m) * d.ldd + n + 4);
          v[0] += d.beta * d0.x; v[1] += d.beta * d0.y; v[2] += d.beta * d0.z; v[3] += d.beta * d0.w;
          v[4] += d.beta * d1.x; v[5] += d.beta * d1.y; v[6] += d.beta * d1.z; v[7] += d.beta * d1.w;
        }
      }
      if constexpr (CT == C_F32) {
        float* cp = reinterpret_cast<float*>(C) + static_cast<int64_t>(m) * d.ldc + n;
        *reinterpret_cast<float4*>(cp) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(cp + 4) = make_float4(v[4], v[5], v[6], v[7]);
      } else {
        *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(C) + static_cast<int64_t>(m) * d.ldc + n) =
            make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7]));
      }
      if (C2)
        *reinterpret_cast<uint4*>(C2 + static_cast<int64_t>(m) * d.ldc2 + n) =
            make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7]));
    }
  }
}

template <int BM, int BN, int AM, int BMD, int CT>
void launch_cfg(const GemmDesc& d, hipStream_t s) {
  constexpr int BK = 64;
  const int tm = (d.M + BM - 1) / BM, tn = (d.N + BN - 1) / BN;
  const dim3 grid(tm * tn, 1, d.batch * d.ksplit);
  if constexpr (AM == A_KCONTIG && CT == C_BF16 && BMD != B_NCONTIG) {
    if (d.dense) {
      hipLaunchKernelGGL((k_gemm_bf16<BM, BN, BK, 2, 2, AM, BMD, CT, 1>), grid, dim3(256), 0, s, d, tm, tn);
      return;
    }
  }
  hipLaunchKernelGGL((k_gemm_bf16<BM, BN, BK, 2, 2, AM, BMD, CT, 0>), grid, dim3(256), 0, s, d, tm, tn);
}

// 256 x 256 tiles when they give at least two workgroups per CU (256 CUs),
// else 128 x 128 tiles for more parallelism.
template <int AM, int BMD, int CT>
void launch_any(const GemmDesc& d, hipStream_t s) {
  const int64_t big = static_cast<int64_t>((d.M + 255) / 256) * ((d.N + 255) / 256) * d.batch * d.ksplit;
  if (d.M >= 256 && d.N >= 256 && big >= 512)
    launch_cfg<256, 256, AM, BMD, CT>(d, s);
  else
    launch_cfg<128, 128, AM, BMD, CT>(d, s);
}

template <int AM, int BMD>
void launch_c(const GemmDesc& d, int ct, hipStream_t s) {
  if (ct == C_F32)
    launch_any<AM, BMD, C_F32>(d, s);
  else
    launch_any<AM, BMD, C_BF16>(d, s);
}

}  // namespace

bool gemm_bf16(const GemmDesc& d, int a_mode, int b_mode, int c_type, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0 || d.batch <= 0) return true;
  if (a_mode == A_KCONTIG) {
    if (b_mode == B_KCONTIG) launch_c<A_KCONTIG, B_KCONTIG>(d, c_type, s);
    else if (b_mode == B_NCONTIG) launch_c<A_KCONTIG, B_NCONTIG>(d, c_type, s);
    else if (b_mode == B_KCONTIG_I8) launch_c<A_KCONTIG, B_KCONTIG_I8>(d, c_type, s);
    else return false;
  } else if (a_mode == A_MCONTIG) {
    if (b_mode == B_NCONTIG) launch_c<A_MCONTIG, B_NCONTIG>(d, c_type, s);
    else if (b_mode == B_KCONTIG) launch_c<A_MCONTIG, B_KCONTIG>(d, c_type, s);
    else return false;
  } else {
    return false;
  }
  return true;
}

}  // namespace poetx
