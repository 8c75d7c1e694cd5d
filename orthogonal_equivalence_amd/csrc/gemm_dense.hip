// Dense product C = A B^T (bfloat16 in, float32 accumulate, bfloat16 out) for
// the layer's two W0 products: Y1 = X2 Wp (B = Wp^T rows) and dX2 = dY1 Wp^T
// (B = Wp rows). Both operands are K-contiguous.
//
// gfx950 design:
//  * 256 x 256 output tile per workgroup, K in steps of 64, 8 waves (two per
//    SIMD, so one wave's LDS waits hide behind the other's MFMAs); each wave
//    owns 128 x 64 outputs as 4 x 2 tiles of v_mfma_f32_32x32x16_bf16.
//  * Operand tiles go global -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging, no LDS write instructions), double-buffered, one barrier per
//    K step. The next stage's loads are spread over the current stage's four
//    K groups (two 1 KB loads per group and wave) rather than issued in one
//    burst, so that their LDS writes interleave with the fragment reads.
//  * LDS rows are 128 bytes, unpadded; 16-byte chunk c of row r sits in slot
//    c ^ swz(r) with swz(r) = (r & 7) ^ ((r >> 3) & 1), which keeps the
//    fragment reads (32 rows, same chunk) free of bank conflicts whether the
//    LDS serves 8 or 16 lanes of a 16-byte read per cycle.
//  * Output tiles are ordered so that each XCD works on one contiguous band
//    of tiles (shared A/B panels stay in that XCD's L2).
//  * When the tiles do not fill a whole number of rounds over the 256 CUs,
//    the tiles of the last, partial round are split along K into k parts
//    (k * tail <= 256), so that round runs on (nearly) every CU. Every part
//    writes its fp32 partial tile, row-major, to the workspace; a second
//    kernel adds the k partials of each tile in part order, applies the
//    column scale and stores bfloat16. The kernel boundary makes the
//    partials visible across XCDs; a hand-off inside the kernel would need
//    device-scope fences, which write back and invalidate a whole XCD's L2
//    under every other workgroup streaming from it.
#include "common.hpp"
#include "gemm.hpp"

namespace poetx {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

#ifndef POETX_DENSE_BK
#define POETX_DENSE_BK 64
#endif
#ifndef POETX_DENSE_STAGES
#define POETX_DENSE_STAGES 2
#endif
#ifndef POETX_DENSE_WN
#define POETX_DENSE_WN 4
#endif

constexpr int BM = 256, BN = 256;
constexpr int BK = POETX_DENSE_BK;           // K depth of one LDS stage
constexpr int NSTAGE = POETX_DENSE_STAGES;   // LDS stages; NSTAGE - 1 in flight
constexpr int WM = 2, WN = POETX_DENSE_WN;
constexpr int NT = 64 * WM * WN;
constexpr int WTM = BM / WM, WTN = BN / WN;  // 128 x 64 per wave
constexpr int TM = WTM / 32, TN = WTN / 32;  // 4 x 2 MFMA tiles
constexpr int kRowBytes = BK * 2;            // 64 or 128
constexpr int kChunks = kRowBytes / 16;      // 16-byte chunks per row
constexpr int kRowsPerInst = 64 / kChunks;   // rows one 1 KB load covers
constexpr int kTileBytes = BM * kRowBytes;   // per operand and stage
constexpr int kStageBytes = 2 * kTileBytes;  // A + B
constexpr int kInstPerTile = kTileBytes / 1024 / (NT / 64);  // loads per wave per operand
constexpr int kSlabStride = WTN + 8;         // epilogue slab row, floats
static_assert(NSTAGE * kStageBytes <= 160 * 1024, "LDS");

// Slot of 16-byte chunk c in row r: c ^ swz(r). For 128-byte rows the bank
// group of a 16-byte read is 8 * (r % 2) + slot (16 lanes a cycle) or slot
// (8 lanes); for 64-byte rows it is 4 * (r % 4) + slot or 4 * (r % 2) + slot.
// Both choices below make the 32 rows of one fragment read conflict-free in
// either model.
__device__ __forceinline__ int swz(int r) {
  if constexpr (kChunks == 8) return (r & 7) ^ ((r >> 3) & 1);
  else return ((r >> 1) & 3) ^ ((r >> 3) & 1);
}

// Direct-to-LDS load of one 256 x BK bfloat16 operand tile. Each wave issues
// kInstPerTile instructions of 1 KB; lane l of an instruction lands in slot
// l % kChunks of row l / kChunks and fetches the chunk that belongs there.
// Rows past `rowlim` re-read row rowlim - 1 (in bounds); their products only
// reach outputs that are never stored.
__device__ __forceinline__ void load_tile(const bf16_t* __restrict__ g, int64_t ld, int row0, int rowlim, int k0,
                                          char* lds, int wave, int lane) {
  const int sub = lane / kChunks, slot = lane % kChunks;
#pragma unroll
  for (int i = 0; i < kInstPerTile; ++i) {
    const int rbase = (wave * kInstPerTile + i) * kRowsPerInst;
    const int r = rbase + sub;
    const int c = slot ^ swz(r);
    int gr = row0 + r;
    gr = gr < rowlim ? gr : rowlim - 1;
    const bf16_t* src = g + static_cast<int64_t>(gr) * ld + k0 + c * 8;
    __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t)(lds + rbase * kRowBytes), 16, 0, 0);
  }
}

__device__ __forceinline__ void load_one(const bf16_t* __restrict__ g, int64_t ld, int row0, int rowlim, int k0,
                                         char* lds, int wave, int lane, int i) {
  const int sub = lane / kChunks, slot = lane % kChunks;
  const int rbase = (wave * kInstPerTile + i) * kRowsPerInst;
  const int r = rbase + sub;
  const int c = slot ^ swz(r);
  int gr = row0 + r;
  gr = gr < rowlim ? gr : rowlim - 1;
  const bf16_t* src = g + static_cast<int64_t>(gr) * ld + k0 + c * 8;
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(src), (lds_void_t)(lds + rbase * kRowBytes), 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Tiles [0, full) run whole; tile full + u / k is computed as part u % k
// (of k) by workgroup full + u. part: the tail tiles' partials,
// [tail][k][BM][BN] floats.
struct DenseSplit {
  float* part;
  int full;
  int k;
};

// Output tile (tm, tn) of tile index pid: groups of GM tile rows, walked
// column by column, so that neighbouring pids share A or B panels.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GM = 8;
  const int group = GM * tiles_n;
  const int first_m = (pid / group) * GM;
  const int gsz = min(tiles_m - first_m, GM);
  tm = first_m + (pid % group) % gsz;
  tn = (pid % group) / gsz;
}

__global__ void __launch_bounds__(NT, 1) k_gemm_dense(const GemmDesc d, int tiles_m, int tiles_n, DenseSplit sp) {
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;

  const int bid = static_cast<int>(blockIdx.x);
  int pid, part = 0;
  if (bid < sp.full) {
    pid = xcd_remap(bid, sp.full);
  } else {
    pid = sp.full + (bid - sp.full) / sp.k;
    part = (bid - sp.full) % sp.k;
  }
  int tm, tn;
  tile_coords(pid, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const bf16_t* A = static_cast<const bf16_t*>(d.A);
  const bf16_t* B = static_cast<const bf16_t*>(d.B);
  // this workgroup's K steps: [kb, kb + nk) (all of them for a whole tile)
  const int nk_all = d.K / BK;
  const int nparts = bid < sp.full ? 1 : sp.k;
  const int kb = part * nk_all / nparts;
  const int nk = (part + 1) * nk_all / nparts - kb;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // per-lane fragment offsets: row (lane % 32) of a 32-row tile, chunk
  // 2*kk + lane/32, swizzled; the swizzle only depends on lane % 16
  const int lrow = lane & 31;
  const int sw = swz(lrow);
  int koff[BK / 16];
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) koff[kk] = lrow * kRowBytes + (((2 * kk + (lane >> 5)) ^ sw) << 4);
  const int abase = wm * WTM * kRowBytes;
  const int bbase = kTileBytes + wn * WTN * kRowBytes;

  // prologue: stages 0 .. NSTAGE-2 in flight
#pragma unroll
  for (int p = 0; p < NSTAGE - 1; ++p) {
    if (p < nk) {
      load_tile(A, d.lda, m0, d.M, (kb + p) * BK, smem + p * kStageBytes, wave, lane);
      load_tile(B, d.ldb, n0, d.N, (kb + p) * BK, smem + p * kStageBytes + kTileBytes, wave, lane);
    }
  }

  for (int it = 0; it < nk; ++it) {
    // stage `it` is the oldest of the (up to NSTAGE - 1) stages in flight;
    // loads complete in order, so waiting until the younger ones remain
    // suffices. Near the end fewer younger stages exist.
    constexpr int kPerStage = 2 * kInstPerTile;
    const int younger = min(NSTAGE - 2, nk - 1 - it);
    if (younger >= 2) wait_vmcnt<2 * kPerStage>();
    else if (younger == 1) wait_vmcnt<kPerStage>();
    else wait_vmcnt<0>();
    __syncthreads();
    const int pf = it + NSTAGE - 1;
    char* nxt = smem + (pf % NSTAGE) * kStageBytes;
    const int kpf = (kb + min(pf, nk - 1)) * BK;
    const char* st = smem + (it % NSTAGE) * kStageBytes;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      // this K group's share of the next stage's loads (branch-free: the last
      // iteration re-loads the last K slice into the idle stage)
#pragma unroll
      for (int u = 0; u < 2 * kInstPerTile / (BK / 16); ++u) {
        const int i = kk * (2 * kInstPerTile / (BK / 16)) + u;
        load_one(i < kInstPerTile ? A : B, i < kInstPerTile ? d.lda : d.ldb, i < kInstPerTile ? m0 : n0,
                 i < kInstPerTile ? d.M : d.N, kpf, nxt + (i < kInstPerTile ? 0 : kTileBytes), wave, lane,
                 i % kInstPerTile);
      }
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(st + abase + i * 32 * kRowBytes + koff[kk]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(st + bbase + j * 32 * kRowBytes + koff[kk]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // the last iteration's re-load of the idle stage must land before the
  // slabs reuse that LDS
  wait_vmcnt<0>();

  // epilogue through per-wave LDS slabs (32 rows x 64 columns), 16-byte stores
  // (a part of a split tile stores its fp32 rows to its partial tile instead)
  bf16_t* C = static_cast<bf16_t*>(d.C);
  const float* S = d.scale;
  float* P = bid >= sp.full
                 ? sp.part + (static_cast<int64_t>(pid - sp.full) * sp.k + part) * (BM * BN)
                 : nullptr;
  float* slab = reinterpret_cast<float*>(smem) + wave * 32 * kSlabStride;
  constexpr int kChunksPerRow = WTN / 8;
  constexpr int kChunksPerLane = 32 * kChunksPerRow / 64;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        slab[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * kSlabStride + j * 32 + lrow] = acc[i][j][r];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kChunksPerLane; ++c) {
      const int ch = lane + c * 64;
      const int row = ch / kChunksPerRow, col = (ch % kChunksPerRow) * 8;
      const int m = m0 + wm * WTM + i * 32 + row;
      const int n = n0 + wn * WTN + col;
      if (P) {
        float* dst = P + (wm * WTM + i * 32 + row) * BN + wn * WTN + col;
        *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(slab + row * kSlabStride + col);
        *reinterpret_cast<float4*>(dst + 4) = *reinterpret_cast<const float4*>(slab + row * kSlabStride + col + 4);
      } else if (m < d.M && n < d.N) {
        const float4 p0 = *reinterpret_cast<const float4*>(slab + row * kSlabStride + col);
        const float4 p1 = *reinterpret_cast<const float4*>(slab + row * kSlabStride + col + 4);
        float v[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        if (S) {
          const float4 s0 = *reinterpret_cast<const float4*>(S + n);
          const float4 s1 = *reinterpret_cast<const float4*>(S + n + 4);
          v[0] *= s0.x; v[1] *= s0.y; v[2] *= s0.z; v[3] *= s0.w;
          v[4] *= s1.x; v[5] *= s1.y; v[6] *= s1.z; v[7] *= s1.w;
        }
        // non-temporal: the output is not read again here, and keeping it
        // out of L2 leaves the operand panels there for the next tiles
        const u32x4_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                           pack_bf16x2(v[6], v[7])};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(C + static_cast<int64_t>(m) * d.ldc + n));
      }
    }
  }
}

// Sum of the k partial tiles of each split tile, in part order, times the
// column scale, to bfloat16: one thread per 8 consecutive columns of a row.
__global__ void __launch_bounds__(256) k_dense_split_sum(const GemmDesc d, int tiles_m, int tiles_n,
                                                         DenseSplit sp) {
  const int slot = blockIdx.x / (BM * BN / 8 / 256);
  const int e = (blockIdx.x % (BM * BN / 8 / 256)) * 256 + threadIdx.x;  // chunk of 8 in the tile
  const int row = e / (BN / 8), col = (e % (BN / 8)) * 8;
  int tm, tn;
  tile_coords(sp.full + slot, tiles_m, tiles_n, tm, tn);
  const int m = tm * BM + row, n = tn * BN + col;
  if (m >= d.M || n >= d.N) return;
  const float* src = sp.part + static_cast<int64_t>(slot) * sp.k * (BM * BN) + row * BN + col;
  float4 a = *reinterpret_cast<const float4*>(src), b = *reinterpret_cast<const float4*>(src + 4);
  for (int p = 1; p < sp.k; ++p) {
    const float4 u = *reinterpret_cast<const float4*>(src + static_cast<int64_t>(p) * (BM * BN));
    const float4 w = *reinterpret_cast<const float4*>(src + static_cast<int64_t>(p) * (BM * BN) + 4);
    a.x += u.x; a.y += u.y; a.z += u.z; a.w += u.w;
    b.x += w.x; b.y += w.y; b.z += w.z; b.w += w.w;
  }
  float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  if (d.scale) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] *= d.scale[n + i];
  }
  bf16_t* C = static_cast<bf16_t*>(d.C);
  *reinterpret_cast<uint4*>(C + static_cast<int64_t>(m) * d.ldc + n) =
      make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
}

}  // namespace

namespace {

constexpr int kCUs = 256;

// Tiles run whole and the split of the last, partial round: k parts per
// tail tile with k * tail <= 256 CUs and at least 8 K steps per part.
struct SplitPlan {
  int tiles, full, k;
};

SplitPlan split_plan(int M, int N, int K) {
  SplitPlan p;
  p.tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int tail = p.tiles % kCUs;
  const int nk = K / BK;
  p.k = 1;
  while (tail > 0 && p.k < 4 && 2 * p.k * tail <= kCUs && nk / (2 * p.k) >= 8) p.k *= 2;
  p.full = p.k > 1 ? p.tiles - tail : p.tiles;
  return p;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

size_t gemm_dense_split_bytes(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const SplitPlan p = split_plan(M, N, K);
  if (p.k == 1) return 0;
  return align256(static_cast<size_t>(p.tiles - p.full) * p.k * BM * BN * sizeof(float));
}

bool gemm_dense_bf16(const GemmDesc& d, void* split_ws, hipStream_t s) {
  if (d.M <= 0 || d.N <= 0) return true;
  if (d.K % 64 != 0 || d.K <= 0 || d.N % 8 != 0) return false;
  const int tm = (d.M + BM - 1) / BM, tn = (d.N + BN - 1) / BN;
  SplitPlan p = split_plan(d.M, d.N, d.K);
  if (!split_ws) p = SplitPlan{p.tiles, p.tiles, 1};
  const DenseSplit sp{static_cast<float*>(split_ws), p.full, p.k};
  const int tail = p.tiles - p.full;
  hipLaunchKernelGGL(k_gemm_dense, dim3(p.full + tail * p.k), dim3(NT), 0, s, d, tm, tn, sp);
  if (tail > 0)
    hipLaunchKernelGGL(k_dense_split_sum, dim3(tail * (BM * BN / 8 / 256)), dim3(256), 0, s, d, tm, tn, sp);
  return true;
}

}  // namespace poetx
