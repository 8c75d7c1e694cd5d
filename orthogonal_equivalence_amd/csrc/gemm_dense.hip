// Dense product C = A B^T (bfloat16 in, float32 accumulate, bfloat16 out) for
// the layer's two W0 products, both on the one resident weight Wp (m x n,
// row-major): Y1 = X2 Wp reads Wp as B[k][n] (N-contiguous rows, K = m) and
// dX2 = dY1 Wp^T reads it as B[n][k] (K-contiguous rows, K = n). A is always
// K-contiguous.
//
// gfx950 design:
//  * 256 x 256 output tile per workgroup, K in steps of 64, 8 waves (two per
//    SIMD, so one wave's LDS waits hide behind the other's MFMAs); each wave
//    owns 128 x 64 outputs as 4 x 2 tiles of v_mfma_f32_32x32x16_bf16.
//  * Operand tiles go global -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging, no LDS write instructions), double-buffered, one barrier per
//    K step. The next stage's loads are spread over the current stage's four
//    K groups (2, 3, 3 and none of the eight 1 KB loads per wave) rather than
//    issued in one burst, so that their LDS writes interleave with the
//    fragment reads and each has a group's MFMAs to land in.
//  * LDS rows are 128 bytes, unpadded; 16-byte chunk c of row r sits in slot
//    c ^ swz(r) with swz(r) = (r & 7) ^ ((r >> 3) & 1), which keeps the
//    fragment reads (32 rows, same chunk) free of bank conflicts whether the
//    LDS serves 8 or 16 lanes of a 16-byte read per cycle.
//  * An N-contiguous B tile is stored as it lies in memory, 64 K rows of 256
//    columns (512 bytes), with chunk c of row r in slot c ^ 4 (r % 4). Its
//    MFMA fragments (8 consecutive k of one column per lane) come from pairs
//    of ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives
//    element j % 4 of the 8 bytes addressed by lane 4e + j / 4 (e = 0..3),
//    so with lane i addressing row k0 + i / 4 at column n0 + 4 (i % 4), lane
//    j gets rows k0 .. k0+3 of column n0 + j. The four rows a read touches
//    then fall in four different 64-byte quarters of the 256-byte bank
//    window, and the 32 columns of a fragment are 64 contiguous bytes.
//  * An int8 B (the quantised base weight) is dequantised inside the
//    product: its tiles go global -> LDS as int8 (half the bytes of bfloat16)
//    into a staging area of two 16 KB buffers, with the direct loads, two K
//    steps ahead (after that step's A loads, so that the wait at the top of a
//    step leaves them in flight). At the end of the step before its own, each
//    wave converts the chunks it loaded itself (no barrier needed) exactly to
//    bfloat16 (|code| <= 127 has at most 8 significant bits) into the same
//    LDS layouts as a bfloat16 B, K-contiguous or N-contiguous. The column
//    scales are applied in the epilogue as for any scaled product. An fp8 B
//    (OCP E4M3 bytes, the same storage with 4-bit exponents) takes the same
//    route with v_cvt_pk_f32_fp8 as the conversion (exact: 4 significant
//    bits, exponents from 2^-9 to 2^8).
//  * Output tiles are ordered so that each XCD works on one contiguous band
//    of tiles (shared A/B panels stay in that XCD's L2).
//  * Whole rounds of whole tiles with a K-contiguous B (the backward) run
//    persistently, one workgroup per CU over its band's tiles, so that each
//    tile boundary overlaps the next tile's first loads and the epilogue's
//    stores (k_gemm_dense_persist); with the N-contiguous B of the forward
//    the same scheme measured slower and is not used.
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

// N-contiguous B tile (BK rows of k, BN columns): instruction i of a wave
// covers two 512-byte rows; lane l lands in slot l % 32 of row l / 32 and
// fetches the chunk that belongs there. Columns past `collim` re-read the
// last chunk of the row (in bounds); they only reach outputs never stored.
constexpr int kNcRowBytes = BN * 2;                 // 512
constexpr int kNcChunks = kNcRowBytes / 16;         // 32
constexpr int kNcRowsPerInst = 64 / kNcChunks;      // 2
static_assert(BK * kNcRowBytes == kTileBytes, "N-contiguous B tile size");

__device__ __forceinline__ int swz_nc(int r) { return (r & 3) << 2; }

// Element offset of lane `lane`'s chunk for instruction i, relative to row
// k0 of the tile (the row term k0 * ld is uniform and added per K step).
__device__ __forceinline__ int64_t nc_offset(int64_t ld, int col0, int collim, int wave, int lane, int i) {
  const int sub = lane / kNcChunks, slot = lane % kNcChunks;
  const int r = (wave * kInstPerTile + i) * kNcRowsPerInst + sub;
  const int c = slot ^ swz_nc(r);
  int col = col0 + c * 8;
  col = col < collim ? col : collim - 8;
  return static_cast<int64_t>(r) * ld + col;
}

__device__ __forceinline__ void load_one_nc(const bf16_t* __restrict__ g_k0, int64_t off, char* lds, int wave, int i) {
  const int rbase = (wave * kInstPerTile + i) * kNcRowsPerInst;
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(g_k0 + off), (lds_void_t)(lds + rbase * kNcRowBytes), 16,
                                   0, 0);
}

// The next stage's 2 kInstPerTile = 8 loads per wave, spread over the current
// stage's four K groups: group kk issues loads [load_first(kk),
// load_first(kk + 1)). Two right after the barrier (all eight waves issue
// theirs at once there), three and three in the next two groups, none in the
// last, so that every load has at least a group's MFMAs to land in; measured
// against an even 2-2-2-2 spread at the 8B shapes: forward 0.820 -> 0.807 ms,
// backward 0.751 -> 0.748 ms.
// Other stage shapes spread their loads evenly, and so does the int8
// N-contiguous (forward) kernel, whose B comes as codes in two loads per wave
// and step: there the even spread measured 0.87-0.90 ms against 0.94 ms.
template <bool EVEN>
__host__ __device__ constexpr int load_first(int kk) {
  constexpr int kGroups = BK / 16, kLoads = 2 * kInstPerTile;
  if constexpr (!EVEN && kGroups == 4 && kLoads == 8) return kk <= 0 ? 0 : (kk == 1 ? 2 : (kk == 2 ? 5 : 8));
  else return kk * kLoads / kGroups;
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

// Sixteen int8 codes as sixteen bfloat16 values (exact): each code widened
// to float, whose low 16 bits are zero for |code| <= 127.
__device__ __forceinline__ void i8x16_to_bf16(const uint4 raw, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t o[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float f0 = static_cast<float>(static_cast<int8_t>(w[q] & 0xffu));
    const float f1 = static_cast<float>(static_cast<int8_t>((w[q] >> 8) & 0xffu));
    const float f2 = static_cast<float>(static_cast<int8_t>((w[q] >> 16) & 0xffu));
    const float f3 = static_cast<float>(static_cast<int8_t>(w[q] >> 24));
    o[2 * q] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
    o[2 * q + 1] = (__float_as_uint(f2) >> 16) | (__float_as_uint(f3) & 0xffff0000u);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// Sixteen E4M3 fp8 codes as sixteen bfloat16 values (exact): v_cvt_pk_f32_fp8
// turns two bytes of a word into two floats (OCP E4M3 on gfx950), whose low
// 16 bits are zero.
__device__ __forceinline__ void f8x16_to_bf16(const uint4 raw, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t o[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[q]), false);  // bytes 0, 1
    const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w[q]), true);   // bytes 2, 3
    o[2 * q] = (__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xffff0000u);
    o[2 * q + 1] = (__float_as_uint(b[0]) >> 16) | (__float_as_uint(b[1]) & 0xffff0000u);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// int8 B tile: 16 KB of codes per stage, two 1 KB direct loads per wave.
constexpr int kI8StageBytes = BN * BK;
constexpr int kI8Chunks = kI8StageBytes / 1024 / (NT / 64);  // 2
static_assert(NSTAGE * 2 * BM * BK * 2 + 2 * kI8StageBytes <= 160 * 1024, "LDS with int8 staging");

// One K group (16 of the stage's K) of a wave's 128 x 64 outputs: A
// fragments from the stage's A rows, B fragments from its B rows (K-contiguous)
// or through transposed reads of its K rows (N-contiguous, inline asm that
// waits for its own results: as the builtin, the read gets a vmcnt(0) in front
// of it while direct loads are in flight), then the 4 x 2 MFMAs.
template <bool BNC>
__device__ __forceinline__ void kgroup_mfma(const char* st, int kk, const int (&koff)[BK / 16], int abase, int bbase,
                                            const uint32_t (&bnc_addr)[TN], f32x16_t (&acc)[TM][TN]) {
  bf16x8_t af[TM], bfr[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(st + abase + i * 32 * kRowBytes + koff[kk]);
  if constexpr (BNC) {
    typedef unsigned long long u64;
    typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
    const uint32_t sb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(st)) + kk * 16 * kNcRowBytes;
    const uint32_t a0 = sb + bnc_addr[0], a1 = sb + bnc_addr[1];
    u64 rb[4];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n ds_read_b64_tr_b16 %1, %4 offset:2048\n"
        "ds_read_b64_tr_b16 %2, %5\n ds_read_b64_tr_b16 %3, %5 offset:2048\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(rb[0]), "=&v"(rb[1]), "=&v"(rb[2]), "=&v"(rb[3])
        : "v"(a0), "v"(a1)
        : "memory");
    bfr[0] = __builtin_bit_cast(bf16x8_t, u64x2{rb[0], rb[1]});
    bfr[1] = __builtin_bit_cast(bf16x8_t, u64x2{rb[2], rb[3]});
  } else {
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bfr[j] = *reinterpret_cast<const bf16x8_t*>(st + bbase + j * 32 * kRowBytes + koff[kk]);
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
}

// BNC: B is N-contiguous (B[k * ldb + n]) instead of K-contiguous.
// BI8: B holds 1-byte codes (ldb in elements = bytes): int8, or with BF8
// OCP E4M3 fp8 bytes.
template <bool BNC, bool BI8, bool BF8 = false>
__global__ void __launch_bounds__(NT, 1) k_gemm_dense(const GemmDesc d, int tiles_m, int tiles_n, DenseSplit sp) {
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * kStageBytes + (BI8 ? 2 * kI8StageBytes : 0)];
  char* const i8st = smem + NSTAGE * kStageBytes;  // int8 staging (BI8 only)

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
  // N-contiguous B: transposed-read address of this lane in the stage for
  // column tile j, first row of K group 0. Lane group G = lane / 16 takes
  // columns 16 (G % 2) .. of the fragment and rows 8 (G / 2) ..; lane i of
  // the group addresses row + i / 4, column + 4 (i % 4). Rows +4 (second half
  // of a fragment) and +16 (next K group) keep the row's swizzle, so they are
  // 2048 and 8192 bytes further.
  uint32_t bnc_addr[TN];
  int64_t bnc_goff[kInstPerTile];
  // int8 B: per chunk, its element offset in B relative to K step k0 (add
  // k0 for K-contiguous rows, k0 * ldb for N-contiguous ones) and the LDS
  // offsets (within a B tile) of the two bfloat16 chunks it becomes
  int64_t i8_goff[kI8Chunks];
  int i8_lds[kI8Chunks][2];
  if constexpr (BI8) {
#pragma unroll
    for (int u = 0; u < kI8Chunks; ++u) {
      // chunk q of the tile: lane `lane` of this wave's direct load u
      const int q = (wave * kI8Chunks + u) * 64 + lane;
      if constexpr (BNC) {
        const int row = q >> 4, part = q & 15;  // K row, 16 columns
        int col = n0 + part * 16;
        col = col < d.N ? col : d.N - 16;
        i8_goff[u] = static_cast<int64_t>(row) * d.ldb + col;
        i8_lds[u][0] = row * kNcRowBytes + (((2 * part) ^ swz_nc(row)) << 4);
        i8_lds[u][1] = row * kNcRowBytes + (((2 * part + 1) ^ swz_nc(row)) << 4);
      } else {
        const int row = q >> 2, part = q & 3;  // N row, 16 K values
        int gr = n0 + row;
        gr = gr < d.N ? gr : d.N - 1;
        i8_goff[u] = static_cast<int64_t>(gr) * d.ldb + part * 16;
        i8_lds[u][0] = row * kRowBytes + (((2 * part) ^ swz(row)) << 4);
        i8_lds[u][1] = row * kRowBytes + (((2 * part + 1) ^ swz(row)) << 4);
      }
    }
  }
  const int8_t* Bq = static_cast<const int8_t*>(d.B);
  // direct loads of this wave's share of stage-K-step k0's codes into
  // staging buffer sb
  auto i8_load = [&](int k0, int sb) {
    const int8_t* base = BNC ? Bq + static_cast<int64_t>(k0) * d.ldb : Bq + k0;
#pragma unroll
    for (int u = 0; u < kI8Chunks; ++u)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(base + i8_goff[u]),
                                       (lds_void_t)(i8st + sb * kI8StageBytes + (wave * kI8Chunks + u) * 1024), 16,
                                       0, 0);
  };
  // this wave's chunks of staging buffer sb, as bfloat16 into B tile btile
  // (the staging reads are inline asm that waits for its own results: read
  // through ordinary loads they get a vmcnt(0) in front of them, which would
  // drain the loads in flight; the caller has waited for this buffer's loads)
  auto i8_convert = [&](int sb, char* btile) {
    static_assert(kI8Chunks == 2, "two staged chunks per lane");
    u32x4_t rawv[2];
    const uint32_t ad = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(i8st)) + sb * kI8StageBytes +
                        wave * kI8Chunks * 1024 + lane * 16;
    asm volatile("ds_read_b128 %0, %2\n ds_read_b128 %1, %2 offset:1024\n s_waitcnt lgkmcnt(0)"
                 : "=&v"(rawv[0]), "=&v"(rawv[1])
                 : "v"(ad)
                 : "memory");
    const uint4 raw[2] = {make_uint4(rawv[0][0], rawv[0][1], rawv[0][2], rawv[0][3]),
                          make_uint4(rawv[1][0], rawv[1][1], rawv[1][2], rawv[1][3])};
    // the writes, likewise from inline asm: as ordinary stores they get a
    // vmcnt(0) in front of them (the direct loads in flight target other
    // LDS: the next stage's A tile and the other staging buffer)
    u32x4_t cv[2][2];
#pragma unroll
    for (int u = 0; u < kI8Chunks; ++u) {
      uint4 lo, hi;
      if constexpr (BF8) f8x16_to_bf16(raw[u], lo, hi);
      else i8x16_to_bf16(raw[u], lo, hi);
      cv[u][0] = u32x4_t{lo.x, lo.y, lo.z, lo.w};
      cv[u][1] = u32x4_t{hi.x, hi.y, hi.z, hi.w};
    }
    const uint32_t bt = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(btile));
    asm volatile(
        "ds_write_b128 %0, %4\n ds_write_b128 %1, %5\n ds_write_b128 %2, %6\n ds_write_b128 %3, %7\n"
        " s_waitcnt lgkmcnt(0)"
        :
        : "v"(bt + i8_lds[0][0]), "v"(bt + i8_lds[0][1]), "v"(bt + i8_lds[1][0]), "v"(bt + i8_lds[1][1]),
          "v"(cv[0][0]), "v"(cv[0][1]), "v"(cv[1][0]), "v"(cv[1][1])
        : "memory");
  };
  if constexpr (BNC) {
#pragma unroll
    for (int i = 0; i < kInstPerTile; ++i) bnc_goff[i] = nc_offset(d.ldb, n0, d.N, wave, lane, i);
    const int grp = lane >> 4, li = lane & 15;
    const int r = 8 * (grp >> 1) + (li >> 2);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = wn * WTN + j * 32 + 16 * (grp & 1) + 4 * (li & 3);
      bnc_addr[j] = static_cast<uint32_t>(kTileBytes + r * kNcRowBytes + (((col >> 3) ^ swz_nc(r)) << 4) +
                                          (col & 7) * 2);
    }
  }

  // prologue: stages 0 .. NSTAGE-2 in flight
#pragma unroll
  for (int p = 0; p < NSTAGE - 1; ++p) {
    if (p < nk) {
      load_tile(A, d.lda, m0, d.M, (kb + p) * BK, smem + p * kStageBytes, wave, lane);
      if constexpr (BI8) {
        i8_load((kb + p) * BK, 0);
        wait_vmcnt<0>();
        i8_convert(0, smem + p * kStageBytes + kTileBytes);
      } else if constexpr (BNC) {
        const bf16_t* Bk = B + static_cast<int64_t>((kb + p) * BK) * d.ldb;
#pragma unroll
        for (int i = 0; i < kInstPerTile; ++i) load_one_nc(Bk, bnc_goff[i], smem + p * kStageBytes + kTileBytes, wave, i);
      } else {
        load_tile(B, d.ldb, n0, d.N, (kb + p) * BK, smem + p * kStageBytes + kTileBytes, wave, lane);
      }
    }
  }

  // int8 B: the codes of the stage after the one being computed, in staging
  // buffer 1 (step `it` converts buffer (it + 1) % 2 and loads into it % 2)
  if constexpr (BI8) i8_load((kb + min(1, nk - 1)) * BK, 1);

  for (int it = 0; it < nk; ++it) {
    // stage `it` is the oldest of the (up to NSTAGE - 1) stages in flight;
    // loads complete in order, so waiting until the younger ones remain
    // suffices. Near the end fewer younger stages exist. With an int8 B the
    // youngest loads are the next stage's codes, which stay in flight.
    constexpr int kPerStage = 2 * kInstPerTile;
    const int younger = min(NSTAGE - 2, nk - 1 - it);
    if constexpr (BI8) {
      // a bare barrier: __syncthreads() would also wait for the codes in flight
      wait_vmcnt<kI8Chunks>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      if (younger >= 2) wait_vmcnt<2 * kPerStage>();
      else if (younger == 1) wait_vmcnt<kPerStage>();
      else wait_vmcnt<0>();
      __syncthreads();
    }
    const int pf = it + NSTAGE - 1;
    char* nxt = smem + (pf % NSTAGE) * kStageBytes;
    const int kpf = (kb + min(pf, nk - 1)) * BK;
    const char* st = smem + (it % NSTAGE) * kStageBytes;
    const bf16_t* Bpf = BNC ? B + static_cast<int64_t>(kpf) * d.ldb : B;

#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      // this K group's share of the next stage's loads (branch-free: the last
      // iteration re-loads the last K slice into the idle stage)
#pragma unroll
      for (int i = load_first<BI8 && BNC>(kk); i < load_first<BI8 && BNC>(kk + 1); ++i) {
        if constexpr (BI8) {
          if (i >= kInstPerTile) {
            // B comes through registers: once the A loads are out
            if (i == kInstPerTile) i8_load((kb + min(it + 2, nk - 1)) * BK, it & 1);
            continue;
          }
        }
        if (BNC && i >= kInstPerTile)
          load_one_nc(Bpf, bnc_goff[i % kInstPerTile], nxt + kTileBytes, wave, i % kInstPerTile);
        else
          load_one(i < kInstPerTile ? A : B, i < kInstPerTile ? d.lda : d.ldb, i < kInstPerTile ? m0 : n0,
                   i < kInstPerTile ? d.M : d.N, kpf, nxt + (i < kInstPerTile ? 0 : kTileBytes), wave, lane,
                   i % kInstPerTile);
      }
      kgroup_mfma<BNC>(st, kk, koff, abase, bbase, bnc_addr, acc);
      if constexpr (BI8) {
        // the next stage's codes, loaded one step ago, into its B tile; younger
        // loads are this step's A loads and the codes two stages ahead
        // (in-order completion). N-contiguous: between the last two K groups,
        // while this group's MFMAs run; K-contiguous: after the last group
        // (each measured faster for its layout).
        if (kk == (BNC ? BK / 16 - 2 : BK / 16 - 1)) {
          wait_vmcnt<kInstPerTile + kI8Chunks>();
          i8_convert((it + 1) & 1, nxt + kTileBytes);
        }
      }
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
  // every wave is done with the stages before the slabs overwrite them; the
  // slabs are per wave, so the passes need no further barrier (one wave's
  // LDS accesses complete in order)
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        slab[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * kSlabStride + j * 32 + lrow] = acc[i][j][r];
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
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

// Persistent variant for a bfloat16 B with M and N multiples of 256, no
// column scale and a tile count that fills whole rounds of the 256 CUs: one
// workgroup per CU walks the tiles that one-tile-per-workgroup launches give
// the workgroups of its XCD band, in the same order. The tile boundary
// overlaps: during a tile's last K step the free stage buffer receives the
// next tile's first K slice; the epilogue goes through 16-row slabs in the
// other buffer; the next tile's first step issues its second slice and runs
// its MFMAs while the epilogue's stores drain (they are waited for only at
// its second step, with that slice).
template <bool BNC>
__global__ void __launch_bounds__(NT, 1) k_gemm_dense_persist(const GemmDesc d, int tiles_m, int tiles_n, int ntiles) {
  static_assert(NSTAGE == 2, "two stage buffers");
  constexpr int kSlabRows = 16;
  static_assert(NT / 64 * kSlabRows * kSlabStride * 4 <= kStageBytes, "slabs fit one stage buffer");
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * kStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WM, wn = wave / WM;
  const bf16_t* A = static_cast<const bf16_t*>(d.A);
  const bf16_t* B = static_cast<const bf16_t*>(d.B);
  bf16_t* C = static_cast<bf16_t*>(d.C);
  const int nk = d.K / BK;
  const int stride = static_cast<int>(gridDim.x);

  const int lrow = lane & 31;
  const int sw = swz(lrow);
  int koff[BK / 16];
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) koff[kk] = lrow * kRowBytes + (((2 * kk + (lane >> 5)) ^ sw) << 4);
  const int abase = wm * WTM * kRowBytes;
  const int bbase = kTileBytes + wn * WTN * kRowBytes;
  uint32_t bnc_addr[TN];
  if constexpr (BNC) {
    const int grp = lane >> 4, li = lane & 15;
    const int r = 8 * (grp >> 1) + (li >> 2);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = wn * WTN + j * 32 + 16 * (grp & 1) + 4 * (li & 3);
      bnc_addr[j] = static_cast<uint32_t>(kTileBytes + r * kNcRowBytes + (((col >> 3) ^ swz_nc(r)) << 4) +
                                          (col & 7) * 2);
    }
  }

  auto coords = [&](int v, int& m0, int& n0) {
    int tm, tn;
    tile_coords(xcd_remap(v, ntiles), tiles_m, tiles_n, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
  };
  int v = static_cast<int>(blockIdx.x);
  int m0, n0;
  coords(v, m0, n0);
  int64_t goff[kInstPerTile];
  if constexpr (BNC) {
#pragma unroll
    for (int i = 0; i < kInstPerTile; ++i) goff[i] = nc_offset(d.ldb, n0, d.N, wave, lane, i);
  }

  // the first tile's first K slice into buffer 0
  load_tile(A, d.lda, m0, d.M, 0, smem, wave, lane);
  if constexpr (BNC) {
#pragma unroll
    for (int i = 0; i < kInstPerTile; ++i) load_one_nc(B, goff[i], smem + kTileBytes, wave, i);
  } else {
    load_tile(B, d.ldb, n0, d.N, 0, smem + kTileBytes, wave, lane);
  }

  int base = 0;  // stage buffer of the current tile's first K step
  bool first = true;
  for (; v < ntiles; v += stride) {
    // the next tile; after the last one, this tile again (a harmless re-load
    // of its first slice into the free buffer)
    int m1 = m0, n1 = n0;
    if (v + stride < ntiles) coords(v + stride, m1, n1);

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    for (int it = 0; it < nk; ++it) {
      // slice `it` has landed once nothing older is in flight; a later tile's
      // first slice was waited for before the epilogue, so its first step
      // leaves the epilogue's stores in flight. The barrier is a bare one
      // (__syncthreads would wait for the stores too).
      if (first || it > 0) wait_vmcnt<0>();
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      const int cur = (base + it) & 1;
      const char* st = smem + cur * kStageBytes;
      char* nxt = smem + (cur ^ 1) * kStageBytes;
      const bool last = it == nk - 1;
      if constexpr (BNC) {
        // the last step loads the next tile: its B offsets replace this one's
        if (last) {
#pragma unroll
          for (int i = 0; i < kInstPerTile; ++i) goff[i] = nc_offset(d.ldb, n1, d.N, wave, lane, i);
        }
      }
      const int kpf = last ? 0 : (it + 1) * BK;
      const int am = last ? m1 : m0, bn = last ? n1 : n0;
      const bf16_t* Bpf = BNC ? B + static_cast<int64_t>(kpf) * d.ldb : B;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
#pragma unroll
        for (int i = load_first<false>(kk); i < load_first<false>(kk + 1); ++i) {
          if (BNC && i >= kInstPerTile)
            load_one_nc(Bpf, goff[i % kInstPerTile], nxt + kTileBytes, wave, i % kInstPerTile);
          else
            load_one(i < kInstPerTile ? A : B, i < kInstPerTile ? d.lda : d.ldb, i < kInstPerTile ? am : bn,
                     i < kInstPerTile ? d.M : d.N, kpf, nxt + (i < kInstPerTile ? 0 : kTileBytes), wave, lane,
                     i % kInstPerTile);
        }
        kgroup_mfma<BNC>(st, kk, koff, abase, bbase, bnc_addr, acc);
      }
    }

    // epilogue: the next tile's first slice has landed in buffer (base + nk)
    // & 1; every wave is past its last reads of the other buffer, which holds
    // the slabs (16 rows x 64 columns per wave and pass)
    wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    float* slab = reinterpret_cast<float*>(smem + ((base + nk - 1) & 1) * kStageBytes) + wave * kSlabRows * kSlabStride;
    constexpr int kChunksPerRow = WTN / 8;
    constexpr int kChunksPerLane = kSlabRows * kChunksPerRow / 64;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int r = 8 * hh; r < 8 * hh + 8; ++r)
            slab[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) - kSlabRows * hh) * kSlabStride + j * 32 + lrow] =
                acc[i][j][r];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int c = 0; c < kChunksPerLane; ++c) {
          const int ch = lane + c * 64;
          const int row = ch / kChunksPerRow, col = (ch % kChunksPerRow) * 8;
          const int m = m0 + wm * WTM + i * 32 + kSlabRows * hh + row;
          const int n = n0 + wn * WTN + col;
          const float4 p0 = *reinterpret_cast<const float4*>(slab + row * kSlabStride + col);
          const float4 p1 = *reinterpret_cast<const float4*>(slab + row * kSlabStride + col + 4);
          const u32x4_t w = {pack_bf16x2(p0.x, p0.y), pack_bf16x2(p0.z, p0.w), pack_bf16x2(p1.x, p1.y),
                             pack_bf16x2(p1.z, p1.w)};
          __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(C + static_cast<int64_t>(m) * d.ldc + n));
        }
        // this pass's slab reads are complete before the next pass's writes
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    }
    base = (base + nk) & 1;
    m0 = m1;
    n0 = n1;
    first = false;
  }
  // the last tile's re-load must land before the workgroup's LDS is released
  wait_vmcnt<0>();
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

bool gemm_dense_bf16(const GemmDesc& d, void* split_ws, hipStream_t s, bool b_ncontig, bool b_int8) {
  if (d.M <= 0 || d.N <= 0) return true;
  if (d.K % 64 != 0 || d.K <= 0 || d.N % 8 != 0) return false;
  if (b_int8 && (d.N % 16 != 0 || d.ldb % 16 != 0)) return false;
  const int tm = (d.M + BM - 1) / BM, tn = (d.N + BN - 1) / BN;
  SplitPlan p = split_plan(d.M, d.N, d.K);
  if (!split_ws) p = SplitPlan{p.tiles, p.tiles, 1};
#ifndef POETX_DENSE_PERSIST
#define POETX_DENSE_PERSIST 1
#endif
  // the persistent kernel for K-contiguous B (the N-contiguous forward
  // measured 10 us slower with it, the backward 15 us faster at the 8B shape)
  if (POETX_DENSE_PERSIST && !b_int8 && !b_ncontig && !d.scale && d.M % BM == 0 && d.N % BN == 0 &&
      p.tiles % kCUs == 0) {
    hipLaunchKernelGGL(k_gemm_dense_persist<false>, dim3(kCUs), dim3(NT), 0, s, d, tm, tn, p.tiles);
    return true;
  }
  const DenseSplit sp{static_cast<float*>(split_ws), p.full, p.k};
  const int tail = p.tiles - p.full;
  const dim3 grid(p.full + tail * p.k);
  if (b_int8) {
    if (d.b_fp8) {
      if (b_ncontig) hipLaunchKernelGGL((k_gemm_dense<true, true, true>), grid, dim3(NT), 0, s, d, tm, tn, sp);
      else hipLaunchKernelGGL((k_gemm_dense<false, true, true>), grid, dim3(NT), 0, s, d, tm, tn, sp);
    } else {
      if (b_ncontig) hipLaunchKernelGGL((k_gemm_dense<true, true>), grid, dim3(NT), 0, s, d, tm, tn, sp);
      else hipLaunchKernelGGL((k_gemm_dense<false, true>), grid, dim3(NT), 0, s, d, tm, tn, sp);
    }
  } else {
    if (b_ncontig) hipLaunchKernelGGL((k_gemm_dense<true, false>), grid, dim3(NT), 0, s, d, tm, tn, sp);
    else hipLaunchKernelGGL((k_gemm_dense<false, false>), grid, dim3(NT), 0, s, d, tm, tn, sp);
  }
  if (tail > 0)
    hipLaunchKernelGGL(k_dense_split_sum, dim3(tail * (BM * BN / 8 / 256)), dim3(256), 0, s, d, tm, tn, sp);
  return true;
}

}  // namespace poetx
