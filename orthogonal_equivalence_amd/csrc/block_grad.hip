// Token reduction of the block gradients: for one 256-wide slice pair of a
// block and one chunk of tokens,
//   part[i][c] = sum_t act[t][a0 + i] * dout[t][d0 + c]      (i, c < 256)
// i.e. dG_j = X1_J^T dX2_J and dH_k = Y1_K^T dY2_K of the backward (W0 is
// frozen, so these b x b sums replace the T x m x n weight gradient; zhichai.net
// digest of arXiv:2603.05500, section "1. 输入中心化架构"). Blocks of 512
// columns are four slice pairs.
//
// gfx950 design: the contraction runs over tokens while the activations are
// stored token-major, so the MFMA fragments (8 consecutive tokens of one
// feature per lane) are columns of the staged tiles. The tiles go global ->
// LDS token-major with global_load_lds_dwordx4 (no register staging), and the
// fragments are read with ds_read_b64_tr_b16: within each group of 16 lanes,
// lane j receives element (j % 4) of the 8 bytes addressed by lane
// 4e + j / 4, for e = 0..3. With lane i addressing token row t0 + i / 4 at
// feature f0 + 4 (i % 4), lane j gets tokens t0 .. t0+3 of feature f0 + j;
// two such reads make one fragment. 32-token sub-tiles in four stages (three
// in flight ahead of the one being multiplied); eight waves each hold a
// 128 x 64 region of the 256 x 256 fp32 partial in registers for the whole
// chunk; one store of the partial at the end.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace poetx {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16* lds_v4i16_t;

constexpr int S = 256;              // slice width
constexpr int TK = 32;              // tokens per sub-tile
constexpr int NT = 512;             // threads
constexpr int NSTAGE = 4;
constexpr int ROWB = S * 2;         // bytes per token row of a tile (512)
constexpr int TILE = TK * ROWB;     // one operand tile (16 KB)
constexpr int STAGE = 2 * TILE;     // act + dout

// Slot of 16-byte chunk c (0..31) in token row r: c ^ (4 (r % 4)). A
// transposed read touches rows t0 .. t0+3 (and t0+8 .. t0+11) at 4
// consecutive chunks c0 .. c0+3 (c0 a multiple of 4): the XOR spreads the
// four rows over all 16 bank groups, two cycles per read.
__device__ __forceinline__ int slot(int r, int c) { return c ^ ((r & 3) << 2); }

// One side's operands: act and dout [T][dim] (row stride dim), partials
// [nsplit][nblk][b][b].
struct GradSide {
  const bf16_t* act;
  const bf16_t* dout;
  float* part;
  int64_t dim;          // row width (short last block)
  int nblk;
};

// Up to two sides with the same block size and token split in one launch:
// workgroups [0, wgs0) take side 0, the rest side 1.
struct GradArgs {
  GradSide side[2];
  int wgs0;
  int64_t T;
  int b;                // block size (256 or 512)
  int slices;           // b / 256
  int tokens_per_wg;
  int nsplit;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__global__ void __launch_bounds__(NT) k_block_grad(const GradArgs g) {
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (side, block, slice pair, split)
  const int pairs = g.slices * g.slices;
  int w = blockIdx.x;
  const bool second = w >= g.wgs0;
  const GradSide sd = second ? g.side[1] : g.side[0];
  if (second) w -= g.wgs0;
  const int split = w % g.nsplit;
  w /= g.nsplit;
  const int pair = w % pairs;
  const int blk = w / pairs;
  const int si = pair / g.slices, sc = pair % g.slices;
  const int64_t blk0 = static_cast<int64_t>(blk) * g.b;
  const int width = static_cast<int>(min(static_cast<int64_t>(g.b), sd.dim - blk0));
  const int a0 = si * S, d0 = sc * S;  // slice offsets inside the block
  const int64_t t_begin = static_cast<int64_t>(split) * g.tokens_per_wg;
  const int64_t t_end = min(g.T, t_begin + g.tokens_per_wg);
  const int nsub = t_end > t_begin ? static_cast<int>((t_end - t_begin + TK - 1) / TK) : 0;

  // loads: a stage is 2 x 16 KB = 32 instructions of 1 KB, four per wave
  // (two act, two dout); lane -> (row, chunk slot) of a 2-row instruction.
  // Features past the block's width re-read its last 8 valid features (their
  // outputs are stored as zeros), so every load stays inside the block even
  // when a whole slice lies past a short block; tokens past the chunk re-read
  // its last token (masked in the act fragments).
  auto issue = [&](int sub, char* st) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int op = u >> 1;                  // 0 act, 1 dout
      const int inst = wave * 2 + (u & 1);    // 0..15 within the operand tile
      const int row = inst * 2 + (lane >> 5);
      const int sl = lane & 31;
      const int c = sl ^ ((row & 3) << 2);    // the chunk that lands in slot sl
      int f = (op ? d0 : a0) + c * 8;         // feature offset inside the block
      f = f < width - 8 ? f : width - 8;
      int64_t t = t_begin + static_cast<int64_t>(sub) * TK + row;
      t = t < t_end ? t : t_end - 1;
      const bf16_t* src = (op ? sd.dout : sd.act) + t * sd.dim + blk0 + f;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src),
                                       (lds_void_t)(st + op * TILE + inst * 1024), 16, 0, 0);
    }
  };

  // wave region: features rw0 .. rw0+127 of act, cw0 .. cw0+63 of dout
  constexpr int TMw = 4, TNw = 2;
  const int rw0 = (wave & 1) * 128, cw0 = (wave >> 1) * 64;
  // transposed-read address of this lane inside a 32-feature x 16-token
  // fragment at (feature base fb, token base kb): group G = lane / 16 takes
  // features fb + 16 (G % 2) .., tokens kb + 8 (G / 2) ..; lane i of the group
  // addresses token row + i / 4, feature + 4 (i % 4)
  const int grp = lane >> 4, li = lane & 15;
  const int f_in = 16 * (grp & 1) + 4 * (li & 3);   // feature offset in the fragment
  const int t_in = 8 * (grp >> 1) + (li >> 2);       // token offset in the fragment (first read)
  auto tr_addr = [&](const char* tile, int fb, int t) {
    const int f = fb + f_in;
    const int c = f >> 3;
    return reinterpret_cast<const v4i16*>(tile + t * ROWB + (slot(t, c) << 4) + (f & 7) * 2);
  };
  // the feature and first token this lane receives in the fragment (for masking)
  const int tok_recv = 8 * (lane >> 5);

  f32x16_t acc[TMw][TNw];
#pragma unroll
  for (int i = 0; i < TMw; ++i)
#pragma unroll
    for (int j = 0; j < TNw; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  for (int p = 0; p < NSTAGE - 1 && p < nsub; ++p) issue(p, smem + p * STAGE);
  for (int s = 0; s < nsub; ++s) {
    // stage s has landed once only the younger stages' loads remain
    const int younger = min(NSTAGE - 2, nsub - 1 - s);
    if (younger >= 2) wait_vmcnt<8>();
    else if (younger == 1) wait_vmcnt<4>();
    else wait_vmcnt<0>();
    // LDS-only barrier (the loads in flight are waited for by count above)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const char* A = smem + (s % NSTAGE) * STAGE;
    const char* B = A + TILE;
    const int valid = static_cast<int>(min(static_cast<int64_t>(TK), t_end - t_begin - static_cast<int64_t>(s) * TK));
    // the loads three stages ahead first, into the buffer the step before
    // read (every wave is past those reads at the barrier; issued here they
    // measured 3 us faster than after the fragment reads), then all fragments
    // of the stage, then the MFMAs.
    if (s + NSTAGE - 1 < nsub) issue(s + NSTAGE - 1, smem + ((s + NSTAGE - 1) % NSTAGE) * STAGE);
    // The transposed reads are issued from inline asm that waits for them
    // itself (every output is complete when the asm statement ends): the
    // compiler otherwise places a vmcnt(0) before each such read while direct
    // loads are in flight, which would drain the prefetched stages. Rows +4
    // (second half of a fragment) and +16 (second K group) keep the row
    // swizzle, so they are immediate offsets of 2048 and 8192 bytes.
    bf16x8_t af[TK / 16][TMw], bfr[TK / 16][TNw];
    {
      uint32_t ad[TMw], bd[TNw];
#pragma unroll
      for (int i = 0; i < TMw; ++i)
        ad[i] = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tr_addr(A, rw0 + i * 32, t_in)));
#pragma unroll
      for (int j = 0; j < TNw; ++j)
        bd[j] = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tr_addr(B, cw0 + j * 32, t_in)));
      typedef unsigned long long u64;
      u64 ra[16], rb[8];
      asm volatile(
          "ds_read_b64_tr_b16 %0, %16\n ds_read_b64_tr_b16 %1, %16 offset:2048\n"
          "ds_read_b64_tr_b16 %2, %16 offset:8192\n ds_read_b64_tr_b16 %3, %16 offset:10240\n"
          "ds_read_b64_tr_b16 %4, %17\n ds_read_b64_tr_b16 %5, %17 offset:2048\n"
          "ds_read_b64_tr_b16 %6, %17 offset:8192\n ds_read_b64_tr_b16 %7, %17 offset:10240\n"
          "ds_read_b64_tr_b16 %8, %18\n ds_read_b64_tr_b16 %9, %18 offset:2048\n"
          "ds_read_b64_tr_b16 %10, %18 offset:8192\n ds_read_b64_tr_b16 %11, %18 offset:10240\n"
          "ds_read_b64_tr_b16 %12, %19\n ds_read_b64_tr_b16 %13, %19 offset:2048\n"
          "ds_read_b64_tr_b16 %14, %19 offset:8192\n ds_read_b64_tr_b16 %15, %19 offset:10240\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(ra[0]), "=&v"(ra[1]), "=&v"(ra[2]), "=&v"(ra[3]), "=&v"(ra[4]), "=&v"(ra[5]), "=&v"(ra[6]),
            "=&v"(ra[7]), "=&v"(ra[8]), "=&v"(ra[9]), "=&v"(ra[10]), "=&v"(ra[11]), "=&v"(ra[12]), "=&v"(ra[13]),
            "=&v"(ra[14]), "=&v"(ra[15])
          : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
          : "memory");
      asm volatile(
          "ds_read_b64_tr_b16 %0, %8\n ds_read_b64_tr_b16 %1, %8 offset:2048\n"
          "ds_read_b64_tr_b16 %2, %8 offset:8192\n ds_read_b64_tr_b16 %3, %8 offset:10240\n"
          "ds_read_b64_tr_b16 %4, %9\n ds_read_b64_tr_b16 %5, %9 offset:2048\n"
          "ds_read_b64_tr_b16 %6, %9 offset:8192\n ds_read_b64_tr_b16 %7, %9 offset:10240\n"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(rb[0]), "=&v"(rb[1]), "=&v"(rb[2]), "=&v"(rb[3]), "=&v"(rb[4]), "=&v"(rb[5]), "=&v"(rb[6]),
            "=&v"(rb[7])
          : "v"(bd[0]), "v"(bd[1])
          : "memory");
      // ra[4 i + 2 kk + h]: fragment i, K group kk, half h (tokens 4h .. 4h+3),
      // 16-bit element e of a half in bits 16 e; fragments are bit copies
      if (valid < TK) {
        // tokens past the chunk: zero their act values (the last sub-tile only)
#pragma unroll
        for (int kk = 0; kk < TK / 16; ++kk)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u64 keep = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (kk * 16 + tok_recv + 4 * h + e < valid) keep |= 0xffffull << (16 * e);
#pragma unroll
            for (int i = 0; i < TMw; ++i) ra[4 * i + 2 * kk + h] &= keep;
          }
      }
      typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int kk = 0; kk < TK / 16; ++kk) {
#pragma unroll
        for (int i = 0; i < TMw; ++i)
          af[kk][i] = __builtin_bit_cast(bf16x8_t, u64x2{ra[4 * i + 2 * kk], ra[4 * i + 2 * kk + 1]});
#pragma unroll
        for (int j = 0; j < TNw; ++j)
          bfr[kk][j] = __builtin_bit_cast(bf16x8_t, u64x2{rb[4 * j + 2 * kk], rb[4 * j + 2 * kk + 1]});
      }
    }
#pragma unroll
    for (int kk = 0; kk < TK / 16; ++kk)
#pragma unroll
      for (int i = 0; i < TMw; ++i)
#pragma unroll
        for (int j = 0; j < TNw; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk][i], bfr[kk][j], acc[i][j], 0, 0, 0);
  }

  // partial for this split: rows a0 + i, columns d0 + c of the b x b block;
  // entries outside a short block are stored as zeros
  float* out = sd.part + (static_cast<int64_t>(split) * sd.nblk + blk) * g.b * g.b;
  const int lrow = lane & 31;
#pragma unroll
  for (int i = 0; i < TMw; ++i)
#pragma unroll
    for (int j = 0; j < TNw; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = a0 + rw0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = d0 + cw0 + j * 32 + lrow;
        out[static_cast<int64_t>(row) * g.b + col] = (row < width && col < width) ? acc[i][j][r] : 0.f;
      }
}

}  // namespace

// Splits of the token range for blocks of b over `dim` features (plus dim1
// more in the same launch): as many as fit one round of workgroups on the
// 256 CUs (one 128 KB-LDS workgroup per CU), so that no partial second round
// doubles the time; at least 8 sub-tiles of tokens per split.
int block_grad_splits(int64_t T, int64_t dim, int b, int64_t dim1) {
  if (b != 256 && b != 512) return 0;
  const int slices = b / S;
  const int64_t nblk = (dim + b - 1) / b + (dim1 + b - 1) / b;
  const int64_t units = nblk * slices * slices;
  int64_t ns = std::max<int64_t>(1, 256 / units);
  ns = std::max<int64_t>(1, std::min<int64_t>(ns, (T + 8 * TK - 1) / (8 * TK)));
  int64_t tpw = (T + ns - 1) / ns;
  tpw = (tpw + TK - 1) / TK * TK;
  return static_cast<int>(std::max<int64_t>(1, (T + tpw - 1) / tpw));
}

bool block_grad2_bf16(const uint16_t* act0, const uint16_t* dout0, float* part0, int64_t dim0,
                      const uint16_t* act1, const uint16_t* dout1, float* part1, int64_t dim1, int64_t T, int b,
                      int nsplit, hipStream_t s) {
  if (b != 256 && b != 512) return false;
  if (T <= 0 || nsplit <= 0) return true;
  GradArgs g;
  g.T = T;
  g.b = b;
  g.slices = b / S;
  int64_t tpw = (T + nsplit - 1) / nsplit;
  tpw = (tpw + TK - 1) / TK * TK;
  g.tokens_per_wg = static_cast<int>(tpw);
  g.nsplit = nsplit;
  const uint16_t* act[2] = {act0, act1};
  const uint16_t* dout[2] = {dout0, dout1};
  float* part[2] = {part0, part1};
  const int64_t dim[2] = {dim0, dim1};
  int wgs[2];
  for (int k = 0; k < 2; ++k) {
    g.side[k].act = reinterpret_cast<const bf16_t*>(act[k]);
    g.side[k].dout = reinterpret_cast<const bf16_t*>(dout[k]);
    g.side[k].part = part[k];
    g.side[k].dim = dim[k];
    g.side[k].nblk = act[k] ? static_cast<int>((dim[k] + b - 1) / b) : 0;
    wgs[k] = g.side[k].nblk * g.slices * g.slices * nsplit;
  }
  g.wgs0 = wgs[0];
  if (wgs[0] + wgs[1] > 0) hipLaunchKernelGGL(k_block_grad, dim3(static_cast<unsigned>(wgs[0] + wgs[1])), dim3(NT), 0, s, g);
  return true;
}

bool block_grad_bf16(const uint16_t* act, const uint16_t* dout, float* part, int64_t ld, int64_t T, int64_t dim,
                     int b, int nsplit, hipStream_t s) {
  if (ld != dim) return false;
  return block_grad2_bf16(act, dout, part, dim, nullptr, nullptr, nullptr, 0, T, b, nsplit, s);
}

}  // namespace poetx
