// Token reduction of the block gradients: for one 256-wide slice pair of a
// block and one chunk of tokens,
//   part[i][c] = sum_t act[t][a0 + i] * dout[t][d0 + c]      (i, c < 256)
// i.e. dG_j = X1_J^T dX2_J and dH_k = Y1_K^T dY2_K of the backward (W0 is
// frozen, so these b x b sums replace the T x m x n weight gradient; zhichai.net
// digest of arXiv:2603.05500, section "1. 输入中心化架构"). Blocks of 512
// columns are four slice pairs.
//
// gfx950 design: the contraction runs over tokens, so both operands must be
// token-contiguous for the MFMA fragments while the activations are stored
// token-major. Each thread loads an 8-token x 8-feature block (eight 16-byte
// row loads), transposes it in registers with v_perm_b32 and writes eight
// 16-byte feature rows into a swizzled feature-major LDS stage; fragment reads
// are then plain 16-byte LDS reads. 64-token sub-tiles, double-buffered, the
// next sub-tile's global loads in flight during the current MFMAs. Eight waves
// each hold a 128 x 64 region of the 256 x 256 fp32 partial in registers for
// the whole chunk; one store of the partial at the end.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace poetx {
namespace {

constexpr int S = 256;       // slice width
constexpr int TK = 64;       // tokens per sub-tile
constexpr int NT = 512;      // threads
constexpr int ROWB = TK * 2; // bytes per feature row of a stage (128)
constexpr int TILE = S * ROWB;  // one operand stage (32 KB)

// Slot of 16-byte chunk c in feature row r (128-byte rows): c ^ swz(r).
// Fragment reads touch 16 consecutive rows at one chunk: the bank group is
// 8 * (r % 2) + slot, and swz takes 8 distinct values on the even and on the
// odd rows of any aligned 16 (and on any aligned 8 rows). The transposed
// writes of one instruction touch rows 8 * fb + e: swz = e ^ (fb & 7) spreads
// them over all 8 slots of their parity.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 7); }

__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
  uint32_t iw[32];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    iw[r * 4 + 0] = in[r].x;
    iw[r * 4 + 1] = in[r].y;
    iw[r * 4 + 2] = in[r].z;
    iw[r * 4 + 3] = in[r].w;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int w = c >> 1;
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = __builtin_amdgcn_perm(iw[(2 * p + 1) * 4 + w], iw[(2 * p) * 4 + w], sel);
    out[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

struct GradArgs {
  const bf16_t* act;
  const bf16_t* dout;
  float* part;          // [nsplit][nblk][b][b]
  int64_t ld;           // row stride of act and dout (elements)
  int64_t dim;          // row width (short last block)
  int64_t T;
  int b;                // block size (256 or 512)
  int nblk;
  int slices;           // b / 256
  int tokens_per_wg;
  int nsplit;
};

__global__ void __launch_bounds__(NT) k_block_grad(const GradArgs g) {
  __shared__ __attribute__((aligned(1024))) char smem[2 * 2 * TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // workgroup -> (block, slice pair, split)
  const int pairs = g.slices * g.slices;
  int w = blockIdx.x;
  const int split = w % g.nsplit;
  w /= g.nsplit;
  const int pair = w % pairs;
  const int blk = w / pairs;
  const int si = pair / g.slices, sc = pair % g.slices;
  const int64_t blk0 = static_cast<int64_t>(blk) * g.b;
  const int width = static_cast<int>(min(static_cast<int64_t>(g.b), g.dim - blk0));
  const int a0 = si * S, d0 = sc * S;  // slice offsets inside the block
  const int64_t t_begin = static_cast<int64_t>(split) * g.tokens_per_wg;
  const int64_t t_end = min(g.T, t_begin + g.tokens_per_wg);
  const int nsub = t_end > t_begin ? static_cast<int>((t_end - t_begin + TK - 1) / TK) : 0;

  // staging: threads [0, 256) load act, [256, 512) load dout; each an 8x8 block
  const int op = tid >> 8;                       // 0 act, 1 dout
  const int q = tid & 255;
  const int fb = q & 31, tb = q >> 5;            // feature block (8 features), token block (8 tokens)
  const bf16_t* src = op == 0 ? g.act : g.dout;
  const int fcol = (op == 0 ? a0 : d0) + fb * 8; // feature offset in the block
  const bool fvalid = fcol < width;
  uint4 reg[8];
  auto gload = [&](int sub) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t t = t_begin + static_cast<int64_t>(sub) * TK + tb * 8 + e;
      if (fvalid && t < t_end)
        reg[e] = *reinterpret_cast<const uint4*>(src + t * g.ld + blk0 + fcol);
      else
        reg[e] = make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int stage) {
    uint4 tr[8];
    transpose8x8(reg, tr);
    char* base = smem + stage * 2 * TILE + op * TILE;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = fb * 8 + e;
      *reinterpret_cast<uint4*>(base + row * ROWB + ((tb ^ swz(row)) << 4)) = tr[e];
    }
  };

  // wave region: rows (wave % 2) * 128 .. + 128, columns (wave / 2) * 64 .. + 64
  constexpr int TMw = 4, TNw = 2;
  const int rw0 = (wave & 1) * 128, cw0 = (wave >> 1) * 64;
  const int lrow = lane & 31;
  // swz depends on row bits 0..5; wave regions start at multiples of 64, so a
  // fragment row is 32 * t + lrow with t the tile index and only t's parity matters
  const int sw0 = swz(lrow), sw1 = swz(32 + lrow);
  f32x16_t acc[TMw][TNw];
#pragma unroll
  for (int i = 0; i < TMw; ++i)
#pragma unroll
    for (int j = 0; j < TNw; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nsub > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (int s = 0; s < nsub; ++s) {
    if (s + 1 < nsub) gload(s + 1);
    const char* A = smem + (s & 1) * 2 * TILE;
    const char* B = A + TILE;
#pragma unroll
    for (int kk = 0; kk < TK / 16; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      const int off0 = lrow * ROWB + ((c ^ sw0) << 4), off1 = lrow * ROWB + ((c ^ sw1) << 4);
      bf16x8_t af[TMw], bfr[TNw];
#pragma unroll
      for (int i = 0; i < TMw; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(A + (rw0 + i * 32) * ROWB + ((i & 1) ? off1 : off0));
#pragma unroll
      for (int j = 0; j < TNw; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(B + (cw0 + j * 32) * ROWB + ((j & 1) ? off1 : off0));
#pragma unroll
      for (int i = 0; i < TMw; ++i)
#pragma unroll
        for (int j = 0; j < TNw; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nsub) lstore((s + 1) & 1);
    __syncthreads();
  }

  // partial for this split: rows a0 + i, columns d0 + c of the b x b block
  // (entries outside a short block are exact zeros: their loads were zero)
  float* out = g.part + (static_cast<int64_t>(split) * g.nblk + blk) * g.b * g.b;
#pragma unroll
  for (int i = 0; i < TMw; ++i)
#pragma unroll
    for (int j = 0; j < TNw; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = a0 + rw0 + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int col = d0 + cw0 + j * 32 + lrow;
        out[static_cast<int64_t>(row) * g.b + col] = acc[i][j][r];
      }
}

}  // namespace

// Splits of the token range: as many as fit one round of workgroups on the
// 256 CUs (one 128 KB-LDS workgroup per CU), so that no partial second round
// doubles the time; at least 4 sub-tiles of tokens per split.
int block_grad_splits(int64_t T, int64_t dim, int b) {
  if (b != 256 && b != 512) return 0;
  const int nblk = static_cast<int>((dim + b - 1) / b);
  const int slices = b / S;
  const int64_t units = static_cast<int64_t>(nblk) * slices * slices;
  int64_t ns = std::max<int64_t>(1, 256 / units);
  ns = std::max<int64_t>(1, std::min<int64_t>(ns, (T + 4 * TK - 1) / (4 * TK)));
  int64_t tpw = (T + ns - 1) / ns;
  tpw = (tpw + TK - 1) / TK * TK;
  return static_cast<int>(std::max<int64_t>(1, (T + tpw - 1) / tpw));
}

bool block_grad_bf16(const uint16_t* act, const uint16_t* dout, float* part, int64_t ld, int64_t T, int64_t dim,
                     int b, int nsplit, hipStream_t s) {
  if (b != 256 && b != 512) return false;
  if (T <= 0 || nsplit <= 0) return true;
  GradArgs g;
  g.act = act;
  g.dout = dout;
  g.part = part;
  g.ld = ld;
  g.dim = dim;
  g.T = T;
  g.b = b;
  g.nblk = static_cast<int>((dim + b - 1) / b);
  g.slices = b / S;
  int64_t tpw = (T + nsplit - 1) / nsplit;
  tpw = (tpw + TK - 1) / TK * TK;
  g.tokens_per_wg = static_cast<int>(tpw);
  g.nsplit = nsplit;
  const unsigned grid = static_cast<unsigned>(g.nblk * g.slices * g.slices * nsplit);
  hipLaunchKernelGGL(k_block_grad, dim3(grid), dim3(NT), 0, s, g);
  return true;
}

}  // namespace poetx
