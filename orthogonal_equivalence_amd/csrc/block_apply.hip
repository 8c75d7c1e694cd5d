// Streaming block-diagonal product on token-major bfloat16 activations:
//   out[t, J_j] = (in[t, J_j] + in[t, J_j] B_j^T) * s[J_j]     (s optional)
// where B_j is one b x b plane of a CNP block buffer ((G-I)^T for the forward
// apply in G, (G-I) for the backward apply in G^T). It is the layer's
// "X1 Diag(G)" / "dY2 Diag(H)^T" step (zhichai.net digest of arXiv:2603.05500,
// section "2. 块随机正交变换"), an HBM-bound pass (b/2 flops per byte).
//
// gfx950 design: one workgroup owns one block and a contiguous run of
// tokens. Each of its b/32 waves keeps its 32 output columns of B_j resident
// in registers as MFMA fragments for the whole run, so B_j is read once per
// workgroup (in whole rows through LDS before the first sub-tile). A 512 x
// 512 plane would fill a CU's whole register file, so for b = 512 two
// workgroups share a block and a token run, each owning 256 of its output
// columns (8 waves of 128 fragment registers) and staging the full
// 512-column input; the two are issued 8 workgroups apart so that they land
// on the same XCD and the second read of the input hits its L2. 32-token
// sub-tiles stream global -> LDS with global_load_lds_dwordx4 into two
// swizzled stages (the next sub-tile is in flight while the current one is
// multiplied); v_mfma_f32_32x32x16_bf16 does the product; a per-wave LDS
// slab turns the accumulator into rows, where the residual (from the staged
// input) is added and 16-byte stores go out.
#include "common.hpp"
#include "kernels.hpp"

#include <algorithm>

namespace poetx {
namespace {

typedef __attribute__((address_space(3))) void* lds_void_t;

constexpr int TT = 32;  // tokens per sub-tile

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void lds_barrier() {
  // LDS-only barrier: the direct loads in flight are waited for by count
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int B>
__device__ __forceinline__ int swz_row(int r) {
  // rows of >= 256 bytes: 16-byte slot bank group = slot % 16, spread by r;
  // 128-byte rows: bank group = 8 * (r % 2) + slot, spread by r / 2
  if constexpr (B >= 128) return r & 15;
  else return (r >> 1) & 7;
}

// Per wave, the MFMA fragments frag[kk] (lane: row 32 wave + lane % 32 of a
// row-major plane of b-element rows, elements 16 kk + 8 (lane / 32) .. +7),
// for NW waves. Loaded straight into registers, each load instruction would
// touch 32 rows for 32 bytes each, so every cache line would reach the CU
// about four times. Instead the rows go through LDS whole: buffer j of
// NBUF holds one wave's 32 rows (chunk c of row r in slot c ^ swz_row(r),
// 1 KB direct loads shared by all waves), NBUF of them in flight, and each
// wave reads its own fragments out of its buffer. Ends with the buffers free.
template <int b, int NW, int NBUF>
__device__ __forceinline__ void stage_frags(const bf16_t* __restrict__ rows, char* lds, int wave, int lane,
                                            bf16x8_t (&frag)[b / 16]) {
  constexpr int ROWB = 2 * b, CPR = ROWB / 16, BUF = 32 * ROWB, LPW = BUF / 1024 / NW;
  static_assert(LPW * NW * 1024 == BUF && NBUF >= 2 && NBUF <= 4 && NBUF <= NW, "fragment staging");
  auto issue = [&](int w, int buf) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int q = (wave * LPW + i) * 64 + lane;
      const int row = q / CPR, slot = q % CPR;
      const int c = slot ^ swz_row<b>(row);
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(rows + static_cast<int64_t>(w * 32 + row) * b + c * 8),
                                       (lds_void_t)(lds + buf * BUF + (wave * LPW + i) * 1024), 16, 0, 0);
    }
  };
  const int r = lane & 31, sw = swz_row<b>(r);
#pragma unroll
  for (int w = 0; w < NBUF; ++w) issue(w, w);
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    // rounds w+1 .. min(w + NBUF, NW) - 1 may still be in flight
    const int younger = (w + NBUF - 1 < NW - 1 ? w + NBUF - 1 : NW - 1) - w;
    if (younger >= 3) wait_vmcnt<3 * LPW>();
    else if (younger == 2) wait_vmcnt<2 * LPW>();
    else if (younger == 1) wait_vmcnt<LPW>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (wave == w) {
      const char* st = lds + (w % NBUF) * BUF;
#pragma unroll
      for (int kk = 0; kk < b / 16; ++kk) {
        const int c = 2 * kk + (lane >> 5);
        frag[kk] = *reinterpret_cast<const bf16x8_t*>(st + r * ROWB + ((c ^ sw) << 4));
      }
    }
    if (w + NBUF < NW) {
      lds_barrier();  // every wave is past its reads of this buffer
      issue(w + NBUF, w % NBUF);
    }
  }
  lds_barrier();
}


// workgroups of 8 waves and b <= 256: two per CU, 4 waves per SIMD; b = 512:
// one per CU (its fragments take 128 registers per lane), 2 waves per SIMD
template <int B>
__global__ void __launch_bounds__(64 * ((B > 256 ? 256 : B) / 32), (B > 256 ? 2 : (B >= 256 ? 4 : 2)))
k_block_apply(const bf16_t* __restrict__ in, bf16_t* __restrict__ out, int64_t ld, const bf16_t* __restrict__ plane,
              const float* __restrict__ scale, int64_t T, int64_t dim, int tokens_per_wg, int wgs_per_block,
              int npairs, const SideJob job) {
  constexpr int NH = B > 256 ? 2 : 1;  // workgroups sharing a block (column halves)
  constexpr int NW = B / NH / 32;      // waves, 32 output columns each
  constexpr int ROWB = B * 2;
  constexpr int CPR = ROWB / 16;
  constexpr int STAGE = TT * ROWB;
  constexpr int LPW = STAGE / 1024 / NW;  // 1 KB direct loads per wave and stage
  constexpr int KS = B / 16;
  constexpr int SLAB = 32 * 33 * 4;  // per wave: 32 rows x 32 fp32 columns (+1 pad)
  constexpr int NSTG = 2;  // stages
  constexpr int SMEM = NSTG * STAGE + NW * SLAB;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  run_side_job(job);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  int blk, part, cofs = 0;  // cofs: first output column of this workgroup within the block
  if constexpr (NH == 2) {
    // in each run of 16 workgroups, the first 8 take half 0 of 8 (block,
    // token run) pairs and the next 8 take half 1 of the same pairs
    const int idx = static_cast<int>(blockIdx.x);
    const int pair = ((idx >> 4) << 3) | (idx & 7);
    if (pair >= npairs) return;
    blk = pair / wgs_per_block;
    part = pair % wgs_per_block;
    cofs = ((idx >> 3) & 1) * (B / NH);
  } else {
    blk = blockIdx.x / wgs_per_block;
    part = blockIdx.x % wgs_per_block;
  }
  const int64_t col0 = static_cast<int64_t>(blk) * B;
  const int width = static_cast<int>(min(static_cast<int64_t>(B), dim - col0));  // short last block
  const int cmax = width / 8 - 1;                                                  // last valid chunk
  const int64_t t_begin = static_cast<int64_t>(part) * tokens_per_wg;
  const int64_t t_end = min(T, t_begin + tokens_per_wg);
  if (t_begin >= t_end) return;
  const int nsub = static_cast<int>((t_end - t_begin + TT - 1) / TT);

  // direct loads: each wave fills LPW x 1 KB of a stage
  auto issue = [&](int sub, int stage) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int q = (wave * LPW + i) * 64 + lane;
      const int row = q / CPR, slot = q % CPR;
      int c = slot ^ swz_row<B>(row);
      c = c < cmax ? c : cmax;
      int64_t t = t_begin + static_cast<int64_t>(sub) * TT + row;
      t = t < t_end ? t : t_end - 1;
      const bf16_t* src = in + t * ld + col0 + c * 8;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src),
                                       (lds_void_t)(smem + stage * STAGE + (wave * LPW + i) * 1024), 16, 0, 0);
    }
  };

  const int arow = lane & 31, lcol = lane & 31;
  const int asw = swz_row<B>(arow);

  // this wave's 32 columns of B_j as MFMA B-operand fragments (lane: column
  // cofs + 32 wave + lane % 32, k's 16 kk + 8 (lane / 32) .. +7): rows of the
  // plane, staged through the stage and slab space
  constexpr int NBUF = SMEM / STAGE < NW ? SMEM / STAGE : NW;
  static_assert(NBUF * STAGE <= SMEM, "fragment staging buffers");
  bf16x8_t gfrag[KS];
  stage_frags<B, NW, (NBUF < 4 ? NBUF : 4)>(plane + (static_cast<int64_t>(blk) * B + cofs) * B, smem, wave, lane, gfrag);

  float* slab = reinterpret_cast<float*>(smem + NSTG * STAGE + wave * SLAB);
  // sub-tile s's product into acc: the MFMA chain over the stage st
  auto product = [&](const char* st, f32x16_t& acc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int c = 2 * kk + (lane >> 5);
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(st + arow * ROWB + ((c ^ asw) << 4));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gfrag[kk], acc, 0, 0, 0);
    }
  };
  // accumulator -> this wave's fp32 slab (32 rows x 32 columns)
  auto to_slab = [&](const f32x16_t& acc) {
#pragma unroll
    for (int r = 0; r < 16; ++r) slab[((r >> 2) * 8 + (lane >> 5) * 4 + (r & 3)) * 33 + lcol] = acc[r];
  };
  // half i of sub-tile s from the slab: per lane 8 consecutive columns of a
  // row, + residual from the staged input st, * column scale, bfloat16, one
  // 16-byte store
  auto store_half = [&](int i, int s, const char* st) {
    const int q = lane + i * 64;
    const int row = q >> 2, c4 = q & 3;
    const int64_t t = t_begin + static_cast<int64_t>(s) * TT + row;
    const int col = cofs + wave * 32 + c4 * 8;
    const int chunk = col >> 3;
    // the residual, read by inline asm that waits for its own result: as an
    // ordinary LDS load it gets a wait for every direct load in flight, the
    // next stage's included
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 xr;
    const uint32_t xa = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>(st + row * ROWB + ((chunk ^ swz_row<B>(row)) << 4)));
    asm volatile("ds_read_b128 %0, %1\n s_waitcnt lgkmcnt(0)" : "=v"(xr) : "v"(xa) : "memory");
    const uint32_t xw[4] = {xr.x, xr.y, xr.z, xr.w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = slab[row * 33 + c4 * 8 + 2 * e] + __uint_as_float(xw[e] << 16);
      v[2 * e + 1] = slab[row * 33 + c4 * 8 + 2 * e + 1] + __uint_as_float(xw[e] & 0xffff0000u);
    }
    if (scale) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] *= scale[col0 + (col < width ? col : 0) + e];
    }
    if (t < t_end && col < width)
      *reinterpret_cast<uint4*>(out + t * ld + col0 + col) =
          make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                     pack_bf16x2(v[6], v[7]));
  };
  auto epilogue = [&](const f32x16_t& acc, int s, const char* st) {
    to_slab(acc);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    store_half(0, s, st);
    store_half(1, s, st);
  };

  issue(0, 0);
  for (int s = 0; s < nsub; ++s) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (s + 1 < nsub) issue(s + 1, (s + 1) & 1);
    const char* st = smem + (s & 1) * STAGE;
    f32x16_t acc;
    product(st, acc);
    epilogue(acc, s, st);
  }
}

// Left block product on a row-major matrix: out[J][c] = in[J][c] + sum_k
// plane[J][i][k] in[J k][c] for the b = 256 row blocks J, i.e. Diag(G) W with
// plane = G - I row-major (the merge's left factor on the rows of W directly).
// Each wave keeps rows 32w .. 32w+31 of its block's plane as MFMA A fragments
// for a whole run of columns; 256-row x 64-column tiles (128-byte row
// segments, whole cache lines) go global -> LDS (global_load_lds_dwordx4, two
// stages), and the B fragments (8 consecutive rows of one column per lane)
// come from ds_read_b64_tr_b16 on the row-major tile: within each group of 16
// lanes, lane j receives element (j % 4) of the 8 bytes addressed by lane
// 4e + j / 4 (e = 0..3), so with lane i addressing row r0 + i / 4 at column
// c0 + 4 (i % 4), lane j gets rows r0 .. r0+3 of column c0 + j. Chunk c of
// tile row r sits in slot c ^ 4 ((r / 2) % 2): the 8 rows one read touches
// (r0 .. r0+3 and r0+8 .. r0+11) then cover each bank twice, the minimum for
// 512 bytes. The epilogue goes through a per-wave float slab of 16 rows x 32
// columns (8-column groups swizzled by row), which keeps a workgroup at
// 80 KB of LDS, two per CU.
__device__ __forceinline__ int left_slot(int r, int c) { return c ^ (((r >> 1) & 1) << 2); }

__global__ void __launch_bounds__(512, 4)
k_block_apply_left(const bf16_t* __restrict__ in, bf16_t* __restrict__ out, int64_t ld,
                   const bf16_t* __restrict__ plane, int64_t rows, int64_t ncols, int cols_per_wg, int wgs_per_block,
                   const SideJob job) {
  constexpr int B = 256, TC = 64, ROWB = TC * 2, STAGE = B * ROWB, KS = B / 16;
  constexpr int SLAB = 16 * 32;  // floats per wave
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE + 8 * SLAB * 4];
  run_side_job(job);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  // the workgroups of one block run on one XCD (one L2 holds its plane)
  const int pid = xcd_remap(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int blk = pid / wgs_per_block;
  const int part = pid % wgs_per_block;
  const int64_t row0 = static_cast<int64_t>(blk) * B;
  const int height = static_cast<int>(min(static_cast<int64_t>(B), rows - row0));  // short last block
  const int64_t c_begin = static_cast<int64_t>(part) * cols_per_wg;
  const int64_t c_end = min(ncols, c_begin + cols_per_wg);
  if (c_begin >= c_end) return;
  const int nsub = static_cast<int>((c_end - c_begin + TC - 1) / TC);

  // A fragments: rows 32w + (l % 32) of the plane, 8 k's at 16 kk + 8 (l / 32),
  // staged through the stage and slab space
  const int lrow = lane & 31;
  static_assert(4 * 32 * B * 2 <= 2 * STAGE + 8 * SLAB * 4, "fragment staging buffers");
  bf16x8_t afrag[KS];
  stage_frags<B, 8, 4>(plane + static_cast<int64_t>(blk) * B * B, smem, wave, lane, afrag);

  // loads: 32 instructions of 8 rows x 128 bytes per stage, four per wave;
  // lane l lands in slot l % 8 of row 8 q + l / 8 and fetches the chunk that
  // belongs there. Rows past a short block re-read its last row, columns past
  // the end its last 8 columns (neither reaches a stored output).
  auto issue = [&](int sub, int stage) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = wave * 4 + u;
      const int r = q * 8 + (lane >> 3);
      const int ch = left_slot(r, lane & 7);
      int64_t c = c_begin + static_cast<int64_t>(sub) * TC + ch * 8;
      c = c < ncols - 8 ? c : ncols - 8;
      const int rr = r < height ? r : height - 1;
      const bf16_t* src = in + (row0 + rr) * ld + c;
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(src),
                                       (lds_void_t)(smem + stage * STAGE + q * 1024), 16, 0, 0);
    }
  };

  // transposed-read address of this lane for K rows kb = 0 and column tile ct:
  // row 8 (G / 2) + i / 4, column 32 ct + 16 (G % 2) + 4 (i % 4). Rows +4
  // (second half of a fragment) and +16 (next K group) keep the row's slot
  // pattern, so they are immediate offsets of 512 and 2048 bytes.
  const int grp = lane >> 4, li = lane & 15;
  const int rd_row = 8 * (grp >> 1) + (li >> 2), rd_col = 16 * (grp & 1) + 4 * (li & 3);
  uint32_t rd_off[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int col = ct * 32 + rd_col;
    rd_off[ct] = static_cast<uint32_t>(rd_row * ROWB + (left_slot(rd_row, col >> 3) << 4) + (col & 7) * 2);
  }
  float* slab = reinterpret_cast<float*>(smem + 2 * STAGE) + wave * SLAB;
  typedef unsigned long long u64;
  typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

  issue(0, 0);
  for (int s = 0; s < nsub; ++s) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (s + 1 < nsub) issue(s + 1, (s + 1) & 1);
    const char* st = smem + (s & 1) * STAGE;
    const uint32_t sbase = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(st));
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x16_t acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
      // 32 transposed reads (16 K groups x 2 halves) in eight self-waiting
      // asm blocks of 2 K groups
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        u64 t[4];
        const uint32_t bh = sbase + rd_off[ct] + h * 2 * 2048;
        asm volatile(
            "ds_read_b64_tr_b16 %0, %4\n ds_read_b64_tr_b16 %1, %4 offset:512\n"
            "ds_read_b64_tr_b16 %2, %4 offset:2048\n ds_read_b64_tr_b16 %3, %4 offset:2560\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3])
            : "v"(bh)
            : "memory");
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              afrag[2 * h + k2], __builtin_bit_cast(bf16x8_t, u64x2{t[2 * k2], t[2 * k2 + 1]}), acc, 0, 0, 0);
      }
      // per half of the wave's 32 rows: accumulators -> slab (16 rows x 32
      // columns), then per lane 8 consecutive columns of a row: + residual
      // from the staged tile, one 16-byte store
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int r = 8 * hh; r < 8 * hh + 8; ++r) {
          const int row = (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3) - 16 * hh;
          slab[row * 32 + ((((lrow >> 3) ^ ((row >> 1) & 3))) << 3) + (lrow & 7)] = acc[r];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int row = lane >> 2, c4 = lane & 3;  // row within the half, 8-column chunk
        const int grow = wave * 32 + 16 * hh + row;
        const int64_t c = c_begin + static_cast<int64_t>(s) * TC + ct * 32 + c4 * 8;
        const uint4 xr = *reinterpret_cast<const uint4*>(st + grow * ROWB + (left_slot(grow, ct * 4 + c4) << 4));
        const float* sp = slab + row * 32 + ((c4 ^ ((row >> 1) & 3)) << 3);
        const float4 a0 = *reinterpret_cast<const float4*>(sp);
        const float4 a1 = *reinterpret_cast<const float4*>(sp + 4);
        const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const uint32_t xw[4] = {xr.x, xr.y, xr.z, xr.w};
        float v[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[2 * e] = av[2 * e] + __uint_as_float(xw[e] << 16);
          v[2 * e + 1] = av[2 * e + 1] + __uint_as_float(xw[e] & 0xffff0000u);
        }
        if (grow < height && c < c_end)
          *reinterpret_cast<uint4*>(out + (row0 + grow) * ld + c) =
              make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                         pack_bf16x2(v[6], v[7]));
        // every lane's slab reads are complete before the next tile's writes
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
    }
  }
}

}  // namespace

bool block_apply_left_bf16(const uint16_t* in, uint16_t* out, int64_t ld, const uint16_t* plane, int64_t rows,
                           int64_t ncols, int b, hipStream_t s, const SideJob& job) {
  if (rows <= 0 || ncols <= 0) return job.empty();  // (no launch to carry the side job)
  if (b != 256 || ncols % 8 != 0 || ncols < 8) return false;
  const int nblk = static_cast<int>((rows + b - 1) / b);
  // two 512-thread workgroups per CU (LDS) -> 512 resident
  int64_t wpb = std::max<int64_t>(1, 512 / nblk);
  int64_t cpw = (ncols + wpb - 1) / wpb;
  cpw = (cpw + 63) / 64 * 64;
  wpb = (ncols + cpw - 1) / cpw;
  hipLaunchKernelGGL(k_block_apply_left, dim3(static_cast<unsigned>(nblk * wpb)), dim3(512), 0, s,
                     reinterpret_cast<const bf16_t*>(in), reinterpret_cast<bf16_t*>(out), ld,
                     reinterpret_cast<const bf16_t*>(plane), rows, ncols, static_cast<int>(cpw),
                     static_cast<int>(wpb), job);
  return true;
}

bool block_apply_bf16(const uint16_t* in, uint16_t* out, int64_t ld, const uint16_t* plane, const float* scale,
                      int64_t T, int64_t dim, int b, hipStream_t s, const SideJob& job) {
  if (T <= 0) return job.empty();  // (no launch to carry the side job)
  if (b != 64 && b != 128 && b != 256 && b != 512) return false;
  const int nblk = static_cast<int>((dim + b - 1) / b);
  const int nh = b == 512 ? 2 : 1;  // workgroups per block and token run
  // Workgroups resident at once on the 256 CUs: b = 512 takes a CU alone
  // (8 waves of up to 256 registers), b = 256 is limited to two per CU by
  // registers (8 waves of up to 128 VGPRs), b = 128 to four (registers and
  // LDS), b = 64 to nine by LDS (eight used). Every workgroup streams the
  // same number of tokens, and one more than fits would cost a whole second
  // round: floor(resident / (blocks x nh)) token runs per block.
  const int64_t resident = 256 * (b == 512 ? 1 : (b == 256 ? 2 : (b == 128 ? 4 : 8)));
  int64_t wpb = std::max<int64_t>(1, resident / (static_cast<int64_t>(nblk) * nh));
  int64_t tpw = (T + wpb - 1) / wpb;
  tpw = (tpw + TT - 1) / TT * TT;
  wpb = (T + tpw - 1) / tpw;
  const int64_t npairs = nblk * wpb;
  const int itpw = static_cast<int>(tpw), iwpb = static_cast<int>(wpb), inp = static_cast<int>(npairs);
  switch (b) {
    case 64:
      hipLaunchKernelGGL(k_block_apply<64>, dim3(static_cast<unsigned>(npairs)), dim3(128), 0, s, in, out, ld, plane,
                         scale, T, dim, itpw, iwpb, inp, job);
      break;
    case 128:
      hipLaunchKernelGGL(k_block_apply<128>, dim3(static_cast<unsigned>(npairs)), dim3(256), 0, s, in, out, ld, plane,
                         scale, T, dim, itpw, iwpb, inp, job);
      break;
    case 256:
      hipLaunchKernelGGL(k_block_apply<256>, dim3(static_cast<unsigned>(npairs)), dim3(512), 0, s, in, out, ld, plane,
                         scale, T, dim, itpw, iwpb, inp, job);
      break;
    default:
      // both halves of every pair, in runs of 16 workgroups (8 pairs each)
      hipLaunchKernelGGL(k_block_apply<512>, dim3(static_cast<unsigned>((npairs + 7) / 8 * 16)), dim3(512), 0, s, in,
                         out, ld, plane, scale, T, dim, itpw, iwpb, inp, job);
      break;
  }
  return true;
}

}  // namespace poetx
