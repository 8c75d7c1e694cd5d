// Bandwidth kernels around the matrix products: column permutations of
// row-major matrices (full rows staged in LDS, so both the HBM reads and the
// HBM writes are 16-byte coalesced and only the permuted accesses hit LDS),
// transposes, the element-wise steps of the Cayley-Neumann map and its
// adjoint, and fixed-order reductions of split-K partial sums.
#include "common.hpp"
#include "kernels.hpp"

namespace poetx {
namespace {

constexpr int kThreads = 256;
// Grid limits kept by every launch here: one-dimensional element-wise grids
// stop at kMaxGrid1 workgroups (2^28 threads, well inside the 2^32 work-items
// a dimension holds) and loop over the rest; y and z stop at the 65535 the
// runtime reports, with a loop where a size could exceed it.
constexpr int64_t kMaxGrid1 = int64_t(1) << 20;
constexpr int64_t kMaxGridYZ = 65535;
#ifndef POETX_GATHER_LDS_KB
#define POETX_GATHER_LDS_KB 32
#endif
constexpr int64_t kRowLdsBudget = POETX_GATHER_LDS_KB * 1024;  // bytes of rows staged per workgroup
constexpr int64_t kRowLdsMax = 64 * 1024;        // wider rows use the direct kernel

template <typename T> struct Pack8;
template <> struct Pack8<uint8_t> { typedef uint2 type; };
template <> struct Pack8<uint16_t> { typedef uint4 type; };

__device__ __forceinline__ uint2 pack8(const uint8_t (&v)[8]) {
  return make_uint2(v[0] | (v[1] << 8) | (v[2] << 16) | (static_cast<uint32_t>(v[3]) << 24),
                    v[4] | (v[5] << 8) | (v[6] << 16) | (static_cast<uint32_t>(v[7]) << 24));
}
__device__ __forceinline__ uint4 pack8(const uint16_t (&v)[8]) {
  return make_uint4(v[0] | (static_cast<uint32_t>(v[1]) << 16), v[2] | (static_cast<uint32_t>(v[3]) << 16),
                    v[4] | (static_cast<uint32_t>(v[5]) << 16), v[6] | (static_cast<uint32_t>(v[7]) << 16));
}

template <typename T>
__device__ __forceinline__ void store8(T* p, const T (&v)[8]) {
  if constexpr (sizeof(T) == 4) {
    reinterpret_cast<uint4*>(p)[0] = make_uint4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<uint4*>(p)[1] = make_uint4(v[4], v[5], v[6], v[7]);
  } else {
    *reinterpret_cast<typename Pack8<T>::type*>(p) = pack8(v);
  }
}

// Column gather with whole rows staged in LDS. Workgroup w handles rows
// [w*rows_per_wg, ...). Phase 1 copies those rows into LDS with 16-byte
// (8-byte for byte rows not a multiple of 16) loads; phase 2 writes 8 output
// elements per lane and row, reading the permuted sources from LDS.
template <typename T>
__global__ void __launch_bounds__(kThreads)
k_gather_cols_lds(const T* __restrict__ in, int64_t ld_in, const int32_t* __restrict__ rmap_in,
                  T* __restrict__ out, int64_t ld_out, const int32_t* __restrict__ rmap_out,
                  const int32_t* __restrict__ cidx, int ncols, int64_t nrows, int rows_per_wg, int chunk) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  T* lds = reinterpret_cast<T*>(lds_raw);
  const int64_t r0 = static_cast<int64_t>(blockIdx.x) * rows_per_wg;
  const int nr = static_cast<int>(min(static_cast<int64_t>(rows_per_wg), nrows - r0));
  const int64_t row_bytes = static_cast<int64_t>(ncols) * sizeof(T);
  const int cpr = static_cast<int>(row_bytes / chunk);
  for (int c = threadIdx.x; c < nr * cpr; c += kThreads) {
    const int rr = c / cpr, cc = c % cpr;
    const int64_t gr = r0 + rr;
    const int64_t src = rmap_in ? clamp_index(rmap_in[gr], nrows) : gr;
    const char* sp = reinterpret_cast<const char*>(in + src * ld_in) + static_cast<int64_t>(cc) * chunk;
    char* dp = lds_raw + rr * row_bytes + static_cast<int64_t>(cc) * chunk;
    if (chunk == 16)
      *reinterpret_cast<uint4*>(dp) = *reinterpret_cast<const uint4*>(sp);
    else
      *reinterpret_cast<uint2*>(dp) = *reinterpret_cast<const uint2*>(sp);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < ncols / 8; c += kThreads) {
    const int4 i0 = reinterpret_cast<const int4*>(cidx)[2 * c];
    const int4 i1 = reinterpret_cast<const int4*>(cidx)[2 * c + 1];
    const int idx[8] = {clamp_index(i0.x, ncols), clamp_index(i0.y, ncols), clamp_index(i0.z, ncols),
                        clamp_index(i0.w, ncols), clamp_index(i1.x, ncols), clamp_index(i1.y, ncols),
                        clamp_index(i1.z, ncols), clamp_index(i1.w, ncols)};
    for (int rr = 0; rr < nr; ++rr) {
      T v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = lds[static_cast<int64_t>(rr) * ncols + idx[e]];
      const int64_t gr = r0 + rr;
      const int64_t dst = rmap_out ? clamp_index(rmap_out[gr], nrows) : gr;
      store8(out + dst * ld_out + static_cast<int64_t>(c) * 8, v);
    }
  }
}

typedef __attribute__((address_space(3))) void* lds_void_t;

// s_waitcnt vmcnt(n) for a run-time n in [0, 63] (the counter's range on
// gfx950; larger n waits for all)
__device__ __forceinline__ void wait_vm63(int n) {
  switch (n) {
#define POETX_VM(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
#define POETX_VM8(k) POETX_VM(k) POETX_VM(k + 1) POETX_VM(k + 2) POETX_VM(k + 3) POETX_VM(k + 4) POETX_VM(k + 5) \
  POETX_VM(k + 6) POETX_VM(k + 7)
    POETX_VM8(1) POETX_VM8(9) POETX_VM8(17) POETX_VM8(25) POETX_VM8(33) POETX_VM8(41) POETX_VM8(49)
    POETX_VM(57) POETX_VM(58) POETX_VM(59) POETX_VM(60) POETX_VM(61) POETX_VM(62) POETX_VM(63)
#undef POETX_VM8
#undef POETX_VM
    default: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
  }
}

// Column gather, streaming version for rows of at most kPipeGroups * 8 * 256
// elements and a multiple of 16 bytes. Each workgroup walks rows
// blockIdx.x, blockIdx.x + gridDim.x, ... through a ring of `nbuf` LDS row
// buffers: rows are copied in with global_load_lds_dwordx4 nbuf - 1 rows
// ahead, and each row is gathered out of LDS and written with 16-byte stores.
// The threads' source indices sit in registers (16-bit), loaded once while
// the first row is already on its way.
//
// Loads and stores share the vector-memory counter, which retires in issue
// order, so the wait for row k counts what this wave issued after that row's
// loads: the loads of the rows still ahead of it and the stores of the rows
// before it. The host keeps that count within the counter's 63.
constexpr int kPipeGroups = 8;  // column groups of 8 per thread
constexpr int kPipeMaxBuf = 8;

template <typename T>
__global__ void __launch_bounds__(kThreads, 2)
k_gather_rows_pipe(const T* __restrict__ in, int64_t ld_in, const int32_t* __restrict__ rmap_in,
                   T* __restrict__ out, int64_t ld_out, const int32_t* __restrict__ rmap_out,
                   const int32_t* __restrict__ cidx, int ncols, int64_t nrows,
                   const int32_t* __restrict__ rmap_pre, const int32_t* __restrict__ cidx_pre, int nbuf,
                   const SideJob job) {
  extern __shared__ __attribute__((aligned(16))) char lds_raw[];
  // the side job's stores go out before every load the waits below count
  run_side_job(job);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row_bytes = ncols * static_cast<int>(sizeof(T));
  const int nchunk = row_bytes >> 4;
  const int ninst = (nchunk + 63) >> 6;  // 1 KB load instructions per row
  const int ngroups = ncols >> 3;
  // rows of this workgroup: blockIdx.x + k * gridDim.x for k < nrow
  const int64_t r0 = blockIdx.x;
  if (r0 >= nrows) return;
  const int nrow = static_cast<int>((nrows - 1 - r0) / gridDim.x + 1);

  auto issue = [&](int k) {
    const int64_t r = r0 + static_cast<int64_t>(k) * gridDim.x;
    const int64_t src = rmap_in ? clamp_index(rmap_in[rmap_pre ? clamp_index(rmap_pre[r], nrows) : r], nrows) : r;
    const char* sp = reinterpret_cast<const char*>(in + src * ld_in);
    char* buf = lds_raw + (k % nbuf) * row_bytes;
    for (int i = wave; i < ninst; i += kThreads / 64) {
      const int ch = i * 64 + lane;
      if (ch < nchunk)
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(sp + static_cast<int64_t>(ch) * 16),
                                         (lds_void_t)(buf + i * 1024), 16, 0, 0);
    }
  };
  issue(0);

  // every group's index loads go out before the first wait (groups past the
  // row's end load the last group again and are never used); with a composed
  // map, column i takes cidx[cidx_pre[i]]
  int4 iv[kPipeGroups][2];
  const int4* const first = reinterpret_cast<const int4*>(cidx_pre ? cidx_pre : cidx);
#pragma unroll
  for (int g = 0; g < kPipeGroups; ++g) {
    const int grp = min(tid + g * kThreads, ngroups - 1);
    iv[g][0] = first[2 * grp];
    iv[g][1] = first[2 * grp + 1];
  }
  if (cidx_pre) {
#pragma unroll
    for (int g = 0; g < kPipeGroups; ++g)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        iv[g][h] = make_int4(cidx[clamp_index(iv[g][h].x, ncols)], cidx[clamp_index(iv[g][h].y, ncols)],
                             cidx[clamp_index(iv[g][h].z, ncols)], cidx[clamp_index(iv[g][h].w, ncols)]);
  }
  uint32_t ix[kPipeGroups][4];
#pragma unroll
  for (int g = 0; g < kPipeGroups; ++g) {
    ix[g][0] = clamp_index(iv[g][0].x, ncols) | (clamp_index(iv[g][0].y, ncols) << 16);
    ix[g][1] = clamp_index(iv[g][0].z, ncols) | (clamp_index(iv[g][0].w, ncols) << 16);
    ix[g][2] = clamp_index(iv[g][1].x, ncols) | (clamp_index(iv[g][1].y, ncols) << 16);
    ix[g][3] = clamp_index(iv[g][1].z, ncols) | (clamp_index(iv[g][1].w, ncols) << 16);
  }
  // the rest of the ring's first fill, after the wait for the indices (which
  // also covers row 0), so that it overlaps the first rows' gathers
  for (int k = 1; k < nbuf - 1 && k < nrow; ++k) issue(k);
  // load and store instructions this wave issues per row
  int my_ld = 0, my_st = 0;
  for (int i = wave; i < ninst; i += kThreads / 64) ++my_ld;
#pragma unroll
  for (int g = 0; g < kPipeGroups; ++g) my_st += (wave * 64 + g * kThreads < ngroups) ? (sizeof(T) == 4 ? 2 : 1) : 0;

  for (int k = 0; k < nrow; ++k) {
    // issued after row k's loads: the loads of rows k+1 .. k+nbuf-2 and the
    // stores of rows k-nbuf+1 .. k-1 (those that exist)
    const int ld_after = min(nbuf - 2, nrow - 1 - k);
    const int st_after = min(nbuf - 1, k);
    wait_vm63(ld_after * my_ld + st_after * my_st);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    // the ring slot of row k - 1 is free: every wave has read it
    if (k + nbuf - 1 < nrow) issue(k + nbuf - 1);
    const T* L = reinterpret_cast<const T*>(lds_raw + (k % nbuf) * row_bytes);
    const int64_t r = r0 + static_cast<int64_t>(k) * gridDim.x;
    const int64_t dst = rmap_out ? clamp_index(rmap_out[r], nrows) : r;
    T* op = out + dst * ld_out;
    // all LDS reads of the row first (independent registers), then the stores
    uint32_t w[kPipeGroups][8];
#pragma unroll
    for (int g = 0; g < kPipeGroups; ++g) {
      if (tid + g * kThreads < ngroups) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[g][2 * e] = L[ix[g][e] & 0xffffu];
          w[g][2 * e + 1] = L[ix[g][e] >> 16];
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kPipeGroups; ++g) {
      const int grp = tid + g * kThreads;
      if (grp < ngroups) {
        T v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = static_cast<T>(w[g][e]);
        store8(op + static_cast<int64_t>(grp) * 8, v);
      }
    }
  }
}

// Fallback for rows wider than LDS: the gather reads global memory directly.
template <typename T>
__global__ void __launch_bounds__(kThreads)
k_gather_cols_direct(const T* __restrict__ in, int64_t ld_in, const int32_t* __restrict__ rmap_in,
                     T* __restrict__ out, int64_t ld_out, const int32_t* __restrict__ rmap_out,
                     const int32_t* __restrict__ cidx, int64_t ncols, int64_t nrows) {
  for (int64_t r = blockIdx.y; r < nrows; r += gridDim.y) {
    const int64_t src = rmap_in ? clamp_index(rmap_in[r], nrows) : r;
    const int64_t dst = rmap_out ? clamp_index(rmap_out[r], nrows) : r;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < ncols;
         i += static_cast<int64_t>(gridDim.x) * kThreads)
      out[dst * ld_out + i] = in[src * ld_in + clamp_index(cidx[i], ncols)];
  }
}

// i = this thread's first element; the loop steps by the whole grid
#define POETX_GRID_STRIDE(i, n)                                                          \
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < (n); \
       i += static_cast<int64_t>(gridDim.x) * kThreads)

__global__ void k_inverse_perm(const int32_t* __restrict__ perm, int32_t* __restrict__ inv, int64_t n) {
  POETX_GRID_STRIDE(i, n) inv[clamp_index(perm[i], n)] = static_cast<int32_t>(i);
}

__global__ void __launch_bounds__(kThreads) k_side_job(const SideJob job) { run_side_job(job); }

__global__ void k_compose_perm(const int32_t* __restrict__ inv0, const int32_t* __restrict__ next0,
                               int32_t* __restrict__ out0, int64_t n0, const int32_t* __restrict__ inv1,
                               const int32_t* __restrict__ next1, int32_t* __restrict__ out1, int64_t n1) {
  POETX_GRID_STRIDE(i, n0 + n1) {
    if (i < n0) out0[i] = inv0[clamp_index(next0[i], n0)];
    else out1[i - n0] = inv1[clamp_index(next1[i - n0], n1)];
  }
}

__global__ void k_gather_f32(const float* __restrict__ in, const int32_t* __restrict__ idx, float* __restrict__ out,
                             int64_t n) {
  POETX_GRID_STRIDE(i, n) out[i] = in[clamp_index(idx[i], n)];
}

// Transpose through a 64 x 64 LDS tile with 16-byte global accesses on both
// sides: each lane reads 16 bytes of an input row and writes 16 bytes of an
// output row (V = 16 / sizeof(T) elements). The LDS tile is padded by one
// element per row so that the column reads spread over the banks.
template <typename T>
__global__ void __launch_bounds__(kThreads) k_transpose(const T* __restrict__ in, T* __restrict__ out, int64_t rows,
                                                       int64_t cols) {
  constexpr int V = 16 / sizeof(T);
  constexpr int CPR = 64 / V;  // 16-byte chunks per 64-element row
  __shared__ T tile[64][64 + 1];
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 64;
  for (int64_t r0 = static_cast<int64_t>(blockIdx.y) * 64; r0 < rows; r0 += static_cast<int64_t>(gridDim.y) * 64) {
    const bool full = (r0 + 64 <= rows) && (c0 + 64 <= cols);
    for (int q = threadIdx.x; q < 64 * CPR; q += kThreads) {
      const int i = q / CPR, j = (q % CPR) * V;
      const int64_t r = r0 + i, c = c0 + j;
      T v[V];
      if (full) {
        const uint4 w = *reinterpret_cast<const uint4*>(in + r * cols + c);
        __builtin_memcpy(v, &w, 16);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) v[e] = (r < rows && c + e < cols) ? in[r * cols + c + e] : T(0);
      }
#pragma unroll
      for (int e = 0; e < V; ++e) tile[i][j + e] = v[e];
    }
    __syncthreads();
    for (int q = threadIdx.x; q < 64 * CPR; q += kThreads) {
      const int i = q / CPR, j = (q % CPR) * V;  // output row c0 + i, columns r0 + j ..
      const int64_t c = c0 + i, r = r0 + j;
      T v[V];
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] = tile[j + e][i];
      if (full) {
        uint4 w;
        __builtin_memcpy(&w, v, 16);
        *reinterpret_cast<uint4*>(out + c * rows + r) = w;
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (c < cols && r + e < rows) out[c * rows + r + e] = v[e];
      }
    }
    __syncthreads();  // the next tile row overwrites the tile
  }
}

__global__ void k_fill_zero(float* p, int64_t n) {
  POETX_GRID_STRIDE(i, n) p[i] = 0.f;
}

// two arrays in one launch: elements [0, n0) of p0, then [0, n1) of p1
__global__ void k_fill_zero2(float* p0, int64_t n0, float* p1, int64_t n1) {
  POETX_GRID_STRIDE(i, n0 + n1) {
    if (i < n0) p0[i] = 0.f;
    else p1[i - n0] = 0.f;
  }
}

// ---- quantized base weight around a merge ----------------------------------
// out[r][c] = value(wq[r][c]) * scale[cmap[c]] (cmap null: identity), the
// byte an int8 code or (fp8) an E4M3 code; 8 columns per thread: 8-byte
// loads, 32-byte stores.
__global__ void k_dequant_i8_cols(const int8_t* __restrict__ wq, const float* __restrict__ scale,
                                  const int32_t* __restrict__ cmap, float* __restrict__ out, int64_t rows,
                                  int64_t cols, int fp8) {
  const int64_t per_row = cols >> 3;
  POETX_GRID_STRIDE(g, rows * per_row) {  // g: 8-column group
    const int64_t r = g / per_row, c0 = (g % per_row) * 8;
    const uint2 q = *reinterpret_cast<const uint2*>(wq + r * cols + c0);
    const uint32_t w[2] = {q.x, q.y};
    float sc[8];
    if (cmap) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sc[e] = scale[clamp_index(cmap[c0 + e], cols)];
    } else {
      const float4 s0 = *reinterpret_cast<const float4*>(scale + c0);
      const float4 s1 = *reinterpret_cast<const float4*>(scale + c0 + 4);
      sc[0] = s0.x; sc[1] = s0.y; sc[2] = s0.z; sc[3] = s0.w;
      sc[4] = s1.x; sc[5] = s1.y; sc[6] = s1.z; sc[7] = s1.w;
    }
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t byte = (w[e >> 2] >> (8 * (e & 3))) & 0xffu;
      v[e] = (fp8 ? e4m3_to_f32(byte) : static_cast<float>(static_cast<int8_t>(byte))) * sc[e];
    }
    float4* o = reinterpret_cast<float4*>(out + r * cols + c0);
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// bfloat16 copy of int8 weight codes: every code (|c| <= 127) is exact in
// bfloat16. One thread per 8 codes: an 8-byte load, a 16-byte store.
__global__ void k_i8_to_bf16(const int8_t* __restrict__ in, uint16_t* __restrict__ out, int64_t n8) {
  POETX_GRID_STRIDE(i, n8) {
    const uint2 q = reinterpret_cast<const uint2*>(in)[i];
    const uint32_t w[2] = {q.x, q.y};
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float a = static_cast<float>(static_cast<int8_t>((w[h] >> (16 * e)) & 0xff));
        const float b = static_cast<float>(static_cast<int8_t>((w[h] >> (16 * e + 8)) & 0xff));
        o[2 * h + e] = (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
      }
    }
    reinterpret_cast<uint4*>(out)[i] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

__global__ void k_bf16_to_f32(const bf16_t* __restrict__ in, float* __restrict__ out, int64_t n) {
  POETX_GRID_STRIDE(i, n) out[i] = bf16_to_f32(in[i]);
}

// amax[c] = max over rows of |w[r][c]|: blockIdx.y takes a band of rows, one
// thread a column; the bands meet in an atomic max on the bit patterns (all
// values are non-negative, so their bits order like the floats). The result
// does not depend on the order.
__global__ void k_col_absmax(const float* __restrict__ w, int64_t rows, int64_t cols, int64_t band,
                             unsigned int* __restrict__ amax) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (c >= cols) return;
  float m = 0.f;
  for (int64_t r0 = static_cast<int64_t>(blockIdx.y) * band; r0 < rows; r0 += static_cast<int64_t>(gridDim.y) * band) {
    const int64_t r1 = r0 + band < rows ? r0 + band : rows;
    for (int64_t r = r0; r < r1; ++r) m = fmaxf(m, fabsf(w[r * cols + c]));
  }
  atomicMax(amax + c, __float_as_uint(m));
}

// Per-column storage. int8: scale[c] = amax[c] / 127 (1 for a zero column),
// wq = clamp(rint(w / scale), -127, 127), rint rounding half to even. fp8:
// scale[c] = amax[c] / 448 (1 for a zero column), wq = the E4M3 byte of
// w / scale. The division is the correctly rounded float32 one.
__global__ void k_quant_i8_cols(const float* __restrict__ w, const unsigned int* __restrict__ amax,
                                int8_t* __restrict__ wq, float* __restrict__ scale, int64_t rows, int64_t cols,
                                int fp8) {
  const int64_t per_row = cols >> 3;
  POETX_GRID_STRIDE(g, rows * per_row) {  // g: 8-column group
    const int64_t r = g / per_row, c0 = (g % per_row) * 8;
    uint32_t out[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t c = c0 + e;
      float sc = __uint_as_float(amax[c]) / (fp8 ? 448.f : 127.f);
      sc = sc > 0.f ? sc : 1.f;
      if (r == 0) scale[c] = sc;
      uint32_t byte;
      if (fp8) {
        byte = f32_to_e4m3(w[r * cols + c] / sc);
      } else {
        const float q = fminf(fmaxf(rintf(w[r * cols + c] / sc), -127.f), 127.f);
        byte = static_cast<uint32_t>(static_cast<int32_t>(q)) & 0xffu;
      }
      out[e >> 2] |= byte << (8 * (e & 3));
    }
    *reinterpret_cast<uint2*>(wq + r * cols + c0) = make_uint2(out[0], out[1]);
  }
}

// packed index of (i, l), i < l, in a block of size r
__device__ __forceinline__ int64_t tri_index(int i, int l, int r) {
  return static_cast<int64_t>(i) * r - static_cast<int64_t>(i) * (i + 1) / 2 + (l - i - 1);
}

// Blocks [0, seg.n0) come from side 0, the next seg.n1 from side 1 (R and P
// share one launch when their block sizes match).
struct Seg2 {
  const float* q0;
  const float* q1;
  int64_t dim0, dim1;
  int n0;
};

__device__ __forceinline__ void seg_pick(const Seg2& sg, int z, const float*& q, int64_t& dim, int& zl) {
  if (z < sg.n0) {
    q = sg.q0;
    dim = sg.dim0;
    zl = z;
  } else {
    q = sg.q1;
    dim = sg.dim1;
    zl = z - sg.n0;
  }
}

// One workgroup per 32 x 32 tile pair (I, L), I <= L, of block z: the packed
// entries of rows i in tile I and columns l in tile L (i < l) are contiguous
// runs of q, read coalesced; Q[i][l] = q and Q[l][i] = -q meet in LDS.
__global__ void __launch_bounds__(kThreads) k_unpack_skew(const Seg2 sg, int b, float* __restrict__ Qf,
                                                         uint16_t* __restrict__ Qh) {
  __shared__ float tile[32][33];
  const int z = blockIdx.z, I = blockIdx.y, Lt = blockIdx.x;
  if (I > Lt) return;
  const float* q;
  int64_t dim;
  int zl;
  seg_pick(sg, z, q, dim, zl);
  const int r = static_cast<int>(min(static_cast<int64_t>(b), dim - static_cast<int64_t>(zl) * b));
  const float* qz = q + static_cast<int64_t>(zl) * (static_cast<int64_t>(b) * (b - 1) / 2);
  const int64_t base = static_cast<int64_t>(z) * b * b;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int k = ty; k < 32; k += 8) {
    const int i = I * 32 + k, l = Lt * 32 + tx;
    float v = 0.f;
    if (i < l && l < r) v = qz[tri_index(i, l, r)];
    tile[k][tx] = v;
    if (i < b && l < b) {
      const int64_t o = base + static_cast<int64_t>(i) * b + l;
      if (I != Lt || i < l) {  // the rest of a diagonal tile is written below
        if (Qf) Qf[o] = v;
        if (Qh) Qh[o] = f32_to_bf16(v);
      }
    }
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int l = Lt * 32 + k, i = I * 32 + tx;  // Q[l][i] = -Q[i][l] for i < l
    if (i < b && l < b && (I != Lt || i <= l)) {
      const float v = (i == l) ? 0.f : -tile[tx][k];
      const int64_t o = base + static_cast<int64_t>(l) * b + i;
      if (Qf) Qf[o] = v;
      if (Qh) Qh[o] = f32_to_bf16(v);
    }
  }
}

// Same result for b a multiple of 64: one workgroup per 64 x 64 tile pair
// (I, L), I <= L, with the upper tile staged in LDS and both the tile and its
// mirror written with 16-byte stores; tile pairs with I > L are not launched.
__global__ void __launch_bounds__(kThreads) k_unpack_skew64(const Seg2 sg, int b, int tiles, float* __restrict__ Qf,
                                                           uint16_t* __restrict__ Qh) {
  __shared__ float tile[64][65];
  // blockIdx.x enumerates the pairs I <= L of one block row-major over I
  int p = blockIdx.x, I = 0;
  while (p >= tiles - I) {
    p -= tiles - I;
    ++I;
  }
  const int Lt = I + p;
  const int z = blockIdx.y;
  const float* q;
  int64_t dim;
  int zl;
  seg_pick(sg, z, q, dim, zl);
  const int r = static_cast<int>(min(static_cast<int64_t>(b), dim - static_cast<int64_t>(zl) * b));
  const float* qz = q + static_cast<int64_t>(zl) * (static_cast<int64_t>(b) * (b - 1) / 2);
  const int64_t base = static_cast<int64_t>(z) * b * b;
  const int tid = threadIdx.x;
  // U[a][c] = Q[I*64 + a][Lt*64 + c] for a row above the diagonal, else 0;
  // all 16 loads of a thread in flight together
  float u[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int i = I * 64 + (tid >> 6) + 4 * k, l = Lt * 64 + (tid & 63);
    u[k] = (i < l && l < r) ? qz[tri_index(i, l, r)] : 0.f;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) tile[(tid >> 6) + 4 * k][tid & 63] = u[k];
  __syncthreads();
  const bool diag = I == Lt;
  if (diag) {
    // complete the diagonal tile in LDS: lower half = -(upper half)^T
    // (reads only touch a < c, writes only a > c)
    float m[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int a = (tid >> 6) + 4 * k, c = tid & 63;
      m[k] = a > c ? -tile[c][a] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int a = (tid >> 6) + 4 * k, c = tid & 63;
      if (a > c) tile[a][c] = m[k];
    }
    __syncthreads();
  }
  // pass 0: tile (I, Lt) = LDS rows; pass 1 (off the diagonal): tile (Lt, I) = -LDS^T
  for (int pass = 0; pass < (diag ? 1 : 2); ++pass) {
    const int R0 = (pass == 0 ? I : Lt) * 64, C0 = (pass == 0 ? Lt : I) * 64;
    const float sg = pass == 0 ? 1.f : -1.f;
    if (Qh) {
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int ch = tid + it * kThreads;
        const int row = ch >> 3, c8 = (ch & 7) * 8;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = sg * (pass == 0 ? tile[row][c8 + e] : tile[c8 + e][row]);
        *reinterpret_cast<uint4*>(Qh + base + static_cast<int64_t>(R0 + row) * b + C0 + c8) =
            make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7]));
      }
    }
    if (Qf) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int ch = tid + it * kThreads;
        const int row = ch >> 4, c4 = (ch & 15) * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = sg * (pass == 0 ? tile[row][c4 + e] : tile[c4 + e][row]);
        *reinterpret_cast<float4*>(Qf + base + static_cast<int64_t>(R0 + row) * b + C0 + c4) =
            make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  }
}

__global__ void k_cnp_mid(const float* __restrict__ Qf, const float* __restrict__ Q2f, uint16_t* __restrict__ Sh,
                          float* __restrict__ Sf, int64_t n) {
  POETX_GRID_STRIDE(e, n) {
    const float s = 2.f * Qf[e] + Q2f[e];
    if (Sh) Sh[e] = f32_to_bf16(s);
    if (Sf) Sf[e] = s;
  }
}

template <typename TG>
__global__ void __launch_bounds__(kThreads) k_cnp_finish(const float* __restrict__ Qf, const float* __restrict__ Q2f,
                                                         const float* __restrict__ Tf, int b, int n0, int n1,
                                                         TG* __restrict__ g0, TG* __restrict__ g1) {
  __shared__ float tile[32][33];
  const int z = blockIdx.z;
  const int i0 = blockIdx.y * 32, l0 = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 8 rows of 32
  const int64_t bb = static_cast<int64_t>(b) * b;
  const int64_t src = static_cast<int64_t>(z) * bb;
  TG* g = z < n0 ? g0 : g1;
  const int nb = z < n0 ? n0 : n1;
  const int zl = z < n0 ? z : z - n0;
  TG* plane0 = g + static_cast<int64_t>(zl) * bb;
  TG* plane1 = g + static_cast<int64_t>(nb) * bb + static_cast<int64_t>(zl) * bb;
  for (int k = ty; k < 32; k += 8) {
    const int i = i0 + k, l = l0 + tx;
    if (i < b && l < b) {
      const int64_t o = src + static_cast<int64_t>(i) * b + l;
      const float v = 2.f * Qf[o] + 2.f * Q2f[o] + Tf[o];
      tile[k][tx] = v;
      store_from_f32(plane0 + static_cast<int64_t>(i) * b + l, v);
    }
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int l = l0 + k, i = i0 + tx;  // plane1[l][i] = (G - I)[i][l]
    if (i < b && l < b) store_from_f32(plane1 + static_cast<int64_t>(l) * b + i, tile[tx][k]);
  }
}

// dq for block z: dq[k(i,l)] = E[i][l] - E[l][i] for i < l < r. One
// workgroup per 32 x 32 tile (I, L), I <= L: the mirror tile (L, I) is read
// row-wise and transposed through LDS.
// Tile pair p of a t x t grid with I <= L, row-major over the upper triangle.
__device__ __forceinline__ void tile_pair(int p, int t, int& I, int& L) {
  int i = 0;
  while (p >= t - i) {
    p -= t - i;
    ++i;
  }
  I = i;
  L = i + p;
}

// dq[k(i, l)] = E[i][l] - E[l][i] for the i < l of a 64 x 64 tile pair (I, L):
// both tiles are read row-wise (256-byte rows), the mirror tile through LDS.
__global__ void __launch_bounds__(kThreads) k_pack_asym(const float* __restrict__ E, const Seg2 sg,
                                                       float* __restrict__ dq0, float* __restrict__ dq1, int b,
                                                       int t) {
  __shared__ float mir[64][65];
  const int z = blockIdx.y;
  int I, Lt;
  tile_pair(static_cast<int>(blockIdx.x), t, I, Lt);
  const float* q;
  int64_t dim;
  int zl;
  seg_pick(sg, z, q, dim, zl);
  float* dq = z < sg.n0 ? dq0 : dq1;
  const int r = static_cast<int>(min(static_cast<int64_t>(b), dim - static_cast<int64_t>(zl) * b));
  const int64_t base = static_cast<int64_t>(z) * b * b;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  // mirror tile (L, I): mir[l - 64 L][i - 64 I] = E[l][i]
#pragma unroll
  for (int k = ty; k < 64; k += 4) {
    const int l = Lt * 64 + k, i = I * 64 + tx;
    mir[k][tx] = (l < b && i < b) ? E[base + static_cast<int64_t>(l) * b + i] : 0.f;
  }
  __syncthreads();
  float* dqz = dq + static_cast<int64_t>(zl) * (static_cast<int64_t>(b) * (b - 1) / 2);
#pragma unroll
  for (int k = ty; k < 64; k += 4) {
    const int i = I * 64 + k, l = Lt * 64 + tx;
    if (i < l && l < r) dqz[tri_index(i, l, r)] = E[base + static_cast<int64_t>(i) * b + l] - mir[tx][k];
  }
}

// U = sum of the split partials (fixed order), written as its symmetric and
// skew parts Us = (U + U^T) / 2, Uk = (U - U^T) / 2 (float, and bfloat16
// copies when requested). One workgroup per tile pair (I, L), I <= L.
// Blocks [0, z_split) take their partials from side 0, the rest from side 1
// (each side has its own split count); the outputs of both sides are one
// array of blocks.
struct SymSkewIn {
  const float* part0;
  const float* part1;
  int64_t blocks_elems0, blocks_elems1;  // stride between splits
  int nsplit0, nsplit1;
  int z_split;
};

__global__ void __launch_bounds__(kThreads) k_reduce_symskew(const SymSkewIn in, int b, float* __restrict__ Us,
                                                            float* __restrict__ Uk, uint16_t* __restrict__ Ush,
                                                            uint16_t* __restrict__ Ukh) {
  __shared__ float ta[32][33];
  __shared__ float tb[32][33];
  const int z = blockIdx.y;
  const bool hi = z >= in.z_split;
  const float* __restrict__ part = hi ? in.part1 : in.part0;
  const int nsplit = hi ? in.nsplit1 : in.nsplit0;
  const int64_t blocks_elems = hi ? in.blocks_elems1 : in.blocks_elems0;
  int I, Lt;
  tile_pair(static_cast<int>(blockIdx.x), (b + 31) / 32, I, Lt);
  const int64_t base_in = static_cast<int64_t>(hi ? z - in.z_split : z) * b * b;  // within the side's partials
  const int64_t base = static_cast<int64_t>(z) * b * b;                          // in the outputs
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  // each thread sums 4 rows of tile (I, L) and 4 of tile (L, I) over the
  // splits, in split order; a group of 4 splits puts all 32 loads in flight
  int64_t oa[4], om[4];
  bool va[4], vm[4];
  float a[4], m[4];
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) {
    const int k = ty + 8 * k4;
    const int i = I * 32 + k, l = Lt * 32 + tx;    // tile (I, L) row-wise
    const int l2 = Lt * 32 + k, i2 = I * 32 + tx;  // tile (L, I) row-wise
    va[k4] = i < b && l < b;
    vm[k4] = l2 < b && i2 < b;
    oa[k4] = va[k4] ? base_in + static_cast<int64_t>(i) * b + l : base_in;
    om[k4] = vm[k4] ? base_in + static_cast<int64_t>(l2) * b + i2 : base_in;
    a[k4] = 0.f;
    m[k4] = 0.f;
  }
  for (int sp = 0; sp < nsplit; sp += 4) {
    float xa[4][4], xm[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* pp = part + static_cast<int64_t>(min(sp + u, nsplit - 1)) * blocks_elems;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        xa[u][k4] = pp[oa[k4]];
        xm[u][k4] = pp[om[k4]];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (sp + u < nsplit) {
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4) {
          a[k4] += xa[u][k4];
          m[k4] += xm[u][k4];
        }
      }
    }
  }
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) {
    ta[ty + 8 * k4][tx] = va[k4] ? a[k4] : 0.f;  // U[i][l]
    tb[ty + 8 * k4][tx] = vm[k4] ? m[k4] : 0.f;  // U[l2][i2]
  }
  __syncthreads();
  // tile (I, L): U[i][l] and U[l][i] = tb[l - L*32][i - I*32]
  for (int k = ty; k < 32; k += 8) {
    const int i = I * 32 + k, l = Lt * 32 + tx;
    if (i < b && l < b) {
      const float u = ta[k][tx], ut = tb[tx][k];
      const int64_t o = base + static_cast<int64_t>(i) * b + l;
      Us[o] = 0.5f * (u + ut);
      Uk[o] = 0.5f * (u - ut);
      if (Ush) Ush[o] = f32_to_bf16(0.5f * (u + ut));
      if (Ukh) Ukh[o] = f32_to_bf16(0.5f * (u - ut));
    }
    const int l2 = Lt * 32 + k, i2 = I * 32 + tx;
    if (I != Lt && l2 < b && i2 < b) {
      const float u = tb[k][tx], ut = ta[tx][k];
      const int64_t o = base + static_cast<int64_t>(l2) * b + i2;
      Us[o] = 0.5f * (u + ut);
      Uk[o] = 0.5f * (u - ut);
      if (Ush) Ush[o] = f32_to_bf16(0.5f * (u + ut));
      if (Ukh) Ukh[o] = f32_to_bf16(0.5f * (u - ut));
    }
  }
}

// H1 = 4 Uk - 2 (P1 - P1^T): tile pairs (I, L), I <= L, through LDS.
__global__ void __launch_bounds__(kThreads) k_cnp_h1(const float* __restrict__ Uk, const float* __restrict__ P1, int b,
                                                    float* __restrict__ Hf, uint16_t* __restrict__ Hh) {
  __shared__ float ta[32][33];
  __shared__ float tb[32][33];
  const int z = blockIdx.y;
  int I, Lt;
  tile_pair(static_cast<int>(blockIdx.x), (b + 31) / 32, I, Lt);
  const int64_t base = static_cast<int64_t>(z) * b * b;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int k = ty; k < 32; k += 8) {
    const int i = I * 32 + k, l = Lt * 32 + tx;
    const int l2 = Lt * 32 + k, i2 = I * 32 + tx;
    ta[k][tx] = (i < b && l < b) ? P1[base + static_cast<int64_t>(i) * b + l] : 0.f;
    tb[k][tx] = (l2 < b && i2 < b) ? P1[base + static_cast<int64_t>(l2) * b + i2] : 0.f;
  }
  __syncthreads();
  for (int k = ty; k < 32; k += 8) {
    const int i = I * 32 + k, l = Lt * 32 + tx;
    if (i < b && l < b) {
      const int64_t o = base + static_cast<int64_t>(i) * b + l;
      const float v = 4.f * Uk[o] - 2.f * (ta[k][tx] - tb[tx][k]);
      if (Hf) Hf[o] = v;
      if (Hh) Hh[o] = f32_to_bf16(v);
    }
    const int l2 = Lt * 32 + k, i2 = I * 32 + tx;
    if (I != Lt && l2 < b && i2 < b) {
      const int64_t o = base + static_cast<int64_t>(l2) * b + i2;
      const float v = 4.f * Uk[o] - 2.f * (tb[k][tx] - ta[tx][k]);
      if (Hf) Hf[o] = v;
      if (Hh) Hh[o] = f32_to_bf16(v);
    }
  }
}

inline unsigned grid1(int64_t n) { return static_cast<unsigned>(std::min<int64_t>((n + kThreads - 1) / kThreads, kMaxGrid1)); }
inline unsigned grid_yz(int64_t n) { return static_cast<unsigned>(std::min<int64_t>(n, kMaxGridYZ)); }

template <typename T>
bool pipe_applies(int64_t ncols) {
  const int64_t row_bytes = ncols * static_cast<int64_t>(sizeof(T));
  return row_bytes % 16 == 0 && ncols <= kPipeGroups * 8 * kThreads && 2 * row_bytes <= 128 * 1024;
}

#ifndef POETX_PIPE_LDS_KB
#define POETX_PIPE_LDS_KB 96
#endif

// Workgroups per CU and ring depth of k_gather_rows_pipe. Rows of at most
// 8 KB: four workgroups per CU, each with a ring of up to 32 KB (four 8 KB
// rows). Wider rows: the most row bytes in flight per CU (per_cu * (nbuf - 1)
// rows) within POETX_PIPE_LDS_KB of LDS per CU, one or two workgroups; but
// with at most 16 rows per CU, two workgroups of two buffers each. The wait
// count of the kernel's deepest wave stays within the counter's 63. At the
// 8B MLP widths: 8 KB rows four workgroups with four buffers (the m-wide
// token gather 0.039 -> 0.034 ms against two with six; more in flight per
// workgroup, e.g. a full 160 KB ring, measured slower); 28 KB rows over 8192
// tokens one workgroup with three buffers; the 4096 rows of 28 KB of the
// weight reframe two with two (0.069 -> 0.065 ms).
template <typename T>
void pipe_shape(int64_t ncols, int64_t nrows, int* per_cu, int* nbuf) {
  const int64_t row_bytes = ncols * static_cast<int64_t>(sizeof(T));
  const int64_t ninst = (row_bytes / 16 + 63) / 64;
  const int64_t ld = (ninst + kThreads / 64 - 1) / (kThreads / 64);
  const int64_t st = ((ncols / 8 + kThreads - 1) / kThreads) * (sizeof(T) == 4 ? 2 : 1);
  auto fit = [&](int d) {
    while (d > 2 && (d - 2) * ld + (d - 1) * st > 63) --d;
    return d;
  };
  if (row_bytes > 8192 && nrows <= 16 * 256 && 4 * row_bytes <= 160 * 1024) {
    *per_cu = 2;
    *nbuf = fit(2);
    return;
  }
  if (row_bytes <= 8192) {
    *per_cu = 4;
    *nbuf = fit(static_cast<int>(std::min<int64_t>(kPipeMaxBuf, 32768 / row_bytes)));
    return;
  }
  int64_t best = -1;
  for (int pc = 1; pc <= 2; ++pc) {
    const int d = fit(static_cast<int>(std::min<int64_t>(kPipeMaxBuf, POETX_PIPE_LDS_KB * 1024 / (pc * row_bytes))));
    if (d < 2) continue;
    const int64_t inflight = pc * (d - 1) * row_bytes;
    if (inflight >= best) {
      best = inflight;
      *per_cu = pc;
      *nbuf = d;
    }
  }
}

template <typename T>
void launch_gather(const void* in, int64_t ld_in, const int32_t* rmap_in, void* out, int64_t ld_out,
                   const int32_t* rmap_out, const int32_t* cidx, int64_t ncols, int64_t nrows, hipStream_t s,
                   const int32_t* rmap_pre = nullptr, const int32_t* cidx_pre = nullptr,
                   const SideJob& job = SideJob()) {
  const int64_t row_bytes = ncols * static_cast<int64_t>(sizeof(T));
  if (pipe_applies<T>(ncols)) {
    int per_cu = 1, nbuf = 2;
    pipe_shape<T>(ncols, nrows, &per_cu, &nbuf);
    const unsigned nwg = static_cast<unsigned>(std::min<int64_t>(nrows, 256 * per_cu));
    hipLaunchKernelGGL(k_gather_rows_pipe<T>, dim3(nwg), dim3(kThreads), static_cast<size_t>(nbuf * row_bytes), s,
                       static_cast<const T*>(in), ld_in, rmap_in, static_cast<T*>(out), ld_out, rmap_out, cidx,
                       static_cast<int>(ncols), nrows, rmap_pre, cidx_pre, nbuf, job);
    return;
  }
  if (!job.empty()) side_job(job, s);
  if (row_bytes <= kRowLdsMax) {
    int rows = static_cast<int>(kRowLdsBudget / row_bytes);
    rows = rows < 1 ? 1 : (rows > 16 ? 16 : rows);
    const int chunk = (row_bytes % 16 == 0) ? 16 : 8;
    const unsigned nwg = static_cast<unsigned>((nrows + rows - 1) / rows);
    hipLaunchKernelGGL(k_gather_cols_lds<T>, dim3(nwg), dim3(kThreads), static_cast<size_t>(rows * row_bytes), s,
                       static_cast<const T*>(in), ld_in, rmap_in, static_cast<T*>(out), ld_out, rmap_out, cidx,
                       static_cast<int>(ncols), nrows, rows, chunk);
  } else {
    const unsigned gx = static_cast<unsigned>(std::min<int64_t>((ncols + kThreads - 1) / kThreads, 1024));
    hipLaunchKernelGGL(k_gather_cols_direct<T>, dim3(gx, grid_yz(nrows)), dim3(kThreads), 0, s,
                       static_cast<const T*>(in), ld_in, rmap_in, static_cast<T*>(out), ld_out, rmap_out, cidx,
                       ncols, nrows);
  }
}

}  // namespace

bool gather_cols(const void* in, int64_t ld_in, const int32_t* rmap_in, void* out, int64_t ld_out,
                 const int32_t* rmap_out, const int32_t* cidx, int64_t ncols, int64_t nrows, int esize,
                 hipStream_t s) {
  if (nrows <= 0 || ncols <= 0) return true;
  if (ncols % 8 != 0) return false;
  switch (esize) {
    case 1: launch_gather<uint8_t>(in, ld_in, rmap_in, out, ld_out, rmap_out, cidx, ncols, nrows, s); return true;
    case 2: launch_gather<uint16_t>(in, ld_in, rmap_in, out, ld_out, rmap_out, cidx, ncols, nrows, s); return true;
    case 4: launch_gather<uint32_t>(in, ld_in, rmap_in, out, ld_out, rmap_out, cidx, ncols, nrows, s); return true;
    default: return false;
  }
}

void inverse_perm(const int32_t* perm, int32_t* inv, int64_t n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_inverse_perm, dim3(grid1(n)), dim3(kThreads), 0, s, perm, inv, n);
}

void side_job(const SideJob& job, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(job.n0) + job.n1 + job.nz0 + job.nz1;
  if (total > 0) hipLaunchKernelGGL(k_side_job, dim3(grid1(total)), dim3(kThreads), 0, s, job);
}

bool reframe_rows_cols(const void* in, const int32_t* inv_r, const int32_t* next_r, void* out,
                       const int32_t* inv_c, const int32_t* next_c, int32_t* rmap, int32_t* cmap, int64_t ncols,
                       int64_t nrows, int esize, hipStream_t s, const SideJob& job) {
  if (ncols % 8 != 0 || (esize != 1 && esize != 2 && esize != 4)) return false;
  if (nrows <= 0 || ncols <= 0) {
    side_job(job, s);
    return true;
  }
  const bool pipe = esize == 2 ? pipe_applies<uint16_t>(ncols)
                               : (esize == 4 ? pipe_applies<uint32_t>(ncols) : pipe_applies<uint8_t>(ncols));
  if (pipe) {
    switch (esize) {
      case 1: launch_gather<uint8_t>(in, ncols, inv_r, out, ncols, nullptr, inv_c, ncols, nrows, s, next_r, next_c, job); return true;
      case 2: launch_gather<uint16_t>(in, ncols, inv_r, out, ncols, nullptr, inv_c, ncols, nrows, s, next_r, next_c, job); return true;
      default: launch_gather<uint32_t>(in, ncols, inv_r, out, ncols, nullptr, inv_c, ncols, nrows, s, next_r, next_c, job); return true;
    }
  }
  side_job(job, s);
  compose_perm(inv_r, next_r, rmap, nrows, inv_c, next_c, cmap, ncols, s);
  return gather_cols(in, ncols, rmap, out, ncols, nullptr, cmap, ncols, nrows, esize, s);
}

void compose_perm(const int32_t* inv0, const int32_t* next0, int32_t* out0, int64_t n0, const int32_t* inv1,
                  const int32_t* next1, int32_t* out1, int64_t n1, hipStream_t s) {
  if (n0 + n1 > 0)
    hipLaunchKernelGGL(k_compose_perm, dim3(grid1(n0 + n1)), dim3(kThreads), 0, s, inv0, next0, out0, n0, inv1, next1,
                       out1, n1);
}

void gather_f32(const float* in, const int32_t* idx, float* out, int64_t n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_gather_f32, dim3(grid1(n)), dim3(kThreads), 0, s, in, idx, out, n);
}

bool dequant_i8_cols(const int8_t* wq, const float* scale, const int32_t* cmap, float* out, int64_t rows,
                     int64_t cols, hipStream_t s, bool fp8) {
  if (rows <= 0 || cols <= 0) return true;
  if (cols % 8 != 0) return false;
  hipLaunchKernelGGL(k_dequant_i8_cols, dim3(grid1(rows * (cols / 8))), dim3(kThreads), 0, s, wq, scale, cmap, out,
                     rows, cols, fp8 ? 1 : 0);
  return true;
}

bool i8_to_bf16(const int8_t* in, uint16_t* out, int64_t n, hipStream_t s) {
  if (n % 8 != 0) return false;
  const int64_t n8 = n / 8;
  if (n8 > 0) hipLaunchKernelGGL(k_i8_to_bf16, dim3(grid1(n8)), dim3(kThreads), 0, s, in, out, n8);
  return true;
}

void bf16_to_f32(const uint16_t* in, float* out, int64_t n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_bf16_to_f32, dim3(grid1(n)), dim3(kThreads), 0, s, in, out, n);
}

bool requant_i8_cols(const float* w, unsigned int* amax, int8_t* wq, float* scale, int64_t rows, int64_t cols,
                     hipStream_t s, bool fp8) {
  if (rows <= 0 || cols <= 0) return true;
  if (cols % 8 != 0) return false;
  fill_zero_f32(reinterpret_cast<float*>(amax), cols, s);  // bit pattern 0 = +0.0
  const int64_t band = 64;
  const dim3 g(static_cast<unsigned>((cols + kThreads - 1) / kThreads), grid_yz((rows + band - 1) / band));
  hipLaunchKernelGGL(k_col_absmax, g, dim3(kThreads), 0, s, w, rows, cols, band, amax);
  hipLaunchKernelGGL(k_quant_i8_cols, dim3(grid1(rows * (cols / 8))), dim3(kThreads), 0, s, w, amax, wq, scale,
                     rows, cols, fp8 ? 1 : 0);
  return true;
}

bool transpose(const void* in, void* out, int64_t rows, int64_t cols, int esize, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return true;
  const dim3 g(static_cast<unsigned>((cols + 63) / 64), grid_yz((rows + 63) / 64));
  switch (esize) {
    case 1: hipLaunchKernelGGL(k_transpose<uint8_t>, g, dim3(kThreads), 0, s, static_cast<const uint8_t*>(in),
                               static_cast<uint8_t*>(out), rows, cols); return true;
    case 2: hipLaunchKernelGGL(k_transpose<uint16_t>, g, dim3(kThreads), 0, s, static_cast<const uint16_t*>(in),
                               static_cast<uint16_t*>(out), rows, cols); return true;
    case 4: hipLaunchKernelGGL(k_transpose<uint32_t>, g, dim3(kThreads), 0, s, static_cast<const uint32_t*>(in),
                               static_cast<uint32_t*>(out), rows, cols); return true;
    default: return false;
  }
}

void fill_zero_f32(float* p, int64_t n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_fill_zero, dim3(grid1(n)), dim3(kThreads), 0, s, p, n);
}

void fill_zero2_f32(float* p0, int64_t n0, float* p1, int64_t n1, hipStream_t s) {
  if (n0 + n1 > 0) hipLaunchKernelGGL(k_fill_zero2, dim3(grid1(n0 + n1)), dim3(kThreads), 0, s, p0, n0, p1, n1);
}

void unpack_skew2(const float* q0, int64_t dim0, int n0, const float* q1, int64_t dim1, int n1, int b, float* Qf,
                  uint16_t* Qh, hipStream_t s) {
  const Seg2 sg{q0, q1, dim0, dim1, n0};
  if (b % 64 == 0) {
    const int t = b / 64;
    hipLaunchKernelGGL(k_unpack_skew64, dim3(static_cast<unsigned>(t * (t + 1) / 2), static_cast<unsigned>(n0 + n1)),
                       dim3(kThreads), 0, s, sg, b, t, Qf, Qh);
    return;
  }
  const unsigned t = static_cast<unsigned>((b + 31) / 32);
  hipLaunchKernelGGL(k_unpack_skew, dim3(t, t, static_cast<unsigned>(n0 + n1)), dim3(kThreads), 0, s, sg, b, Qf, Qh);
}

void cnp_mid(const float* Qf, const float* Q2f, uint16_t* Sh, float* Sf, int64_t n, hipStream_t s) {
  hipLaunchKernelGGL(k_cnp_mid, dim3(grid1(n)), dim3(kThreads), 0, s, Qf, Q2f, Sh, Sf, n);
}

void cnp_finish2(const float* Qf, const float* Q2f, const float* Tf, int b, int n0, void* g0, int n1, void* g1,
                 bool bf16, hipStream_t s) {
  const unsigned t = static_cast<unsigned>((b + 31) / 32);
  const dim3 g(t, t, static_cast<unsigned>(n0 + n1));
  if (bf16)
    hipLaunchKernelGGL(k_cnp_finish<uint16_t>, g, dim3(kThreads), 0, s, Qf, Q2f, Tf, b, n0, n1,
                       static_cast<uint16_t*>(g0), static_cast<uint16_t*>(g1));
  else
    hipLaunchKernelGGL(k_cnp_finish<float>, g, dim3(kThreads), 0, s, Qf, Q2f, Tf, b, n0, n1,
                       static_cast<float*>(g0), static_cast<float*>(g1));
}

void pack_asym2(const float* E, int b, int64_t dim0, int n0, float* dq0, int64_t dim1, int n1, float* dq1,
                hipStream_t s) {
  const Seg2 sg{nullptr, nullptr, dim0, dim1, n0};
  const int t = (b + 63) / 64;
  hipLaunchKernelGGL(k_pack_asym, dim3(static_cast<unsigned>(t * (t + 1) / 2), static_cast<unsigned>(n0 + n1)),
                     dim3(kThreads), 0, s, E, sg, dq0, dq1, b, t);
}

void reduce_symskew2(const float* part0, int nsplit0, int nblk0, const float* part1, int nsplit1, int nblk1, int b,
                     float* Us, float* Uk, uint16_t* Ush, uint16_t* Ukh, hipStream_t s) {
  if (nblk0 + nblk1 <= 0) return;
  const unsigned t = static_cast<unsigned>((b + 31) / 32);
  const int64_t bb = static_cast<int64_t>(b) * b;
  const SymSkewIn in{part0, part1, nblk0 * bb, nblk1 * bb, nsplit0, nsplit1, nblk0};
  hipLaunchKernelGGL(k_reduce_symskew, dim3(t * (t + 1) / 2, static_cast<unsigned>(nblk0 + nblk1)), dim3(kThreads),
                     0, s, in, b, Us, Uk, Ush, Ukh);
}

void cnp_h1(const float* Uk, const float* P1, int b, int nblk, float* Hf, uint16_t* Hh, hipStream_t s) {
  const unsigned t = static_cast<unsigned>((b + 31) / 32);
  hipLaunchKernelGGL(k_cnp_h1, dim3(t * (t + 1) / 2, static_cast<unsigned>(nblk)), dim3(kThreads), 0, s, Uk, P1, b,
                     Hf, Hh);
}

}  // namespace poetx
