// Seeded permutation draws for Psi and Phi.
//
// The permutations of R = Psi^T Diag(G) Psi and P = Phi^T Diag(H) Phi are
// random (zhichai.net digest of arXiv:2603.05500, section "2. 块随机正交变换")
// and are drawn again whenever a merge restarts the rotations (section
// "代码与部署"). A draw takes word i mod 4 of the Philox4x64-10 block at
// counter (i div 4, draw, 0, 0) under key (seed, tag) (Salmon, Moraes, Dror
// and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), keeps its
// top 44 bits as index i's key, and lists the indices in ascending order of
// (key, index).
//
// With dim <= 2^20 the pair packs into one word, key * 2^20 + i, and these
// words are distinct; index i's rank is the number of smaller words, and
// perm[rank_i] = i writes every entry exactly once.
//
// Layer widths (dim <= kLdsPermMax) take one workgroup that keeps every word
// in LDS: a histogram of the words' top 10 bits, its exclusive scan, a
// scatter of the indices into their buckets, and each index ranked as its
// bucket's start plus the number of smaller words in its bucket (about
// dim / 1024 of them). The keys are uniform, so the work grows as dim; one
// CU does it, leaving the others to whatever else runs. Slot order inside a
// bucket depends on the order of the LDS atomics, but a rank does not.
//
// Wider draws: k_perm_keys writes the words once; k_perm_rank ranks index i
// by counting the smaller words with wave-uniform (scalar) loads of the
// words, one 64-bit compare per pair (dim^2 in all).

#include "kernels.hpp"

namespace poetx {
namespace {

constexpr uint64_t kPhiloxMul0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxMul1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxWeyl0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxWeyl1 = 0xBB67AE8584CAA73Bull;

// Philox4x64-10 in place on the counter c under key (k0, k1): each round
// takes the 128-bit products of words 0 and 2 with the round multipliers and
// forms (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key gains the Weyl
// increments before every round after the first.
__device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kPhiloxWeyl0;
      k1 += kPhiloxWeyl1;
    }
    const uint64_t lo0 = kPhiloxMul0 * c[0], hi0 = __umul64hi(kPhiloxMul0, c[0]);
    const uint64_t lo1 = kPhiloxMul1 * c[2], hi1 = __umul64hi(kPhiloxMul1, c[2]);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

constexpr int kKeyShift = 20;     // index bits of a packed key (dim <= 2^20)
constexpr int kRankWaves = 16;    // waves of one workgroup splitting the comparisons
constexpr int kRankUnroll = 32;   // words per scalar-load batch (64 SGPRs)

// comp[i] = (top 44 bits of index i's word) * 2^20 + i; one Philox block
// (four indices) per thread.
__global__ __launch_bounds__(256) void k_perm_keys(int n, uint64_t seed, uint64_t tag, uint64_t draw,
                                                   uint64_t* __restrict__ comp) {
  const int blk = blockIdx.x * 256 + threadIdx.x;
  const int i0 = 4 * blk;
  if (i0 >= n) return;
  uint64_t c[4] = {static_cast<uint64_t>(blk), draw, 0, 0};
  philox4x64_10(c, seed, tag);
  constexpr uint64_t kKeyMask = ~((uint64_t(1) << kKeyShift) - 1);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    if (i0 + k < n) comp[i0 + k] = (c[k] & kKeyMask) | static_cast<uint64_t>(i0 + k);
}

// One workgroup ranks 64 indices (one per lane); its waves split [0, n) into
// kRankWaves ranges and each counts, for every lane, the words of its range
// below the lane's word. The range bounds are wave-uniform, so the words
// arrive through scalar loads and every lane compares against the same one.
__global__ __launch_bounds__(64 * kRankWaves) void k_perm_rank(const uint64_t* __restrict__ comp, int n,
                                                               int32_t* __restrict__ perm) {
  __shared__ int part[kRankWaves][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int i = blockIdx.x * 64 + lane;
  const uint64_t ci = comp[min(i, n - 1)];
  // scalar loads complete out of order, so a wave cannot overlap its next
  // batch with the current one; other waves on the SIMD hide the latency
  const int q = ((n + kRankWaves - 1) / kRankWaves + kRankUnroll - 1) / kRankUnroll * kRankUnroll;
  const int a = min(w * q, n), e = min(a + q, n);
  int cnt = 0;
  int j = a;
  for (; j + kRankUnroll <= e; j += kRankUnroll) {
#pragma unroll
    for (int t = 0; t < kRankUnroll; ++t) cnt += comp[j + t] < ci;
  }
  for (; j < e; ++j) cnt += comp[j] < ci;
  part[w][lane] = cnt;
  __syncthreads();
  if (w == 0 && i < n) {
    int r = 0;
#pragma unroll
    for (int k = 0; k < kRankWaves; ++k) r += part[k][lane];
    perm[r] = i;
  }
}

constexpr int kLdsBuckets = 1024;  // top 10 bits of a word
constexpr int kLdsThreads = 1024;

// Block-wide exclusive scan of kLdsBuckets counters in LDS (one per thread).
__device__ __forceinline__ void scan_exclusive(uint32_t* cnt, uint32_t* wave_sum) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const uint32_t v = cnt[t];
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_sum[w] = x;
  __syncthreads();
  if (w == 0) {
    uint32_t s = lane < kLdsThreads / 64 ? wave_sum[lane] : 0u;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < kLdsThreads / 64) wave_sum[lane] = s;  // inclusive over waves
  }
  __syncthreads();
  cnt[t] = x - v + (w ? wave_sum[w - 1] : 0u);
  __syncthreads();
}

// The whole draw in one workgroup (dim <= kLdsPermMax): the words, the
// indices in bucket order, the bucket counters and the scan's wave sums all
// sit in LDS (157 KB at the largest dim).
__global__ __launch_bounds__(kLdsThreads) void k_perm_lds(int n, uint64_t seed, uint64_t tag, uint64_t draw,
                                                          int32_t* __restrict__ perm) {
  __shared__ uint64_t words[kLdsPermMax];
  __shared__ uint16_t idx[kLdsPermMax];
  __shared__ uint32_t cnt[kLdsBuckets];
  __shared__ uint32_t wave_sum[kLdsThreads / 64];
  const int t = threadIdx.x;
  constexpr int kShift = 64 - 10;
  cnt[t] = 0;
  __syncthreads();
  // words and the histogram of their top 10 bits
  constexpr uint64_t kKeyMask = ~((uint64_t(1) << kKeyShift) - 1);
  for (int blk = t; 4 * blk < n; blk += kLdsThreads) {
    uint64_t c[4] = {static_cast<uint64_t>(blk), draw, 0, 0};
    philox4x64_10(c, seed, tag);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * blk + k;
      if (i < n) {
        const uint64_t w = (c[k] & kKeyMask) | static_cast<uint64_t>(i);
        words[i] = w;
        atomicAdd(&cnt[w >> kShift], 1u);
      }
    }
  }
  __syncthreads();
  scan_exclusive(cnt, wave_sum);  // cnt[b] = first slot of bucket b
  // indices into their buckets; afterwards cnt[b] = end of bucket b
  for (int i = t; i < n; i += kLdsThreads) {
    const uint32_t slot = atomicAdd(&cnt[words[i] >> kShift], 1u);
    idx[slot] = static_cast<uint16_t>(i);
  }
  __syncthreads();
  for (int i = t; i < n; i += kLdsThreads) {
    const uint64_t w = words[i];
    const uint32_t b = static_cast<uint32_t>(w >> kShift);
    const uint32_t lo = b ? cnt[b - 1] : 0u, hi = cnt[b];
    uint32_t r = lo;
    for (uint32_t s = lo; s < hi; ++s) r += words[idx[s]] < w;
    perm[r] = i;
  }
}

}  // namespace

bool sample_perm(int64_t n, uint64_t seed, uint64_t tag, uint64_t draw, int32_t* perm, uint64_t* keys,
                 hipStream_t stream) {
  if (n < 1 || n > kMaxPermDim) return false;
  if (n <= kLdsPermMax) {
    hipLaunchKernelGGL(k_perm_lds, dim3(1), dim3(kLdsThreads), 0, stream, static_cast<int>(n), seed,
                       tag, draw, perm);
    return true;
  }
  const int nb = static_cast<int>((n + 3) / 4);
  k_perm_keys<<<(nb + 255) / 256, 256, 0, stream>>>(static_cast<int>(n), seed, tag, draw, keys);
  k_perm_rank<<<static_cast<int>((n + 63) / 64), 64 * kRankWaves, 0, stream>>>(keys, static_cast<int>(n), perm);
  return true;
}

}  // namespace poetx
