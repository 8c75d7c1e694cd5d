// C ABI of libpoetx.so (include/poetx.h): argument validation, workspace
// layout and the kernel sequence of each entry point.
//
// Data flow (row form Z = X R W0 P, R = Psi^T Diag(G) Psi, P = Phi^T Diag(H)
// Phi; zhichai.net digest of arXiv:2603.05500, sections "1. 输入中心化架构" and
// "2. 块随机正交变换"). Activations stay token-major; everything between the
// boundary tensors lives in the permuted frames, where every diagonal block is
// a contiguous run of b columns:
//   forward   X1 = X[:, perm_r]            column gather (saved)
//             X2 = X1 + X1 (G - I)         batched block product, MFMA
//             Y1 = X2 Wp, Wp = Psi W0 Phi^T dense product, MFMA (saved)
//             Y2 = Y1 + Y1 (H - I)         batched block product
//             Z  = Y2 scattered by perm_p  column gather with perm_p^-1
//   backward  dY2 = dZ[:, perm_p]; dY1 = dY2 H^T; dH = sum_t Y1^T dY2
//             dX2 = dY1 Wp^T; dX1 = dX2 G^T; dG = sum_t X1^T dX2
//             dX = dX1 scattered by perm_r; dq = skew-packed CNP adjoint of dG, dH
// Because Wp already carries both permutations, the two dense products need
// no gather at all. Wp is the only copy of the base weight the library keeps:
// the forward reads it N-contiguous, the backward K-contiguous, and a merge
// writes the merged weight straight into the frame of the next permutations.
// W0 in the original frame exists only on request (poetx_weight_export).
#include "../../include/poetx.h"
#include "common.hpp"
#include "gemm.hpp"
#include "kernels.hpp"

#include <algorithm>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

using namespace poetx;

namespace {

struct Side {
  int64_t dim;
  int b;
  int nblk;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// every pointer non-null and 16-byte aligned
bool ptrs_ok(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p || !aligned16(p)) return false;
  return true;
}

// Size limits. Tokens: every token count the kernels form (T rounded up to a
// tile, a split's share) stays an int. Blocks: the CNP launches put the
// blocks of both sides in one grid dimension, whose reported limit is 65535.
constexpr int64_t kMaxTokens = int64_t(1) << 30;
constexpr int64_t kMaxFeatures = int64_t(1) << 24;
constexpr int64_t kMaxBlocks = 65535;

bool tokens_ok(int64_t T) { return T >= 0 && T <= kMaxTokens; }

bool layer_ok(const poetx_layer* L) {
  if (!L) return false;
  if (L->m < 8 || L->n < 8 || L->m % 8 || L->n % 8) return false;
  if (L->m > kMaxFeatures || L->n > kMaxFeatures) return false;
  for (int b : {L->b_r, L->b_p})
    if (b < 8 || b > 1024 || b % 8) return false;
  if ((L->m + L->b_r - 1) / L->b_r + (L->n + L->b_p - 1) / L->b_p > kMaxBlocks) return false;
  if (L->act_dtype == POETX_F32) return L->w_dtype == POETX_F32;
  if (L->act_dtype == POETX_BF16) {
    if (L->w_dtype == POETX_BF16) return true;
    if (L->w_dtype == POETX_I8) return L->m % 16 == 0 && L->n % 16 == 0;
    // fp8 codes are only read by the dense kernel, whose shape rules then
    // hold for both products
    if (L->w_dtype == POETX_F8) return L->m % 64 == 0 && L->n % 64 == 0;
  }
  return false;
}

Side side_of(const poetx_layer* L, int side) {
  Side s;
  s.dim = side == POETX_SIDE_R ? L->m : L->n;
  s.b = side == POETX_SIDE_R ? L->b_r : L->b_p;
  s.nblk = static_cast<int>((s.dim + s.b - 1) / s.b);
  return s;
}

bool is_bf16(const poetx_layer* L) { return L->act_dtype == POETX_BF16; }
int act_size(const poetx_layer* L) { return is_bf16(L) ? 2 : 4; }
int w_size(const poetx_layer* L) { return L->w_dtype == POETX_F32 ? 4 : (L->w_dtype == POETX_BF16 ? 2 : 1); }
// a 1-byte base weight with per-column scales: int8 codes or E4M3 fp8 bytes
bool quantized(const poetx_layer* L) { return L->w_dtype == POETX_I8 || L->w_dtype == POETX_F8; }
bool fp8_weight(const poetx_layer* L) { return L->w_dtype == POETX_F8; }
int64_t block_elems(const Side& s) { return static_cast<int64_t>(s.nblk) * s.b * s.b; }
int64_t packed_len(const Side& s) {
  const int64_t last = s.dim - static_cast<int64_t>(s.nblk - 1) * s.b;
  return static_cast<int64_t>(s.nblk - 1) * (static_cast<int64_t>(s.b) * (s.b - 1) / 2) + last * (last - 1) / 2;
}

// Bump allocator over the caller's workspace (256-byte aligned pieces).
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* p) : base(static_cast<char*>(p)) {}
  template <typename T>
  T* take(int64_t count, size_t esize = sizeof(T)) {
    const size_t o = off;
    off = (off + static_cast<size_t>(count) * esize + 255) & ~static_cast<size_t>(255);
    return base ? reinterpret_cast<T*>(base + o) : nullptr;
  }
};

// Split of a token reduction over T so that about `target` workgroups run.
struct Split {
  int nsplit;
  int kchunk;
};

// Both sides' token sums in one launch after the rest of the backward
// (nothing needs dH before the CNP adjoint): one split count sized for the
// blocks of both sides, which halves the float partials against two launches
// each filling the GPU on its own.
bool grads_merged(const poetx_layer* L) {
  return is_bf16(L) && L->b_r == L->b_p && (L->b_r == 256 || L->b_r == 512);
}

Split token_split(const poetx_layer* L, const Side& s, int64_t T) {
  if (is_bf16(L) && (s.b == 256 || s.b == 512)) {
    Split r;
    r.nsplit = std::max(1, grads_merged(L) ? block_grad_splits(T, L->m, s.b, L->n) : block_grad_splits(T, s.dim, s.b));
    r.kchunk = 0;
    return r;
  }
  int tiles;
  if (is_bf16(L)) {
    const int t = s.b >= 256 ? 256 : 128;
    tiles = ((s.b + t - 1) / t) * ((s.b + t - 1) / t);
  } else {
    tiles = ((s.b + 63) / 64) * ((s.b + 63) / 64);
  }
  const int64_t target = 512;
  int64_t ns = (target + static_cast<int64_t>(s.nblk) * tiles - 1) / (static_cast<int64_t>(s.nblk) * tiles);
  ns = std::max<int64_t>(1, std::min<int64_t>(ns, std::max<int64_t>(1, T / 256)));
  ns = std::min<int64_t>(ns, std::max<int64_t>(1, 65535 / s.nblk));
  int64_t kchunk = (T + ns - 1) / ns;
  kchunk = std::max<int64_t>(64, (kchunk + 63) / 64 * 64);
  Split r;
  r.kchunk = static_cast<int>(kchunk);
  r.nsplit = static_cast<int>(std::max<int64_t>(1, (T + kchunk - 1) / kchunk));
  return r;
}

// Blocks processed in one batch: side 0's n0 blocks followed by side 1's n1
// blocks (n1 = 0 for one side alone). Both sides share a batch when their
// block sizes match.
struct Group {
  int b;
  int64_t dim0, dim1;
  int n0, n1;
  int64_t elems() const { return static_cast<int64_t>(n0 + n1) * b * b; }
};

Group group_of(const Side& s) { return Group{s.b, s.dim, 0, s.nblk, 0}; }
Group group_of(const Side& s0, const Side& s1) { return Group{s0.b, s0.dim, s1.dim, s0.nblk, s1.nblk}; }

// Upper bound of the block elements any CNP batch of this layer holds.
int64_t cnp_batch_elems(const poetx_layer* L) {
  const Side R = side_of(L, POETX_SIDE_R), P = side_of(L, POETX_SIDE_P);
  if (R.b == P.b) return block_elems(R) + block_elems(P);
  return std::max(block_elems(R), block_elems(P));
}

// ---------------------------------------------------------------------------
// workspace plans (a null base only measures)
// ---------------------------------------------------------------------------

struct CnpWs {
  float *Qf, *Q2f, *Tf, *Sf;
  uint16_t *Qh, *Q2h, *Sh;
};

// bfloat16 blocks of 256 take the two-launch build: unpack to bfloat16 Q,
// then every product of the chain with Q kept in LDS (cnp_fused.hip).
bool cnp_fused_applies(const poetx_layer* L, int b) { return is_bf16(L) && b == 256; }

CnpWs plan_cnp(const poetx_layer* L, int64_t bb, Carve& c) {
  CnpWs w{};
  if (cnp_fused_applies(L, L->b_r) && cnp_fused_applies(L, L->b_p)) {
    w.Qh = c.take<uint16_t>(bb);
    return w;
  }
  w.Qf = c.take<float>(bb);
  w.Q2f = c.take<float>(bb);
  w.Tf = c.take<float>(bb);
  if (is_bf16(L)) {
    w.Qh = c.take<uint16_t>(bb);
    w.Q2h = c.take<uint16_t>(bb);
    w.Sh = c.take<uint16_t>(bb);
  } else {
    w.Sf = c.take<float>(bb);
  }
  return w;
}

struct CnpBwdWs {
  float *Qf, *P1, *Hf, *F, *E;
  uint16_t *Qh, *Hh, *Fh;
};

CnpBwdWs plan_cnp_bwd(const poetx_layer* L, int64_t bb, Carve& c) {
  CnpBwdWs w{};
  w.Qf = c.take<float>(bb);
  w.P1 = c.take<float>(bb);
  w.F = c.take<float>(bb);
  w.E = c.take<float>(bb);
  if (is_bf16(L)) {
    w.Qh = c.take<uint16_t>(bb);
    w.Hh = c.take<uint16_t>(bb);
    w.Fh = c.take<uint16_t>(bb);
  } else {
    w.Hf = c.take<float>(bb);
  }
  return w;
}

struct FwdWs {
  void* buf;
  int32_t* inv_p;
  void* split;  // the dense product's split of a partial last round (or null)
  void* wdeq;   // int8 weight the dense kernel cannot take: bfloat16 copy of its codes (or null)
};

size_t dense_split_bytes(const poetx_layer* L, int64_t M, int64_t N, int64_t K);
bool i8_staging(const poetx_layer* L);

FwdWs plan_fwd(const poetx_layer* L, int64_t T, Carve& c) {
  FwdWs w;
  w.buf = c.take<char>(T * std::max(L->m, L->n) * act_size(L));
  w.inv_p = c.take<int32_t>(L->n);
  const size_t sb = dense_split_bytes(L, T, L->n, L->m);
  w.split = sb ? c.take<char>(static_cast<int64_t>(sb)) : nullptr;
  w.wdeq = i8_staging(L) ? c.take<uint16_t>(L->m * L->n) : nullptr;
  return w;
}

struct BwdWs {
  void *bufA, *bufB;
  void* bufC;         // [T][m]: keeps dY2 alive for the merged token sums (or null)
  void* wh;           // Wp H (m x n), when the backward folds H into the weight
  int32_t* inv_r;
  float *part_r, *part_p;
  float *Us, *Uk;     // symmetric / skew parts of dG (side R) and dH (side P)
  uint16_t *Ush, *Ukh;
  void* split;        // the dense product's split of a partial last round (or null)
  size_t cnp_off;     // the CNP adjoint scratch starts here
};

// dX2 = dY2 H^T Wp^T = dY2 (Wp H)^T: with a float or bf16 weight and fewer
// weight rows than tokens it is cheaper to multiply the m x n weight by H once
// than the T x n gradient by H^T (dH only needs dY2 and Y1, never dY1).
bool fold_h(const poetx_layer* L, int64_t T) { return !quantized(L) && L->m < T; }

BwdWs plan_bwd(const poetx_layer* L, int64_t T, Carve& c) {
  BwdWs w;
  const int64_t rowmax = std::max(L->m, L->n);
  const Side R = side_of(L, POETX_SIDE_R), P = side_of(L, POETX_SIDE_P);
  const int64_t Tn = std::max<int64_t>(T, 1);
  w.bufA = c.take<char>(T * rowmax * act_size(L));
  w.bufB = c.take<char>(T * rowmax * act_size(L));
  w.bufC = grads_merged(L) ? c.take<char>(T * L->m * act_size(L)) : nullptr;
  w.wh = fold_h(L, T) ? c.take<char>(L->m * L->n * w_size(L)) : nullptr;
  w.inv_r = c.take<int32_t>(L->m);
  w.part_r = c.take<float>(static_cast<int64_t>(token_split(L, R, Tn).nsplit) * block_elems(R));
  w.part_p = c.take<float>(static_cast<int64_t>(token_split(L, P, Tn).nsplit) * block_elems(P));
  const int64_t all = block_elems(R) + block_elems(P);
  w.Us = c.take<float>(all);
  w.Uk = c.take<float>(all);
  w.Ush = c.take<uint16_t>(all);
  w.Ukh = c.take<uint16_t>(all);
  const size_t sb = dense_split_bytes(L, T, L->m, L->n);
  w.split = sb ? c.take<char>(static_cast<int64_t>(sb)) : nullptr;
  w.cnp_off = c.off;
  Carve m(nullptr);
  plan_cnp_bwd(L, cnp_batch_elems(L), m);
  c.off += m.off;
  return w;
}

struct MergeWs {
  void *C1, *C2;
  int32_t *inv_r, *inv_p;  // inverses of the current permutations
  int32_t *rmap, *cmap;    // merged-weight row / column for each row / column of the next frame
  // int8 weights: the merge runs in float on a float copy of both CNP buffers
  float *gr32, *gp32;
  unsigned int* amax;
};

MergeWs plan_merge(const poetx_layer* L, Carve& c) {
  MergeWs w;
  const bool i8 = quantized(L);
  const int64_t es = i8 ? 4 : w_size(L);
  w.C1 = c.take<char>(L->m * L->n * es);
  w.C2 = c.take<char>(L->m * L->n * es);
  w.inv_r = c.take<int32_t>(L->m);
  w.inv_p = c.take<int32_t>(L->n);
  w.rmap = c.take<int32_t>(L->m);
  w.cmap = c.take<int32_t>(L->n);
  w.gr32 = w.gp32 = nullptr;
  w.amax = nullptr;
  if (i8) {
    const Side R = side_of(L, POETX_SIDE_R), P = side_of(L, POETX_SIDE_P);
    w.gr32 = c.take<float>(2 * block_elems(R));
    w.gp32 = c.take<float>(2 * block_elems(P));
    w.amax = c.take<unsigned int>(L->n);
  }
  return w;
}

size_t cnp_build_bytes(const poetx_layer* L) {
  Carve m(nullptr);
  plan_cnp(L, cnp_batch_elems(L), m);
  return m.off;
}

// X1 (T x m) then Y1 (T x n), activation dtype: the forward's saved tensors
int64_t saved_region(const poetx_layer* L, int64_t T) { return T * (L->m + L->n) * act_size(L); }

// Scratch of one permutation draw: one packed 64-bit key per index.
size_t perm_ws_bytes(int64_t dim) { return static_cast<size_t>(dim) * sizeof(uint64_t); }

size_t ws_bytes_for(const poetx_layer* L, int64_t T, int op) {
  Carve c(nullptr);
  switch (op) {
    case POETX_OP_CNP_BUILD: return cnp_build_bytes(L);
    case POETX_OP_WEIGHT_PREPARE: return 0;
    case POETX_OP_WEIGHT_EXPORT: return static_cast<size_t>(L->n) * sizeof(int32_t);
    case POETX_OP_FORWARD: plan_fwd(L, T, c); return c.off;
    case POETX_OP_BACKWARD: plan_bwd(L, T, c); return c.off;
    case POETX_OP_MERGE: plan_merge(L, c); return c.off;
    case POETX_OP_FORWARD_MEM: {
      // X1 and Y1 live in the workspace
      c.take<char>(saved_region(L, T));
      plan_fwd(L, T, c);
      return c.off;
    }
    case POETX_OP_BACKWARD_MEM: {
      // X1 and Y1 recomputed into the workspace; the recompute's scratch and
      // the backward's share what follows
      c.take<char>(saved_region(L, T));
      Carve f = c, b = c;
      plan_fwd(L, T, f);
      plan_bwd(L, T, b);
      return std::max(f.off, b.off);
    }
    case POETX_OP_SAMPLE_PERM: return perm_ws_bytes(std::max(L->m, L->n));
    default: return 0;
  }
}

// ---------------------------------------------------------------------------
// optional kernel timing log (poetx_profile_*): HIP events around each step
// ---------------------------------------------------------------------------

struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct ProfScope {
  bool on = false;
  hipStream_t st;
  ProfRec rec{};
  ProfScope(const char* name, hipStream_t s) : st(s) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (!g_prof_on) return;
    rec.name = name;
    rec.start = prof_event();
    rec.stop = prof_event();
    if (!rec.start || !rec.stop) return;
    on = hipEventRecord(rec.start, st) == hipSuccess;
  }
  ~ProfScope() {
    if (!on) return;
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (hipEventRecord(rec.stop, st) == hipSuccess) g_prof.push_back(rec);
  }
};

// ---------------------------------------------------------------------------
// building blocks
// ---------------------------------------------------------------------------

bool gemm(const poetx_layer* L, const GemmDesc& d, int am, int bm, int ct, hipStream_t st) {
  if (is_bf16(L)) return gemm_bf16(d, am, bm, ct, st);
  return gemm_f32(d, am, bm, st);
}

// The dense W0 product: the specialised kernel when its shape constraints
// hold, else the general engine.
bool dense_kernel_applies(const poetx_layer* L, int N, int K) {
  return is_bf16(L) && K % 64 == 0 && N % 8 == 0;
}

// ... with B as int8 codes, converted inside the kernel: the code rows must
// also be whole 16-byte chunks (see i8_staging for the other widths)
bool dense_i8_applies(const poetx_layer* L, int N, int K, int64_t ldb) {
  return dense_kernel_applies(L, N, K) && N % 16 == 0 && ldb % 16 == 0;
}

// The quantised variant stores the base weight as int8 and dequantises it at
// run time (section "POET-XQ"): the dense kernel reads the int8 codes and
// turns them into bfloat16 on their way into LDS (exact); its epilogue (or
// the preceding apply, in the backward) applies the column scales. Where the
// dense kernel's int8 shape rules fail, the backward's general engine reads
// the codes itself, and the forward (which reads Wp N-contiguous) copies them
// to bfloat16 in the workspace first.
bool i8_staging(const poetx_layer* L) {
  return L->w_dtype == POETX_I8 && !dense_i8_applies(L, static_cast<int>(L->n), static_cast<int>(L->m), L->n);
}

// Workspace of the dense kernel's split of a partial last round of tiles.
size_t dense_split_bytes(const poetx_layer* L, int64_t M, int64_t N, int64_t K) {
  if (!dense_kernel_applies(L, static_cast<int>(N), static_cast<int>(K))) return 0;
  return gemm_dense_split_bytes(static_cast<int>(M), static_cast<int>(N), static_cast<int>(K));
}

// b_ncontig: B is Wp itself read as [K][N] (the forward); otherwise B rows
// are K-contiguous (the backward). i8: B holds int8 codes (K-contiguous only).
bool dense_product(const poetx_layer* L, const GemmDesc& d, bool i8, bool b_ncontig, void* split_ws,
                   hipStream_t st) {
  if (i8 ? dense_i8_applies(L, d.N, d.K, d.ldb) : dense_kernel_applies(L, d.N, d.K))
    return gemm_dense_bf16(d, split_ws, st, b_ncontig, i8);
  if (i8 && d.b_fp8) return false;  // (the layer's shape rules keep fp8 on the dense kernel)
  if (b_ncontig) return !i8 && gemm(L, d, A_KCONTIG, B_NCONTIG, is_bf16(L) ? C_BF16 : C_F32, st);
  return gemm(L, d, A_KCONTIG, i8 ? B_KCONTIG_I8 : B_KCONTIG, is_bf16(L) ? C_BF16 : C_F32, st);
}

// Planes of a CNP block buffer: 0 = G - I row-major, 1 = (G - I)^T row-major.
const void* plane(const poetx_layer* L, const void* g, const Side& s, int p) {
  return static_cast<const char*>(g) + static_cast<int64_t>(p) * block_elems(s) * act_size(L);
}

// The side job that writes inv = the inverse of the permutation perm of [0, n).
SideJob inverse_job(const int32_t* perm, int32_t* inv, int64_t n) {
  SideJob j;
  j.src0 = perm;
  j.dst0 = inv;
  j.n0 = static_cast<int>(n);
  return j;
}

// out[:, blocks] = in + in (G - I)^{T or not} for every diagonal block
// (plane 1 gives in G, plane 0 gives in G^T), optional per-column scale.
// job (optional): work for later launches, done in the same launch where the
// apply kernel runs, else in a launch of its own.
bool block_apply(const poetx_layer* L, const Side& s, int64_t T, const void* in, void* out, const void* gbuf,
                 int p, const float* colscale, hipStream_t st, const SideJob& job = SideJob()) {
  if (is_bf16(L) && (s.b == 64 || s.b == 128 || s.b == 256 || s.b == 512) && T > 0)
    return block_apply_bf16(static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out), s.dim,
                            static_cast<const uint16_t*>(plane(L, gbuf, s, p)), colscale, T, s.dim, s.b, st, job);
  side_job(job, st);
  if (T <= 0) return true;
  GemmDesc d;
  d.A = in;
  d.lda = s.dim;
  d.sA = s.b;
  d.B = plane(L, gbuf, s, p);
  d.ldb = s.b;
  d.sB = static_cast<int64_t>(s.b) * s.b;
  d.R = in;
  d.ldr = s.dim;
  d.sR = s.b;
  d.C = out;
  d.ldc = s.dim;
  d.sC = s.b;
  d.scale = colscale;
  d.sScale = s.b;
  d.M = static_cast<int>(T);
  d.N = d.K = s.b;
  d.batch = s.nblk;
  d.ragged_dim = static_cast<int>(s.dim);
  d.ragged_blk = s.b;
  d.ragged_mask = 2 | 4;
  return gemm(L, d, A_KCONTIG, B_KCONTIG, is_bf16(L) ? C_BF16 : C_F32, st);
}

// part[s][z] = sum over the tokens of split s of A_z^T dO_z (b x b per block)
bool block_token_grad(const poetx_layer* L, const Side& s, int64_t T, const void* act, const void* dout,
                      float* part, const Split& sp, hipStream_t st) {
  if (is_bf16(L) && (s.b == 256 || s.b == 512))
    return block_grad_bf16(static_cast<const uint16_t*>(act), static_cast<const uint16_t*>(dout), part, s.dim, T,
                           s.dim, s.b, sp.nsplit, st);
  GemmDesc d;
  d.A = act;
  d.lda = s.dim;
  d.sA = s.b;
  d.B = dout;
  d.ldb = s.dim;
  d.sB = s.b;
  d.C = part;
  d.ldc = s.b;
  d.sC = static_cast<int64_t>(s.b) * s.b;
  d.sCsplit = block_elems(s);
  d.M = d.N = s.b;
  d.K = static_cast<int>(T);
  d.batch = s.nblk;
  d.ksplit = sp.nsplit;
  d.kchunk = sp.kchunk;
  d.ragged_dim = static_cast<int>(s.dim);
  d.ragged_blk = s.b;
  d.ragged_mask = 1 | 2;
  d.store_full = 1;
  return gemm(L, d, A_MCONTIG, B_NCONTIG, C_F32, st);
}

// Batched b x b product C = alpha A B^T-form (see gemm.hpp) with optional
// addend and bf16 copy, over the nblk blocks of one side.
bool sq(const poetx_layer* L, const Group& g, const void* A, int am, const void* B, int bm, float* C, uint16_t* C2,
        float alpha, const float* D, hipStream_t st, float beta = 1.f) {
  GemmDesc d;
  const Side s{0, g.b, g.n0 + g.n1};
  const int64_t bb = static_cast<int64_t>(s.b) * s.b;
  d.A = A;
  d.lda = s.b;
  d.sA = bb;
  d.B = B;
  d.ldb = s.b;
  d.sB = bb;
  d.C = C;
  d.ldc = s.b;
  d.sC = bb;
  d.C2 = C2;
  d.ldc2 = s.b;
  d.sC2 = bb;
  d.D = D;
  d.ldd = s.b;
  d.sD = bb;
  d.beta = D ? beta : 0.f;
  d.alpha = alpha;
  d.M = d.N = d.K = s.b;
  d.batch = s.nblk;
  return gemm(L, d, am, bm, C_F32, st);
}

// G - I for every block of a group: Q2 = Q Q, S = 2Q + Q2, T = S Q2,
// G - I = 2Q + 2Q2 + T  (= (I+Q)(I+Q+Q^2+Q^3) - I with every higher term
// formed from Q and Q^2, section "3. Cayley-Neumann 参数化优化").
bool cnp_group(const poetx_layer* L, const Group& g, const float* q0, const float* q1, void* g0, void* g1, void* ws,
               hipStream_t st) {
  Carve c(ws);
  CnpWs w = plan_cnp(L, g.elems(), c);
  if (cnp_fused_applies(L, g.b)) {
    uint16_t* Qh = w.Qh;
    unpack_skew2(q0, g.dim0, g.n0, q1, g.dim1, g.n1, g.b, nullptr, Qh, st);
    return cnp_build_fused(Qh, g.n0, g.n1, g.b, g0, g1, st);
  }
  const bool bf = is_bf16(L);
  unpack_skew2(q0, g.dim0, g.n0, q1, g.dim1, g.n1, g.b, w.Qf, bf ? w.Qh : nullptr, st);
  if (bf && g.b % 128 == 0) {
    // two fused block products: Q2 = -Q Q^T with S = 2Q + Q2 in the epilogue,
    // then G - I = S Q2 + 2Q + 2Q2 written as both planes
    BlockProdDesc p;
    p.A1 = w.Qh;
    p.B1 = w.Qh;
    p.b = g.b;
    p.nblk = g.n0 + g.n1;
    p.alpha = -1.f;
    p.out1 = w.Q2h;
    p.Eh = w.Qh;
    p.alpha2 = -1.f;
    p.gamma2 = 2.f;
    p.out2 = w.Sh;
    if (!block_prod_bf16(p, st)) return false;
    const int64_t bb = static_cast<int64_t>(g.b) * g.b;
    BlockProdDesc t;
    t.A1 = w.Sh;
    t.B1 = w.Q2h;  // Q2 symmetric: its rows are the rows of Q2^T
    t.b = g.b;
    t.nblk = g.n0 + g.n1;
    t.alpha = 1.f;
    t.beta = 2.f;
    t.Ef = w.Qf;
    t.gamma = 2.f;
    t.Eh = w.Q2h;
    t.out1 = g0;
    t.out1t = g0 ? static_cast<uint16_t*>(g0) + g.n0 * bb : nullptr;
    t.z_split = g.n0;
    t.out1_hi = g1;
    t.out1t_hi = g1 ? static_cast<uint16_t*>(g1) + g.n1 * bb : nullptr;
    return block_prod_bf16(t, st);
  }
  const void* Qop = bf ? static_cast<const void*>(w.Qh) : w.Qf;
  // Q Q = -Q Q^T: the NT product with B = Q and alpha = -1 (Q skew)
  if (!sq(L, g, Qop, A_KCONTIG, Qop, B_KCONTIG, w.Q2f, bf ? w.Q2h : nullptr, -1.f, nullptr, st)) return false;
  cnp_mid(w.Qf, w.Q2f, bf ? w.Sh : nullptr, bf ? nullptr : w.Sf, g.elems(), st);
  // S Q2 with Q2 symmetric: B rows = Q2 rows
  const void* Sop = bf ? static_cast<const void*>(w.Sh) : w.Sf;
  const void* Q2op = bf ? static_cast<const void*>(w.Q2h) : w.Q2f;
  if (!sq(L, g, Sop, A_KCONTIG, Q2op, B_KCONTIG, w.Tf, nullptr, 1.f, nullptr, st)) return false;
  cnp_finish2(w.Qf, w.Q2f, w.Tf, g.b, g.n0, g0, g.n1, g1, bf, st);
  return true;
}

// dq from the block gradients U = dL/dG of a group, given as Us = (U+U^T)/2
// and Uk = (U-U^T)/2. The packed gradient only sees the skew part of dL/dQ,
// and with Q skew the adjoint of G = (I+Q)(I+Q+Q^2+Q^3) (a sum of
// Q^a U Q^c with coefficients 2, -2, 2, -1 for a + c = 0..3) reduces to
//   dq = pack(E),  E = 2 Uk + Q F,  F = -4 Us + 2 Uk Q + Q H1,
//   H1 = 4 Uk - 2 (Q Us - (Q Us)^T),
// four b x b products per block (pack(M)[k(i,l)] = M[i][l] - M[l][i]).
bool cnp_bwd_group(const poetx_layer* L, const Group& g, const float* q0, const float* q1, const float* Us,
                   const float* Uk, const uint16_t* Ush, const uint16_t* Ukh, float* dq0, float* dq1, void* cnp_ws,
                   hipStream_t st) {
  Carve c(cnp_ws);
  CnpBwdWs w = plan_cnp_bwd(L, g.elems(), c);
  const bool bf = is_bf16(L);
  const int nb = g.n0 + g.n1;
  if (bf && g.b % 128 == 0) {
    // Same recurrence as below in three fused block products (Q skew, Us
    // symmetric, Uk skew, so every right factor is read by rows):
    //   H1/2 = 2 Uk - (Q Us + Us Q),          Q Us = NT(Q, Us), Us Q = -NT(Us, Q)
    //   F    = -4 Us - 2 (NT(Uk, Q) + NT(Q, H1/2)),   written transposed
    //   E    = 2 Uk + NT(Q, F^T), of which only E - E^T is needed:
    //   E - E^T = 4 Uk + NT(Q, F^T) - NT(F^T, Q)  (Uk skew; (Q F)^T = F^T Q^T),
    //   one product whose epilogue writes dq packed
    unpack_skew2(q0, g.dim0, g.n0, q1, g.dim1, g.n1, g.b, nullptr, w.Qh, st);
    BlockProdDesc h;
    h.A1 = w.Qh;
    h.B1 = Ush;
    h.A2 = Ush;
    h.B2 = w.Qh;
    h.neg2 = 1;
    h.b = g.b;
    h.nblk = nb;
    h.alpha = -1.f;
    h.beta = 2.f;
    h.Ef = Uk;
    h.out1 = w.Hh;
    if (!block_prod_bf16(h, st)) return false;
    BlockProdDesc f;
    f.A1 = Ukh;
    f.B1 = w.Qh;
    f.A2 = w.Qh;
    f.B2 = w.Hh;
    f.b = g.b;
    f.nblk = nb;
    f.alpha = -2.f;
    f.beta = -4.f;
    f.Ef = Us;
    f.out1t = w.Fh;
    if (!block_prod_bf16(f, st)) return false;
    BlockProdDesc e;
    e.A1 = w.Qh;
    e.B1 = w.Fh;
    e.A2 = w.Fh;
    e.B2 = w.Qh;
    e.neg2 = 1;
    e.b = g.b;
    e.nblk = nb;
    e.alpha = 1.f;
    e.beta = 4.f;
    e.Ef = Uk;
    e.z_split = g.n0;
    e.pk = dq0;
    e.pk_dim = g.dim0;
    e.pk_hi = dq1;
    e.pk_dim_hi = g.dim1;
    return block_prod_bf16(e, st);
  }
  unpack_skew2(q0, g.dim0, g.n0, q1, g.dim1, g.n1, g.b, w.Qf, bf ? w.Qh : nullptr, st);
  const void* Q = bf ? static_cast<const void*>(w.Qh) : w.Qf;
  const void* UsOp = bf ? static_cast<const void*>(Ush) : Us;
  const void* UkOp = bf ? static_cast<const void*>(Ukh) : Uk;
  // P1 = Q Us (Us symmetric: B rows = Us rows)
  bool ok = sq(L, g, Q, A_KCONTIG, UsOp, B_KCONTIG, w.P1, nullptr, 1.f, nullptr, st);
  cnp_h1(Uk, w.P1, g.b, nb, bf ? nullptr : w.Hf, bf ? w.Hh : nullptr, st);
  const void* H1 = bf ? static_cast<const void*>(w.Hh) : w.Hf;
  // F = 2 Uk Q - 4 Us  (Uk Q = -Uk Q^T: B rows = Q rows, alpha = -2), then += Q H1
  ok = ok && sq(L, g, UkOp, A_KCONTIG, Q, B_KCONTIG, w.F, nullptr, -2.f, Us, st, -4.f);
  ok = ok && sq(L, g, Q, A_KCONTIG, H1, B_NCONTIG, w.F, bf ? w.Fh : nullptr, 1.f, w.F, st, 1.f);
  const void* F = bf ? static_cast<const void*>(w.Fh) : w.F;
  // E = 2 Uk + Q F
  ok = ok && sq(L, g, Q, A_KCONTIG, F, B_NCONTIG, w.E, nullptr, 1.f, Uk, st, 2.f);
  if (!ok) return false;
  pack_asym2(w.E, g.b, g.dim0, g.n0, dq0, g.dim1, g.n1, dq1, st);
  return true;
}

thread_local hipError_t g_last_hip = hipSuccess;
thread_local std::string g_last_hip_msg;

// Drops a HIP error left pending by earlier calls of other code on this
// thread, so that launch_status() sees only this entry point's launches.
void clear_pending_error() { (void)hipGetLastError(); }

int launch_status() {
  const hipError_t e = hipGetLastError();
  if (e == hipSuccess) return POETX_OK;
  g_last_hip = e;
  return POETX_EHIP;
}

int check_ws(const poetx_layer* L, int64_t T, int op, const void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_for(L, T, op);
  if (need == 0) return POETX_OK;
  if (ws_bytes < need) return POETX_EWORKSPACE;
  if (!ws || !aligned16(ws)) return POETX_EINVAL;
  return POETX_OK;
}

// Forward steps up to Y1 = X2 Wp, then (when z is given) Y2 = Y1 Diag(H) and
// the scatter to z. X1, Y1: where the saved tensors go (the caller's buffer,
// or the workspace in the memory variant). `recompute` only renames the
// profiled steps: the memory variant's backward runs the first three again.
bool forward_core(const poetx_layer* L, int64_t T, const void* x, const int32_t* perm_r, const int32_t* perm_p,
                  const void* g_r, const void* g_p, const void* wp, const float* wscale_p, void* z, void* X1,
                  void* Y1, const FwdWs& w, bool recompute, hipStream_t stream) {
  const Side R = side_of(L, POETX_SIDE_R), P = side_of(L, POETX_SIDE_P);
  const int es = act_size(L);
  const bool i8 = quantized(L);
  bool ok;
  {
    ProfScope p(recompute ? "recompute_gather_x" : "gather_x", stream);
    ok = gather_cols(x, L->m, nullptr, X1, L->m, nullptr, perm_r, L->m, T, es, stream);
  }
  {
    ProfScope p(recompute ? "recompute_apply_r" : "apply_r_fwd", stream);
    ok = ok && block_apply(L, R, T, X1, w.buf, g_r, 1, nullptr, stream);
  }
  // Y1 = X2 Wp with Wp read as B[k][n] (N-contiguous)
  GemmDesc d;
  d.dense = 1;
  d.b_fp8 = fp8_weight(L);
  d.A = w.buf;
  d.lda = L->m;
  d.B = wp;
  d.ldb = L->n;
  d.C = Y1;
  d.ldc = L->n;
  d.scale = i8 ? wscale_p : nullptr;
  d.M = static_cast<int>(T);
  d.N = static_cast<int>(L->n);
  d.K = static_cast<int>(L->m);
  if (w.wdeq) {
    ProfScope p(recompute ? "recompute_dequant_w" : "dequant_w_fwd", stream);
    ok = ok && i8_to_bf16(static_cast<const int8_t*>(wp), static_cast<uint16_t*>(w.wdeq), L->m * L->n, stream);
    d.B = w.wdeq;
  }
  {
    ProfScope p(recompute ? "recompute_gemm_dense" : "gemm_dense_fwd", stream);
    ok = ok && dense_product(L, d, i8 && !w.wdeq, true, w.split, stream);
  }
  if (!z) return ok;
  {
    ProfScope p("apply_p_fwd", stream);
    // the same launch inverts perm_p for the scatter
    ok = ok && block_apply(L, P, T, Y1, w.buf, g_p, 1, nullptr, stream, inverse_job(perm_p, w.inv_p, L->n));
  }
  {
    ProfScope p("scatter_z", stream);
    ok = ok && gather_cols(w.buf, L->n, nullptr, z, L->n, nullptr, w.inv_p, L->n, T, es, stream);
  }
  return ok;
}

// Backward from the saved X1, Y1 to dq_r, dq_p and dx (T > 0).
bool backward_core(const poetx_layer* L, int64_t T, const void* X1, const void* Y1, const void* dz,
                   const int32_t* perm_r, const int32_t* perm_p, const float* q_r, const float* q_p,
                   const void* g_r, const void* g_p, const void* wp, const float* wscale_p, float* dq_r,
                   float* dq_p, void* dx, const BwdWs& w, void* cnp_ws, hipStream_t stream) {
  const Side R = side_of(L, POETX_SIDE_R), P = side_of(L, POETX_SIDE_P);
  const bool i8 = quantized(L);
  const int es = act_size(L);
  // P side: dY2 = dZ Phi^T, dH = sum_t Y1^T dY2, and either dY1 = dY2 H^T
  // (times the column scales for int8 weights, which belong to Wp's columns)
  // for dX2 = dY1 Wp^T, or the fold dX2 = dY2 (Wp H)^T
  const bool fold = fold_h(L, T);
  bool ok;
  {
    ProfScope p("gather_dz", stream);
    ok = gather_cols(dz, L->n, nullptr, w.bufA, L->n, nullptr, perm_p, L->n, T, es, stream);
  }
  const Split spP = token_split(L, P, T);
  const bool merged = grads_merged(L);
  void* const dY2 = w.bufA;
  if (!merged) {
    ProfScope p("grad_h", stream);
    ok = ok && block_token_grad(L, P, T, Y1, dY2, w.part_p, spP, stream);
  }
  // buffers: dY2 in bufA; with the merged token sums it stays there until
  // the end, and the [T][m] results use bufB and bufC
  GemmDesc d;
  d.dense = 1;
  d.b_fp8 = fp8_weight(L);
  void* dX1;
  if (fold) {
    ProfScope p("fold_h_bwd", stream);
    ok = ok && block_apply(L, P, L->m, wp, w.wh, g_p, 1, nullptr, stream);
    d.A = dY2;
    d.B = w.wh;
    d.C = w.bufB;
    dX1 = merged ? w.bufC : w.bufA;
  } else {
    ProfScope p("apply_p_bwd", stream);
    ok = ok && block_apply(L, P, T, dY2, w.bufB, g_p, 0, i8 ? wscale_p : nullptr, stream);
    d.A = w.bufB;
    d.B = wp;
    d.C = merged ? w.bufC : w.bufA;
    dX1 = w.bufB;
  }
  void* const dX2 = d.C;
  d.lda = L->n;
  d.ldb = L->n;
  d.ldc = L->m;
  d.M = static_cast<int>(T);
  d.N = static_cast<int>(L->m);
  d.K = static_cast<int>(L->n);
  {
    ProfScope p("gemm_dense_bwd", stream);
    ok = ok && dense_product(L, d, i8, false, w.split, stream);
  }
  // R side: dX1 = dX2 G^T, dG = sum_t X1^T dX2, dX = dX1 Psi
  {
    ProfScope p("apply_r_bwd", stream);
    // the same launch inverts perm_r for the scatter of dx
    ok = ok && block_apply(L, R, T, dX2, dX1, g_r, 0, nullptr, stream, inverse_job(perm_r, w.inv_r, L->m));
  }
  const Split spR = token_split(L, R, T);
  if (!merged) {
    ProfScope p("grad_g", stream);
    ok = ok && block_token_grad(L, R, T, X1, dX2, w.part_r, spR, stream);
  }
  {
    ProfScope p("scatter_dx", stream);
    ok = ok && gather_cols(dX1, L->m, nullptr, dx, L->m, nullptr, w.inv_r, L->m, T, es, stream);
  }
  if (merged) {
    ProfScope p("grad_gh", stream);
    ok = ok && block_grad2_bf16(static_cast<const uint16_t*>(X1), static_cast<const uint16_t*>(dX2), w.part_r, L->m,
                                static_cast<const uint16_t*>(Y1), static_cast<const uint16_t*>(dY2), w.part_p, L->n,
                                T, R.b, spR.nsplit, stream);
  }
  // dq_r, dq_p from the token sums dG, dH
  {
    ProfScope p("cnp_bwd", stream);
    const bool bf = is_bf16(L);
    const int64_t eR = block_elems(R);
    // both sides' blocks in one launch when their block sizes match
    if (R.b == P.b) {
      reduce_symskew2(w.part_r, spR.nsplit, R.nblk, w.part_p, spP.nsplit, P.nblk, R.b, w.Us, w.Uk,
                      bf ? w.Ush : nullptr, bf ? w.Ukh : nullptr, stream);
    } else {
      reduce_symskew2(w.part_r, spR.nsplit, R.nblk, nullptr, 0, 0, R.b, w.Us, w.Uk, bf ? w.Ush : nullptr,
                      bf ? w.Ukh : nullptr, stream);
      reduce_symskew2(w.part_p, spP.nsplit, P.nblk, nullptr, 0, 0, P.b, w.Us + eR, w.Uk + eR,
                      bf ? w.Ush + eR : nullptr, bf ? w.Ukh + eR : nullptr, stream);
    }
    if (R.b == P.b) {
      ok = ok && cnp_bwd_group(L, group_of(R, P), q_r, q_p, w.Us, w.Uk, w.Ush, w.Ukh, dq_r, dq_p, cnp_ws, stream);
    } else {
      ok = ok && cnp_bwd_group(L, group_of(R), q_r, nullptr, w.Us, w.Uk, w.Ush, w.Ukh, dq_r, nullptr, cnp_ws,
                               stream);
      ok = ok && cnp_bwd_group(L, group_of(P), q_p, nullptr, w.Us + eR, w.Uk + eR, w.Ush + eR, w.Ukh + eR, dq_p,
                               nullptr, cnp_ws, stream);
    }
  }
  return ok;
}

}  // namespace

// Scratch of poetx_sample_perm_static, the draw for callers that cannot
// allocate: one packed key per index of the largest accepted draw (2^20
// indices, 8 MiB). Every device the library runs on holds its own copy from
// the load of the code object until the process ends. In host code the name
// `scratch` is only a host-side stand-in: kernels must get the device address
// that hipGetSymbolAddress returns for the device they run on.
static __device__ __align__(256) uint64_t scratch[kMaxPermDim];

namespace {

std::mutex g_scratch_mu;
std::vector<uint64_t*> g_scratch_ptr;  // device address of `scratch`, per device

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream), looked up once per device with that device
// current.
int static_scratch(hipStream_t stream, uint64_t** out) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess || dev < 0) {
    g_last_hip = e != hipSuccess ? e : hipErrorInvalidDevice;
    return POETX_EHIP;
  }
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (static_cast<size_t>(dev) >= g_scratch_ptr.size()) g_scratch_ptr.resize(static_cast<size_t>(dev) + 1, nullptr);
  if (!g_scratch_ptr[static_cast<size_t>(dev)]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess || !p) {
      g_last_hip = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return POETX_EHIP;
    }
    g_scratch_ptr[static_cast<size_t>(dev)] = static_cast<uint64_t*>(p);
  }
  *out = g_scratch_ptr[static_cast<size_t>(dev)];
  return POETX_OK;
}

}  // namespace

extern "C" {

int poetx_abi_version(void) { return POETX_ABI_VERSION; }

const char* poetx_last_hip_error(void) {
  g_last_hip_msg = std::string(hipGetErrorName(g_last_hip)) + ": " + hipGetErrorString(g_last_hip);
  return g_last_hip_msg.c_str();
}

const char* poetx_strerror(int status) {
  switch (status) {
    case POETX_OK: return "ok";
    case POETX_EINVAL: return "invalid argument (pointer, alignment, shape, dtype or size)";
    case POETX_EUNSUPPORTED: return "valid request the library does not implement";
    case POETX_EHIP: return "HIP kernel launch failed";
    case POETX_EWORKSPACE: return "workspace smaller than poetx_workspace_bytes()";
    default: return "unknown status";
  }
}

size_t poetx_packed_len(const poetx_layer* L, int side) {
  if (!layer_ok(L) || (side != POETX_SIDE_R && side != POETX_SIDE_P)) return 0;
  return static_cast<size_t>(packed_len(side_of(L, side)));
}

size_t poetx_gbuf_bytes(const poetx_layer* L, int side) {
  if (!layer_ok(L) || (side != POETX_SIDE_R && side != POETX_SIDE_P)) return 0;
  return static_cast<size_t>(2 * block_elems(side_of(L, side)) * act_size(L));
}

size_t poetx_saved_bytes(const poetx_layer* L, int64_t T) {
  if (!layer_ok(L) || !tokens_ok(T)) return 0;
  return static_cast<size_t>(T * (L->m + L->n) * act_size(L));
}

size_t poetx_wbuf_bytes(const poetx_layer* L) {
  if (!layer_ok(L)) return 0;
  return static_cast<size_t>(L->m * L->n * w_size(L));
}

size_t poetx_workspace_bytes(const poetx_layer* L, int64_t T, int op) {
  if (!layer_ok(L) || !tokens_ok(T)) return 0;
  return ws_bytes_for(L, T, op);
}

int poetx_cnp_build(const poetx_layer* L, const float* q_r, const float* q_p, void* g_r, void* g_p, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  if (!layer_ok(L)) return POETX_EINVAL;
  if ((q_r == nullptr) != (g_r == nullptr) || (q_p == nullptr) != (g_p == nullptr)) return POETX_EINVAL;
  for (const void* p : {static_cast<const void*>(q_r), static_cast<const void*>(q_p), static_cast<const void*>(g_r),
                        static_cast<const void*>(g_p)})
    if (p && !aligned16(p)) return POETX_EINVAL;
  if (const int e = check_ws(L, 0, POETX_OP_CNP_BUILD, ws, ws_bytes)) return e;
  clear_pending_error();
  bool ok = true;
  const Side R = side_of(L, POETX_SIDE_R), P = side_of(L, POETX_SIDE_P);
  if (q_r && q_p && R.b == P.b) {
    ProfScope p("cnp_build", stream);
    ok = cnp_group(L, group_of(R, P), q_r, q_p, g_r, g_p, ws, stream);
  } else {
    if (q_r) {
      ProfScope p("cnp_build_r", stream);
      ok = ok && cnp_group(L, group_of(R), q_r, nullptr, g_r, nullptr, ws, stream);
    }
    if (q_p) {
      ProfScope p("cnp_build_p", stream);
      ok = ok && cnp_group(L, group_of(P), q_p, nullptr, g_p, nullptr, ws, stream);
    }
  }
  if (!ok) return POETX_EUNSUPPORTED;
  return launch_status();
}

int poetx_weight_prepare(const poetx_layer* L, const void* w0, const float* w_scale, const int32_t* perm_r,
                         const int32_t* perm_p, void* wp, float* wscale_p, hipStream_t stream) {
  if (!layer_ok(L)) return POETX_EINVAL;
  if (!ptrs_ok({w0, perm_r, perm_p, wp})) return POETX_EINVAL;
  const bool i8 = quantized(L);
  if (i8 && !ptrs_ok({w_scale, wscale_p})) return POETX_EINVAL;
  clear_pending_error();
  {
    ProfScope p("prepare_permute", stream);
    if (!gather_cols(w0, L->n, perm_r, wp, L->n, nullptr, perm_p, L->n, L->m, w_size(L), stream))
      return POETX_EUNSUPPORTED;
    if (i8) gather_f32(w_scale, perm_p, wscale_p, L->n, stream);
  }
  return launch_status();
}

int poetx_weight_export(const poetx_layer* L, const void* wp, const float* wscale_p, const int32_t* perm_r,
                        const int32_t* perm_p, void* w0, float* w_scale, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  if (!layer_ok(L)) return POETX_EINVAL;
  if (!ptrs_ok({wp, perm_r, perm_p, w0})) return POETX_EINVAL;
  const bool i8 = quantized(L);
  if (i8 && !ptrs_ok({wscale_p, w_scale})) return POETX_EINVAL;
  if (const int e = check_ws(L, 0, POETX_OP_WEIGHT_EXPORT, ws, ws_bytes)) return e;
  clear_pending_error();
  // W0[perm_r[i]][c] = Wp[i][inv_p[c]], w_scale[c] = wscale_p[inv_p[c]]
  int32_t* inv_p = static_cast<int32_t*>(ws);
  {
    ProfScope p("export_permute", stream);
    inverse_perm(perm_p, inv_p, L->n, stream);
    if (!gather_cols(wp, L->n, nullptr, w0, L->n, perm_r, inv_p, L->n, L->m, w_size(L), stream))
      return POETX_EUNSUPPORTED;
    if (i8) gather_f32(wscale_p, inv_p, w_scale, L->n, stream);
  }
  return launch_status();
}

int poetx_forward(const poetx_layer* L, int64_t T, const void* x, const int32_t* perm_r, const int32_t* perm_p,
                  const void* g_r, const void* g_p, const void* wp, const float* wscale_p, void* z, void* saved,
                  void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!layer_ok(L) || !tokens_ok(T)) return POETX_EINVAL;
  if (T == 0) return POETX_OK;
  if (!ptrs_ok({x, perm_r, perm_p, g_r, g_p, wp, z, saved})) return POETX_EINVAL;
  if (quantized(L) && (!wscale_p || !aligned16(wscale_p))) return POETX_EINVAL;
  if (const int e = check_ws(L, T, POETX_OP_FORWARD, ws, ws_bytes)) return e;
  clear_pending_error();
  Carve c(ws);
  const FwdWs w = plan_fwd(L, T, c);
  void* X1 = saved;
  void* Y1 = static_cast<char*>(saved) + T * L->m * act_size(L);
  if (!forward_core(L, T, x, perm_r, perm_p, g_r, g_p, wp, wscale_p, z, X1, Y1, w, false, stream))
    return POETX_EUNSUPPORTED;
  return launch_status();
}

int poetx_forward_mem(const poetx_layer* L, int64_t T, const void* x, const int32_t* perm_r,
                      const int32_t* perm_p, const void* g_r, const void* g_p, const void* wp,
                      const float* wscale_p, void* z, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!layer_ok(L) || !tokens_ok(T)) return POETX_EINVAL;
  if (T == 0) return POETX_OK;
  if (!ptrs_ok({x, perm_r, perm_p, g_r, g_p, wp, z})) return POETX_EINVAL;
  if (quantized(L) && (!wscale_p || !aligned16(wscale_p))) return POETX_EINVAL;
  if (const int e = check_ws(L, T, POETX_OP_FORWARD_MEM, ws, ws_bytes)) return e;
  clear_pending_error();
  Carve c(ws);
  char* X1 = c.take<char>(saved_region(L, T));
  char* Y1 = X1 + T * L->m * act_size(L);
  const FwdWs w = plan_fwd(L, T, c);
  if (!forward_core(L, T, x, perm_r, perm_p, g_r, g_p, wp, wscale_p, z, X1, Y1, w, false, stream))
    return POETX_EUNSUPPORTED;
  return launch_status();
}

int poetx_backward(const poetx_layer* L, int64_t T, const void* saved, const void* dz, const int32_t* perm_r,
                   const int32_t* perm_p, const float* q_r, const float* q_p, const void* g_r, const void* g_p,
                   const void* wp, const float* wscale_p, float* dq_r, float* dq_p, void* dx, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  if (!layer_ok(L) || !tokens_ok(T)) return POETX_EINVAL;
  if (!ptrs_ok({dq_r, dq_p})) return POETX_EINVAL;
  const Side R = side_of(L, POETX_SIDE_R), P = side_of(L, POETX_SIDE_P);
  clear_pending_error();
  if (T == 0) {
    fill_zero2_f32(dq_r, packed_len(R), dq_p, packed_len(P), stream);
    return launch_status();
  }
  if (!ptrs_ok({saved, dz, perm_r, perm_p, q_r, q_p, g_r, g_p, wp, dx})) return POETX_EINVAL;
  if (quantized(L) && (!wscale_p || !aligned16(wscale_p))) return POETX_EINVAL;
  if (const int e = check_ws(L, T, POETX_OP_BACKWARD, ws, ws_bytes)) return e;
  Carve c(ws);
  const BwdWs w = plan_bwd(L, T, c);
  void* cnp_ws = static_cast<char*>(ws) + w.cnp_off;
  const void* X1 = saved;
  const void* Y1 = static_cast<const char*>(saved) + T * L->m * act_size(L);
  if (!backward_core(L, T, X1, Y1, dz, perm_r, perm_p, q_r, q_p, g_r, g_p, wp, wscale_p, dq_r, dq_p, dx, w,
                     cnp_ws, stream))
    return POETX_EUNSUPPORTED;
  return launch_status();
}

int poetx_backward_mem(const poetx_layer* L, int64_t T, const void* x, const void* dz, const int32_t* perm_r,
                       const int32_t* perm_p, const float* q_r, const float* q_p, const void* g_r,
                       const void* g_p, const void* wp, const float* wscale_p, float* dq_r, float* dq_p, void* dx,
                       void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!layer_ok(L) || !tokens_ok(T)) return POETX_EINVAL;
  if (!ptrs_ok({dq_r, dq_p})) return POETX_EINVAL;
  const Side R = side_of(L, POETX_SIDE_R), P = side_of(L, POETX_SIDE_P);
  clear_pending_error();
  if (T == 0) {
    fill_zero2_f32(dq_r, packed_len(R), dq_p, packed_len(P), stream);
    return launch_status();
  }
  if (!ptrs_ok({x, dz, perm_r, perm_p, q_r, q_p, g_r, g_p, wp, dx})) return POETX_EINVAL;
  if (quantized(L) && (!wscale_p || !aligned16(wscale_p))) return POETX_EINVAL;
  if (const int e = check_ws(L, T, POETX_OP_BACKWARD_MEM, ws, ws_bytes)) return e;
  Carve c(ws);
  char* X1 = c.take<char>(saved_region(L, T));
  char* Y1 = X1 + T * L->m * act_size(L);
  // the recompute's scratch and the backward's start at the same offset: the
  // recompute is done (in stream order) before the backward touches it
  Carve f = c, b = c;
  const FwdWs fw = plan_fwd(L, T, f);
  const BwdWs w = plan_bwd(L, T, b);
  void* cnp_ws = static_cast<char*>(ws) + w.cnp_off;
  if (!forward_core(L, T, x, perm_r, perm_p, g_r, g_p, wp, wscale_p, nullptr, X1, Y1, fw, true, stream))
    return POETX_EUNSUPPORTED;
  if (!backward_core(L, T, X1, Y1, dz, perm_r, perm_p, q_r, q_p, g_r, g_p, wp, wscale_p, dq_r, dq_p, dx, w,
                     cnp_ws, stream))
    return POETX_EUNSUPPORTED;
  return launch_status();
}

int poetx_merge(const poetx_layer* L, void* wp, float* wscale_p, const int32_t* perm_r, const int32_t* perm_p,
                const int32_t* perm_r_next, const int32_t* perm_p_next, hipEvent_t next_ready, const void* g_r,
                const void* g_p, float* q_r, float* q_p, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!layer_ok(L)) return POETX_EINVAL;
  if (!ptrs_ok({wp, perm_r, perm_p, perm_r_next, perm_p_next, g_r, g_p, q_r, q_p})) return POETX_EINVAL;
  const bool i8 = quantized(L);
  if (i8 && !ptrs_ok({wscale_p})) return POETX_EINVAL;
  if (const int e = check_ws(L, 0, POETX_OP_MERGE, ws, ws_bytes)) return e;
  clear_pending_error();
  const Side R = side_of(L, POETX_SIDE_R), P = side_of(L, POETX_SIDE_P);
  Carve c(ws);
  MergeWs w = plan_merge(L, c);
  // R W0 P = Psi^T Diag(G) Wp Diag(H) Phi with Wp = Psi W0 Phi^T. In the next
  // frame (Psi', Phi') the merged weight is Psi' Psi^T M Phi Phi'^T with
  // M = Diag(G) Wp Diag(H): row i of it is row inv_r[perm_r_next[i]] of M,
  // column c is column inv_p[perm_p_next[c]].
  int wait_status = POETX_OK;
  auto wait_next = [&]() -> bool {
    if (next_ready) {
      const hipError_t e = hipStreamWaitEvent(stream, next_ready, 0);
      if (e != hipSuccess) {
        g_last_hip = e;
        wait_status = POETX_EHIP;
        return false;
      }
    }
    return true;
  };
  // inv_r, inv_p: written by the right block product's launch (workspace
  // only, so a failed wait leaves wp and q as they were)
  SideJob inv_job = inverse_job(perm_r, w.inv_r, L->m);
  inv_job.src1 = perm_p;
  inv_job.dst1 = w.inv_p;
  inv_job.n1 = static_cast<int>(L->n);
  // q <- 0 in the reframe's launch (the merge reads only the CNP planes)
  SideJob zero_q;
  zero_q.z0 = q_r;
  zero_q.nz0 = packed_len(R);
  zero_q.z1 = q_p;
  zero_q.nz1 = packed_len(P);
  bool ok;
  if (i8) {
    // Dequantize Wp with its column scales, merge in float with float copies
    // of the (G - I) planes, gather into the next frame, store per column
    // again.
    poetx_layer Lf = *L;
    Lf.act_dtype = POETX_F32;
    Lf.w_dtype = POETX_F32;
    {
      ProfScope p("merge_dequant", stream);
      ok = dequant_i8_cols(static_cast<const int8_t*>(wp), wscale_p, nullptr, static_cast<float*>(w.C1), L->m,
                           L->n, stream, fp8_weight(L));
      bf16_to_f32(static_cast<const uint16_t*>(g_r), w.gr32, 2 * block_elems(R), stream);
      bf16_to_f32(static_cast<const uint16_t*>(g_p), w.gp32, 2 * block_elems(P), stream);
    }
    {
      ProfScope p("merge_left", stream);
      ok = ok && transpose(w.C1, w.C2, L->m, L->n, 4, stream);
      ok = ok && block_apply(&Lf, R, L->n, w.C2, w.C1, w.gr32, 0, nullptr, stream);
    }
    {
      ProfScope p("merge_transpose", stream);
      ok = ok && transpose(w.C1, w.C2, L->n, L->m, 4, stream);
    }
    {
      ProfScope p("merge_right", stream);
      ok = ok && block_apply(&Lf, P, L->m, w.C2, w.C1, w.gp32, 1, nullptr, stream, inv_job);
    }
    {
      ProfScope p("merge_reframe", stream);
      ok = ok && wait_next();
      ok = ok && reframe_rows_cols(w.C1, w.inv_r, perm_r_next, w.C2, w.inv_p, perm_p_next, w.rmap, w.cmap, L->n,
                                   L->m, 4, stream, zero_q);
    }
    {
      ProfScope p("merge_requant", stream);
      ok = ok && requant_i8_cols(static_cast<const float*>(w.C2), w.amax, static_cast<int8_t*>(wp), wscale_p, L->m,
                                 L->n, stream, fp8_weight(L));
    }
    if (wait_status) return wait_status;
    if (!ok) return POETX_EUNSUPPORTED;
    return launch_status();
  }
  void* M;  // Diag(G) Wp Diag(H), m x n
  if (is_bf16(L) && R.b == 256) {
    // the left block product on the rows of Wp, then Diag(H) on the right
    {
      ProfScope p("merge_left", stream);
      ok = block_apply_left_bf16(static_cast<const uint16_t*>(wp), static_cast<uint16_t*>(w.C2), L->n,
                                 static_cast<const uint16_t*>(plane(L, g_r, R, 0)), L->m, L->n, R.b, stream);
    }
    {
      ProfScope p("merge_right", stream);
      ok = ok && block_apply(L, P, L->m, w.C2, w.C1, g_p, 1, nullptr, stream, inv_job);
    }
    M = w.C1;
  } else {
    // Diag(G) Wp = (Wp^T Diag(G)^T)^T: a right block product on the rows of
    // Wp^T with the (G - I) plane between two transposes
    {
      ProfScope p("merge_left", stream);
      ok = transpose(wp, w.C1, L->m, L->n, w_size(L), stream);
      ok = ok && block_apply(L, R, L->n, w.C1, w.C2, g_r, 0, nullptr, stream);
    }
    {
      ProfScope p("merge_transpose", stream);
      ok = ok && transpose(w.C2, w.C1, L->n, L->m, w_size(L), stream);
    }
    {
      ProfScope p("merge_right", stream);
      ok = ok && block_apply(L, P, L->m, w.C1, w.C2, g_p, 1, nullptr, stream, inv_job);
    }
    M = w.C2;
  }
  {
    ProfScope p("merge_reframe", stream);
    ok = ok && wait_next();
    ok = ok && reframe_rows_cols(M, w.inv_r, perm_r_next, wp, w.inv_p, perm_p_next, w.rmap, w.cmap, L->n, L->m,
                                 w_size(L), stream, zero_q);
  }
  if (wait_status) return wait_status;
  if (!ok) return POETX_EUNSUPPORTED;
  return launch_status();
}

int poetx_sample_perm(int64_t dim, uint64_t seed, uint64_t tag, uint64_t draw, int32_t* perm, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  if (dim < 1 || !perm || !aligned16(perm)) return POETX_EINVAL;
  if (dim > kMaxPermDim) return POETX_EUNSUPPORTED;
  if (ws_bytes < perm_ws_bytes(dim)) return POETX_EWORKSPACE;
  if (!ws || !aligned16(ws)) return POETX_EINVAL;
  clear_pending_error();
  {
    ProfScope p("sample_perm", stream);
    if (!sample_perm(dim, seed, tag, draw, perm, static_cast<uint64_t*>(ws), stream)) return POETX_EUNSUPPORTED;
  }
  return launch_status();
}

int poetx_sample_perm_static(int64_t dim, uint64_t seed, uint64_t tag, uint64_t draw, int32_t* perm,
                             hipStream_t stream) {
  if (dim < 1 || !perm || !aligned16(perm)) return POETX_EINVAL;
  if (dim > kMaxPermDim) return POETX_EUNSUPPORTED;
  clear_pending_error();
  uint64_t* keys = nullptr;
  if (const int e = static_scratch(stream, &keys)) return e;
  {
    ProfScope p("sample_perm", stream);
    if (!sample_perm(dim, seed, tag, draw, perm, keys, stream)) return POETX_EUNSUPPORTED;
  }
  return launch_status();
}

int poetx_profile_enable(int enable) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  if (enable) {
    for (const ProfRec& r : g_prof) {
      g_prof_pool.push_back(r.start);
      g_prof_pool.push_back(r.stop);
    }
    g_prof.clear();
  }
  g_prof_on = enable != 0;
  return POETX_OK;
}

int poetx_profile_count(void) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  return static_cast<int>(g_prof.size());
}

int poetx_profile_get(int i, const char** name, float* ms) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  if (i < 0 || i >= static_cast<int>(g_prof.size()) || !name || !ms) return POETX_EINVAL;
  const ProfRec& r = g_prof[static_cast<size_t>(i)];
  if (hipEventSynchronize(r.stop) != hipSuccess) return POETX_EHIP;
  float t = 0.f;
  if (hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess) return POETX_EHIP;
  *name = r.name;
  *ms = t;
  return POETX_OK;
}

}  // extern "C"
