/*
 * poetx.h - C ABI of libpoetx.so: the POET-X reparameterized linear layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (zhichai.net digest of arXiv:2603.05500, sections
 * "1. 输入中心化架构", "2. 块随机正交变换", "3. Cayley-Neumann 参数化优化"):
 *
 *   z = P^T (W0^T (R^T x)),  R = Psi^T Diag(G_1..G_ceil(m/b)) Psi,
 *                            P = Phi^T Diag(H_1..H_ceil(n/b)) Phi,
 *   G_j = (I + Q_j)(I + Q_j + Q_j^2 + Q_j^3),  Q_j skew, stored as its packed
 *   strict upper triangle (b(b-1)/2 floats per block).
 *
 * Row form used throughout: a batch X (T tokens x m features, row-major) maps
 * to Z = X R W0 P (T x n). W0 is m x n and frozen; only the packed q_R, q_P
 * are trained. Psi[i, perm_r[i]] = 1, i.e. (X Psi^T)[:, i] = X[:, perm_r[i]].
 * Block j covers permuted indices [j*b, min((j+1)*b, dim)); only the last
 * block can be shorter. Block j's packed parameters start at j*b(b-1)/2 and
 * list Q_j[i][l], i < l, in row-major order (Q_j[l][i] = -Q_j[i][l]).
 *
 * Conventions shared by every entry point:
 *  - Every pointer is a device pointer owned by the caller (hipMalloc or a
 *    torch CUDA tensor). The library allocates no device memory and keeps no
 *    state between calls apart from the optional timing log below; scratch
 *    memory is the caller's workspace `ws`.
 *  - Everything is asynchronous and stream-ordered on `stream`; no entry point
 *    synchronises the host. Inputs are read-only unless stated otherwise.
 *  - Arguments are validated before any launch: on any error nothing is
 *    launched and no output is touched. POETX_EHIP reports a failed launch.
 *  - Element types: `act_dtype` (x, z, dz, dx, saved activations, the CNP
 *    block buffers) is POETX_F32 or POETX_BF16. `w_dtype` is POETX_F32 with
 *    F32 activations, POETX_BF16, POETX_I8 or POETX_F8 with BF16 activations
 *    (I8 = int8 weight with one float scale per output column: W0[r][c] =
 *    s[c] * q[r][c], the quantised-base-weight variant POET-XQ of section
 *    "POET-XQ"; F8 = the same with q[r][c] an OCP E4M3 fp8 byte (sign, 4-bit
 *    exponent with bias 7, 3-bit mantissa; largest finite 448; the NaN
 *    bytes 0x7F / 0xFF are never stored), the lower-precision format the
 *    section expects to work as well).
 *  - Shapes: m, n, b_r, b_p multiples of 8 (m, n multiples of 16 for I8 and
 *    of 64 for F8); 8 <= b <= 1024; m, n <= 2^24;
 *    ceil(m / b_r) + ceil(n / b_p) <= 65535 blocks; 0 <= T <= 2^30 tokens.
 *    Outside these the entry points return POETX_EINVAL and the size queries
 *    return 0.
 *  - Permutations must be permutations of [0, dim). Out-of-range entries are
 *    not reported, but every index is clamped, so a bad permutation gives
 *    wrong values, never an access outside the buffers.
 */
#ifndef POETX_H
#define POETX_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define POETX_API __attribute__((visibility("default")))
#else
#define POETX_API
#endif

#define POETX_ABI_VERSION 2

enum {
  POETX_OK = 0,
  POETX_EINVAL = 1,        /* bad pointer, shape, dtype or size */
  POETX_EUNSUPPORTED = 2,  /* valid request the library does not implement */
  POETX_EHIP = 3,          /* a HIP launch failed */
  POETX_EWORKSPACE = 4     /* ws_bytes smaller than poetx_workspace_bytes() */
};

enum { POETX_F32 = 0, POETX_BF16 = 1, POETX_I8 = 2, POETX_F8 = 3 };

enum { POETX_SIDE_R = 0, POETX_SIDE_P = 1 };

enum {
  POETX_OP_CNP_BUILD = 0,
  POETX_OP_WEIGHT_PREPARE = 1,
  POETX_OP_FORWARD = 2,
  POETX_OP_BACKWARD = 3,
  POETX_OP_MERGE = 4,
  POETX_OP_FORWARD_MEM = 5,
  POETX_OP_BACKWARD_MEM = 6,
  POETX_OP_SAMPLE_PERM = 7,
  POETX_OP_WEIGHT_EXPORT = 8
};

typedef struct poetx_layer {
  int64_t m;          /* input features (rows of W0) */
  int64_t n;          /* output features (columns of W0) */
  int32_t b_r;        /* block size of R: ceil(m / b_r) blocks */
  int32_t b_p;        /* block size of P: ceil(n / b_p) blocks */
  int32_t act_dtype;  /* POETX_F32 or POETX_BF16 */
  int32_t w_dtype;    /* POETX_F32, POETX_BF16, POETX_I8 or POETX_F8 (see above) */
} poetx_layer;

/* Version of this ABI (POETX_ABI_VERSION). */
POETX_API int poetx_abi_version(void);

/* Static message for a status code; never NULL. */
POETX_API const char* poetx_strerror(int status);

/* Name and description of the HIP error behind the last POETX_EHIP returned
 * to the calling thread ("hipSuccess: no error" if there was none); never
 * NULL, valid until the thread's next call. The compute entry points clear
 * HIP's per-thread last-error state before they launch, so POETX_EHIP reports
 * errors raised by their own launches only. */
POETX_API const char* poetx_last_hip_error(void);

/* Number of packed float parameters of one side: sum over its blocks of
 * r(r-1)/2 (section "3. Cayley-Neumann 参数化优化"). 0 for an invalid layer. */
POETX_API size_t poetx_packed_len(const poetx_layer* L, int side);

/* Bytes of one side's CNP block buffer (output of poetx_cnp_build): two
 * planes of nblk x b x b elements of act_dtype. Plane 0 holds G_j - I
 * row-major, plane 1 holds (G_j - I)^T row-major; for a short last block of
 * size r, entries with a row or column >= r are zero. 0 for an invalid layer. */
POETX_API size_t poetx_gbuf_bytes(const poetx_layer* L, int side);

/* Bytes of the activations poetx_forward saves for poetx_backward:
 * X1 = X Psi^T (T x m) followed by Y1 = X R W0 Phi^T (T x n), act_dtype,
 * row-major. */
POETX_API size_t poetx_saved_bytes(const poetx_layer* L, int64_t T);

/* Bytes of the permuted-frame weight wp (m x n elements of w_dtype), the one
 * copy of the base weight a layer keeps (section "1. 输入中心化架构": the
 * method adds no second m x n weight). */
POETX_API size_t poetx_wbuf_bytes(const poetx_layer* L);

/* Workspace bytes an operation needs for T tokens (T ignored by CNP build,
 * weight preparation and export, merge and permutation draws). 0 means
 * none. */
POETX_API size_t poetx_workspace_bytes(const poetx_layer* L, int64_t T, int op);

/* CNP build (section "3. Cayley-Neumann 参数化优化": G = (I+Q)(I+Q+Q^2+Q^3),
 * every higher term formed from Q and Q^2).
 *   q_r [poetx_packed_len(L, R)] float, q_p likewise: packed skew parameters.
 *   g_r, g_p: CNP block buffers (poetx_gbuf_bytes), overwritten.
 * Either side may be skipped by passing NULL for both its q and g. */
POETX_API int poetx_cnp_build(const poetx_layer* L, const float* q_r, const float* q_p,
                    void* g_r, void* g_p, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* Permuted-frame base weight from W0 in the original frame (loading a
 * weight or a checkpoint): wp = Psi W0 Phi^T, i.e. wp[i][c] =
 * w0[perm_r[i]][perm_p[c]] (m x n, w_dtype); for I8 and F8 also wscale_p[c] =
 * w_scale[perm_p[c]] (n floats; w_scale and wscale_p are ignored otherwise
 * and may be NULL). wp is the weight every other entry point takes: the
 * forward reads it N-contiguous, the backward K-contiguous, and poetx_merge
 * rewrites it in the frame of the next permutations. w0 may be freed after
 * the call has run. */
POETX_API int poetx_weight_prepare(const poetx_layer* L, const void* w0, const float* w_scale,
                         const int32_t* perm_r, const int32_t* perm_p,
                         void* wp, float* wscale_p, hipStream_t stream);

/* The inverse of poetx_weight_prepare, for checkpoints: w0[perm_r[i]][
 * perm_p[c]] = wp[i][c] (m x n, w_dtype) and, for I8 and F8, w_scale[perm_p[c]] =
 * wscale_p[c]. ws: poetx_workspace_bytes(L, 0, POETX_OP_WEIGHT_EXPORT)
 * bytes (n int32). With q = 0 (right after a merge) the layer's function is
 * x -> x w0, whatever the permutations. */
POETX_API int poetx_weight_export(const poetx_layer* L, const void* wp, const float* wscale_p,
                        const int32_t* perm_r, const int32_t* perm_p,
                        void* w0, float* w_scale, void* ws, size_t ws_bytes, hipStream_t stream);

/* Forward, input-centric (section "1. 输入中心化架构"): Z = X R W0 P without
 * forming R W0 P.
 *   x [T][m], act_dtype. z [T][n], act_dtype, overwritten.
 *   g_r, g_p: CNP block buffers from poetx_cnp_build.
 *   wp: permuted-frame weight (poetx_weight_prepare, poetx_merge);
 *   wscale_p: its column scales (I8 and F8 only, else ignored).
 *   saved: poetx_saved_bytes(L, T) bytes, overwritten with X1 and Y1.
 * An int8 or fp8 weight is dequantised at run time (section "POET-XQ"): the
 * dense product turns its codes into bfloat16 (exact for both formats) on
 * their way into on-chip memory and applies the column scales in its
 * epilogue; for int8 with m or n not a multiple of 64 the codes are first
 * copied to bfloat16 in the workspace.
 * T == 0 launches nothing. */
POETX_API int poetx_forward(const poetx_layer* L, int64_t T, const void* x,
                  const int32_t* perm_r, const int32_t* perm_p,
                  const void* g_r, const void* g_p,
                  const void* wp, const float* wscale_p,
                  void* z, void* saved, void* ws, size_t ws_bytes,
                  hipStream_t stream);

/* Backward of L = <dz, z> for the forward that wrote `saved`:
 *   dq_r, dq_p: packed gradients (float, poetx_packed_len), overwritten.
 *   dx [T][m], act_dtype, overwritten.
 *   q_r, q_p: the packed parameters the CNP buffers were built from.
 *   wp, wscale_p: the forward's permuted-frame weight (m x n).
 * No W0 gradient exists (W0 is frozen). Outputs are overwritten, not
 * accumulated; T == 0 writes zero gradients. When the weight is not I8 or F8 and
 * m < T, the P-side product dY1 = dY2 H^T is not formed: the dense product
 * takes dY2 and the weight Wp H (built in the workspace), which is the same
 * dX2 = dY2 H^T Wp^T with fewer bytes moved. For an I8 or F8 weight, dY1 takes the
 * column scales and the dense product reads Wp's codes, converting them to
 * bfloat16 (exact) itself. */
POETX_API int poetx_backward(const poetx_layer* L, int64_t T, const void* saved, const void* dz,
                   const int32_t* perm_r, const int32_t* perm_p,
                   const float* q_r, const float* q_p,
                   const void* g_r, const void* g_p,
                   const void* wp, const float* wscale_p,
                   float* dq_r, float* dq_p, void* dx,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/* Memory variant (section "三种变体，三种场景", POET-X mem; the pages give no
 * mechanism, the reading here is recomputation): the forward saves nothing
 * and the backward recomputes what it needs from x.
 * poetx_forward_mem: poetx_forward without `saved` (X1 and Y1 go to the
 *   workspace, poetx_workspace_bytes(L, T, POETX_OP_FORWARD_MEM)).
 * poetx_backward_mem: poetx_backward with x in place of `saved`. It recomputes
 *   X1 = X Psi^T, X2 = X1 Diag(G) and Y1 = X2 Wp (the forward's first three
 *   steps, same kernels) into the workspace
 *   (poetx_workspace_bytes(L, T, POETX_OP_BACKWARD_MEM)), then runs the
 *   backward; results equal poetx_backward's for the same inputs.
 *   x [T][m], act_dtype.
 * Costs one more dense product per step and saves poetx_saved_bytes(L, T) of
 * activations per layer. */
POETX_API int poetx_forward_mem(const poetx_layer* L, int64_t T, const void* x,
                      const int32_t* perm_r, const int32_t* perm_p,
                      const void* g_r, const void* g_p,
                      const void* wp, const float* wscale_p,
                      void* z, void* ws, size_t ws_bytes, hipStream_t stream);

POETX_API int poetx_backward_mem(const poetx_layer* L, int64_t T, const void* x, const void* dz,
                       const int32_t* perm_r, const int32_t* perm_p,
                       const float* q_r, const float* q_p,
                       const void* g_r, const void* g_p,
                       const void* wp, const float* wscale_p,
                       float* dq_r, float* dq_p, void* dx,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Merge (section "代码与部署", merge_if_needed): W0 <- R W0 P with the current
 * permutations and blocks, then q_r, q_p <- 0, with the merged weight written
 * straight into the frame of the permutations that follow the merge (the
 * rotations restart from Q = 0, when the layer no longer depends on the
 * permutations, and a training loop draws new ones).
 *   wp [m][n], w_dtype, in-out: in, the permuted-frame weight of perm_r,
 *       perm_p; out, Psi' R W0 P Phi'^T for Psi', Phi' of perm_r_next,
 *       perm_p_next (which may be perm_r, perm_p themselves: no new frame).
 *   wscale_p [n] float, I8 and F8 weights only, in-out: the column scales
 *       of wp. The merged weight is stored again the way W0 was (section
 *       "POET-XQ：量化训练的额外红利" stores the base weight quantized; how a
 *       merged weight is stored again is a reading): per column c, I8:
 *       scale[c] = max_r |W0'[r][c]| / 127 (1 for a zero column) and code =
 *       clamp(rint(W0'[r][c] / scale[c]), -127, 127), rounding half to even
 *       in float32; F8: scale[c] = max_r |W0'[r][c]| / 448 (1 for a zero
 *       column) and code = the E4M3 byte nearest W0'[r][c] / scale[c]
 *       (float32), ties to the even code, magnitudes past 448 saturated.
 *       The merge itself runs in float for both.
 *   next_ready: NULL, or an event the stream waits for (hipStreamWaitEvent)
 *       after the block products and before perm_r_next / perm_p_next are
 *       read, so that their draw can run on another stream beside the block
 *       products. If that wait cannot be enqueued, POETX_EHIP is returned
 *       with the block products launched but wp and q untouched.
 *   g_r, g_p: the CNP block buffers of q_r, q_p.
 * The caller then builds the CNP blocks of q = 0 and uses perm_r_next,
 * perm_p_next from here on. */
POETX_API int poetx_merge(const poetx_layer* L, void* wp, float* wscale_p,
                const int32_t* perm_r, const int32_t* perm_p,
                const int32_t* perm_r_next, const int32_t* perm_p_next, hipEvent_t next_ready,
                const void* g_r, const void* g_p, float* q_r, float* q_p,
                void* ws, size_t ws_bytes, hipStream_t stream);

/* Draw of a uniformly random permutation of [0, dim) for Psi or Phi. The
 * permutations are random (section "2. 块随机正交变换"); a merge restarts
 * the rotations every merge_interval steps (section "代码与部署"), and a
 * training loop then draws both permutations again. Index i's key is the top
 * 44 bits of word (i mod 4) of Philox4x64-10 (Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011) at counter
 * (i div 4, draw, 0, 0) under key (seed, tag); perm lists the indices in
 * ascending order of (key, index). The same (dim, seed, tag, draw) gives the
 * same permutation on every device and in every process.
 *   seed: run seed; tag: separates layers and the two sides; draw: number of
 *       the draw (0 = initial, k = after the k-th merge).
 *   perm [dim] int32, overwritten.
 *   ws: at least 8 * dim bytes of scratch (poetx_workspace_bytes(L, 0,
 *       POETX_OP_SAMPLE_PERM) covers both sides of a layer L).
 * 1 <= dim <= 2^20 (POETX_EUNSUPPORTED above). Up to dim = 15360 the draw
 * runs in one workgroup and leaves ws untouched (its keys stay in on-chip
 * memory, the work grows as dim); wider draws rank each index by counting
 * smaller keys over the whole GPU, and their work grows as dim^2. */
POETX_API int poetx_sample_perm(int64_t dim, uint64_t seed, uint64_t tag, uint64_t draw,
                      int32_t* perm, void* ws, size_t ws_bytes, hipStream_t stream);

/* poetx_sample_perm without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that
 * forbid hipMalloc). Same arguments, draw and result as poetx_sample_perm,
 * but the keys go to a scratch array inside the library: 2^20 64-bit words
 * (8 MiB) per device, held by each device the library runs on until the
 * process ends. The call allocates nothing.
 *   dim: 1 <= dim <= 2^20, the scratch's size (POETX_EUNSUPPORTED above it,
 *       POETX_EINVAL below 1 or for a null or unaligned perm).
 *   perm [dim] int32, overwritten.
 * The device is the one that runs `stream` (the current device for the null
 * stream). The first call on a device looks up the scratch's device address
 * (POETX_EHIP if that fails); make it outside graph capture. All calls on one
 * device share the scratch: calls that can overlap on one device (different
 * streams without ordering between them, host threads) race and may return
 * wrong permutations. Calls ordered on one stream are safe: nothing in the
 * scratch carries over from one call to the next. */
POETX_API int poetx_sample_perm_static(int64_t dim, uint64_t seed, uint64_t tag, uint64_t draw,
                                       int32_t* perm, hipStream_t stream);

/* Kernel timing log (tracing). poetx_profile_enable(1) clears the log and
 * starts recording: from then on every step of every entry point (e.g.
 * "gemm_dense_fwd", "apply_p_bwd", "grad_h", "cnp_build_r") is bracketed by a
 * pair of HIP events recorded on the caller's stream. poetx_profile_enable(0)
 * stops recording (the log is kept). The log is process-wide and guarded by a
 * mutex; it is the only state the library keeps between calls. */
POETX_API int poetx_profile_enable(int enable);

/* Number of steps recorded since the last poetx_profile_enable call. */
POETX_API int poetx_profile_count(void);

/* Name (static string) and elapsed milliseconds of recorded step i; waits
 * for that step's stop event. POETX_EINVAL for i out of range. */
POETX_API int poetx_profile_get(int i, const char** name, float* ms);

#ifdef __cplusplus
}
#endif

#endif /* POETX_H */
