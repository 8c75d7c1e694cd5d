"""POET-X layer, float64 NumPy reference (test infrastructure, CPU only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use this
module. Nothing here is shared with the HIP library.

Source of every formula: the zhichai.net digest of arXiv:2603.05500 (page title
"POET-X：单卡H100训练130亿参数模型..."). Sections cited below:
  [IC]  "1. 输入中心化架构" - the layer output z = P^T (W^T (R^T x)) evaluated
        input-first, versus the weight-first z = (R W0 P)^T x of original POET.
  [BS]  "2. 块随机正交变换" - R = Psi^T Diag(G_1, ..., G_ceil(m/b)) Psi with b x b
        orthogonal blocks G_j and a random permutation matrix Psi.
  [CNP] "3. Cayley-Neumann 参数化优化" - G = (I+Q)(I+Q+Q^2+Q^3) with Q skew, only
        the b(b-1)/2 upper-triangle entries of Q stored.
  [MG]  "代码与部署" - the training loop calls merge_if_needed(step) every
        merge_interval steps: W0 absorbs R and P, and the rotations restart.
  [XQ]  "POET-XQ：量化训练的额外红利" - base weight stored quantized and
        dequantized at run time.

Conventions (readings where the page is silent; all listed in the design notes):
  * Row form.  A batch X (T x m, one token per row) maps to Z = X R W0 P
    (T x n), the transpose of [IC]'s column form z = P^T W0^T R^T x.
  * Permutation.  perm is an int array with Psi[i, perm[i]] = 1, so
    (X Psi^T)[:, i] = X[:, perm[i]] (a column gather) and
    (V Psi)[:, perm[i]] = V[:, i] (a column scatter).
  * P has the same form as R: P = Phi^T Diag(H_1..H_ceil(n/b)) Phi.
  * Blocks.  Block j covers permuted indices [j*b, min((j+1)*b, dim)); only the
    last block can be smaller (ceil(dim/b) blocks, [BS]).
  * Packing.  Block j's parameters start at j*b*(b-1)/2 and hold the strict
    upper triangle of Q_j in row-major order (numpy.triu_indices(r, 1)):
    Q[i, l] = q[k], Q[l, i] = -q[k] for i < l, zero diagonal ([CNP]).
  * Gradients are for the scalar L = <dZ, Z> (ordinary back-propagation of the
    upstream gradient dZ). W0 is frozen, so it has none.
"""

import numpy as np

__all__ = [
    "block_sizes", "packed_offsets", "packed_len", "skew_from_packed",
    "project_to_packed", "cnp", "cnp_adjoint", "cnp_blocks", "gather_cols",
    "scatter_cols", "block_diag_right", "block_diag_left", "permutation_matrix",
    "dense_block_orthogonal", "dequantize", "permuted_weight", "forward",
    "backward", "backward_blocks", "merge", "weight_centric_forward", "inner",
    "requantize_int8_per_col", "merge_xq", "philox4x64_10", "perm_words",
    "FP8_MAX", "fp8_e4m3_values", "fp8_e4m3_decode", "fp8_e4m3_encode",
    "dequantize_fp8", "requantize_fp8_per_col",
    "perm_keys", "sample_perm", "merge_due", "PERM_KEY_BITS",
]


# ----------------------------------------------------------------------------
# block structure and packed storage  ([BS], [CNP])
# ----------------------------------------------------------------------------

def block_sizes(dim, b):
    """Sizes of the ceil(dim/b) diagonal blocks of R (or P) [BS]."""
    nblk = -(-dim // b)
    return [b] * (nblk - 1) + [dim - (nblk - 1) * b]


def packed_offsets(dim, b):
    """Start of each block's packed parameters; block j starts at j*b(b-1)/2."""
    sizes = block_sizes(dim, b)
    offs = [j * (b * (b - 1) // 2) for j in range(len(sizes))]
    return offs, sizes


def packed_len(dim, b):
    """Total packed parameter count: sum over blocks of r(r-1)/2 [CNP]."""
    return sum(r * (r - 1) // 2 for r in block_sizes(dim, b))


def skew_from_packed(qblk, r):
    """Skew-symmetric Q (r x r) from its packed strict upper triangle [CNP]."""
    qblk = np.asarray(qblk, dtype=np.float64)
    assert qblk.shape == (r * (r - 1) // 2,)
    Q = np.zeros((r, r), dtype=np.float64)
    iu = np.triu_indices(r, 1)
    Q[iu] = qblk
    Q[(iu[1], iu[0])] = -qblk
    return Q


def project_to_packed(M):
    """Gradient w.r.t. the packed entries given the gradient M w.r.t. Q.

    Entry k sits at Q[i, l] with sign + and at Q[l, i] with sign -, so
    dL/dq_k = M[i, l] - M[l, i].
    """
    M = np.asarray(M, dtype=np.float64)
    iu = np.triu_indices(M.shape[0], 1)
    return M[iu] - M.T[iu]


# ----------------------------------------------------------------------------
# Cayley-Neumann map and its adjoint  ([CNP])
# ----------------------------------------------------------------------------

def cnp(Q):
    """G = (I + Q)(I + Q + Q^2 + Q^3), written as the page's product [CNP]."""
    Q = np.asarray(Q, dtype=np.float64)
    I = np.eye(Q.shape[0])
    Q2 = Q @ Q
    Q3 = Q2 @ Q
    return (I + Q) @ (I + Q + Q2 + Q3)


def cnp_adjoint(Q, U):
    """dL/dQ for dL/dG = U, by the product rule on G = A S [CNP].

    A = I + Q, S = I + Q + Q^2 + Q^3.  With <U, dG> = <U S^T, dA> + <A^T U, dS>
    and dS = dQ + dQ Q + Q dQ + dQ Q^2 + Q dQ Q + Q^2 dQ, moving every factor
    to the other side of the inner product gives, with V = A^T U,
      dL/dQ = U S^T + V + V Q^T + Q^T V + V Q^T Q^T + Q^T V Q^T + Q^T Q^T V.
    Q is treated as an unconstrained matrix here; project_to_packed() then
    applies the skew constraint.
    """
    Q = np.asarray(Q, dtype=np.float64)
    U = np.asarray(U, dtype=np.float64)
    I = np.eye(Q.shape[0])
    A = I + Q
    S = I + Q + Q @ Q + Q @ Q @ Q
    V = A.T @ U
    Qt = Q.T
    return (U @ S.T + V + V @ Qt + Qt @ V + V @ Qt @ Qt + Qt @ V @ Qt
            + Qt @ Qt @ V)


def cnp_blocks(q, dim, b):
    """All G_j of one side from its packed parameters [BS], [CNP]."""
    q = np.asarray(q, dtype=np.float64)
    offs, sizes = packed_offsets(dim, b)
    assert q.shape == (packed_len(dim, b),)
    out = []
    for o, r in zip(offs, sizes):
        out.append(cnp(skew_from_packed(q[o:o + r * (r - 1) // 2], r)))
    return out


# ----------------------------------------------------------------------------
# permutations and block-diagonal products  ([BS])
# ----------------------------------------------------------------------------

def gather_cols(V, perm):
    """V Psi^T: out[:, i] = V[:, perm[i]]."""
    return np.asarray(V)[:, np.asarray(perm)]


def scatter_cols(V, perm):
    """V Psi: out[:, perm[i]] = V[:, i]."""
    V = np.asarray(V)
    out = np.empty_like(V)
    out[:, np.asarray(perm)] = V
    return out


def block_diag_right(V, blocks, b):
    """V Diag(B_0, B_1, ...) for V with one column per permuted index."""
    V = np.asarray(V, dtype=np.float64)
    out = np.empty_like(V)
    for j, B in enumerate(blocks):
        s = j * b
        e = s + B.shape[0]
        out[:, s:e] = V[:, s:e] @ B
    return out


def block_diag_left(blocks, V, b):
    """Diag(B_0, B_1, ...) V for V with one row per permuted index."""
    V = np.asarray(V, dtype=np.float64)
    out = np.empty_like(V)
    for j, B in enumerate(blocks):
        s = j * b
        e = s + B.shape[0]
        out[s:e, :] = B @ V[s:e, :]
    return out


def permutation_matrix(perm):
    """Psi with Psi[i, perm[i]] = 1 (dense; small sizes only)."""
    perm = np.asarray(perm)
    Psi = np.zeros((perm.size, perm.size))
    Psi[np.arange(perm.size), perm] = 1.0
    return Psi


def dense_block_orthogonal(blocks, perm, b):
    """R = Psi^T Diag(G_0, ...) Psi as a dense matrix [BS] (small sizes only)."""
    dim = len(perm)
    D = np.zeros((dim, dim))
    for j, B in enumerate(blocks):
        s = j * b
        e = s + B.shape[0]
        D[s:e, s:e] = B
    Psi = permutation_matrix(perm)
    return Psi.T @ D @ Psi


# ----------------------------------------------------------------------------
# base weight  ([XQ], and the permuted frame used by the library)
# ----------------------------------------------------------------------------

def dequantize(Wq, scale):
    """Run-time dequantization of a per-output-column int8 base weight [XQ]:
    W0[r, c] = scale[c] * Wq[r, c]."""
    return np.asarray(Wq, dtype=np.float64) * np.asarray(scale, np.float64)[None, :]


def permuted_weight(W0, perm_r, perm_p):
    """Psi W0 Phi^T: W0 with rows in perm_r order and columns in perm_p order."""
    W0 = np.asarray(W0)
    return W0[np.asarray(perm_r)][:, np.asarray(perm_p)]


# ----------------------------------------------------------------------------
# the layer  ([IC], [BS], [CNP], [MG])
# ----------------------------------------------------------------------------

def forward(X, W0, q_r, q_p, perm_r, perm_p, b_r, b_p):
    """Input-centric forward Z = ((X R) W0) P, never forming R W0 P [IC].

    Returns every intermediate: X1 = X Psi^T, X2 = X1 Diag(G), X3 = X2 Psi,
    Y = X3 W0, Y1 = Y Phi^T, Y2 = Y1 Diag(H), Z = Y2 Phi, plus the blocks.
    """
    X = np.asarray(X, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    m, n = W0.shape
    assert X.shape[1] == m
    G = cnp_blocks(q_r, m, b_r)
    H = cnp_blocks(q_p, n, b_p)
    X1 = gather_cols(X, perm_r)
    X2 = block_diag_right(X1, G, b_r)
    X3 = scatter_cols(X2, perm_r)
    Y = X3 @ W0
    Y1 = gather_cols(Y, perm_p)
    Y2 = block_diag_right(Y1, H, b_p)
    Z = scatter_cols(Y2, perm_p)
    return dict(Z=Z, X1=X1, X2=X2, X3=X3, Y=Y, Y1=Y1, Y2=Y2, G=G, H=H)


def backward(X, dZ, W0, q_r, q_p, perm_r, perm_p, b_r, b_p):
    """Gradients of L = <dZ, Z> w.r.t. q_r, q_p and X, by reverse-mode
    differentiation of forward() step by step [IC], [BS], [CNP].

    W0 is frozen, so there is no X^T dZ weight-gradient product; the block
    gradients are token sums dG_j = X1_J^T dX2_J and dH_k = Y1_K^T dY2_K.
    """
    X = np.asarray(X, dtype=np.float64)
    dZ = np.asarray(dZ, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    m, n = W0.shape
    f = forward(X, W0, q_r, q_p, perm_r, perm_p, b_r, b_p)
    G, H = f["G"], f["H"]
    # Z = Y2 Phi  ->  dY2 = dZ Phi^T (gather)
    dY2 = gather_cols(dZ, perm_p)
    # Y2 = Y1 Diag(H)
    dH = []
    for k, Hk in enumerate(H):
        s = k * b_p
        e = s + Hk.shape[0]
        dH.append(f["Y1"][:, s:e].T @ dY2[:, s:e])
    dY1 = block_diag_right(dY2, [Hk.T for Hk in H], b_p)
    # Y1 = Y Phi^T  ->  dY = dY1 Phi (scatter)
    dY = scatter_cols(dY1, perm_p)
    # Y = X3 W0
    dX3 = dY @ W0.T
    # X3 = X2 Psi  ->  dX2 = dX3 Psi^T (gather)
    dX2 = gather_cols(dX3, perm_r)
    # X2 = X1 Diag(G)
    dG = []
    for j, Gj in enumerate(G):
        s = j * b_r
        e = s + Gj.shape[0]
        dG.append(f["X1"][:, s:e].T @ dX2[:, s:e])
    dX1 = block_diag_right(dX2, [Gj.T for Gj in G], b_r)
    # X1 = X Psi^T  ->  dX = dX1 Psi (scatter)
    dX = scatter_cols(dX1, perm_r)
    # G_j = cnp(Q_j(q))  ->  packed gradients
    dq_r = _packed_grad(q_r, m, b_r, dG)
    dq_p = _packed_grad(q_p, n, b_p, dH)
    return dict(dq_r=dq_r, dq_p=dq_p, dX=dX, dG=dG, dH=dH, dY2=dY2, dY1=dY1,
                dX2=dX2, dX1=dX1, fwd=f)


def backward_blocks(X, dZ, W0, q_r, q_p, perm_r, perm_p, b_r, b_p, blocks_r, blocks_p):
    """Packed gradients of chosen blocks only, for sizes where backward() is
    too costly. Same steps as backward(), restricted to the needed columns:
    dH_k = Y1_K^T dY2_K with Y1_K = X3 W0[:, perm_p[K]], and
    dG_j = X1_J^T dX2_J with dX2_J = dY W0[perm_r[J], :]^T.
    Returns ({j: dq_r block j}, {k: dq_p block k})."""
    X = np.asarray(X, dtype=np.float64)
    dZ = np.asarray(dZ, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    perm_r, perm_p = np.asarray(perm_r), np.asarray(perm_p)
    m, n = W0.shape
    offs_r, sizes_r = packed_offsets(m, b_r)
    offs_p, sizes_p = packed_offsets(n, b_p)
    G = cnp_blocks(q_r, m, b_r)
    H = cnp_blocks(q_p, n, b_p)
    q_r = np.asarray(q_r, np.float64)
    q_p = np.asarray(q_p, np.float64)
    X1 = gather_cols(X, perm_r)
    dY2 = gather_cols(dZ, perm_p)
    out_p = {}
    if len(blocks_p):
        X3 = scatter_cols(block_diag_right(X1, G, b_r), perm_r)
        for k in blocks_p:
            s, r = k * b_p, sizes_p[k]
            Y1K = X3 @ W0[:, perm_p[s:s + r]]
            dHk = Y1K.T @ dY2[:, s:s + r]
            Q = skew_from_packed(q_p[offs_p[k]:offs_p[k] + r * (r - 1) // 2], r)
            out_p[k] = project_to_packed(cnp_adjoint(Q, dHk))
    out_r = {}
    if len(blocks_r):
        dY = scatter_cols(block_diag_right(dY2, [Hk.T for Hk in H], b_p), perm_p)
        for j in blocks_r:
            s, r = j * b_r, sizes_r[j]
            dX2J = dY @ W0[perm_r[s:s + r], :].T
            dGj = X1[:, s:s + r].T @ dX2J
            Q = skew_from_packed(q_r[offs_r[j]:offs_r[j] + r * (r - 1) // 2], r)
            out_r[j] = project_to_packed(cnp_adjoint(Q, dGj))
    return out_r, out_p


def _packed_grad(q, dim, b, dblocks):
    q = np.asarray(q, dtype=np.float64)
    offs, sizes = packed_offsets(dim, b)
    out = np.zeros(packed_len(dim, b))
    for o, r, U in zip(offs, sizes, dblocks):
        L = r * (r - 1) // 2
        Q = skew_from_packed(q[o:o + L], r)
        out[o:o + L] = project_to_packed(cnp_adjoint(Q, U))
    return out


def merge(W0, q_r, q_p, perm_r, perm_p, b_r, b_p):
    """W0 <- R W0 P, after which the rotations restart from Q = 0 [MG].

    R W0 P = Psi^T Diag(G) (Psi W0 Phi^T) Diag(H) Phi, evaluated block by
    block on the permuted weight. Returns the new W0; the caller zeroes q.
    """
    W0 = np.asarray(W0, dtype=np.float64)
    m, n = W0.shape
    G = cnp_blocks(q_r, m, b_r)
    H = cnp_blocks(q_p, n, b_p)
    A = permuted_weight(W0, perm_r, perm_p)
    B = block_diag_right(block_diag_left(G, A, b_r), H, b_p)
    out = np.empty_like(B)
    out[np.ix_(np.asarray(perm_r), np.asarray(perm_p))] = B
    return out


def requantize_int8_per_col(W):
    """Per-output-column int8 storage of a float weight [XQ], in the reading
    taken of the page's quantized base weight: scale[c] = max_r |W[r, c]| / 127,
    code = clip(rint(W / scale), -127, 127) with rint rounding half to even,
    and a zero column stored with scale 1. The page fixes no precision for
    the decision, so it is taken in float32, the kernels' precision."""
    W32 = np.asarray(W, dtype=np.float64).astype(np.float32)
    amax = np.abs(W32).max(axis=0)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.rint(W32 / scale[None, :]), -127, 127).astype(np.int8)
    return codes, scale


# ----------------------------------------------------------------------------
# fp8 base weight  ([XQ] extension)
# ----------------------------------------------------------------------------
#
# [XQ] stores the base weight in int8 and expects lower-precision formats such
# as FP8 to need no quantization-aware training either. The format taken is
# E4M3 of the OCP 8-bit floating point specification (OFP8): a code byte is a
# sign bit, a 4-bit exponent field e with bias 7 and a 3-bit mantissa m; e > 0
# gives (1 + m/8) 2^(e-7), e = 0 gives the subnormal m 2^-9, and e = 15 with
# m = 7 is NaN (there is no infinity), so the largest finite magnitude is 448.
# Storage per output column as for int8, a reading: scale[c] = max_r |W[r, c]|
# / 448 in float32 (1 for a zero column) and the code of W / scale (float32)
# is the nearest E4M3 value, ties to the even code, magnitudes past 448 kept
# at 448, and the sign bit that of W / scale.

FP8_MAX = 448.0


def fp8_e4m3_values():
    """Magnitudes of the finite non-negative E4M3 codes 0..126, in code order
    (increasing)."""
    c = np.arange(127)
    e, m = c >> 3, c & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


def fp8_e4m3_decode(codes):
    """Value of each E4M3 code byte; NaN for 0x7F and 0xFF."""
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
    low = c & 0x7F
    v = np.where(low == 0x7F, np.nan, fp8_e4m3_values()[np.minimum(low, 126)])
    return np.where(c & 0x80, -v, v)


def fp8_e4m3_encode(x):
    """E4M3 code byte of each finite value: the nearest code, ties to the even
    code, magnitudes past 448 saturated, the sign bit that of x."""
    x = np.asarray(x, dtype=np.float64)
    vals = fp8_e4m3_values()
    a = np.minimum(np.abs(x), FP8_MAX)
    hi = np.minimum(np.searchsorted(vals, a, side="left"), 126)  # first value >= a
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - vals[lo], vals[hi] - a
    mag = np.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    return (mag | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def dequantize_fp8(Wq, scale):
    """Run-time dequantization of a per-output-column E4M3 base weight:
    W0[r, c] = scale[c] * value(Wq[r, c])."""
    return fp8_e4m3_decode(Wq) * np.asarray(scale, np.float64)[None, :]


def requantize_fp8_per_col(W):
    """Per-output-column E4M3 storage of a float weight (see above); the
    division and the decision are taken in float32, the kernels' precision."""
    W32 = np.asarray(W, dtype=np.float64).astype(np.float32)
    amax = np.abs(W32).max(axis=0)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    codes = fp8_e4m3_encode((W32 / scale[None, :]).astype(np.float32))
    return codes, scale


def merge_xq(Wq, scale, q_r, q_p, perm_r, perm_p, b_r, b_p, fmt="i8"):
    """Merge of a quantized base weight [XQ], [MG] (fmt "i8": int8 codes,
    "f8": E4M3 code bytes). The page does not say how the merged weight is
    stored again; reading: dequantize, W0 <- R W0 P in float64, then store
    per output column as the input was stored. Returns (codes, scale, merged
    float64 weight before storage)."""
    deq, req = (dequantize_fp8, requantize_fp8_per_col) if fmt == "f8" else (dequantize, requantize_int8_per_col)
    W = merge(deq(Wq, scale), q_r, q_p, perm_r, perm_p, b_r, b_p)
    codes, new_scale = req(W)
    return codes, new_scale, W


# ----------------------------------------------------------------------------
# permutation draws and the merge schedule  ([BS], [MG])
# ----------------------------------------------------------------------------
#
# [BS] makes Psi and Phi random permutations and [MG] restarts the rotations
# at every merge, but the pages say neither how a permutation is drawn nor
# when a new one is. Reading: after every merge both permutations are drawn
# again, uniformly, from a counter-based generator, so that any device can
# reproduce a draw from (seed, tag, draw number) alone. The generator is
# Philox4x64 with 10 rounds, as defined by Salmon, Moraes, Dror and Shaw,
# "Parallel random numbers: as easy as 1, 2, 3" (SC 2011).

_PHILOX_MUL = (0xD2E7470EE14C6C93, 0xCA5A826395121157)  # round multipliers
_PHILOX_WEYL = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)  # key increments
_U32 = np.uint64(0xFFFFFFFF)


def _mulhilo64(a, b):
    """Full 128-bit product of uint64 arrays, as (high, low) words, from
    32-bit limbs (NumPy has no 128-bit integers)."""
    s32 = np.uint64(32)
    al, ah = a & _U32, a >> s32
    bl, bh = b & _U32, b >> s32
    ll, lh, hl, hh = al * bl, al * bh, ah * bl, ah * bh
    mid = (ll >> s32) + (lh & _U32) + (hl & _U32)
    lo = (ll & _U32) | ((mid & _U32) << s32)
    hi = hh + (lh >> s32) + (hl >> s32) + (mid >> s32)
    return hi, lo


def philox4x64_10(ctr, key):
    """Philox4x64-10 of counters ctr (N x 4 uint64) under key (2 uint64).

    Each round multiplies counter words 0 and 2 by the two round multipliers
    and forms the new counter (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the
    key gains the two Weyl increments before every round after the first.
    Returns N x 4 uint64 output words."""
    c = np.array(ctr, dtype=np.uint64).reshape(-1, 4).copy()
    k0, k1 = (np.uint64(int(v)) for v in key)
    m0, m1 = (np.uint64(v) for v in _PHILOX_MUL)
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k0 = k0 + np.uint64(_PHILOX_WEYL[0])
                k1 = k1 + np.uint64(_PHILOX_WEYL[1])
            hi0, lo0 = _mulhilo64(np.full(len(c), m0), c[:, 0])
            hi1, lo1 = _mulhilo64(np.full(len(c), m1), c[:, 2])
            c = np.stack([hi1 ^ c[:, 1] ^ k0, lo1, hi0 ^ c[:, 3] ^ k1, lo0], axis=1)
    return c


def perm_words(dim, seed, tag, draw):
    """Random 64-bit word of every index i < dim: word i mod 4 of the Philox
    block at counter (i div 4, draw, 0, 0) under key (seed, tag). `tag` keeps
    the draws of different layers and sides apart; `draw` numbers the draws
    of one permutation."""
    nb = (dim + 3) // 4
    ctr = np.zeros((nb, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(nb, dtype=np.uint64)
    ctr[:, 1] = np.uint64(draw)
    return philox4x64_10(ctr, (seed, tag)).reshape(-1)[:dim]


PERM_KEY_BITS = 44  # random bits of a sort key; dim <= 2**20 keeps the index in the rest


def perm_keys(dim, seed, tag, draw):
    """Sort key of every index: the top 44 bits of its random word."""
    return perm_words(dim, seed, tag, draw) >> np.uint64(64 - PERM_KEY_BITS)


def sample_perm(dim, seed, tag, draw):
    """A uniformly random permutation of range(dim) [BS]: the indices in
    ascending order of their keys, equal keys in ascending index order. (With
    dim <= 2**20 two keys of 44 random bits are equal with probability below
    dim**2 / 2**45, so the index order decides almost never.)"""
    assert 1 <= dim <= 1 << 20
    return np.argsort(perm_keys(dim, seed, tag, draw), kind="stable").astype(np.int64)


def merge_due(step, interval):
    """[MG]: the training loop asks after optimizer step `step` (counted from
    0) whether to merge. Reading: a merge follows every `interval`-th update,
    so after steps interval-1, 2*interval-1, ...; the k-th merge is followed by
    draw k of both permutations (draw 0 being the initial one)."""
    return (step + 1) % interval == 0


def weight_centric_forward(X, W0, q_r, q_p, perm_r, perm_p, b_r, b_p):
    """Original POET's weight-first evaluation X (R W0 P) with dense R and P
    ([IC], the form POET-X avoids). Small sizes only; used as a cross-check."""
    W0 = np.asarray(W0, dtype=np.float64)
    m, n = W0.shape
    R = dense_block_orthogonal(cnp_blocks(q_r, m, b_r), perm_r, b_r)
    P = dense_block_orthogonal(cnp_blocks(q_p, n, b_p), perm_p, b_p)
    return np.asarray(X, dtype=np.float64) @ (R @ W0 @ P)


def inner(A, B):
    """<A, B> = sum of elementwise products (the scalar loss for gradients)."""
    return float(np.sum(np.asarray(A, np.float64) * np.asarray(B, np.float64)))
