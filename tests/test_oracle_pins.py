"""Pins of the float64 oracle against facts fixed by the pages and by algebra.

Each test compares the oracle with something it does not compute itself: a
closed form, a hand-derived fixture under tests/golden/, a textbook or library
routine (numpy.linalg), a dense formulation, or central finite differences.
Source of the method: the zhichai.net digest of arXiv:2603.05500, sections
"1. 输入中心化架构", "2. 块随机正交变换", "3. Cayley-Neumann 参数化优化" and
"代码与部署" (merge_if_needed).
"""

import os

import numpy as np
import pytest

import oracle as O
from orthogonal_equivalence_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    return np.loadtxt(os.path.join(GOLDEN, name), comments="#", ndmin=2)


def _rand_skew(rng, r, sigma):
    A = rng.standard_normal((r, r)) * sigma
    return np.triu(A, 1) - np.triu(A, 1).T


def _cayley(Q):
    I = np.eye(Q.shape[0])
    return np.linalg.solve((I - Q).T, (I + Q).T).T  # (I+Q)(I-Q)^-1


def _tiny(seed=0, T=6, m=12, n=20, b_r=4, b_p=8, sigma_q=0.1):
    cfg = synth.LayerConfig("pin", 90 + seed, T, m, n, b_r, b_p, "f32", "f32",
                            sigma_q=sigma_q, sigma_w=0.5)
    L = synth.make_layer(cfg, seed)
    A = synth.make_activations(cfg, seed)
    return cfg, L, A


# --- packing -----------------------------------------------------------------

def test_packing_order_fixture():
    rows = _load("packing_order_b4.txt").astype(int)
    b = 4
    for k, i, l in rows:
        q = np.zeros(b * (b - 1) // 2)
        q[k] = 1.0
        Q = O.skew_from_packed(q, b)
        E = np.zeros((b, b))
        E[i, l], E[l, i] = 1.0, -1.0
        assert np.array_equal(Q, E)
        # the gradient projection reads the same position with the same signs
        M = np.zeros((b, b))
        M[i, l], M[l, i] = 3.0, 5.0
        g = O.project_to_packed(M)
        assert g[k] == -2.0 and np.count_nonzero(g) == 1


def test_cnp_onehot_fixture_exact():
    (s, g_off, g_diag), = _load("cnp_onehot_b4.txt")
    b = 4
    iu = np.triu_indices(b, 1)
    for k in range(b * (b - 1) // 2):
        q = np.zeros(b * (b - 1) // 2)
        q[k] = s
        G = O.cnp(O.skew_from_packed(q, b))
        i, l = iu[0][k], iu[1][k]
        E = np.eye(b)
        E[i, l], E[l, i] = g_off, -g_off
        E[i, i] = E[l, l] = g_diag
        assert np.array_equal(G, E), k  # dyadic values: exact in float64


def test_cnp_b2_closed_form_fixture():
    for s, g00, g01 in _load("cnp_b2_closed_form.txt"):
        G = O.cnp(O.skew_from_packed(np.array([s]), 2))
        assert np.array_equal(G, np.array([[g00, g01], [-g01, g00]]))


# --- Cayley-Neumann truncation (section 3) ------------------------------------

@pytest.mark.parametrize("r", [3, 8, 16])
def test_cnp_gram_closed_form(r):
    # (I+Q+Q^2+Q^3)(I-Q) = I - Q^4, so G = C (I - Q^4) with C the exact Cayley
    # transform; C orthogonal and Q^4 symmetric give G^T G = (I - Q^4)^2.
    rng = np.random.default_rng(r)
    Q = _rand_skew(rng, r, 0.2)
    G = O.cnp(Q)
    Q4 = np.linalg.matrix_power(Q, 4)
    I = np.eye(r)
    assert np.allclose(G.T @ G, (I - Q4) @ (I - Q4), atol=1e-13, rtol=0)


@pytest.mark.parametrize("r", [4, 9, 16])
def test_cnp_vs_exact_cayley_spectral(r):
    rng = np.random.default_rng(100 + r)
    Q = _rand_skew(rng, r, 0.3)
    C = _cayley(Q)
    assert np.allclose(C.T @ C, np.eye(r), atol=1e-13)
    smax = np.linalg.svd(Q, compute_uv=False).max()
    err = np.linalg.norm(O.cnp(Q) - C, 2)
    assert err == pytest.approx(smax ** 4, rel=1e-9)


def test_cnp_singular_values():
    rng = np.random.default_rng(7)
    Q = _rand_skew(rng, 10, 0.4)
    sq = np.linalg.svd(Q, compute_uv=False)
    sg = np.sort(np.linalg.svd(O.cnp(Q), compute_uv=False))
    assert np.allclose(sg, np.sort(np.abs(1 - sq ** 4)), atol=1e-13)


def test_cnp_truncation_order_four():
    # ||G^T G - I||_F shrinks like t^4 when Q is scaled by t (4-term truncation)
    rng = np.random.default_rng(11)
    Q = _rand_skew(rng, 12, 1.0)
    Q = Q / np.linalg.norm(Q, 2)
    ts = np.array([1e-1, 3e-2, 1e-2])
    d = [np.linalg.norm(O.cnp(t * Q).T @ O.cnp(t * Q) - np.eye(12)) for t in ts]
    slope = np.polyfit(np.log(ts), np.log(d), 1)[0]
    assert abs(slope - 4.0) < 0.02
    # leading term 2 ||Q^4||_F
    t = 1e-2
    assert d[-1] == pytest.approx(2 * np.linalg.norm(np.linalg.matrix_power(t * Q, 4)), rel=1e-3)


def test_cnp_zero_is_identity():
    assert np.array_equal(O.cnp(np.zeros((5, 5))), np.eye(5))


# --- block structure, permutation, input- vs weight-centric (sections 1, 2) --

@pytest.mark.parametrize("shape", [(12, 20, 4, 8), (10, 14, 4, 6), (16, 24, 16, 24)])
def test_input_centric_equals_weight_centric(shape):
    m, n, b_r, b_p = shape  # (10, 14, 4, 6) has ragged last blocks on both sides
    _, L, A = _tiny(0, 5, m, n, b_r, b_p)
    args = (L["W0"], L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], b_r, b_p)
    Z = O.forward(A["X"], *args)["Z"]
    Zw = O.weight_centric_forward(A["X"], *args)
    assert np.allclose(Z, Zw, atol=1e-13, rtol=1e-12)


def test_dense_R_is_block_diagonal_in_permuted_frame():
    rng = np.random.default_rng(3)
    perm = rng.permutation(10)
    blocks = [O.cnp(_rand_skew(rng, r, 0.2)) for r in (4, 4, 2)]
    R = O.dense_block_orthogonal(blocks, perm, 4)
    x = rng.standard_normal(10)
    # R^T x computed by hand: gather x by perm, apply G_j^T per block, scatter
    xp = x[perm]
    yp = np.concatenate([blocks[0].T @ xp[0:4], blocks[1].T @ xp[4:8], blocks[2].T @ xp[8:10]])
    y = np.empty(10)
    y[perm] = yp
    assert np.allclose(R.T @ x, y, atol=1e-14)


def test_spectrum_preserved_under_exact_cayley():
    rng = np.random.default_rng(5)
    m, n, b = 12, 8, 4
    perm_r, perm_p = rng.permutation(m), rng.permutation(n)
    W0 = rng.standard_normal((m, n))
    R = O.dense_block_orthogonal([_cayley(_rand_skew(rng, b, 0.5)) for _ in range(m // b)], perm_r, b)
    P = O.dense_block_orthogonal([_cayley(_rand_skew(rng, b, 0.5)) for _ in range(n // b)], perm_p, b)
    assert np.allclose(np.linalg.svd(R @ W0 @ P, compute_uv=False),
                       np.linalg.svd(W0, compute_uv=False), atol=1e-12)


def test_cnp_layer_spectrum_bounds():
    # with the truncated map, sigma_i(R W0 P) lies in
    # [smin(G) smin(H) sigma_i(W0), smax(G) smax(H) sigma_i(W0)], smax <= 1
    _, L, _ = _tiny(2, 4, 12, 8, 4, 4, sigma_q=0.3)
    m, n = 12, 8
    G = O.cnp_blocks(L["q_r"], m, 4)
    H = O.cnp_blocks(L["q_p"], n, 4)
    R = O.dense_block_orthogonal(G, L["perm_r"], 4)
    P = O.dense_block_orthogonal(H, L["perm_p"], 4)
    sw = np.linalg.svd(L["W0"].astype(np.float64), compute_uv=False)
    s = np.linalg.svd(R @ L["W0"] @ P, compute_uv=False)
    sR = np.linalg.svd(R, compute_uv=False)
    sP = np.linalg.svd(P, compute_uv=False)
    assert sR.max() <= 1 + 1e-12 and sP.max() <= 1 + 1e-12
    lo = sR.min() * sP.min() * sw
    assert np.all(s >= lo - 1e-12) and np.all(s <= sw + 1e-12)


def test_zero_q_is_plain_matmul_and_single_block_textbook():
    _, L, A = _tiny(1, 4, 8, 8, 4, 4)
    zq_r, zq_p = np.zeros_like(L["q_r"]), np.zeros_like(L["q_p"])
    Z = O.forward(A["X"], L["W0"], zq_r, zq_p, L["perm_r"], L["perm_p"], 4, 4)["Z"]
    assert np.array_equal(Z, A["X"].astype(np.float64) @ L["W0"].astype(np.float64))
    # b = m, identity permutation: R = G, P = H (one block each)
    ident = np.arange(8)
    Z1 = O.forward(A["X"], L["W0"], np.resize(L["q_r"], 28), np.resize(L["q_p"], 28),
                   ident, ident, 8, 8)["Z"]
    G = O.cnp(O.skew_from_packed(np.resize(L["q_r"], 28), 8))
    H = O.cnp(O.skew_from_packed(np.resize(L["q_p"], 28), 8))
    assert np.allclose(Z1, A["X"] @ G @ L["W0"] @ H, atol=1e-13)


# --- gradients ----------------------------------------------------------------

def _loss(X, dZ, L, q_r, q_p, b_r, b_p, W0=None):
    W0 = L["W0"] if W0 is None else W0
    return O.inner(dZ, O.forward(X, W0, q_r, q_p, L["perm_r"], L["perm_p"], b_r, b_p)["Z"])


@pytest.mark.parametrize("shape", [(12, 20, 4, 8), (10, 14, 4, 6)])
def test_dq_matches_central_differences_full_sweep(shape):
    m, n, b_r, b_p = shape
    _, L, A = _tiny(4, 5, m, n, b_r, b_p, sigma_q=0.1)
    X, dZ = A["X"].astype(np.float64), A["dZ"].astype(np.float64)
    g = O.backward(X, dZ, L["W0"], L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], b_r, b_p)
    h = 1e-6
    for side in ("r", "p"):
        q = L["q_" + side].astype(np.float64)
        fd = np.empty_like(q)
        for k in range(q.size):
            qp, qm = q.copy(), q.copy()
            qp[k] += h
            qm[k] -= h
            if side == "r":
                fd[k] = (_loss(X, dZ, L, qp, L["q_p"], b_r, b_p) - _loss(X, dZ, L, qm, L["q_p"], b_r, b_p)) / (2 * h)
            else:
                fd[k] = (_loss(X, dZ, L, L["q_r"], qp, b_r, b_p) - _loss(X, dZ, L, L["q_r"], qm, b_r, b_p)) / (2 * h)
        got = g["dq_" + side]
        assert np.allclose(got, fd, rtol=1e-6, atol=1e-7 * np.abs(fd).max()), side


def test_dx_dense_and_finite_difference():
    _, L, A = _tiny(5, 4, 12, 8, 4, 4, sigma_q=0.2)
    X, dZ = A["X"].astype(np.float64), A["dZ"].astype(np.float64)
    args = (L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], 4, 4)
    g = O.backward(X, dZ, L["W0"], *args)
    R = O.dense_block_orthogonal(O.cnp_blocks(L["q_r"], 12, 4), L["perm_r"], 4)
    P = O.dense_block_orthogonal(O.cnp_blocks(L["q_p"], 8, 4), L["perm_p"], 4)
    assert np.allclose(g["dX"], dZ @ (R @ L["W0"] @ P).T, atol=1e-13)
    h = 1e-6
    for (t, c) in [(0, 0), (1, 5), (3, 11)]:
        Xp, Xm = X.copy(), X.copy()
        Xp[t, c] += h
        Xm[t, c] -= h
        fd = (_loss(Xp, dZ, L, L["q_r"], L["q_p"], 4, 4) - _loss(Xm, dZ, L, L["q_r"], L["q_p"], 4, 4)) / (2 * h)
        assert g["dX"][t, c] == pytest.approx(fd, rel=1e-7, abs=1e-9)


def test_block_gradient_token_sum_equals_dense_route():
    # dG_j = X1_J^T dX2_J equals the diagonal blocks of Psi X^T dZ (W0 P)^T Psi^T
    _, L, A = _tiny(6, 7, 12, 8, 4, 4, sigma_q=0.2)
    X, dZ = A["X"].astype(np.float64), A["dZ"].astype(np.float64)
    g = O.backward(X, dZ, L["W0"], L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], 4, 4)
    P = O.dense_block_orthogonal(O.cnp_blocks(L["q_p"], 8, 4), L["perm_p"], 4)
    Psi = O.permutation_matrix(L["perm_r"])
    D = Psi @ X.T @ dZ @ (L["W0"] @ P).T @ Psi.T
    for j, dG in enumerate(g["dG"]):
        assert np.allclose(dG, D[4 * j:4 * j + 4, 4 * j:4 * j + 4], atol=1e-12)


def test_dq_is_linear_in_token_shards():
    _, L, A = _tiny(7, 9, 12, 20, 4, 8, sigma_q=0.1)
    X, dZ = A["X"].astype(np.float64), A["dZ"].astype(np.float64)
    args = (L["W0"], L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], 4, 8)
    full = O.backward(X, dZ, *args)
    a = O.backward(X[:4], dZ[:4], *args)
    b = O.backward(X[4:], dZ[4:], *args)
    for k in ("dq_r", "dq_p"):
        assert np.allclose(full[k], a[k] + b[k], atol=1e-12)
    assert np.allclose(full["dX"], np.vstack([a["dX"], b["dX"]]), atol=1e-13)


# --- merge (merge_if_needed) ---------------------------------------------------

def test_merge_preserves_function_and_zero_q_is_identity():
    _, L, A = _tiny(8, 6, 12, 20, 4, 8, sigma_q=0.2)
    m, n = 12, 20
    args = (L["perm_r"], L["perm_p"], 4, 8)
    W1 = O.merge(L["W0"], L["q_r"], L["q_p"], *args)
    z0 = np.zeros_like(L["q_r"]), np.zeros_like(L["q_p"])
    before = O.forward(A["X"], L["W0"], L["q_r"], L["q_p"], *args)["Z"]
    after = O.forward(A["X"], W1, z0[0], z0[1], *args)["Z"]
    assert np.allclose(before, after, atol=1e-13)
    # dense definition R W0 P
    R = O.dense_block_orthogonal(O.cnp_blocks(L["q_r"], m, 4), L["perm_r"], 4)
    P = O.dense_block_orthogonal(O.cnp_blocks(L["q_p"], n, 8), L["perm_p"], 8)
    assert np.allclose(W1, R @ L["W0"] @ P, atol=1e-14)
    # merging with q = 0 leaves W0 bit for bit
    W2 = O.merge(L["W0"], z0[0], z0[1], *args)
    assert np.array_equal(W2, L["W0"].astype(np.float64))
    # after a merge the perms can be resampled without changing the function
    rng = np.random.default_rng(1)
    after2 = O.forward(A["X"], W1, z0[0], z0[1], rng.permutation(m), rng.permutation(n), 4, 8)["Z"]
    assert np.allclose(after2, after, atol=1e-13)


def test_permuted_weight_is_psi_w_phit():
    rng = np.random.default_rng(9)
    W = rng.standard_normal((6, 5))
    pr, pp = rng.permutation(6), rng.permutation(5)
    assert np.array_equal(O.permuted_weight(W, pr, pp),
                          O.permutation_matrix(pr) @ W @ O.permutation_matrix(pp).T)


# --- quantised base weight -----------------------------------------------------

def test_dequantize_exact_and_roundtrip_bound():
    Wq = np.array([[1, -127], [64, 3]], dtype=np.int8)
    s = np.array([0.5, 2.0 ** -10], dtype=np.float32)
    assert np.array_equal(O.dequantize(Wq, s), np.array([[0.5, -127 * 2.0 ** -10], [32.0, 3 * 2.0 ** -10]]))
    cfg = synth.CONFIGS["xq_llama8b_mlp_up"]
    L = synth.make_layer(cfg, 0, m=64, n=48)
    W = synth._draw(synth._rng(0, cfg.cfg_id, 0), (64, 48), cfg.sigma_w).astype(np.float64)
    Wd = O.dequantize(L["W0_raw"], L["w_scale"])
    # absmax quantisation error is at most half a step per column
    assert np.all(np.abs(Wd - W) <= 0.5 * L["w_scale"][None, :].astype(np.float64) * (1 + 1e-6))


def test_requantize_rounds_half_to_even_and_stores_zero_columns():
    # column 0: scale 0.25 (a power of two, exact) and codes at exact half steps;
    # column 1 is all zero
    s = 0.25
    v = np.array([127, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, -126.5])
    W = np.stack([v * s, np.zeros_like(v)], axis=1)
    codes, scale = O.requantize_int8_per_col(W)
    assert scale.dtype == np.float32 and np.array_equal(scale, np.array([0.25, 1.0], np.float32))
    assert np.array_equal(codes[:, 0], np.array([127, 2, 4, -2, 0, 0, 2, -126], np.int8))
    assert np.array_equal(codes[:, 1], np.zeros(8, np.int8))
    # sign symmetry
    c2, s2 = O.requantize_int8_per_col(-W)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scale)


def test_xq_merge_with_zero_q_keeps_the_codes():
    # merging with q = 0 is the identity on the weight; storing it again gives
    # back every code, and the scales of that storage
    cfg = synth.CONFIGS["xq_llama8b_mlp_up"]
    L = synth.make_layer(cfg, 0, m=64, n=96)
    zr = np.zeros(O.packed_len(64, 16))
    zp = np.zeros(O.packed_len(96, 16))
    pr, pp = np.random.default_rng(3).permutation(64), np.random.default_rng(4).permutation(96)
    codes, scale, W = O.merge_xq(L["W0_raw"], L["w_scale"], zr, zp, pr, pp, 16, 16)
    assert np.array_equal(W, O.dequantize(L["W0_raw"], L["w_scale"]))
    assert np.array_equal(codes, L["W0_raw"])
    assert np.allclose(scale, L["w_scale"], rtol=2.0 ** -22, atol=0)


def test_xq_merge_stores_the_float_merge_within_half_a_step():
    cfg = synth.CONFIGS["xq_llama8b_mlp_up"]
    L = synth.make_layer(cfg, 0, m=48, n=64)
    rng = np.random.default_rng(5)
    qr = rng.standard_normal(O.packed_len(48, 16)) * 0.05
    qp = rng.standard_normal(O.packed_len(64, 16)) * 0.05
    pr, pp = rng.permutation(48), rng.permutation(64)
    codes, scale, W = O.merge_xq(L["W0_raw"], L["w_scale"], qr, qp, pr, pp, 16, 16)
    # the merged float weight is R W0 P of the dequantized weight
    R = O.dense_block_orthogonal(O.cnp_blocks(qr, 48, 16), pr, 16)
    P = O.dense_block_orthogonal(O.cnp_blocks(qp, 64, 16), pp, 16)
    assert np.allclose(W, R @ O.dequantize(L["W0_raw"], L["w_scale"]) @ P, atol=1e-14)
    # every column uses its full code range and stores within half a step
    assert np.all(np.abs(codes.astype(np.int32)).max(axis=0) == 127)
    assert np.all(np.abs(O.dequantize(codes, scale) - W) <= 0.5 * scale[None, :] * (1 + 1e-5))
    assert not np.array_equal(codes, L["W0_raw"])


def test_packed_len_matches_block_count():
    assert O.packed_len(4096, 256) == 16 * 256 * 255 // 2
    assert O.packed_len(10, 4) == 6 + 6 + 1
    assert synth.packed_count(10, 4) == O.packed_len(10, 4)
    assert synth.packed_count(14336, 256) == O.packed_len(14336, 256)


def test_block_restricted_gradients_agree_with_full_backward():
    _, L, A = _tiny(12, 7, 16, 24, 8, 8, sigma_q=0.1)
    args = (L["W0"], L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], 8, 8)
    full = O.backward(A["X"], A["dZ"], *args)
    r, p = O.backward_blocks(A["X"], A["dZ"], *args, [0, 1], [2])
    assert np.allclose(r[0], full["dq_r"][0:28], atol=1e-13)
    assert np.allclose(r[1], full["dq_r"][28:56], atol=1e-13)
    assert np.allclose(p[2], full["dq_p"][56:84], atol=1e-13)


# --- permutation draws and the merge schedule -------------------------------
# NumPy's Philox bit generator implements the same published Philox4x64-10;
# it increments its 256-bit counter (word 0 lowest) before each block.

_U64 = (1 << 64) - 1


def _numpy_philox_words(key, start_ctr, count):
    g = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=np.array(start_ctr, dtype=np.uint64))
    return g.random_raw(count).astype(np.uint64)


@pytest.mark.parametrize("key,ctr", [((0, 0), (0, 0, 0, 0)), ((123, 456), (5, 9, 0, 0)),
                                     ((_U64, 7), (_U64 - 1, 3, 1, 2)), ((2**63 + 11, 1), (40, 0, 0, 2**62))])
def test_philox_is_numpy_philox(key, ctr):
    ref = _numpy_philox_words(key, ctr, 12).reshape(3, 4)
    c = np.array(ctr, dtype=object)
    mine = []
    for _ in range(3):
        # the next counter, carried through the four words as NumPy does
        v = int(c[0]) + int(c[1]) * 2**64 + int(c[2]) * 2**128 + int(c[3]) * 2**192 + 1
        c = np.array([(v >> (64 * w)) & _U64 for w in range(4)], dtype=object)
        mine.append(O.philox4x64_10(np.array(c, dtype=np.uint64)[None, :], key)[0])
    assert np.array_equal(np.array(mine, dtype=np.uint64), ref)


@pytest.mark.parametrize("dim,draw", [(1, 0), (13, 0), (64, 3), (1031, 2**40)])
def test_perm_words_are_the_philox_stream_from_counter_zero(dim, draw):
    seed, tag = 987654321, 5
    # a start one block before (0, draw, 0, 0): NumPy increments before drawing
    start = (_U64, _U64, _U64, _U64) if draw == 0 else (_U64, draw - 1, 0, 0)
    ref = _numpy_philox_words((seed, tag), start, dim)
    assert np.array_equal(O.perm_words(dim, seed, tag, draw), ref)
    # the sort keys are the words' top 44 bits
    assert np.array_equal(O.perm_keys(dim, seed, tag, draw), np.array([int(v) >> 20 for v in ref], dtype=np.uint64))


def test_sample_perm_sorts_by_key_then_index():
    for dim in (1, 2, 37, 300):
        words = O.perm_words(dim, 11, 3, 1)
        p = O.sample_perm(dim, 11, 3, 1)
        assert sorted(p.tolist()) == list(range(dim))
        brute = sorted(range(dim), key=lambda i: (int(words[i]) >> 20, i))
        assert p.tolist() == brute
    # different tags and draws give different permutations
    assert not np.array_equal(O.sample_perm(300, 11, 3, 1), O.sample_perm(300, 11, 4, 1))
    assert not np.array_equal(O.sample_perm(300, 11, 3, 1), O.sample_perm(300, 11, 3, 2))


def test_sample_perm_is_uniform_on_four_elements():
    # 2400 draws of a 4-element permutation: each of the 24 appears about 100
    # times (binomial standard deviation 9.8)
    counts = {}
    for d in range(2400):
        k = tuple(O.sample_perm(4, 2024, 9, d).tolist())
        counts[k] = counts.get(k, 0) + 1
    assert len(counts) == 24
    assert min(counts.values()) >= 60 and max(counts.values()) <= 140


def test_merge_schedule_merges_after_every_interval_updates():
    due = [s for s in range(1000) if O.merge_due(s, 200)]
    assert due == [199, 399, 599, 799, 999]
    assert all(O.merge_due(s, 1) for s in range(10))


# --- fp8 (E4M3) base weight -------------------------------------------------

def test_fp8_decode_matches_published_values_and_torch():
    g = _load("fp8_e4m3_published_values.txt")
    assert np.array_equal(O.fp8_e4m3_decode(g[:, 0].astype(np.uint8)), g[:, 1])
    assert np.isnan(O.fp8_e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    # every byte against torch's float8_e4m3fn (a library implementation of
    # the same OCP format)
    import torch

    c = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    d = O.fp8_e4m3_decode(c)
    assert np.array_equal(np.isnan(d), np.isnan(t))
    assert np.array_equal(d[~np.isnan(d)], t[~np.isnan(t)])


def test_fp8_encode_rounds_to_nearest_even_and_saturates():
    import torch

    vals = O.fp8_e4m3_values()
    # every finite code back to itself; midpoints to the even neighbour
    assert np.array_equal(O.fp8_e4m3_encode(vals), np.arange(127, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    assert np.array_equal(O.fp8_e4m3_encode(mids), (np.arange(126) + 1) // 2 * 2)
    # hand-derived ties: 1.0625 halfway 1 (0x38) / 1.125 (0x39) -> 0x38;
    # 1.1875 halfway 1.125 / 1.25 (0x3A) -> 0x3A; 2^-10 halfway 0 / 2^-9 -> 0
    assert O.fp8_e4m3_encode([1.0625, 1.1875, 2.0 ** -10]).tolist() == [0x38, 0x3A, 0x00]
    # saturation and signs
    assert O.fp8_e4m3_encode([449.0, 1e9, -1e9, -1.0, -0.0]).tolist() == [0x7E, 0x7E, 0xFE, 0xB8, 0x80]
    # random float32 values within range against torch's conversion
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.standard_normal(4000) * 0.01,
                        mids, -mids]).astype(np.float32)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.fp8_e4m3_encode(x), t)


def test_fp8_requantize_and_merge():
    W = np.random.default_rng(12).standard_normal((40, 24)) * 0.02
    W[:, 3] = 0.0
    codes, scale = O.requantize_fp8_per_col(W)
    assert scale[3] == 1.0 and np.all(codes[:, 3] == 0)
    # the column maximum takes the largest code; every value within half a
    # code step (relative 2^-4 for normals, 2^-10 absolute on the code scale)
    big = np.argmax(np.abs(W), axis=0)
    for c in (0, 1, 5):
        assert codes[big[c], c] & 0x7F == 0x7E
    Wd = O.dequantize_fp8(codes, scale)
    step = np.maximum(np.abs(W) / scale * 2.0 ** -4, 2.0 ** -10) * scale
    assert np.all(np.abs(Wd - W) <= step * (1 + 1e-6))
    # the synthetic fp8 weight is that storage of the drawn float weight
    cfg = synth.CONFIGS["xf8_llama8b_mlp_up"]
    L = synth.make_layer(cfg, 0, m=32, n=48)
    c2, s2 = O.requantize_fp8_per_col(O.dequantize_fp8(L["W0_raw"], L["w_scale"]))
    assert np.array_equal(c2, L["W0_raw"])
    assert np.allclose(s2, L["w_scale"], rtol=2.0 ** -22, atol=0)
    # merge with q = 0 keeps every code
    zr, zp = np.zeros(O.packed_len(32, 16)), np.zeros(O.packed_len(48, 16))
    pr, pp = np.random.default_rng(13).permutation(32), np.random.default_rng(14).permutation(48)
    codes, scale, W = O.merge_xq(L["W0_raw"], L["w_scale"], zr, zp, pr, pp, 16, 16, fmt="f8")
    assert np.array_equal(codes, L["W0_raw"])
