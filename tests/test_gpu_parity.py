"""Parity of the HIP path (libpoetx.so through its C ABI) with the float64
oracle on the same seeded inputs.

Bar: relative Frobenius error ||gpu - ref|| / ||ref|| per output tensor of at
most 1e-5 for float32 layers and 2e-2 for bfloat16 layers (the tolerances the
layer's specification states), bit-exact for pure index work (packing of the
skew parameters, permutations). Full-size workloads are checked on sampled
outputs: token rows of z and dx (both token-local), whole blocks of dq, and
the whole merged weight.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from orthogonal_equivalence_amd import synth  # noqa: E402
from orthogonal_equivalence_amd import poetx as px  # noqa: E402
from orthogonal_equivalence_amd.device import DeviceLayer, to_device, to_host_f64  # noqa: E402

TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    torch.cuda.init()


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _cfg(name, T, m, n, b_r, b_p, act, weight, cfg_id):
    return synth.LayerConfig(name, cfg_id, T, m, n, b_r, b_p, act, weight)


def _w0_values(cfg, L):
    if cfg.weight == "i8":
        return O.dequantize(L["W0_raw"], L["w_scale"])
    if cfg.weight == "f8":
        return O.dequantize_fp8(L["W0_raw"], L["w_scale"])
    return L["W0"].astype(np.float64)


def _run(cfg, seed=0, merge=False):
    print(f"\n[gpu] {cfg.name} T={cfg.T} m={cfg.m} n={cfg.n} b={cfg.b_r}/{cfg.b_p} "
          f"{cfg.act}/{cfg.weight} seed={seed}", flush=True)
    L = synth.make_layer(cfg, seed)
    A = synth.make_activations(cfg, seed)
    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, cfg.act, cfg.weight, cfg.T)
    dl.load(L)
    dl.cnp_build()
    x = to_device(A["X_raw"], cfg.act)
    dz = to_device(A["dZ_raw"], cfg.act)
    z = dl.forward(x)
    dq_r, dq_p, dx = dl.backward(dz)
    x1, y1 = dl.saved_views(cfg.T)
    out = dict(z=to_host_f64(z), dq_r=to_host_f64(dq_r), dq_p=to_host_f64(dq_p), dx=to_host_f64(dx),
               x1=to_host_f64(x1), y1=to_host_f64(y1),
               g_r=to_host_f64(dl.g_planes(px.POETX_SIDE_R)), g_p=to_host_f64(dl.g_planes(px.POETX_SIDE_P)))
    if merge:
        # merged into the frame of freshly drawn permutations, as a training
        # loop does; W0 in the original frame is exported for the comparison
        rng = np.random.default_rng([seed, cfg.cfg_id, 99])
        nr, np_ = rng.permutation(cfg.m).astype(np.int32), rng.permutation(cfg.n).astype(np.int32)
        dl.merge(to_device(nr, "i32"), to_device(np_, "i32"))
        out["w0_merged"] = to_host_f64(dl.export_w0()[0])
        out["wp_merged"] = to_host_f64(dl.wp)
        out["perm_next"] = (nr, np_)
        out["q_after"] = to_host_f64(torch.cat([dl.q_r, dl.q_p]))
    torch.cuda.synchronize()
    return L, A, out, dl


def _expected_planes(q, dim, b):
    G = O.cnp_blocks(q, dim, b)
    nblk = len(G)
    P = np.zeros((2, nblk, b, b))
    for j, g in enumerate(G):
        r = g.shape[0]
        P[0, j, :r, :r] = g - np.eye(r)
        P[1, j, :r, :r] = (g - np.eye(r)).T
    return P


# ---------------------------------------------------------------------------
# full parity on sizes the oracle finishes in seconds
# ---------------------------------------------------------------------------

SMALL = [
    # the float32 workload itself (256 tokens, 512 x 512, b = 64)
    synth.CONFIGS["tiny_f32"],
    # float32 with short last blocks on both sides and a ragged token count
    _cfg("f32_ragged", 77, 200, 136, 64, 64, "f32", "f32", 20),
    # bfloat16, several 256-row tiles, ragged T, b = 256
    _cfg("bf16_multitile", 1000, 768, 1280, 256, 256, "bf16", "bf16", 21),
    # bfloat16 with short last blocks (640 = 2*256 + 128, 1088 = 4*256 + 64)
    _cfg("bf16_ragged_blocks", 777, 640, 1088, 256, 256, "bf16", "bf16", 22),
    # b = 512: four output tiles per block in the token reductions
    _cfg("bf16_b512", 300, 1024, 1536, 512, 512, "bf16", "bf16", 23),
    # small blocks and different R / P block sizes
    _cfg("bf16_b32_b64", 130, 256, 192, 32, 64, "bf16", "bf16", 24),
    # int8 base weight with per-column scales
    _cfg("xq_small", 520, 512, 768, 128, 128, "bf16", "i8", 25),
    # fp8 (E4M3) base weight with per-column scales
    _cfg("xf8_small", 520, 512, 768, 128, 128, "bf16", "f8", 66),
    # a single token
    _cfg("bf16_one_token", 1, 256, 512, 128, 128, "bf16", "bf16", 26),
    # float32 with more tokens than weight rows: the backward folds H into the weight
    _cfg("f32_fold", 300, 128, 192, 64, 64, "f32", "f32", 27),
    # the largest block size (general engine for the applies and token sums,
    # 8 x 8 tiles per block in the CNP products)
    _cfg("bf16_b1024", 200, 2048, 1024, 1024, 1024, "bf16", "bf16", 28),
    # b = 512 with a short last block on R (1280 = 2*512 + 256)
    _cfg("bf16_b512_ragged", 260, 1280, 1024, 512, 512, "bf16", "bf16", 29),
    # b = 512 with a last P block shorter than half a block (1672 = 3*512 + 136)
    # and a ragged token count
    _cfg("bf16_b512_ragged_p", 97, 1024, 1672, 512, 512, "bf16", "bf16", 35),
    # b = 128 with short last blocks on both sides (704 = 5*128 + 64, 392 = 3*128 + 8)
    _cfg("bf16_b128_ragged", 150, 704, 392, 128, 128, "bf16", "bf16", 32),
    # shallowest dense products: K = 64 forward (one K step), K = 128 backward (two)
    _cfg("bf16_k64", 300, 64, 128, 32, 64, "bf16", "bf16", 33),
    # ragged token count and output width across several 256 x 256 output tiles
    _cfg("bf16_ragged_tiles", 1100, 320, 1800, 64, 64, "bf16", "bf16", 34),
    # fewer output tiles than CUs and K >= 2048: both dense products split
    # every tile into four K parts, whose fp32 partial tiles a second kernel
    # adds in fixed part order
    _cfg("bf16_split_k", 300, 2048, 2304, 256, 256, "bf16", "bf16", 36),
    # the same with an int8 weight: codes converted to bfloat16 inside the
    # dense kernel, column scales in the split sum's epilogue
    _cfg("xq_split_k", 300, 2048, 2304, 256, 256, "bf16", "i8", 39),
    _cfg("xf8_split_k", 300, 2048, 2304, 256, 256, "bf16", "f8", 67),
    # one block per side: R's block size exceeds m (a single short block of
    # 64), P is exactly one block
    _cfg("f32_single_block", 50, 64, 128, 128, 128, "f32", "f32", 47),
    _cfg("bf16_single_block", 130, 192, 256, 256, 256, "bf16", "bf16", 48),
    # block sizes that are multiples of 8 but not powers of two, with short
    # last blocks (general engine for applies, token sums and CNP products)
    _cfg("bf16_b96_b40", 210, 480, 600, 96, 40, "bf16", "bf16", 49),
    _cfg("f32_b24_b56", 70, 120, 200, 24, 56, "f32", "f32", 53),
    # the smallest block size the library takes, b = 8
    _cfg("f32_b8", 40, 48, 64, 8, 8, "f32", "f32", 54),
    _cfg("bf16_b8", 40, 48, 64, 8, 8, "bf16", "bf16", 55),
    # a weight width that ends inside a 64-column tile of the merge's left
    # product (1000 = 15*64 + 40), with a short last P block (1000 = 3*256 + 232)
    _cfg("bf16_left_ragged_cols", 200, 512, 1000, 256, 256, "bf16", "bf16", 56),
    # int8 weight whose widths are not multiples of 64 (the dense kernel's K
    # step): the forward multiplies a bfloat16 copy of the codes in the general
    # engine, the backward reads the codes in the general engine; short last
    # blocks of 16 on both sides (528 = 4*128 + 16, 1040 = 8*128 + 16)
    _cfg("xq_widths_not_64", 200, 528, 1040, 128, 128, "bf16", "i8", 57),
    # weight rows wider than the LDS-staged gathers take (float32 65 568 bytes,
    # bfloat16 past 16384 columns): the z scatter, the dx scatter and the
    # merge's reframe gather from global memory, and the work the apply and
    # gather launches otherwise carry (inverse permutations, q <- 0) runs in
    # launches of its own; last P blocks of 8 and 16
    _cfg("f32_wide_rows", 8, 64, 16392, 64, 512, "f32", "f32", 60),
    _cfg("bf16_wide_rows", 8, 64, 16400, 64, 256, "bf16", "bf16", 61),
    # the backward dense product in its persistent form (whole rounds of
    # 256 x 256 tiles over the 256 CUs): two tiles per workgroup, the second's
    # first K slice loaded during the first's last step (8192 x 4096 output,
    # K = 1024), and one tile per workgroup (4096 x 4096, K = 512)
    _cfg("bf16_persistent_bwd", 8192, 4096, 1024, 256, 256, "bf16", "bf16", 62),
    _cfg("bf16_persistent_bwd_one", 4096, 4096, 512, 256, 256, "bf16", "bf16", 63),
]


@pytest.mark.parametrize("cfg", SMALL, ids=lambda c: c.name)
def test_layer_parity(cfg):
    L, A, out, _ = _run(cfg, merge=(cfg.weight not in ("i8", "f8")))
    W0 = _w0_values(cfg, L)
    args = (W0, L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], cfg.b_r, cfg.b_p)
    ref = O.backward(A["X"], A["dZ"], *args)
    f = ref["fwd"]
    tol = TOL[cfg.act]
    errs = {
        "cnp_r": rel(out["g_r"], _expected_planes(L["q_r"], cfg.m, cfg.b_r)),
        "cnp_p": rel(out["g_p"], _expected_planes(L["q_p"], cfg.n, cfg.b_p)),
        "x1": rel(out["x1"], f["X1"]),
        "y1": rel(out["y1"], f["Y1"]),
        "z": rel(out["z"], f["Z"]),
        "dq_r": rel(out["dq_r"], ref["dq_r"]),
        "dq_p": rel(out["dq_p"], ref["dq_p"]),
        "dx": rel(out["dx"], ref["dX"]),
    }
    if "w0_merged" in out:
        errs["merge"] = rel(out["w0_merged"], O.merge(*args))
        assert np.all(out["q_after"] == 0.0)
        # the resident weight is the merged one in the next frame, exactly
        assert np.array_equal(out["wp_merged"], O.permuted_weight(out["w0_merged"], *out["perm_next"]))
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad
    # X1 is a pure permutation of X: bit-exact
    assert np.array_equal(out["x1"], A["X"][:, L["perm_r"]].astype(np.float64))


def test_merge_preserves_the_layer_function():
    cfg = _cfg("merge_invariant", 64, 256, 384, 64, 64, "f32", "f32", 27)
    L, A, out, dl = _run(cfg, merge=True)
    # after the merge q = 0 and the forward through the merged weight must
    # reproduce the forward before it
    dl.cnp_build()
    z2 = to_host_f64(dl.forward(to_device(A["X_raw"], cfg.act)))
    torch.cuda.synchronize()
    assert rel(z2, out["z"]) <= 1e-5


@pytest.mark.parametrize("cfg", [
    _cfg("merge_resample_f32", 96, 256, 384, 64, 64, "f32", "f32", 37),
    _cfg("merge_resample_bf16", 300, 512, 768, 256, 256, "bf16", "bf16", 38),
], ids=lambda c: c.name)
def test_merge_then_new_permutations_keep_the_function(cfg):
    # after a merge q = 0, so the layer no longer depends on its permutations:
    # the weight merged into the frame of fresh ones (as drawn at a merge)
    # must give the forward from before the merge
    L, A, out, dl = _run(cfg, merge=True)
    dl.cnp_build()
    z2 = to_host_f64(dl.forward(to_device(A["X_raw"], cfg.act)))
    torch.cuda.synchronize()
    err = rel(z2, out["z"])
    print(f"rel {err:.2e}", flush=True)
    assert err <= TOL[cfg.act]


@pytest.mark.parametrize("cfg", [
    # b = 256 on the R side: left block product on the rows of Wp
    _cfg("merge_zero_q_b256", 16, 640, 1088, 256, 256, "bf16", "bf16", 35),
    # other block sizes: the left product between two transposes
    _cfg("merge_zero_q_b128", 16, 384, 704, 128, 128, "bf16", "bf16", 36),
], ids=lambda c: c.name)
def test_merge_with_zero_q_leaves_w0_unchanged(cfg):
    # q = 0 makes every G and H the identity, so R W0 P = W0 exactly; both
    # roundings to bfloat16 then return the stored values bit for bit, in the
    # same frame and, after a merge into new permutations, in theirs
    print(f"\n[gpu] {cfg.name} m={cfg.m} n={cfg.n} b={cfg.b_r}/{cfg.b_p}", flush=True)
    L = synth.make_layer(cfg, 0)
    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, cfg.act, cfg.weight, cfg.T)
    dl.load(L)
    dl.q_r.zero_()
    dl.q_p.zero_()
    dl.cnp_build()
    before = dl.wp.clone()
    dl.merge()
    torch.cuda.synchronize()
    assert torch.equal(dl.wp.view(torch.int16), before.view(torch.int16))
    rng = np.random.default_rng(12)
    nr, np_ = rng.permutation(cfg.m).astype(np.int32), rng.permutation(cfg.n).astype(np.int32)
    dl.merge(to_device(nr, "i32"), to_device(np_, "i32"))
    torch.cuda.synchronize()
    bits = L["W0_raw"].view(np.int16)[nr][:, np_]
    assert np.array_equal(dl.wp.view(torch.int16).cpu().numpy(), bits)


# ---------------------------------------------------------------------------
# bit-exact index work
# ---------------------------------------------------------------------------

def _round_robin(b):
    """b-1 perfect matchings of {0..b-1} that together cover every pair once."""
    rounds = []
    for r in range(b - 1):
        pairs = [(r, b - 1)]
        for k in range(1, b // 2):
            pairs.append(((r + k) % (b - 1), (r - k) % (b - 1)))
        rounds.append([(min(p), max(p)) for p in pairs])
    return rounds


@pytest.mark.parametrize("act,s,b", [("f32", 2.0 ** -4, 16), ("bf16", 0.25, 16), ("bf16", 0.25, 128),
                                      ("bf16", 0.25, 256)])
def test_packing_bit_exact(act, s, b):
    # One perfect matching of nonzero q per block: every Q is a direct sum of
    # 2 x 2 rotation generators, so G - I has exactly representable entries
    # diag -2s^2 + s^4 and off-diagonal +-(2s - 2s^3) at the matched pairs
    # (as are Q^2, 2Q + Q^2 and their product on the way). b = 16 runs the
    # general product engine, b = 128 and 256 the fused block products.
    nblk = 4
    m = n = b * nblk
    dl = DeviceLayer(m, n, b, b, act, act, 8)
    rounds = _round_robin(b)
    iu = {p: k for k, p in enumerate(zip(*np.triu_indices(b, 1)))}
    L = b * (b - 1) // 2
    seen = set()
    for call in range(-(-len(rounds) // nblk)):
        q = np.zeros(nblk * L, np.float32)
        expect = np.zeros((nblk, b, b))
        for z in range(nblk):
            ridx = (call * nblk + z) % len(rounds)
            for (i, l) in rounds[ridx]:
                q[z * L + iu[(i, l)]] = s
                expect[z, i, i] = expect[z, l, l] = -2 * s * s + s ** 4
                expect[z, i, l] = 2 * s - 2 * s ** 3
                expect[z, l, i] = -(2 * s - 2 * s ** 3)
                seen.add((i, l))
        dl.q_r.copy_(torch.from_numpy(q))
        dl.q_p.copy_(torch.from_numpy(q))
        dl.cnp_build()
        torch.cuda.synchronize()
        for side in (px.POETX_SIDE_R, px.POETX_SIDE_P):
            planes = to_host_f64(dl.g_planes(side))
            assert np.array_equal(planes[0], expect), (call, side)
            assert np.array_equal(planes[1], expect.transpose(0, 2, 1)), (call, side)
    assert len(seen) == L


def _shift(b, k):
    S = np.zeros((b, b))
    S[np.arange(b), (np.arange(b) + k) % b] = 1.0
    return S


@pytest.mark.parametrize("act,b,T", [("f32", 16, 40), ("bf16", 16, 40), ("bf16", 256, 1100)])
def test_permutations_bit_exact(act, b, T):
    # G_j, H_k cyclic shifts (0/1 matrices), W0 = I and small-integer X, dZ:
    # every value stays a small integer, so z and dx are exact index shuffles
    # of the inputs and any correct implementation matches bit for bit.
    # b = 256 with T > m runs the dedicated apply kernel and the backward's
    # fold of H into the weight.
    nblk = 4
    m = n = b * nblk
    rng = np.random.default_rng(5)
    perm_r, perm_p = rng.permutation(m), rng.permutation(n)
    X = rng.integers(-8, 9, size=(T, m)).astype(np.float32)
    dZ = rng.integers(-8, 9, size=(T, n)).astype(np.float32)
    Gs = [_shift(b, 1 + j % 3) for j in range(nblk)]
    Hs = [_shift(b, 2 + k % 5) for k in range(nblk)]
    dl = DeviceLayer(m, n, b, b, act, act, T)
    eye = np.eye(m, dtype=np.float32)
    dl.load(dict(W0_raw=synth.bf16_bits(eye) if act == "bf16" else eye, w_scale=None,
                 perm_r=perm_r, perm_p=perm_p, q_r=np.zeros(dl.q_r.numel(), np.float32),
                 q_p=np.zeros(dl.q_p.numel(), np.float32)))
    for side, blocks in ((px.POETX_SIDE_R, Gs), (px.POETX_SIDE_P, Hs)):
        D = np.stack([g - np.eye(b) for g in blocks])
        host = np.stack([D, D.transpose(0, 2, 1)]).astype(np.float32)
        dev = to_device(synth.bf16_bits(host) if act == "bf16" else host, act)
        dl.g_planes(side).copy_(dev.view(dl.g_planes(side).shape))
    raw = (lambda a: synth.bf16_bits(a)) if act == "bf16" else (lambda a: a)
    z = to_host_f64(dl.forward(to_device(raw(X), act)))
    _, _, dx = dl.backward(to_device(raw(dZ), act))
    dx = to_host_f64(dx)
    torch.cuda.synchronize()
    R = O.dense_block_orthogonal(Gs, perm_r, b)
    P = O.dense_block_orthogonal(Hs, perm_p, b)
    Weff = R @ np.eye(m) @ P
    assert np.array_equal(z, X.astype(np.float64) @ Weff)
    assert np.array_equal(dx, dZ.astype(np.float64) @ Weff.T)
    # the permuted-frame weight is Psi W0 Phi^T exactly
    assert np.array_equal(to_host_f64(dl.wp), O.permuted_weight(np.eye(m), perm_r, perm_p))
    # and the export returns W0 itself
    assert np.array_equal(to_host_f64(dl.export_w0()[0]), np.eye(m))


# ---------------------------------------------------------------------------
# determinism, empty input, token-shard linearity
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [
    _cfg("determinism", 1024, 512, 768, 128, 128, "bf16", "bf16", 28),
    # dense products split along K: the partials are summed in part order by
    # a second kernel, so the result must not depend on which part ends first
    _cfg("determinism_split_k", 300, 2048, 2304, 256, 256, "bf16", "bf16", 36),
], ids=lambda c: c.name)
def test_layer_is_deterministic(cfg):
    _, A, out1, dl = _run(cfg)
    for _ in range(2):
        z = dl.forward(to_device(A["X_raw"], cfg.act))
        dq_r, dq_p, dx = dl.backward(to_device(A["dZ_raw"], cfg.act))
        torch.cuda.synchronize()
        assert np.array_equal(to_host_f64(z), out1["z"])
        assert np.array_equal(to_host_f64(dq_r), out1["dq_r"])
        assert np.array_equal(to_host_f64(dq_p), out1["dq_p"])
        assert np.array_equal(to_host_f64(dx), out1["dx"])


def test_zero_tokens():
    dl = DeviceLayer(64, 64, 16, 16, "bf16", "bf16", 0)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    z = dl.forward(x)
    assert z.shape == (0, 64)
    dq_r = torch.full_like(dl.q_r, 7.0)
    dq_p = torch.full_like(dl.q_p, 7.0)
    dl.backward(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), dq_r, dq_p)
    torch.cuda.synchronize()
    assert float(dq_r.abs().max()) == 0.0 and float(dq_p.abs().max()) == 0.0


def test_token_shard_linearity():
    # data parallelism exchanges only the packed gradients: the dq of a batch
    # equals the sum of the dq of its token shards
    cfg = _cfg("shards", 300, 256, 320, 64, 64, "f32", "f32", 29)
    L = synth.make_layer(cfg, 0)
    A = synth.make_activations(cfg, 0)
    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, "f32", "f32", cfg.T)
    dl.load(L)
    dl.cnp_build()
    res = []
    for sl in (slice(0, 300), slice(0, 120), slice(120, 300)):
        dl.forward(to_device(A["X_raw"][sl], "f32"))
        dq_r, dq_p, _ = dl.backward(to_device(A["dZ_raw"][sl], "f32"))
        res.append((to_host_f64(dq_r), to_host_f64(dq_p)))
    torch.cuda.synchronize()
    assert rel(res[1][0] + res[2][0], res[0][0]) <= 1e-5
    assert rel(res[1][1] + res[2][1], res[0][1]) <= 1e-5


# ---------------------------------------------------------------------------
# full-size workloads, sampled outputs
# ---------------------------------------------------------------------------

FULL = ["llama3b_proj", "llama8b_mlp_up", "llama13b_q_proj", "llama13b_down_proj", "xq_llama8b_mlp_up",
        "xf8_llama8b_mlp_up"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    cfg = synth.CONFIGS[name]
    L, A, out, _ = _run(cfg, merge=cfg.merge)
    W0 = _w0_values(cfg, L)
    args = (W0, L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], cfg.b_r, cfg.b_p)
    rng = np.random.default_rng(123)
    rows = np.sort(rng.choice(cfg.T, size=16, replace=False))
    rows[-1] = cfg.T - 1
    sub = O.backward(A["X"][rows], A["dZ"][rows], *args)
    nR, nP = -(-cfg.m // cfg.b_r), -(-cfg.n // cfg.b_p)
    br, bp = [0, nR - 1], [nP // 2]
    dqr_ref, dqp_ref = O.backward_blocks(A["X"], A["dZ"], *args, br, bp)
    Lr, Lp = cfg.b_r * (cfg.b_r - 1) // 2, cfg.b_p * (cfg.b_p - 1) // 2
    errs = {
        "z_rows": rel(out["z"][rows], sub["fwd"]["Z"]),
        "dx_rows": rel(out["dx"][rows], sub["dX"]),
        "y1_rows": rel(out["y1"][rows], sub["fwd"]["Y1"]),
    }
    for j in br:
        errs[f"dq_r[{j}]"] = rel(out["dq_r"][j * Lr:j * Lr + dqr_ref[j].size], dqr_ref[j])
    for k in bp:
        errs[f"dq_p[{k}]"] = rel(out["dq_p"][k * Lp:k * Lp + dqp_ref[k].size], dqp_ref[k])
    if cfg.merge:
        errs["merge"] = rel(out["w0_merged"], O.merge(*args))
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    bad = {k: v for k, v in errs.items() if not v <= TOL[cfg.act]}
    assert not bad, bad


def test_profile_log_records_every_step():
    cfg = _cfg("profile", 128, 256, 384, 64, 64, "bf16", "bf16", 30)
    px.poetx_profile_enable(1)
    try:
        _run(cfg)
    finally:
        px.poetx_profile_enable(0)
    names = [px.poetx_profile_get(i)[0] for i in range(px.poetx_profile_count())]
    for want in ("cnp_build", "gather_x", "apply_r_fwd", "gemm_dense_fwd", "apply_p_fwd",
                 "scatter_z", "gather_dz", "apply_p_bwd", "grad_h", "gemm_dense_bwd",
                 "apply_r_bwd", "grad_g", "cnp_bwd", "scatter_dx", "prepare_permute"):
        assert want in names, want
    assert all(px.poetx_profile_get(i)[1] >= 0.0 for i in range(len(names)))


def test_profile_log_fold_path():
    # more tokens than weight rows: the backward builds Wp H instead of dY2 H^T
    cfg = _cfg("profile_fold", 640, 256, 384, 128, 128, "bf16", "bf16", 31)
    px.poetx_profile_enable(1)
    try:
        _run(cfg)
    finally:
        px.poetx_profile_enable(0)
    names = [px.poetx_profile_get(i)[0] for i in range(px.poetx_profile_count())]
    assert "fold_h_bwd" in names and "apply_p_bwd" not in names, names


def test_profile_log_merged_token_sums():
    # equal bf16 block sizes of 256: one token-sum launch for both sides at
    # the end of the backward
    cfg = _cfg("profile_merged", 300, 512, 768, 256, 256, "bf16", "bf16", 59)
    px.poetx_profile_enable(1)
    try:
        _run(cfg)
    finally:
        px.poetx_profile_enable(0)
    names = [px.poetx_profile_get(i)[0] for i in range(px.poetx_profile_count())]
    assert "grad_gh" in names and "grad_g" not in names and "grad_h" not in names, names
