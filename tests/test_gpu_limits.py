"""The HIP path at the edges of its size limits, against the float64 oracle.

- Token batches whose n-wide activations hold more than 2^31 elements (every
  offset into z, Y1 and dz past that point needs 64-bit arithmetic).
- Rows too wide for LDS staging (float32, n = 16392: 65 568 bytes) over more
  than 65535 tokens, so the row gathers loop past their capped grid.
- A tall int8 weight (m = 65537 * 64) whose transposes and column maxima run
  over more than 65535 row tiles and row bands.

The oracle cannot run the full backward at these sizes, so the tests use
properties that hold at any size. z and dx are token-local: their sampled rows
equal the oracle's on those rows alone. The packed gradients are linear in dz:
with dz zero outside the sampled rows they equal the oracle's gradients over
those rows, and every other row of dx is exactly zero. With q = 0 both
rotations are the identity, so the layer is z = x W0 (a plain matrix product),
and a merge stores the weight again exactly as the oracle's requantization of
it does, bit for bit.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from orthogonal_equivalence_amd import synth  # noqa: E402
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


def _w0_values(cfg, L):
    if cfg.weight == "i8":
        return O.dequantize(L["W0_raw"], L["w_scale"])
    return L["W0"].astype(np.float64)


def _sample_rows(T, must, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, size=16, replace=False).tolist()) | {0, T - 1} | set(must)
    return np.array(sorted(rows), dtype=np.int64)


def _sparse_dz(cfg, rows, seed):
    """dz rows for the sampled tokens: N(0, 1) in the activation type."""
    d = (np.random.default_rng(seed).standard_normal((len(rows), cfg.n), dtype=np.float32))
    if cfg.act == "bf16":
        bits = synth.bf16_bits(d)
        return synth.from_bf16_bits(bits), bits
    return d, d


BIG = [
    # Llama-style MLP width with a short input side: T * n = 2 148 020 224 > 2^31
    synth.LayerConfig("tokens_past_2e31_bf16", 70, 149834, 256, 14336, 256, 256, "bf16", "bf16"),
    synth.LayerConfig("tokens_past_2e31_xq", 71, 149834, 256, 14336, 256, 256, "bf16", "i8"),
    # float32 rows of 65 568 bytes over 65 736 tokens; last P block 8 wide
    synth.LayerConfig("wide_rows_f32", 72, 65736, 64, 16392, 64, 512, "f32", "f32"),
]


@pytest.mark.parametrize("cfg", BIG, ids=lambda c: c.name)
def test_large_batches_sampled(cfg):
    print(f"\n[gpu] {cfg.name} T={cfg.T} m={cfg.m} n={cfg.n} b={cfg.b_r}/{cfg.b_p} "
          f"{cfg.act}/{cfg.weight}", flush=True)
    L = synth.make_layer(cfg, 0)
    A = synth.make_activations(cfg, 0, n=8)    # X only; dz is built sparse below
    T = cfg.T
    past = -(-(1 << 31) // cfg.n)              # first token whose z row starts past 2^31 elements
    rows = _sample_rows(T, [r for r in (past, past + 1, 65535, 65536) if r < T], cfg.cfg_id)
    dz_vals, dz_raw = _sparse_dz(cfg, rows, cfg.cfg_id)

    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, cfg.act, cfg.weight, T)
    dl.load(L)
    dl.cnp_build()
    x = to_device(A["X_raw"], cfg.act)
    z = dl.forward(x)
    rows_d = torch.from_numpy(rows).cuda()
    z_rows = to_host_f64(z.index_select(0, rows_d))
    del z
    dz = torch.zeros((T, cfg.n), dtype=x.dtype, device="cuda")
    dz[rows_d] = to_device(dz_raw, cfg.act)
    dq_r, dq_p, dx = dl.backward(dz)
    keep = torch.ones(T, dtype=torch.bool, device="cuda")
    keep[rows_d] = False
    dx_rest_max = float(dx[keep].abs().max())
    dx_rows = to_host_f64(dx.index_select(0, rows_d))
    torch.cuda.synchronize()

    W0 = _w0_values(cfg, L)
    args = (W0, L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], cfg.b_r, cfg.b_p)
    ref = O.backward(A["X"][rows], dz_vals, *args)
    errs = {
        "z_rows": rel(z_rows, ref["fwd"]["Z"]),
        "dx_rows": rel(dx_rows, ref["dX"]),
        "dq_r": rel(to_host_f64(dq_r), ref["dq_r"]),
        "dq_p": rel(to_host_f64(dq_p), ref["dq_p"]),
    }
    print({k: f"{v:.2e}" for k, v in errs.items()}, f"rows {rows.tolist()}", flush=True)
    assert dx_rest_max == 0.0
    bad = {k: v for k, v in errs.items() if not v <= TOL[cfg.act]}
    assert not bad, bad


def test_tall_int8_weight_with_identity_rotations():
    cfg = synth.LayerConfig("tall_xq", 73, 40, 65537 * 64, 16, 128, 16, "bf16", "i8")
    print(f"\n[gpu] {cfg.name} T={cfg.T} m={cfg.m} n={cfg.n} b={cfg.b_r}/{cfg.b_p}", flush=True)
    L = synth.make_layer(cfg, 0)
    A = synth.make_activations(cfg, 0)
    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, cfg.act, cfg.weight, cfg.T)
    dl.load(L)
    dl.q_r.zero_()
    dl.q_p.zero_()
    dl.cnp_build()
    z = to_host_f64(dl.forward(to_device(A["X_raw"], cfg.act)))
    _, _, dx = dl.backward(to_device(A["dZ_raw"], cfg.act))
    dx = to_host_f64(dx)
    dl.merge()
    w0, w_scale = dl.export_w0()
    torch.cuda.synchronize()
    codes = w0.cpu().numpy().view(np.int8).reshape(cfg.m, cfg.n)
    scale = w_scale.cpu().numpy().astype(np.float32)

    W0 = _w0_values(cfg, L)
    X = A["X"].astype(np.float64)
    dZ = A["dZ"].astype(np.float64)
    errs = {"z": rel(z, X @ W0), "dx": rel(dx, dZ @ W0.T)}
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert max(errs.values()) <= TOL["bf16"], errs
    # with R = P = I the oracle's merge_xq is the weight stored again
    ref_codes, ref_scale = O.requantize_int8_per_col(O.dequantize(L["W0_raw"], L["w_scale"]))
    assert np.array_equal(codes, ref_codes)
    assert np.array_equal(scale, ref_scale)
