"""Merge of an int8 or fp8 (E4M3) base weight on the GPU against the float64
oracle's merge_xq (dequantize, W0 <- R W0 P, store per output column again).

The code of an element is decided in float32 on both sides, from merged
values that differ by rounding (the oracle's are float64, the GPU's come from
bfloat16 CNP planes and float32 products). So codes must agree exactly
wherever the oracle's unrounded value lies clear of a rounding boundary, and
within one step everywhere; the scales (column maxima) within the products'
rounding.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from orthogonal_equivalence_amd import synth  # noqa: E402
from orthogonal_equivalence_amd.device import DeviceLayer, to_device  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    torch.cuda.init()


def _cfg(name, T, m, n, b_r, b_p, cfg_id, weight="i8"):
    return synth.LayerConfig(name, cfg_id, T, m, n, b_r, b_p, "bf16", weight)


def _merge_on_gpu(cfg, L, zero_q=False):
    # merged into the frame of new permutations (as at a training loop's
    # merge), then exported to the original frame for the comparison
    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, cfg.act, cfg.weight, 16)
    dl.load(L)
    if zero_q:
        dl.q_r.zero_()
        dl.q_p.zero_()
    dl.cnp_build()
    rng = np.random.default_rng([cfg.cfg_id, 98])
    nr, np_ = rng.permutation(cfg.m).astype(np.int32), rng.permutation(cfg.n).astype(np.int32)
    dl.merge(to_device(nr, "i32"), to_device(np_, "i32"))
    w0, w_scale = dl.export_w0()
    torch.cuda.synchronize()
    codes = w0.cpu().numpy().view(np.uint8 if cfg.weight == "f8" else np.int8).reshape(cfg.m, cfg.n)
    scale = w_scale.cpu().numpy().astype(np.float32)
    # the resident codes and scales are those in the new frame, exactly
    assert np.array_equal(dl.wp.cpu().numpy(), codes[nr][:, np_])
    assert np.array_equal(dl.wscale_p.cpu().numpy(), scale[np_])
    q_after = torch.cat([dl.q_r, dl.q_p]).cpu().numpy()
    return codes, scale, q_after


CASES = [
    _cfg("xq_merge_b128", 16, 512, 768, 128, 128, 50),
    # short last blocks on both sides
    _cfg("xq_merge_ragged", 16, 640, 1088, 256, 256, 51),
    # the Llama-8B MLP up-projection in int8
    synth.CONFIGS["xq_llama8b_mlp_up"],
    # the same three with an fp8 (E4M3) weight
    _cfg("xf8_merge_b128", 16, 512, 768, 128, 128, 64, "f8"),
    _cfg("xf8_merge_ragged", 16, 640, 1088, 256, 256, 65, "f8"),
    synth.CONFIGS["xf8_llama8b_mlp_up"],
]


def _fp8_boundaries(v):
    """For each unrounded code value v (float64): its distance from the
    nearest rounding boundary (midpoint between neighbouring E4M3 values),
    in units of the local step, and that step."""
    vals = O.fp8_e4m3_values()
    a = np.minimum(np.abs(v), O.FP8_MAX)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 1, 126)
    lo = hi - 1
    step = vals[hi] - vals[lo]
    return np.abs(a - (vals[lo] + vals[hi]) / 2) / step, step


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_xq_merge_matches_the_oracle(cfg):
    print(f"\n[gpu] {cfg.name} m={cfg.m} n={cfg.n} b={cfg.b_r}/{cfg.b_p}", flush=True)
    L = synth.make_layer(cfg, 0)
    codes, scale, q_after = _merge_on_gpu(cfg, L)
    assert np.all(q_after == 0.0)
    ref_codes, ref_scale, W = O.merge_xq(L["W0_raw"], L["w_scale"], L["q_r"], L["q_p"], L["perm_r"],
                                         L["perm_p"], cfg.b_r, cfg.b_p, fmt=cfg.weight)
    s_err = np.abs(scale.astype(np.float64) / ref_scale - 1.0).max()
    v = W / ref_scale.astype(np.float64)[None, :]             # the oracle's unrounded codes
    if cfg.weight == "f8":
        # The GPU's merged values carry an absolute error against the
        # oracle's (float32 products of bfloat16 CNP planes); the int8 case
        # below bounds it by 0.05 of an int8 step, 0.05 / 127 of the column
        # maximum, which is 0.05 * 448 / 127 = 0.176 in E4M3 code units.
        # E4M3 steps shrink towards zero (2^-9 code units for subnormals), so
        # a code is decided there by that absolute error: "clear of a
        # boundary" takes both 0.05 of the local step and 0.176 code units,
        # and the stored values agree within the larger of one step and twice
        # that error.
        ABS = 0.05 * 448 / 127
        dist, step_v = _fp8_boundaries(v)
        clear = (dist >= 0.05) & (dist * step_v >= ABS)
        differ = codes != ref_codes
        flips = int(np.count_nonzero(differ))
        print(f"scale rel err {s_err:.2e}; codes differing {flips} of {codes.size} "
              f"({np.count_nonzero(~clear)} elements near a boundary)", flush=True)
        assert s_err <= 1e-3
        assert not np.any(differ[clear])
        assert flips <= 0.01 * codes.size
        A = O.dequantize_fp8(codes, scale)
        B = O.dequantize_fp8(ref_codes, ref_scale)
        bound = (np.maximum(step_v, 2 * ABS) * (1 + 1e-6) + 448 * s_err) * ref_scale.astype(np.float64)[None, :]
        assert np.all(np.abs(A - B) <= bound + 1e-12)
        return
    clear = np.abs(np.abs(v - np.floor(v)) - 0.5) >= 0.05     # clear of a rounding boundary
    d = codes.astype(np.int32) - ref_codes.astype(np.int32)
    flips = int(np.count_nonzero(d))
    print(f"scale rel err {s_err:.2e}; codes differing {flips} of {d.size} "
          f"({np.count_nonzero(~clear)} elements near a boundary)", flush=True)
    assert s_err <= 1e-3
    assert np.abs(d).max() <= 1
    assert not np.any(d[clear])
    assert flips <= 0.01 * d.size
    # the stored weight against the oracle's: within one step everywhere, plus
    # what the scale difference makes of a code of up to 127
    A = O.dequantize(codes, scale)
    B = O.dequantize(ref_codes, ref_scale)
    step = ref_scale.astype(np.float64)[None, :]
    assert np.all(np.abs(A - B) <= step * (1 + 128 * s_err) + 1e-12)


@pytest.mark.parametrize("weight", ["i8", "f8"])
def test_xq_merge_with_zero_q_keeps_the_codes(weight):
    cfg = _cfg(f"{weight}_merge_zero_q", 16, 512, 768, 128, 128, 52, weight)
    print(f"\n[gpu] {cfg.name}", flush=True)
    L = synth.make_layer(cfg, 0)
    codes, scale, _ = _merge_on_gpu(cfg, L, zero_q=True)
    zr, zp = np.zeros_like(L["q_r"]), np.zeros_like(L["q_p"])
    ref_codes, ref_scale, _ = O.merge_xq(L["W0_raw"], L["w_scale"], zr, zp, L["perm_r"], L["perm_p"],
                                         cfg.b_r, cfg.b_p, fmt=weight)
    assert np.array_equal(codes, L["W0_raw"])
    assert np.array_equal(codes, ref_codes)
    assert np.array_equal(scale, ref_scale)
