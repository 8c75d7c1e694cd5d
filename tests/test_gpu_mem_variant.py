"""Memory variant (forward saves nothing, backward recomputes X1 and Y1 from x)
against the saving variant and the float64 oracle.

The recompute runs the forward's own kernels on the same inputs, and every
kernel is deterministic, so z, dq_r, dq_p and dx must equal the saving
variant's bit for bit; one case also goes to the oracle at the layer's
tolerance.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from orthogonal_equivalence_amd import synth  # noqa: E402
from orthogonal_equivalence_amd.device import DeviceLayer, to_device, to_host_f64  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    torch.cuda.init()


def _cfg(name, T, m, n, b_r, b_p, act, weight, cfg_id):
    return synth.LayerConfig(name, cfg_id, T, m, n, b_r, b_p, act, weight)


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32)


CASES = [
    # bf16, more tokens than weight rows: the backward folds H into the weight
    _cfg("mem_bf16_fold", 700, 512, 768, 256, 256, "bf16", "bf16", 40),
    # bf16, fewer tokens than weight rows: dY1 = dY2 H^T is formed
    _cfg("mem_bf16_nofold", 200, 768, 512, 128, 128, "bf16", "bf16", 41),
    # float32 with short last blocks and a ragged token count
    _cfg("mem_f32_ragged", 77, 200, 136, 64, 64, "f32", "f32", 42),
    # int8 weight with per-column scales
    _cfg("mem_xq", 300, 512, 768, 128, 128, "bf16", "i8", 43),
    # the Llama-8B MLP up-projection itself
    synth.CONFIGS["llama8b_mlp_up"],
    # fewer output tiles than CUs and K >= 2048: both dense products split
    # along K, their partials in the workspace the recompute shares
    _cfg("mem_split_k", 300, 2048, 2304, 256, 256, "bf16", "bf16", 45),
    # the same with an int8 weight (its bfloat16 code copy is workspace too)
    _cfg("mem_xq_split_k", 300, 2048, 2304, 256, 256, "bf16", "i8", 46),
    # fp8 (E4M3) weight with per-column scales
    _cfg("mem_xf8", 300, 512, 768, 128, 128, "bf16", "f8", 47),
]


@pytest.mark.parametrize("cfg", CASES, ids=lambda c: c.name)
def test_memory_variant_equals_saving_variant(cfg):
    print(f"\n[gpu] {cfg.name} T={cfg.T} m={cfg.m} n={cfg.n} b={cfg.b_r}/{cfg.b_p} {cfg.act}/{cfg.weight}",
          flush=True)
    L = synth.make_layer(cfg, 0)
    A = synth.make_activations(cfg, 0)
    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, cfg.act, cfg.weight, cfg.T)
    dl.load(L)
    dl.cnp_build()
    x = to_device(A["X_raw"], cfg.act)
    dz = to_device(A["dZ_raw"], cfg.act)
    z = dl.forward(x)
    dq_r, dq_p, dx = dl.backward(dz)
    z_m = dl.forward_mem(x)
    dq_r_m, dq_p_m, dx_m = dl.backward_mem(x, dz)
    torch.cuda.synchronize()
    assert torch.equal(_bits(z_m), _bits(z))
    assert torch.equal(_bits(dq_r_m), _bits(dq_r))
    assert torch.equal(_bits(dq_p_m), _bits(dq_p))
    assert torch.equal(_bits(dx_m), _bits(dx))


def test_memory_variant_against_the_oracle():
    cfg = _cfg("mem_oracle", 300, 256, 384, 64, 64, "f32", "f32", 44)
    print(f"\n[gpu] {cfg.name} T={cfg.T} m={cfg.m} n={cfg.n}", flush=True)
    L = synth.make_layer(cfg, 0)
    A = synth.make_activations(cfg, 0)
    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, cfg.act, cfg.weight, cfg.T)
    dl.load(L)
    dl.cnp_build()
    x = to_device(A["X_raw"], cfg.act)
    dz = to_device(A["dZ_raw"], cfg.act)
    z = to_host_f64(dl.forward_mem(x))
    dq_r, dq_p, dx = (to_host_f64(t) for t in dl.backward_mem(x, dz))
    torch.cuda.synchronize()
    args = (L["W0"].astype(np.float64), L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], cfg.b_r, cfg.b_p)
    ref = O.backward(A["X"], A["dZ"], *args)

    def rel(a, b):
        return float(np.linalg.norm(a - b) / np.linalg.norm(b))

    errs = {"z": rel(z, ref["fwd"]["Z"]), "dq_r": rel(dq_r, ref["dq_r"]), "dq_p": rel(dq_p, ref["dq_p"]),
            "dx": rel(dx, ref["dX"])}
    print({k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
    assert all(v <= 1e-5 for v in errs.values()), errs
