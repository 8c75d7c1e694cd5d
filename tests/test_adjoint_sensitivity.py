"""The large-rotation GPU parity cases can see every product of the
Cayley-Neumann adjoint (CPU, oracle only).

The library forms dq from the block gradient U = dL/dG with a reduced
recurrence instead of the literal product rule. With Q skew, Us = (U + U^T)/2
and Uk = (U - U^T)/2 (zhichai.net digest of arXiv:2603.05500, section
"3. Cayley-Neumann 参数化优化", G = (I+Q)(I+Q+Q^2+Q^3)):

    H1 = 4 Uk - 2 (Q Us + Us Q)
    F  = -4 Us + 2 Uk Q + Q H1
    E  = 2 Uk + Q F,            dq = pack(E - E^T)

Five b x b products per block: Q Us, Us Q, Uk Q, Q H1, Q F. This test writes
the recurrence out on its own, checks that it equals the oracle's literal
adjoint, and then drops one product at a time. On the inputs of every case in
large_q_cases.py the change in dq must be large against the parity tolerance,
so a kernel that got any one product wrong would fail the GPU parity test of
that case. It also checks that the rotation is a large share of z, dx and the
merged weight there, so that the GPU test's comparison of those deltas
(z - X W0 and so on) measures the rotation arithmetic itself.
"""

import numpy as np
import pytest

import oracle as O
from large_q_cases import CASES
from orthogonal_equivalence_amd import synth

TOL = {"f32": 1e-5, "bf16": 2e-2}
PRODUCTS = ("QUs", "UsQ", "UkQ", "QH1", "QF")


def _recurrence(Q, U, drop=None):
    Us = (U + U.T) / 2
    Uk = (U - U.T) / 2
    zero = np.zeros_like(Q)
    QUs = zero if drop == "QUs" else Q @ Us
    UsQ = zero if drop == "UsQ" else Us @ Q
    H1 = 4 * Uk - 2 * (QUs + UsQ)
    UkQ = zero if drop == "UkQ" else Uk @ Q
    QH1 = zero if drop == "QH1" else Q @ H1
    F = -4 * Us + 2 * UkQ + QH1
    QF = zero if drop == "QF" else Q @ F
    E = 2 * Uk + QF
    return E[np.triu_indices(Q.shape[0], 1)] - E.T[np.triu_indices(Q.shape[0], 1)]


def _w0(cfg, L):
    if cfg.weight == "i8":
        return O.dequantize(L["W0_raw"], L["w_scale"])
    if cfg.weight == "f8":
        return O.dequantize_fp8(L["W0_raw"], L["w_scale"])
    return L["W0"].astype(np.float64)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("cfg,strength", CASES, ids=[c.name for c, _ in CASES])
def test_each_adjoint_product_is_visible(cfg, strength):
    L = synth.make_layer(cfg, 0)
    A = synth.make_activations(cfg, 0)
    W0 = _w0(cfg, L)
    args = (W0, L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], cfg.b_r, cfg.b_p)
    ref = O.backward(A["X"], A["dZ"], *args)
    tol = TOL[cfg.act]
    worst = {}
    for q, dim, b, blocks, want in ((L["q_r"], cfg.m, cfg.b_r, ref["dG"], ref["dq_r"]),
                                    (L["q_p"], cfg.n, cfg.b_p, ref["dH"], ref["dq_p"])):
        offs, sizes = O.packed_offsets(dim, b)
        Qs = [O.skew_from_packed(q[o:o + r * (r - 1) // 2], r) for o, r in zip(offs, sizes)]
        full = np.concatenate([_recurrence(Q, U) for Q, U in zip(Qs, blocks)])
        # the recurrence is the oracle's adjoint, rearranged
        assert _rel(full, want) < 1e-12
        # dq with Q set to zero inside the adjoint (U unchanged): the
        # Q-independent part, which the GPU test subtracts
        base = np.concatenate([O.project_to_packed(O.cnp_adjoint(np.zeros_like(Q), U))
                               for Q, U in zip(Qs, blocks)])
        for p in PRODUCTS:
            cut = np.concatenate([_recurrence(Q, U, p) for Q, U in zip(Qs, blocks)])
            whole = _rel(cut, full)
            delta = float(np.linalg.norm(cut - full) / np.linalg.norm(full - base))
            worst[p] = min(worst.get(p, (9, 9))[0], whole), min(worst.get(p, (9, 9))[1], delta)
    print(cfg.name, {p: f"{w:.3f}/{d:.3f}" for p, (w, d) in worst.items()})
    for p, (whole, delta) in worst.items():
        if strength == "strong":
            assert whole >= 4 * tol and delta >= 5 * tol, (p, whole, delta)
        else:
            assert delta >= 1.5 * tol, (p, delta)
    # the rotation's share of each compared tensor
    f = ref["fwd"]
    X = A["X"].astype(np.float64)
    dZ = A["dZ"].astype(np.float64)
    share = {
        "z": np.linalg.norm(f["Z"] - X @ W0) / np.linalg.norm(f["Z"]),
        "dx": np.linalg.norm(ref["dX"] - dZ @ W0.T) / np.linalg.norm(ref["dX"]),
        "merge": np.linalg.norm(O.merge(*args) - W0) / np.linalg.norm(W0),
    }
    assert min(share.values()) >= (0.5 if strength == "mid" else 0.85), share
