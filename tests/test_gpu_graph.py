"""The layer step captured in a HIP graph (through torch.cuda.CUDAGraph) and
replayed: CNP build, forward, backward, draws of the next permutations and the
merge into their frame.

Every replay starts from the same layer state as an eager reference step and
must reproduce its outputs bit for bit. Eager steps and synchronisations run
between the replays, so a node that only works on its first replay would show.
"""

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from orthogonal_equivalence_amd import poetx as px  # noqa: E402
from orthogonal_equivalence_amd import synth  # noqa: E402
from orthogonal_equivalence_amd.device import DeviceLayer, to_device  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    torch.cuda.init()


def test_graph_replays_match_the_eager_step():
    cfg = synth.LayerConfig("graph_bf16", 90, 1000, 768, 1280, 256, 256, "bf16", "bf16")
    print(f"\n[gpu] {cfg.name} T={cfg.T} m={cfg.m} n={cfg.n}", flush=True)
    L = synth.make_layer(cfg, 0)
    A = synth.make_activations(cfg, 0)
    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, cfg.act, cfg.weight, cfg.T)
    dl.load(L)
    x = to_device(A["X_raw"], cfg.act)
    dz = to_device(A["dZ_raw"], cfg.act)
    z = dl.act_tensor(cfg.T, cfg.n)
    dx = dl.act_tensor(cfg.T, cfg.m)
    dq_r = torch.empty_like(dl.q_r)
    dq_p = torch.empty_like(dl.q_p)
    wp_0, qr_0, qp_0 = dl.wp.clone(), dl.q_r.clone(), dl.q_p.clone()
    cur_r, cur_p = dl.perm_r, dl.perm_p
    pr_0, pp_0 = cur_r.clone(), cur_p.clone()
    next_r, next_p = torch.empty_like(cur_r), torch.empty_like(cur_p)
    draw_ws = torch.empty(8 * max(cfg.m, cfg.n), dtype=torch.uint8, device="cuda")

    def reset():
        dl.wp.copy_(wp_0)
        dl.q_r.copy_(qr_0)
        dl.q_p.copy_(qp_0)
        cur_r.copy_(pr_0)
        cur_p.copy_(pp_0)
        dl.perm_r, dl.perm_p = cur_r, cur_p

    def step(stream=None):
        dl.cnp_build(stream)
        dl.forward(x, z, stream)
        dl.backward(dz, dq_r, dq_p, dx, stream)
        px.poetx_sample_perm(cfg.m, 7, 0, 1, next_r, draw_ws, None, stream)
        px.poetx_sample_perm(cfg.n, 7, 1, 1, next_p, draw_ws, None, stream)
        dl.merge(next_r, next_p, None, stream)
        dl.cnp_build(stream)

    def outputs():
        return [t.clone() for t in (z, dx, dq_r, dq_p, dl.wp, next_r, next_p, dl.q_r, dl.q_p, dl.g_r, dl.g_p)]

    reset()
    step()
    torch.cuda.synchronize()
    ref = outputs()

    # warm up on a side stream, then capture from the reset state
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs()
        names = ("z", "dx", "dq_r", "dq_p", "wp", "perm_r", "perm_p", "q_r", "q_p", "g_r", "g_p")
        bad = [nm for nm, a, b in zip(names, got, ref) if not torch.equal(a.view(torch.uint8), b.view(torch.uint8))]
        print(f"replay {rep}: {'bit-identical' if not bad else bad}", flush=True)
        assert not bad, (rep, bad)
        step()  # eager work between the replays
        torch.cuda.synchronize()
