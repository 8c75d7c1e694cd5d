"""poetx_sample_perm_static (the permutation draw that allocates nothing)
against poetx_sample_perm (the same draw with a caller's workspace).

A draw is index work, so the two must agree bit for bit. Two calls in a row,
the second smaller than the first, check that nothing the first call leaves
in the shared scratch reaches the second; a third at the largest accepted
size checks the scratch's full extent.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
from orthogonal_equivalence_amd import poetx as px  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    torch.cuda.init()


def _with_workspace(dim, seed, tag, draw):
    perm = torch.full((dim,), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(8 * dim, dtype=torch.uint8, device="cuda")
    px.poetx_sample_perm(dim, seed, tag, draw, perm, ws)
    return perm


def _static(dim, seed, tag, draw):
    perm = torch.full((dim,), -1, dtype=torch.int32, device="cuda")
    px.poetx_sample_perm_static(dim, seed, tag, draw, perm)
    return perm


@pytest.mark.parametrize("calls", [
    [(14336, 2024, 1, 1), (4096, 2024, 0, 1)],
    [(100003, 7, 9, 3), (65, 7, 3, 1), (1 << 20, 3, 6, 7)],
], ids=["8b_widths", "odd_then_largest"])
def test_static_draw_equals_workspace_draw(calls):
    for dim, seed, tag, draw in calls:
        print(f"\n[gpu] sample_perm_static dim={dim} seed={seed} tag={tag} draw={draw}", flush=True)
        got = _static(dim, seed, tag, draw)
        want = _with_workspace(dim, seed, tag, draw)
        torch.cuda.synchronize()
        assert torch.equal(got, want), dim
        if dim <= 1 << 17:
            assert np.array_equal(got.cpu().numpy().astype(np.int64), O.sample_perm(dim, seed, tag, draw))


def test_static_draw_on_a_side_stream():
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = torch.full((4096,), -1, dtype=torch.int32, device="cuda")
        px.poetx_sample_perm_static(4096, 5, 6, 7, got, stream=s)
    s.synchronize()
    want = _with_workspace(4096, 5, 6, 7)
    torch.cuda.synchronize()
    assert torch.equal(got, want)


def test_static_draw_rejects_sizes_beyond_the_scratch():
    perm = torch.empty(16, dtype=torch.int32, device="cuda")
    with pytest.raises(px.PoetxError) as e:
        px.poetx_sample_perm_static((1 << 20) + 1, 1, 2, 3, perm)
    assert e.value.status == px.POETX_EUNSUPPORTED
