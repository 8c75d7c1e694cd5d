"""Two layers driven at once from two host threads, each on its own stream.

The library keeps no state between calls (its only process-wide state is the
optional timing log, and the last-error record is per thread), so layers that
run concurrently on different streams must give exactly what they give when
run one after the other: the results are compared bit for bit.
"""

import threading

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from orthogonal_equivalence_amd import synth  # noqa: E402
from orthogonal_equivalence_amd.device import DeviceLayer, to_device  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible AMD GPU"
    torch.cuda.init()


CFGS = [
    synth.LayerConfig("conc_bf16", 80, 1000, 768, 1280, 256, 256, "bf16", "bf16"),
    synth.LayerConfig("conc_f32", 81, 300, 512, 384, 64, 64, "f32", "f32"),
]


def _setup(cfg):
    L = synth.make_layer(cfg, 0)
    A = synth.make_activations(cfg, 0)
    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, cfg.act, cfg.weight, cfg.T)
    dl.load(L)
    torch.cuda.synchronize()
    return dl, to_device(A["X_raw"], cfg.act), to_device(A["dZ_raw"], cfg.act)


def _step(dl, x, dz, out, stream):
    dl.cnp_build(stream=stream)
    dl.forward(x, out["z"], stream=stream)
    dl.backward(dz, out["dq_r"], out["dq_p"], out["dx"], stream=stream)


def _buffers(dl, x, dz):
    return {"z": torch.empty((x.shape[0], dl.n), dtype=x.dtype, device="cuda"),
            "dq_r": torch.empty_like(dl.q_r), "dq_p": torch.empty_like(dl.q_p), "dx": torch.empty_like(x)}


def test_two_layers_on_two_streams_match_sequential_runs():
    print("\n[gpu] two layers, two streams, two host threads", flush=True)
    layers = [_setup(c) for c in CFGS]
    ref = []
    for dl, x, dz in layers:
        out = _buffers(dl, x, dz)
        _step(dl, x, dz, out, torch.cuda.current_stream())
        torch.cuda.synchronize()
        ref.append({k: v.clone() for k, v in out.items()})

    streams = [torch.cuda.Stream() for _ in layers]
    outs = [_buffers(dl, x, dz) for dl, x, dz in layers]
    errors = []

    def run(i):
        try:
            dl, x, dz = layers[i]
            with torch.cuda.stream(streams[i]):
                for _ in range(3):
                    _step(dl, x, dz, outs[i], streams[i])
            streams[i].synchronize()
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(layers))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i, cfg in enumerate(CFGS):
        for k in ref[i]:
            assert torch.equal(outs[i][k], ref[i][k]), (cfg.name, k)
