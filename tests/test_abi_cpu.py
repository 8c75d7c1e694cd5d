"""Host-side checks of libpoetx.so: it loads, exports every entry point that
include/poetx.h declares, reports sizes consistent with the layer's block
structure, and rejects invalid arguments before launching anything.

No test here reaches a kernel launch: every call either only computes sizes or
fails validation (fake but aligned pointers are never dereferenced)."""

import ctypes
import os
import re

import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "poetx.h")

px = pytest.importorskip("orthogonal_equivalence_amd.poetx", reason="libpoetx.so not built")

FAKE = 1 << 20  # aligned, never dereferenced


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"POETX_API\s+[\w\s\*]+?\b(poetx_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) == 21
    lib = ctypes.CDLL(px.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(px.EXPORTED) == names


def test_profile_log_host_side():
    px.poetx_profile_enable(1)
    assert px.poetx_profile_count() == 0
    with pytest.raises(px.PoetxError):
        px.poetx_profile_get(0)
    px.poetx_profile_enable(0)


def test_version_and_messages():
    assert px.poetx_abi_version() == 2
    for s in range(5):
        assert px.poetx_strerror(s)
    assert px.poetx_strerror(99) == "unknown status"


@pytest.mark.parametrize("m,n,b_r,b_p", [(512, 512, 64, 64), (4096, 14336, 256, 256), (40, 24, 16, 16),
                                         (13824, 5120, 512, 512)])
def test_sizes_match_block_structure(m, n, b_r, b_p):
    L = px.make_layer(m, n, b_r, b_p, "bf16", "bf16")
    assert px.poetx_packed_len(L, px.POETX_SIDE_R) == O.packed_len(m, b_r)
    assert px.poetx_packed_len(L, px.POETX_SIDE_P) == O.packed_len(n, b_p)
    nR, nP = -(-m // b_r), -(-n // b_p)
    assert px.poetx_gbuf_bytes(L, px.POETX_SIDE_R) == 2 * nR * b_r * b_r * 2
    assert px.poetx_gbuf_bytes(L, px.POETX_SIDE_P) == 2 * nP * b_p * b_p * 2
    assert px.poetx_saved_bytes(L, 100) == 100 * (m + n) * 2
    assert px.poetx_wbuf_bytes(L) == m * n * 2
    Lf = px.make_layer(m, n, b_r, b_p, "f32", "f32")
    assert px.poetx_saved_bytes(Lf, 3) == 3 * (m + n) * 4
    Lq = px.make_layer(m, n, b_r, b_p, "bf16", "i8")
    assert px.poetx_wbuf_bytes(Lq) == (m * n if m % 16 == 0 and n % 16 == 0 else 0)
    L8 = px.make_layer(m, n, b_r, b_p, "bf16", "f8")
    assert px.poetx_wbuf_bytes(L8) == (m * n if m % 64 == 0 and n % 64 == 0 else 0)
    for op in range(5):
        assert px.poetx_workspace_bytes(L, 4096, op) >= 0
    assert px.poetx_workspace_bytes(L, 4096, px.POETX_OP_FORWARD) >= 4096 * max(m, n) * 2


@pytest.mark.parametrize("bad", [
    dict(m=12, n=16, b_r=8, b_p=8),          # m not a multiple of 8
    dict(m=16, n=16, b_r=4, b_p=8),          # block below 8
    dict(m=16, n=16, b_r=12, b_p=8),         # block not a multiple of 8
    dict(m=16, n=16, b_r=2048, b_p=8),       # block above 1024
    dict(m=16, n=16, b_r=8, b_p=8, act="f32", weight="bf16"),
    dict(m=16, n=16, b_r=8, b_p=8, act="f32", weight="i8"),
    dict(m=24, n=32, b_r=8, b_p=8, act="bf16", weight="i8"),   # int8 rows need 16-byte multiples
    dict(m=16, n=16, b_r=8, b_p=8, act="f32", weight="f8"),
    dict(m=64, n=96, b_r=8, b_p=8, act="bf16", weight="f8"),   # fp8 widths need multiples of 64
    dict(m=(1 << 24) + 8, n=16, b_r=1024, b_p=8),               # more than 2^24 features
    dict(m=8 * 65535, n=8, b_r=8, b_p=8),                       # 65536 blocks over the two sides
])
def test_invalid_layers_are_rejected(bad):
    kw = dict(act="bf16", weight="bf16")
    kw.update(bad)
    L = px.make_layer(kw["m"], kw["n"], kw["b_r"], kw["b_p"], kw["act"], kw["weight"])
    assert px.poetx_packed_len(L, 0) == 0
    assert px.poetx_gbuf_bytes(L, 1) == 0
    with pytest.raises(px.PoetxError) as e:
        px.poetx_cnp_build(L, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, stream=0)
    assert e.value.status == px.POETX_EINVAL


def test_size_limits_at_their_edges():
    # the largest accepted feature count and block count
    L = px.make_layer(1 << 24, 8, 1024, 8, "bf16", "bf16")
    assert px.poetx_packed_len(L, px.POETX_SIDE_R) == O.packed_len(1 << 24, 1024)
    L = px.make_layer(8 * 65534, 8, 8, 8, "bf16", "bf16")     # 65534 + 1 blocks
    assert px.poetx_packed_len(L, px.POETX_SIDE_R) == O.packed_len(8 * 65534, 8)
    # tokens: up to 2^30
    L = px.make_layer(64, 64, 16, 16, "bf16", "bf16")
    assert px.poetx_saved_bytes(L, 1 << 30) == (1 << 30) * 128 * 2
    assert px.poetx_workspace_bytes(L, 1 << 30, px.POETX_OP_FORWARD) > 0
    assert px.poetx_saved_bytes(L, (1 << 30) + 1) == 0
    assert px.poetx_workspace_bytes(L, (1 << 30) + 1, px.POETX_OP_BACKWARD) == 0
    for call in (lambda T: px.poetx_forward(L, T, *([FAKE] * 9), FAKE, 1 << 62, stream=0),
                 lambda T: px.poetx_backward(L, T, *([FAKE] * 13), FAKE, 1 << 62, stream=0),
                 lambda T: px.poetx_forward_mem(L, T, *([FAKE] * 8), FAKE, 1 << 62, stream=0),
                 lambda T: px.poetx_backward_mem(L, T, *([FAKE] * 13), FAKE, 1 << 62, stream=0)):
        with pytest.raises(px.PoetxError) as e:
            call((1 << 30) + 1)
        assert e.value.status == px.POETX_EINVAL


def test_argument_errors_before_any_launch():
    L = px.make_layer(64, 64, 16, 16, "bf16", "bf16")
    ws_f = px.poetx_workspace_bytes(L, 32, px.POETX_OP_FORWARD)
    ws_b = px.poetx_workspace_bytes(L, 32, px.POETX_OP_BACKWARD)
    fwd = [FAKE] * 9
    # null / misaligned pointers
    for i in range(len(fwd)):
        args = list(fwd)
        args[i] = None if i % 2 == 0 else FAKE + 2
        if i == 6:   # wscale_p is ignored for bf16 weights
            continue
        with pytest.raises(px.PoetxError) as e:
            px.poetx_forward(L, 32, args[0], args[1], args[2], args[3], args[4], args[5], args[6], args[7],
                             args[8], FAKE, ws_f, stream=0)
        assert e.value.status == px.POETX_EINVAL, i
    # workspace too small
    with pytest.raises(px.PoetxError) as e:
        px.poetx_forward(L, 32, *([FAKE] * 9), FAKE, ws_f - 1, stream=0)
    assert e.value.status == px.POETX_EWORKSPACE
    with pytest.raises(px.PoetxError) as e:
        px.poetx_backward(L, 32, *([FAKE] * 13), FAKE, ws_b - 1, stream=0)
    assert e.value.status == px.POETX_EWORKSPACE
    # negative T
    with pytest.raises(px.PoetxError) as e:
        px.poetx_forward(L, -1, *([FAKE] * 9), FAKE, ws_f, stream=0)
    assert e.value.status == px.POETX_EINVAL
    # T = 0 forward is a no-op (no launch, no pointer use)
    px.poetx_forward(L, 0, *([None] * 9), None, 0, stream=0)
    # memory variant: its own workspace sizes, the same checks
    ws_fm = px.poetx_workspace_bytes(L, 32, px.POETX_OP_FORWARD_MEM)
    ws_bm = px.poetx_workspace_bytes(L, 32, px.POETX_OP_BACKWARD_MEM)
    saved = px.poetx_saved_bytes(L, 32)
    assert ws_fm == ws_f + saved
    assert ws_bm >= max(ws_f, ws_b) + saved
    with pytest.raises(px.PoetxError) as e:
        px.poetx_forward_mem(L, 32, *([FAKE] * 8), FAKE, ws_fm - 1, stream=0)
    assert e.value.status == px.POETX_EWORKSPACE
    with pytest.raises(px.PoetxError) as e:
        px.poetx_backward_mem(L, 32, *([FAKE] * 13), FAKE, ws_bm - 1, stream=0)
    assert e.value.status == px.POETX_EWORKSPACE
    with pytest.raises(px.PoetxError) as e:
        px.poetx_backward_mem(L, 32, None, *([FAKE] * 12), FAKE, ws_bm, stream=0)
    assert e.value.status == px.POETX_EINVAL
    px.poetx_forward_mem(L, 0, *([None] * 8), None, 0, stream=0)
    # cnp build: q without g
    with pytest.raises(px.PoetxError) as e:
        px.poetx_cnp_build(L, FAKE, None, None, None, FAKE, 1 << 30, stream=0)
    assert e.value.status == px.POETX_EINVAL
    # merge: every pointer but the event is required; an int8 weight needs
    # its scales (in and out)
    ws_mb = px.poetx_workspace_bytes(L, 0, px.POETX_OP_MERGE)
    margs = [FAKE, None, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE]
    for i in (0, 2, 3, 4, 5, 7, 8, 9, 10):
        a = list(margs)
        a[i] = None
        with pytest.raises(px.PoetxError) as e:
            px.poetx_merge(L, *a, FAKE, ws_mb, stream=0)
        assert e.value.status == px.POETX_EINVAL, i
    with pytest.raises(px.PoetxError) as e:
        px.poetx_merge(L, *margs, FAKE, ws_mb - 1, stream=0)
    assert e.value.status == px.POETX_EWORKSPACE
    Lq = px.make_layer(64, 64, 16, 16, "bf16", "i8")
    ws_m = px.poetx_workspace_bytes(Lq, 0, px.POETX_OP_MERGE)
    assert ws_m >= 2 * 64 * 64 * 4
    with pytest.raises(px.PoetxError) as e:
        px.poetx_merge(Lq, *margs, FAKE, ws_m, stream=0)
    assert e.value.status == px.POETX_EINVAL
    # int8 and fp8 weights need their scales
    for Lw in (Lq, px.make_layer(64, 64, 16, 16, "bf16", "f8")):
        with pytest.raises(px.PoetxError) as e:
            px.poetx_weight_prepare(Lw, FAKE, None, FAKE, FAKE, FAKE, FAKE, stream=0)
        assert e.value.status == px.POETX_EINVAL
    with pytest.raises(px.PoetxError) as e:
        px.poetx_weight_export(Lq, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 20, stream=0)
    assert e.value.status == px.POETX_EINVAL
    # export needs n int32 of workspace
    assert px.poetx_workspace_bytes(L, 0, px.POETX_OP_WEIGHT_EXPORT) == 64 * 4
    with pytest.raises(px.PoetxError) as e:
        px.poetx_weight_export(L, FAKE, None, FAKE, FAKE, FAKE, None, FAKE, 64 * 4 - 1, stream=0)
    assert e.value.status == px.POETX_EWORKSPACE


def test_sample_perm_argument_errors():
    big = 8 << 20
    for dim, ptr, ws, ws_bytes, status in [
            (0, FAKE, FAKE, big, px.POETX_EINVAL), (-5, FAKE, FAKE, big, px.POETX_EINVAL),
            (16, None, FAKE, big, px.POETX_EINVAL), (16, FAKE + 4, FAKE, big, px.POETX_EINVAL),
            ((1 << 20) + 1, FAKE, FAKE, 2 * big, px.POETX_EUNSUPPORTED),
            (16, FAKE, FAKE, 127, px.POETX_EWORKSPACE), (16, FAKE, None, 128, px.POETX_EINVAL),
            (16, FAKE, FAKE + 8, 128, px.POETX_EINVAL)]:
        with pytest.raises(px.PoetxError) as e:
            px.poetx_sample_perm(dim, 1, 2, 3, ptr, ws, ws_bytes, stream=0)
        assert e.value.status == status, (dim, ptr, ws, ws_bytes)
    # the layer's workspace query covers the wider side
    L = px.make_layer(4096, 14336, 256, 256, "bf16", "bf16")
    assert px.poetx_workspace_bytes(L, 0, px.POETX_OP_SAMPLE_PERM) == 8 * 14336


def test_sample_perm_static_argument_errors():
    # rejected on the host before the scratch is looked up or anything runs
    for dim, ptr, status in [(0, FAKE, px.POETX_EINVAL), (-5, FAKE, px.POETX_EINVAL),
                             (16, None, px.POETX_EINVAL), (16, FAKE + 4, px.POETX_EINVAL),
                             ((1 << 20) + 1, FAKE, px.POETX_EUNSUPPORTED),
                             (1 << 40, FAKE, px.POETX_EUNSUPPORTED)]:
        with pytest.raises(px.PoetxError) as e:
            px.poetx_sample_perm_static(dim, 1, 2, 3, ptr, stream=0)
        assert e.value.status == status, (dim, ptr)


def test_last_hip_error_without_failure():
    assert px.poetx_last_hip_error().startswith("hipSuccess")
