"""ctypes binding of libpoetx.so (declared in include/poetx.h).

Argument marshalling only: every function has the name and argument order of
its C counterpart, pointers may be given as ints or as torch tensors (their
data_ptr()), ``stream=None`` means torch's current HIP stream, and a non-zero
status raises PoetxError. All computation happens in the library's HIP
kernels; importing this module fails if the library is not built.
"""

import ctypes
import os

# torch first: its libraries load the HIP runtime it ships (soname
# libamdhip64.so.7), which then also satisfies libpoetx.so's dependency, so the
# process holds one HIP runtime. Loaded the other way round, libpoetx.so would
# pull in the system runtime and torch a second one, and the two need not
# agree on the devices.
import torch  # noqa: F401,E402

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpoetx.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m orthogonal_equivalence_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

POETX_OK, POETX_EINVAL, POETX_EUNSUPPORTED, POETX_EHIP, POETX_EWORKSPACE = 0, 1, 2, 3, 4
POETX_F32, POETX_BF16, POETX_I8, POETX_F8 = 0, 1, 2, 3
POETX_SIDE_R, POETX_SIDE_P = 0, 1
(POETX_OP_CNP_BUILD, POETX_OP_WEIGHT_PREPARE, POETX_OP_FORWARD, POETX_OP_BACKWARD,
 POETX_OP_MERGE, POETX_OP_FORWARD_MEM, POETX_OP_BACKWARD_MEM, POETX_OP_SAMPLE_PERM,
 POETX_OP_WEIGHT_EXPORT) = range(9)

EXPORTED = [
    "poetx_abi_version", "poetx_strerror", "poetx_last_hip_error", "poetx_packed_len", "poetx_gbuf_bytes",
    "poetx_saved_bytes", "poetx_wbuf_bytes", "poetx_workspace_bytes", "poetx_cnp_build",
    "poetx_weight_prepare", "poetx_weight_export", "poetx_forward", "poetx_backward", "poetx_forward_mem", "poetx_backward_mem",
    "poetx_merge", "poetx_sample_perm", "poetx_sample_perm_static",
    "poetx_profile_enable", "poetx_profile_count", "poetx_profile_get",
]

_DTYPES = {"f32": POETX_F32, "bf16": POETX_BF16, "i8": POETX_I8, "f8": POETX_F8}


class poetx_layer(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("b_r", ctypes.c_int32),
                ("b_p", ctypes.c_int32), ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32)]


def make_layer(m, n, b_r, b_p, act="bf16", weight="bf16"):
    """poetx_layer from sizes and dtype names ("f32", "bf16", "i8")."""
    return poetx_layer(m, n, b_r, b_p, _DTYPES[act], _DTYPES[weight])


class PoetxError(RuntimeError):
    def __init__(self, fn, status):
        msg = f"{fn}: {poetx_strerror(status)} (status {status})"
        if status == POETX_EHIP:
            msg += f" [{poetx_last_hip_error()}]"
        super().__init__(msg)
        self.status = status


_P = ctypes.c_void_p
_L = ctypes.POINTER(poetx_layer)
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_sig = {
    "poetx_abi_version": (ctypes.c_int, []),
    "poetx_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "poetx_last_hip_error": (ctypes.c_char_p, []),
    "poetx_packed_len": (_SZ, [_L, ctypes.c_int]),
    "poetx_gbuf_bytes": (_SZ, [_L, ctypes.c_int]),
    "poetx_saved_bytes": (_SZ, [_L, _I64]),
    "poetx_wbuf_bytes": (_SZ, [_L]),
    "poetx_workspace_bytes": (_SZ, [_L, _I64, ctypes.c_int]),
    "poetx_cnp_build": (ctypes.c_int, [_L, _P, _P, _P, _P, _P, _SZ, _P]),
    "poetx_weight_prepare": (ctypes.c_int, [_L, _P, _P, _P, _P, _P, _P, _P]),
    "poetx_weight_export": (ctypes.c_int, [_L, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "poetx_forward": (ctypes.c_int, [_L, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "poetx_backward": (ctypes.c_int, [_L, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      _P, _P, _SZ, _P]),
    "poetx_forward_mem": (ctypes.c_int, [_L, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "poetx_backward_mem": (ctypes.c_int, [_L, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                          _P, _P, _SZ, _P]),
    "poetx_merge": (ctypes.c_int, [_L, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "poetx_sample_perm": (ctypes.c_int, [_I64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, _P, _P, _SZ,
                                         _P]),
    "poetx_sample_perm_static": (ctypes.c_int, [_I64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, _P,
                                                _P]),
    "poetx_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "poetx_profile_count": (ctypes.c_int, []),
    "poetx_profile_get": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                         ctypes.POINTER(ctypes.c_float)]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _size(ws, ws_bytes):
    if ws_bytes is not None:
        return ws_bytes
    if ws is None or isinstance(ws, int):
        return 0
    return ws.numel() * ws.element_size()


def _call(name, *args):
    st = getattr(_lib, name)(*args)
    if st != POETX_OK:
        raise PoetxError(name, st)


def poetx_abi_version():
    return _lib.poetx_abi_version()


def poetx_strerror(status):
    return _lib.poetx_strerror(status).decode()


def poetx_last_hip_error():
    return _lib.poetx_last_hip_error().decode()


def poetx_packed_len(L, side):
    return _lib.poetx_packed_len(ctypes.byref(L), side)


def poetx_gbuf_bytes(L, side):
    return _lib.poetx_gbuf_bytes(ctypes.byref(L), side)


def poetx_saved_bytes(L, T):
    return _lib.poetx_saved_bytes(ctypes.byref(L), T)


def poetx_wbuf_bytes(L):
    return _lib.poetx_wbuf_bytes(ctypes.byref(L))


def poetx_workspace_bytes(L, T, op):
    return _lib.poetx_workspace_bytes(ctypes.byref(L), T, op)


def poetx_cnp_build(L, q_r, q_p, g_r, g_p, ws=None, ws_bytes=None, stream=None):
    _call("poetx_cnp_build", ctypes.byref(L), _ptr(q_r), _ptr(q_p), _ptr(g_r), _ptr(g_p), _ptr(ws),
          _size(ws, ws_bytes), _stream(stream))


def poetx_weight_prepare(L, w0, w_scale, perm_r, perm_p, wp, wscale_p, stream=None):
    _call("poetx_weight_prepare", ctypes.byref(L), _ptr(w0), _ptr(w_scale), _ptr(perm_r), _ptr(perm_p),
          _ptr(wp), _ptr(wscale_p), _stream(stream))


def poetx_weight_export(L, wp, wscale_p, perm_r, perm_p, w0, w_scale, ws=None, ws_bytes=None, stream=None):
    _call("poetx_weight_export", ctypes.byref(L), _ptr(wp), _ptr(wscale_p), _ptr(perm_r), _ptr(perm_p),
          _ptr(w0), _ptr(w_scale), _ptr(ws), _size(ws, ws_bytes), _stream(stream))


def poetx_forward(L, T, x, perm_r, perm_p, g_r, g_p, wp, wscale_p, z, saved, ws=None, ws_bytes=None,
                  stream=None):
    _call("poetx_forward", ctypes.byref(L), T, _ptr(x), _ptr(perm_r), _ptr(perm_p), _ptr(g_r), _ptr(g_p),
          _ptr(wp), _ptr(wscale_p), _ptr(z), _ptr(saved), _ptr(ws), _size(ws, ws_bytes), _stream(stream))


def poetx_backward(L, T, saved, dz, perm_r, perm_p, q_r, q_p, g_r, g_p, wp, wscale_p, dq_r, dq_p, dx,
                   ws=None, ws_bytes=None, stream=None):
    _call("poetx_backward", ctypes.byref(L), T, _ptr(saved), _ptr(dz), _ptr(perm_r), _ptr(perm_p),
          _ptr(q_r), _ptr(q_p), _ptr(g_r), _ptr(g_p), _ptr(wp), _ptr(wscale_p), _ptr(dq_r), _ptr(dq_p),
          _ptr(dx), _ptr(ws), _size(ws, ws_bytes), _stream(stream))


def poetx_forward_mem(L, T, x, perm_r, perm_p, g_r, g_p, wp, wscale_p, z, ws=None, ws_bytes=None,
                      stream=None):
    _call("poetx_forward_mem", ctypes.byref(L), T, _ptr(x), _ptr(perm_r), _ptr(perm_p), _ptr(g_r), _ptr(g_p),
          _ptr(wp), _ptr(wscale_p), _ptr(z), _ptr(ws), _size(ws, ws_bytes), _stream(stream))


def poetx_backward_mem(L, T, x, dz, perm_r, perm_p, q_r, q_p, g_r, g_p, wp, wscale_p, dq_r, dq_p, dx,
                       ws=None, ws_bytes=None, stream=None):
    _call("poetx_backward_mem", ctypes.byref(L), T, _ptr(x), _ptr(dz), _ptr(perm_r), _ptr(perm_p),
          _ptr(q_r), _ptr(q_p), _ptr(g_r), _ptr(g_p), _ptr(wp), _ptr(wscale_p), _ptr(dq_r),
          _ptr(dq_p), _ptr(dx), _ptr(ws), _size(ws, ws_bytes), _stream(stream))


def _event(e):
    if e is None or isinstance(e, int):
        return e
    return e.cuda_event


def poetx_merge(L, wp, wscale_p, perm_r, perm_p, perm_r_next, perm_p_next, next_ready, g_r, g_p, q_r, q_p,
                ws=None, ws_bytes=None, stream=None):
    """next_ready: None, a raw hipEvent_t handle, or a torch.cuda.Event
    (recorded before the call)."""
    _call("poetx_merge", ctypes.byref(L), _ptr(wp), _ptr(wscale_p), _ptr(perm_r), _ptr(perm_p),
          _ptr(perm_r_next), _ptr(perm_p_next), _event(next_ready), _ptr(g_r), _ptr(g_p), _ptr(q_r), _ptr(q_p),
          _ptr(ws), _size(ws, ws_bytes), _stream(stream))


def poetx_sample_perm(dim, seed, tag, draw, perm, ws=None, ws_bytes=None, stream=None):
    _call("poetx_sample_perm", dim, seed, tag, draw, _ptr(perm), _ptr(ws), _size(ws, ws_bytes), _stream(stream))


def poetx_sample_perm_static(dim, seed, tag, draw, perm, stream=None):
    _call("poetx_sample_perm_static", dim, seed, tag, draw, _ptr(perm), _stream(stream))


def poetx_profile_enable(enable):
    _call("poetx_profile_enable", 1 if enable else 0)


def poetx_profile_count():
    return _lib.poetx_profile_count()


def poetx_profile_get(i):
    """(name, milliseconds) of recorded step i."""
    name = ctypes.c_char_p()
    ms = ctypes.c_float()
    _call("poetx_profile_get", i, ctypes.byref(name), ctypes.byref(ms))
    return name.value.decode(), ms.value
