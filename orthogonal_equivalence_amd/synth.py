"""Seeded synthetic inputs for the POET-X layer.

This module only draws random numbers and rounds them to the storage types; it
holds none of the layer's arithmetic. Tests, the benchmark and the smoke check
feed the same arrays to the HIP library and to the float64 reference.

Every tensor comes from ``numpy.random.default_rng([seed, cfg_id, tensor_id])``
so that each one can be regenerated on its own:

  tensor_id 0  W0      ~ N(0, 0.02^2), shape (m, n)
  tensor_id 1  q_R     ~ N(0, sigma_q^2), packed upper triangles of R's blocks
  tensor_id 2  q_P     ~ N(0, sigma_q^2), packed upper triangles of P's blocks
  tensor_id 3  perm_R  = rng.permutation(m)
  tensor_id 4  perm_P  = rng.permutation(n)
  tensor_id 5  X       ~ N(0, 1), shape (T, m)
  tensor_id 6  dZ      ~ N(0, 1), shape (T, n)

Values are drawn in float32 and then rounded to the layer's storage type:
bfloat16 by round-to-nearest-even of the float32 bits; int8 base weights by
symmetric per-output-column absmax/127 quantisation with round-half-even and a
clamp to [-127, 127] (the storage format the quantised variant starts from);
fp8 base weights likewise per output column, scale absmax/448 and each value
w / scale converted to the OCP E4M3 byte by torch's float8_e4m3fn conversion
(round to nearest even).
"""

from dataclasses import dataclass
import numpy as np

__all__ = ["LayerConfig", "CONFIGS", "bf16_round", "bf16_bits", "from_bf16_bits",
           "quantize_int8_per_col", "quantize_fp8_per_col", "make_layer", "make_activations",
           "packed_count"]


@dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int
    T: int
    m: int
    n: int
    b_r: int
    b_p: int
    act: str            # "f32" or "bf16"
    weight: str         # "f32", "bf16", "i8" or "f8" (E4M3 byte)
    merge: bool = False
    sigma_w: float = 0.02
    sigma_q: float = 1e-3

    @property
    def tokens(self):
        return self.T


# Workloads of the pages' pre-training runs (Llama 3B / 8B / 13B at sequence
# length 2048), as single POET-X layers at one GPU's micro-batch.
CONFIGS = {
    c.name: c for c in [
        LayerConfig("tiny_f32", 0, 256, 512, 512, 64, 64, "f32", "f32"),
        LayerConfig("llama3b_proj", 1, 8 * 2048, 3072, 3072, 256, 256, "bf16", "bf16"),
        LayerConfig("llama8b_mlp_up", 2, 4 * 2048, 4096, 14336, 256, 256, "bf16", "bf16",
                    merge=True),
        LayerConfig("llama13b_q_proj", 3, 2 * 2048, 5120, 5120, 512, 512, "bf16", "bf16"),
        LayerConfig("llama13b_down_proj", 4, 2 * 2048, 13824, 5120, 512, 512, "bf16", "bf16"),
        LayerConfig("xq_llama8b_mlp_up", 5, 4 * 2048, 4096, 14336, 256, 256, "bf16", "i8"),
        LayerConfig("xf8_llama8b_mlp_up", 6, 4 * 2048, 4096, 14336, 256, 256, "bf16", "f8"),
    ]
}


def packed_count(dim, b):
    """Number of packed parameters for ceil(dim/b) blocks (last may be short)."""
    nblk = -(-dim // b)
    last = dim - (nblk - 1) * b
    return (nblk - 1) * (b * (b - 1) // 2) + last * (last - 1) // 2


def _rng(seed, cfg_id, tensor_id):
    return np.random.default_rng([seed, cfg_id, tensor_id])


def bf16_bits(x):
    """uint16 bfloat16 bit patterns of float32 x, round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def from_bf16_bits(h):
    """float32 values of uint16 bfloat16 bit patterns."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def bf16_round(x):
    """float32 array holding the bfloat16-rounded values of x."""
    return from_bf16_bits(bf16_bits(x))


def quantize_int8_per_col(w):
    """Symmetric per-column int8 storage: scale[c] = max_r |w[r, c]| / 127 in
    float32, q = clip(rint(w / scale), -127, 127)."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=0)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    q = np.clip(np.rint(w / scale[None, :]), -127, 127).astype(np.int8)
    return q, scale


def quantize_fp8_per_col(w):
    """Per-column E4M3 storage: scale[c] = max_r |w[r, c]| / 448 in float32,
    code = the E4M3 byte of w / scale (clamped to +-448 first: the float32
    division can land just past it)."""
    import torch

    w = np.asarray(w, dtype=np.float32)
    amax = np.abs(w).max(axis=0)
    scale = (amax / np.float32(448.0)).astype(np.float32)
    scale = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    x = np.clip(w / scale[None, :], -448.0, 448.0).astype(np.float32)
    q = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return q, scale


def _draw(rng, shape, sigma):
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def _store(x, kind):
    """Round a float32 array to the storage type; returns (values_f32, raw)."""
    if kind == "f32":
        return x, x
    if kind == "bf16":
        bits = bf16_bits(x)
        return from_bf16_bits(bits), bits
    raise ValueError(kind)


def make_layer(cfg, seed=0, m=None, n=None):
    """Layer state: W0 (values + raw storage), packed q_R, q_P, perm_R, perm_P.

    Returns a dict. ``W0`` is the float32 value array (exactly representable in
    the storage type), ``W0_raw`` the storage array (float32, uint16 bfloat16
    bits, int8, or uint8 E4M3 bytes), ``w_scale`` the per-column scale of an
    int8 or fp8 weight (else None).
    """
    m = cfg.m if m is None else m
    n = cfg.n if n is None else n
    w = _draw(_rng(seed, cfg.cfg_id, 0), (m, n), cfg.sigma_w)
    if cfg.weight in ("i8", "f8"):
        wq, scale = (quantize_int8_per_col if cfg.weight == "i8" else quantize_fp8_per_col)(w)
        # values are scale[c] * wq[r, c]; kept as (wq, scale) so that the
        # consumer forms the product in its own precision
        out = dict(W0_raw=wq, w_scale=scale, W0=None)
    else:
        vals, raw = _store(w, cfg.weight)
        out = dict(W0_raw=raw, w_scale=None, W0=vals)
    out["q_r"] = _draw(_rng(seed, cfg.cfg_id, 1), (packed_count(m, cfg.b_r),), cfg.sigma_q)
    out["q_p"] = _draw(_rng(seed, cfg.cfg_id, 2), (packed_count(n, cfg.b_p),), cfg.sigma_q)
    out["perm_r"] = _rng(seed, cfg.cfg_id, 3).permutation(m).astype(np.int32)
    out["perm_p"] = _rng(seed, cfg.cfg_id, 4).permutation(n).astype(np.int32)
    out["m"], out["n"] = m, n
    return out


def make_activations(cfg, seed=0, T=None, m=None, n=None):
    """X (T x m) and dZ (T x n) ~ N(0, 1) in the activation storage type.

    Returns dict with X, dZ (float32 values) and X_raw, dZ_raw (storage).
    """
    T = cfg.T if T is None else T
    m = cfg.m if m is None else m
    n = cfg.n if n is None else n
    x = _draw(_rng(seed, cfg.cfg_id, 5), (T, m), 1.0)
    dz = _draw(_rng(seed, cfg.cfg_id, 6), (T, n), 1.0)
    X, X_raw = _store(x, cfg.act)
    dZ, dZ_raw = _store(dz, cfg.act)
    return dict(X=X, X_raw=X_raw, dZ=dZ, dZ_raw=dZ_raw, T=T)
