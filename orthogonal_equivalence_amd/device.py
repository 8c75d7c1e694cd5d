"""Device-resident POET-X layer state driven through the C ABI.

Holds the torch device buffers one layer needs (the permuted-frame base
weight, the only copy of it the layer keeps; packed parameters; permutations;
CNP block buffers; saved activations and a workspace sized by
poetx_workspace_bytes) and calls the ABI entry points in order, including the
merge schedule a training loop runs (new permutation draws beside the merge,
which writes the merged weight straight into their frame). It allocates,
marshals and orders work on streams; all arithmetic runs in libpoetx.so.
"""

import numpy as np
import torch

from . import poetx as px

_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8, "f8": torch.uint8}
_QUANTIZED = ("i8", "f8")  # 1-byte codes with per-column scales


def to_device(arr, kind, device="cuda"):
    """Host storage array -> device tensor. bf16 arrays are uint16 bit patterns."""
    arr = np.ascontiguousarray(arr)
    if kind == "bf16":
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    if kind == "f8":
        return torch.from_numpy(arr.astype(np.uint8)).to(device)
    if kind == "i8":
        return torch.from_numpy(arr.astype(np.int8)).to(device)
    if kind == "i32":
        return torch.from_numpy(arr.astype(np.int32)).to(device)
    return torch.from_numpy(arr.astype(np.float32)).to(device)


def to_host_f64(t):
    """Device tensor (float32 / bfloat16 / int8) -> float64 numpy array."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


class DeviceLayer:
    """One POET-X layer on one GPU, for up to ``T_max`` tokens per call."""

    def __init__(self, m, n, b_r, b_p, act="bf16", weight="bf16", T_max=0, device="cuda"):
        self.m, self.n, self.b_r, self.b_p = m, n, b_r, b_p
        self.act, self.weight, self.device = act, weight, device
        self.L = px.make_layer(m, n, b_r, b_p, act, weight)
        if px.poetx_gbuf_bytes(self.L, px.POETX_SIDE_R) == 0:
            raise ValueError("invalid layer shape or dtypes for libpoetx")
        dev = device
        u8 = torch.uint8
        # Psi W0 Phi^T, and for an int8 weight the scales of its columns
        self.wp = torch.empty((m, n), dtype=_TORCH[weight], device=dev)
        self.wscale_p = torch.ones(n, dtype=torch.float32, device=dev) if weight in _QUANTIZED else None
        self.perm_r = torch.arange(m, dtype=torch.int32, device=dev)
        self.perm_p = torch.arange(n, dtype=torch.int32, device=dev)
        self.q_r = torch.zeros(px.poetx_packed_len(self.L, px.POETX_SIDE_R), dtype=torch.float32, device=dev)
        self.q_p = torch.zeros(px.poetx_packed_len(self.L, px.POETX_SIDE_P), dtype=torch.float32, device=dev)
        self.g_r = torch.empty(px.poetx_gbuf_bytes(self.L, px.POETX_SIDE_R), dtype=u8, device=dev)
        self.g_p = torch.empty(px.poetx_gbuf_bytes(self.L, px.POETX_SIDE_P), dtype=u8, device=dev)
        self.T_max = 0
        self.saved = None
        self.ws = torch.empty(0, dtype=u8, device=dev)
        # merge cycle: second stream, spare permutations, the draws' own
        # workspace and the event the merge waits for before reading them
        self._side = None
        self._next_r = self._next_p = self._draw_ws = self._drawn = None
        self._pending = None
        self.reserve(T_max)

    # -- buffers --------------------------------------------------------------
    def reserve(self, T):
        """Grow the saved-activation buffer and workspace for T tokens."""
        if T <= self.T_max and self.saved is not None:
            return
        self.T_max = max(T, self.T_max)
        self.saved = torch.empty(max(px.poetx_saved_bytes(self.L, self.T_max), 16), dtype=torch.uint8,
                                 device=self.device)
        need = max(px.poetx_workspace_bytes(self.L, self.T_max, op) for op in range(9))
        if need > self.ws.numel():
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)

    def load(self, layer, stream=None):
        """Upload a layer dict from ``synth.make_layer``: permutations, packed
        parameters, and W0 (original frame), which becomes the permuted-frame
        weight; the original-frame copy is not kept."""
        self.perm_r.copy_(to_device(layer["perm_r"], "i32", self.device))
        self.perm_p.copy_(to_device(layer["perm_p"], "i32", self.device))
        self.q_r.copy_(to_device(layer["q_r"], "f32", self.device))
        self.q_p.copy_(to_device(layer["q_p"], "f32", self.device))
        w0 = to_device(layer["W0_raw"], self.weight, self.device)
        scale = to_device(layer["w_scale"], "f32", self.device) if self.weight in _QUANTIZED else None
        self.set_weight(w0, scale, stream)

    def set_weight(self, w0, w_scale=None, stream=None):
        """Permuted-frame weight from W0 [m][n] in the original frame (and its
        column scales for an int8 or fp8 weight), for the current permutations."""
        px.poetx_weight_prepare(self.L, w0, w_scale, self.perm_r, self.perm_p, self.wp, self.wscale_p, stream)

    def export_w0(self, stream=None):
        """W0 in the original frame (and, for an int8 or fp8 weight, its column
        scales), e.g. for a checkpoint. Returns (w0, w_scale or None)."""
        w0 = torch.empty((self.m, self.n), dtype=_TORCH[self.weight], device=self.device)
        scale = torch.empty(self.n, dtype=torch.float32, device=self.device) if self.weight in _QUANTIZED else None
        px.poetx_weight_export(self.L, self.wp, self.wscale_p, self.perm_r, self.perm_p, w0, scale, self.ws, None,
                               stream)
        return w0, scale

    def act_tensor(self, rows, cols):
        return torch.empty((rows, cols), dtype=_TORCH[self.act], device=self.device)

    def saved_views(self, T):
        es = 4 if self.act == "f32" else 2
        x1 = self.saved[: T * self.m * es].view(_TORCH[self.act]).view(T, self.m)
        y1 = self.saved[T * self.m * es: T * (self.m + self.n) * es].view(_TORCH[self.act]).view(T, self.n)
        return x1, y1

    def g_planes(self, side):
        g, dim, b = (self.g_r, self.m, self.b_r) if side == px.POETX_SIDE_R else (self.g_p, self.n, self.b_p)
        nblk = -(-dim // b)
        return g.view(_TORCH[self.act]).view(2, nblk, b, b)

    # -- hot path ---------------------------------------------------------------
    def cnp_build(self, stream=None):
        px.poetx_cnp_build(self.L, self.q_r, self.q_p, self.g_r, self.g_p, self.ws, None, stream)

    def forward(self, x, z=None, stream=None):
        T = x.shape[0]
        self.reserve(T)
        if z is None:
            z = self.act_tensor(T, self.n)
        px.poetx_forward(self.L, T, x, self.perm_r, self.perm_p, self.g_r, self.g_p, self.wp, self.wscale_p,
                         z, self.saved, self.ws, None, stream)
        return z

    def backward(self, dz, dq_r=None, dq_p=None, dx=None, stream=None):
        T = dz.shape[0]
        if dq_r is None:
            dq_r = torch.empty_like(self.q_r)
        if dq_p is None:
            dq_p = torch.empty_like(self.q_p)
        if dx is None:
            dx = self.act_tensor(T, self.m)
        px.poetx_backward(self.L, T, self.saved, dz, self.perm_r, self.perm_p, self.q_r, self.q_p, self.g_r,
                          self.g_p, self.wp, self.wscale_p, dq_r, dq_p, dx, self.ws, None, stream)
        return dq_r, dq_p, dx

    def forward_mem(self, x, z=None, stream=None):
        """Memory variant: nothing saved (X1 and Y1 only in the workspace)."""
        T = x.shape[0]
        self.reserve(T)
        if z is None:
            z = self.act_tensor(T, self.n)
        px.poetx_forward_mem(self.L, T, x, self.perm_r, self.perm_p, self.g_r, self.g_p, self.wp,
                             self.wscale_p, z, self.ws, None, stream)
        return z

    def backward_mem(self, x, dz, dq_r=None, dq_p=None, dx=None, stream=None):
        """Memory variant: recomputes X1 and Y1 from x, then the backward."""
        T = dz.shape[0]
        self.reserve(T)
        if dq_r is None:
            dq_r = torch.empty_like(self.q_r)
        if dq_p is None:
            dq_p = torch.empty_like(self.q_p)
        if dx is None:
            dx = self.act_tensor(T, self.m)
        px.poetx_backward_mem(self.L, T, x, dz, self.perm_r, self.perm_p, self.q_r, self.q_p, self.g_r,
                              self.g_p, self.wp, self.wscale_p, dq_r, dq_p, dx, self.ws, None, stream)
        return dq_r, dq_p, dx

    def merge(self, perm_r_next=None, perm_p_next=None, next_ready=None, stream=None):
        """W0 <- R W0 P with q <- 0. With new permutations (device int32
        tensors, drawn before the call or, with ``next_ready``, on another
        stream up to that recorded event) the merged weight lands in their
        frame and they become the layer's permutations; without, the frame
        stays."""
        nr = self.perm_r if perm_r_next is None else perm_r_next
        np_ = self.perm_p if perm_p_next is None else perm_p_next
        px.poetx_merge(self.L, self.wp, self.wscale_p, self.perm_r, self.perm_p, nr, np_, next_ready, self.g_r,
                       self.g_p, self.q_r, self.q_p, self.ws, None, stream)
        self.perm_r, self.perm_p = nr, np_

    def begin_draw(self, seed, tag, draw, stream=None):
        """Start draw ``draw`` of both permutations (Psi under tag 2*tag, Phi
        under 2*tag + 1; ``tag`` names the layer) on a second stream (default
        priority) into spare buffers, and record an event when they are done.
        A draw depends on nothing, so a training loop can start it well before
        the merge that uses it (merge_cycle with the same arguments then only
        waits for the event); merge_cycle starts it itself otherwise."""
        main = stream if stream is not None else torch.cuda.current_stream(self.device)
        if self._side is None:
            self._side = torch.cuda.Stream(device=self.device)
            self._next_r = torch.empty_like(self.perm_r)
            self._next_p = torch.empty_like(self.perm_p)
            need = px.poetx_workspace_bytes(self.L, 0, px.POETX_OP_SAMPLE_PERM)
            self._draw_ws = torch.empty(max(need, 16), dtype=torch.uint8, device=self.device)
            self._drawn = torch.cuda.Event()
        # the spare buffers' earlier readers (the last merge) are on the main stream
        self._side.wait_stream(main)
        px.poetx_sample_perm(self.m, seed, 2 * tag, draw, self._next_r, self._draw_ws, None, self._side)
        px.poetx_sample_perm(self.n, seed, 2 * tag + 1, draw, self._next_p, self._draw_ws, None, self._side)
        self._drawn.record(self._side)
        self._pending = (seed, tag, draw)

    def merge_cycle(self, seed, tag, draw, stream=None):
        """Draw ``draw`` of both permutations (see begin_draw), then
        W0 <- R W0 P with q <- 0 written into their frame. The merge's block
        products do not wait for the draws; its final gather does (an event
        wait on the stream). The old permutations become the spares."""
        main = stream if stream is not None else torch.cuda.current_stream(self.device)
        if getattr(self, "_pending", None) != (seed, tag, draw):
            self.begin_draw(seed, tag, draw, main)
        self._pending = None
        old_r, old_p = self.perm_r, self.perm_p
        self.merge(self._next_r, self._next_p, self._drawn, main)
        self._next_r, self._next_p = old_r, old_p

    def merge_if_needed(self, step, interval, seed, tag, stream=None):
        """Called after optimizer step ``step`` (counted from 0). After every
        ``interval``-th update: CNP blocks of the current q, draw k = (step +
        1) / interval of both permutations, W0 <- R W0 P with q <- 0 in their
        frame, and the CNP blocks of q = 0. Returns whether it merged."""
        if (step + 1) % interval:
            return False
        self.cnp_build(stream)
        self.merge_cycle(seed, tag, (step + 1) // interval, stream)
        self.cnp_build(stream)
        return True
