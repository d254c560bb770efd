"""ctypes binding of ``libmoe_decode.so`` (the C ABI in include/moe_decode.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels of the library.  PyTorch provides device memory and streams.  The
binding fails loudly when the library has not been built; there is no other
implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_decode.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_WORKSPACE = 0, -1, -2, -3, -4
MOE_ROUTER_BF16, MOE_ROUTER_F32 = 0, 1

_lib = None


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("latent", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("expert_inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_top_k", ctypes.c_int32), ("router_dtype", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("router_w", "router_bias", "lat_down", "lat_up", "w13_q", "w13_s", "w2_q",
                 "w2_s", "sh_w13", "sh_w2")]


class DispatchInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("batch", "top_k", "col_tiles", "split_in", "split_out", "split_w13",
                 "split_w2", "grid_in", "grid_w13", "grid_w2", "grid_out", "router_f32",
                 "n_kernels", "fused", "grid_step", "out_staged", "routing", "ordered",
                  "in_staged")]


class Debug(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("score", "key", "z", "act", "ylat", "ash", "n_active")]


MODE_FUSED, MODE_FOUR_LAUNCHES, MODE_TWO_LAUNCHES, MODE_SIDE_STREAM = 0, 1, 2, 3
MODE_LATE_ROUTING, MODE_DENSE_ROUTING, MODE_ORDERED = 4, 5, 6
DEFAULT_MODE = MODE_FOUR_LAUNCHES  # what moe_decode_init selects

EXPORTED = ("moe_decode_validate_config", "moe_decode_workspace_size", "moe_decode_init",
            "moe_decode_step", "moe_decode_destroy", "moe_decode_status_string",
            "moe_decode_last_hip_error", "moe_decode_graph_create", "moe_decode_graph_launch",
            "moe_decode_graph_destroy", "moe_decode_last_dispatch", "moe_decode_debug_export",
            "moe_decode_debug_dequant", "moe_decode_set_timing_events", "moe_decode_set_mode",
            "moe_decode_read_flags", "moe_decode_set_next_layer", "moe_decode_step_static")

STATIC_WORKSPACE_BYTES = 64 << 20  # MOE_DECODE_STATIC_WORKSPACE_BYTES


class MoEError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Loads the library (it must have been built: __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MoEError(f"{LIB_PATH} is missing: build the HIP library first "
                       "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.moe_decode_validate_config.argtypes = [ctypes.POINTER(Config)]
    L.moe_decode_validate_config.restype = i32
    L.moe_decode_workspace_size.argtypes = [ctypes.POINTER(Config)]
    L.moe_decode_workspace_size.restype = ctypes.c_size_t
    L.moe_decode_init.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), vp,
                                  ctypes.c_size_t, ctypes.POINTER(vp)]
    L.moe_decode_init.restype = i32
    L.moe_decode_step.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp]
    L.moe_decode_step.restype = i32
    L.moe_decode_destroy.argtypes = [vp]
    L.moe_decode_destroy.restype = i32
    L.moe_decode_status_string.argtypes = [i32]
    L.moe_decode_status_string.restype = ctypes.c_char_p
    L.moe_decode_last_hip_error.argtypes = [vp]
    L.moe_decode_last_hip_error.restype = i32
    L.moe_decode_graph_create.argtypes = [ctypes.POINTER(vp), i32, ctypes.POINTER(vp), i32, i32,
                                          ctypes.POINTER(vp), ctypes.POINTER(vp),
                                          ctypes.POINTER(vp), ctypes.POINTER(vp)]
    L.moe_decode_graph_create.restype = i32
    L.moe_decode_graph_launch.argtypes = [vp, vp]
    L.moe_decode_graph_launch.restype = i32
    L.moe_decode_graph_destroy.argtypes = [vp]
    L.moe_decode_graph_destroy.restype = i32
    L.moe_decode_last_dispatch.argtypes = [vp, ctypes.POINTER(DispatchInfo)]
    L.moe_decode_last_dispatch.restype = i32
    L.moe_decode_debug_export.argtypes = [vp, i32, i32, ctypes.POINTER(Debug), vp]
    L.moe_decode_debug_export.restype = i32
    L.moe_decode_debug_dequant.argtypes = [vp, vp, i64, vp, vp]
    L.moe_decode_debug_dequant.restype = i32
    L.moe_decode_set_timing_events.argtypes = [vp, ctypes.POINTER(vp), i32]
    L.moe_decode_set_timing_events.restype = i32
    L.moe_decode_set_mode.argtypes = [vp, i32]
    L.moe_decode_set_mode.restype = i32
    L.moe_decode_read_flags.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32)]
    L.moe_decode_read_flags.restype = i32
    L.moe_decode_set_next_layer.argtypes = [vp, vp]
    L.moe_decode_set_next_layer.restype = i32
    L.moe_decode_step_static.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), vp,
                                         i32, i32, vp, vp, vp, vp]
    L.moe_decode_step_static.restype = i32
    _lib = L
    return L


def _check(rc: int, what: str, ctx=None) -> None:
    if rc != MOE_OK:
        msg = lib().moe_decode_status_string(rc).decode()
        extra = ""
        if ctx is not None and rc == MOE_ERR_HIP:
            extra = f" (hip error {lib().moe_decode_last_hip_error(ctx)})"
        raise MoEError(f"{what}: {msg}{extra} [{rc}]")


def make_config(dims, max_batch: int, max_top_k: int) -> Config:
    return Config(dims.hidden, dims.latent, dims.n_experts, dims.expert_inter, dims.shared_inter,
                  max_batch, max_top_k, MOE_ROUTER_F32 if dims.router_f32 else MOE_ROUTER_BF16)


def workspace_size(dims, max_batch: int, max_top_k: int) -> int:
    cfg = make_config(dims, max_batch, max_top_k)
    return int(lib().moe_decode_workspace_size(ctypes.byref(cfg)))


def validate(dims, max_batch: int, max_top_k: int) -> int:
    cfg = make_config(dims, max_batch, max_top_k)
    return int(lib().moe_decode_validate_config(ctypes.byref(cfg)))


def _stream_ptr(stream) -> Optional[int]:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream or None


# ---------------------------------------------------------------------------
# Device-resident layer weights
# ---------------------------------------------------------------------------

def _dev(arr, device):
    """numpy array -> contiguous torch device tensor with the same bytes
    (uint16 bf16 patterns travel as int16)."""
    import numpy as np
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DeviceLayer:
    """The weights of one layer (a synth.Layer) copied to the GPU."""

    NAMES = ("router_w", "bias", "lat_down", "lat_up", "w13_q", "w13_s", "w2_q", "w2_s",
             "sh_w13", "sh_w2")

    def __init__(self, layer, device="cuda"):
        self.dims = layer.dims
        self.t: Dict[str, object] = {}
        for n in self.NAMES:
            v = getattr(layer, n)
            self.t[n] = None if v is None else _dev(v, device)

    def with_bias(self, bias) -> "DeviceLayer":
        """The same device weights with another router bias (numpy f32 [E])."""
        other = DeviceLayer.__new__(DeviceLayer)
        other.dims = self.dims
        other.t = dict(self.t)
        other.t["bias"] = None if bias is None else _dev(bias, self.t["lat_down"].device)
        return other

    def weights_struct(self) -> Weights:
        t = self.t
        p = lambda n: None if t[n] is None else t[n].data_ptr()  # noqa: E731
        return Weights(p("router_w"), p("bias"), p("lat_down"), p("lat_up"), p("w13_q"),
                       p("w13_s"), p("w2_q"), p("w2_s"), p("sh_w13"), p("sh_w2"))


# ---------------------------------------------------------------------------
# One layer's decode context
# ---------------------------------------------------------------------------

class MoEDecode:
    """A library context over device weights, with its own workspace
    (or a shared one)."""

    def __init__(self, dev_layer: DeviceLayer, max_batch: int, max_top_k: int,
                 workspace=None):
        import torch
        self.layer = dev_layer
        self.dims = dev_layer.dims
        self.max_batch, self.max_top_k = max_batch, max_top_k
        self.cfg = make_config(self.dims, max_batch, max_top_k)
        size = int(lib().moe_decode_workspace_size(ctypes.byref(self.cfg)))
        if size == 0:
            _check(lib().moe_decode_validate_config(ctypes.byref(self.cfg)), "config")
        if workspace is None:
            workspace = torch.empty(size, dtype=torch.uint8, device="cuda")
        if workspace.numel() < size:
            raise MoEError("shared workspace too small")
        self.workspace = workspace
        self.weights = dev_layer.weights_struct()
        h = ctypes.c_void_p()
        _check(lib().moe_decode_init(ctypes.byref(self.cfg), ctypes.byref(self.weights),
                                     workspace.data_ptr(), workspace.numel(), ctypes.byref(h)),
               "moe_decode_init")
        self.handle = h

    def step(self, x, top_k: int, out=None, idx=None, w=None, stream=None):
        """x: int16 [B][H] device tensor of bf16 patterns.  Returns (out, idx, w)."""
        import torch
        B = x.shape[0]
        if out is None:
            out = torch.empty((B, self.dims.hidden), dtype=torch.int16, device=x.device)
        if idx is None:
            idx = torch.empty((B, top_k), dtype=torch.int32, device=x.device)
        if w is None:
            w = torch.empty((B, top_k), dtype=torch.float32, device=x.device)
        rc = lib().moe_decode_step(self.handle, x.data_ptr(), B, top_k, out.data_ptr(),
                                   idx.data_ptr() if idx is not False else None,
                                   w.data_ptr() if w is not False else None,
                                   _stream_ptr(stream))
        _check(rc, "moe_decode_step", self.handle)
        return out, idx, w

    def set_timing_events(self, events) -> None:
        """torch.cuda.Event(enable_timing=True) objects (already recorded once,
        so their handles exist), a start and a stop event per kernel of the
        step, attached to the kernels' dispatches; None switches off."""
        if not events:
            _check(lib().moe_decode_set_timing_events(self.handle, None, 0), "timing events")
            return
        arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
        _check(lib().moe_decode_set_timing_events(self.handle, arr, len(events)), "timing events")

    def set_mode(self, mode: int) -> None:
        """MODE_FOUR_LAUNCHES (default), MODE_SIDE_STREAM (shared expert on
        the context's second stream), MODE_TWO_LAUNCHES or MODE_FUSED (one
        persistent launch where the shape has one)."""
        _check(lib().moe_decode_set_mode(self.handle, mode), "set_mode")

    def set_next_layer(self, nxt: Optional["MoEDecode"]) -> None:
        """Prefetch nxt's router and latent-down rows while this context's
        steps route (None: off); nxt must outlive this setting."""
        self._next = nxt
        _check(lib().moe_decode_set_next_layer(self.handle, nxt.handle if nxt else None),
               "set_next_layer")

    def read_flags(self) -> int:
        """Sticky fault flags of the context's fused steps (0: none)."""
        v = ctypes.c_uint32(0)
        _check(lib().moe_decode_read_flags(self.handle, ctypes.byref(v)), "read_flags")
        return int(v.value)

    def last_dispatch(self) -> dict:
        info = DispatchInfo()
        _check(lib().moe_decode_last_dispatch(self.handle, ctypes.byref(info)), "last_dispatch")
        return {n: getattr(info, n) for n, _ in DispatchInfo._fields_}

    def debug_export(self, batch: int, top_k: int, stream=None) -> dict:
        """Intermediates of the last step as f32 device tensors."""
        import torch
        d = self.dims
        dev = "cuda"
        r = {"score": torch.empty((batch, d.n_experts), device=dev),
             "key": torch.empty((batch, d.n_experts), device=dev),
             "z": torch.empty((batch, d.latent), device=dev),
             "act": torch.empty((batch, top_k, d.expert_inter), device=dev),
             "ylat": torch.empty((batch, d.latent), device=dev),
             "ash": torch.empty((batch, d.shared_inter), device=dev),
             "n_active": torch.empty((1,), dtype=torch.int32, device=dev)}
        dbg = Debug(*[r[n].data_ptr() for n in ("score", "key", "z", "act", "ylat", "ash",
                                                  "n_active")])
        _check(lib().moe_decode_debug_export(self.handle, batch, top_k, ctypes.byref(dbg),
                                             _stream_ptr(stream)), "debug_export", self.handle)
        return r

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib().moe_decode_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Graph:
    """Several layers' steps captured into one HIP graph."""

    def __init__(self, ctxs: Sequence[MoEDecode], xs, batch: int, top_k: int, outs, idxs=None,
                 ws=None, prefetch_next: bool = False):
        """prefetch_next: each layer's step prefetches the next layer's
        router and latent-down rows while it routes (captured that way; the
        contexts' own setting is restored afterwards)."""
        n = len(ctxs)
        if prefetch_next:
            for i in range(n - 1):
                if ctxs[i + 1] is not ctxs[i]:
                    lib().moe_decode_set_next_layer(ctxs[i].handle, ctxs[i + 1].handle)
        VP = ctypes.c_void_p
        arr = lambda vals: (VP * n)(*vals)  # noqa: E731
        self._keep = (ctxs, xs, outs, idxs, ws)
        g = VP()
        rc = lib().moe_decode_graph_create(
            arr([c.handle for c in ctxs]), n, arr([x.data_ptr() for x in xs]), batch, top_k,
            arr([o.data_ptr() for o in outs]),
            arr([i.data_ptr() for i in idxs]) if idxs is not None else None,
            arr([w.data_ptr() for w in ws]) if ws is not None else None, ctypes.byref(g))
        if prefetch_next:
            for c in ctxs:
                nxt = getattr(c, "_next", None)
                lib().moe_decode_set_next_layer(c.handle, nxt.handle if nxt else None)
        _check(rc, "moe_decode_graph_create", ctxs[0].handle)
        self.handle = g

    def launch(self, stream=None) -> None:
        _check(lib().moe_decode_graph_launch(self.handle, _stream_ptr(stream)), "graph_launch")

    def close(self) -> None:
        if getattr(self, "handle", None):
            lib().moe_decode_graph_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def step_static(dev_layer: DeviceLayer, max_batch: int, max_top_k: int, x, top_k: int,
                out=None, idx=None, w=None, stream=None):
    """moe_decode_step_static: one step of the layer with the library's static
    workspace (no context, no allocation by the library).  x: int16 [B][H]
    device tensor.  Returns (out, idx, w)."""
    import torch
    cfg = make_config(dev_layer.dims, max_batch, max_top_k)
    weights = dev_layer.weights_struct()
    B = x.shape[0]
    if out is None:
        out = torch.empty((B, dev_layer.dims.hidden), dtype=torch.int16, device=x.device)
    if idx is None:
        idx = torch.empty((B, top_k), dtype=torch.int32, device=x.device)
    if w is None:
        w = torch.empty((B, top_k), dtype=torch.float32, device=x.device)
    _check(lib().moe_decode_step_static(ctypes.byref(cfg), ctypes.byref(weights), x.data_ptr(),
                                        B, top_k, out.data_ptr(), idx.data_ptr(), w.data_ptr(),
                                        _stream_ptr(stream)), "moe_decode_step_static")
    return out, idx, w


def dequant(q, s, stream=None):
    """MXFP4 codes/scales (uint8 device tensors) -> f32 via the library."""
    import torch
    n = q.numel() * 2
    out = torch.empty(n, dtype=torch.float32, device=q.device)
    _check(lib().moe_decode_debug_dequant(q.data_ptr(), s.data_ptr(), n, out.data_ptr(),
                                          _stream_ptr(stream)), "debug_dequant")
    return out
