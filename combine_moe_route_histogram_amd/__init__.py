"""Python binding of libmoe.so, the MI355X MoE expert-layer library.

Argument marshalling only: every function here has the name of the C entry
point it calls (declared in include/moe.h), takes torch tensors that live on
the GPU, checks their dtype/shape/contiguity, and passes their device pointers
and the current HIP stream through ctypes.  Every step of the layer runs in the
library's HIP kernels; there is no fallback of any kind -- if libmoe.so is
missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "Dims", "MoeError", "F32", "BF16", "lib_path", "load", "moe_init", "moe_status_str",
    "moe_last_error", "moe_workspace_bytes", "moe_route", "moe_dispatch", "moe_expert_ffn_up",
    "moe_expert_ffn_down", "moe_expert_ffn", "moe_combine", "moe_dispatch_ffn",
    "moe_ffn_combine", "moe_combine_bwd", "moe_expert_ffn_bwd_data",
    "moe_expert_ffn_bwd_weight", "moe_dispatch_bwd", "moe_route_bwd", "moe_expert_ffn_bwd_act",
    "moe_expert_ffn_bwd_input", "moe_expert_ffn_bwd_weight_gate_up", "moe_expert_ffn_bwd_weight_down",
    "moe_expert_ffn_bwd", "moe_sync_status", "moe_route_noalloc", "Tuning", "moe_get_tuning",
    "moe_tuning_predict",
]

F32, BF16 = 0, 1
_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}

_PKG = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(_PKG, "libmoe.so")


class Dims(ctypes.Structure):
    """moe_dims.  I_shared defaults to I when there are shared experts."""
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("E", ctypes.c_int32),
                ("K", ctypes.c_int32), ("I", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("I_shared", ctypes.c_int32), ("dtype", ctypes.c_int32)]

    def __init__(self, T=0, H=0, E=0, K=0, I=0, n_shared=0, I_shared=None, dtype=BF16):
        if I_shared is None:
            I_shared = I if n_shared else 0
        super().__init__(T, H, E, K, I, n_shared, I_shared, dtype)

    @property
    def R(self) -> int:
        return self.T * self.K

    @property
    def RA(self) -> int:
        return self.T * self.K + self.n_shared * self.T

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]


class Tuning(ctypes.Structure):
    """moe_tuning: the schedule knobs (band heights, fused task sizes)."""
    _fields_ = [("band_up", ctypes.c_int32), ("band_act", ctypes.c_int32),
                ("small_group", ctypes.c_int32), ("band_wgrad_up", ctypes.c_int32),
                ("band_wgrad_down", ctypes.c_int32), ("combine_tokens", ctypes.c_int32),
                ("copy_tokens", ctypes.c_int32), ("copy_in_tiles", ctypes.c_int32)]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


class MoeError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name} failed: {moe_status_str(status)}: {detail}")
        self.status = status


_P = ctypes.c_void_p
_D = ctypes.POINTER(Dims)
_SIGS = {
    "moe_init": (ctypes.c_int, [ctypes.c_int]),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_workspace_bytes": (ctypes.c_size_t, [_D]),
    "moe_get_tuning": (ctypes.c_int, [_D, ctypes.POINTER(Tuning)]),
    "moe_tuning_predict": (ctypes.c_double, [_D, ctypes.c_char_p, ctypes.c_int]),
    "moe_sync_status": (ctypes.c_int, [_P]),
    "moe_route": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_route_noalloc": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_route_ranks_workspace_bytes": (ctypes.c_size_t, [_D, ctypes.c_int]),
    "moe_route_ranks": (ctypes.c_int, [_D, _P, ctypes.c_int, _P, _P, _P, _P, _P, _P, _P,
                                       ctypes.c_size_t, _P]),
    "moe_dispatch": (ctypes.c_int, [_D, _P, _P, _P, _P]),
    "moe_expert_ffn_up": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_ffn_down": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_ffn": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                      ctypes.c_size_t, _P]),
    "moe_combine": (ctypes.c_int, [_D, _P, _P, _P, _P, _P]),
    "moe_dispatch_ffn": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                        ctypes.c_size_t, _P]),
    "moe_ffn_combine": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_combine_bwd": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P]),
    "moe_expert_ffn_bwd_data": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                               _P, ctypes.c_size_t, _P]),
    "moe_expert_ffn_bwd_weight": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                 _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_ffn_bwd": (ctypes.c_int, [_D] + [_P] * 22 + [ctypes.c_size_t, _P]),
    "moe_expert_ffn_bwd_act": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_ffn_bwd_input": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_expert_ffn_bwd_weight_gate_up": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                                         ctypes.c_size_t, _P]),
    "moe_expert_ffn_bwd_weight_down": (ctypes.c_int, [_D, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "moe_dispatch_bwd": (ctypes.c_int, [_D, _P, _P, _P, _P]),
    "moe_route_bwd": (ctypes.c_int, [_D, _P, _P, _P, _P, _P]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libmoe.so (once).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m combine_moe_route_histogram_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def moe_status_str(status: int) -> str:
    return load().moe_status_str(status).decode()


def moe_last_error() -> str:
    return load().moe_last_error().decode()


def moe_init(device: int = 0) -> None:
    st = load().moe_init(device)
    if st:
        raise MoeError(st, "moe_init", moe_last_error())


def moe_sync_status(stream=None) -> None:
    """Wait for `stream`; raise MoeError (MOE_ETIMEOUT) if a bounded wait inside
    a kernel gave up since the last check, or on a HIP error."""
    _call("moe_sync_status", _stream(stream))


def moe_get_tuning(d: Dims) -> Tuning:
    """The schedule knobs the library uses for these dims."""
    t = Tuning()
    _call("moe_get_tuning", ctypes.byref(d), ctypes.byref(t))
    return t


def moe_tuning_predict(d: Dims, knob: str, value: int) -> float:
    """The band model's predicted bytes beyond L2 per flop (negative: not modelled)."""
    return float(load().moe_tuning_predict(ctypes.byref(d), knob.encode(), int(value)))


def moe_workspace_bytes(d: Dims) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(d)))


# ---------------------------------------------------------------- marshalling

def _ptr(t, name, dtype=None, numel=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor or None")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ws(ws):
    if ws is None:
        return None, 0
    return _ptr(ws, "ws", torch.uint8), ws.numel()


def _call(name, *args):
    st = getattr(load(), name)(*args)
    if st:
        raise MoeError(st, name, moe_last_error())


# ---------------------------------------------------------------- forward

def moe_route(d: Dims, logits, topk_idx, topk_w, counts, offsets, slot, slot_src, ws, stream=None):
    T, E, K, R = d.T, d.E, d.K, d.R
    wp, wn = _ws(ws)
    _call("moe_route", ctypes.byref(d), _ptr(logits, "logits", torch.float32, T * E),
          _ptr(topk_idx, "topk_idx", torch.int32, T * K), _ptr(topk_w, "topk_w", torch.float32, T * K),
          _ptr(counts, "counts", torch.int32, E), _ptr(offsets, "offsets", torch.int32, E + 1),
          _ptr(slot, "slot", torch.int32, T * K), _ptr(slot_src, "slot_src", torch.int32, R),
          wp, wn, _stream(stream))


def moe_route_noalloc(d: Dims, logits, topk_idx, topk_w, counts, offsets, slot, slot_src,
                      stream=None):
    T, E, K, R = d.T, d.E, d.K, d.R
    _call("moe_route_noalloc", ctypes.byref(d), _ptr(logits, "logits", torch.float32, T * E),
          _ptr(topk_idx, "topk_idx", torch.int32, T * K), _ptr(topk_w, "topk_w", torch.float32, T * K),
          _ptr(counts, "counts", torch.int32, E), _ptr(offsets, "offsets", torch.int32, E + 1),
          _ptr(slot, "slot", torch.int32, T * K), _ptr(slot_src, "slot_src", torch.int32, R),
          _stream(stream))


def moe_route_ranks_workspace_bytes(d: Dims, G: int) -> int:
    return int(load().moe_route_ranks_workspace_bytes(ctypes.byref(d), int(G)))


def moe_route_ranks(d: Dims, topk_idx, G: int, rank_counts, rank_base, counts, offsets, slot,
                    slot_src, ws, stream=None):
    T, E, K, R = d.T, d.E, d.K, d.R
    wp, wn = _ws(ws)
    _call("moe_route_ranks", ctypes.byref(d), _ptr(topk_idx, "topk_idx", torch.int32, T * K),
          int(G), _ptr(rank_counts, "rank_counts", torch.int32, G * E),
          _ptr(rank_base, "rank_base", torch.int32, G * E),
          _ptr(counts, "counts", torch.int32, E), _ptr(offsets, "offsets", torch.int32, E + 1),
          _ptr(slot, "slot", torch.int32, T * K), _ptr(slot_src, "slot_src", torch.int32, R),
          wp, wn, _stream(stream))


def moe_dispatch(d: Dims, x, slot, x_perm, stream=None):
    dt = d.torch_dtype
    _call("moe_dispatch", ctypes.byref(d), _ptr(x, "x", dt, d.T * d.H),
          _ptr(slot, "slot", torch.int32, d.T * d.K), _ptr(x_perm, "x_perm", dt, d.R * d.H),
          _stream(stream))


def moe_expert_ffn_up(d: Dims, x_perm, x, offsets, w1, w3, ws1, ws3, ab, h, ws, stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    wp, wn = _ws(ws)
    _call("moe_expert_ffn_up", ctypes.byref(d), _ptr(x_perm, "x_perm", dt, d.R * H),
          _ptr(x, "x", dt, d.T * H), _ptr(offsets, "offsets", torch.int32, E + 1),
          _ptr(w1, "w1", dt, E * H * I), _ptr(w3, "w3", dt, E * H * I),
          _ptr(ws1, "ws1", dt, Ns * H * I), _ptr(ws3, "ws3", dt, Ns * H * I),
          _ptr(ab, "ab", dt, d.RA * 2 * I), _ptr(h, "h", dt, d.RA * I), wp, wn, _stream(stream))


def moe_expert_ffn_down(d: Dims, h, offsets, w2, ws2, y, ws, stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    wp, wn = _ws(ws)
    _call("moe_expert_ffn_down", ctypes.byref(d), _ptr(h, "h", dt, d.RA * I),
          _ptr(offsets, "offsets", torch.int32, E + 1), _ptr(w2, "w2", dt, E * I * H),
          _ptr(ws2, "ws2", dt, Ns * I * H), _ptr(y, "y", dt, d.RA * H), wp, wn, _stream(stream))


def moe_expert_ffn(d: Dims, x_perm, x, offsets, w1, w3, w2, ws1, ws3, ws2, ab, h, y, ws, stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    wp, wn = _ws(ws)
    _call("moe_expert_ffn", ctypes.byref(d), _ptr(x_perm, "x_perm", dt, d.R * H),
          _ptr(x, "x", dt, d.T * H), _ptr(offsets, "offsets", torch.int32, E + 1),
          _ptr(w1, "w1", dt, E * H * I), _ptr(w3, "w3", dt, E * H * I), _ptr(w2, "w2", dt, E * I * H),
          _ptr(ws1, "ws1", dt, Ns * H * I), _ptr(ws3, "ws3", dt, Ns * H * I),
          _ptr(ws2, "ws2", dt, Ns * I * H), _ptr(ab, "ab", dt, d.RA * 2 * I),
          _ptr(h, "h", dt, d.RA * I), _ptr(y, "y", dt, d.RA * H), wp, wn, _stream(stream))


def moe_combine(d: Dims, y, slot, topk_w, out, stream=None):
    dt = d.torch_dtype
    _call("moe_combine", ctypes.byref(d), _ptr(y, "y", dt, d.RA * d.H),
          _ptr(slot, "slot", torch.int32, d.T * d.K), _ptr(topk_w, "topk_w", torch.float32, d.T * d.K),
          _ptr(out, "out", dt, d.T * d.H), _stream(stream))


def moe_dispatch_ffn(d: Dims, x, slot_src, slot, offsets, w1, w3, ws1, ws3, x_perm, ab, h, ws,
                     stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    wp, wn = _ws(ws)
    _call("moe_dispatch_ffn", ctypes.byref(d), _ptr(x, "x", dt, d.T * H),
          _ptr(slot_src, "slot_src", torch.int32, d.R), _ptr(slot, "slot", torch.int32, d.T * d.K),
          _ptr(offsets, "offsets", torch.int32, E + 1),
          _ptr(w1, "w1", dt, E * H * I), _ptr(w3, "w3", dt, E * H * I),
          _ptr(ws1, "ws1", dt, Ns * H * I), _ptr(ws3, "ws3", dt, Ns * H * I),
          _ptr(x_perm, "x_perm", dt, d.R * H), _ptr(ab, "ab", dt, d.RA * 2 * I),
          _ptr(h, "h", dt, d.RA * I), wp, wn, _stream(stream))


def moe_ffn_combine(d: Dims, h, offsets, w2, ws2, slot, topk_w, y, out, ws, stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    wp, wn = _ws(ws)
    _call("moe_ffn_combine", ctypes.byref(d), _ptr(h, "h", dt, d.RA * I),
          _ptr(offsets, "offsets", torch.int32, E + 1), _ptr(w2, "w2", dt, E * I * H),
          _ptr(ws2, "ws2", dt, Ns * I * H), _ptr(slot, "slot", torch.int32, d.T * d.K),
          _ptr(topk_w, "topk_w", torch.float32, d.T * d.K), _ptr(y, "y", dt, d.RA * H),
          _ptr(out, "out", dt, d.T * H), wp, wn, _stream(stream))


# ---------------------------------------------------------------- backward

def moe_combine_bwd(d: Dims, dout, y, slot, topk_w, dy, dtopk_w, stream=None):
    dt = d.torch_dtype
    _call("moe_combine_bwd", ctypes.byref(d), _ptr(dout, "dout", dt, d.T * d.H),
          _ptr(y, "y", dt, d.R * d.H), _ptr(slot, "slot", torch.int32, d.T * d.K),
          _ptr(topk_w, "topk_w", torch.float32, d.T * d.K), _ptr(dy, "dy", dt, d.R * d.H),
          _ptr(dtopk_w, "dtopk_w", torch.float32, d.T * d.K), _stream(stream))


def moe_expert_ffn_bwd_data(d: Dims, dy, dout, offsets, w1, w3, w2, ws1, ws3, ws2, ab, dab, dx_rows,
                            ws, stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    wp, wn = _ws(ws)
    _call("moe_expert_ffn_bwd_data", ctypes.byref(d), _ptr(dy, "dy", dt, d.R * H),
          _ptr(dout, "dout", dt, d.T * H), _ptr(offsets, "offsets", torch.int32, E + 1),
          _ptr(w1, "w1", dt, E * H * I), _ptr(w3, "w3", dt, E * H * I), _ptr(w2, "w2", dt, E * I * H),
          _ptr(ws1, "ws1", dt, Ns * H * I), _ptr(ws3, "ws3", dt, Ns * H * I),
          _ptr(ws2, "ws2", dt, Ns * I * H), _ptr(ab, "ab", dt, d.RA * 2 * I),
          _ptr(dab, "dab", dt, d.RA * 2 * I), _ptr(dx_rows, "dx_rows", dt, d.RA * H), wp, wn,
          _stream(stream))


def moe_expert_ffn_bwd_weight(d: Dims, x_perm, x, h, dy, dout, dab, offsets, dw1, dw3, dw2,
                              dws1, dws3, dws2, ws, stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    f32 = torch.float32
    wp, wn = _ws(ws)
    _call("moe_expert_ffn_bwd_weight", ctypes.byref(d), _ptr(x_perm, "x_perm", dt, d.R * H),
          _ptr(x, "x", dt, d.T * H), _ptr(h, "h", dt, d.RA * I), _ptr(dy, "dy", dt, d.R * H),
          _ptr(dout, "dout", dt, d.T * H), _ptr(dab, "dab", dt, d.RA * 2 * I),
          _ptr(offsets, "offsets", torch.int32, E + 1), _ptr(dw1, "dw1", f32, E * H * I),
          _ptr(dw3, "dw3", f32, E * H * I), _ptr(dw2, "dw2", f32, E * I * H),
          _ptr(dws1, "dws1", f32, Ns * H * I), _ptr(dws3, "dws3", f32, Ns * H * I),
          _ptr(dws2, "dws2", f32, Ns * I * H), wp, wn, _stream(stream))


def moe_expert_ffn_bwd(d: Dims, dy, dout, offsets, w1, w3, w2, ws1, ws3, ws2, ab, x_perm, x, h,
                       dab, dx_rows, dw1, dw3, dw2, dws1, dws3, dws2, ws, stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    f32 = torch.float32
    wp, wn = _ws(ws)
    _call("moe_expert_ffn_bwd", ctypes.byref(d), _ptr(dy, "dy", dt, d.R * H),
          _ptr(dout, "dout", dt, d.T * H), _ptr(offsets, "offsets", torch.int32, E + 1),
          _ptr(w1, "w1", dt, E * H * I), _ptr(w3, "w3", dt, E * H * I), _ptr(w2, "w2", dt, E * I * H),
          _ptr(ws1, "ws1", dt, Ns * H * I), _ptr(ws3, "ws3", dt, Ns * H * I),
          _ptr(ws2, "ws2", dt, Ns * I * H), _ptr(ab, "ab", dt, d.RA * 2 * I),
          _ptr(x_perm, "x_perm", dt, d.R * H), _ptr(x, "x", dt, d.T * H), _ptr(h, "h", dt, d.RA * I),
          _ptr(dab, "dab", dt, d.RA * 2 * I), _ptr(dx_rows, "dx_rows", dt, d.RA * H),
          _ptr(dw1, "dw1", f32, E * H * I), _ptr(dw3, "dw3", f32, E * H * I),
          _ptr(dw2, "dw2", f32, E * I * H), _ptr(dws1, "dws1", f32, Ns * H * I),
          _ptr(dws3, "dws3", f32, Ns * H * I), _ptr(dws2, "dws2", f32, Ns * I * H), wp, wn,
          _stream(stream))


def moe_expert_ffn_bwd_act(d: Dims, dy, dout, offsets, w2, ws2, ab, dab, ws, stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    wp, wn = _ws(ws)
    _call("moe_expert_ffn_bwd_act", ctypes.byref(d), _ptr(dy, "dy", dt, d.R * H),
          _ptr(dout, "dout", dt, d.T * H), _ptr(offsets, "offsets", torch.int32, E + 1),
          _ptr(w2, "w2", dt, E * I * H), _ptr(ws2, "ws2", dt, Ns * I * H),
          _ptr(ab, "ab", dt, d.RA * 2 * I), _ptr(dab, "dab", dt, d.RA * 2 * I), wp, wn,
          _stream(stream))


def moe_expert_ffn_bwd_input(d: Dims, dab, offsets, w1, w3, ws1, ws3, dx_rows, ws, stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    wp, wn = _ws(ws)
    _call("moe_expert_ffn_bwd_input", ctypes.byref(d), _ptr(dab, "dab", dt, d.RA * 2 * I),
          _ptr(offsets, "offsets", torch.int32, E + 1), _ptr(w1, "w1", dt, E * H * I),
          _ptr(w3, "w3", dt, E * H * I), _ptr(ws1, "ws1", dt, Ns * H * I),
          _ptr(ws3, "ws3", dt, Ns * H * I), _ptr(dx_rows, "dx_rows", dt, d.RA * H), wp, wn,
          _stream(stream))


def moe_expert_ffn_bwd_weight_gate_up(d: Dims, x_perm, x, dab, offsets, dw1, dw3, dws1, dws3, ws,
                                      stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    f32 = torch.float32
    wp, wn = _ws(ws)
    _call("moe_expert_ffn_bwd_weight_gate_up", ctypes.byref(d), _ptr(x_perm, "x_perm", dt, d.R * H),
          _ptr(x, "x", dt, d.T * H), _ptr(dab, "dab", dt, d.RA * 2 * I),
          _ptr(offsets, "offsets", torch.int32, E + 1), _ptr(dw1, "dw1", f32, E * H * I),
          _ptr(dw3, "dw3", f32, E * H * I), _ptr(dws1, "dws1", f32, Ns * H * I),
          _ptr(dws3, "dws3", f32, Ns * H * I), wp, wn, _stream(stream))


def moe_expert_ffn_bwd_weight_down(d: Dims, h, dy, dout, offsets, dw2, dws2, ws, stream=None):
    dt, H, I, E, Ns = d.torch_dtype, d.H, d.I, d.E, d.n_shared
    f32 = torch.float32
    wp, wn = _ws(ws)
    _call("moe_expert_ffn_bwd_weight_down", ctypes.byref(d), _ptr(h, "h", dt, d.RA * I),
          _ptr(dy, "dy", dt, d.R * H), _ptr(dout, "dout", dt, d.T * H),
          _ptr(offsets, "offsets", torch.int32, E + 1), _ptr(dw2, "dw2", f32, E * I * H),
          _ptr(dws2, "dws2", f32, Ns * I * H), wp, wn, _stream(stream))


def moe_dispatch_bwd(d: Dims, dx_rows, slot, dx, stream=None):
    dt = d.torch_dtype
    _call("moe_dispatch_bwd", ctypes.byref(d), _ptr(dx_rows, "dx_rows", dt, d.RA * d.H),
          _ptr(slot, "slot", torch.int32, d.T * d.K), _ptr(dx, "dx", dt, d.T * d.H), _stream(stream))


def moe_route_bwd(d: Dims, dtopk_w, topk_w, topk_idx, dlogits, stream=None):
    f32 = torch.float32
    _call("moe_route_bwd", ctypes.byref(d), _ptr(dtopk_w, "dtopk_w", f32, d.T * d.K),
          _ptr(topk_w, "topk_w", f32, d.T * d.K), _ptr(topk_idx, "topk_idx", torch.int32, d.T * d.K),
          _ptr(dlogits, "dlogits", f32, d.T * d.E), _stream(stream))
