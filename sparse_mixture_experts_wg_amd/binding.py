"""Thin ctypes binding of libmoe.so (include/moe.h) for torch tensors.

Only argument marshalling happens here: shape/dtype/device checks, output
allocation with torch.empty when the caller passes none, and the current HIP
stream. Every step of the layer runs in the library's kernels. There is no
fallback: if libmoe.so is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libmoe.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "moe.h")

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_HIP = range(7)
F32, BF16 = 0, 1
PATH_AUTO, PATH_STREAM, PATH_TILED = 0, 1, 2
_DTYPES = {"f32": F32, "bf16": BF16}
_PATHS = {"auto": PATH_AUTO, "stream": PATH_STREAM, "tiled": PATH_TILED}
FLAG_DOWN_PARTIALS = 1


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("h", ctypes.c_int64),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("path", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]

    @property
    def S(self) -> int:
        return int(self.T) * int(self.K)


def problem(T: int, d: int, h: int, E: int = 8, K: int = 2, dtype: str = "bf16",
            out_dtype: str = "f32", path: str = "auto", flags: int = 0,
            capacity: int = 0) -> Problem:
    return Problem(T, d, h, E, K, _DTYPES[dtype], _DTYPES[out_dtype], _PATHS[path], flags,
                   capacity, 0)


def capacity_rows(T: int, K: int, E: int, capacity_factor) -> int:
    """Rows per expert for a capacity factor, ceil(cf * T * K / E), computed by the
    library in exact integer arithmetic. cf is taken as the exact rational of its
    decimal text (1.1 means 11/10), or given as a fractions.Fraction or a
    (numerator, denominator) pair."""
    from fractions import Fraction

    if isinstance(capacity_factor, tuple):
        cf = Fraction(int(capacity_factor[0]), int(capacity_factor[1]))
    elif isinstance(capacity_factor, Fraction):
        cf = capacity_factor
    else:
        cf = Fraction(repr(float(capacity_factor)))
    n = lib.moe_capacity_rows(int(T), int(K), int(E), cf.numerator, cf.denominator)
    if n < 0:
        raise MoeError(-n, last_error())
    return int(n)


def header_functions(path: str = HEADER):
    """Names of the functions include/moe.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def _load() -> ctypes.CDLL:
    # torch ships its own HIP runtime. Loading it first makes libmoe.so bind to
    # that same runtime (the dynamic linker matches libamdhip64.so.7 by SONAME);
    # loading libmoe.so first would put a second HIP runtime into the process.
    import torch  # noqa: F401

    if not os.path.exists(LIBRARY):
        raise ImportError(f"{LIBRARY} is not built; run __graft_entry__.build() or "
                          "python sparse_mixture_experts_wg_amd/build.py")
    lib = ctypes.CDLL(LIBRARY)
    P, vp, i32 = ctypes.POINTER(Problem), ctypes.c_void_p, ctypes.c_int
    sz = ctypes.c_size_t
    sig = {
        "moe_status_string": ([i32], ctypes.c_char_p),
        "moe_capacity_rows": ([ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                               ctypes.c_int64], ctypes.c_int64),
        "moe_forward_noalloc": ([P, vp, vp, vp, vp, vp, vp, vp, vp, vp], i32),
        "moe_last_error": ([], ctypes.c_char_p),
        "moe_resolve_path": ([P], i32),
        "moe_down_parts": ([P], i32),
        "moe_route": ([P, vp, vp, vp, vp, vp, vp], i32),
        "moe_permute": ([P, vp, vp, vp, vp, vp, vp, vp], i32),
        "moe_expert_gate_up": ([P, vp, vp, vp, vp, vp, vp], i32),
        "moe_expert_gate_up_rows": ([P, vp, vp, vp, vp, vp, vp, vp], i32),
        "moe_expert_down": ([P, vp, vp, vp, vp, vp], i32),
        "moe_expert_workspace_bytes": ([P], sz),
        "moe_expert_swiglu": ([P, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_combine": ([P, vp, vp, vp, vp, vp], i32),
        "moe_forward_workspace_bytes": ([P], sz),
        "moe_forward": ([P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp], i32),
        "moe_forward_profiled": ([P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp], i32),
        "moe_rmsnorm": ([P, vp, vp, ctypes.c_float, vp, vp], i32),
        "moe_combine_residual": ([P, vp, vp, vp, vp, vp, vp], i32),
        "moe_block_workspace_bytes": ([P], sz),
        "moe_block_forward": ([P, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
                              i32),
        "moe_block_forward_profiled": ([P, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp,
                                        sz, vp, vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


def last_error() -> str:
    return lib.moe_last_error().decode()


def _check(status: int):
    if status != OK:
        raise MoeError(status, last_error())


def resolve_path(p: Problem) -> int:
    return lib.moe_resolve_path(ctypes.byref(p))


def expert_workspace_bytes(p: Problem) -> int:
    return lib.moe_expert_workspace_bytes(ctypes.byref(p))


def down_parts(p: Problem) -> int:
    """Partial sums per row that the down projection writes into o_perm for `p`."""
    n = lib.moe_down_parts(ctypes.byref(p))
    if n < 0:
        raise MoeError(-n, last_error())
    return n


def _o_shape(p: Problem):
    parts = down_parts(p)
    return (p.S, int(p.d)) if parts == 1 else (parts, p.S, int(p.d))


def forward_workspace_bytes(p: Problem) -> int:
    return lib.moe_forward_workspace_bytes(ctypes.byref(p))


# ---- torch marshalling -----------------------------------------------------------

def _torch():
    import torch

    return torch


def _tdtype(code: int):
    torch = _torch()
    return torch.bfloat16 if code == BF16 else torch.float32


def _ptr(t, name: str, shape=None, dtype=None):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _empty(shape, dtype, like):
    return _torch().empty(shape, dtype=dtype, device=like.device)


def route(p: Problem, x, w_g, topk_idx=None, topk_w=None, logits=None, want_logits=False,
          stream=None):
    torch = _torch()
    T, d, E, K = int(p.T), int(p.d), int(p.E), int(p.K)
    dt = _tdtype(p.dtype)
    topk_idx = _empty((T, K), torch.int32, x) if topk_idx is None else topk_idx
    topk_w = _empty((T, K), torch.float32, x) if topk_w is None else topk_w
    if logits is None and want_logits:
        logits = _empty((T, E), torch.float32, x)
    _check(lib.moe_route(ctypes.byref(p), _ptr(x, "x", (T, d), dt), _ptr(w_g, "w_g", (d, E), dt),
                         _ptr(topk_idx, "topk_idx", (T, K), torch.int32),
                         _ptr(topk_w, "topk_w", (T, K), torch.float32),
                         _ptr(logits, "logits", (T, E), torch.float32), _stream(stream)))
    return topk_idx, topk_w, logits


def permute(p: Problem, x, topk_idx, offsets=None, perm_token=None, slot_pos=None, x_perm=None,
            stream=None, gather: bool = True):
    """gather=False: the index arrays only (x_perm is returned as None; x may be
    None), for expert_gate_up_rows."""
    torch = _torch()
    T, d, E, K, S = int(p.T), int(p.d), int(p.E), int(p.K), p.S
    dt = _tdtype(p.dtype)
    offsets = _empty((E + 1,), torch.int32, topk_idx) if offsets is None else offsets
    perm_token = _empty((S,), torch.int32, topk_idx) if perm_token is None else perm_token
    slot_pos = _empty((T, K), torch.int32, topk_idx) if slot_pos is None else slot_pos
    if not gather:
        x_perm = None
    elif x_perm is None:
        x_perm = _empty((S, d), dt, x)
    _check(lib.moe_permute(ctypes.byref(p), _ptr(x, "x", (T, d), dt),
                           _ptr(topk_idx, "topk_idx", (T, K), torch.int32),
                           _ptr(offsets, "offsets", (E + 1,), torch.int32),
                           _ptr(perm_token, "perm_token", (S,), torch.int32),
                           _ptr(slot_pos, "slot_pos", (T, K), torch.int32),
                           _ptr(x_perm, "x_perm", (S, d), dt), _stream(stream)))
    return offsets, perm_token, slot_pos, x_perm


def expert_gate_up(p: Problem, x_perm, offsets, w1, w3, act=None, stream=None):
    torch = _torch()
    d, h, E, S = int(p.d), int(p.h), int(p.E), p.S
    dt = _tdtype(p.dtype)
    act = _empty((S, h), dt, x_perm) if act is None else act
    _check(lib.moe_expert_gate_up(ctypes.byref(p), _ptr(x_perm, "x_perm", (S, d), dt),
                                  _ptr(offsets, "offsets", (E + 1,), torch.int32),
                                  _ptr(w1, "w1", (E, h, d), dt), _ptr(w3, "w3", (E, h, d), dt),
                                  _ptr(act, "act", (S, h), dt), _stream(stream)))
    return act


def expert_gate_up_rows(p: Problem, x, perm_token, offsets, w1, w3, act=None, stream=None):
    torch = _torch()
    T, d, h, E, S = int(p.T), int(p.d), int(p.h), int(p.E), p.S
    dt = _tdtype(p.dtype)
    act = _empty((S, h), dt, x) if act is None else act
    _check(lib.moe_expert_gate_up_rows(ctypes.byref(p), _ptr(x, "x", (T, d), dt),
                                       _ptr(perm_token, "perm_token", (S,), torch.int32),
                                       _ptr(offsets, "offsets", (E + 1,), torch.int32),
                                       _ptr(w1, "w1", (E, h, d), dt), _ptr(w3, "w3", (E, h, d), dt),
                                       _ptr(act, "act", (S, h), dt), _stream(stream)))
    return act


def expert_down(p: Problem, act, offsets, w2, o_perm=None, stream=None):
    torch = _torch()
    d, h, E, S = int(p.d), int(p.h), int(p.E), p.S
    dt = _tdtype(p.dtype)
    o_shape = _o_shape(p)
    o_perm = _empty(o_shape, torch.float32, act) if o_perm is None else o_perm
    _check(lib.moe_expert_down(ctypes.byref(p), _ptr(act, "act", (S, h), dt),
                               _ptr(offsets, "offsets", (E + 1,), torch.int32),
                               _ptr(w2, "w2", (E, d, h), dt),
                               _ptr(o_perm, "o_perm", o_shape, torch.float32), _stream(stream)))
    return o_perm


def expert_swiglu(p: Problem, x_perm, offsets, w1, w3, w2, o_perm=None, ws=None, stream=None):
    torch = _torch()
    d, h, E, S = int(p.d), int(p.h), int(p.E), p.S
    dt = _tdtype(p.dtype)
    o_shape = _o_shape(p)
    o_perm = _empty(o_shape, torch.float32, x_perm) if o_perm is None else o_perm
    need = expert_workspace_bytes(p)
    ws = _empty((max(need, 1),), torch.uint8, x_perm) if ws is None else ws
    _check(lib.moe_expert_swiglu(ctypes.byref(p), _ptr(x_perm, "x_perm", (S, d), dt),
                                 _ptr(offsets, "offsets", (E + 1,), torch.int32),
                                 _ptr(w1, "w1", (E, h, d), dt), _ptr(w3, "w3", (E, h, d), dt),
                                 _ptr(w2, "w2", (E, d, h), dt),
                                 _ptr(o_perm, "o_perm", o_shape, torch.float32), _ptr(ws, "ws"),
                                 ws.numel() * ws.element_size(), _stream(stream)))
    return o_perm


def block_workspace_bytes(p: Problem) -> int:
    return lib.moe_block_workspace_bytes(ctypes.byref(p))


def rmsnorm(p: Problem, h, norm_w, eps: float, x=None, stream=None):
    T, d = int(p.T), int(p.d)
    dt = _tdtype(p.dtype)
    x = _empty((T, d), dt, h) if x is None else x
    _check(lib.moe_rmsnorm(ctypes.byref(p), _ptr(h, "h", (T, d), dt),
                           _ptr(norm_w, "norm_w", (d,), dt), ctypes.c_float(eps),
                           _ptr(x, "x", (T, d), dt), _stream(stream)))
    return x


def combine_residual(p: Problem, o_perm, slot_pos, topk_w, residual, y=None, stream=None):
    torch = _torch()
    T, d, K = int(p.T), int(p.d), int(p.K)
    yd = _tdtype(p.out_dtype)
    y = _empty((T, d), yd, o_perm) if y is None else y
    _check(lib.moe_combine_residual(ctypes.byref(p),
                                    _ptr(o_perm, "o_perm", _o_shape(p), torch.float32),
                                    _ptr(slot_pos, "slot_pos", (T, K), torch.int32),
                                    _ptr(topk_w, "topk_w", (T, K), torch.float32),
                                    _ptr(residual, "residual", (T, d), _tdtype(p.dtype)),
                                    _ptr(y, "y", (T, d), yd), _stream(stream)))
    return y


def block_forward(p: Problem, h, norm_w, eps: float, w_g, w1, w3, w2, y=None, topk_idx=None,
                  topk_w=None, ws=None, stream=None, events=None):
    """Pre-norm block: y = h + MoE(RMSNorm(h) * norm_w); `events` as for forward."""
    torch = _torch()
    T, d, hd, E, K = int(p.T), int(p.d), int(p.h), int(p.E), int(p.K)
    dt = _tdtype(p.dtype)
    yd = _tdtype(p.out_dtype)
    y = _empty((T, d), yd, h) if y is None else y
    need = block_workspace_bytes(p)
    ws = _empty((max(need, 1),), torch.uint8, h) if ws is None else ws
    args = (ctypes.byref(p), _ptr(h, "h", (T, d), dt), _ptr(norm_w, "norm_w", (d,), dt),
            ctypes.c_float(eps), _ptr(w_g, "w_g", (d, E), dt), _ptr(w1, "w1", (E, hd, d), dt),
            _ptr(w3, "w3", (E, hd, d), dt), _ptr(w2, "w2", (E, d, hd), dt),
            _ptr(y, "y", (T, d), yd), _ptr(topk_idx, "topk_idx", (T, K), torch.int32),
            _ptr(topk_w, "topk_w", (T, K), torch.float32), _ptr(ws, "ws"),
            ws.numel() * ws.element_size(), _stream(stream))
    if events is None:
        _check(lib.moe_block_forward(*args))
    else:
        _check(lib.moe_block_forward_profiled(*args, *_events(events)))
    return y


def combine(p: Problem, o_perm, slot_pos, topk_w, y=None, stream=None):
    torch = _torch()
    T, d, K, S = int(p.T), int(p.d), int(p.K), p.S
    yd = _tdtype(p.out_dtype)
    y = _empty((T, d), yd, o_perm) if y is None else y
    _check(lib.moe_combine(ctypes.byref(p), _ptr(o_perm, "o_perm", _o_shape(p), torch.float32),
                           _ptr(slot_pos, "slot_pos", (T, K), torch.int32),
                           _ptr(topk_w, "topk_w", (T, K), torch.float32),
                           _ptr(y, "y", (T, d), yd), _stream(stream)))
    return y


def _events(events):
    """(begin, end) torch.cuda.Event pair -> two raw hipEvent_t handles (the events
    must have been recorded once, which creates them), or two NULLs."""
    if events is None:
        return None, None
    handles = [int(ev.cuda_event) for ev in events]
    if len(handles) != 2 or not all(handles):
        raise ValueError("events: a pair of torch.cuda.Event that have been recorded once")
    return ctypes.c_void_p(handles[0]), ctypes.c_void_p(handles[1])


def forward(p: Problem, x, w_g, w1, w3, w2, y=None, topk_idx=None, topk_w=None, ws=None,
            stream=None, events=None):
    """The whole layer (moe_forward); with `events` (a pair of recorded
    torch.cuda.Event) moe_forward_profiled, which records them around the gate-up."""
    torch = _torch()
    T, d, h, E, K = int(p.T), int(p.d), int(p.h), int(p.E), int(p.K)
    dt = _tdtype(p.dtype)
    yd = _tdtype(p.out_dtype)
    y = _empty((T, d), yd, x) if y is None else y
    need = forward_workspace_bytes(p)
    ws = _empty((max(need, 1),), torch.uint8, x) if ws is None else ws
    args = (ctypes.byref(p), _ptr(x, "x", (T, d), dt), _ptr(w_g, "w_g", (d, E), dt),
            _ptr(w1, "w1", (E, h, d), dt), _ptr(w3, "w3", (E, h, d), dt),
            _ptr(w2, "w2", (E, d, h), dt), _ptr(y, "y", (T, d), yd),
            _ptr(topk_idx, "topk_idx", (T, K), torch.int32),
            _ptr(topk_w, "topk_w", (T, K), torch.float32), _ptr(ws, "ws"),
            ws.numel() * ws.element_size(), _stream(stream))
    if events is None:
        _check(lib.moe_forward(*args))
    else:
        _check(lib.moe_forward_profiled(*args, *_events(events)))
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES


def forward_noalloc(p: Problem, x, w_g, w1, w3, w2, y=None, topk_idx=None, topk_w=None,
                    stream=None):
    """moe_forward_noalloc: the whole layer with the library's static scratch array
    as its workspace (no device allocation by the library)."""
    torch = _torch()
    T, d, h, E, K = int(p.T), int(p.d), int(p.h), int(p.E), int(p.K)
    dt = _tdtype(p.dtype)
    yd = _tdtype(p.out_dtype)
    y = _empty((T, d), yd, x) if y is None else y
    _check(lib.moe_forward_noalloc(ctypes.byref(p), _ptr(x, "x", (T, d), dt),
                                   _ptr(w_g, "w_g", (d, E), dt), _ptr(w1, "w1", (E, h, d), dt),
                                   _ptr(w3, "w3", (E, h, d), dt), _ptr(w2, "w2", (E, d, h), dt),
                                   _ptr(y, "y", (T, d), yd),
                                   _ptr(topk_idx, "topk_idx", (T, K), torch.int32),
                                   _ptr(topk_w, "topk_w", (T, K), torch.float32),
                                   _stream(stream)))
    return y
