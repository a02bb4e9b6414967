"""Python binding of libmoe_mi355x, the routed MoE layer for MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libmoe_mi355x.so``; torch tensors supply device memory and the stream.  The
functions carry the C ABI's names (``include/moe.h``).  There is no fallback:
if the library is not built, importing works but the first call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK = 0
MOE_E_TIMEOUT = 8
MOE_E_RANGE = 9
MOE_E_OVERLAP = 10
FMT_Q8_0, FMT_Q4 = 0, 1
STAGE_FULL, STAGE_DOWN = 0, 1
F_RESIDUAL, F_DETERMINISTIC, F_PRENORM, F_FP16_ACT, F_BANDED = 1, 2, 4, 8, 16
BLOCK_BYTES = {FMT_Q8_0: 34, FMT_Q4: 18}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_str(status)})")


class moe_experts(ctypes.Structure):
    _fields_ = [
        ("num_experts", ctypes.c_int32), ("d_model", ctypes.c_int32),
        ("d_ff", ctypes.c_int32), ("format", ctypes.c_int32),
        ("w_gate", ctypes.c_void_p), ("gate_stride", ctypes.c_int64),
        ("w_up", ctypes.c_void_p), ("up_stride", ctypes.c_int64),
        ("w_down", ctypes.c_void_p), ("down_stride", ctypes.c_int64),
    ]


class moe_attn_weights(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("format", ctypes.c_int32),
        ("w_qkv", ctypes.c_void_p), ("attn_gain", ctypes.c_void_p), ("q_gain", ctypes.c_void_p),
        ("k_gain", ctypes.c_void_p),
    ]


class moe_stack_layer(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("experts", moe_experts)]


_lib = None
_P = ctypes.c_void_p
_I32, _I64, _SZ, _F32 = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_SIGS = {
    "moe_abi_version": (_I32, []),
    "moe_status_str": (ctypes.c_char_p, [_I32]),
    "moe_workspace_bytes": (_SZ, [_I64, _I32, _I32, _I32, _I32, _I32, _I32]),
    "moe_route": (_I32, [_P, _I64, _I32, _P, _P, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "moe_group": (_I32, [_P, _I64, _I32, _I32, _P, _P, _P, _SZ, _P]),
    "moe_expert_ffn": (_I32, [_P, _I32, ctypes.POINTER(moe_experts), _P, _P, _P, _P, _I64, _I32,
                              _P, _P, _I32, _P, _SZ, _P]),
    "moe_combine": (_I32, [_P, _P, _I64, _I32, _I32, _P, _P, _P]),
    "moe_layer": (_I32, [_P, _P, _P, ctypes.POINTER(moe_experts), _I64, _I32, _I32, _P, _P, _P,
                         _P, _P, _P, _SZ, _P]),
    "moe_rmsnorm": (_I32, [_P, _I64, _I32, _F32, _P, _P]),
    "moe_decode_stack": (_I32, [_P, _I32, ctypes.POINTER(moe_stack_layer), _I32, _I32, _P, _P,
                                _P, _P, _SZ, _P]),
    "moe_workspace_status": (_I32, [_P, _SZ, _I32, _P]),
    "moe_layer_noalloc": (_I32, [_P, _P, _P, ctypes.POINTER(moe_experts), _I64, _I32, _I32, _P, _P,
                                 _P, _P, _P, _P]),
    "moe_attn_workspace_bytes": (_SZ, [_I64, ctypes.POINTER(moe_attn_weights)]),
    "moe_attn_prep": (_I32, [_P, _I64, ctypes.POINTER(moe_attn_weights), _P, _F32, _F32, _P, _P,
                             _P, _I32, _P, _SZ, _P]),
}
EXPORTS = tuple(_SIGS)


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_routed_lineargate_amd.build`; "
                               "there is no non-HIP implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def abi_version() -> int:
    return lib().moe_abi_version()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _need(t, dtype, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Experts:
    """One layer's experts: device byte buffer(s) plus geometry.

    ``base`` is a uint8 device tensor; expert e's gate/up/down matrices start at
    ``base + gate_off + e*stride`` etc.
    """

    def __init__(self, base, E: int, D: int, F: int, fmt: int, stride: int,
                 gate_off: int, up_off: int, down_off: int):
        import torch
        _need(base, torch.uint8, "experts")
        self.base, self.E, self.D, self.F, self.fmt, self.stride = base, E, D, F, fmt, stride
        p = base.data_ptr()
        self.c = moe_experts(E, D, F, fmt, p + gate_off, stride, p + up_off, stride,
                             p + down_off, stride)

    @classmethod
    def from_blobs(cls, blobs, D: int, F: int, fmt: int):
        """``blobs`` uint8 [E][stride]: per expert gate rows, then up rows, then down rows."""
        bb = BLOCK_BYTES[fmt]
        g = F * (D // 32) * bb
        return cls(blobs, blobs.shape[0], D, F, fmt, blobs.stride(0), 0, g, 2 * g)


def moe_workspace_bytes(T: int, D: int, F: int, E: int, k: int, fmt: int = FMT_Q8_0,
                        flags: int = 0) -> int:
    return int(lib().moe_workspace_bytes(T, D, F, E, k, fmt, flags))


def workspace(T: int, D: int, F: int, E: int, k: int, fmt: int = FMT_Q8_0, flags: int = 0,
              device="cuda"):
    import torch
    n = moe_workspace_bytes(T, D, F, E, k, fmt, flags)
    # zero-filled: the fused kernels keep grid-barrier counters at its start
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def moe_route(x, gate, bias, k: int, topk_ids, topk_w, ws, stream=None):
    import torch
    for t, dt, n in ((x, torch.float32, "x"), (gate, torch.float32, "gate"),
                     (bias, torch.float32, "bias"), (topk_ids, torch.int32, "topk_ids"),
                     (topk_w, torch.float32, "topk_w"), (ws, torch.uint8, "ws")):
        _need(t, dt, n)
    T, D = x.shape
    E = gate.shape[1]
    _check("moe_route", lib().moe_route(_ptr(x), T, D, _ptr(gate), _ptr(bias), E, k,
                                        _ptr(topk_ids), _ptr(topk_w), _ptr(ws),
                                        0 if ws is None else ws.numel(), _stream(stream)))


def moe_group(topk_ids, E: int, expert_offsets, sorted_rows, ws=None, stream=None):
    import torch
    for t, n in ((topk_ids, "topk_ids"), (expert_offsets, "expert_offsets"),
                 (sorted_rows, "sorted_rows")):
        _need(t, torch.int32, n)
    T, k = topk_ids.shape
    _check("moe_group", lib().moe_group(_ptr(topk_ids), T, k, E, _ptr(expert_offsets),
                                        _ptr(sorted_rows), _ptr(ws),
                                        0 if ws is None else ws.numel(), _stream(stream)))


def moe_expert_ffn(inp, stage: int, experts: Experts, topk_ids, topk_w, expert_offsets,
                   sorted_rows, y=None, out=None, flags: int = 0, ws=None, stream=None):
    import torch
    for t, dt, n in ((inp, torch.float32, "in"), (topk_ids, torch.int32, "topk_ids"),
                     (topk_w, torch.float32, "topk_w"), (expert_offsets, torch.int32, "offsets"),
                     (sorted_rows, torch.int32, "sorted_rows"), (y, torch.float32, "y"),
                     (out, torch.float32, "out"), (ws, torch.uint8, "ws")):
        _need(t, dt, n)
    T, k = topk_ids.shape
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        _ptr(inp), stage, ctypes.byref(experts.c), _ptr(topk_ids), _ptr(topk_w),
        _ptr(expert_offsets), _ptr(sorted_rows), T, k, _ptr(y), _ptr(out), flags, _ptr(ws),
        0 if ws is None else ws.numel(), _stream(stream)))


def moe_combine(y, topk_w, out, residual=None, stream=None):
    import torch
    for t, n in ((y, "y"), (topk_w, "topk_w"), (out, "out"), (residual, "residual")):
        _need(t, torch.float32, n)
    T, k = topk_w.shape
    D = out.shape[1]
    _check("moe_combine", lib().moe_combine(_ptr(y), _ptr(topk_w), T, k, D, _ptr(residual),
                                            _ptr(out), _stream(stream)))


def moe_layer(x, gate, bias, experts: Experts, k: int, out, flags: int = 0, topk_ids=None,
              topk_w=None, expert_offsets=None, sorted_rows=None, ws=None, stream=None):
    import torch
    for t, dt, n in ((x, torch.float32, "x"), (gate, torch.float32, "gate"),
                     (bias, torch.float32, "bias"), (out, torch.float32, "out"),
                     (topk_ids, torch.int32, "topk_ids"), (topk_w, torch.float32, "topk_w"),
                     (expert_offsets, torch.int32, "offsets"),
                     (sorted_rows, torch.int32, "sorted_rows"), (ws, torch.uint8, "ws")):
        _need(t, dt, n)
    T = x.shape[0]
    _check("moe_layer", lib().moe_layer(
        _ptr(x), _ptr(gate), _ptr(bias), ctypes.byref(experts.c), T, k, flags, _ptr(out),
        _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_rows), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(stream)))


def moe_workspace_status(ws, reset: bool = False, stream=None) -> int:
    """Status of the workspace's device-side error word (synchronous: waits for
    ``stream``).  MOE_OK; MOE_E_TIMEOUT when a fused kernel's bounded wait gave
    up, else MOE_E_RANGE when a decode stack met a value outside its fixed-point
    range (the outputs hold NaN either way); ``reset`` zero-fills the exchange
    region after an error so the workspace can be used again."""
    import torch
    _need(ws, torch.uint8, "ws")
    return int(lib().moe_workspace_status(_ptr(ws), ws.numel(), 1 if reset else 0,
                                          _stream(stream)))


def check_workspace(ws, stream=None):
    """Raise MoeError if a fused kernel recorded an error on this workspace (a
    bounded wait that gave up, or a decode-stack value out of range)."""
    st = moe_workspace_status(ws, stream=stream)
    if st != MOE_OK:
        raise MoeError("moe_workspace_status", st)


def moe_layer_noalloc(x, gate, bias, experts: Experts, k: int, out, flags: int = 0,
                      topk_ids=None, topk_w=None, expert_offsets=None, sorted_rows=None,
                      stream=None):
    """moe_layer with the library's static workspace (no allocation; see moe.h)."""
    import torch
    for t, dt, n in ((x, torch.float32, "x"), (gate, torch.float32, "gate"),
                     (bias, torch.float32, "bias"), (out, torch.float32, "out"),
                     (topk_ids, torch.int32, "topk_ids"), (topk_w, torch.float32, "topk_w"),
                     (expert_offsets, torch.int32, "offsets"),
                     (sorted_rows, torch.int32, "sorted_rows")):
        _need(t, dt, n)
    T = x.shape[0]
    _check("moe_layer_noalloc", lib().moe_layer_noalloc(
        _ptr(x), _ptr(gate), _ptr(bias), ctypes.byref(experts.c), T, k, flags, _ptr(out),
        _ptr(topk_ids), _ptr(topk_w), _ptr(expert_offsets), _ptr(sorted_rows), _stream(stream)))


def moe_rmsnorm(x, out, eps: float = 1e-6, stream=None):
    import torch
    _need(x, torch.float32, "x")
    _need(out, torch.float32, "out")
    T, D = x.shape
    _check("moe_rmsnorm", lib().moe_rmsnorm(_ptr(x), T, D, eps, _ptr(out), _stream(stream)))


class StackLayers:
    """Host array of moe_stack_layer entries for moe_decode_stack (keeps the
    tensors it points at alive)."""

    def __init__(self, gates, biases, experts):
        import torch
        if not (len(gates) == len(biases) == len(experts)) or not gates:
            raise ValueError("gates, biases and experts need one entry per layer")
        for g, b in zip(gates, biases):
            _need(g, torch.float32, "gate")
            _need(b, torch.float32, "bias")
        self.keep = (list(gates), list(biases), list(experts))
        self.n = len(gates)
        self.c = (moe_stack_layer * self.n)()
        for i, (g, b, ex) in enumerate(zip(gates, biases, experts)):
            self.c[i] = moe_stack_layer(_ptr(g), _ptr(b), ex.c)


def moe_decode_stack(x, layers: StackLayers, k: int, outs, flags: int = 0, topk_ids=None,
                     topk_w=None, ws=None, stream=None):
    """Single-token decode through ``layers.n`` layers: outs [L][D] gets o_l."""
    import torch
    for t, dt, n in ((x, torch.float32, "x"), (outs, torch.float32, "outs"),
                     (topk_ids, torch.int32, "topk_ids"), (topk_w, torch.float32, "topk_w"),
                     (ws, torch.uint8, "ws")):
        _need(t, dt, n)
    if outs.shape[0] != layers.n or (topk_ids is not None and topk_ids.shape != (layers.n, k)) or (
            topk_w is not None and topk_w.shape != (layers.n, k)):
        raise ValueError("outs / topk_ids / topk_w need one row per layer")
    _check("moe_decode_stack", lib().moe_decode_stack(
        _ptr(x), layers.n, layers.c, k, flags, _ptr(outs), _ptr(topk_ids), _ptr(topk_w),
        _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


class AttnWeights:
    """One layer's attention-side weights for moe_attn_prep (keeps the tensors alive).

    ``w_qkv`` uint8 device tensor of (Hq + 2 Hkv) * hd stored rows of D/32 blocks (q
    heads, then k heads, then v heads); gains fp32 device tensors [D], [hd], [hd]."""

    def __init__(self, w_qkv, attn_gain, q_gain, k_gain, D: int, n_q: int, n_kv: int,
                 head_dim: int, fmt: int):
        import torch
        _need(w_qkv, torch.uint8, "w_qkv")
        for t, n in ((attn_gain, "attn_gain"), (q_gain, "q_gain"), (k_gain, "k_gain")):
            _need(t, torch.float32, n)
        self.keep = (w_qkv, attn_gain, q_gain, k_gain)
        self.n_q, self.n_kv, self.hd, self.D = n_q, n_kv, head_dim, D
        self.c = moe_attn_weights(D, n_q, n_kv, head_dim, fmt, _ptr(w_qkv), _ptr(attn_gain),
                                  _ptr(q_gain), _ptr(k_gain))


def attn_workspace(T: int, W: AttnWeights, device="cuda"):
    """Zero-filled workspace for moe_attn_prep (its arrival counters start at zero)."""
    import torch
    n = int(lib().moe_attn_workspace_bytes(T, ctypes.byref(W.c)))
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


def moe_attn_prep(x, W: AttnWeights, pos, q, k_cache, v_cache, rope_theta: float = 1e6,
                  eps: float = 1e-6, ws=None, stream=None):
    """q [T][Hq][hd] <- normalised, rotated q; k_cache / v_cache [max_pos][Hkv][hd]
    get row pos[t] (see moe.h)."""
    import torch
    for t, dt, n in ((x, torch.float32, "x"), (pos, torch.int32, "pos"), (q, torch.float32, "q"),
                     (k_cache, torch.float32, "k_cache"), (v_cache, torch.float32, "v_cache"),
                     (ws, torch.uint8, "ws")):
        _need(t, dt, n)
    T = x.shape[0]
    max_pos = 0 if k_cache is None else k_cache.shape[0]
    _check("moe_attn_prep", lib().moe_attn_prep(
        _ptr(x), T, ctypes.byref(W.c), _ptr(pos), rope_theta, eps, _ptr(q), _ptr(k_cache),
        _ptr(v_cache), max_pos, _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))
