"""Python binding of libmoe.so (include/moe.h): argument marshalling only.

Every step of the block runs in the library's HIP kernels.  PyTorch supplies
device memory and the current HIP stream; this module turns tensors into the
C descriptors, allocates the caller-side workspace as a torch byte tensor and
raises MoeError on any non-OK status.  If libmoe.so has not been built the
import of the entry points fails loudly: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_SHAPE, MOE_ERR_QUANT, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE, MOE_ERR_UNSUPPORTED = range(7)
MOE_F32, MOE_BF16, MOE_F16 = 0, 1, 2
MOE_SIGMOID, MOE_SOFTMAX = 0, 1
MOE_W_DENSE, MOE_W_AFFINE4, MOE_W_MXFP4 = 0, 1, 2
MOE_SHARED_NONE, MOE_SHARED_ADD, MOE_SHARED_BLEND = 0, 1, 2

FMT_CODES = {"dense": MOE_W_DENSE, "affine4": MOE_W_AFFINE4, "mxfp4": MOE_W_MXFP4}
SHARED_CODES = {"none": MOE_SHARED_NONE, "add": MOE_SHARED_ADD, "blend": MOE_SHARED_BLEND}
SCORING_CODES = {"sigmoid": MOE_SIGMOID, "softmax": MOE_SOFTMAX}

EXPORTS = ("moe_route", "moe_permute", "moe_experts_forward", "moe_block_forward", "moe_pack_weights",
           "moe_timing_enable", "moe_timing_read", "moe_status_str", "moe_last_error", "moe_abi_version")

# kernel classes of moe_timing_enable
TIMING_GATEUP, TIMING_DOWN, TIMING_ROUTER, TIMING_TOPK, TIMING_PERM, TIMING_COMBINE, TIMING_PLAIN = range(1, 8)


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


# ----------------------------------------------------------------------------
# C structs
# ----------------------------------------------------------------------------

class MoeLinear(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("dense_dtype", ctypes.c_int32), ("n", ctypes.c_int32),
                ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("w", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("qbias", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("packed", ctypes.c_void_p)]


class MoeMLP(ctypes.Structure):
    _fields_ = [("gate", MoeLinear), ("up", MoeLinear), ("down", MoeLinear), ("swiglu_limit", ctypes.c_float)]


class MoeRouter(ctypes.Structure):
    _fields_ = [("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("scoring", ctypes.c_int32),
                ("norm_topk", ctypes.c_int32), ("routed_scale", ctypes.c_float), ("w", ctypes.c_void_p),
                ("logit_bias", ctypes.c_void_p), ("select_bias", ctypes.c_void_p)]


class MoeBlock(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("expert_dim", ctypes.c_int32), ("router", MoeRouter),
                ("experts", MoeMLP), ("shared_mode", ctypes.c_int32), ("shared", MoeMLP),
                ("coef_w", ctypes.c_void_p), ("coef_b", ctypes.c_void_p), ("latent_down", MoeLinear),
                ("latent_up", MoeLinear), ("latent_norm_w", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("inter_dtype", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by build.py).  Raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m sparse_mixture_experts_bias_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)
        L.moe_route.argtypes = [vp, i32, i64, i32, ctypes.POINTER(MoeRouter), vp, vp, vp, vp, sz, vp]
        L.moe_permute.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_experts_forward.argtypes = [vp, i32, i64, i32, ctypes.POINTER(MoeMLP), i32, i32, vp, vp, vp, vp, vp,
                                          i32, vp, vp, sz, vp]
        L.moe_block_forward.argtypes = [vp, i32, i64, ctypes.POINTER(MoeBlock), vp, i32, vp, vp, vp, sz, vp]
        L.moe_pack_weights.argtypes = [ctypes.POINTER(MoeLinear), ctypes.POINTER(MoeLinear), vp, sz, vp]
        for f in ("moe_route", "moe_permute", "moe_experts_forward", "moe_block_forward", "moe_pack_weights"):
            getattr(L, f).restype = ctypes.c_int32
        L.moe_status_str.argtypes = [i32]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_timing_enable.argtypes = [i32]
        L.moe_timing_enable.restype = ctypes.c_int32
        L.moe_timing_read.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_double)]
        L.moe_timing_read.restype = ctypes.c_int32
        L.moe_abi_version.argtypes = []
        L.moe_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def _status_name(st: int) -> str:
    try:
        return lib().moe_status_str(st).decode()
    except Exception:
        return f"status {st}"


def _check(st: int):
    if st != MOE_OK:
        raise MoeError(st, lib().moe_last_error().decode())


# ----------------------------------------------------------------------------
# descriptors
# ----------------------------------------------------------------------------

def dtype_code(t: torch.dtype) -> int:
    return {torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.float16: MOE_F16}[t]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors handed to libmoe must be contiguous")
    return t.data_ptr()


class Desc:
    """A ctypes descriptor plus the tensors it points into (kept alive with it)."""

    def __init__(self, c, keep):
        self.c = c
        self.keep = keep


def linear(fmt: str, w: torch.Tensor, scales=None, qbias=None, bias=None, group_size: int = 0) -> Desc:
    """Stacked weights: dense [n, rows, cols]; affine4 int32 [n, rows, cols/8];
    mxfp4 uint8 [n, rows, cols/2]."""
    n, rows = int(w.shape[0]), int(w.shape[1])
    code = FMT_CODES[fmt]
    if code == MOE_W_DENSE:
        cols, dd = int(w.shape[2]), dtype_code(w.dtype)
    elif code == MOE_W_AFFINE4:
        cols, dd = int(w.shape[2]) * 8, 0
    else:
        cols, dd = int(w.shape[2]) * 2, 0
        group_size = 32
    c = MoeLinear(code, dd, n, rows, cols, int(group_size), 0 if code == MOE_W_DENSE else 4,
                  _ptr(w), _ptr(scales), _ptr(qbias), _ptr(bias))
    return Desc(c, [w, scales, qbias, bias])


def _packable(d: Desc) -> bool:
    c = d.c
    return c.fmt != MOE_W_DENSE or c.dense_dtype == MOE_BF16


def _on_gpu(d: Desc) -> bool:
    return d.keep[0] is not None and d.keep[0].is_cuda


def packed_bytes(a: Desc, b: Optional[Desc] = None) -> int:
    """Size of the packed stream moe_pack_weights writes for a (gate/up pair: a, b)."""
    n = ctypes.c_size_t(0)
    _check(lib().moe_pack_weights(ctypes.byref(a.c), ctypes.byref(b.c) if b is not None else None, None,
                                  ctypes.byref(n), None))
    return n.value


def moe_pack_weights(a: Desc, b: Optional[Desc] = None, stream=None) -> torch.Tensor:
    """The packed stream of stack a (or of the gate/up pair a, b) in a new 256-byte
    aligned device buffer; the descriptor is not modified."""
    nbytes = packed_bytes(a, b)
    dev = a.keep[0].device
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    off = (-buf.data_ptr()) % 256
    out = buf[off:off + nbytes]
    n = ctypes.c_size_t(nbytes)
    _check(lib().moe_pack_weights(ctypes.byref(a.c), ctypes.byref(b.c) if b is not None else None, out.data_ptr(),
                                  ctypes.byref(n), _stream(stream)))
    return out


def attach_packed(d: Desc, b: Optional[Desc] = None):
    """Pack d (the gate/up pair d, b) and point d.packed at the stream (kept alive by d)."""
    t = moe_pack_weights(d, b)
    d.c.packed = t.data_ptr()
    d.keep.append(t)


def mlp(gate: Desc, up: Desc, down: Desc, swiglu_limit: float = 0.0) -> Desc:
    """SwiGLU stack; on the GPU the gate/up pair and the down stack are packed here."""
    if _on_gpu(gate) and _packable(gate):
        attach_packed(gate, up)
        attach_packed(down)
    return Desc(MoeMLP(gate.c, up.c, down.c, float(swiglu_limit)), [gate, up, down])


def router(w: torch.Tensor, top_k: int, scoring: str = "sigmoid", norm_topk: bool = True, routed_scale: float = 1.0,
           logit_bias: Optional[torch.Tensor] = None, select_bias: Optional[torch.Tensor] = None) -> Desc:
    c = MoeRouter(int(w.shape[0]), int(top_k), SCORING_CODES[scoring], int(bool(norm_topk)), float(routed_scale),
                  _ptr(w), _ptr(logit_bias), _ptr(select_bias))
    return Desc(c, [w, logit_bias, select_bias])


def block(hidden: int, router_d: Desc, experts: Desc, shared: Optional[Desc] = None, shared_mode: str = "none",
          coef_w=None, coef_b=None, latent_down: Optional[Desc] = None, latent_up: Optional[Desc] = None,
          latent_norm_w=None, norm_eps: float = 1e-5, inter_dtype: int = MOE_BF16) -> Desc:
    D = experts.c.gate.cols
    for lin in (latent_down, latent_up):
        if lin is not None and _on_gpu(lin) and _packable(lin) and not lin.c.packed:
            attach_packed(lin)
    empty_mlp = MoeMLP()
    c = MoeBlock(int(hidden), int(D), router_d.c, experts.c, SHARED_CODES[shared_mode],
                 shared.c if shared is not None else empty_mlp, _ptr(coef_w), _ptr(coef_b),
                 latent_down.c if latent_down is not None else MoeLinear(),
                 latent_up.c if latent_up is not None else MoeLinear(), _ptr(latent_norm_w), float(norm_eps),
                 int(inter_dtype))
    return Desc(c, [router_d, experts, shared, coef_w, coef_b, latent_down, latent_up, latent_norm_w])


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------

def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    nbytes = max(nbytes, 256)
    if ws is not None and ws.numel() >= nbytes:
        return ws, ws.numel()
    t = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + nbytes], nbytes


def route_ws_bytes(x: torch.Tensor, r: Desc, with_logits: bool) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_route(None, dtype_code(x.dtype), x.shape[0], x.shape[1], ctypes.byref(r.c), None, None,
                           1 if with_logits else None, None, ctypes.byref(n), None))
    return n.value


def moe_route(x: torch.Tensor, r: Desc, topk_idx: torch.Tensor, topk_w: torch.Tensor,
              logits: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    L = lib()
    n = ctypes.c_size_t(0)
    _check(L.moe_route(_ptr(x), dtype_code(x.dtype), x.shape[0], x.shape[1], ctypes.byref(r.c), _ptr(topk_idx),
                       _ptr(topk_w), _ptr(logits), None, ctypes.byref(n), None))
    w, nb = _workspace(n.value, x.device, ws)
    n = ctypes.c_size_t(nb)
    _check(L.moe_route(_ptr(x), dtype_code(x.dtype), x.shape[0], x.shape[1], ctypes.byref(r.c), _ptr(topk_idx),
                       _ptr(topk_w), _ptr(logits), _ptr(w),
                       ctypes.byref(n), _stream(stream)))
    return w


def moe_permute(topk_idx: torch.Tensor, E: int, counts, offsets, sorted_slot, slot_pos,
                ws: Optional[torch.Tensor] = None, stream=None):
    L = lib()
    T, K = int(topk_idx.shape[0]), int(topk_idx.shape[1])
    n = ctypes.c_size_t(0)
    args = (_ptr(topk_idx), T, K, int(E), _ptr(counts), _ptr(offsets), _ptr(sorted_slot), _ptr(slot_pos))
    _check(L.moe_permute(*args, None, ctypes.byref(n), None))
    w, nb = _workspace(n.value, topk_idx.device, ws)
    n = ctypes.c_size_t(nb)
    _check(L.moe_permute(*args, _ptr(w), ctypes.byref(n), _stream(stream)))
    return w


def moe_experts_forward(z: torch.Tensor, experts: Desc, E: int, topk_idx, topk_w, offsets, sorted_slot, slot_pos,
                        y_routed: torch.Tensor, inter_dtype: int = MOE_BF16, ws: Optional[torch.Tensor] = None,
                        stream=None):
    L = lib()
    T, K = int(topk_idx.shape[0]), int(topk_idx.shape[1])
    args = (_ptr(z), dtype_code(z.dtype), T, int(z.shape[1]), ctypes.byref(experts.c), int(E), K, _ptr(topk_idx),
            _ptr(topk_w), _ptr(offsets), _ptr(sorted_slot), _ptr(slot_pos), int(inter_dtype), _ptr(y_routed))
    n = ctypes.c_size_t(0)
    _check(L.moe_experts_forward(*args, None, ctypes.byref(n), None))
    w, nb = _workspace(n.value, z.device, ws)
    n = ctypes.c_size_t(nb)
    _check(L.moe_experts_forward(*args, _ptr(w), ctypes.byref(n), _stream(stream)))
    return w


def block_ws_bytes(x: torch.Tensor, b: Desc, with_topk: bool = False) -> int:
    n = ctypes.c_size_t(0)
    dummy = 1 if with_topk else None
    _check(lib().moe_block_forward(None, dtype_code(x.dtype), x.shape[0], ctypes.byref(b.c), None, MOE_F32, dummy,
                                   dummy, None, ctypes.byref(n), None))
    return n.value


def moe_block_forward(x: torch.Tensor, b: Desc, y: torch.Tensor, topk_idx: Optional[torch.Tensor] = None,
                      topk_w: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    L = lib()
    args = (_ptr(x), dtype_code(x.dtype), int(x.shape[0]), ctypes.byref(b.c), _ptr(y), dtype_code(y.dtype),
            _ptr(topk_idx), _ptr(topk_w))
    n = ctypes.c_size_t(0)
    _check(L.moe_block_forward(*args, None, ctypes.byref(n), None))
    w, nb = _workspace(n.value, x.device, ws)
    n = ctypes.c_size_t(nb)
    _check(L.moe_block_forward(*args, _ptr(w), ctypes.byref(n), _stream(stream)))
    return w


def moe_timing_enable(kind: int):
    _check(lib().moe_timing_enable(int(kind)))


def moe_timing_read():
    """-> (number of timed launches, summed milliseconds); clears the record."""
    n, ms = ctypes.c_int32(0), ctypes.c_double(0.0)
    _check(lib().moe_timing_read(ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def abi_version() -> int:
    return lib().moe_abi_version()
