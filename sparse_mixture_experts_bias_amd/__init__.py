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

EXPORTS = ("moe_route", "moe_permute", "moe_experts_forward", "moe_block_forward", "moe_block_forward_noalloc",
           "moe_pack_weights", "moe_pack_weights_scaled", "moe_set_decode_fusion", "moe_timing_enable", "moe_timing_read", "moe_status_str",
           "moe_last_error", "moe_abi_version")
NOALLOC_SCRATCH_BYTES = 32 << 20   # MOE_NOALLOC_SCRATCH_BYTES of include/moe.h

# kernel classes of moe_timing_enable
TIMING_GATEUP, TIMING_DOWN, TIMING_ROUTER, TIMING_TOPK, TIMING_PERM, TIMING_COMBINE, TIMING_PLAIN, TIMING_FUSED = \
    range(1, 9)


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
                ("qbias", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("packed", ctypes.c_void_p),
                ("packed_scaled", ctypes.c_void_p)]


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
        L.moe_pack_weights_scaled.argtypes = [ctypes.POINTER(MoeLinear), ctypes.POINTER(MoeLinear), vp, sz, vp]
        L.moe_block_forward_noalloc.argtypes = [vp, i32, i64, ctypes.POINTER(MoeBlock), vp, i32, vp, vp, vp]
        for f in ("moe_route", "moe_permute", "moe_experts_forward", "moe_block_forward", "moe_pack_weights",
                  "moe_pack_weights_scaled",
                  "moe_block_forward_noalloc"):
            getattr(L, f).restype = ctypes.c_int32
        L.moe_status_str.argtypes = [i32]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_set_decode_fusion.argtypes = [i32]
        L.moe_set_decode_fusion.restype = ctypes.c_int32
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


def packed_bytes(a: Desc, b: Optional[Desc] = None, scaled: bool = False) -> int:
    """Size of the packed stream moe_pack_weights (scaled: moe_pack_weights_scaled) writes
    for a (gate/up pair: a, b)."""
    n = ctypes.c_size_t(0)
    fn = lib().moe_pack_weights_scaled if scaled else lib().moe_pack_weights
    _check(fn(ctypes.byref(a.c), ctypes.byref(b.c) if b is not None else None, None, ctypes.byref(n), None))
    return n.value


def moe_pack_weights(a: Desc, b: Optional[Desc] = None, stream=None, scaled: bool = False) -> torch.Tensor:
    """The packed stream of stack a (or of the gate/up pair a, b) in a new 256-byte
    aligned device buffer; the descriptor is not modified.  scaled: the stream of the
    block-scaled MFMA (moe_pack_weights_scaled, MXFP4 only)."""
    nbytes = packed_bytes(a, b, scaled)
    dev = a.keep[0].device
    buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=dev)
    off = (-buf.data_ptr()) % 256
    out = buf[off:off + nbytes]
    n = ctypes.c_size_t(nbytes)
    fn = lib().moe_pack_weights_scaled if scaled else lib().moe_pack_weights
    _check(fn(ctypes.byref(a.c), ctypes.byref(b.c) if b is not None else None, out.data_ptr(), ctypes.byref(n),
              _stream(stream)))
    return out


def attach_packed(d: Desc, b: Optional[Desc] = None, scaled: bool = False):
    """Pack d (the gate/up pair d, b) and point d.packed (scaled: d.packed_scaled) at the
    stream (kept alive by d)."""
    t = moe_pack_weights(d, b, scaled=scaled)
    if scaled:
        d.c.packed_scaled = t.data_ptr()
    else:
        d.c.packed = t.data_ptr()
    d.keep.append(t)


def mlp(gate: Desc, up: Desc, down: Desc, swiglu_limit: float = 0.0, scaled: bool = False) -> Desc:
    """SwiGLU stack; on the GPU the gate/up pair and the down stack are packed here.
    scaled (MXFP4): also the streams of the block-scaled MFMA (moe_linear.packed_scaled)."""
    if _on_gpu(gate) and _packable(gate):
        attach_packed(gate, up)
        attach_packed(down)
        if scaled and gate.c.fmt == MOE_W_MXFP4:
            attach_packed(gate, up, scaled=True)
            attach_packed(down, scaled=True)
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
# argument checks (the C ABI sees pointers only: every size it relies on is
# checked here, before the first C call)
# ----------------------------------------------------------------------------

_INT32_LIMIT = 2 ** 31


def _bad(msg: str):
    raise ValueError(msg)


def _tensor(t, name: str, shape, dtypes, device=None) -> torch.Tensor:
    """t must be a contiguous tensor of one of `dtypes` with exactly `shape`
    (a tuple of ints) on `device` (when given)."""
    if not isinstance(t, torch.Tensor):
        _bad(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in dtypes:
        _bad(f"{name} has dtype {t.dtype}, expected {' or '.join(str(d) for d in dtypes)}")
    if tuple(t.shape) != tuple(shape):
        _bad(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        _bad(f"{name} must be contiguous")
    if device is not None and t.device != device:
        _bad(f"{name} is on {t.device}, expected {device} (every tensor of a call lives on one device)")
    return t


def _tokens(x: torch.Tensor, name: str, width: int, what: str) -> int:
    """Rows of x seen as [tokens, width]: every leading dimension flattens into
    the token count (the product is exact in Python integers and bounded here,
    as libmir-metal's ClampedRoutedExperts::forward bounds its checked product)."""
    if not isinstance(x, torch.Tensor):
        _bad(f"{name} must be a torch.Tensor, got {type(x).__name__}")
    if x.dim() < 1:
        _bad(f"{name} must have at least one dimension ([..., {what}])")
    if int(x.shape[-1]) != width:
        _bad(f"{name} has last dimension {int(x.shape[-1])}, expected {what} = {width}")
    T = 1
    for d in x.shape[:-1]:
        T *= int(d)
    if T * max(width, 1) >= 2 ** 62:
        _bad(f"{name}: {T} tokens x {width} elements overflows the token product")
    if not x.is_contiguous():
        _bad(f"{name} must be contiguous")
    return T


def _gpu(device: torch.device):
    if device.type != "cuda":
        _bad(f"tensors are on {device}: libmoe runs on a GPU (HIP) device only")


def _slots(T: int, K: int):
    if T * K >= _INT32_LIMIT:
        _bad(f"{T} tokens x top_k {K} = {T * K} slots exceeds the int32 slot numbering")


def _desc_device(d: "Desc") -> torch.device:
    """The one device every tensor of a descriptor lives on."""
    devs = set()

    def walk(obj):
        if isinstance(obj, torch.Tensor):
            devs.add(obj.device)
        elif isinstance(obj, Desc):
            for k in obj.keep:
                walk(k)
        elif isinstance(obj, (list, tuple)):
            for k in obj:
                walk(k)
    walk(d)
    if len(devs) != 1:
        _bad(f"descriptor tensors live on {sorted(str(v) for v in devs) or 'no device'}, expected one device")
    return devs.pop()


_ACT = (torch.float32, torch.bfloat16)
_INTER_DT = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16, MOE_F16: torch.float16}


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------

def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    nbytes = max(nbytes, 256)
    if ws is not None:
        if not isinstance(ws, torch.Tensor) or ws.dtype != torch.uint8 or ws.dim() != 1 or ws.device != device:
            _bad(f"ws must be a 1-D uint8 tensor on {device}")
        if ws.data_ptr() % 256:
            _bad("ws must be 256-byte aligned")
        if ws.numel() >= nbytes:
            return ws, ws.numel()
    t = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-t.data_ptr()) % 256
    return t[off:off + nbytes], nbytes


def _router_shape(r: Desc):
    w = r.keep[0]
    return int(w.shape[0]), int(w.shape[1]), w.dtype


def route_ws_bytes(x: torch.Tensor, r: Desc, with_logits: bool) -> int:
    E, H, _ = _router_shape(r)
    T = _tokens(x, "x", H, "hidden")
    n = ctypes.c_size_t(0)
    _check(lib().moe_route(None, dtype_code(x.dtype), T, H, ctypes.byref(r.c), None, None,
                           1 if with_logits else None, None, ctypes.byref(n), None))
    return n.value


def moe_route(x: torch.Tensor, r: Desc, topk_idx: torch.Tensor, topk_w: torch.Tensor,
              logits: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """x [..., H]; topk_idx int32 / topk_w float32 [..., K] (or [T, K]); logits float32
    [..., E] (or [T, E]) or None."""
    E, H, wdt = _router_shape(r)
    K = int(r.c.top_k)
    T = _tokens(x, "x", H, "hidden (router weight columns)")
    if x.dtype != wdt:
        _bad(f"x has dtype {x.dtype}, the router weight {wdt}")
    if x.dtype not in _ACT:
        _bad(f"x has dtype {x.dtype}, expected float32 or bfloat16")
    _slots(T, K)
    dev = x.device
    lead = tuple(x.shape[:-1])
    for t, name, width, dt in ((topk_idx, "topk_idx", K, torch.int32), (topk_w, "topk_w", K, torch.float32),
                               (logits, "logits", E, torch.float32)):
        if t is None:
            if name == "logits":
                continue
            _bad(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            _bad(f"{name} must be a torch.Tensor")
        _tensor(t, name, (*lead, width) if tuple(t.shape[:-1]) == lead else (T, width), (dt,), dev)
    if _desc_device(r) != dev:
        _bad(f"the router weights are on {_desc_device(r)}, x on {dev}")
    _gpu(dev)
    L = lib()
    n = ctypes.c_size_t(0)
    _check(L.moe_route(_ptr(x), dtype_code(x.dtype), T, H, ctypes.byref(r.c), _ptr(topk_idx),
                       _ptr(topk_w), _ptr(logits), None, ctypes.byref(n), None))
    w, nb = _workspace(n.value, dev, ws)
    n = ctypes.c_size_t(nb)
    _check(L.moe_route(_ptr(x), dtype_code(x.dtype), T, H, ctypes.byref(r.c), _ptr(topk_idx),
                       _ptr(topk_w), _ptr(logits), _ptr(w),
                       ctypes.byref(n), _stream(stream)))
    return w


def moe_permute(topk_idx: torch.Tensor, E: int, counts, offsets, sorted_slot, slot_pos,
                ws: Optional[torch.Tensor] = None, stream=None):
    """topk_idx int32 [T, K]; counts int32 [E]; offsets int32 [E+1]; sorted_slot,
    slot_pos int32 [T*K]."""
    if not isinstance(topk_idx, torch.Tensor) or topk_idx.dim() != 2:
        _bad("topk_idx must be a 2-D tensor [T, K]")
    T, K = int(topk_idx.shape[0]), int(topk_idx.shape[1])
    E = int(E)
    _slots(T, K)
    dev = topk_idx.device
    i32 = (torch.int32,)
    _tensor(topk_idx, "topk_idx", (T, K), i32, dev)
    _tensor(counts, "counts", (E,), i32, dev)
    _tensor(offsets, "offsets", (E + 1,), i32, dev)
    _tensor(sorted_slot, "sorted_slot", (T * K,), i32, dev)
    _tensor(slot_pos, "slot_pos", (T * K,), i32, dev)
    _gpu(dev)
    L = lib()
    n = ctypes.c_size_t(0)
    args = (_ptr(topk_idx), T, K, E, _ptr(counts), _ptr(offsets), _ptr(sorted_slot), _ptr(slot_pos))
    _check(L.moe_permute(*args, None, ctypes.byref(n), None))
    w, nb = _workspace(n.value, dev, ws)
    n = ctypes.c_size_t(nb)
    _check(L.moe_permute(*args, _ptr(w), ctypes.byref(n), _stream(stream)))
    return w


def moe_experts_forward(z: torch.Tensor, experts: Desc, E: int, topk_idx, topk_w, offsets, sorted_slot, slot_pos,
                        y_routed: torch.Tensor, inter_dtype: int = MOE_BF16, ws: Optional[torch.Tensor] = None,
                        stream=None):
    """z [T, D]; topk_idx int32 / topk_w float32 [T, K]; offsets int32 [E+1];
    sorted_slot, slot_pos int32 [T*K]; y_routed float32 [T, D]."""
    D = int(experts.c.gate.cols)
    if int(E) != int(experts.c.gate.n):
        _bad(f"E = {E} but the expert stack holds {experts.c.gate.n} experts")
    if not isinstance(z, torch.Tensor) or z.dim() != 2:
        _bad("z must be a 2-D tensor [T, D]")
    T = _tokens(z, "z", D, "expert input width (gate columns)")
    if z.dtype not in (torch.float32, torch.bfloat16, torch.float16):
        _bad(f"z has dtype {z.dtype}, expected float32, bfloat16 or float16")
    if not isinstance(topk_idx, torch.Tensor) or topk_idx.dim() != 2:
        _bad("topk_idx must be a 2-D tensor [T, K]")
    K = int(topk_idx.shape[1])
    _slots(T, K)
    dev = z.device
    i32 = (torch.int32,)
    _tensor(topk_idx, "topk_idx", (T, K), i32, dev)
    _tensor(topk_w, "topk_w", (T, K), (torch.float32,), dev)
    _tensor(offsets, "offsets", (int(E) + 1,), i32, dev)
    _tensor(sorted_slot, "sorted_slot", (T * K,), i32, dev)
    _tensor(slot_pos, "slot_pos", (T * K,), i32, dev)
    _tensor(y_routed, "y_routed", (T, D), (torch.float32,), dev)
    if _desc_device(experts) != dev:
        _bad(f"the expert weights are on {_desc_device(experts)}, z on {dev}")
    _gpu(dev)
    L = lib()
    args = (_ptr(z), dtype_code(z.dtype), T, D, ctypes.byref(experts.c), int(E), K, _ptr(topk_idx),
            _ptr(topk_w), _ptr(offsets), _ptr(sorted_slot), _ptr(slot_pos), int(inter_dtype), _ptr(y_routed))
    n = ctypes.c_size_t(0)
    _check(L.moe_experts_forward(*args, None, ctypes.byref(n), None))
    w, nb = _workspace(n.value, dev, ws)
    n = ctypes.c_size_t(nb)
    _check(L.moe_experts_forward(*args, _ptr(w), ctypes.byref(n), _stream(stream)))
    return w


def block_ws_bytes(x: torch.Tensor, b: Desc, with_topk: bool = False) -> int:
    T = _tokens(x, "x", int(b.c.hidden), "hidden")
    n = ctypes.c_size_t(0)
    dummy = 1 if with_topk else None
    _check(lib().moe_block_forward(None, dtype_code(x.dtype), T, ctypes.byref(b.c), None, MOE_F32, dummy,
                                   dummy, None, ctypes.byref(n), None))
    return n.value


def _check_block_call(x, b: Desc, y, topk_idx, topk_w):
    H, K = int(b.c.hidden), int(b.c.router.top_k)
    T = _tokens(x, "x", H, "hidden")
    if x.dtype not in _ACT:
        _bad(f"x has dtype {x.dtype}, expected float32 or bfloat16")
    _slots(T, K)
    dev = x.device
    lead = tuple(x.shape[:-1])
    shape_of = lambda t, w: (*lead, w) if isinstance(t, torch.Tensor) and tuple(t.shape[:-1]) == lead else (T, w)
    _tensor(y, "y", shape_of(y, H), _ACT, dev)
    if x.dtype == torch.float32 and y.dtype != torch.float32:
        _bad("float32 x needs a float32 y")
    if topk_idx is not None:
        _tensor(topk_idx, "topk_idx", shape_of(topk_idx, K), (torch.int32,), dev)
    if topk_w is not None:
        _tensor(topk_w, "topk_w", shape_of(topk_w, K), (torch.float32,), dev)
    if _desc_device(b) != dev:
        _bad(f"the block's weights are on {_desc_device(b)}, x on {dev}")
    return T, dev


def moe_block_forward(x: torch.Tensor, b: Desc, y: torch.Tensor, topk_idx: Optional[torch.Tensor] = None,
                      topk_w: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None, stream=None):
    """x [..., H] (leading dimensions flatten into the token count); y [..., H] or
    [T, H] float32/bfloat16; topk_idx int32 / topk_w float32 [..., K] or [T, K].
    Returns the workspace used: after the call it begins with the routing state
    (see routing_state)."""
    T, dev = _check_block_call(x, b, y, topk_idx, topk_w)
    _gpu(dev)
    L = lib()
    args = (_ptr(x), dtype_code(x.dtype), T, ctypes.byref(b.c), _ptr(y), dtype_code(y.dtype),
            _ptr(topk_idx), _ptr(topk_w))
    n = ctypes.c_size_t(0)
    _check(L.moe_block_forward(*args, None, ctypes.byref(n), None))
    w, nb = _workspace(n.value, dev, ws)
    n = ctypes.c_size_t(nb)
    _check(L.moe_block_forward(*args, _ptr(w), ctypes.byref(n), _stream(stream)))
    return w


def moe_block_forward_noalloc(x: torch.Tensor, b: Desc, y: torch.Tensor, topk_idx: Optional[torch.Tensor] = None,
                              topk_w: Optional[torch.Tensor] = None, stream=None):
    """moe_block_forward on the library's fixed per-GPU scratch array (no workspace is
    allocated anywhere); same arguments and checks.  Calls that overlap on one GPU race."""
    T, dev = _check_block_call(x, b, y, topk_idx, topk_w)
    _gpu(dev)
    _check(lib().moe_block_forward_noalloc(_ptr(x), dtype_code(x.dtype), T, ctypes.byref(b.c), _ptr(y),
                                           dtype_code(y.dtype), _ptr(topk_idx), _ptr(topk_w), _stream(stream)))


def routing_state(ws: torch.Tensor, T: int, K: int, E: int):
    """Views of the routing state a moe_block_forward call left at the start of its
    workspace (include/moe.h): counts [E], offsets [E+1], sorted_slot [T*K],
    slot_pos [T*K], each int32 and 256-byte aligned, in that order."""
    al = lambda n: (n + 255) // 256 * 256
    o_counts = 0
    o_offsets = o_counts + al(4 * E)
    o_ss = o_offsets + al(4 * (E + 1))
    o_sp = o_ss + al(4 * T * K)
    v = lambda off, n: ws[off:off + 4 * n].view(torch.int32)
    return v(o_counts, E), v(o_offsets, E + 1), v(o_ss, T * K), v(o_sp, T * K)


def call_status(ws: torch.Tensor, T: int, K: int, E: int) -> torch.Tensor:
    """The status word after the routing state (0: every bounded wait completed)."""
    al = lambda n: (n + 255) // 256 * 256
    off = al(4 * E) + al(4 * (E + 1)) + 2 * al(4 * T * K)
    return ws[off:off + 4].view(torch.int32)


DECODE_SEPARATE, DECODE_THREE_LAUNCHES, DECODE_SINGLE_LAUNCH = 0, 1, 2


def moe_set_decode_fusion(mode):
    """Decode-sized batches: True / DECODE_THREE_LAUNCHES (default: routing, experts and
    combine launches), DECODE_SINGLE_LAUNCH (one launch up to 16 tokens, three above), or
    False / DECODE_SEPARATE (the separate router, routing, gate/up, down and combine launches)."""
    _check(lib().moe_set_decode_fusion(int(mode)))


def moe_timing_enable(kind: int):
    _check(lib().moe_timing_enable(int(kind)))


def moe_timing_read():
    """-> (number of timed launches, summed milliseconds); clears the record."""
    n, ms = ctypes.c_int32(0), ctypes.c_double(0.0)
    _check(lib().moe_timing_read(ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def abi_version() -> int:
    return lib().moe_abi_version()
