"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every entry point include/moe.h declares, and
reject every hostile argument with the right status before anything would be
launched (mlxcel issue #974: bounds checks assert on the returned status and
never run a forward pass; each hostile case has a positive control).  All
calls below are workspace queries or fail validation, so no HIP call is made.
"""
import copy
import ctypes
import math
import os
import re

import pytest
import torch

import synth
import sparse_mixture_experts_bias_amd as moe
from synth.descs import block_desc

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "moe.h")


def header_functions():
    txt = open(HEADER).read()
    return re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", txt)


def test_library_exports_every_declared_function():
    names = header_functions()
    assert set(names) == {"moe_route", "moe_permute", "moe_experts_forward", "moe_block_forward", "moe_pack_weights",
                          "moe_pack_weights_scaled",
                          "moe_block_forward_noalloc", "moe_set_decode_fusion", "moe_status_str",
                          "moe_last_error", "moe_abi_version", "moe_timing_enable", "moe_timing_read"}
    L = moe.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(moe.EXPORTS) == set(names)


def test_status_strings_and_version():
    L = moe.lib()
    for code, name in enumerate(["MOE_OK", "MOE_ERR_ARG", "MOE_ERR_SHAPE", "MOE_ERR_QUANT", "MOE_ERR_WORKSPACE",
                                 "MOE_ERR_DEVICE", "MOE_ERR_UNSUPPORTED"]):
        assert L.moe_status_str(code).decode() == name
    assert L.moe_status_str(99).decode() == "MOE_ERR_UNKNOWN"
    assert moe.abi_version() >> 16 == 3   # 3: moe_linear.packed_scaled and moe_pack_weights_scaled
    assert L.moe_timing_enable(42) == moe.MOE_ERR_ARG
    assert L.moe_set_decode_fusion(3) == moe.MOE_ERR_ARG
    assert L.moe_set_decode_fusion(2) == moe.MOE_OK
    assert L.moe_set_decode_fusion(-1) == moe.MOE_ERR_ARG
    assert L.moe_set_decode_fusion(1) == moe.MOE_OK
    assert L.moe_timing_enable(0) == moe.MOE_OK
    assert moe.moe_timing_read() == (0, 0.0)


def test_struct_layouts_match_c():
    """ctypes mirrors of the C structs have the C sizes (x86-64 SysV alignment)."""
    assert ctypes.sizeof(moe.MoeLinear) == 7 * 4 + 4 + 6 * 8
    assert moe.MoeLinear.packed_scaled.offset == 7 * 4 + 4 + 5 * 8
    assert ctypes.sizeof(moe.MoeMLP) == 3 * ctypes.sizeof(moe.MoeLinear) + 8
    assert ctypes.sizeof(moe.MoeRouter) == 5 * 4 + 4 + 3 * 8


# ----------------------------------------------------------------------------
# hostile arguments (block descriptor), each with its positive control
# ----------------------------------------------------------------------------

@pytest.fixture(scope="module")
def layers():
    out = {}
    for cfg in ("c1", "c2", "c5"):
        b = synth.make_block(synth.SMALL_SPECS[cfg], "cpu")
        out[cfg] = b
    return out


_HOST_PACKED = []


def host_packed(desc):
    """Point every packed stream of a host-side block descriptor at an aligned host buffer.
    Only validation runs on these descriptors (workspace queries and rejected calls), which
    checks the pointers and never reads through them."""
    buf = (ctypes.c_uint8 * 1024)()
    _HOST_PACKED.append(buf)
    addr = ctypes.addressof(buf) + ((-ctypes.addressof(buf)) % 256)
    c = desc.c
    for lin in (c.experts.gate, c.experts.down, c.shared.gate, c.shared.down, c.latent_down, c.latent_up):
        if lin.n > 0 and not (lin.fmt == moe.MOE_W_DENSE and lin.dense_dtype == moe.MOE_F32):
            lin.packed = addr
    return desc


def bdesc(b):
    return host_packed(block_desc(b))


def query_block(b, desc, T=None, x_dtype=None, y_dtype=None):
    n = ctypes.c_size_t(0)
    T = b.T if T is None else T
    xd = moe.dtype_code(b.x.dtype) if x_dtype is None else x_dtype
    yd = moe.MOE_F32 if y_dtype is None else y_dtype
    st = moe.lib().moe_block_forward(None, xd, T, ctypes.byref(desc.c), None, yd, None, None, None, ctypes.byref(n),
                                     None)
    return st, n.value


def _set(path):
    def f(c, v):
        obj = c
        parts = path.split(".")
        for p in parts[:-1]:
            obj = getattr(obj, p)
        setattr(obj, parts[-1], v)
    return f


# (layer, field path, hostile value, expected status)
HOSTILE = [
    ("c2", "router.top_k", 0, moe.MOE_ERR_SHAPE),
    ("c2", "router.top_k", 33, moe.MOE_ERR_SHAPE),                 # > num_experts (32)
    ("c2", "router.num_experts", 0, moe.MOE_ERR_SHAPE),
    ("c2", "router.num_experts", 513, moe.MOE_ERR_SHAPE),
    ("c2", "router.scoring", 7, moe.MOE_ERR_ARG),
    ("c2", "router.norm_topk", 2, moe.MOE_ERR_ARG),
    ("c2", "router.routed_scale", float("nan"), moe.MOE_ERR_ARG),
    ("c2", "router.w", None, moe.MOE_ERR_ARG),
    ("c2", "hidden", 0, moe.MOE_ERR_SHAPE),
    ("c2", "experts.gate.bits", 0, moe.MOE_ERR_QUANT),
    ("c2", "experts.gate.bits", 8, moe.MOE_ERR_QUANT),
    ("c2", "experts.gate.group_size", 0, moe.MOE_ERR_QUANT),
    ("c2", "experts.down.group_size", 48, moe.MOE_ERR_QUANT),
    ("c2", "experts.up.n", 31, moe.MOE_ERR_SHAPE),                  # fewer planes than num_experts
    ("c2", "experts.up.rows", 0, moe.MOE_ERR_SHAPE),                # zero checked before divisibility
    ("c2", "experts.down.cols", 100, moe.MOE_ERR_SHAPE),
    ("c2", "experts.gate.fmt", 9, moe.MOE_ERR_ARG),
    ("c2", "experts.gate.packed", None, moe.MOE_ERR_ARG),          # the GEMM reads only the packed stream
    ("c2", "experts.down.packed", "misaligned", moe.MOE_ERR_ARG),
    ("c2", "experts.gate.packed_scaled", 1 << 20, moe.MOE_ERR_ARG),  # the scaled stream is MXFP4-only
    ("c5", "experts.down.packed_scaled", (1 << 20) + 64, moe.MOE_ERR_ARG),  # not 256-byte aligned
    ("c2", "experts.up.fmt", moe.MOE_W_MXFP4, moe.MOE_ERR_QUANT),  # up checked on its own first (group 64)
    ("c5", "latent_down.packed", None, moe.MOE_ERR_ARG),
    ("c2", "experts.swiglu_limit", float("inf"), moe.MOE_ERR_ARG),
    ("c2", "shared_mode", 5, moe.MOE_ERR_ARG),
    ("c2", "coef_w", None, moe.MOE_ERR_ARG),                        # blend without its coefficient head
    ("c2", "inter_dtype", 7, moe.MOE_ERR_ARG),
    ("c2", "shared.down.rows", 64, moe.MOE_ERR_SHAPE),
    ("c5", "experts.gate.group_size", 64, moe.MOE_ERR_QUANT),     # MXFP4 blocks are 32
    ("c5", "experts.gate.bits", 0, moe.MOE_ERR_QUANT),
    ("c5", "norm_eps", 0.0, moe.MOE_ERR_ARG),
    ("c5", "norm_eps", float("nan"), moe.MOE_ERR_ARG),
    ("c5", "latent_up.cols", 64, moe.MOE_ERR_SHAPE),
    ("c5", "latent_down.fmt", moe.MOE_W_AFFINE4, moe.MOE_ERR_QUANT),
    ("c5", "shared_mode", moe.MOE_SHARED_BLEND, moe.MOE_ERR_ARG),  # blend needs coef_w (none on c5)
    ("c1", "inter_dtype", moe.MOE_BF16, moe.MOE_ERR_UNSUPPORTED),  # f32 layer keeps f32 intermediates
    ("c1", "experts.gate.dense_dtype", 5, moe.MOE_ERR_ARG),
]


@pytest.mark.parametrize("case", range(len(HOSTILE)), ids=[f"{h[0]}:{h[1]}={h[2]}" for h in HOSTILE])
def test_hostile_block_argument(case, layers):
    cfg, path, val, want = HOSTILE[case]
    b = layers[cfg]
    desc = bdesc(b)
    st, need = query_block(b, desc)
    assert st == moe.MOE_OK and need > 0, "positive control must validate"
    bad = bdesc(b)
    if val == "misaligned":
        obj = bad.c
        for part in path.split(".")[:-1]:
            obj = getattr(obj, part)
        val = getattr(obj, path.split(".")[-1]) + 8
    _set(path)(bad.c, val)
    st, _ = query_block(b, bad)
    assert st == want, (path, val, moe.lib().moe_status_str(st), moe.lib().moe_last_error())
    assert moe.lib().moe_last_error().decode() != ""


def test_token_count_guards(layers):
    b = layers["c2"]
    d = bdesc(b)
    assert query_block(b, d, T=-1)[0] == moe.MOE_ERR_SHAPE
    assert query_block(b, d, T=2 ** 40)[0] == moe.MOE_ERR_SHAPE     # T*K would overflow int32 slot ids
    st, n0 = query_block(b, d, T=0)
    assert st == moe.MOE_OK
    assert query_block(b, d, x_dtype=moe.MOE_F16)[0] == moe.MOE_ERR_ARG
    assert query_block(b, d, y_dtype=moe.MOE_F16)[0] == moe.MOE_ERR_ARG
    assert query_block(layers["c1"], bdesc(layers["c1"]), y_dtype=moe.MOE_BF16)[0] == moe.MOE_ERR_UNSUPPORTED


def test_workspace_grows_with_tokens(layers):
    b = layers["c2"]
    d = bdesc(b)
    sizes = [query_block(b, d, T=t)[1] for t in (1, 64, 1024)]
    assert sizes[0] < sizes[1] < sizes[2]


def test_workspace_too_small_or_misaligned(layers):
    b = layers["c2"]
    d = bdesc(b)
    st, need = query_block(b, d)
    buf = (ctypes.c_uint8 * (need + 512))()
    base = ctypes.addressof(buf)
    aligned = base + ((-base) % 256)
    L = moe.lib()
    n = ctypes.c_size_t(need - 1)
    st = L.moe_block_forward(None, moe.MOE_BF16, b.T, ctypes.byref(d.c), None, moe.MOE_F32, None, None, aligned,
                             ctypes.byref(n), None)
    assert st == moe.MOE_ERR_WORKSPACE
    n = ctypes.c_size_t(need)
    st = L.moe_block_forward(None, moe.MOE_BF16, b.T, ctypes.byref(d.c), None, moe.MOE_F32, None, None, aligned + 8,
                             ctypes.byref(n), None)
    assert st == moe.MOE_ERR_WORKSPACE
    # right size and alignment, but no input pointers: rejected before any launch
    st = L.moe_block_forward(None, moe.MOE_BF16, b.T, ctypes.byref(d.c), None, moe.MOE_F32, None, None, aligned,
                             ctypes.byref(n), None)
    assert st == moe.MOE_ERR_ARG


def test_route_permute_experts_queries(layers):
    L = moe.lib()
    b = layers["c2"]
    r = synth.descs.router_desc(b)
    n = ctypes.c_size_t(0)
    assert L.moe_route(None, moe.MOE_BF16, b.T, b.H, ctypes.byref(r.c), None, None, None, None, ctypes.byref(n),
                       None) == moe.MOE_OK
    assert n.value >= b.T * b.E * 4
    assert L.moe_route(None, moe.MOE_BF16, b.T, 0, ctypes.byref(r.c), None, None, None, None, ctypes.byref(n),
                       None) == moe.MOE_ERR_SHAPE
    assert L.moe_route(None, moe.MOE_BF16, b.T, 100, ctypes.byref(r.c), None, None, None, None, ctypes.byref(n),
                       None) == moe.MOE_ERR_SHAPE
    assert L.moe_permute(None, 1000, 8, 256, None, None, None, None, None, ctypes.byref(n), None) == moe.MOE_OK
    assert n.value > 0
    assert L.moe_permute(None, 10, 0, 256, None, None, None, None, None, ctypes.byref(n), None) == moe.MOE_ERR_SHAPE
    assert L.moe_permute(None, 10, 9, 8, None, None, None, None, None, ctypes.byref(n), None) == moe.MOE_ERR_SHAPE
    assert L.moe_permute(None, 10, 2, 8, None, None, None, None, None, None, None) == moe.MOE_ERR_ARG
    ex = synth.descs.mlp_desc(b.experts)
    buf = (ctypes.c_uint8 * 512)()
    _HOST_PACKED.append(buf)
    ex.c.gate.packed = ex.c.down.packed = ctypes.addressof(buf) + ((-ctypes.addressof(buf)) % 256)
    assert L.moe_experts_forward(None, moe.MOE_BF16, b.T, b.H, ctypes.byref(ex.c), b.E, b.K, None, None, None, None,
                                 None, moe.MOE_BF16, None, None, ctypes.byref(n), None) == moe.MOE_OK
    assert L.moe_experts_forward(None, moe.MOE_BF16, b.T, b.H, ctypes.byref(ex.c), b.E + 1, b.K, None, None, None,
                                 None, None, moe.MOE_BF16, None, None, ctypes.byref(n), None) == moe.MOE_ERR_SHAPE
    assert L.moe_experts_forward(None, moe.MOE_BF16, b.T, b.H, ctypes.byref(ex.c), b.E, b.K, None, None, None, None,
                                 None, moe.MOE_F32, None, None, ctypes.byref(n), None) == moe.MOE_ERR_ARG


# ----------------------------------------------------------------------------
# moe_pack_weights: size queries and rejected arguments (nothing is launched)
# ----------------------------------------------------------------------------

def _pack_query(a, b=None):
    n = ctypes.c_size_t(0)
    st = moe.lib().moe_pack_weights(ctypes.byref(a.c), ctypes.byref(b.c) if b is not None else None, None,
                                    ctypes.byref(n), None)
    return st, n.value


def test_pack_sizes_follow_the_documented_layout(layers):
    """n * row blocks * chunks * record bytes; records are 4096 bytes of weights plus the
    chunk's scales (affine: 4 bytes per row and group, mxfp4: 1 byte per row and block)."""
    from synth.descs import linear_desc
    b2 = layers["c2"]
    g, u, d = (linear_desc(m) for m in (b2.experts.gate, b2.experts.up, b2.experts.down))
    E, I, H, G = b2.E, b2.I, b2.H, b2.experts.gate.group_size
    ceil = lambda a, q: -(-a // q)
    rec_aff = 4096 + 32 * (256 // G) * 4
    assert _pack_query(g, u) == (moe.MOE_OK, E * ceil(I, 16) * ceil(H, 256) * rec_aff)
    assert _pack_query(d) == (moe.MOE_OK, E * ceil(H, 32) * ceil(I, 256) * rec_aff)
    b5 = layers["c5"]
    g5, u5 = linear_desc(b5.experts.gate), linear_desc(b5.experts.up)
    assert _pack_query(g5, u5) == (moe.MOE_OK, b5.E * ceil(b5.I, 16) * ceil(b5.D, 256) * (4096 + 32 * 8))
    ld = linear_desc(b5.latent_down)
    assert _pack_query(ld) == (moe.MOE_OK, ceil(b5.D, 32) * ceil(b5.H, 64) * 4096)
    # the block-scaled MFMA's stream: the same records (1 KB pieces and 256 scale bytes)
    n = ctypes.c_size_t(0)
    assert moe.lib().moe_pack_weights_scaled(ctypes.byref(g5.c), ctypes.byref(u5.c), None, ctypes.byref(n),
                                             None) == moe.MOE_OK
    assert n.value == b5.E * ceil(b5.I, 16) * ceil(b5.D, 256) * (4096 + 256)


def test_pack_rejects_bad_arguments(layers):
    from synth.descs import linear_desc
    L = moe.lib()
    b2 = layers["c2"]
    g, u = linear_desc(b2.experts.gate), linear_desc(b2.experts.up)
    assert _pack_query(g, u)[0] == moe.MOE_OK
    bad = linear_desc(b2.experts.gate)
    bad.c.scales = None                                   # the source planes are read by the packing
    assert _pack_query(bad)[0] == moe.MOE_ERR_ARG
    f32 = linear_desc(layers["c1"].experts.gate)          # dense f32 has no packed form
    assert _pack_query(f32)[0] == moe.MOE_ERR_UNSUPPORTED
    u5 = linear_desc(layers["c5"].experts.up)             # gate and up must share one format and shape
    assert _pack_query(g, u5)[0] in (moe.MOE_ERR_SHAPE, moe.MOE_ERR_UNSUPPORTED)
    assert L.moe_pack_weights(ctypes.byref(g.c), None, None, None, None) == moe.MOE_ERR_ARG
    st, need = _pack_query(g)
    buf = (ctypes.c_uint8 * 1024)()
    base = ctypes.addressof(buf) + ((-ctypes.addressof(buf)) % 256)
    n = ctypes.c_size_t(need - 1)
    assert L.moe_pack_weights(ctypes.byref(g.c), None, base, ctypes.byref(n), None) == moe.MOE_ERR_WORKSPACE
    n = ctypes.c_size_t(need)
    assert L.moe_pack_weights(ctypes.byref(g.c), None, base + 8, ctypes.byref(n), None) == moe.MOE_ERR_ARG
    # the scaled stream exists for MXFP4 weights only
    n = ctypes.c_size_t(0)
    assert L.moe_pack_weights_scaled(ctypes.byref(g.c), None, None, ctypes.byref(n), None) == moe.MOE_ERR_UNSUPPORTED
    assert L.moe_pack_weights_scaled(None, None, None, ctypes.byref(n), None) == moe.MOE_ERR_ARG


def test_noalloc_rejects_more_than_its_scratch(layers):
    """moe_block_forward_noalloc: a call whose workspace would exceed the fixed scratch
    array fails with MOE_ERR_WORKSPACE before any HIP call (no pointers needed); a
    call that fits passes that check (and then needs its tensors: MOE_ERR_ARG)."""
    L = moe.lib()
    b = layers["c2"]
    d = bdesc(b)
    for T, want in ((1 << 16, moe.MOE_ERR_WORKSPACE), (b.T, moe.MOE_ERR_ARG)):
        need = ctypes.c_size_t(0)
        assert L.moe_block_forward(None, moe.MOE_BF16, T, ctypes.byref(d.c), None, moe.MOE_F32, None, None, None,
                                   ctypes.byref(need), None) == moe.MOE_OK
        assert (need.value > moe.NOALLOC_SCRATCH_BYTES) == (want == moe.MOE_ERR_WORKSPACE)
        st = L.moe_block_forward_noalloc(None, moe.MOE_BF16, T, ctypes.byref(d.c), None, moe.MOE_F32, None, None,
                                         None)
        assert st == want, L.moe_last_error()
        if want == moe.MOE_ERR_WORKSPACE:
            assert "scratch" in L.moe_last_error().decode()
