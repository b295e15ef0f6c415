"""The Python binding checks every tensor before the first C call (CPU only).

The C ABI receives raw pointers and sizes, so a tensor of the wrong shape,
dtype or device would be read or written out of bounds on the GPU.  The
binding flattens leading dimensions into the token count with a bounded
product (libmir-metal's ClampedRoutedExperts::forward flattens to
[tokens, hidden] and rejects an overflowing product) and raises ValueError
for every mismatch.  Every case here fails in the binding, before libmoe is
called; the positive controls get as far as the check that a GPU is needed.
"""
import pytest
import torch

import synth
import sparse_mixture_experts_bias_amd as moe
from synth.descs import block_desc, mlp_desc, router_desc


@pytest.fixture(scope="module")
def c2():
    b = synth.make_block(synth.SMALL_SPECS["c2"], "cpu")
    return b, block_desc(b)


def out_tensors(b, lead=None, y_dtype=torch.float32):
    lead = lead if lead is not None else (b.T,)
    return (torch.empty(*lead, b.H, dtype=y_dtype), torch.empty(*lead, b.K, dtype=torch.int32),
            torch.empty(*lead, b.K, dtype=torch.float32))


def expect(msg, fn, *a, **kw):
    with pytest.raises(ValueError, match=msg):
        fn(*a, **kw)


def test_positive_control_reaches_the_gpu_check(c2):
    b, d = c2
    y, i, w = out_tensors(b)
    expect("GPU", moe.moe_block_forward, b.x, d, y, i, w)


def test_leading_dims_flatten(c2):
    """[B, S, H] input with [B, S, ...] or [T, ...] outputs passes every shape check."""
    b, d = c2
    x3 = b.x[:36].reshape(4, 9, b.H)
    y, i, w = out_tensors(b, (4, 9))
    expect("GPU", moe.moe_block_forward, x3, d, y, i, w)
    y2, i2, w2 = out_tensors(b, (36,))
    expect("GPU", moe.moe_block_forward, x3, d, y2, i2, w2)


@pytest.mark.parametrize("case", ["x_width", "x_dtype", "x_noncontig", "x_scalar", "y_shape", "y_dtype",
                                  "y_f32_needed", "idx_dtype", "idx_shape", "w_dtype", "w_shape", "device"])
def test_block_forward_rejects(c2, case):
    b, d = c2
    x = b.x
    y, i, w = out_tensors(b)
    if case == "x_width":
        x = torch.zeros(b.T, b.H + 8, dtype=torch.bfloat16)
    elif case == "x_dtype":
        x = b.x.to(torch.float16)
    elif case == "x_noncontig":
        x = torch.zeros(b.H, b.T, dtype=torch.bfloat16).t()
        expect("last dimension|contiguous", moe.moe_block_forward, x, d, y, i, w)
        x = torch.zeros(b.T, 2 * b.H, dtype=torch.bfloat16)[:, ::2]
        expect("contiguous", moe.moe_block_forward, x, d, y, i, w)
        return
    elif case == "x_scalar":
        x = torch.tensor(1.0, dtype=torch.bfloat16)
    elif case == "y_shape":
        y = torch.empty(b.T, b.H - 8)
    elif case == "y_dtype":
        y = torch.empty(b.T, b.H, dtype=torch.float16)
    elif case == "y_f32_needed":
        x = b.x.float()
        y = torch.empty(b.T, b.H, dtype=torch.bfloat16)
    elif case == "idx_dtype":
        i = torch.empty(b.T, b.K, dtype=torch.int64)
    elif case == "idx_shape":
        i = torch.empty(b.T, b.K + 1, dtype=torch.int32)
    elif case == "w_dtype":
        w = torch.empty(b.T, b.K, dtype=torch.bfloat16)
    elif case == "w_shape":
        w = torch.empty(b.T - 1, b.K, dtype=torch.float32)
    elif case == "device":
        y = torch.empty(b.T, b.H, device="meta")
    # the error names the culprit, not the GPU requirement
    with pytest.raises(ValueError) as ei:
        moe.moe_block_forward(x, d, y, i, w)
    assert "GPU" not in str(ei.value)


def test_token_product_overflow(c2):
    """2^40 tokens (leading dims 2^20 x 2^20) times top_k overflows the int32 slot ids."""
    b, d = c2
    x = torch.empty(2 ** 20, 2 ** 20, b.H, dtype=torch.bfloat16, device="meta")
    y = torch.empty(2 ** 20, 2 ** 20, b.H, dtype=torch.float32, device="meta")
    expect("slot", moe.moe_block_forward, x, d, y)


def test_weights_on_another_device(c2):
    b, d = c2
    x = b.x.to("meta")
    y = torch.empty(b.T, b.H, device="meta")
    expect("weights are on", moe.moe_block_forward, x, d, y)


def test_route_rejects(c2):
    b, _ = c2
    r = router_desc(b)
    i = torch.empty(b.T, b.K, dtype=torch.int32)
    w = torch.empty(b.T, b.K, dtype=torch.float32)
    lg = torch.empty(b.T, b.E, dtype=torch.float32)
    expect("GPU", moe.moe_route, b.x, r, i, w, lg)
    expect("last dimension", moe.moe_route, torch.zeros(b.T, b.H // 2, dtype=torch.bfloat16), r, i, w)
    expect("dtype", moe.moe_route, b.x.float(), r, i, w)
    expect("topk_idx", moe.moe_route, b.x, r, i.long(), w)
    expect("topk_w", moe.moe_route, b.x, r, i, w[:, :-1].contiguous())
    expect("logits", moe.moe_route, b.x, r, i, w, torch.empty(b.T, b.E + 2))
    expect("required", moe.moe_route, b.x, r, None, w)


def test_permute_rejects(c2):
    b, _ = c2
    T, K, E = b.T, b.K, b.E
    idx = torch.zeros(T, K, dtype=torch.int32)
    i32 = lambda *s: torch.empty(*s, dtype=torch.int32)
    args = [i32(E), i32(E + 1), i32(T * K), i32(T * K)]
    expect("GPU", moe.moe_permute, idx, E, *args)
    expect("topk_idx", moe.moe_permute, idx.reshape(-1), E, *args)
    for k, bad in enumerate([i32(E + 1), i32(E), i32(T * K - 1), torch.empty(T * K, dtype=torch.int64)]):
        a = list(args)
        a[k] = bad
        expect("counts|offsets|sorted_slot|slot_pos", moe.moe_permute, idx, E, *a)


def test_experts_forward_rejects(c2):
    b, _ = c2
    ex = mlp_desc(b.experts)
    T, K, E, D = b.T, b.K, b.E, b.H
    i32 = lambda *s: torch.empty(*s, dtype=torch.int32)
    idx, tw = i32(T, K), torch.empty(T, K)
    rest = [i32(E + 1), i32(T * K), i32(T * K)]
    yr = torch.empty(T, D)
    expect("GPU", moe.moe_experts_forward, b.x, ex, E, idx, tw, *rest, yr)
    expect("last dimension", moe.moe_experts_forward, b.x[:, : D // 2].contiguous(), ex, E, idx, tw, *rest, yr)
    expect("experts", moe.moe_experts_forward, b.x, ex, E + 1, idx, tw, *rest, yr)
    expect("y_routed", moe.moe_experts_forward, b.x, ex, E, idx, tw, *rest, yr.to(torch.bfloat16))
    expect("topk_w", moe.moe_experts_forward, b.x, ex, E, idx, tw[:-1], *rest, yr)
    expect("z", moe.moe_experts_forward, b.x.reshape(1, T, D), ex, E, idx, tw, *rest, yr)


def test_routing_state_offsets():
    """The workspace prefix of moe_block_forward: counts, offsets, sorted_slot, slot_pos
    at 256-byte aligned offsets in that order."""
    T, K, E = 37, 8, 32
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    c, o, s, p = moe.routing_state(ws, T, K, E)
    base = ws.data_ptr()
    offs = [t.data_ptr() - base for t in (c, o, s, p)]
    assert offs == [0, 256, 512, 512 + 1280]
    assert [t.numel() for t in (c, o, s, p)] == [E, E + 1, T * K, T * K]
