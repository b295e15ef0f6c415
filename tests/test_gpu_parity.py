"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Every case prints its name, shape and seed before touching the GPU.
Inputs are drawn on the GPU by the seeded generator; the oracle reads the
same stored bytes copied to the host.
"""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth
import sparse_mixture_experts_bias_amd as moe
from synth.descs import block_desc, mlp_desc, inter_dtype_for

from parity import check_output, check_permutation, check_routing, np32, run_block, run_route

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def announce(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.lib()
    yield


def _full_check(b: synth.Block, label: str, y_dtype=torch.float32):
    announce(f"{label}: T={b.T} H={b.H} E={b.E} K={b.K} seed={b.seed}")
    y, idx, w, state = run_block(b, y_dtype, with_state=True)
    check_permutation(idx, b.E, state)
    gidx, gw, glog = run_route(b)
    assert torch.equal(gidx, idx), "moe_route and moe_block_forward disagree on the selection"
    assert torch.equal(gw, w)
    ob = O.from_block(b)
    routing, rep = check_routing(ob, np32(idx).astype(np.int64), np32(w), np32(glog),
                                 w_tol=(1e-5, 1e-6) if b.x.dtype == torch.float32 else (1e-4, 1e-5))
    ref = O.block_forward(ob, routing=routing)["y"]
    f32 = b.x.dtype == torch.float32
    stats = check_output(np32(y), ref, f32, label)
    print(f"[ok] {label}: {stats} {rep}", flush=True)
    return y, idx, w, ob, routing


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4", "c5"])
def test_block_small(cfg):
    b = synth.make_block(synth.SMALL_SPECS[cfg], DEV)
    _full_check(b, f"{cfg}-small")


@pytest.mark.parametrize("T", [64, 65, 255, 256, 257])
def test_block_path_boundaries(T):
    """Token counts at the switches between launch paths: one-launch routing (T <= 64) or
    top-k + permutation kernels; the decode router or the tiled one (T >= 256); the
    single-workgroup permutation (T <= 256) or the three-kernel one."""
    b = synth.make_block(synth.SMALL_SPECS["c2"], DEV, T=T)
    _full_check(b, f"c2-small T={T}")


@pytest.mark.parametrize("T,H,E", [(256, 544, 72), (301, 2080, 136), (300, 1024, 130)])
def test_router_tiled_ragged(T, H, E):
    """Router for many tokens: the tiled GEMM with its reduction split into slices (a
    slice and the reduction ending inside a chunk, ragged token and expert tiles, the
    blend head's two rows in the last tile), and an expert count the tiled GEMM does not
    take (not a multiple of 8)."""
    from dataclasses import replace
    spec = replace(synth.FULL_SPECS["c3"], name="router-tiled", T=T, H=H, E=E, K=6, I=64, I_s=64,
                   group=32, seed=T + E)
    _full_check(synth.make_block(spec, DEV), f"router-tiled T={T} H={H} E={E}")


def test_block_full_c1():
    b = synth.make_block(synth.FULL_SPECS["c1"], DEV)
    _full_check(b, "c1-full")


def test_block_full_c2_decode():
    """The decode layer at its full size, every token through the oracle."""
    b = synth.make_block(synth.FULL_SPECS["c2"], DEV)
    _full_check(b, "c2-full")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg,inter", [("c3", None), ("c4", None), ("c5", None), ("c3", "bf16"), ("c4", "bf16")])
def test_block_full_every_token(cfg, inter):
    """Full-size layers in the launch configuration of the benchmark: routing, the
    permutation the experts ran on, and the output of every token against the oracle
    (the oracle decodes each expert once and applies it to all of its tokens).  "bf16":
    the layer with bf16 intermediates instead of its default."""
    spec = synth.FULL_SPECS[cfg]
    b = synth.make_block(spec, DEV)
    announce(f"{cfg}-full inter={inter}: T={b.T} H={b.H} E={b.E} K={b.K} seed={b.seed}")
    y, idx, w, state = run_block(b, inter=moe.MOE_BF16 if inter == "bf16" else None, with_state=True)
    check_permutation(idx, b.E, state)
    gidx, gw, glog = run_route(b)
    assert torch.equal(gidx, idx) and torch.equal(gw, w)
    ob = O.from_block(b)
    routing, rep = check_routing(ob, np32(idx).astype(np.int64), np32(w), np32(glog))
    print(f"[routing] {cfg}-full {rep}; m-tile rows per expert: max {int(state[0].max())}", flush=True)
    ref = O.block_forward(ob, routing=routing)["y"]
    stats = check_output(np32(y), ref, False, f"{cfg}-full")
    print(f"[ok] {cfg}-full, all {b.T} tokens: {stats}", flush=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("cfg", ["c2", "c3", "c4", "c5"])
@pytest.mark.parametrize("seed", [101, 102, 103])
def test_block_full_other_seeds(cfg, seed):
    """The full-size layers drawn from three more seeds (a robustness check of the parity:
    skew, near-ties and segment sizes change with the draw): routing, permutation and every
    token's output against the oracle."""
    b = synth.make_block(synth.FULL_SPECS[cfg], DEV, seed=seed)
    announce(f"{cfg}-full seed {seed}: T={b.T} H={b.H} E={b.E} K={b.K}")
    y, idx, w, state = run_block(b, with_state=True)
    check_permutation(idx, b.E, state)
    gidx, gw, glog = run_route(b)
    assert torch.equal(gidx, idx) and torch.equal(gw, w)
    ob = O.from_block(b)
    routing, rep = check_routing(ob, np32(idx).astype(np.int64), np32(w), np32(glog))
    ref = O.block_forward(ob, routing=routing)["y"]
    stats = check_output(np32(y), ref, False, f"{cfg}-full seed {seed}")
    print(f"[ok] {cfg}-full seed {seed}: {stats} {rep}", flush=True)


def _check_permute(idx: torch.Tensor, E: int):
    T, K = idx.shape
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    ss = torch.empty(T * K, dtype=torch.int32, device=DEV)
    sp = torch.empty(T * K, dtype=torch.int32, device=DEV)
    moe.moe_permute(idx, E, counts, offsets, ss, sp)
    torch.cuda.synchronize()
    c, o, s, p = O.permute(idx.cpu().numpy(), E)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(ss.cpu().numpy(), s)
    assert np.array_equal(sp.cpu().numpy(), p)
    return counts, offsets, ss, sp


@pytest.mark.parametrize("T,E,K", [(1, 8, 2), (37, 32, 8), (256, 64, 6), (257, 16, 4), (1000, 384, 8),
                                   (4096, 256, 8)])
def test_permute_bit_exact(T, E, K):
    announce(f"permute T={T} E={E} K={K}")
    g = torch.Generator().manual_seed(T * 7 + E)
    # skewed random selections: distinct experts per token, ascending
    pri = torch.rand(T, E, generator=g) + torch.linspace(0, 2, E)[torch.randperm(E, generator=g)]
    idx = pri.topk(K, dim=1).indices.sort(dim=1).values.to(torch.int32).to(DEV)
    _check_permute(idx, E)


def test_route_entry_exports_logits():
    b = synth.make_block(synth.SMALL_SPECS["c4"], DEV)
    announce("moe_route c4-small")
    idx, w, logits = run_route(b)
    ob = O.from_block(b)
    ref = O.router_logits(ob.x, ob.router_w, ob.logit_bias)
    assert np.allclose(np32(logits), ref, rtol=1e-4, atol=1e-4)
    check_routing(ob, np32(idx).astype(np.int64), np32(w), np32(logits))


@pytest.mark.parametrize("cfg", ["c2", "c5"])
def test_experts_forward_entry(cfg):
    """moe_experts_forward alone: routed sum on z = x (or the stored latent z)."""
    b = synth.make_block(synth.SMALL_SPECS[cfg], DEV)
    announce(f"moe_experts_forward {cfg}-small")
    idx, w, _ = run_route(b)
    counts, offsets, ss, sp = _check_permute(idx, b.E)
    if b.latent_down is None:
        z = b.x
    else:  # an arbitrary fp16 latent input
        g = torch.Generator(device=DEV).manual_seed(99)
        z = torch.randn(b.T, b.D, generator=g, device=DEV).to(torch.float16)
    inter = inter_dtype_for(b)
    yr = torch.empty(b.T, z.shape[1], dtype=torch.float32, device=DEV)
    moe.moe_experts_forward(z, mlp_desc(b.experts), b.E, idx, w, offsets, ss, sp, yr, inter_dtype=inter)
    torch.cuda.synchronize()
    ob = O.from_block(b)
    zf = z.double().cpu().numpy()
    routing = {"idx": idx.cpu().numpy().astype(np.int64), "w": w.double().cpu().numpy()}
    o = O.routed_outputs(ob, zf, routing)
    ref = np.einsum("tk,tkd->td", routing["w"], o)
    check_output(np32(yr), ref, False, f"experts-{cfg}")


def test_mxfp4_scale_extremes():
    """E8M0 scale bytes 0 (2^-127) and 255 (NaN, OCP MX) in routed MXFP4 weights: the
    kernels hand the byte to the scaled FP4 conversion as its scale exponent.  NaN reaches
    exactly the output rows the oracle's does (every token routed to the poisoned expert);
    an expert whose scales are all 0 contributes ~nothing; the rest matches the oracle."""
    b = synth.make_block(synth.SMALL_SPECS["c5"], DEV)
    announce("MXFP4 scale bytes 0 and 255, c5-small")
    idx, w, _ = run_route(b)
    e_nan, e_tiny = int(idx[0, 0]), int(idx[0, 1])
    sc = b.experts.gate.scales.clone()
    sc[e_nan, 3, 0] = 255
    sc[e_tiny] = 0
    b.experts.gate.scales = sc
    counts, offsets, ss, sp = _check_permute(idx, b.E)
    g = torch.Generator(device=DEV).manual_seed(98)
    z = torch.randn(b.T, b.D, generator=g, device=DEV).to(torch.float16)
    yr = torch.empty(b.T, b.D, dtype=torch.float32, device=DEV)
    moe.moe_experts_forward(z, mlp_desc(b.experts), b.E, idx, w, offsets, ss, sp, yr, inter_dtype=inter_dtype_for(b))
    torch.cuda.synchronize()
    ob = O.from_block(b)
    routing = {"idx": idx.cpu().numpy().astype(np.int64), "w": w.double().cpu().numpy()}
    with np.errstate(invalid="ignore"):
        o = O.routed_outputs(ob, z.double().cpu().numpy(), routing)
        ref = np.einsum("tk,tkd->td", routing["w"], o)
    got = np32(yr)
    nan_ref, nan_got = np.isnan(ref).all(axis=1), np.isnan(got).all(axis=1)
    assert nan_ref[0] and (nan_ref == nan_got).all(), "NaN rows differ from the oracle's"
    assert not np.isnan(got[~nan_got]).any() and not np.isnan(ref[~nan_ref]).any()
    check_output(got[~nan_ref], ref[~nan_ref], False, "mxfp4-scale-extremes")


def test_zero_tokens_is_noop():
    b = synth.make_block(synth.SMALL_SPECS["c2"], DEV, T=0)
    announce("T=0")
    y, idx, w = run_block(b)
    assert y.shape == (0, b.H)


@pytest.mark.parametrize("cfg", ["c2", "c5"])
def test_single_token(cfg):
    b = synth.make_block(synth.SMALL_SPECS[cfg], DEV, T=1)
    _full_check(b, f"{cfg}-T1")


def test_all_equal_scores_tie_rule():
    """Zero router weights, no biases: every key ties; experts 0..K-1 are chosen."""
    b = synth.make_block(synth.SMALL_SPECS["c2"], DEV)
    b.router_w = torch.zeros_like(b.router_w)
    b.logit_bias = None
    b.select_bias = None
    announce("tie rule c2-small")
    y, idx, w = run_block(b)
    assert (idx.cpu() == torch.arange(b.K, dtype=torch.int32)).all()
    assert torch.allclose(w.cpu(), torch.full_like(w.cpu(), 1.0 / b.K), rtol=1e-6, atol=0)
    _full_check(b, "tie-c2")


def test_topk_equals_experts_softmax():
    """K = E with softmax scores: every expert is chosen (the dense mixture)."""
    spec = synth.replace(synth.SMALL_SPECS["c4"], E=8, K=8, T=40, seed=41)
    b = synth.make_block(spec, DEV)
    y, idx, w = _full_check(b, "K=E softmax")[:3]
    assert (idx.cpu() == torch.arange(8, dtype=torch.int32)).all()


def test_zero_routed_branch_blend():
    """Down weights zeroed (scales and qbias 0): y = coef[1] * shared."""
    b = synth.make_block(synth.SMALL_SPECS["c2"], DEV)
    b.experts.down.scales = torch.zeros_like(b.experts.down.scales)
    b.experts.down.qbias = torch.zeros_like(b.experts.down.qbias)
    y, idx, w, ob, routing = _full_check(b, "zero-routed c2")
    out = O.block_forward(ob, routing=routing)
    assert np.array_equal(out["y_routed"], np.zeros_like(out["y_routed"]))


@pytest.mark.parametrize("cfg", ["c2", "c5"])
def test_batch_invariance_bitwise(cfg):
    """A token's output does not depend on the other tokens in the batch (rows of
    a segment never mix): bitwise equal when run alone."""
    b = synth.make_block(synth.SMALL_SPECS[cfg], DEV)
    announce(f"batch invariance {cfg}")
    y, idx, w = run_block(b)
    for t in (0, b.T // 2, b.T - 1):
        yt, it, wt = run_block(synth.token_subset(b, [t]))
        assert torch.equal(it[0], idx[t]) and torch.equal(wt[0], w[t])
        assert torch.equal(yt[0], y[t]), f"token {t} differs when run alone"


def test_determinism_bitwise():
    b = synth.make_block(synth.SMALL_SPECS["c3"], DEV)
    announce("determinism c3-small")
    y1, i1, w1 = run_block(b)
    y2, i2, w2 = run_block(b)
    assert torch.equal(y1, y2) and torch.equal(i1, i2) and torch.equal(w1, w2)


def test_bf16_output_is_rounded_f32_output():
    b = synth.make_block(synth.SMALL_SPECS["c2"], DEV)
    announce("bf16 output c2-small")
    y32, _, _ = run_block(b, torch.float32)
    y16, _, _ = run_block(b, torch.bfloat16)
    assert torch.equal(y16, y32.to(torch.bfloat16))


def test_fp16_intermediates_on_bf16_layer():
    """The intermediate storage type is a free choice: fp16 on a bf16 layer."""
    b = synth.make_block(synth.SMALL_SPECS["c3"], DEV)
    announce("fp16 inter c3-small")
    y, idx, w = run_block(b, inter=moe.MOE_F16)
    ob = O.from_block(b)
    gidx, gw, glog = run_route(b)
    routing, _ = check_routing(ob, np32(idx).astype(np.int64), np32(w), np32(glog))
    check_output(np32(y), O.block_forward(ob, routing=routing)["y"], False, "c3-f16")


@pytest.mark.parametrize("group", [32, 128])
def test_affine_group_sizes(group):
    spec = synth.replace(synth.SMALL_SPECS["c2"], group=group, I=256, I_s=256, seed=50 + group)
    b = synth.make_block(spec, DEV)
    _full_check(b, f"affine g{group}")


def test_swiglu_limit_engages():
    """A small clamp limit on the MXFP4 latent layer (reading: both pre-activations
    clamped to [-L, L]) - checked against the oracle's reading; parity unpinned."""
    spec = synth.replace(synth.SMALL_SPECS["c5"], swiglu_limit=0.5, seed=77)
    b = synth.make_block(spec, DEV)
    _full_check(b, "clamp 0.5")


@pytest.mark.parametrize("T", [1, 37, 64])
def test_decode_routing_state_bit_exact(T):
    """T <= 64 routes and permutes in one launch; the counts, offsets, sorted_slot and
    slot_pos it leaves for the experts equal the oracle's permutation bit for bit."""
    b = synth.make_block(synth.FULL_SPECS["c2"], DEV, T=T)
    announce(f"decode routing state c2 T={T}")
    y, idx, w, state = run_block(b, with_state=True)
    check_permutation(idx, b.E, state)
    gidx, gw, glog = run_route(b)
    assert torch.equal(gidx, idx) and torch.equal(gw, w)
    check_routing(O.from_block(b), np32(idx).astype(np.int64), np32(w), np32(glog))


def test_topk_above_16():
    """K > 16 takes the wave-per-token selection kernel (one chosen expert per lane)."""
    spec = synth.replace(synth.SMALL_SPECS["c2"], name="K20", E=64, K=20, T=45, I=128, I_s=128, seed=61)
    _full_check(synth.make_block(spec, DEV), "K=20 of 64")


def test_sigmoid_without_renorm():
    spec = synth.replace(synth.SMALL_SPECS["c2"], name="sig-norenorm", norm_topk=False, seed=62)
    b = synth.make_block(spec, DEV)
    y, idx, w = _full_check(b, "sigmoid, no renorm")[:3]
    assert not torch.allclose(w.sum(1).cpu(), torch.ones(b.T))


@pytest.mark.parametrize("cfg,scale", [("c2", 2.5), ("c4", 0.375)])
def test_routed_scale(cfg, scale):
    """routed_scale multiplies the (renormalised) routing weights."""
    b = synth.make_block(synth.SMALL_SPECS[cfg], DEV)
    b.routed_scale = scale
    y, idx, w = _full_check(b, f"{cfg} routed_scale={scale}")[:3]
    if b.norm_topk:
        assert torch.allclose(w.sum(1).cpu(), torch.full((b.T,), scale), rtol=1e-5)


def test_zero_routed_branch_add():
    """Add mode with the down weights zeroed: y is the shared expert alone."""
    b = synth.make_block(synth.SMALL_SPECS["c4"], DEV)
    b.experts.down.scales = torch.zeros_like(b.experts.down.scales)
    b.experts.down.qbias = torch.zeros_like(b.experts.down.qbias)
    y, idx, w, ob, routing = _full_check(b, "zero-routed c4 (add)")
    out = O.block_forward(ob, routing=routing)
    assert np.array_equal(out["y_routed"], np.zeros_like(out["y_routed"]))
    check_output(np32(y), out["shared"], False, "y == shared")


# ----------------------------------------------------------------------------
# the one-launch decode experts (gate/up + down + combine) against the separate launches
# ----------------------------------------------------------------------------

def _decode_specs():
    c2s = synth.SMALL_SPECS["c2"]
    return {
        "c2-full": (synth.FULL_SPECS["c2"], None),
        "c2-full-T1": (synth.FULL_SPECS["c2"], 1),
        "c2s-blend": (c2s, None),
        "c2s-add": (synth.replace(c2s, name="c2s-add", shared_mode="add", seed=71), None),
        "c2s-none": (synth.replace(c2s, name="c2s-none", shared_mode="none", seed=72), 64),
        "c2s-g128": (synth.replace(c2s, name="c2s-g128", group=128, I=256, I_s=384, seed=73), 29),
        "mxfp4-add": (synth.replace(c2s, name="mxfp4", E=48, K=6, H=1024, I=256, I_s=320, expert_fmt=synth.FMT_MXFP4,
                                    shared_fmt=synth.FMT_MXFP4, group=32, shared_mode="add", swiglu_limit=7.0,
                                    expert_bias=True, seed=74), 24),
    }


def _run_separate(b, y_dtype=torch.float32):
    moe.moe_set_decode_fusion(False)
    try:
        return run_block(b, y_dtype=y_dtype)
    finally:
        moe.moe_set_decode_fusion(True)


@pytest.mark.parametrize("name", list(_decode_specs()))
def test_decode_fused_matches_oracle_and_separate_launches(name):
    """Decode-sized batches run the router, selection and permutation in one launch and
    gate/up and down in one persistent launch by default.  The result matches the oracle
    (C16) and, bit for bit, the separate launches (the same arithmetic in the same order);
    the status word stays 0 (every wait between workgroups completed), also on a second
    call (the counters are left zero)."""
    spec, T = _decode_specs()[name]
    b = synth.make_block(spec, DEV, T=T)
    y, idx, w, ob, routing = _full_check(b, f"fused decode {name}")
    announce(f"status + other modes {name}")
    dev = b.x.device
    ym = torch.empty(b.T, b.H, dtype=torch.float32, device=dev)
    ws = moe.moe_block_forward(b.x, block_desc(b), ym)
    torch.cuda.synchronize()
    assert int(moe.call_status(ws, b.T, b.K, b.E)[0]) == 0
    assert torch.equal(ym, y), "the fused path is not deterministic"
    yu, iu, wu = _run_separate(b)
    assert torch.equal(iu, idx) and torch.equal(wu, w), "routing differs from the separate launches"
    d = (yu - y).abs().max().item()
    assert torch.equal(yu, y), f"decode launches vs separate launches differ: max |diff| {d:.3g}"
    y1, _, _ = run_block(b, y_dtype=torch.bfloat16)
    y0, _, _ = _run_separate(b, torch.bfloat16)
    assert torch.equal(y1, y0), "bf16 output: decode launches vs separate launches differ"


def test_decode_fused_call_sequence():
    """Calls of different sizes and layers in a row on one stream, each bit-identical to the
    separate launches: every call starts from the counters the one before left."""
    c2s = synth.SMALL_SPECS["c2"]
    blocks = [synth.make_block(synth.FULL_SPECS["c2"], DEV),
              synth.make_block(c2s, DEV, T=5),
              synth.make_block(synth.replace(c2s, name="c2s-none", shared_mode="none", seed=72), DEV, T=48),
              synth.make_block(synth.FULL_SPECS["c2"], DEV, T=1)]
    announce("fused call sequence: expected outputs from the separate launches")
    want = [_run_separate(b)[0] for b in blocks]
    for rep in range(2):
        for i, b in enumerate(blocks):
            announce(f"fused call sequence rep {rep} block {i} (T={b.T})")
            y, _, _ = run_block(b)
            torch.cuda.synchronize()
            assert torch.equal(y, want[i]), f"rep {rep} block {i}: one launch differs from separate launches"


def _run_mode(b, mode, y_dtype=torch.float32, with_state=False):
    moe.moe_set_decode_fusion(mode)
    try:
        return run_block(b, y_dtype=y_dtype, with_state=with_state)
    finally:
        moe.moe_set_decode_fusion(moe.DECODE_THREE_LAUNCHES)


def _single_specs():
    c2s = synth.SMALL_SPECS["c2"]
    d = _decode_specs()
    return {
        "c2-full-T1": (synth.FULL_SPECS["c2"], 1),
        "c2-full-T8": (synth.FULL_SPECS["c2"], 8),
        "c2-full-T16": (synth.FULL_SPECS["c2"], 16),
        "c2s-blend-T7": (c2s, 7),
        "c2s-add-T5": (d["c2s-add"][0], 5),
        "c2s-none-T3": (d["c2s-none"][0], 3),
        "c2s-g128-T9": (d["c2s-g128"][0], 9),
        "mxfp4-add-T4": (d["mxfp4-add"][0], 4),
    }


@pytest.mark.parametrize("name", list(_single_specs()))
def test_decode_single_launch(name):
    """The opt-in single launch (up to 16 tokens: router tiles, selection, permutation,
    gate/up, down and the combine of each 32-column block by the wave that completes it)
    matches the oracle (C16), gives the three launches' and the separate launches' bits for
    f32 and bf16 outputs, leaves the oracle's permutation in the workspace and a zero status
    word, and stays bit-identical on a second call (the counter blocks alternate)."""
    spec, T = _single_specs()[name]
    b = synth.make_block(spec, DEV, T=T)
    announce(f"single launch {name}: expected outputs")
    y3, i3, w3 = _run_mode(b, moe.DECODE_THREE_LAUNCHES)
    y0, _, _ = _run_mode(b, moe.DECODE_SEPARATE)
    assert torch.equal(y3, y0)
    yb3, _, _ = _run_mode(b, moe.DECODE_THREE_LAUNCHES, y_dtype=torch.bfloat16)
    moe.moe_set_decode_fusion(moe.DECODE_SINGLE_LAUNCH)
    try:
        y1, i1, w1 = _full_check(b, f"single launch {name}")[:3]
        assert torch.equal(i1, i3) and torch.equal(w1, w3), "routing differs from the three launches"
        d = (y1 - y3).abs().max().item()
        assert torch.equal(y1, y3), f"single launch vs three launches differ: max |diff| {d:.3g}"
        ym = torch.empty(b.T, b.H, dtype=torch.float32, device=b.x.device)
        ws = moe.moe_block_forward(b.x, block_desc(b), ym)
        torch.cuda.synchronize()
        assert int(moe.call_status(ws, b.T, b.K, b.E)[0]) == 0
        assert torch.equal(ym, y1), "second call differs"
        yb1, _, _ = run_block(b, y_dtype=torch.bfloat16)
        assert torch.equal(yb1, yb3), "bf16 output: single launch vs three launches differ"
    finally:
        moe.moe_set_decode_fusion(moe.DECODE_THREE_LAUNCHES)


def test_block_forward_under_graph_capture():
    """A decode block captured in a HIP graph (torch.cuda.graph) takes the separate launches
    (the decode launches keep per-stream counters that a replay elsewhere could share) and
    every replay, with eager calls of the decode launches between replays, equals the eager
    result bit for bit."""
    b = synth.make_block(synth.FULL_SPECS["c2"], DEV)
    desc = block_desc(b)
    announce("graph capture: eager reference")
    y_ref, _, _ = run_block(b)
    y = torch.empty_like(y_ref)
    ws = moe.moe_block_forward(b.x, desc, y)          # the workspace, allocated outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_block_forward(b.x, desc, y, ws=ws)
    for rep in range(3):
        announce(f"graph capture: replay {rep}")
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep} differs from the eager result"
        y_e, _, _ = run_block(b)                          # eager decode launches between replays
        assert torch.equal(y_e, y_ref)


# ----------------------------------------------------------------------------
# the packed weight stream: a pure permutation of the stored planes
# ----------------------------------------------------------------------------

def _pair_order(v):
    """AFFINE4 word, element j in bits 4j..4j+3 -> element 2j at bits 4j, 2j+1 at 16+4j."""
    v = v.astype(np.uint32)
    r = np.zeros_like(v)
    for j in range(4):
        r |= ((v >> np.uint32(8 * j)) & np.uint32(0xF)) << np.uint32(4 * j)
        r |= ((v >> np.uint32(8 * j + 4)) & np.uint32(0xF)) << np.uint32(16 + 4 * j)
    return r


def _expect_packed(lins, gateup: bool, fmt: str, group: int):
    """The stream rebuilt in numpy from the layout stated in include/moe.h / moe_kernels.h:
    per matrix, per 32-row block, per chunk: 4096 bytes of weights (piece (i, lane) at
    i*1024 + lane*16 holds words 4i..4i+3 of the lane's sequence q = (unit*2 + half)*LPU + w)
    followed by the chunk's scales; zero past the rows and columns; AFFINE4 codes in pair
    order (element 2j at bit 4j, element 2j+1 at bit 16+4j)."""
    a = lins[0]
    n, R, K = a.n, a.rows, a.cols
    dense = fmt == synth.FMT_DENSE
    aff = fmt == synth.FMT_AFFINE4
    KC = 64 if dense else 256
    UE = group if aff else (64 if fmt == synth.FMT_MXFP4 else 32)
    QE = UE // 4
    LPU = (2 * QE if dense else QE // 2) // 4
    NU = KC // UE
    SW = (32 * NU) if aff else (64 if fmt == synth.FMT_MXFP4 else 0)   # scale words per record
    nblk = -(-R // 16) if gateup else -(-R // 32)
    nch = -(-K // KC)
    words = [l.w.cpu().contiguous().view(torch.int32).numpy().view(np.uint32).reshape(n, R, -1) for l in lins]
    wpr = words[0].shape[2]
    out = np.zeros((n, nblk, nch, 1024 + SW), dtype=np.uint32)
    lane = np.arange(64)
    n16, kq = lane % 16, lane // 16
    for q in range(16):
        i, j = q // 4, q % 4
        uu, h, wi = q // (2 * LPU), (q // LPU) % 2, q % LPU
        for bk in range(nblk):
            src = words[h] if gateup else words[0]
            row = (16 * bk + n16) if gateup else (32 * bk + 16 * h + n16)
            for c in range(nch):
                e0 = c * KC + uu * UE + kq * QE
                word = (e0 // 2 + wi) if dense else (e0 // 8 + wi)
                ok = (row < R) & (e0 < K)
                vals = np.where(ok[None, :], src[:, np.minimum(row, R - 1), np.minimum(word, wpr - 1)], 0)
                if aff:
                    vals = _pair_order(vals)
                out[:, bk, c, i * 256 + lane * 4 + j] = vals
    if aff:
        G = K // group
        sc = [l.scales.cpu().view(torch.int16).numpy().astype(np.uint16).reshape(n, R, G) for l in lins]
        qb = [l.qbias.cpu().view(torch.int16).numpy().astype(np.uint16).reshape(n, R, G) for l in lins]
        for h in range(2):
            for r16 in range(16):
                for un in range(NU):
                    ent = h * 16 * NU + r16 * NU + un
                    for bk in range(nblk):
                        li = h if gateup else 0
                        row = (16 * bk + r16) if gateup else (32 * bk + 16 * h + r16)
                        for c in range(nch):
                            g = c * KC // group + un
                            if row < R and g < G:
                                out[:, bk, c, 1024 + ent] = (sc[li][:, row, g].astype(np.uint32) |
                                                            (qb[li][:, row, g].astype(np.uint32) << 16))
    elif fmt == synth.FMT_MXFP4:
        NB = K // 32
        e8 = [l.scales.cpu().contiguous().numpy().view(np.uint8).reshape(n, R, NB) for l in lins]
        by = np.zeros((n, nblk, nch, 256), dtype=np.uint32)
        for h in range(2):
            for r16 in range(16):
                for jj in range(8):
                    for bk in range(nblk):
                        li = h if gateup else 0
                        row = (16 * bk + r16) if gateup else (32 * bk + 16 * h + r16)
                        for c in range(nch):
                            g = c * KC // 32 + jj
                            if row < R and g < NB:
                                by[:, bk, c, h * 128 + r16 * 8 + jj] = e8[li][:, row, g]
        b4 = by.reshape(n, nblk, nch, 64, 4)
        out[..., 1024:] = b4[..., 0] | (b4[..., 1] << 8) | (b4[..., 2] << 16) | (b4[..., 3] << 24)
    return out.reshape(-1)


@pytest.mark.parametrize("cfg,which", [("c2", "gateup"), ("c4", "down"), ("c5", "gateup"), ("c5", "latent_down")])
def test_packed_stream_is_the_documented_permutation(cfg, which):
    from synth.descs import linear_desc
    announce(f"packed layout {cfg} {which}")
    b = synth.make_block(synth.SMALL_SPECS[cfg], "cuda:0")
    if which == "gateup":
        lins, gu = [b.experts.gate, b.experts.up], True
        got = moe.moe_pack_weights(linear_desc(lins[0]), linear_desc(lins[1]))
    elif which == "down":
        lins, gu = [b.experts.down], False
        got = moe.moe_pack_weights(linear_desc(lins[0]))
    else:
        lins, gu = [b.latent_down], False
        got = moe.moe_pack_weights(linear_desc(lins[0]))
    torch.cuda.synchronize()
    want = _expect_packed(lins, gu, lins[0].fmt, lins[0].group_size)
    have = got.cpu().numpy().view(np.uint32)
    assert have.shape == want.shape
    assert np.array_equal(have, want)


def _expect_packed_scaled(lins, gateup: bool):
    """The block-scaled MFMA's stream rebuilt in numpy from include/moe.h: per matrix, per
    32-row block, per 256-element record: piece i = 2*stage + half holds at lane l the 16
    stored bytes of tile row (half, l % 16) at elements 128*stage + 32*(l // 16) .. +32, then
    one word per lane whose byte 2*stage + half is the E8M0 scale of those elements; zero
    past the rows and columns."""
    a = lins[0]
    n, R, K = a.n, a.rows, a.cols
    nblk = -(-R // 16) if gateup else -(-R // 32)
    nch = -(-K // 256)
    words = [l.w.cpu().contiguous().numpy().view(np.uint32).reshape(n, R, -1) for l in lins]
    e8 = [l.scales.cpu().contiguous().numpy().view(np.uint8).reshape(n, R, K // 32) for l in lins]
    wpr = words[0].shape[2]
    out = np.zeros((n, nblk, nch, 1024 + 64), dtype=np.uint32)
    lane = np.arange(64)
    n16, kq = lane % 16, lane // 16
    for st in range(2):
        for h in range(2):
            src, sc = (words[h], e8[h]) if gateup else (words[0], e8[0])
            for bk in range(nblk):
                row = (16 * bk + n16) if gateup else (32 * bk + 16 * h + n16)
                for c in range(nch):
                    e0 = c * 256 + 128 * st + 32 * kq
                    ok = (row < R) & (e0 < K)
                    r_ = np.minimum(row, R - 1)
                    for j in range(4):
                        word = np.minimum(e0 // 8 + j, wpr - 1)
                        out[:, bk, c, (2 * st + h) * 256 + lane * 4 + j] = np.where(ok[None, :], src[:, r_, word], 0)
                    g = np.minimum(e0 // 32, K // 32 - 1)
                    byte = np.where(ok[None, :], sc[:, r_, g], 0).astype(np.uint32)
                    out[:, bk, c, 1024 + lane] |= byte << (8 * (2 * st + h))
    return out.reshape(-1)


@pytest.mark.parametrize("which", ["gateup", "down"])
def test_packed_scaled_stream_is_the_documented_permutation(which):
    from synth.descs import linear_desc
    announce(f"scaled packed layout c5 {which}")
    b = synth.make_block(synth.SMALL_SPECS["c5"], "cuda:0")
    if which == "gateup":
        lins, gu = [b.experts.gate, b.experts.up], True
        got = moe.moe_pack_weights(linear_desc(lins[0]), linear_desc(lins[1]), scaled=True)
    else:
        lins, gu = [b.experts.down], False
        got = moe.moe_pack_weights(linear_desc(lins[0]), scaled=True)
    torch.cuda.synchronize()
    want = _expect_packed_scaled(lins, gu)
    have = got.cpu().numpy().view(np.uint32)
    assert have.shape == want.shape
    assert np.array_equal(have, want)


def _scaled_check(b, label, engaged=True):
    """The latent layer with its routed experts on the block-scaled FP4 x FP8 MFMA: routing
    bit-exact as everywhere, outputs against the oracle within the bf16 tolerance."""
    announce(f"{label}: T={b.T} H={b.H} E={b.E} K={b.K} seed={b.seed} (block-scaled MFMA)")
    dev = b.x.device
    y = torch.empty(b.T, b.H, dtype=torch.float32, device=dev)
    idx = torch.empty(b.T, b.K, dtype=torch.int32, device=dev)
    w = torch.empty(b.T, b.K, dtype=torch.float32, device=dev)
    used = moe.moe_block_forward(b.x, block_desc(b, scaled=True), y, idx, w)
    torch.cuda.synchronize()
    state = tuple(t.cpu().numpy().copy() for t in moe.routing_state(used, b.T, b.K, b.E))
    check_permutation(idx, b.E, state)
    y16, idx16, w16 = run_block(b)
    assert torch.equal(idx, idx16) and torch.equal(w, w16), "the selection must not depend on the GEMM path"
    # the two GEMM paths round differently: equal bits mean the scaled path did not run
    assert torch.equal(y, y16) != engaged, "block-scaled path engaged" if not engaged else "block-scaled path not taken"
    ob = O.from_block(b)
    gidx, gw, glog = run_route(b)
    routing, rep = check_routing(ob, np32(idx).astype(np.int64), np32(w), np32(glog))
    ref = O.block_forward(ob, routing=routing)["y"]
    stats = check_output(np32(y), ref, False, label)
    stats16 = check_output(np32(y16), ref, False, label + " (16-bit path)")
    print(f"[ok] {label}: scaled {stats}; 16-bit {stats16}", flush=True)
    return y


_SCALED_SPECS = {
    # several m-tiles per expert and column blocks; widths of 4 and 2 stages per record
    "c5-scaled-a": dict(T=256, D=512, I=256, E=48),
    # ragged m-tiles, an odd number of 128-element stages (3) in both reductions, top-6
    "c5-scaled-b": dict(T=301, D=384, I=384, E=24, K=6, seed=16),
}


@pytest.mark.parametrize("name", list(_SCALED_SPECS))
def test_block_scaled_mfma_small(name):
    from dataclasses import replace
    b = synth.make_block(replace(synth.SMALL_SPECS["c5"], name=name, **_SCALED_SPECS[name]), DEV)
    _scaled_check(b, name)


@pytest.mark.timeout(600)
def test_block_scaled_mfma_full_every_token():
    """The c5 layer at full size on the block-scaled MFMA: every token against the oracle."""
    b = synth.make_block(synth.FULL_SPECS["c5"], DEV)
    _scaled_check(b, "c5-full scaled")


def test_block_scaled_mfma_deterministic_and_fallbacks():
    """Two calls give the same bits; a decode-sized batch, and a layer whose latent width is
    not a whole number of 128-blocks, keep the 16-bit path with the scaled streams attached."""
    from dataclasses import replace
    b = synth.make_block(replace(synth.SMALL_SPECS["c5"], name="c5-scaled-a", **_SCALED_SPECS["c5-scaled-a"]), DEV)
    d = block_desc(b, scaled=True)
    outs = []
    for _ in range(2):
        y = torch.empty(b.T, b.H, dtype=torch.float32, device=DEV)
        moe.moe_block_forward(b.x, d, y)
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    bs = synth.make_block(replace(synth.SMALL_SPECS["c5"], **_SCALED_SPECS["c5-scaled-a"]), DEV, T=3)
    _scaled_check(bs, "c5-scaled-a T=3 (16-bit path)", engaged=False)
    _scaled_check(synth.make_block(synth.SMALL_SPECS["c5"], DEV), "c5-small D=448 (16-bit path)", engaged=False)


def test_block_scaled_mfma_scale_extremes():
    """E8M0 scale bytes 255 (NaN) and 0 in the routed gate weights on the block-scaled MFMA
    path: the NaN reaches the same output rows as on the 16-bit path and in the oracle (the
    split keeps a NaN activation NaN); the other rows match the oracle."""
    from dataclasses import replace
    b = synth.make_block(replace(synth.SMALL_SPECS["c5"], name="c5-scaled-a", **_SCALED_SPECS["c5-scaled-a"]), DEV)
    announce("MXFP4 scale bytes 0 and 255 on the block-scaled MFMA, c5-scaled-a")
    idx, w, _ = run_route(b)
    e_nan, e_tiny = int(idx[0, 0]), int(idx[0, 1])
    sc = b.experts.gate.scales.clone()
    sc[e_nan, 3, 0] = 255
    sc[e_tiny] = 0
    b.experts.gate.scales = sc
    ys = torch.empty(b.T, b.H, dtype=torch.float32, device=DEV)
    moe.moe_block_forward(b.x, block_desc(b, scaled=True), ys)
    y16, _, _ = run_block(b)
    torch.cuda.synchronize()
    ob = O.from_block(b)
    with np.errstate(invalid="ignore"):
        ref = O.block_forward(ob)["y"]
    got, got16 = np32(ys), np32(y16)
    nan_ref, nan_got, nan16 = np.isnan(ref).any(axis=1), np.isnan(got).any(axis=1), np.isnan(got16).any(axis=1)
    assert nan_ref[0] and (nan_got == nan_ref).all() and (nan16 == nan_ref).all(), "NaN rows differ"
    check_output(got[~nan_ref], ref[~nan_ref], False, "scaled-mfma-scale-extremes")
