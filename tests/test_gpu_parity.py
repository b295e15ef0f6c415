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

from parity import check_output, check_routing, np32, run_block, run_route

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
    y, idx, w = run_block(b, y_dtype)
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


@pytest.mark.parametrize("cfg,nsample", [("c3", 16), ("c4", 16), ("c5", 6)])
def test_block_full_sampled(cfg, nsample):
    """Full-size layers in the launch configuration of the benchmark; routing and
    permutation checked on every token, outputs on a sample of tokens."""
    spec = synth.FULL_SPECS[cfg]
    b = synth.make_block(spec, DEV)
    announce(f"{cfg}-full: T={b.T} H={b.H} E={b.E} K={b.K} seed={b.seed}")
    y, idx, w = run_block(b)
    gidx, gw, glog = run_route(b)
    assert torch.equal(gidx, idx) and torch.equal(gw, w)
    # routing on every token
    from synth import raw
    ob_all = O.OBlock(x=raw(b.x), router_w=raw(b.router_w), scoring=b.scoring, K=b.K, norm_topk=b.norm_topk,
                      routed_scale=b.routed_scale, experts=None, logit_bias=raw(b.logit_bias),
                      select_bias=raw(b.select_bias))
    routing, rep = check_routing(ob_all, np32(idx).astype(np.int64), np32(w), np32(glog))
    print(f"[routing] {cfg}-full {rep}", flush=True)
    # permutation on every token
    _check_permute(idx, b.E)
    # outputs on sampled tokens
    g = torch.Generator().manual_seed(1234)
    toks = torch.randperm(b.T, generator=g)[:nsample].sort().values.tolist()
    sub = synth.token_subset(b, toks)
    ob = O.from_block(sub)
    r_sub = {k: (v[toks] if isinstance(v, np.ndarray) and v.ndim >= 1 and v.shape[0] == b.T else v)
             for k, v in routing.items()}
    ref = O.block_forward(ob, routing=r_sub)["y"]
    stats = check_output(np32(y)[toks], ref, False, f"{cfg}-full")
    print(f"[ok] {cfg}-full sampled {toks}: {stats}", flush=True)


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
