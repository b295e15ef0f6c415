"""Pins of the oracle to facts outside itself (CPU only).

Each test ties a part of the oracle to something the pages or mathematics fix:
the page-4 worked example (ferrox-models latent_moe.rs tests), the blend and
selection-bias contracts of mlxcel PR #1044, closed forms, exhaustive
enumeration on tiny inputs, the OCP MX encoding tables, and library routines.
Mutation tests plant plausible mistakes in the oracle and check that a pin
catches each one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "latent_moe_page4.json")


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def dense(*mats):
    return O.OLinear("dense", np.stack([np.asarray(m, dtype=np.float64) for m in mats]))


def golden_block(with_norm=True):
    g = json.load(open(GOLDEN))
    H, D, E, I, Is = g["hidden"], g["latent"], g["experts"], g["intermediate"], g["shared_intermediate"]
    M = lambda v, r, c: np.asarray(v, dtype=np.float64).reshape(r, c)
    ex = O.OMLP(dense(*[M(e["w1_gate"], I, D) for e in g["experts_w"]]),
                dense(*[M(e["w3_up"], I, D) for e in g["experts_w"]]),
                dense(*[M(e["w2_down"], D, I) for e in g["experts_w"]]))
    sh = O.OMLP(dense(M(g["shared"]["w1_gate"], Is, H)), dense(M(g["shared"]["w3_up"], Is, H)),
                dense(M(g["shared"]["w2_down"], H, Is)))
    b = O.OBlock(x=np.asarray([g["input"]]), router_w=M(g["router_weight"], E, H), scoring="sigmoid",
                 K=g["top_k"], norm_topk=g["renormalize"], routed_scale=g["routed_scaling_factor"], experts=ex,
                 select_bias=np.asarray(g["e_score_correction_bias"]), shared=sh, shared_mode="add",
                 latent_down=dense(M(g["down_proj"], D, H)), latent_up=dense(M(g["up_proj"], H, D)),
                 latent_norm_w=np.asarray(g["routed_norm_weight"]) if with_norm else None,
                 norm_eps=g["norm_eps"])
    return b, np.asarray(g["golden_out"]), g["tolerance_abs"]


def golden_error():
    b, ref, _ = golden_block()
    return float(np.max(np.abs(O.block_forward(b)["y"][0] - ref)))


def rand_block(rng, T=5, H=12, E=6, K=2, I=7, scoring="sigmoid", norm=True, sbias=True, lbias=False,
               shared_mode="blend", latent=0, limit=0.0, Is=5):
    D = latent or H
    r = lambda *s: rng.standard_normal(s)
    ex = O.OMLP(dense(*[0.5 * r(I, D) for _ in range(E)]), dense(*[0.5 * r(I, D) for _ in range(E)]),
                dense(*[0.5 * r(D, I) for _ in range(E)]), limit)
    sh = None
    if shared_mode != "none":
        sh = O.OMLP(dense(0.5 * r(Is, H)), dense(0.5 * r(Is, H)), dense(0.5 * r(H, Is)))
    return O.OBlock(
        x=r(T, H), router_w=r(E, H) / math.sqrt(H), scoring=scoring, K=K, norm_topk=norm, routed_scale=1.0,
        experts=ex, logit_bias=r(E) if lbias else None, select_bias=0.3 * r(E) if sbias else None, shared=sh,
        shared_mode=shared_mode, coef_w=0.3 * r(2, H) if shared_mode == "blend" else None,
        coef_b=0.3 * r(2) if shared_mode == "blend" else None,
        latent_down=dense(0.3 * r(D, H)) if latent else None, latent_up=dense(0.3 * r(H, D)) if latent else None,
        latent_norm_w=1 + 0.1 * r(D) if latent else None)


# ----------------------------------------------------------------------------
# P1: the page-4 worked example
# ----------------------------------------------------------------------------

def test_golden_latent_moe_page4():
    """ferrox-models latent_moe.rs, test matches_independent_python_reference:
    six outputs within 1e-3 of the printed golden values (SwiGLU stands in for
    situ, whose definition is not on the pages)."""
    b, ref, tol = golden_block()
    y = O.block_forward(b)["y"][0]
    assert np.all(np.abs(y - ref) < tol), (y, ref)
    # the per-token literal flow gives the same numbers
    assert np.allclose(O.block_forward_loop(b)[0], y, rtol=0, atol=1e-14)


def test_golden_without_routed_norm_differs():
    """latent_moe.rs, test without_routed_norm_output_still_finite_and_differs."""
    b, ref, _ = golden_block(with_norm=False)
    y = O.block_forward(b)["y"][0]
    assert np.all(np.isfinite(y))
    assert abs(y[0] - ref[0]) > 1e-6


def _wrong_route_biased_weights(x, router_w, scoring, K, norm_topk, routed_scale=1.0, logit_bias=None,
                                select_bias=None, logits=None):
    r = ORIG_ROUTE(x, router_w, scoring, K, norm_topk, routed_scale, logit_bias, select_bias, logits)
    w = np.take_along_axis(r["sel"], r["idx"].astype(np.int64), axis=1)
    r["w"] = w / w.sum(axis=1, keepdims=True) if norm_topk else w
    return r


ORIG_ROUTE = O.route

MUTANTS = {
    # weights gathered from the biased selection keys instead of the unbiased scores
    "weights_from_biased_scores": ("route", _wrong_route_biased_weights),
    # the selection bias ignored
    "no_selection_bias": ("route", lambda x, rw, sc, K, nt, rs=1.0, lb=None, sb=None, logits=None:
                          ORIG_ROUTE(x, rw, sc, K, nt, rs, lb, None, logits)),
    # renormalisation skipped
    "no_renorm": ("route", lambda x, rw, sc, K, nt, rs=1.0, lb=None, sb=None, logits=None:
                  ORIG_ROUTE(x, rw, sc, K, False, rs, lb, sb, logits)),
    # gate and up exchanged inside SwiGLU
    "gate_up_swapped": ("swiglu", lambda g, u, limit=0.0: O.silu(u) * g),
    # eps outside the square root
    "eps_outside_sqrt": ("rms_norm", lambda v, w, eps: v / (np.sqrt(np.mean(v * v, -1, keepdims=True)) + eps)
                         * O.as_f64(w)),
    # norm weight dropped
    "no_norm_weight": ("rms_norm", lambda v, w, eps: v / np.sqrt(np.mean(v * v, -1, keepdims=True) + eps)),
    # the weights applied transposed
    "transposed_apply": ("apply_linear", None),
    # softmax instead of sigmoid scores
    "softmax_scores": ("scores_from_logits", lambda l, scoring: O.softmax(l, axis=-1)),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_golden_catches_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    if name == "transposed_apply":
        def fn(lin, e, z):
            m = lin.matrix(e)
            if m.shape[0] == m.shape[1]:
                m = m.T
            else:  # square-free weights: reshape the stored buffer the other way round
                m = m.reshape(m.shape[1], m.shape[0]).T.reshape(m.shape)
            return z @ m.T
    monkeypatch.setattr(O, attr, fn)
    err = golden_error()
    assert err > 1e-3, f"mutant {name} still matches the golden vector (err {err})"


# ----------------------------------------------------------------------------
# stored-format decoding
# ----------------------------------------------------------------------------

def test_e2m1_table():
    """OCP MX v1.0 FP4 E2M1 value table (codes 0..7 positive, 8..15 negative)."""
    table = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    got = O.e2m1_decode(np.arange(16))
    assert list(got[:8]) == table
    assert list(-got[8:]) == table
    assert np.signbit(got[8])  # code 8 is -0


def test_e8m0_values():
    v = O.e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255]))
    assert v[0] == 2.0 ** -127 and v[1] == 2.0 ** -126 and v[2] == 0.5 and v[3] == 1.0 and v[4] == 2.0
    assert v[5] == 2.0 ** 127 and np.isnan(v[6])


def test_nibble_unpack_against_python_ints():
    rng = np.random.default_rng(0)
    words = rng.integers(0, 2 ** 32, size=(3, 5), dtype=np.uint64).astype(np.uint32)
    q = O.unpack_nibbles_u32(words)
    for r in range(3):
        for j in range(5):
            w = int(words[r, j])
            for i in range(8):
                assert q[r, 8 * j + i] == (w // 16 ** i) % 16


def test_bf16_decode_against_torch():
    x = torch.randn(1000, dtype=torch.float32) * 10
    xb = x.to(torch.bfloat16)
    assert np.array_equal(O.bf16_to_f64(synth.raw(xb)), xb.double().numpy())


@pytest.mark.parametrize("group", [32, 64, 128])
def test_affine4_roundtrip(group):
    """Encoder (torch, synth) and decoder (numpy, oracle) are separate code: every
    decoded weight is scale*q + qbias with q in 0..15 and lies within half a
    quantisation step of the original."""
    g = torch.Generator().manual_seed(group)
    w = torch.randn(3, 16, 256, generator=g) * 0.02
    words, sc, qb = synth.encode_affine4(w, group)
    deq = O.dequant_affine4(synth.raw(words), synth.raw(sc), synth.raw(qb), group)
    s = O.bf16_to_f64(synth.raw(sc))
    b = O.bf16_to_f64(synth.raw(qb))
    srep = np.repeat(s, group, axis=-1)
    brep = np.repeat(b, group, axis=-1)
    q = (deq - brep) / srep
    assert np.allclose(q, np.round(q), atol=1e-9) and q.min() >= -1e-9 and q.max() <= 15 + 1e-9
    # within half a step plus the bf16 rounding of scale and qbias
    slack = srep * 0.5 + np.abs(brep) * 2 ** -8 + srep * 15 * 2 ** -8
    assert np.all(np.abs(deq - w.double().numpy()) <= slack + 1e-12)


def test_mxfp4_roundtrip():
    g = torch.Generator().manual_seed(7)
    w = torch.randn(2, 8, 128, generator=g) * 0.02
    w[0, 0, :32] = 0.0                       # an all-zero block
    codes, e8 = synth.encode_mxfp4(w)
    deq = O.dequant_mxfp4(synth.raw(codes), synth.raw(e8))
    assert np.all(deq[0, 0, :32] == 0)
    scale = np.repeat(O.e8m0_decode(synth.raw(e8)), 32, axis=-1)
    # every value lies on the E2M1 grid times its block scale
    grid = set([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    assert set(np.unique(np.abs(deq / scale))).issubset(grid)
    # nearest grid point (below saturation: largest element of a block may clip at 6*scale)
    err = np.abs(deq - w.double().numpy())
    below = np.abs(w.double().numpy()) <= 6 * scale
    assert np.all(err[below] <= 0.5 * scale[below] * 2 + 1e-15)   # grid spacing <= 2 in scaled units
    assert np.all(np.abs(deq) <= 6 * scale)


def test_mxfp4_known_bytes():
    """Hand-built bytes: low nibble = even element; code 0x3 = 1.5, 0xA = -1.0."""
    blocks = np.zeros((1, 16), dtype=np.uint8)
    blocks[0, 0] = 0xA3          # elements 0 -> 1.5, 1 -> -1.0
    scales = np.array([[128]], dtype=np.uint8)  # 2.0
    v = O.dequant_mxfp4(blocks, scales)
    assert v[0, 0] == 3.0 and v[0, 1] == -2.0 and np.all(v[0, 2:] == 0)


# ----------------------------------------------------------------------------
# routing
# ----------------------------------------------------------------------------

def test_all_equal_scores_pick_lowest_ids():
    """W_r = 0 and no biases: every score is equal, the tie rule picks experts
    0..K-1 and renormalised weights are 1/K (sigmoid(0) = 1/2 before)."""
    x = np.ones((3, 4))
    for scoring in ("sigmoid", "softmax"):
        r = O.route(x, np.zeros((7, 4)), scoring, 3, True)
        assert (r["idx"] == np.arange(3)).all()
        assert np.allclose(r["w"], 1 / 3, rtol=0, atol=1e-15)
    r = O.route(x, np.zeros((7, 4)), "sigmoid", 3, False)
    assert np.all(r["w"] == 0.5)
    r = O.route(x, np.zeros((7, 4)), "softmax", 3, False)
    assert np.allclose(r["w"], 1 / 7, rtol=0, atol=1e-15)


def test_selection_bias_moves_selection_not_weights():
    """mlxcel PR #1044 point 3: bias on a copy used for selection, weights from the
    unbiased scores.  Expert 0 has the largest score but a bias pushes it out."""
    logits = np.array([[3.0, 1.0, 0.5, 0.0, -1.0]])
    bias = np.array([-10.0, 0.0, 0.0, 0.0, 0.0])
    r = O.route(None, None, "sigmoid", 2, True, select_bias=bias, logits=logits)
    assert list(r["idx"][0]) == [1, 2]
    s = 1 / (1 + np.exp(-np.array([1.0, 0.5])))
    assert np.allclose(r["w"][0], s / s.sum(), rtol=1e-15)
    assert not np.allclose(r["w"][0], (s - 10) / (s - 10).sum())
    # a positive bias pulls in the smallest-score expert; its weight is its own score
    bias2 = np.array([0.0, 0.0, 0.0, 0.0, 5.0])
    r2 = O.route(None, None, "sigmoid", 2, False, select_bias=bias2, logits=logits)
    assert list(r2["idx"][0]) == [0, 4]
    assert math.isclose(r2["w"][0, 1], 1 / (1 + math.exp(1.0)), rel_tol=1e-15)


def test_logit_offset_moves_weights_too():
    logits = np.array([[0.0, 0.0, 0.0]])
    r = O.route(None, None, "sigmoid", 1, False, logits=logits + np.array([0.0, 2.0, 0.0]))
    assert r["idx"][0, 0] == 1 and math.isclose(r["w"][0, 0], 1 / (1 + math.exp(-2.0)), rel_tol=1e-15)


def test_sigmoid_softmax_closed_forms():
    l = np.array([[0.0, math.log(3.0)]])
    assert np.allclose(O.scores_from_logits(l, "sigmoid"), [[0.5, 0.75]], rtol=1e-15)
    assert np.allclose(O.scores_from_logits(l, "softmax"), [[0.25, 0.75]], rtol=1e-15)


@pytest.mark.parametrize("seed", range(6))
def test_selection_brute_force(seed):
    """The chosen set is the unique K-subset whose smallest key exceeds every key
    outside it (found by enumerating all subsets)."""
    rng = np.random.default_rng(seed)
    E, K = 8, 3
    b = rand_block(rng, T=6, E=E, K=K, lbias=True)
    r = O.route(b.x, b.router_w, b.scoring, K, True, 1.0, b.logit_bias, b.select_bias)
    for t in range(6):
        sel = r["sel"][t]
        good = [S for S in itertools.combinations(range(E), K)
                if min(sel[list(S)]) > max(sel[[e for e in range(E) if e not in S]])]
        assert len(good) == 1 and list(good[0]) == list(r["idx"][t])
        assert O.topk_margin(r["sel"][t:t + 1], K)[0] == pytest.approx(
            min(sel[list(good[0])]) - max(sel[[e for e in range(E) if e not in good[0]]]), rel=1e-12)


def test_block_brute_force_sum_over_chosen_experts():
    """y equals the plain sum over the enumerated chosen set of w_e * expert_e(x)
    plus the blended shared branch, computed with library SiLU (torch)."""
    rng = np.random.default_rng(11)
    b = rand_block(rng, T=4, E=6, K=2)
    y = O.block_forward(b)["y"]
    tt = lambda a: torch.tensor(a, dtype=torch.float64)
    for t in range(4):
        x = tt(b.x[t])
        logits = tt(b.router_w) @ x
        s = torch.sigmoid(logits)
        sel = s + tt(b.select_bias)
        best = max(itertools.combinations(range(6), 2), key=lambda S: float(sel[list(S)].sum()))
        w = s[list(best)] / s[list(best)].sum()

        def mlp(m, e, v):
            g = tt(m.gate.matrix(e)) @ v
            u = tt(m.up.matrix(e)) @ v
            return tt(m.down.matrix(e)) @ (torch.nn.functional.silu(g) * u)

        yr = sum(w[i] * mlp(b.experts, e, x) for i, e in enumerate(best))
        sh = mlp(b.shared, 0, x)
        c = torch.softmax(tt(b.coef_w) @ x + tt(b.coef_b), dim=0)
        ref = c[0] * yr + c[1] * sh
        assert np.allclose(y[t], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_topk_equals_expert_count_is_dense_mixture():
    """Softmax scores with K = E: the block is the dense mixture
    sum_e softmax_e(x) * expert_e(x), with or without renormalisation."""
    rng = np.random.default_rng(3)
    for norm in (False, True):
        b = rand_block(rng, T=5, E=5, K=5, scoring="softmax", norm=norm, sbias=False, shared_mode="none")
        y = O.block_forward(b)["y"]
        l = b.x @ b.router_w.T
        p = np.exp(l - l.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        ref = np.zeros_like(y)
        for e in range(5):
            g = b.x @ b.experts.gate.matrix(e).T
            u = b.x @ b.experts.up.matrix(e).T
            h = g / (1 + np.exp(-g)) * u
            ref += p[:, e:e + 1] * (h @ b.experts.down.matrix(e).T)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# shared expert: add vs blend (mlxcel PR #1044 point 2)
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("mode", ["blend", "add"])
def test_zero_routed_branch(mode):
    """Routed branch zeroed (down weights 0): blend gives exactly coef[1]*shared,
    add gives exactly shared."""
    rng = np.random.default_rng(5)
    b = rand_block(rng, shared_mode=mode)
    b.experts.down = O.OLinear("dense", np.zeros_like(b.experts.down.w))
    out = O.block_forward(b)
    s = out["shared"]
    if mode == "blend":
        c = O.coef_head(b.x, b.coef_w, b.coef_b)
        assert np.array_equal(out["y"], c[:, 1:] * s + c[:, :1] * 0.0)
        assert not np.allclose(out["y"], s)
    else:
        assert np.array_equal(out["y"], s)


def test_zero_routed_branch_quantized():
    """Same with a 4-bit affine down plane whose scales and qbias are 0."""
    spec = synth.SMALL_SPECS["c2"]
    blk = synth.make_block(spec, "cpu")
    ob = O.from_block(blk)
    shape = tuple(blk.experts.down.scales.shape)
    ob.experts.down = O.OLinear("affine4", ob.experts.down.w, np.zeros(shape, np.uint16),
                                np.zeros(shape, np.uint16), None, spec.group)
    out = O.block_forward(ob)
    c = out["coef"]
    assert np.array_equal(out["y"], c[:, 1:] * out["shared"] + c[:, :1] * 0.0)


def test_coefficient_index_one_weights_shared():
    """Sweeping the coefficient bias towards index 1 moves y to the shared output;
    towards index 0, to the routed mixture."""
    rng = np.random.default_rng(8)
    b = rand_block(rng)
    b.coef_w = np.zeros_like(b.coef_w)
    b.coef_b = np.array([0.0, 40.0])
    out = O.block_forward(b)
    assert np.allclose(out["y"], out["shared"], rtol=1e-12, atol=1e-12)
    b.coef_b = np.array([40.0, 0.0])
    out = O.block_forward(b)
    assert np.allclose(out["y"], out["y_routed"], rtol=1e-12, atol=1e-12)
    b.coef_b = np.array([0.0, 0.0])
    out = O.block_forward(b)
    assert np.allclose(out["y"], 0.5 * out["y_routed"] + 0.5 * out["shared"], rtol=1e-14)


# ----------------------------------------------------------------------------
# permutation, invariances, reductions
# ----------------------------------------------------------------------------

def test_permutation_matches_stable_argsort():
    rng = np.random.default_rng(2)
    E, K, T = 9, 3, 40
    idx = np.stack([np.sort(rng.choice(E, K, replace=False)) for _ in range(T)]).astype(np.int32)
    counts, offsets, ss, sp = O.permute(idx, E)
    flat = idx.reshape(-1)
    assert counts.sum() == T * K and np.all(np.diff(offsets) >= 0) and offsets[-1] == T * K
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert np.array_equal(ss, np.argsort(flat, kind="stable"))
    assert np.array_equal(sp[ss], np.arange(T * K))


def test_vectorised_equals_per_token_loop():
    rng = np.random.default_rng(4)
    for kw in (dict(), dict(scoring="softmax", norm=False, sbias=False, shared_mode="add"),
               dict(latent=5, shared_mode="add", limit=0.7), dict(shared_mode="none", lbias=True)):
        b = rand_block(rng, T=6, **kw)
        assert np.allclose(O.block_forward(b)["y"], O.block_forward_loop(b), rtol=1e-13, atol=1e-14)


def test_batch_invariance():
    """A token's output does not depend on the other tokens (mlxcel PR #1044,
    the causality check in "Validation")."""
    rng = np.random.default_rng(6)
    b = rand_block(rng, T=7, latent=4, shared_mode="add")
    y = O.block_forward(b)["y"]
    for t in (0, 3, 6):
        bt = O.OBlock(**{**b.__dict__, "x": b.x[t:t + 1]})
        assert np.allclose(O.block_forward(bt)["y"][0], y[t], rtol=1e-14, atol=1e-15)


def test_single_expert_reduces_to_swiglu_mlp():
    """E = K = 1, no shared: the block is one SwiGLU MLP (checked against torch's
    SiLU and matmul in float64)."""
    rng = np.random.default_rng(9)
    b = rand_block(rng, E=1, K=1, shared_mode="none")
    y = O.block_forward(b)["y"]
    x = torch.tensor(b.x)
    g = x @ torch.tensor(b.experts.gate.matrix(0)).T
    u = x @ torch.tensor(b.experts.up.matrix(0)).T
    ref = (torch.nn.functional.silu(g) * u) @ torch.tensor(b.experts.down.matrix(0)).T
    assert np.allclose(y, ref.numpy(), rtol=1e-13, atol=1e-14)


def test_rms_norm_closed_form():
    v = np.full((1, 8), 3.0)
    w = np.arange(1, 9, dtype=np.float64)
    assert np.allclose(O.rms_norm(v, w, 1e-5), 3.0 / math.sqrt(9.0 + 1e-5) * w, rtol=1e-15)
    v2 = np.array([[3.0, -4.0]])      # mean square 12.5
    assert np.allclose(O.rms_norm(v2, np.ones(2), 0.0), v2 / math.sqrt(12.5), rtol=1e-15)


def test_clamp_properties():
    """Clamped SwiGLU (reading: both pre-activations limited to [-L, L]).  Parity
    unpinned; only its own properties are checked: a huge limit is the plain
    SwiGLU and the output is bounded by silu(L)*L."""
    rng = np.random.default_rng(1)
    g, u = 5 * rng.standard_normal(1000), 5 * rng.standard_normal(1000)
    assert np.array_equal(O.swiglu(g, u, 1e9), O.silu(g) * u)
    L = 2.0
    h = O.swiglu(g, u, L)
    assert np.all(np.abs(h) <= L / (1 + math.exp(-L)) * L + 1e-12)
    inside = (np.abs(g) <= L) & (np.abs(u) <= L)
    assert np.array_equal(h[inside], (O.silu(g) * u)[inside])


# ----------------------------------------------------------------------------
# generated layers: structure of the five workloads
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c4", "c5"])
def test_small_layers_run_and_loop_agrees(cfg):
    spec = synth.SMALL_SPECS[cfg]
    blk = synth.make_block(spec, "cpu")
    ob = O.from_block(blk)
    out = O.block_forward(ob)
    y = out["y"]
    assert y.shape == (spec.T, spec.H) and np.all(np.isfinite(y))
    r = out["routing"]
    assert r["idx"].shape == (spec.T, spec.K)
    assert np.all(np.diff(r["idx"], axis=1) > 0)
    if spec.norm_topk:
        assert np.allclose(r["w"].sum(1), 1.0, rtol=1e-14)
    # a few tokens through the literal per-token loop
    sub = O.OBlock(**{**ob.__dict__, "x": np.asarray(ob.x)[:3]})
    assert np.allclose(O.block_forward_loop(sub), y[:3], rtol=1e-12, atol=1e-13)


def test_c1_brute_force_selection():
    """Workload 1 (4 tokens, 8 experts, top-2): all 28 subsets enumerated."""
    blk = synth.make_block(synth.FULL_SPECS["c1"], "cpu")
    ob = O.from_block(blk)
    r = O.block_forward(ob)["routing"]
    for t in range(4):
        sel = r["sel"][t]
        good = [S for S in itertools.combinations(range(8), 2)
                if min(sel[list(S)]) > max(sel[[e for e in range(8) if e not in S]])]
        assert len(good) == 1 and list(good[0]) == list(r["idx"][t])
