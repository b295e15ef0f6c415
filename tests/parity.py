"""Shared helpers of the GPU parity tests: run the library, compare with the oracle.

Routing comparison (expert indices are integers decided by floating point):
  (i)  the GPU's chosen set must equal, on every token, the selection the
       oracle recomputes in float64 from the GPU's own fp32 logits; a token may
       differ only when its K-th/(K+1)-th keys recomputed that way are closer
       than TIE_EPS (an arithmetic tie of the fp32 scores) and such tokens are
       counted;
  (ii) against the oracle's own float64 logits the sets must be equal on every
       token whose top-k margin exceeds DELTA; tokens at or below DELTA are
       near-ties, where the GPU's set only has to be a valid top-k up to DELTA.
Output comparison uses the oracle's float64 weights on the GPU's selection.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
import synth
import sparse_mixture_experts_bias_amd as moe
from synth.descs import block_desc, router_desc

TIE_EPS = 2.0 ** -22
DELTA = 1e-5
TOL_F32 = 1e-5           # normwise, f32 layer
TOL_BF16 = 2e-2          # normwise, bf16 activations
MAE_BF16 = 2e-3          # mean absolute error, bf16 activations


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def run_block(b: synth.Block, y_dtype=torch.float32, inter=None, ws=None, with_state=False):
    """One moe_block_forward; with_state also returns the routing state the experts
    ran on (counts, offsets, sorted_slot, slot_pos, read back from the workspace)."""
    dev = b.x.device
    y = torch.empty(b.T, b.H, dtype=y_dtype, device=dev)
    idx = torch.empty(b.T, b.K, dtype=torch.int32, device=dev)
    w = torch.empty(b.T, b.K, dtype=torch.float32, device=dev)
    used = moe.moe_block_forward(b.x, block_desc(b, inter), y, idx, w, ws=ws)
    torch.cuda.synchronize()
    if with_state:
        state = tuple(t.cpu().numpy().copy() for t in moe.routing_state(used, b.T, b.K, b.E))
        return y, idx, w, state
    return y, idx, w


def check_permutation(idx: torch.Tensor, E: int, state):
    """The routing state (counts, offsets, sorted_slot, slot_pos) equals the oracle's
    permutation of the selection bit for bit."""
    c, o, s, p = O.permute(idx.cpu().numpy().astype(np.int64), E)
    names = ("counts", "offsets", "sorted_slot", "slot_pos")
    for name, got, want in zip(names, state, (c, o, s, p)):
        assert np.array_equal(got.astype(np.int64), want), f"{name} differs from the oracle's permutation"


def run_route(b: synth.Block):
    dev = b.x.device
    idx = torch.empty(b.T, b.K, dtype=torch.int32, device=dev)
    w = torch.empty(b.T, b.K, dtype=torch.float32, device=dev)
    logits = torch.empty(b.T, b.E, dtype=torch.float32, device=dev)
    moe.moe_route(b.x, router_desc(b), idx, w, logits)
    torch.cuda.synchronize()
    return idx, w, logits


def check_routing(ob: O.OBlock, gidx: np.ndarray, gw: np.ndarray, glogits: np.ndarray, w_tol=(1e-4, 1e-5)):
    """Applies rules (i) and (ii); returns (routing for the output comparison, report)."""
    K = ob.K
    gidx = gidx.astype(np.int64)
    # (i) selection from the GPU's logits, float64
    rg = O.route(None, None, ob.scoring, K, ob.norm_topk, ob.routed_scale, None, ob.select_bias,
                 logits=glogits.astype(np.float64))
    diff_i = np.nonzero((rg["idx"] != gidx).any(axis=1))[0]
    ties = 0
    for t in diff_i:
        m = O.topk_margin(rg["sel"][t:t + 1], K)[0]
        assert m < TIE_EPS, f"token {t}: GPU set {gidx[t]} != set {rg['idx'][t]} from its own logits (margin {m:.3g})"
        ties += 1
    # (ii) against the oracle's float64 logits
    ro = O.route(ob.x, ob.router_w, ob.scoring, K, ob.norm_topk, ob.routed_scale, ob.logit_bias, ob.select_bias)
    margin = O.topk_margin(ro["sel"], K)
    decided = margin > DELTA
    bad = np.nonzero(decided & (ro["idx"] != gidx).any(axis=1))[0]
    assert bad.size == 0, f"tokens {bad[:10]} choose differently with margin > {DELTA}"
    near = np.nonzero(~decided)[0]
    for t in near:
        sel = ro["sel"][t]
        chosen = np.zeros(sel.shape[0], bool)
        chosen[gidx[t]] = True
        if (~chosen).any():
            assert sel[chosen].min() >= sel[~chosen].max() - DELTA, f"token {t}: GPU set is not a top-{K} within DELTA"
    # weights: float64 weights of the GPU's selection
    w_ref = O.weights_for(ro["scores"], gidx, ob.norm_topk, ob.routed_scale)
    rtol, atol = w_tol
    assert np.allclose(gw, w_ref, rtol=rtol, atol=atol), f"weights differ: max {np.abs(gw - w_ref).max():.3g}"
    routing = dict(ro)
    routing["idx"] = gidx
    routing["w"] = w_ref
    return routing, {"arith_ties": ties, "near_ties": int(near.size), "min_margin": float(margin.min())}


def check_output(got: np.ndarray, ref: np.ndarray, f32: bool, label: str = ""):
    d = np.abs(got.astype(np.float64) - ref)
    normwise = d.max() / max(np.abs(ref).max(), 1e-30)
    mae = d.mean()
    if f32:
        assert normwise <= TOL_F32, f"{label}: normwise {normwise:.3g} > {TOL_F32}"
    else:
        assert normwise <= TOL_BF16, f"{label}: normwise {normwise:.3g} > {TOL_BF16}"
        assert mae < MAE_BF16, f"{label}: mean abs error {mae:.3g} >= {MAE_BF16}"
    return {"normwise": float(normwise), "mae": float(mae)}
