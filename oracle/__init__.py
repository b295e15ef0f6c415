"""Double-precision CPU oracle for the sparse MoE FFN block (test infrastructure).

This package is test infrastructure.  Only the test suite, the smoke check of
the package entry point and the CPU-baseline leg of the benchmark may import
it; the GPU library never does, and it shares no code with the GPU library.

It computes, plainly and slowly, in float64 NumPy, what the pages define:

  * router projection and sigmoid/softmax scoring, a per-expert bias used for
    selection only, top-k, optional renormalisation (mlxcel PR #1044, point 3:
    the routing uses sigmoid scores and applies no routed scaling factor;
    ferrox-models latent_moe.rs, kimi_latent_moe_forward and its
    route_top_k_sigmoid_with_bias call);
  * the per-expert SwiGLU MLP with w1 = gate, w3 = up, w2 = down
    (latent_moe.rs, KimiExpertWeights::forward; SwitchGLU in mlx-swift-lm
    PR #364 and mlxcel issue #974), optionally clamped (libmir-metal
    clamped_routed/experts/mod.rs, the swiglu_limit passed to the gate/up
    kernel);
  * stored weights decoded exactly: 4-bit affine groups (mlxcel issue #974,
    the gather_qmm "affine" plane with weight/scales/biases) and MXFP4 blocks
    (libmir-metal ExpertLayout::Native/Mlx; E2M1 and E8M0 from the OCP
    Microscaling Formats specification v1.0);
  * the weighted combine, the latent variant (down_proj -> experts in latent
    space -> weighted sum -> RMSNorm -> up_proj, latent_moe.rs module doc) and
    the shared expert, added at weight 1 or mixed with the routed sum through
    a per-token 2-way softmax coefficient head (mlxcel PR #1044, point 2: the
    two branches are weighted by that head's coefficients rather than summed).

Readings where the pages are silent (each one is listed with its reason in
the design notes): selection ties go to the lowest expert index; the K slots
of a token are reported in ascending expert order; the bias for selection is
added to the post-activation scores; renormalisation divides by the sum of
the K gathered weights, before routed_scale; the clamp limits both the gate
and the up pre-activation to [-L, L] (parity unpinned: no page gives the
formula or a worked example); RMSNorm is v / sqrt(mean(v^2) + eps) * w.

Nothing here rounds an intermediate.  Intermediates are float64 throughout.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

# ----------------------------------------------------------------------------
# exact decoding of the stored formats
# ----------------------------------------------------------------------------


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64.  bf16 is the top half of an IEEE
    binary32, so widening the bits to 32 and reading them as float32 is exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def as_f64(a) -> np.ndarray:
    """Stored dense values (float32/float64 numbers or bf16 bits) -> float64."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


def unpack_nibbles_u32(words) -> np.ndarray:
    """uint32 words [..., c/8] -> 4-bit codes [..., c]; element 8j+i sits in
    bits 4i..4i+3 of word j."""
    w = np.asarray(words, dtype=np.uint32)
    shifts = (np.arange(8, dtype=np.uint32) * np.uint32(4))
    q = (w[..., None] >> shifts) & np.uint32(0xF)
    return q.reshape(*w.shape[:-1], w.shape[-1] * 8)


def dequant_affine4(words, scales_bits, qbias_bits, group: int) -> np.ndarray:
    """4-bit affine group dequantisation, weight = scale * q + qbias per group
    along the input dimension (mlxcel issue #974: gather_qmm in "affine" mode
    over a packed uint32 plane with scales and biases, group 64, 4 bits).
    Exact in float64."""
    q = unpack_nibbles_u32(words).astype(np.float64)
    s = bf16_to_f64(scales_bits)
    b = bf16_to_f64(qbias_bits)
    cols = q.shape[-1]
    qg = q.reshape(*q.shape[:-1], cols // group, group)
    return (s[..., None] * qg + b[..., None]).reshape(q.shape)


def e2m1_decode(code) -> np.ndarray:
    """OCP MX FP4 (E2M1): sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
    exponent 0 is subnormal: value = m * 0.5; otherwise 2^(e-1) * (1 + m/2)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, np.exp2(e - 1.0) * (1.0 + m / 2.0))
    return sign * mag


def e8m0_decode(code) -> np.ndarray:
    """OCP MX E8M0 shared scale: 2^(code-127); code 255 is NaN."""
    c = np.asarray(code, dtype=np.int64)
    v = np.exp2(c.astype(np.float64) - 127.0)
    return np.where(c == 255, np.nan, v)


def dequant_mxfp4(blocks, scales) -> np.ndarray:
    """MXFP4 dequantisation: two E2M1 codes per byte (even element in the low
    nibble), one E8M0 scale per 32 consecutive elements of a row.  Each code
    is looked up in the table of its 16 values (e2m1_decode of every code), so
    a whole expert decodes in one gather."""
    b = np.asarray(blocks, dtype=np.uint8)
    codes = np.empty((*b.shape[:-1], b.shape[-1] * 2), dtype=np.uint8)
    codes[..., 0::2] = b & 0xF
    codes[..., 1::2] = b >> 4
    v = E2M1_VALUES[codes]
    sc = e8m0_decode(scales)
    cols = v.shape[-1]
    return (v.reshape(*v.shape[:-1], cols // 32, 32) * sc[..., None]).reshape(v.shape)


E2M1_VALUES = e2m1_decode(np.arange(16))


# ----------------------------------------------------------------------------
# containers (plain numpy)
# ----------------------------------------------------------------------------


@dataclass
class OLinear:
    """n stacked matrices [rows=out, cols=in] in a stored format; y = W x + bias."""
    fmt: str                      # "dense" | "affine4" | "mxfp4"
    w: np.ndarray
    scales: Optional[np.ndarray] = None
    qbias: Optional[np.ndarray] = None
    bias: Optional[np.ndarray] = None
    group: int = 0

    def matrix(self, e: int) -> np.ndarray:
        if self.fmt == "dense":
            return as_f64(self.w[e])
        if self.fmt == "affine4":
            return dequant_affine4(self.w[e], self.scales[e], self.qbias[e], self.group)
        if self.fmt == "mxfp4":
            return dequant_mxfp4(self.w[e], self.scales[e])
        raise ValueError(self.fmt)

    def out_bias(self, e: int):
        return None if self.bias is None else as_f64(self.bias[e])


@dataclass
class OMLP:
    gate: OLinear
    up: OLinear
    down: OLinear
    limit: float = 0.0


@dataclass
class OBlock:
    x: np.ndarray
    router_w: np.ndarray
    scoring: str
    K: int
    norm_topk: bool
    routed_scale: float
    experts: OMLP
    logit_bias: Optional[np.ndarray] = None
    select_bias: Optional[np.ndarray] = None
    shared: Optional[OMLP] = None
    shared_mode: str = "none"
    coef_w: Optional[np.ndarray] = None
    coef_b: Optional[np.ndarray] = None
    latent_down: Optional[OLinear] = None
    latent_up: Optional[OLinear] = None
    latent_norm_w: Optional[np.ndarray] = None
    norm_eps: float = 1e-5

    @property
    def E(self) -> int:
        return self.router_w.shape[0]


# ----------------------------------------------------------------------------
# the steps
# ----------------------------------------------------------------------------


def apply_linear(lin: OLinear, e: int, z: np.ndarray) -> np.ndarray:
    """Rows z [n, cols] -> [n, rows] = z W^T (+ bias): W is stored [out, in]
    row-major and applied as W x (latent_moe.rs, WeightMatrix::apply on
    [ffn_dim, in_dim] matrices)."""
    out = z @ lin.matrix(e).T
    b = lin.out_bias(e)
    return out if b is None else out + b


def sigmoid(v: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-v))


def softmax(v: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(v, axis=axis, keepdims=True)
    ex = np.exp(v - m)
    return ex / np.sum(ex, axis=axis, keepdims=True)


def router_logits(x, router_w, logit_bias=None) -> np.ndarray:
    """logits [T,E] = x W_r^T (+ a per-expert logit offset): the gate projection
    (mlxcel PR #1044 point 3, self.gate(x); latent_moe.rs, router_weight.apply)."""
    l = as_f64(x) @ as_f64(router_w).T
    if logit_bias is not None:
        l = l + as_f64(logit_bias)
    return l


def scores_from_logits(logits, scoring: str) -> np.ndarray:
    """Sigmoid (mlxcel PR #1044 point 3) or softmax over experts."""
    if scoring == "sigmoid":
        return sigmoid(logits)
    if scoring == "softmax":
        return softmax(logits, axis=-1)
    raise ValueError(scoring)


def select_topk(sel: np.ndarray, K: int) -> np.ndarray:
    """Per token, the K experts with the largest selection key; equal keys go
    to the lower expert index; the chosen ids are reported in ascending order."""
    T, E = sel.shape
    idx = np.empty((T, K), dtype=np.int32)
    ids = np.arange(E)
    for t in range(T):
        order = np.lexsort((ids, -sel[t]))   # primary -sel, secondary id
        idx[t] = np.sort(order[:K])
    return idx


def topk_margin(sel: np.ndarray, K: int) -> np.ndarray:
    """Gap between the K-th and (K+1)-th largest selection key of each token
    (infinite when K equals the expert count)."""
    T, E = sel.shape
    if K >= E:
        return np.full(T, np.inf)
    s = -np.sort(-sel, axis=1)
    return s[:, K - 1] - s[:, K]


def route(x, router_w, scoring, K, norm_topk, routed_scale=1.0, logit_bias=None, select_bias=None,
          logits=None):
    """Router + top-k.  Selection ranks scores + select_bias; the returned
    weights are gathered from the unbiased scores, renormalised to sum 1 if
    norm_topk, then multiplied by routed_scale (mlxcel PR #1044 point 3;
    latent_moe.rs, route_top_k_sigmoid_with_bias(logits, bias, k, renormalize,
    scaling)).  `logits` may be given to recompute the selection from
    externally computed logits."""
    if logits is None:
        logits = router_logits(x, router_w, logit_bias)
    logits = np.asarray(logits, dtype=np.float64)
    s = scores_from_logits(logits, scoring)
    sel = s if select_bias is None else s + as_f64(select_bias)[None, :]
    idx = select_topk(sel, K)
    w = weights_for(s, idx, norm_topk, routed_scale)
    return {"idx": idx, "w": w, "logits": logits, "scores": s, "sel": sel}


def weights_for(scores, idx, norm_topk, routed_scale=1.0) -> np.ndarray:
    """Weights of a given selection: the unbiased scores of the chosen experts,
    divided by their sum if norm_topk, times routed_scale (mlxcel PR #1044
    point 3; latent_moe.rs route_top_k_sigmoid_with_bias argument order)."""
    w = np.take_along_axis(np.asarray(scores, dtype=np.float64), np.asarray(idx, dtype=np.int64), axis=1)
    if norm_topk:
        w = w / np.sum(w, axis=1, keepdims=True)
    return w * routed_scale


def coef_head(x, coef_w, coef_b) -> np.ndarray:
    """[T,2] = softmax(x W_c^T + b_c): the per-token 2-way blend coefficients
    (mlxcel PR #1044 point 2: a [2, hidden] projection with a [2] bias)."""
    return softmax(as_f64(x) @ as_f64(coef_w).T + as_f64(coef_b)[None, :], axis=-1)


def permute(idx: np.ndarray, E: int):
    """Group the T*K (token, slot) pairs by expert.  Slot p = t*K + j.
    counts[e] = number of slots routed to e; offsets = exclusive prefix sum;
    sorted_slot lists, for e ascending, the slots of e in ascending p;
    slot_pos is its inverse."""
    T, K = idx.shape
    flat = idx.reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    for e in flat:
        counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    sorted_slot = np.empty(T * K, dtype=np.int64)
    fill = offsets[:-1].copy()
    for p in range(T * K):
        e = flat[p]
        sorted_slot[fill[e]] = p
        fill[e] += 1
    slot_pos = np.empty(T * K, dtype=np.int64)
    slot_pos[sorted_slot] = np.arange(T * K)
    return counts, offsets, sorted_slot, slot_pos


def clamp_preact(v: np.ndarray, limit: float) -> np.ndarray:
    """swiglu_limit (libmir-metal, passed to the gate/up kernel).  The formula is
    not on the pages; reading: clamp to [-limit, limit].  Parity unpinned."""
    if limit and limit > 0:
        return np.clip(v, -limit, limit)
    return v


def silu(v: np.ndarray) -> np.ndarray:
    return v * sigmoid(v)


def swiglu(g: np.ndarray, u: np.ndarray, limit: float = 0.0) -> np.ndarray:
    """silu(gate) * up (SwitchGLU), after the optional clamp."""
    return silu(clamp_preact(g, limit)) * clamp_preact(u, limit)


def mlp_forward(mlp: OMLP, e: int, z: np.ndarray) -> np.ndarray:
    """One expert on rows z: down(swiglu(gate z, up z)) with w1 = gate, w3 = up,
    w2 = down (latent_moe.rs, KimiExpertWeights::forward)."""
    g = apply_linear(mlp.gate, e, z)
    u = apply_linear(mlp.up, e, z)
    return apply_linear(mlp.down, e, swiglu(g, u, mlp.limit))


def rms_norm(v: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """v / sqrt(mean(v^2) + eps) * w over the last axis (latent_moe.rs,
    rms_norm(&combined, w, rms_norm_eps))."""
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * as_f64(w)


# ----------------------------------------------------------------------------
# the block
# ----------------------------------------------------------------------------


def latent_input(b: OBlock) -> np.ndarray:
    """Expert input z: x itself, or down_proj(x) for the latent variant."""
    x = as_f64(b.x)
    if b.latent_down is None:
        return x
    return apply_linear(b.latent_down, 0, x)


def routed_outputs(b: OBlock, z: np.ndarray, routing) -> np.ndarray:
    """o[t, j] = expert_{idx[t,j]}(z_t), computed one expert at a time over the
    tokens routed to it (each expert's weights are decoded once)."""
    idx = routing["idx"]
    T, K = idx.shape
    o = np.zeros((T, K, z.shape[1]), dtype=np.float64)
    for e in np.unique(idx):
        tt, jj = np.nonzero(idx == e)
        o[tt, jj] = mlp_forward(b.experts, int(e), z[tt])
    return o


def block_forward(b: OBlock, routing=None):
    """The whole block for every token of b.x.  Returns y and the intermediates.

    y_r[t] = sum_j w[t,j] * expert_{idx[t,j]}(z_t), j ascending
    latent:  y_r = up_proj(rms_norm(y_r))            (latent_moe.rs flow)
    shared:  y = y_r + s (add)  |  y = c0*y_r + c1*s (blend, mlxcel PR #1044)
    """
    if routing is None:
        routing = route(b.x, b.router_w, b.scoring, b.K, b.norm_topk, b.routed_scale,
                        b.logit_bias, b.select_bias)
    z = latent_input(b)
    o = routed_outputs(b, z, routing)
    y_r = np.einsum("tk,tkd->td", routing["w"], o)
    if b.latent_down is not None:
        if b.latent_norm_w is not None:
            y_r = rms_norm(y_r, b.latent_norm_w, b.norm_eps)
        y_r = apply_linear(b.latent_up, 0, y_r)
    out = {"routing": routing, "z": z, "o": o, "y_routed": y_r}
    if b.shared is None or b.shared_mode == "none":
        out["y"] = y_r
        return out
    s = mlp_forward(b.shared, 0, as_f64(b.x))
    out["shared"] = s
    if b.shared_mode == "add":
        out["y"] = y_r + s
    elif b.shared_mode == "blend":
        c = coef_head(b.x, b.coef_w, b.coef_b)
        out["coef"] = c
        out["y"] = c[:, :1] * y_r + c[:, 1:] * s
    else:
        raise ValueError(b.shared_mode)
    return out


def block_forward_loop(b: OBlock):
    """The same block written token by token straight from its defining
    equations, for tiny inputs.  For token t with expert input z_t:

      rank_t(e)  = #{e' : sel[e'] > sel[e]} + #{e' < e : sel[e'] == sel[e]}
      e chosen  <=> rank_t(e) < K            (the K largest keys, ties to low ids)
      w_t(e)     = s[e] / sum_{chosen} s     (or s[e] without renormalisation),
                   times routed_scale; 0 for an expert not chosen
      y_r[t]     = sum over every expert e of w_t(e) * f_e(z_t), e ascending
      latent:      y_r[t] = W_up rms_norm(y_r[t])
      y[t]       = y_r[t] + f_shared(x_t)  or  c0 * y_r[t] + c1 * f_shared(x_t)

    i.e. the sparse mixture as a dense sum masked by the selection (mlxcel PR
    #1044 points 2 and 3; the latent flow of latent_moe.rs's module doc).  It
    shares only the per-matrix steps (decoding, one SwiGLU MLP, RMSNorm) with
    block_forward, not its selection or combine."""
    x = as_f64(b.x)
    T, H = x.shape
    E = b.router_w.shape[0]
    W_r = as_f64(b.router_w)
    ys = []
    for t in range(T):
        xt = x[t]
        logit = np.array([float(np.dot(W_r[e], xt)) for e in range(E)])
        if b.logit_bias is not None:
            logit = logit + as_f64(b.logit_bias)
        if b.scoring == "sigmoid":
            s = np.array([1.0 / (1.0 + math.exp(-v)) for v in logit])
        else:
            ex = np.array([math.exp(v - logit.max()) for v in logit])
            s = ex / ex.sum()
        sel = s + (0.0 if b.select_bias is None else as_f64(b.select_bias))
        rank = [sum(1 for f in range(E) if sel[f] > sel[e] or (sel[f] == sel[e] and f < e)) for e in range(E)]
        chosen = [rank[e] < b.K for e in range(E)]
        total = sum(s[e] for e in range(E) if chosen[e])
        zt = xt[None, :] if b.latent_down is None else apply_linear(b.latent_down, 0, xt[None, :])
        acc = np.zeros(zt.shape[1])
        for e in range(E):
            if not chosen[e]:
                continue
            w = (s[e] / total if b.norm_topk else s[e]) * b.routed_scale
            acc = acc + w * mlp_forward(b.experts, e, zt)[0]
        if b.latent_down is not None:
            if b.latent_norm_w is not None:
                acc = acc / math.sqrt(float(np.mean(acc * acc)) + b.norm_eps) * as_f64(b.latent_norm_w)
            acc = apply_linear(b.latent_up, 0, acc[None, :])[0]
        if b.shared is not None and b.shared_mode != "none":
            sh = mlp_forward(b.shared, 0, xt[None, :])[0]
            if b.shared_mode == "add":
                acc = acc + sh
            else:
                h = as_f64(b.coef_w) @ xt + as_f64(b.coef_b)
                c0 = 1.0 / (1.0 + math.exp(h[1] - h[0]))
                acc = c0 * acc + (1.0 - c0) * sh
        ys.append(acc)
    return np.stack(ys)


# ----------------------------------------------------------------------------
# input marshalling from the seeded generator's containers
# ----------------------------------------------------------------------------


class _PerMatrix:
    """Indexable view of a stacked stored tensor that copies one matrix's bits to
    host memory on access (full-size layers are several GB; the oracle only
    decodes the experts it needs)."""

    def __init__(self, t, raw):
        self.t, self.raw = t, raw

    def __getitem__(self, e):
        return self.raw(self.t[e])

    @property
    def shape(self):
        return tuple(self.t.shape)


def _olin(lin, raw) -> OLinear:
    lazy = lambda t: None if t is None else (_PerMatrix(t, raw) if t.shape[0] > 1 else raw(t))
    return OLinear(lin.fmt, lazy(lin.w), lazy(lin.scales), lazy(lin.qbias), lazy(lin.bias), lin.group_size)


def _omlp(m, raw) -> OMLP:
    return OMLP(_olin(m.gate, raw), _olin(m.up, raw), _olin(m.down, raw), m.swiglu_limit)


def from_block(b) -> OBlock:
    """Build the oracle's numpy view of a generated layer (its stored bits)."""
    from synth import raw
    return OBlock(
        x=raw(b.x), router_w=raw(b.router_w), scoring=b.scoring, K=b.K, norm_topk=b.norm_topk,
        routed_scale=b.routed_scale, experts=_omlp(b.experts, raw), logit_bias=raw(b.logit_bias),
        select_bias=raw(b.select_bias), shared=None if b.shared is None else _omlp(b.shared, raw),
        shared_mode=b.shared_mode, coef_w=raw(b.coef_w), coef_b=raw(b.coef_b),
        latent_down=None if b.latent_down is None else _olin(b.latent_down, raw),
        latent_up=None if b.latent_up is None else _olin(b.latent_up, raw),
        latent_norm_w=raw(b.latent_norm_w), norm_eps=b.norm_eps)
