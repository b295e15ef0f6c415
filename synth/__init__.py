"""Seeded synthetic inputs for the sparse MoE FFN block.

This module only draws random tensors and encodes them into the stored
formats that both the GPU library and the oracle read (bf16, packed 4-bit
affine groups, MXFP4 blocks).  It evaluates nothing of the block itself:
no routing, no matmul, no activation.  Decoding those stored bytes back to
numbers is done independently on each side.

Everything is drawn with torch on a caller-chosen device, so the same code
makes small CPU cases for the oracle's own tests and full-size layers
directly in GPU memory.  A given (spec, seed, device type) always yields the
same bytes.

Stored formats (the conventions shared by both sides):
  * bf16: torch.bfloat16 (round-to-nearest-even from float32).
  * affine 4-bit, group g along the input dim: int32 words [n, rows, cols/8],
    element 8*j+i in bits 4*i..4*i+3 of word j; bf16 scales and bf16 qbias
    [n, rows, cols/g]; the weight is scale*q + qbias with q in 0..15
    (the "weight, scales, biases / affine / group 64 / 4-bit" plane of
    mlxcel issue #974, sections "What exists" and "Evidence gathered").
  * MXFP4: uint8 [n, rows, cols/2], two E2M1 codes per byte, even element in
    the low nibble; uint8 E8M0 exponents [n, rows, cols/32]; optional bf16
    output bias [n, rows] (the blocks/scales/bias planes of libmir-metal's
    ExpertLayout::Native / Mlx variants).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import torch

# ----------------------------------------------------------------------------
# containers
# ----------------------------------------------------------------------------

FMT_DENSE = "dense"
FMT_AFFINE4 = "affine4"
FMT_MXFP4 = "mxfp4"


@dataclass
class Linear:
    """n stacked matrices [rows=out, cols=in]; y = W x (+ bias)."""
    fmt: str
    n: int
    rows: int
    cols: int
    w: torch.Tensor                       # dense f32/bf16 [n,rows,cols]; affine4 int32 [n,rows,cols/8]; mxfp4 uint8 [n,rows,cols/2]
    scales: Optional[torch.Tensor] = None  # affine4 bf16 [n,rows,cols/g]; mxfp4 uint8 [n,rows,cols/32]
    qbias: Optional[torch.Tensor] = None   # affine4 bf16 [n,rows,cols/g]
    bias: Optional[torch.Tensor] = None    # bf16 [n,rows] output bias (or f32 for dense f32)
    group_size: int = 0

    def to(self, device) -> "Linear":
        mv = lambda t: None if t is None else t.to(device)
        return replace(self, w=mv(self.w), scales=mv(self.scales), qbias=mv(self.qbias), bias=mv(self.bias))

    def nbytes_per_matrix(self) -> int:
        b = self.w[0].numel() * self.w.element_size()
        for t in (self.scales, self.qbias, self.bias):
            if t is not None:
                b += t[0].numel() * t.element_size()
        return b


@dataclass
class MLP:
    gate: Linear
    up: Linear
    down: Linear
    swiglu_limit: float = 0.0   # <= 0: no clamp

    def to(self, device) -> "MLP":
        return replace(self, gate=self.gate.to(device), up=self.up.to(device), down=self.down.to(device))


@dataclass
class Block:
    name: str
    T: int
    H: int
    D: int
    E: int
    K: int
    I: int
    I_s: int
    x: torch.Tensor                      # [T,H] f32 or bf16
    router_w: torch.Tensor               # [E,H] same dtype as x
    scoring: str                         # "sigmoid" | "softmax"
    norm_topk: bool
    routed_scale: float
    experts: MLP
    logit_bias: Optional[torch.Tensor] = None   # [E] f32, added to logits
    select_bias: Optional[torch.Tensor] = None  # [E] f32, added to scores for selection only
    shared: Optional[MLP] = None
    shared_mode: str = "none"            # "none" | "add" | "blend"
    coef_w: Optional[torch.Tensor] = None  # [2,H] same dtype as x
    coef_b: Optional[torch.Tensor] = None  # [2] f32
    latent_down: Optional[Linear] = None   # n=1, [D,H] dense bf16
    latent_up: Optional[Linear] = None     # n=1, [H,D] dense bf16
    latent_norm_w: Optional[torch.Tensor] = None  # [D] f32
    norm_eps: float = 1e-5
    seed: int = 0
    meta: dict = field(default_factory=dict)

    def to(self, device) -> "Block":
        mv = lambda t: None if t is None else t.to(device)
        return replace(
            self, x=mv(self.x), router_w=mv(self.router_w), experts=self.experts.to(device),
            logit_bias=mv(self.logit_bias), select_bias=mv(self.select_bias),
            shared=None if self.shared is None else self.shared.to(device),
            coef_w=mv(self.coef_w), coef_b=mv(self.coef_b),
            latent_down=None if self.latent_down is None else self.latent_down.to(device),
            latent_up=None if self.latent_up is None else self.latent_up.to(device),
            latent_norm_w=mv(self.latent_norm_w))

    @property
    def act_dtype(self) -> torch.dtype:
        return self.x.dtype


# ----------------------------------------------------------------------------
# encoders (storage formats only)
# ----------------------------------------------------------------------------

def _to_i32_bits(v: torch.Tensor) -> torch.Tensor:
    """int64 holding a value in [0, 2^32) -> int32 with the same 32 bits."""
    v = torch.where(v >= 2 ** 31, v - 2 ** 32, v)
    return v.to(torch.int32)


def encode_affine4(w: torch.Tensor, group: int):
    """Float weights [..., cols] -> (packed int32 [..., cols/8], scales bf16, qbias bf16).

    Per group: qbias = min, scale = (max-min)/15, both rounded to bf16;
    q = clip(rint((w - qbias)/scale), 0, 15).
    """
    cols = w.shape[-1]
    assert cols % group == 0 and cols % 8 == 0
    wg = w.float().reshape(*w.shape[:-1], cols // group, group)
    lo = wg.amin(dim=-1)
    hi = wg.amax(dim=-1)
    scale = ((hi - lo) / 15.0)
    scale = torch.where(scale > 0, scale, torch.ones_like(scale))
    scale_b = scale.to(torch.bfloat16)
    qbias_b = lo.to(torch.bfloat16)
    q = torch.round((wg - qbias_b.float().unsqueeze(-1)) / scale_b.float().unsqueeze(-1))
    q = q.clamp(0, 15).to(torch.int64).reshape(*w.shape[:-1], cols // 8, 8)
    shifts = torch.arange(8, device=w.device, dtype=torch.int64) * 4
    packed = (q << shifts).sum(dim=-1)
    return _to_i32_bits(packed), scale_b, qbias_b


# E2M1 magnitudes by 3-bit code (OCP Microscaling Formats v1.0, FP4 E2M1).
_E2M1_MAG = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def encode_mxfp4(w: torch.Tensor):
    """Float weights [..., cols] -> (uint8 codes [..., cols/2], uint8 e8m0 [..., cols/32]).

    Shared exponent per 32-element block: floor(log2(amax)) - 2 (E2M1's
    largest exponent is 2); elements rounded to the nearest E2M1 value
    (ties to the even code), saturating at +-6.
    """
    cols = w.shape[-1]
    assert cols % 32 == 0
    wb = w.float().reshape(*w.shape[:-1], cols // 32, 32)
    amax = wb.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(torch.where(amax > 0, amax, torch.ones_like(amax)))) - 2,
                    torch.zeros_like(amax))
    e = e.clamp(-127, 127)
    code8 = (e + 127).to(torch.uint8)
    v = wb / torch.exp2(e).unsqueeze(-1)
    a = v.abs()
    # midpoints between consecutive E2M1 magnitudes; ties go to the even code
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], device=w.device)
    mag = torch.bucketize(a, mids, right=False)     # a <= mid -> lower code
    # bucketize(right=False) puts a == mid into the lower bucket; fix ties whose lower code is odd
    tie = (a.unsqueeze(-1) == mids).any(dim=-1)
    mag = torch.where(tie & (mag % 2 == 1), mag + 1, mag)
    mag = mag.clamp(0, 7)
    sign = (v < 0).to(torch.int64)
    code = (sign << 3) | mag.to(torch.int64)
    code = code.reshape(*w.shape[:-1], cols // 2, 2)
    byte = (code[..., 0] | (code[..., 1] << 4)).to(torch.uint8)
    return byte, code8


# ----------------------------------------------------------------------------
# layer specs
# ----------------------------------------------------------------------------

@dataclass
class Spec:
    name: str
    T: int
    H: int
    E: int
    K: int
    I: int
    I_s: int
    D: int = 0                    # latent width (0: same as H)
    act: str = "bf16"             # "f32" | "bf16"
    expert_fmt: str = FMT_AFFINE4
    shared_fmt: str = FMT_AFFINE4
    group: int = 64
    scoring: str = "sigmoid"
    norm_topk: bool = True
    select_bias: bool = True
    logit_offsets: bool = False
    shared_mode: str = "blend"
    swiglu_limit: float = 0.0
    expert_bias: bool = False     # MXFP4 output biases
    latent_norm: bool = False
    w_std: float = 0.02
    seed: int = 1

    @property
    def Dz(self) -> int:
        return self.D if self.D else self.H


# The five layers of the workload list (hidden, experts, top-k, widths, formats).
FULL_SPECS = {
    "c1": Spec("c1", T=4, H=64, E=8, K=2, I=128, I_s=128, act="f32", expert_fmt=FMT_DENSE,
               shared_fmt=FMT_DENSE, scoring="sigmoid", norm_topk=True, select_bias=True,
               shared_mode="blend", seed=1),
    "c2": Spec("c2", T=32, H=2048, E=256, K=8, I=768, I_s=768, logit_offsets=True, seed=2),
    "c3": Spec("c3", T=4096, H=2048, E=256, K=8, I=768, I_s=768, logit_offsets=True, seed=3),
    "c4": Spec("c4", T=2048, H=2816, E=128, K=8, I=704, I_s=2112, scoring="softmax", norm_topk=False,
               select_bias=False, shared_mode="add", seed=4),
    "c5": Spec("c5", T=1024, H=7168, D=3584, E=384, K=8, I=2048, I_s=2048, expert_fmt=FMT_MXFP4,
               shared_fmt=FMT_DENSE, group=32, scoring="sigmoid", norm_topk=True, select_bias=True,
               shared_mode="add", swiglu_limit=7.0, expert_bias=True, latent_norm=True, seed=5),
}

# Reduced versions with the same structure, small enough for the oracle to finish
# in seconds, still spanning several tiles and ragged tails.
SMALL_SPECS = {
    "c1": FULL_SPECS["c1"],
    "c2": replace(FULL_SPECS["c2"], name="c2s", T=37, H=512, E=32, K=8, I=192, I_s=256, seed=12),
    "c3": replace(FULL_SPECS["c3"], name="c3s", T=333, H=512, E=16, K=4, I=256, I_s=192, seed=13),
    "c4": replace(FULL_SPECS["c4"], name="c4s", T=150, H=704, E=24, K=6, I=192, I_s=320, seed=14),
    "c5": replace(FULL_SPECS["c5"], name="c5s", T=70, H=1024, D=448, E=48, K=8, I=256, I_s=320, seed=15),
}


def _randn(gen, shape, std, device, dtype=torch.float32):
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32).mul_(std).to(dtype)


def _dense(gen, n, rows, cols, std, device, dtype) -> Linear:
    w = _randn(gen, (n, rows, cols), std, device, dtype)
    return Linear(FMT_DENSE, n, rows, cols, w)


def _stack_encoded(gen, fmt, n, rows, cols, std, group, device, with_bias, chunk=8) -> Linear:
    """Draw n matrices in chunks and encode each chunk (bounded peak memory)."""
    ws, ss, qs = [], [], []
    for s in range(0, n, chunk):
        c = min(chunk, n - s)
        w = _randn(gen, (c, rows, cols), std, device)
        if fmt == FMT_AFFINE4:
            p, sc, qb = encode_affine4(w, group)
            ws.append(p); ss.append(sc); qs.append(qb)
        else:
            p, sc = encode_mxfp4(w)
            ws.append(p); ss.append(sc)
        del w
    lin = Linear(fmt, n, rows, cols, torch.cat(ws), torch.cat(ss),
                 torch.cat(qs) if qs else None, None, group if fmt == FMT_AFFINE4 else 32)
    if with_bias:
        lin.bias = _randn(gen, (n, rows), std, device, torch.bfloat16)
    return lin


def _linear(gen, fmt, n, rows, cols, spec: Spec, device, with_bias=False) -> Linear:
    if fmt == FMT_DENSE:
        dt = torch.float32 if spec.act == "f32" else torch.bfloat16
        lin = _dense(gen, n, rows, cols, spec.w_std, device, dt)
        if with_bias:
            lin.bias = _randn(gen, (n, rows), spec.w_std, device, dt)
        return lin
    return _stack_encoded(gen, fmt, n, rows, cols, spec.w_std, spec.group, device, with_bias)


def make_block(spec: Spec, device="cpu", seed: Optional[int] = None, T: Optional[int] = None) -> Block:
    """Draw a layer for `spec`.  Fixed draw order: x, router, logit offsets,
    selection bias, coefficient head, routed experts (gate, up, down), shared
    expert, latent projections, latent norm weight."""
    seed = spec.seed if seed is None else seed
    T = spec.T if T is None else T
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    adt = torch.float32 if spec.act == "f32" else torch.bfloat16
    H, D = spec.H, spec.Dz
    x = _randn(gen, (T, H), 1.0, device, adt)
    router_w = _randn(gen, (spec.E, H), 1.0 / H ** 0.5, device, adt)
    logit_bias = _randn(gen, (spec.E,), 1.0, device) if spec.logit_offsets else None
    select_bias = _randn(gen, (spec.E,), 0.1, device) if spec.select_bias else None
    coef_w = coef_b = None
    if spec.shared_mode == "blend":
        coef_w = _randn(gen, (2, H), spec.w_std, device, adt)
        coef_b = _randn(gen, (2,), spec.w_std, device)
    eb = spec.expert_bias
    experts = MLP(_linear(gen, spec.expert_fmt, spec.E, spec.I, D, spec, device, eb),
                  _linear(gen, spec.expert_fmt, spec.E, spec.I, D, spec, device, eb),
                  _linear(gen, spec.expert_fmt, spec.E, D, spec.I, spec, device, eb),
                  spec.swiglu_limit)
    shared = None
    if spec.shared_mode != "none":
        shared = MLP(_linear(gen, spec.shared_fmt, 1, spec.I_s, H, spec, device),
                     _linear(gen, spec.shared_fmt, 1, spec.I_s, H, spec, device),
                     _linear(gen, spec.shared_fmt, 1, H, spec.I_s, spec, device), 0.0)
    latent_down = latent_up = norm_w = None
    if spec.D:
        latent_down = _dense(gen, 1, D, H, spec.w_std, device, torch.bfloat16)
        latent_up = _dense(gen, 1, H, D, spec.w_std, device, torch.bfloat16)
        if spec.latent_norm:
            norm_w = 1.0 + _randn(gen, (D,), 0.1, device)
    return Block(spec.name, T, H, D, spec.E, spec.K, spec.I, spec.I_s, x, router_w, spec.scoring,
                 spec.norm_topk, 1.0, experts, logit_bias, select_bias, shared, spec.shared_mode,
                 coef_w, coef_b, latent_down, latent_up, norm_w, 1e-5, seed,
                 meta={"spec": spec})


def token_subset(b: Block, tokens) -> Block:
    """The same layer applied to a subset of its tokens (rows of x)."""
    idx = torch.as_tensor(tokens, device=b.x.device, dtype=torch.long)
    return replace(b, x=b.x.index_select(0, idx).contiguous(), T=int(idx.numel()))


# ----------------------------------------------------------------------------
# raw storage as numpy (what the oracle reads)
# ----------------------------------------------------------------------------

def raw(t: Optional[torch.Tensor]):
    """Tensor -> numpy array of its stored bits (bf16 as uint16, int32 words as uint32)."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.int32:
        return t.numpy().view("uint32")
    return t.numpy()


def clone_weights(b: Block) -> Block:
    """A copy of the layer whose weight tensors live in fresh memory (x is shared)."""
    cl = lambda t: None if t is None else t.clone()

    def lin(l: Optional[Linear]):
        return None if l is None else replace(l, w=cl(l.w), scales=cl(l.scales), qbias=cl(l.qbias), bias=cl(l.bias))

    def mlp(m: Optional[MLP]):
        return None if m is None else replace(m, gate=lin(m.gate), up=lin(m.up), down=lin(m.down))

    return replace(b, router_w=cl(b.router_w), experts=mlp(b.experts), logit_bias=cl(b.logit_bias),
                   select_bias=cl(b.select_bias), shared=mlp(b.shared), coef_w=cl(b.coef_w), coef_b=cl(b.coef_b),
                   latent_down=lin(b.latent_down), latent_up=lin(b.latent_up), latent_norm_w=cl(b.latent_norm_w))
