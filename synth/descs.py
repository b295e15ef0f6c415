"""libmoe descriptors for a generated layer (glue for the tests and the benchmark)."""
from __future__ import annotations

import sparse_mixture_experts_bias_amd as moe

from . import Block, Linear, MLP


def linear_desc(l: Linear) -> "moe.Desc":
    return moe.linear(l.fmt, l.w, l.scales, l.qbias, l.bias, l.group_size)


def mlp_desc(m: MLP, scaled: bool = False) -> "moe.Desc":
    return moe.mlp(linear_desc(m.gate), linear_desc(m.up), linear_desc(m.down), m.swiglu_limit, scaled=scaled)


def router_desc(b: Block) -> "moe.Desc":
    return moe.router(b.router_w, b.K, b.scoring, b.norm_topk, b.routed_scale, b.logit_bias, b.select_bias)


def inter_dtype_for(b: Block) -> int:
    """f32 layers keep f32 intermediates; the latent layer keeps fp16 ones (its
    unit-scale outputs need them to stay inside the error budget), and so do prefill-sized
    batches (more than 64 tokens), whose GEMMs then also dequantise and multiply in f16;
    decode-sized batches of the other layers keep bf16 (the decode launches take bf16)."""
    if b.x.dtype.is_floating_point and b.x.element_size() == 4:
        return moe.MOE_F32
    return moe.MOE_F16 if (b.latent_down is not None or b.T > 64) else moe.MOE_BF16


def block_desc(b: Block, inter_dtype: int = None, scaled: bool = False) -> "moe.Desc":
    """scaled: MXFP4 routed experts also get the block-scaled MFMA's streams."""
    if inter_dtype is None:
        inter_dtype = inter_dtype_for(b)
    return moe.block(
        b.H, router_desc(b), mlp_desc(b.experts, scaled),
        shared=None if b.shared is None else mlp_desc(b.shared), shared_mode=b.shared_mode,
        coef_w=b.coef_w, coef_b=b.coef_b,
        latent_down=None if b.latent_down is None else linear_desc(b.latent_down),
        latent_up=None if b.latent_up is None else linear_desc(b.latent_up),
        latent_norm_w=b.latent_norm_w, norm_eps=b.norm_eps, inter_dtype=inter_dtype)
