"""Which activation precision the MFMA may take (CPU only).

fp8 activations on the prefill GEMMs, and the block-scaled f8f6f4 MFMA for MXFP4
experts (which takes its activations in an 8-, 6- or 4-bit format too), would double or
quadruple the matrix peak.  Simulated with the float64 oracle on the small layers of the
workloads -- expert inputs and SwiGLU outputs rounded to e4m3 (per-row scale, or per-32
block scale as MXFP8), everything else exact -- the block misses the output tolerance
(normwise 2e-2 with mean absolute error under 2e-3) on each of c3, c4 and c5, while bf16
rounding of the same two intermediates stays an order of magnitude inside it.  The bf16
case also pins the precision budget the GPU path relies on.

Split into two e4m3 terms with their own E8M0 block scales (hi = e4m3(v / 2^Eh), then the
remainder as lo = e4m3((v - hi 2^Eh) / 2^El), Eh and El the smallest exponents that keep
the block's largest magnitude within 448) -- what the block-scaled MFMA path of the MXFP4
experts does -- the same intermediates land inside the tolerance with room to spare, closer
than bf16 rounding.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth

TOL, MAE = 2e-2, 2e-3


def _q_e4m3(a, block):
    t = torch.tensor(a, dtype=torch.float32)
    if block:
        sh = t.shape
        tb = t.reshape(*sh[:-1], sh[-1] // block, block)
        amax = tb.abs().amax(-1, keepdim=True).clamp_min(1e-30)
        sc = torch.exp2(torch.floor(torch.log2(448.0 / amax)))
        return ((tb * sc).to(torch.float8_e4m3fn).float() / sc).reshape(sh).double().numpy()
    amax = t.abs().amax(-1, keepdim=True).clamp_min(1e-30)
    sc = 448.0 / amax
    return ((t * sc).to(torch.float8_e4m3fn).float() / sc).double().numpy()


def _q_bf16(a):
    return torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).double().numpy()


def _errors(cfg, qa, monkeypatch):
    b = synth.make_block(synth.SMALL_SPECS[cfg], "cpu")
    ob = O.from_block(b)
    ref = O.block_forward(ob)

    def mlp_q(mlp, e, z):
        zq = qa(z)
        g, u = O.apply_linear(mlp.gate, e, zq), O.apply_linear(mlp.up, e, zq)
        return O.apply_linear(mlp.down, e, qa(O.swiglu(g, u, mlp.limit)))

    with monkeypatch.context() as m:
        m.setattr(O, "mlp_forward", mlp_q)
        y = O.block_forward(ob, routing=ref["routing"])["y"]
    d = np.abs(y - ref["y"])
    return d.max() / np.abs(ref["y"]).max(), d.mean()


@pytest.mark.parametrize("cfg", ["c3", "c4", "c5"])
def test_fp8_activations_miss_the_tolerance(cfg, monkeypatch):
    for block in (0, 32):
        nw, mae = _errors(cfg, lambda a: _q_e4m3(a, block), monkeypatch)
        assert nw > TOL or mae >= MAE, (cfg, block, nw, mae)


@pytest.mark.parametrize("cfg", ["c3", "c4", "c5"])
def test_bf16_activations_fit_the_tolerance(cfg, monkeypatch):
    nw, mae = _errors(cfg, _q_bf16, monkeypatch)
    assert nw < TOL / 5 and mae < MAE / 2, (cfg, nw, mae)


def _e8m0_exp(amax):
    """The smallest E with amax / 2^E <= 448 (448 = 0.875 * 2^9), per block."""
    m, x = np.frexp(amax)
    E = np.where(m <= 0.875, x - 9, x - 8)
    return np.where(amax > 0, E, 0)


def _q_split_e4m3(a):
    """v -> hi 2^Eh + lo 2^El, both e4m3 with per-32 E8M0 scales (the MFMA path's split)."""
    sh = a.shape
    blk = a.reshape(*sh[:-1], sh[-1] // 32, 32)
    eh = _e8m0_exp(np.abs(blk).max(-1, keepdims=True))
    hi = torch.tensor(blk / 2.0 ** eh, dtype=torch.float32).to(torch.float8_e4m3fn).double().numpy() * 2.0 ** eh
    r = blk - hi
    el = _e8m0_exp(np.abs(r).max(-1, keepdims=True))
    lo = torch.tensor(r / 2.0 ** el, dtype=torch.float32).to(torch.float8_e4m3fn).double().numpy() * 2.0 ** el
    return (hi + lo).reshape(sh)


def test_split_e4m3_pair_is_exact_on_representable_values():
    """Values that one e4m3 term already holds come back exactly (lo = 0); a block's largest
    magnitude lands on 448 or below."""
    v = np.array([[1.0, -0.5, 448.0, 3.0, 0.0, 0.125, -2.0, 6.0] * 4])
    assert np.array_equal(_q_split_e4m3(v), v)
    w = np.array([[1000.0] + [0.0] * 31])
    assert _e8m0_exp(np.array([1000.0])) == 2 and np.array_equal(_q_split_e4m3(w), w)


@pytest.mark.parametrize("cfg", ["c3", "c4", "c5"])
def test_split_e4m3_activations_fit_the_tolerance(cfg, monkeypatch):
    nw, mae = _errors(cfg, _q_split_e4m3, monkeypatch)
    nwb, maeb = _errors(cfg, _q_bf16, monkeypatch)
    assert nw < TOL / 10 and mae < MAE / 10, (cfg, nw, mae)
    assert nw < nwb and mae < maeb, (cfg, nw, nwb, mae, maeb)
