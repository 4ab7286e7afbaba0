"""Parity of the chain-corner scan (resolvent_chain, through the C ABI) with
the fp64 oracle's gated chain.

At switches (0, 0, g) the head's readout is O_i = sum_{j<=i} G_ij V_j, the
chain y_i = a_i y_{i-1} + V_i with y_0 = V_0 ("Resolvent Operator" page,
section "The path-product corner is a resolvent"); the oracle's reference is
``oracle.chain(oracle.gates(u, theta, g), V[:, c], y0_from_b0=True)`` per
channel, itself pinned to the page by the CPU tests.

Tolerance, from the arithmetic: inside a 64-position tile the device runs at
most 64 fp32 recurrence steps with |a| <= 1 on fp32-rounded gates (about
4 * 64 * 2^-24 = 1.5e-5 relative to the largest |y|), and the carry between
tiles is folded in f64; the fp32 path's bound 1e-4 of the metric
max |dO| / (max |O| + 1e-6) covers it with margin.  Small shapes are
compared in full (several tiles, ragged tails); the headline shape is also
compared in full, since the reference is O(n dv) per head.
"""
import numpy as np
import pytest
import torch

import oracle
from gated_causal_attention_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"
TOL_CHAIN = 1e-4


def announce(*a):
    print("case:", *a, flush=True)


def gpu_chain(inp, g):
    t = inputs.as_torch(inp, DEV)
    o_re, o_im = binding.resolvent_chain(t["u"], t["theta"], t["v"], g)
    return o_re.double().cpu().numpy() + 1j * o_im.double().cpu().numpy()


def oracle_chain(inp, g, heads=None):
    B, H, n = inp["u"].shape
    dv = inp["v"].shape[-1]
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    out = np.zeros((len(heads), n, dv), dtype=np.complex128)
    for x, (b, h) in enumerate(heads):
        st, a = oracle.gates(inp["u"][b, h], inp["theta"][b, h], g)
        assert st == oracle.OK
        for c in range(dv):
            out[x, :, c] = oracle.chain(a, inp["v"][b, h, :, c], y0_from_b0=True)
    return out


def compare(inp, g, got, heads=None):
    B, H, _ = inp["u"].shape
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_chain(inp, g, heads)
    return gu.rel_err(np.stack([got[b, h] for b, h in heads]), ref)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 200, 257, 520])
@pytest.mark.parametrize("dv,v_dtype", [(64, inputs.F32), (128, inputs.BF16)])
def test_chain_small_in_full(n, dv, v_dtype):
    announce(f"chain n={n} dv={dv} v={'f32' if v_dtype == inputs.F32 else 'bf16'}")
    inp = inputs.draw(2, 2, n, 64, seed=100 + n, v_dtype=v_dtype, dv=dv)
    got = gpu_chain(inp, 1.0)
    err = compare(inp, 1.0, got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_CHAIN


@pytest.mark.parametrize("dv,v_dtype", [(256, inputs.BF16), (192, inputs.BF16),
                                        (128, inputs.F32), (320, inputs.F32)])
def test_chain_value_widths(dv, v_dtype):
    """Widths of the 16-byte aggregate (256 bf16, 128 fp32) and of the
    per-channel fallback (192, 320), over ragged lengths and more tiles than
    the carry fold has segments."""
    announce(f"chain dv={dv} v={'f32' if v_dtype == inputs.F32 else 'bf16'}")
    for n in (70, 1300):
        inp = inputs.draw(1, 2, n, 64, seed=n + dv, v_dtype=v_dtype, dv=dv, u_range=(0.8, 1.0))
        got = gpu_chain(inp, 1.0)
        err = compare(inp, 1.0, got)
        print(f"  n={n}: rel err {err:.3e}")
        assert err <= TOL_CHAIN


@pytest.mark.parametrize("g", [0.0, 0.5, 1.0, 2.5])
def test_chain_gate_switch(g):
    announce(f"chain g={g}")
    inp = inputs.draw(1, 3, 700, 64, seed=7, v_dtype=inputs.F32, u_range=(0.9, 1.0), dv=64)
    got = gpu_chain(inp, g)
    err = compare(inp, g, got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_CHAIN
    if g == 0.0:  # every gate is 1: the readout is the running sum, O_im == 0
        assert np.all(got.imag == 0)


def test_chain_headline_shape_in_full():
    announce("chain at the headline shape (workload 3 inputs, every head and channel)")
    inp = inputs.make_config(3)
    got = gpu_chain(inp, 1.0)
    assert np.all(np.isfinite(got))
    err = compare(inp, 1.0, got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_CHAIN


def test_chain_closed_gates_cut_exactly():
    """A closed gate (m_k = 0) cuts the chain: y_k = V_k exactly, bitwise
    (pathProd_eq_zero_iff); the rest within tolerance."""
    announce("chain with bedM gates")
    inp = inputs.make_config(4, n=4096, H=4)
    got = gpu_chain(inp, 1.0)
    closed = inp["u"] == 0.0
    assert closed.sum() > 0
    v = inp["v"]
    for b, h, k in zip(*np.nonzero(closed)):
        if k == 0:
            continue
        assert np.all(got[b, h, k].real == v[b, h, k].astype(np.float64))
        assert np.all(got[b, h, k].imag == 0)
    err = compare(inp, 1.0, got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_CHAIN


def test_chain_equals_forward_at_the_corner():
    """resolvent_chain(u, theta, v, g) == resolvent_forward(..., 0, 0, g): on
    the fp32 path to 1e-4, on the bf16 path (bf16 weights) to 2e-2."""
    announce("chain vs forward at (0, 0, g)")
    for idx, n, tol in ((1, 256, gu.TOL_F32), (3, 1024, gu.TOL_BF16)):
        inp = inputs.make_config(idx, n=n, B=1, H=2 if idx == 3 else 1)
        for g in (1.0, 0.5):
            fwd = gu.gpu_forward(inp, (0.0, 0.0, g))
            got = gpu_chain(inp, g)
            err = gu.rel_err(got, fwd)
            print(f"  workload {idx} g={g}: rel diff {err:.3e} (tol {tol})")
            assert err <= tol


def test_chain_refusals_and_empty():
    announce("chain refusals")
    inp = inputs.draw(1, 1, 130, 64, seed=3, v_dtype=inputs.F32, dv=64)
    t = inputs.as_torch(inp, DEV)
    for name in ("u", "theta"):
        bad = t[name].clone()
        bad[0, 0, 0] = float("nan")  # index 0 is checked although a_0 is never read
        args = dict(t)
        args[name] = bad
        with pytest.raises(binding.ResolventError) as e:
            binding.resolvent_chain(args["u"], args["theta"], args["v"], 1.0)
        assert e.value.status == binding.Status.NONFINITE
    with pytest.raises(binding.ResolventError) as e:
        binding.resolvent_chain(t["u"], t["theta"], t["v"], float("inf"))
    assert e.value.status == binding.Status.NONFINITE
    empty = torch.empty((1, 1, 0, 64), device=DEV)
    o_re, o_im = binding.resolvent_chain(torch.empty((1, 1, 0), device=DEV),
                                         torch.empty((1, 1, 0), device=DEV), empty, 1.0)
    assert o_re.shape == (1, 1, 0, 64)
