"""Parity of resolvent_forward_grouped (value width dv free, k/v heads shared
by groups of query heads) with the fp64 oracle, through the C ABI.

Query head h of batch entry b reads k/v head h / (H / Hkv) and keeps its own
gates; the oracle's reference for it is the head's readout (section "Object"
of the "Resolvent Operator" page, with the Rust API's value_dim) on those
keys and values.  Tolerances are the workloads': 2e-2 with bf16 q,k, 1e-4 on
the fp32 path, of max |dO| / (max |O| + 1e-6).
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


def announce(*a):
    print("case:", *a, flush=True)


def grouped_inputs(B, H, Hkv, n, d, dv, seed, qk_dtype=inputs.BF16, v_dtype=inputs.BF16,
                   u_range=(0.5, 1.0)):
    inp = inputs.draw(B, H, n, d, seed, qk_dtype=qk_dtype, v_dtype=v_dtype, dv=dv,
                      u_range=u_range)
    inp["k"] = np.ascontiguousarray(inp["k"][:, :Hkv])
    inp["v"] = np.ascontiguousarray(inp["v"][:, :Hkv])
    inp["Hkv"] = Hkv
    return inp


def gpu_grouped(inp, sw):
    t = inputs.as_torch(inp, DEV)
    o_re, o_im = binding.resolvent_forward_grouped(t["q"], t["k"], t["u"], t["theta"], t["v"],
                                                   *sw)
    return o_re.double().cpu().numpy() + 1j * o_im.double().cpu().numpy()


def oracle_grouped(inp, sw, heads, rows):
    H, Hkv = inp["q"].shape[1], inp["Hkv"]
    group = H // Hkv
    out = []
    for b, h in heads:
        st, ref = oracle.forward_rows(inp["q"][b, h], inp["k"][b, h // group], inp["u"][b, h],
                                      inp["theta"][b, h], inp["v"][b, h // group], *sw,
                                      rows=rows)
        assert st == oracle.OK
        out.append(ref)
    return np.stack(out)


def compare(inp, sw, got, heads=None, rows=None):
    B, H, n = inp["u"].shape
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    rows = np.arange(n) if rows is None else rows
    ref = oracle_grouped(inp, sw, heads, rows)
    return gu.rel_err(np.stack([got[b, h][rows] for b, h in heads]), ref)


@pytest.mark.parametrize("d,dv", [(64, 128), (128, 64), (64, 64), (128, 128)])
@pytest.mark.parametrize("Hkv", [4, 2, 1])
@pytest.mark.parametrize("n", [200, 257])
def test_grouped_bf16_in_full(d, dv, Hkv, n):
    announce(f"grouped bf16 d={d} dv={dv} H=4 Hkv={Hkv} n={n}")
    inp = grouped_inputs(1, 4, Hkv, n, d, dv, seed=11 + n + d + dv + Hkv)
    sw = (1, 1, 1)
    got = gpu_grouped(inp, sw)
    assert got.shape == (1, 4, n, dv)
    err = compare(inp, sw, got)
    print(f"  rel err {err:.3e}")
    assert err <= gu.TOL_BF16


@pytest.mark.parametrize("d,dv", [(64, 128), (128, 64)])
def test_grouped_fp32_in_full(d, dv):
    announce(f"grouped fp32 d={d} dv={dv}")
    inp = grouped_inputs(1, 4, 2, 300, d, dv, seed=5, qk_dtype=inputs.F32, v_dtype=inputs.F32,
                         u_range=(0.0, 1.0))
    for sw in ((1, 1, 0), (0.5, 0.7, 0.5)):
        got = gpu_grouped(inp, sw)
        err = compare(inp, sw, got)
        print(f"  switches {sw}: rel err {err:.3e}")
        assert err <= gu.TOL_F32


@pytest.mark.parametrize("sw", [(1, 0, 1), (0, 0, 1), (0, 1, 0)])
def test_grouped_switches(sw):
    announce(f"grouped switches {sw}")
    inp = grouped_inputs(2, 4, 2, 320, 128, 64, seed=21)
    got = gpu_grouped(inp, sw)
    err = compare(inp, sw, got)
    print(f"  rel err {err:.3e}")
    assert err <= gu.TOL_BF16


def test_grouped_equals_forward_without_grouping_bitwise():
    """Hkv = H and dv = d: resolvent_forward_grouped runs the same kernels as
    resolvent_forward, so the outputs agree bit for bit."""
    announce("grouped with Hkv = H, dv = d vs resolvent_forward")
    inp = inputs.make_config(2, n=700, B=1, H=4)
    inp["Hkv"] = 4
    t = inputs.as_torch(inp, DEV)
    a = binding.resolvent_forward(t["q"], t["k"], t["u"], t["theta"], t["v"], 1, 1, 1)
    b = binding.resolvent_forward_grouped(t["q"], t["k"], t["u"], t["theta"], t["v"], 1, 1, 1)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_grouped_large_sampled():
    announce("grouped B=2 H=16 Hkv=2 n=4096 d=128 dv=64 (sampled rows)")
    inp = grouped_inputs(2, 16, 2, 4096, 128, 64, seed=31, u_range=(0.95, 1.0))
    sw = (1, 1, 1)
    got = gpu_grouped(inp, sw)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(31)
    err = compare(inp, sw, got, heads=[(0, 0), (0, 7), (0, 8), (1, 15)],
                  rows=gu.sample_rows(4096, rng))
    print(f"  rel err {err:.3e}")
    assert err <= gu.TOL_BF16
