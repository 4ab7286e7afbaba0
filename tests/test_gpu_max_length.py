"""The longest sequence the boundary accepts, n = 2^22, on the forward pass,
the decode step and the chain-corner scan (one head, d = 128): every index of
the kernels at its largest, compared with the fp64 oracle on sampled rows.

Gates u ~ U(0.5, 1): the carried gate modulus reaches exactly 0 in float32
within a few key tiles, so the forward's early exit and the oracle's row loop
(which stops once the f64 modulus is exactly 0) both stay short; rows near
the start, the end, and tile and chunk boundaries are sampled.  Tolerances as
elsewhere: 2e-2 on the bf16 forward, 1e-4 for the float32-weight decode step
and the chain.
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
N = 1 << 22


def announce(*a):
    print("case:", *a, flush=True)


@pytest.fixture(scope="module")
def big():
    announce(f"drawing one head at n = {N}")
    return inputs.draw(1, 1, N, 128, seed=2024, u_range=(0.5, 1.0))


def rows_of(n, rng):
    fixed = [0, 1, 63, 64, 255, 256, 257, n // 2, n - 257, n - 256, n - 65, n - 2, n - 1]
    return np.array(sorted(set(fixed + rng.integers(0, n, size=6).tolist())), dtype=np.int64)


def test_forward_at_max_length(big):
    announce(f"forward bf16 n={N} d=128 (sampled rows)")
    t = inputs.as_torch(big, DEV)
    o_re, o_im = binding.resolvent_forward(t["q"], t["k"], t["u"], t["theta"], t["v"], 1, 1, 1)
    rows = rows_of(N, np.random.default_rng(1))
    got = (o_re[0, 0, rows].double() + 1j * o_im[0, 0, rows].double()).cpu().numpy()
    del o_re, o_im
    ref = gu.oracle_rows(big, (1, 1, 1), 0, 0, rows)
    err = gu.rel_err(got, ref)
    print(f"  rel err {err:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= gu.TOL_BF16


def test_decode_at_max_length(big):
    announce(f"decode n={N} d=128")
    t = inputs.as_torch(big, DEV)
    q = t["q"][:, :, N - 1].contiguous()
    o_re, o_im = binding.resolvent_decode(q, t["k"], t["u"], t["theta"], t["v"], 1, 1, 1)
    got = (o_re.double() + 1j * o_im.double()).cpu().numpy()[0, 0]
    st, ref = oracle.forward_rows(big["q"][0, 0], big["k"][0, 0], big["u"][0, 0],
                                  big["theta"][0, 0], big["v"][0, 0], 1, 1, 1, rows=[N - 1])
    assert st == oracle.OK
    err = gu.rel_err(got, ref[0])
    print(f"  rel err {err:.3e}")
    assert err <= 1e-4


def test_chain_at_max_length(big):
    announce(f"chain n={N} dv=128 (sampled positions, 8 channels)")
    t = inputs.as_torch(big, DEV)
    o_re, o_im = binding.resolvent_chain(t["u"], t["theta"], t["v"], 1.0)
    rows = rows_of(N, np.random.default_rng(2))
    chans = [0, 1, 37, 64, 100, 125, 126, 127]
    got = (o_re[0, 0][rows][:, chans].double()
           + 1j * o_im[0, 0][rows][:, chans].double()).cpu().numpy()
    del o_re, o_im
    st, a = oracle.gates(big["u"][0, 0], big["theta"][0, 0], 1.0)
    assert st == oracle.OK
    ref = np.stack([oracle.chain(a, big["v"][0, 0, :, c], y0_from_b0=True)[rows] for c in chans],
                   axis=1)
    err = gu.rel_err(got, ref)
    print(f"  rel err {err:.3e}")
    assert err <= 1e-4
