"""Helpers shared by the GPU parity tests: run the HIP path, run the oracle on
the same seeded inputs, and measure the parity metric
max |dO| / (max |O| + 1e-6) over the compared outputs (complex moduli)."""
import numpy as np

import oracle
from gated_causal_attention_amd import binding, inputs

TOL_BF16 = 2e-2
TOL_F32 = 1e-4


def tol_for(inp):
    return TOL_F32 if inp["qk_dtype"] == inputs.F32 else TOL_BF16


def gpu_forward(inp, sw, device="cuda:0", **kw):
    t = inputs.as_torch(inp, device)
    o_re, o_im = binding.resolvent_forward(t["q"], t["k"], t["u"], t["theta"], t["v"], *sw, **kw)
    return o_re.double().cpu().numpy() + 1j * o_im.double().cpu().numpy()


def oracle_rows(inp, sw, b, h, rows):
    st, ref = oracle.forward_rows(inp["q"][b, h], inp["k"][b, h], inp["u"][b, h],
                                  inp["theta"][b, h], inp["v"][b, h], *sw, rows=rows)
    assert st == oracle.OK, st
    return ref


def rel_err(got, ref):
    return float(np.abs(got - ref).max() / (np.abs(ref).max() + 1e-6))


def sample_rows(n, rng, extra=24):
    fixed = [0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 129, 255, 256, n // 2, n - 129, n - 128,
             n - 65, n - 64, n - 2, n - 1]
    rnd = rng.integers(0, n, size=extra).tolist()
    return np.array(sorted({r for r in fixed + rnd if 0 <= r < n}), dtype=np.int64)


def compare_sampled(inp, sw, got, heads, rows):
    """Worst parity metric over the sampled heads (all share the max|O| of the
    compared set)."""
    refs, gots = [], []
    for b, h in heads:
        refs.append(oracle_rows(inp, sw, b, h, rows))
        gots.append(got[b, h][rows])
    return rel_err(np.stack(gots), np.stack(refs))


def compare_full(inp, sw, got):
    B, H, n = inp["u"].shape
    rows = np.arange(n)
    return compare_sampled(inp, sw, got, [(b, h) for b in range(B) for h in range(H)], rows)
