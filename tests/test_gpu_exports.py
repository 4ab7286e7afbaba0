"""Parity of the materialising exports with the fp64 oracle, through the C ABI.

resolvent_path_product follows the "Resolvent Operator" page's path_product
(Rust API) in the order the page fixes (k = i down to j + 1, no fused
multiply-adds), so it is compared with ``oracle.path_product`` bit for bit.

resolvent_operator writes W_ij = G_ij e^{qk s_ij} / Z_i^beta (section
"Object") in float32; the reference is ``oracle.operator`` per head.
Tolerance, from the arithmetic: float32 logits (a few 2^-24 of
sum_e |q_e k_e| |c|), exp2 of them, gate scans in f64 rounded to float once
and combined by two float32 complex products, and a normaliser summed per
lane over its keys (one per 64-key tile, at most n/64 terms) and then over the
64 keys' lanes in a tree: a few 1e-6 of the largest weight, held to the fp32
bar 1e-4 of max |dW| / (max |W| + 1e-6) per head.  Entries the definition makes exactly zero (above the diagonal,
behind a closed gate) are checked to be exactly zero.
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
TOL_OP = 1e-4


def announce(*a):
    print("case:", *a, flush=True)


def gates_of(inp, g):
    B, H, n = inp["u"].shape
    a = np.zeros((B, H, n), dtype=np.complex128)
    for b in range(B):
        for h in range(H):
            st, a[b, h] = oracle.gates(inp["u"][b, h], inp["theta"][b, h], g)
            assert st == oracle.OK
    return a


def gpu_path_product(a):
    ar = torch.from_numpy(np.ascontiguousarray(a.real)).to(DEV)
    ai = torch.from_numpy(np.ascontiguousarray(a.imag)).to(DEV)
    g_re, g_im = binding.resolvent_path_product(ar, ai)
    torch.cuda.synchronize()
    return g_re.cpu().numpy(), g_im.cpu().numpy()


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 130, 257])
def test_path_product_bitwise(n):
    announce(f"path_product n={n}")
    inp = inputs.draw(1, 3, n, 64, seed=300 + n, u_range=(0.0, 1.0))
    a = gates_of(inp, 0.7)[0]  # [3, n]
    g_re, g_im = gpu_path_product(a)
    assert g_re.shape == (3, n, n)
    for h in range(3):
        ref = oracle.path_product(a[h])
        assert np.array_equal(g_re[h], ref.real), h
        assert np.array_equal(g_im[h], ref.imag), h


def test_path_product_special_gates():
    """Closed gates zero everything behind them exactly; unit phases keep
    |G| = 1; a_0 is never read (a NaN there changes nothing)."""
    announce("path_product special gates")
    n = 150
    rng = np.random.default_rng(5)
    a = np.exp(1j * rng.uniform(-np.pi, np.pi, size=n))
    a[[10, 77]] = 0.0
    a[0] = np.nan
    g_re, g_im = gpu_path_product(a[None])
    G = g_re[0] + 1j * g_im[0]
    ref = oracle.path_product(a)
    assert np.array_equal(G.real, ref.real) and np.array_equal(G.imag, ref.imag)
    assert np.all(G[77:, :77] == 0) and np.all(G[10:, :10] == 0)
    assert np.all(np.triu(G, 1) == 0) and np.all(np.diag(G) == 1)
    assert np.allclose(np.abs(G[78:, 78:][np.tril_indices(n - 78)]), 1.0, atol=1e-12)


def gpu_operator(inp, sw):
    t = inputs.as_torch(inp, DEV)
    w_re, w_im = binding.resolvent_operator(t["q"], t["k"], t["u"], t["theta"], *sw)
    return w_re.double().cpu().numpy() + 1j * w_im.double().cpu().numpy()


def operator_err(inp, sw, W):
    B, H, _ = inp["u"].shape
    worst = 0.0
    for b in range(B):
        for h in range(H):
            st, ref = oracle.operator(inp["q"][b, h], inp["k"][b, h], inp["u"][b, h],
                                      inp["theta"][b, h], *sw)
            assert st == oracle.OK
            assert np.all(np.triu(W[b, h], 1) == 0)  # causal: exactly zero
            worst = max(worst, gu.rel_err(W[b, h], ref))
    return worst


@pytest.mark.parametrize("n", [1, 2, 64, 65, 200, 300])
@pytest.mark.parametrize("d,qdt", [(64, inputs.BF16), (128, inputs.BF16), (128, inputs.F32)])
def test_operator_shapes(n, d, qdt):
    announce(f"operator n={n} d={d} qk dtype {qdt}")
    inp = inputs.draw(1, 2, n, d, seed=n + d, qk_dtype=qdt, u_range=(0.6, 1.0))
    W = gpu_operator(inp, (1, 1, 1))
    assert W.shape == (1, 2, n, n)
    err = operator_err(inp, (1, 1, 1), W)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_OP


@pytest.mark.parametrize("B,H,n,d,qdt,seed", [(1, 1, 1000, 128, inputs.BF16, 51),
                                               (1, 3, 700, 64, inputs.F32, 52),
                                               (2, 1, 1500, 64, inputs.BF16, 53)])
def test_operator_many_tiles(B, H, n, d, qdt, seed):
    """Rows that span many 64-key tiles (the carried product across tiles),
    a ragged last block, and several heads per launch."""
    announce(f"operator B={B} H={H} n={n} d={d} qk dtype {qdt}")
    inp = inputs.draw(B, H, n, d, seed=seed, qk_dtype=qdt, u_range=(0.97, 1.0),
                      theta_range=(-0.3, 0.3))
    W = gpu_operator(inp, (1, 1, 1))
    err = operator_err(inp, (1, 1, 1), W)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_OP


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
@pytest.mark.parametrize("qk", [0.0, 1.0])
@pytest.mark.parametrize("g", [0.0, 0.5, 1.0])
def test_operator_switches(beta, qk, g):
    sw = (beta, qk, g)
    announce(f"operator switches {sw}")
    inp = inputs.draw(1, 2, 180, 64, seed=4, qk_scale=0.3, u_range=(0.5, 1.0))
    W = gpu_operator(inp, sw)
    err = operator_err(inp, sw, W)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_OP


def test_operator_closed_gates_and_readout():
    """Exact-masking gates: W_ij is exactly 0 behind a closed gate; and the
    readout W V of the export equals the hot path's output (fp32 path)."""
    announce("operator closed gates, readout vs forward")
    inp = inputs.make_config(4, n=400, H=2)
    W = gpu_operator(inp, (1, 1, 1))
    err = operator_err(inp, (1, 1, 1), W)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_OP
    closed = inp["u"] == 0.0
    for b, h in [(0, 0), (0, 1)]:
        ks = np.nonzero(closed[b, h])[0]
        for k in ks:
            if k > 0:
                assert np.all(W[b, h, k:, :k] == 0)
    inp32 = inputs.draw(1, 2, 333, 64, seed=8, qk_dtype=inputs.F32, v_dtype=inputs.F32,
                        u_range=(0.7, 1.0))
    W32 = gpu_operator(inp32, (0.5, 1, 1))
    O = gu.gpu_forward(inp32, (0.5, 1, 1))
    WV = W32 @ inp32["v"].astype(np.float64)
    diff = gu.rel_err(WV, O)
    print(f"  W V vs resolvent_forward: rel diff {diff:.3e}")
    assert diff <= gu.TOL_F32


def test_operator_refusals():
    announce("operator refusals")
    inp = inputs.draw(1, 1, 100, 64, seed=2)
    t = inputs.as_torch(inp, DEV)
    for name, where in (("q", (0, 0, 50, 3)), ("k", (0, 0, 0, 0)), ("u", (0, 0, 99)),
                        ("theta", (0, 0, 7))):
        bad = t[name].clone()
        bad[where] = float("nan")
        args = dict(t)
        args[name] = bad
        with pytest.raises(binding.ResolventError) as e:
            binding.resolvent_operator(args["q"], args["k"], args["u"], args["theta"], 1, 1, 1)
        assert e.value.status == binding.Status.NONFINITE, name
    binding.resolvent_operator(t["q"], t["k"], t["u"], t["theta"], 1, 1, 1)


def test_operator_overflow_at_beta_zero():
    """an_overflowing_logit_never_becomes_nan on the export: at beta = 0 the
    weights whose logits pass the float32 range read +inf exactly where the
    oracle's do, every other entry matches the oracle, the imaginary part (g = 0:
    exactly zero lanes of G) stays 0, and no entry is NaN."""
    announce("operator overflow at beta = 0")
    n, d = 200, 64
    inp = inputs.draw(1, 1, n, d, seed=93, qk_dtype=inputs.F32)
    inp["q"][0, 0, 120:] = np.abs(inp["q"][0, 0, 120:]) * 40.0
    inp["k"][0, 0, 120:] = np.abs(inp["k"][0, 0, 120:]) * 40.0
    sw = (0, 1, 0)
    W = gpu_operator(inp, sw)[0, 0]
    st, ref = oracle.operator(inp["q"][0, 0], inp["k"][0, 0], inp["u"][0, 0],
                              inp["theta"][0, 0], *sw)
    assert st == oracle.OK
    assert not np.isnan(W.real).any() and not np.isnan(W.imag).any()
    assert np.all(W.imag == 0)
    big = np.isinf(ref.real)
    assert big.any()
    # float32 overflows earlier than f64: every oracle inf is an inf here, and
    # an entry that is inf only here has a float32-overflowing weight
    assert np.all(np.isposinf(W.real[big]))
    fin = np.isfinite(W.real)
    assert np.all(ref.real[~fin] > 3.0e38)
    # the finite weights here reach 1e38: their float32 logits near 88 carry an
    # absolute rounding error of a few 1e-4 (64-term dot products of entries
    # near 1e2), so they are held to the bf16 bound, as in the forward's large-
    # logit test
    assert gu.rel_err(W[fin & ~big], ref[fin & ~big]) <= gu.TOL_BF16
