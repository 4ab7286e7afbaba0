"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test cites the passage of the "Resolvent Operator" page (teerth.dev,
Aether-Lang/integrated/resolvent) -- or of the "Op Specs" page (The Formal Era)
or the proof page "A position-only causal softmax head is a causal
convolution divided by a prefix normalizer" (proofs.blah.dev) -- that fixes the
expected value.  None of them re-types the oracle's own evaluation: each
compares against a brute force in 50-digit arithmetic, a library routine, a
closed form, a different formulation (the chain recurrence, the resolvent
inverse, a convolution) or an invariant.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests import brute

rng_global = np.random.default_rng(12345)


def rand_head(rng, n, d, dv=None, u_lo=0.0, u_hi=1.0, th=3.0, scale=1.0):
    dv = d if dv is None else dv
    q = rng.standard_normal((n, d)) * scale
    k = rng.standard_normal((n, d)) * scale
    v = rng.standard_normal((n, dv))
    u = rng.uniform(u_lo, u_hi, n)
    theta = rng.uniform(-th, th, n)
    return q, k, v, u, theta


def W_of(q, k, u, theta, beta, qk, g):
    st, W = oracle.operator(q, k, u, theta, beta, qk, g)
    assert st == oracle.OK
    return W


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("n,d", [(1, 1), (2, 3), (3, 2), (5, 4), (8, 3)])
def test_brute_force_definition(n, d):
    """Section "Object": the literal definition in 50 digits (dense Z^beta,
    ascending products) agrees with the oracle to 1e-13 on a switch grid that
    includes interior and extreme values and gates that the clamp cuts."""
    rng = np.random.default_rng(100 + n * 10 + d)
    q, k, v, _, _ = rand_head(rng, n, d)
    u = rng.uniform(-0.5, 1.5, n)
    theta = rng.uniform(-4, 4, n)
    grid = [(1, 1, 0), (0, 1, 0), (0, 0, 1), (0.5, 0.7, 0.5), (0.3, -1.3, 1.4),
            (1.7, 0.4, -0.3), (1, 1, 1), (0, 0, 0)]
    for beta, qk, g in grid:
        W = W_of(q, k, u, theta, beta, qk, g)
        Wb = brute.weights(q.tolist(), k.tolist(), u.tolist(), theta.tolist(), beta, qk, g)
        Wb = np.array([[complex(x) for x in row] for row in Wb])
        scale = max(1.0, np.abs(Wb).max())
        assert np.abs(W - Wb).max() <= 1e-13 * scale, (beta, qk, g)
        st, O = oracle.forward_rows(q, k, u, theta, v, beta, qk, g, rows=np.arange(n))
        assert st == oracle.OK
        Ob = np.array([[complex(x) for x in row] for row in brute.readout(Wb.tolist(), v.tolist())])
        assert np.abs(O - Ob).max() <= 1e-13 * max(1.0, np.abs(Ob).max()), (beta, qk, g)
        # the Rust API's readout applied to the operator: the same rows
        Or = oracle.readout(W, v)
        assert np.abs(Or - Ob).max() <= 1e-13 * max(1.0, np.abs(Ob).max()), (beta, qk, g)
        assert np.abs(Or - O).max() <= 1e-13 * max(1.0, np.abs(O).max()), (beta, qk, g)


@pytest.mark.parametrize("n,dv", [(1, 1), (4, 7), (9, 2), (16, 16)])
def test_readout_is_causal_product(n, dv):
    """Sections "Rust API" (readout of W [seq, seq] and V [seq, value_dim])
    and "Object" (O_i sums W_ij V_j over j <= i only): for any complex W,
    including entries above the diagonal that the readout must ignore, the
    oracle's readout equals tril(W) V from numpy's matrix product, real and
    imaginary parts separately, to 1e-13."""
    rng = np.random.default_rng(900 + 10 * n + dv)
    W = rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))
    v = rng.standard_normal((n, dv))
    got = oracle.readout(W, v)
    want = np.tril(W) @ v
    assert got.shape == (n, dv)
    assert np.abs(got - want).max() <= 1e-13 * max(1.0, np.abs(want).max())
    # a change above the diagonal leaves the readout bitwise unchanged
    W2 = W + np.triu(rng.standard_normal((n, n)), 1)
    assert np.array_equal(oracle.readout(W2, v), got)


# ------------------------------------------------------------------- corners
def test_softmax_corner_is_library_softmax(page_values):
    """Corner (1,1,0) is causal softmax ("The three corners"; test
    the_softmax_corner_is_causal_softmax...): torch SDPA in fp64 with a causal
    mask; imaginary part exactly 0 at g = 0."""
    rng = np.random.default_rng(1)
    n, d = 37, 16
    q, k, v, u, theta = rand_head(rng, n, d)
    st, O = oracle.forward_rows(q, k, u, theta, v, 1, 1, 0, rows=np.arange(n))
    assert st == oracle.OK
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], is_causal=True)[0, 0].numpy()
    assert np.abs(O.real - ref).max() <= 10 * page_values["softmax_corner"]["tol"]
    assert np.all(O.imag == 0.0)
    W = W_of(q, k, u, theta, 1, 1, 0)
    assert np.all(W.imag == 0.0)


def test_kernel_corner_is_bare_exponential_bitwise():
    """Corner (0,1,0): W_ij = e^{s_ij} bitwise (test
    the_unnormalized_kernel_corner_is_the_bare_exponential_bitwise); s_ij is
    summed here in ascending order and divided by sqrt(d), exp from libm."""
    rng = np.random.default_rng(2)
    n, d = 12, 5
    q, k, v, u, theta = rand_head(rng, n, d)
    W = W_of(q, k, u, theta, 0, 1, 0)
    for i in range(n):
        for j in range(n):
            if j > i:
                assert W[i, j] == 0
                continue
            dot = 0.0
            for e in range(d):
                dot += float(q[i, e]) * float(k[j, e])
            assert W[i, j].real == math.exp(dot / math.sqrt(d))
            assert W[i, j].imag == 0.0
    st, O = oracle.forward_rows(q, k, u, theta, v, 0, 1, 0, rows=np.arange(n))
    ref = (np.exp(q @ k.T / np.sqrt(d)) * np.tril(np.ones((n, n)))) @ v
    assert np.abs(O.real - ref).max() <= 1e-12 * np.abs(ref).max()


def triple_loop_G(a):
    n = len(a)
    G = np.zeros((n, n), dtype=complex)
    for i in range(n):
        for j in range(i + 1):
            x = complex(1.0, 0.0)
            for kk in range(i, j, -1):
                x = x * complex(a[kk])
            G[i, j] = x
    return G


def test_path_product_corner_is_gate_product_bitwise():
    """Corner (0,0,1): W = G bitwise against a triple loop with closed and unit
    gates (test the_path_product_corner_is_the_gate_product_bitwise); the loop
    multiplies a_i, ..., a_{j+1} in the order the "Rust API" section fixes."""
    rng = np.random.default_rng(3)
    n, d = 14, 3
    q, k, v, u, theta = rand_head(rng, n, d)
    u[4] = 0.0
    u[9] = 1.0
    theta[9] = 0.0
    W = W_of(q, k, u, theta, 0, 0, 1)
    a = [complex(u[x] * math.cos(theta[x]), u[x] * math.sin(theta[x])) for x in range(n)]
    G = triple_loop_G(a)
    assert np.array_equal(W, G)
    assert np.array_equal(oracle.path_product(np.array(a)), G)


def test_corners_are_distinct(page_values):
    """corners_are_distinct: at g = 0, qk = 0, entry (1,0) is 1/2 at beta = 1
    and 1 at beta = 0; random inputs separate every pair of corners by > 0.5."""
    pv = page_values["corner_entry_1_0"]
    z = np.zeros((2, 1))
    u = np.array([0.3, 0.8])
    th = np.array([0.2, -1.0])
    assert W_of(z, z, u, th, 1, 0, 0)[1, 0] == pv["W10_beta1"]
    assert W_of(z, z, u, th, 0, 0, 0)[1, 0] == pv["W10_beta0"]
    rng = np.random.default_rng(4)
    q, k, v, u, theta = rand_head(rng, 16, 8)
    Ws = [W_of(q, k, u, theta, *c) for c in [(1, 1, 0), (0, 1, 0), (0, 0, 1)]]
    for x in range(3):
        for y in range(x + 1, 3):
            assert np.abs(Ws[x] - Ws[y]).max() > pv["random_pair_separation"]


# ---------------------------------------------------------- row sums / modulus
@pytest.mark.parametrize("qk,g", [(1, 0), (1, 1), (0.7, 0.5), (0, 1), (-2, 0.8)])
def test_beta_one_rows_sum_to_one(qk, g, page_values):
    """softmax_row_sum_one / beta_one_row_is_one: at beta = 1 the moduli of a
    row sum to 1 with gates on or off (reading: sum |W_ij| for complex gates,
    sum W_ij when every blended phase is 0)."""
    tol = page_values["row_sums"]["beta1_tol"]
    rng = np.random.default_rng(5)
    q, k, v, u, theta = rand_head(rng, 20, 6)
    W = W_of(q, k, u, theta, 1, qk, g)
    assert np.abs(np.abs(W).sum(1) - 1).max() <= tol * 4
    W0 = W_of(q, k, u, np.zeros_like(theta), 1, qk, g)
    assert np.abs(W0.sum(1) - 1).max() <= tol * 4


def test_bare_row_sums_to_i_plus_one():
    """gate_zero_beta_zero_row_not_one: at (0,0,0) row i sums to exactly i+1."""
    rng = np.random.default_rng(6)
    n = 25
    q, k, v, u, theta = rand_head(rng, n, 4)
    W = W_of(q, k, u, theta, 0, 0, 0)
    for i in range(n):
        assert W[i].sum() == i + 1
    st, O = oracle.forward_rows(q, k, u, theta, np.ones((n, 1)), 0, 0, 0, rows=np.arange(n))
    assert np.array_equal(O[:, 0].real, np.arange(1, n + 1, dtype=float))


def test_modulus_is_product_of_magnitudes(page_values):
    """pathProd_abs: |G_ij| = prod m_k (1e-14), |G| <= 1, and |G_ij| = 1 exactly
    when every magnitude on the path is 1."""
    rng = np.random.default_rng(7)
    n = 30
    m = rng.uniform(0.2, 1.0, n)
    m[10:16] = 1.0
    th = rng.uniform(-3, 3, n)
    a = m * np.exp(1j * th)
    G = oracle.path_product(a)
    R = oracle.modulus(m)
    for i in range(n):
        for j in range(i + 1):
            ref = 1.0
            for kk in range(j + 1, i + 1):
                ref *= m[kk]
            assert abs(R[i, j] - ref) <= page_values["modulus"]["tol"] * max(ref, 1e-300)
            assert abs(abs(G[i, j]) - ref) <= page_values["modulus"]["tol"]
            assert abs(G[i, j]) <= 1 + 1e-15
    for i in range(10, 16):
        for j in range(9, i + 1):
            assert abs(abs(G[i, j]) - 1) <= 1e-15


@pytest.mark.parametrize("beta,qk,g", [(1, 1, 1), (0, 1, 1), (0, 0, 1), (0.5, 0.7, 0.5),
                                       (1, 0, 1), (2, -1, 0.7)])
def test_closed_gate_annihilates_exactly(beta, qk, g):
    """pathProd_eq_zero_iff / no_prefix_scan_represents_a_zero_gate: a closed
    gate (m_k = 0) makes every W_ij with j < k <= i exactly 0 under every
    switch setting with g != 0 (at g = 0 no gate is closed)."""
    rng = np.random.default_rng(8)
    n = 18
    q, k, v, u, theta = rand_head(rng, n, 5)
    if g != 1:
        u[7] = -(1 - g) / g  # lerp(1, u, g) = 0 exactly
        assert (1 - g) * 1 + g * u[7] == 0.0
    else:
        u[7] = 0.0
    W = W_of(q, k, u, theta, beta, qk, g)
    G = oracle.path_product(np.array([oracle.gate(*oracle.blend(u[x], theta[x], g))
                                      for x in range(n)]))
    for i in range(7, n):
        for j in range(7):
            assert W[i, j] == 0
            assert G[i, j] == 0
    assert np.all(W[7:, 7:].diagonal() != 0)


def test_bedm_values(page_values):
    """bedM_gate_exact: -1, 0, +1 are the gates (m,theta) = (1,pi), (0,0),
    (1,0); exact real parts, imaginary residue of sin(pi) below 1.3e-16."""
    pv = page_values["bedm"]
    for m, th, val in pv["gates_m_theta_value"]:
        th = math.pi if th == "pi" else th
        mm, tp = oracle.blend(m, th, 1.0)
        a = oracle.gate(mm, tp)
        assert a.real == val
        assert abs(a.imag) <= pv["imag_bound"]


def test_vector_gates_hold_the_page_values(page_values):
    """oracle.gates over a whole head: the bedM gates -1, 0, +1 (exact real
    parts, sin(pi) residue below 1.3e-16), the identity gate 1 at g = 0
    ("g = 0 removes the gates exactly"), and the refusal of a non-finite u,
    theta or g*theta."""
    pv = page_values["bedm"]
    us = [m for m, _, _ in pv["gates_m_theta_value"]] * 3
    ths = [math.pi if th == "pi" else th for _, th, _ in pv["gates_m_theta_value"]] * 3
    st, a = oracle.gates(us, ths, 1.0)
    assert st == oracle.OK
    assert list(a.real) == [val for _, _, val in pv["gates_m_theta_value"]] * 3
    assert np.abs(a.imag).max() <= pv["imag_bound"]
    st, a = oracle.gates(np.linspace(0, 1, 7), np.linspace(-3, 3, 7), 0.0)
    assert st == oracle.OK and np.all(a == 1.0)
    assert oracle.gates([0.5, float("nan")], [0.0, 0.0], 1.0)[0] == oracle.NONFINITE
    assert oracle.gates([0.5, 0.5], [0.0, float("inf")], 1.0)[0] == oracle.NONFINITE
    assert oracle.gates([0.5], [1e308], 1e10)[0] == oracle.NONFINITE  # g*theta overflows


def test_constant_phase_is_rope_kernel(page_values):
    """constant_phase_gate_is_rope / cumulative_phase_is_separable: unit gates of
    constant phase w give G_ij = e^{i w (i-j)} (Toeplitz, 1e-13); the readout
    of a ones channel is the geometric sum (1 - e^{iw(i+1)}) / (1 - e^{iw});
    any phase schedule gives e^{i(Theta_i - Theta_j)} with Theta the prefix sum."""
    tol = page_values["constant_phase"]["tol"]
    n, w = 40, 0.37
    z = np.zeros((n, 2))
    W = W_of(z, z, np.ones(n), np.full(n, w), 0, 0, 1)
    for i in range(n):
        for j in range(i + 1):
            assert abs(W[i, j] - np.exp(1j * w * (i - j))) <= tol
    st, O = oracle.forward_rows(z, z, np.ones(n), np.full(n, w), np.ones((n, 1)), 0, 0, 1,
                                rows=np.arange(n))
    idx = np.arange(n)
    geo = (1 - np.exp(1j * w * (idx + 1))) / (1 - np.exp(1j * w))
    assert np.abs(O[:, 0] - geo).max() <= tol * n
    rng = np.random.default_rng(9)
    th = rng.uniform(-2, 2, n)
    W = W_of(z, z, np.ones(n), th, 0, 0, 1)
    Theta = np.cumsum(th)
    for i in range(n):
        for j in range(i + 1):
            assert abs(W[i, j] - np.exp(1j * (Theta[i] - Theta[j]))) <= tol


def test_scalar_gates_commute_within_window(page_values):
    """PhaseH.scalar_gate_commutes: permuting real gates inside (p, r] leaves
    G_ij unchanged for windows containing them (1e-15) and bitwise for windows
    disjoint from them."""
    tol = page_values["commute"]["tol"]
    rng = np.random.default_rng(10)
    n, p, r = 24, 6, 15
    a = rng.uniform(0.3, 1.0, n) * rng.choice([-1.0, 1.0], n)
    perm = a.copy()
    perm[p + 1:r + 1] = rng.permutation(a[p + 1:r + 1])
    G1, G2 = oracle.path_product(a + 0j), oracle.path_product(perm + 0j)
    for i in range(n):
        for j in range(i + 1):
            if j <= p and i >= r:
                assert abs(G1[i, j] - G2[i, j]) <= tol * abs(G1[i, j]) + 1e-300
            elif i <= p or j >= r:
                assert G1[i, j] == G2[i, j]


def test_path_product_corner_is_chain_and_resolvent(page_values):
    """"The path-product corner is a resolvent": the readout at (0,0,1) is the
    chain y_i = a_i y_{i-1} + b_i (1e-12; b_0 = 0 as on the page, and the
    y_0 = b_0 variant), G (I - A) = I with A_{i,i-1} = a_i (1e-14, both sides),
    and beta = 1 breaks the chain (planted negative)."""
    pv = page_values["chain"]
    rng = np.random.default_rng(11)
    n = 50
    q, k, v, u, theta = rand_head(rng, n, 3, dv=4, u_lo=0.5)
    a = np.array([oracle.gate(*oracle.blend(u[x], theta[x], 1.0)) for x in range(n)])
    v[0, 0] = 0.0
    st, O = oracle.forward_rows(q, k, u, theta, v, 0, 0, 1, rows=np.arange(n))
    for c in range(4):
        y = [complex(v[0, c])]
        for i in range(1, n):
            y.append(a[i] * y[-1] + v[i, c])
        y = np.array(y)
        assert np.abs(O[:, c] - y).max() <= pv["chain_tol"]
        if c == 0:
            assert np.abs(oracle.chain(a, v[:, 0]) - y).max() <= pv["chain_tol"]
        assert np.abs(oracle.chain(a, v[:, c], y0_from_b0=True) - y).max() <= pv["chain_tol"]
    G = oracle.path_product(a)
    A = np.zeros((n, n), dtype=complex)
    for i in range(1, n):
        A[i, i - 1] = a[i]
    I = np.eye(n)
    assert np.abs(G @ (I - A) - I).max() <= pv["inverse_tol"]
    assert np.abs((I - A) @ G - I).max() <= pv["inverse_tol"]
    st, O1 = oracle.forward_rows(q, k, u, theta, v, 1, 0, 1, rows=np.arange(n))
    assert np.abs(O1 - O).max() > 1e-3


# ------------------------------------------------ causality / switches / edges
def test_future_never_moves_the_past():
    """perturbing_the_future_never_moves_the_past: rows <= t are bitwise
    unchanged when later q, k, v, u, theta change; W above the diagonal is 0."""
    rng = np.random.default_rng(12)
    n, t = 30, 17
    q, k, v, u, theta = rand_head(rng, n, 6)
    for sw in [(1, 1, 1), (0.5, 0.7, 0.5), (0, 1, 0), (0, 0, 1)]:
        st, O1 = oracle.forward_rows(q, k, u, theta, v, *sw, rows=np.arange(n))
        q2, k2, v2, u2, th2 = (x.copy() for x in (q, k, v, u, theta))
        for x in (q2, k2, v2, u2, th2):
            x[t + 1:] = rng.standard_normal(x[t + 1:].shape)
        st, O2 = oracle.forward_rows(q2, k2, u2, th2, v2, *sw, rows=np.arange(n))
        assert np.array_equal(O1[:t + 1], O2[:t + 1])
        W = W_of(q, k, u, theta, *sw)
        assert np.all(np.triu(W, 1) == 0)


def test_off_switch_deletes_its_term_exactly():
    """an_off_switch_deletes_its_term_exactly: g = 0 removes u and theta
    exactly (and leaves Im O = 0); qk = 0 removes q and k exactly, even when
    their dot product would overflow."""
    rng = np.random.default_rng(13)
    n = 20
    q, k, v, u, theta = rand_head(rng, n, 5)
    _, _, _, u2, th2 = rand_head(rng, n, 5)
    st, A = oracle.forward_rows(q, k, u, theta, v, 0.5, 0.8, 0, rows=np.arange(n))
    st, B = oracle.forward_rows(q, k, u2, th2, v, 0.5, 0.8, 0, rows=np.arange(n))
    assert np.array_equal(A, B) and np.all(A.imag == 0)
    big = np.full((n, 5), 1e200)
    st1, C = oracle.forward_rows(q, k, u, theta, v, 0.5, 0, 1, rows=np.arange(n))
    st2, D = oracle.forward_rows(big, -big, u, theta, v, 0.5, 0, 1, rows=np.arange(n))
    assert st1 == st2 == oracle.OK
    assert np.array_equal(C, D)


def test_large_logits_stay_finite_at_beta_one(page_values):
    """logits_of_ten_thousand_stay_finite_at_beta_one: with logits past 1e4
    the rows stay finite, stochastic to 1e-9 and equal to softmax (torch SDPA,
    fp64) to 1e-9."""
    pv = page_values["large_logits"]
    rng = np.random.default_rng(14)
    n, d = 16, 4
    q, k, v, u, theta = rand_head(rng, n, d)
    q *= 100.0
    k *= 100.0
    logits = q @ k.T / np.sqrt(d)
    assert np.abs(np.tril(logits)).max() > pv["logit_magnitude"]
    W = W_of(q, k, u, theta, 1, 1, 0)
    assert np.all(np.isfinite(W))
    assert np.abs(W.sum(1) - 1).max() <= pv["tol"]
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None], torch.from_numpy(k)[None, None],
        torch.from_numpy(v)[None, None], is_causal=True)[0, 0].numpy()
    st, O = oracle.forward_rows(q, k, u, theta, v, 1, 1, 0, rows=np.arange(n))
    assert np.abs(O.real - ref).max() <= pv["tol"]


def test_overflowing_logit_is_inf_never_nan(page_values):
    """an_overflowing_logit_never_becomes_nan: at beta = 0 a logit of 2e4 reads
    +inf; the zero imaginary lane (g = 0) stays 0 instead of 0*inf."""
    pv = page_values["overflow"]
    q = np.array([[pv["logit"]], [1.0]])
    k = np.array([[1.0], [0.5]])
    W = W_of(q, k, np.ones(2), np.zeros(2), pv["beta"], 1, 0)
    assert W[0, 0].real == math.inf and W[0, 0].imag == 0
    assert not np.any(np.isnan(W.real)) and not np.any(np.isnan(W.imag))


def test_non_finite_input_is_refused():
    """non_finite_input_is_refused: each non-finite class (q, k, u, theta,
    each switch), an overflowing g*theta and an overflowing logit are refused;
    index 0 of u and theta is checked although a_0 is never read; with qk = 0
    an overflowing dot product is accepted."""
    rng = np.random.default_rng(15)
    n, d = 6, 3
    q, k, v, u, theta = rand_head(rng, n, d)
    good = dict(q=q, k=k, u=u, theta=theta)

    def st_of(beta=1.0, qk=1.0, g=0.5, **over):
        args = {**good, **over}
        return oracle.forward_rows(args["q"], args["k"], args["u"], args["theta"], v,
                                   beta, qk, g, rows=np.arange(n))[0]

    assert st_of() == oracle.OK
    for name in ("q", "k", "u", "theta"):
        for bad in (np.nan, np.inf, -np.inf):
            x = good[name].copy()
            x.flat[0] = bad
            assert st_of(**{name: x}) == oracle.NONFINITE, (name, bad)
    for sw in ("beta", "qk", "g"):
        for bad in (np.nan, np.inf):
            assert st_of(**{sw: bad}) == oracle.NONFINITE
    assert st_of(g=1e300, theta=np.full(n, 1e10)) == oracle.NONFINITE
    assert st_of(qk=1e300, q=q * 1e10, k=k * 1e10) == oracle.NONFINITE
    big = np.full((n, d), 1e200)
    assert st_of(qk=0.0, q=big, k=big) == oracle.OK
    assert oracle.operator(q, k, u, theta, 1, 1, 0)[0] == oracle.OK


def test_empty_sequence_and_no_all_masked_row():
    """an_empty_sequence_is_empty_and_no_row_is_ever_all_masked: n = 0 gives
    an empty result; with every gate shut each row keeps only its own key, so W
    is I at beta = 1 and diag(e^{qk s_ii}) at beta = 0; head_dim = 0 with n > 0
    is a shape error."""
    e = np.zeros((0, 4))
    st, O = oracle.forward_rows(e, e, np.zeros(0), np.zeros(0), e, 1, 1, 1, rows=[])
    assert st == oracle.OK and O.shape == (0, 4)
    rng = np.random.default_rng(16)
    n = 9
    q, k, v, u, theta = rand_head(rng, n, 4)
    W = W_of(q, k, np.zeros(n), theta, 1, 1, 1)
    assert np.array_equal(W, np.eye(n))
    W0 = W_of(q, k, np.zeros(n), theta, 0, 1, 1)
    s = np.array([sum(q[i, e] * k[i, e] for e in range(4)) / 2.0 for i in range(n)])
    assert np.allclose(np.diag(W0).real, np.exp(s), rtol=1e-15, atol=0)
    assert np.all(W0 - np.diag(np.diag(W0)) == 0)
    st, _ = oracle.operator(np.zeros((3, 0)), np.zeros((3, 0)), np.ones(3), np.zeros(3), 1, 1, 1)
    assert st == oracle.BAD_SHAPE


# -------------------------------------------------------- derived identities
def test_beta_is_log_linear():
    """From "Object": O(beta) = O(0) Z^{-beta} with Z = O(0)/O(1) real,
    positive and the same for every channel of a row (pins interior beta from
    the corners)."""
    rng = np.random.default_rng(17)
    n = 24
    q, k, v, u, theta = rand_head(rng, n, 5, dv=3)
    rows = np.arange(n)
    O0 = oracle.forward_rows(q, k, u, theta, v, 0, 0.9, 0.6, rows=rows)[1]
    O1 = oracle.forward_rows(q, k, u, theta, v, 1, 0.9, 0.6, rows=rows)[1]
    Z = O0 / O1
    assert np.abs(Z.imag).max() <= 1e-12 * np.abs(Z).max()
    Zr = Z.real[:, :1]
    assert np.all(Zr > 0)
    assert np.abs(Z.real - Zr).max() <= 1e-11 * Zr.max()
    for b in (0.5, 0.3, 1.6):
        Ob = oracle.forward_rows(q, k, u, theta, v, b, 0.9, 0.6, rows=rows)[1]
        assert np.abs(Ob - O0 * Zr ** (-b)).max() <= 1e-12 * np.abs(Ob).max()


def test_qk_scales_the_query():
    """From "Object": the logit is qk * s_ij, so qk = c equals qk = 1 with the
    query scaled by c (up to rounding)."""
    rng = np.random.default_rng(18)
    n = 20
    q, k, v, u, theta = rand_head(rng, n, 5)
    for c in (0.4, -1.7, 3.0):
        A = oracle.forward_rows(q, k, u, theta, v, 0.7, c, 0.5, rows=np.arange(n))[1]
        B = oracle.forward_rows(q * c, k, u, theta, v, 0.7, 1, 0.5, rows=np.arange(n))[1]
        assert np.abs(A - B).max() <= 1e-12 * np.abs(A).max()


def test_g_enters_only_through_blend():
    """From "Object": (u, theta, g) gives the same head as the pre-blended gate
    u' = clamp(lerp(1, u, g), 0, 1), theta'' = g*theta at g = 1 -- bitwise,
    since lerp(1, u', 1) = u' exactly."""
    rng = np.random.default_rng(19)
    n = 20
    q, k, v, u, theta = rand_head(rng, n, 5, u_lo=-0.3, u_hi=1.4)
    g = 0.63
    ub = np.array([oracle.blend(u[x], theta[x], g)[0] for x in range(n)])
    tb = np.array([oracle.blend(u[x], theta[x], g)[1] for x in range(n)])
    A = oracle.forward_rows(q, k, u, theta, v, 0.4, 1.1, g, rows=np.arange(n))[1]
    B = oracle.forward_rows(q, k, ub, tb, v, 0.4, 1.1, 1.0, rows=np.arange(n))[1]
    assert np.array_equal(A, B)


def rope(x, pos, base=10000.0):
    """Op Specs, rope with rot = denom = D, active = D/2: rotate the pairs
    (i, i + D/2) by pos * invFreq(i), invFreq(i) = base^(-2i/D)."""
    D = x.shape[-1]
    half = D // 2
    out = x.copy()
    for i in range(half):
        ang = pos * base ** (-(2 * i) / D)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = x[i] * c - x[i + half] * s
        out[i + half] = x[i] * s + x[i + half] * c
    return out


def test_position_only_head_is_causal_convolution():
    """Proof page "A position-only causal softmax head is a causal convolution
    divided by a prefix normalizer": when the score depends only on i - j the
    beta = 1 output is sum_d e^{a(d)} v_{i-d} / sum_d e^{a(d)}.  Two heads of
    that kind: (a) qk = 0, g = 1 with a constant real gate r, score d*ln r, whose
    normaliser has the closed form (1 - r^{i+1})/(1 - r); (b) g = 0 with
    RoPE-rotated constant q, k (Op Specs, rope), score <q, R(-d) k>/sqrt(D)."""
    rng = np.random.default_rng(20)
    n, D, r = 33, 8, 0.8
    v = rng.standard_normal((n, 3))
    z = np.zeros((n, D))
    O = oracle.forward_rows(z, z, np.full(n, r), np.zeros(n), v, 1, 0, 1, rows=np.arange(n))[1]
    for i in range(n):
        num = sum(r ** dd * v[i - dd] for dd in range(i + 1))
        den = (1 - r ** (i + 1)) / (1 - r)
        assert np.abs(O[i] - num / den).max() <= 1e-13
    q0, k0 = rng.standard_normal(D), rng.standard_normal(D)
    q = np.stack([rope(q0, i) for i in range(n)])
    k = np.stack([rope(k0, j) for j in range(n)])
    O = oracle.forward_rows(q, k, np.ones(n), np.zeros(n), v, 1, 1, 0, rows=np.arange(n))[1]
    a = np.array([rope(k0, -dd) @ q0 / math.sqrt(D) for dd in range(n)])
    for i in range(n):
        w = np.exp(a[:i + 1])
        num = sum(w[dd] * v[i - dd] for dd in range(i + 1))
        assert np.abs(O[i] - num / w.sum()).max() <= 1e-12
        assert np.all(O[i].imag == 0)


def test_rows_subset_equals_full_forward():
    """The sampled-row entry point computes the same rows as the full one."""
    rng = np.random.default_rng(21)
    B, H, n, d = 2, 3, 17, 4
    q = rng.standard_normal((B, H, n, d))
    k = rng.standard_normal((B, H, n, d))
    v = rng.standard_normal((B, H, n, d))
    u = rng.uniform(0, 1, (B, H, n))
    th = rng.uniform(-3, 3, (B, H, n))
    st, O = oracle.forward(q, k, u, th, v, 0.5, 0.7, 0.5)
    assert st == oracle.OK
    rows = np.array([16, 0, 5])
    st, Or = oracle.forward_rows(q[1, 2], k[1, 2], u[1, 2], th[1, 2], v[1, 2], 0.5, 0.7, 0.5,
                                 rows=rows)
    assert np.array_equal(Or, O[1, 2][rows])
