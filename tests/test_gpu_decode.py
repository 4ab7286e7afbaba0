"""Parity of the decode step (resolvent_decode) and of the chain corner's
one-step update (resolvent_chain_step) with the fp64 oracle, through the C ABI.

resolvent_decode's result is the last row, i = n-1, of the head's readout
("Resolvent Operator" page, section "Object"), with query head h reading k/v
head h / (H / Hkv) as decodeGQA does on the Op Specs page; the oracle's
reference is ``oracle.forward_rows(..., rows=[n-1])`` on the same inputs.

Tolerance, from the arithmetic: the decode path keeps every weight in
float32 (no bf16 rounding), so it is held to the fp32 bar 1e-4 of
max |dO| / (max |O| + 1e-6) at every dtype.  Per key the float32 logit carries
a relative error of a few 2^-24 times sum_e |q_e k_e| |c| (a few 1e-6 in
log2 units for N(0,1) inputs at d = 128), exp2 turns that into the same
relative error of the weight, the gate products add a few ulps, and the sums
run at most 64 + 32 terms deep in float32 (a lane's rows of one chunk, then
the chunk merge): about 1e-5 of the summed magnitudes, which stays under
1e-4 of max |O| while the readout does not cancel by more than ~10x.
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
TOL_DEC = 1e-4


def announce(*a):
    print("case:", *a, flush=True)


def decode_inputs(B, H, Hkv, n, d, dv, seed, qk_dtype=inputs.BF16, v_dtype=inputs.BF16,
                  u_range=(0.5, 1.0), qk_scale=1.0, gates="uniform"):
    """Seeded draws of the forward's recipe; the decode query is q[:, :, n-1]."""
    inp = inputs.draw(B, H, n, d, seed, qk_dtype=qk_dtype, v_dtype=v_dtype, dv=dv,
                      u_range=u_range, qk_scale=qk_scale, gates=gates)
    inp["k"] = np.ascontiguousarray(inp["k"][:, :Hkv])
    inp["v"] = np.ascontiguousarray(inp["v"][:, :Hkv])
    inp["Hkv"] = Hkv
    return inp


def gpu_decode(inp, sw, cap=None):
    """Run resolvent_decode on the draws; with ``cap`` the caches hold cap
    positions per head, of which the first n are the draws."""
    t = inputs.as_torch(inp, DEV)
    n = inp["u"].shape[2]
    q = t["q"][:, :, n - 1].contiguous()
    k, v, u, th = t["k"], t["v"], t["u"], t["theta"]
    if cap is not None and cap > n:
        def grow(x):
            shape = list(x.shape)
            shape[2] = cap
            y = torch.full(shape, float("nan"), device=DEV, dtype=x.dtype)
            y[:, :, :n] = x
            return y
        k, v, u, th = grow(k), grow(v), grow(u), grow(th)
    o_re, o_im = binding.resolvent_decode(q, k, u, th, v, *sw, n=n)
    return o_re.double().cpu().numpy() + 1j * o_im.double().cpu().numpy()


def oracle_decode(inp, sw, heads=None):
    B, H, n = inp["u"].shape
    group = H // inp["Hkv"]
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    out = []
    for b, h in heads:
        st, ref = oracle.forward_rows(inp["q"][b, h], inp["k"][b, h // group], inp["u"][b, h],
                                      inp["theta"][b, h], inp["v"][b, h // group], *sw,
                                      rows=[n - 1])
        assert st == oracle.OK
        out.append(ref[0])
    return np.stack(out)


def decode_err(inp, sw, got, heads=None):
    B, H, _ = inp["u"].shape
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_decode(inp, sw, heads)
    return gu.rel_err(np.stack([got[b, h] for b, h in heads]), ref)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 200, 256, 257, 520, 1100])
def test_decode_lengths(n):
    """Ragged and tile-aligned lengths, one and several chunks of 4 key tiles."""
    announce(f"decode bf16 d=128 dv=128 H=4 Hkv=4 n={n}")
    inp = decode_inputs(2, 4, 4, n, 128, 128, seed=40 + n)
    got = gpu_decode(inp, (1, 1, 1))
    err = decode_err(inp, (1, 1, 1), got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_DEC


@pytest.mark.parametrize("d,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtypes", ["bf16", "bf16-f32v", "f32"])
@pytest.mark.parametrize("Hkv", [4, 1])
def test_decode_shapes_dtypes_groups(d, dv, dtypes, Hkv):
    qdt = inputs.F32 if dtypes == "f32" else inputs.BF16
    vdt = inputs.BF16 if dtypes == "bf16" else inputs.F32
    announce(f"decode {dtypes} d={d} dv={dv} H=4 Hkv={Hkv} n=333")
    inp = decode_inputs(1, 4, Hkv, 333, d, dv, seed=d + dv + Hkv, qk_dtype=qdt, v_dtype=vdt,
                        u_range=(0.9, 1.0))
    got = gpu_decode(inp, (1, 1, 1))
    assert got.shape == (1, 4, dv)
    err = decode_err(inp, (1, 1, 1), got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_DEC


@pytest.mark.parametrize("beta", [0.0, 0.5, 1.0])
@pytest.mark.parametrize("qk", [0.0, 1.0])
@pytest.mark.parametrize("g", [0.0, 1.0, 0.5])
def test_decode_switches(beta, qk, g):
    """The switch sweep, q,k scaled by 0.3 as in the batch-scale workload so
    that the unnormalised corner stays in range."""
    sw = (beta, qk, g)
    announce(f"decode switches {sw}")
    inp = decode_inputs(1, 4, 2, 700, 128, 128, seed=9, qk_scale=0.3, u_range=(0.5, 1.0))
    got = gpu_decode(inp, sw)
    err = decode_err(inp, sw, got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_DEC


def test_decode_cache_capacity():
    """Caches allocated for more positions than are filled: the unfilled tail
    (NaN here) is never read."""
    announce("decode with cap > n")
    inp = decode_inputs(2, 4, 2, 300, 64, 128, seed=17)
    got = gpu_decode(inp, (1, 1, 1), cap=389)
    assert np.all(np.isfinite(got))
    err = decode_err(inp, (1, 1, 1), got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_DEC


def test_decode_equals_forward_last_row():
    """resolvent_decode == row n-1 of resolvent_forward_grouped: on the fp32
    path to 1e-4; on the bf16 path the forward rounds its weights to bf16, so
    to that path's 2e-2."""
    announce("decode vs forward's last row")
    for qdt, tol in ((inputs.F32, gu.TOL_F32), (inputs.BF16, gu.TOL_BF16)):
        inp = decode_inputs(1, 4, 2, 777, 128, 128, seed=5, qk_dtype=qdt,
                            v_dtype=inputs.F32 if qdt == inputs.F32 else inputs.BF16)
        t = inputs.as_torch(inp, DEV)
        f_re, f_im = binding.resolvent_forward_grouped(t["q"], t["k"], t["u"], t["theta"],
                                                       t["v"], 1, 1, 1)
        fwd = (f_re[:, :, -1].double() + 1j * f_im[:, :, -1].double()).cpu().numpy()
        got = gpu_decode(inp, (1, 1, 1))
        err = gu.rel_err(got, fwd)
        print(f"  qk dtype {qdt}: rel diff {err:.3e} (tol {tol})")
        assert err <= tol


def test_decode_closed_gates():
    """Gates from {-1, 0, +1} (the exact-masking workload's recipe): a closed
    gate at k > j removes key j from the last row exactly; compared with the
    oracle, and the result does not change when every key before the last
    closed gate is replaced by garbage."""
    announce("decode with closed gates")
    inp = inputs.make_config(4, n=4096, H=4)
    inp["Hkv"] = 4
    got = gpu_decode(inp, (1, 1, 1))
    err = decode_err(inp, (1, 1, 1), got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_DEC
    closed = inp["u"] == 0.0
    inp2 = dict(inp)
    inp2["k"], inp2["v"] = inp["k"].copy(), inp["v"].copy()
    for b in range(closed.shape[0]):
        for h in range(closed.shape[1]):
            ks = np.nonzero(closed[b, h])[0]
            last = ks.max()
            assert last > 0
            inp2["k"][b, h, :last] = inp["k"][b, h, :last][::-1]
            inp2["v"][b, h, :last] = -inp["v"][b, h, :last]
    got2 = gpu_decode(inp2, (1, 1, 1))
    assert np.array_equal(got, got2)


def test_decode_headline_shape():
    """B=4, H=16, n=8192, d=128 (the headline workload's recipe), every head."""
    announce("decode B=4 H=16 n=8192 d=128")
    inp = inputs.make_config(3)
    inp["Hkv"] = inp["k"].shape[1]
    got = gpu_decode(inp, (1, 1, 1))
    assert np.all(np.isfinite(got))
    err = decode_err(inp, (1, 1, 1), got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_DEC


@pytest.mark.parametrize("n,dv", [(20000, 64), (8192, 128), (16384, 64), (8193, 128)])
def test_decode_merge_paths(n, dv):
    """Heads of up to 32 (dv = 128) or 64 (dv = 64) chunks take the one-trip
    merge, longer ones the general merge: both sides of each boundary."""
    announce(f"decode merge path n={n} dv={dv}")
    inp = decode_inputs(1, 2, 1, n, 128, dv, seed=n + dv, u_range=(0.995, 1.0), qk_scale=0.3)
    got = gpu_decode(inp, (1, 1, 1))
    err = decode_err(inp, (1, 1, 1), got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_DEC


def test_decode_long_cache():
    """n = 32768 with slowly decaying gates (u in (0.999, 1)): far keys keep
    weight, so the chunks' partial sums and their merge all matter."""
    announce("decode B=1 H=4 n=32768 d=128, u in (0.999, 1)")
    inp = decode_inputs(1, 4, 2, 32768, 128, 128, seed=77, u_range=(0.999, 1.0),
                        qk_scale=0.3)
    got = gpu_decode(inp, (1, 1, 1))
    err = decode_err(inp, (1, 1, 1), got)
    print(f"  rel err {err:.3e}")
    assert err <= TOL_DEC


def test_decode_overflow_at_beta_zero():
    """an_overflowing_logit_never_becomes_nan on a decode step: at beta = 0 and
    g = 0 a query whose logits pass the float32 range reads +inf (all values
    positive, so no inf - inf), and the imaginary part stays exactly 0."""
    announce("decode overflow at beta = 0")
    n = 300
    inp = decode_inputs(1, 2, 2, n, 64, 64, seed=95, qk_dtype=inputs.F32, v_dtype=inputs.F32)
    inp["v"] = np.abs(inp["v"]) + 0.5
    inp["q"][0, 1] = np.abs(inp["q"][0, 1]) * 40.0
    inp["k"][0, 1] = np.abs(inp["k"][0, 1]) * 40.0
    sw = (0, 1, 0)
    got = gpu_decode(inp, sw)
    ref = oracle_decode(inp, sw)
    assert not np.isnan(got.real).any() and not np.isnan(got.imag).any()
    assert np.all(got.imag == 0)
    assert np.isinf(ref[1].real).all() and np.all(np.isposinf(got[0, 1].real))
    assert gu.rel_err(got[0, 0], ref[0]) <= TOL_DEC


def test_decode_refusals_and_empty():
    announce("decode refusals")
    inp = decode_inputs(1, 2, 1, 300, 64, 64, seed=3)
    t = inputs.as_torch(inp, DEV)
    q = t["q"][:, :, -1].contiguous()

    def run(**over):
        a = dict(q=q, k=t["k"], u=t["u"], theta=t["theta"], v=t["v"])
        a.update(over)
        return binding.resolvent_decode(a["q"], a["k"], a["u"], a["theta"], a["v"], 1, 1, 1)

    for name, where in (("q", (0, 1, 5)), ("k", (0, 0, 0, 3)), ("u", (0, 1, 0)),
                        ("theta", (0, 0, 299))):
        src = {"q": q, "k": t["k"], "u": t["u"], "theta": t["theta"]}[name]
        bad = src.clone()
        bad[where] = float("nan")
        with pytest.raises(binding.ResolventError) as e:
            run(**{name: bad})
        assert e.value.status == binding.Status.NONFINITE, name
    big = t["k"].clone()
    big[0, 0, 7] = 1e38  # finite keys whose logit (64e38 c with q = 1) overflows float32
    ones = torch.ones_like(q)
    run(q=ones)  # the query of ones alone is accepted
    with pytest.raises(binding.ResolventError) as e:
        run(q=ones, k=big)
    assert e.value.status == binding.Status.NONFINITE
    run()  # the clean inputs still pass after the refusals
    o_re, _ = binding.resolvent_decode(q, t["k"][:, :, :0].contiguous(), t["u"][:, :, :0],
                                       t["theta"][:, :, :0], t["v"][:, :, :0].contiguous(),
                                       1, 1, 1)
    assert o_re.shape == (1, 2, 64)


def chain_oracle(inp, g):
    B, H, n = inp["u"].shape
    dv = inp["v"].shape[-1]
    out = np.zeros((B, H, n, dv), dtype=np.complex128)
    for b in range(B):
        for h in range(H):
            st, a = oracle.gates(inp["u"][b, h], inp["theta"][b, h], g)
            assert st == oracle.OK
            for c in range(dv):
                out[b, h, :, c] = oracle.chain(a, inp["v"][b, h, :, c], y0_from_b0=True)
    return out


@pytest.mark.parametrize("v_dtype,g", [(inputs.F32, 1.0), (inputs.BF16, 0.5)])
def test_chain_step_walks_the_chain(v_dtype, g):
    """Starting from y = 0, n calls of resolvent_chain_step give the chain
    corner's readout O_i after step i (section "The path-product corner is a
    resolvent"); every step is compared with the oracle's chain."""
    announce(f"chain step, v dtype {v_dtype}, g={g}")
    n = 150
    inp = inputs.draw(2, 3, n, 64, seed=12, v_dtype=v_dtype, dv=64, u_range=(0.8, 1.0))
    t = inputs.as_torch(inp, DEV)
    ref = chain_oracle(inp, g)
    y_re = torch.zeros((2, 3, 64), device=DEV)
    y_im = torch.zeros((2, 3, 64), device=DEV)
    worst = 0.0
    for i in range(n):
        binding.resolvent_chain_step(y_re, y_im, t["u"][:, :, i].contiguous(),
                                     t["theta"][:, :, i].contiguous(),
                                     t["v"][:, :, i].contiguous(), g, check=(i == n - 1))
        got = y_re.double().cpu().numpy() + 1j * y_im.double().cpu().numpy()
        worst = max(worst, gu.rel_err(got, ref[:, :, i]))
    print(f"  worst rel err over the steps {worst:.3e}")
    assert worst <= TOL_DEC


def test_chain_step_refusal_keeps_the_state():
    announce("chain step refusal")
    y_re = torch.ones((1, 2, 64), device=DEV)
    y_im = torch.zeros((1, 2, 64), device=DEV)
    u = torch.tensor([[0.5, float("nan")]], device=DEV)
    th = torch.zeros((1, 2), device=DEV)
    v = torch.ones((1, 2, 64), device=DEV)
    with pytest.raises(binding.ResolventError) as e:
        binding.resolvent_chain_step(y_re, y_im, u, th, v, 1.0)
    assert e.value.status == binding.Status.NONFINITE
    assert torch.all(y_re[0, 1] == 1) and torch.all(y_im[0, 1] == 0)  # refused head unchanged
    assert torch.all(y_re[0, 0] == 1.5)  # 0.5 * 1 + 1
