"""resolvent_forward_noalloc (the entry point whose workspace is the library's
fixed device scratch) against resolvent_forward on the same inputs: calls in a
row, each smaller than the one before, must give bitwise the outputs of the
entry point that takes a workspace, and those stay within the parity
tolerance of the oracle on sampled rows.  Collected last on purpose: the
scratch array must also serve after every other test has run."""
import numpy as np
import pytest

from gated_causal_attention_amd import binding, inputs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

# (B, H, n, d, qk dtype, switches, seed): the first fills 36.6 of the 64 MiB;
# the later ones are smaller, ragged, and change d and the switches
CALLS = [
    (1, 16, 8192, 128, inputs.BF16, (1.0, 1.0, 1.0), 41),
    (1, 2, 1000, 64, inputs.BF16, (0.5, 1.0, 1.0), 42),
    (1, 1, 300, 128, inputs.F32, (1.0, 1.0, 1.0), 43),
]


def _run_both(B, H, n, d, dt, sw, seed):
    import torch

    dev = torch.device("cuda:0")
    inp = inputs.draw(B, H, n, d, seed, qk_dtype=dt, v_dtype=dt, u_range=(0.95, 1.0),
                      theta_range=(-0.05, 0.05))
    t = inputs.as_torch(inp, dev)
    o_re = torch.full((B, H, n, d), float("nan"), device=dev, dtype=torch.float32)
    o_im = torch.full_like(o_re, float("nan"))
    status = torch.full((1,), -1, device=dev, dtype=torch.int32)
    binding.resolvent_forward_noalloc(t["q"], t["k"], t["u"], t["theta"], t["v"], *sw,
                                      o_re=o_re, o_im=o_im, status=status)
    r_re, r_im = binding.resolvent_forward(t["q"], t["k"], t["u"], t["theta"], t["v"], *sw)
    return inp, o_re, o_im, r_re, r_im


def test_noalloc_matches_workspace_entry_point():
    assert binding.resolvent_noalloc_scratch_bytes() == 64 << 20
    rng = np.random.default_rng(7)
    for B, H, n, d, dt, sw, seed in CALLS:
        print(f"noalloc call B={B} H={H} n={n} d={d} dtype={dt} switches={sw}", flush=True)
        code = binding.BF16 if dt == inputs.BF16 else binding.F32
        assert binding.resolvent_workspace_bytes(B, H, n, d, code, code) <= 64 << 20
        inp, o_re, o_im, r_re, r_im = _run_both(B, H, n, d, dt, sw, seed)
        assert bool((o_re == r_re).all()) and bool((o_im == r_im).all())
        got = o_re.double().cpu().numpy() + 1j * o_im.double().cpu().numpy()
        rows = gu.sample_rows(n, rng, extra=8)
        heads = [(0, 0), (B - 1, H - 1)]
        err = gu.compare_sampled(inp, sw, got, heads, rows)
        assert err <= gu.tol_for(inp), err


def test_noalloc_rejects_beyond_scratch():
    import torch

    dev = torch.device("cuda:0")
    B, H, n, d = 4, 16, 65536, 128
    assert binding.resolvent_workspace_bytes(B, H, n, d) > 64 << 20
    # a too-large problem is refused on the host before any pointer is used,
    # so small stand-in buffers suffice
    small = torch.zeros(16, device=dev, dtype=torch.float32)
    status = torch.zeros(1, device=dev, dtype=torch.int32)
    lib = binding._load()
    rc = lib.resolvent_forward_noalloc(
        small.data_ptr(), small.data_ptr(), small.data_ptr(), small.data_ptr(),
        small.data_ptr(), 1.0, 1.0, 1.0, B, H, n, d, binding.BF16, binding.BF16,
        small.data_ptr(), small.data_ptr(), status.data_ptr(), None)
    assert rc == binding.Status.TOO_LARGE
