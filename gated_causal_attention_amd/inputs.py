"""Seeded synthetic inputs for the resolvent head.

This module holds no arithmetic of the method: it only draws random numbers,
rounds them to the storage type of each workload and hands the same values to
the HIP path and to the fp64 oracle.  The pages measure nothing on a dataset,
so these draws stand in for the workloads (five shapes, see ``WORKLOADS``).

Draw order for a workload: q, k, v (``standard_normal(float32)`` over
[B, H, n, d], then scaled), then u, then theta ([B, H, n]), all from
``numpy.random.Generator(PCG64(seed))``.  bf16 storage is round-to-nearest-even
from the float32 draw (done by torch); the returned float32 arrays hold exactly
the stored values, so the oracle reads what the device reads.
"""
from dataclasses import dataclass, field

import numpy as np

BF16, F32 = "bf16", "f32"


@dataclass(frozen=True)
class Workload:
    """One synthetic workload: shape, storage types, value distributions."""

    idx: int
    B: int
    H: int
    n: int
    d: int
    qk_dtype: str
    v_dtype: str
    qk_scale: float
    gates: str  # "uniform" | "bedm"
    u_range: tuple = (0.0, 1.0)
    theta_range: tuple = (-np.pi, np.pi)  # (lo, hi); lo == hi means constant
    switches: tuple = field(default_factory=tuple)
    description: str = ""


WORKLOADS = {
    1: Workload(1, 1, 1, 256, 64, F32, F32, 1.0, "uniform", (0.0, 1.0), (-np.pi, np.pi),
                ((1, 1, 0), (0, 1, 0), (0, 0, 1), (0.5, 0.7, 0.5)),
                "single head, fp32; q,k scaled by 0.3 at the (0,1,0) corner"),
    2: Workload(2, 2, 8, 2048, 64, BF16, F32, 1.0, "uniform", (0.9, 1.0), (0.01, 0.01),
                ((1, 1, 1), (1, 1, 0.5)),
                "bf16 q,k, fp32 v, constant phase 0.01"),
    3: Workload(3, 4, 16, 8192, 128, BF16, BF16, 1.0, "uniform", (0.95, 1.0), (-0.05, 0.05),
                ((1, 1, 1),), "headline: B=4 H=16 n=8192 d=128 bf16"),
    4: Workload(4, 1, 16, 32768, 128, BF16, BF16, 1.0, "bedm", (0.0, 1.0), (0.0, 0.0),
                ((1, 1, 1),), "gates in {-1, 0, +1} with p = (0.05, 0.01, 0.94)"),
    5: Workload(5, 8, 32, 4096, 128, BF16, BF16, 0.3, "uniform", (0.5, 1.0), (-np.pi, np.pi),
                tuple((b, q, g) for b in (0, 0.5, 1) for q in (0, 1) for g in (0, 1)),
                "switch sweep at batch scale"),
}

# probabilities of the gates (m, theta) = (1, pi), (0, 0), (1, 0) in workload 4
BEDM_P = (0.05, 0.01, 0.94)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 (round to nearest even) -> float32, exact values kept."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def draw(B, H, n, d, seed, qk_dtype=BF16, v_dtype=BF16, qk_scale=1.0, gates="uniform",
         u_range=(0.0, 1.0), theta_range=(-np.pi, np.pi), dv=None):
    """Draw one set of inputs; returns a dict of float32 numpy arrays + meta."""
    dv = d if dv is None else dv
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, n, d), dtype=np.float32)
    k = rng.standard_normal((B, H, n, d), dtype=np.float32)
    v = rng.standard_normal((B, H, n, dv), dtype=np.float32)
    if qk_scale != 1.0:
        q *= np.float32(qk_scale)
        k *= np.float32(qk_scale)
    if gates == "bedm":
        c = rng.choice(3, size=(B, H, n), p=BEDM_P)
        u = np.array([1.0, 0.0, 1.0], dtype=np.float32)[c]
        theta = np.array([np.pi, 0.0, 0.0], dtype=np.float32)[c]
    else:
        lo, hi = u_range
        u = rng.uniform(lo, hi, size=(B, H, n)).astype(np.float32)
        tlo, thi = theta_range
        if tlo == thi:
            theta = np.full((B, H, n), tlo, dtype=np.float32)
        else:
            theta = rng.uniform(tlo, thi, size=(B, H, n)).astype(np.float32)
    if qk_dtype == BF16:
        q, k = round_bf16(q), round_bf16(k)
    if v_dtype == BF16:
        v = round_bf16(v)
    return {"q": q, "k": k, "v": v, "u": u, "theta": theta, "qk_dtype": qk_dtype,
            "v_dtype": v_dtype, "B": B, "H": H, "n": n, "d": d, "seed": seed}


def draw_complex_gates(batch, n, seed, mod_range=(0.95, 1.0), arg_range=(-0.05, 0.05)):
    """Random complex numbers r e^{i phi} (float64 planes [batch, n]) with
    r ~ U(mod_range), phi ~ U(arg_range): ready-made gates for the path-product
    export, drawn directly rather than from u and theta."""
    rng = np.random.Generator(np.random.PCG64(seed))
    r = rng.uniform(*mod_range, size=(batch, n))
    phi = rng.uniform(*arg_range, size=(batch, n))
    return r * np.cos(phi), r * np.sin(phi)


def make_config(idx: int, switches=None, seed=None, n=None, B=None, H=None):
    """Inputs of workload ``idx`` (seed = idx unless given).  ``switches``
    selects the workload-1 variant whose q,k are scaled by 0.3 at (0,1,0).
    ``n``/``B``/``H`` shrink the shape for tests while keeping the recipe."""
    w = WORKLOADS[idx]
    scale = w.qk_scale
    if idx == 1 and switches is not None and tuple(switches) == (0, 1, 0):
        scale = 0.3
    return draw(B or w.B, H or w.H, n or w.n, w.d, idx if seed is None else seed,
                w.qk_dtype, w.v_dtype, scale, w.gates, w.u_range, w.theta_range)


def as_torch(inp: dict, device):
    """Move a drawn input set to ``device`` in its storage types (exact)."""
    import torch

    qdt = torch.bfloat16 if inp["qk_dtype"] == BF16 else torch.float32
    vdt = torch.bfloat16 if inp["v_dtype"] == BF16 else torch.float32
    out = {
        "q": torch.from_numpy(inp["q"]).to(device=device, dtype=qdt).contiguous(),
        "k": torch.from_numpy(inp["k"]).to(device=device, dtype=qdt).contiguous(),
        "v": torch.from_numpy(inp["v"]).to(device=device, dtype=vdt).contiguous(),
        "u": torch.from_numpy(inp["u"]).to(device=device, dtype=torch.float32).contiguous(),
        "theta": torch.from_numpy(inp["theta"]).to(device=device,
                                                    dtype=torch.float32).contiguous(),
    }
    return out
