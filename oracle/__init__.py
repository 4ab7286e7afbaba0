"""fp64 CPU oracle of the resolvent operator head.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path
(``gated_causal_attention_amd``) never imports it and shares no code with it.

Every function restates the "Resolvent Operator" page (teerth.dev,
Aether-Lang/integrated/resolvent): sections "Object", "Evaluation and
refusals", "Rust API" and "The path-product corner is a resolvent".  The
arithmetic lives in ``resolvent_oracle.c``; this module only marshals numpy
arrays (converted to float64, which is exact for the fp32 and bf16 values the
inputs hold) into it.
"""
import ctypes
import os

import numpy as np

from .build import LIBRARY, build_oracle

OK, NONFINITE, BAD_SHAPE, BAD_ARG = 0, 1, 2, 3

_lib = None
_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        build_oracle()
    lib = ctypes.CDLL(LIBRARY)
    d, i64, i32 = ctypes.c_double, ctypes.c_int64, ctypes.c_int32
    lib.oracle_blend.argtypes = [d, d, d, _dp, _dp]
    lib.oracle_gate.argtypes = [d, d, _dp, _dp]
    lib.oracle_gates.argtypes = [_dp, _dp, ctypes.c_int64, d, _dp, _dp]
    lib.oracle_gates.restype = ctypes.c_int
    lib.oracle_path_product.argtypes = [_dp, _dp, i64, _dp, _dp]
    lib.oracle_modulus.argtypes = [_dp, i64, _dp]
    lib.oracle_chain.argtypes = [_dp, _dp, _dp, i64, i32, _dp, _dp]
    lib.oracle_readout.argtypes = [_dp, _dp, _dp, i64, i64, _dp, _dp]
    lib.oracle_operator.argtypes = [_dp, _dp, _dp, _dp, i64, i64, d, d, d, _dp, _dp]
    lib.oracle_operator.restype = ctypes.c_int
    lib.oracle_forward_rows.argtypes = [_dp, _dp, _dp, _dp, _dp, i64, i64, i64, d, d, d,
                                        _i64p, i64, _dp, _dp, i32]
    lib.oracle_forward_rows.restype = ctypes.c_int
    lib.oracle_forward.argtypes = [_dp, _dp, _dp, _dp, _dp, i64, i64, i64, i64, i64, d, d, d,
                                   _dp, _dp, i32]
    lib.oracle_forward.restype = ctypes.c_int
    lib.oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(_dp)


def default_threads() -> int:
    """Threads for the oracle: OMP_NUM_THREADS when set (the host's CPU share),
    else every core this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    cores = len(os.sched_getaffinity(0))
    return min(int(env), cores) if env.isdigit() and int(env) > 0 else cores


def blend(u, theta, g):
    """blend(u, theta, g) -> (m, theta'): clamp((1-g)*1 + g*u, 0, 1), g*theta."""
    m, t = ctypes.c_double(), ctypes.c_double()
    _load().oracle_blend(float(u), float(theta), float(g), ctypes.byref(m), ctypes.byref(t))
    return m.value, t.value


def gate(m, theta_p):
    """gate(m, theta') = m e^{i theta'} as a Python complex."""
    re, im = ctypes.c_double(), ctypes.c_double()
    _load().oracle_gate(float(m), float(theta_p), ctypes.byref(re), ctypes.byref(im))
    return complex(re.value, im.value)


def gates(u, theta, g):
    """Gates a [n] (complex) of one head: gate(blend(u_k, theta_k, g)) for every
    k.  Returns (status, a)."""
    u, theta = _f64(u), _f64(theta)
    n = u.shape[0]
    ar, ai = np.zeros(n), np.zeros(n)
    st = _load().oracle_gates(_ptr(u), _ptr(theta), n, float(g), _ptr(ar), _ptr(ai))
    return st, ar + 1j * ai


def path_product(a):
    """G [n, n] complex from gates a [n] (a[0] is never read)."""
    a = np.asarray(a, dtype=np.complex128)
    n = a.shape[0]
    ar, ai = _f64(a.real), _f64(a.imag)
    gr, gi = np.zeros((n, n)), np.zeros((n, n))
    _load().oracle_path_product(_ptr(ar), _ptr(ai), n, _ptr(gr), _ptr(gi))
    return gr + 1j * gi


def modulus(m):
    """R [n, n] with R_ij = prod_{k=j+1..i} m_k."""
    m = _f64(m)
    n = m.shape[0]
    r = np.zeros((n, n))
    _load().oracle_modulus(_ptr(m), n, _ptr(r))
    return r


def chain(a, b, y0_from_b0=False):
    """Gated chain y_i = a_i y_{i-1} + b_i; y_0 = 0 (page form) or b_0."""
    a = np.asarray(a, dtype=np.complex128)
    b = _f64(b)
    n = b.shape[0]
    ar, ai = _f64(a.real), _f64(a.imag)
    yr, yi = np.zeros(n), np.zeros(n)
    _load().oracle_chain(_ptr(ar), _ptr(ai), _ptr(b), n, int(bool(y0_from_b0)), _ptr(yr), _ptr(yi))
    return yr + 1j * yi


def readout(w, v):
    """O = W V for W [n, n] complex and real V [n, dv]."""
    w = np.asarray(w, dtype=np.complex128)
    v = _f64(v)
    n, dv = v.shape
    wr, wi = _f64(w.real), _f64(w.imag)
    orr, oi = np.zeros((n, dv)), np.zeros((n, dv))
    _load().oracle_readout(_ptr(wr), _ptr(wi), _ptr(v), n, dv, _ptr(orr), _ptr(oi))
    return orr + 1j * oi


def operator(q, k, u, theta, beta, qk, g):
    """W [n, n] complex for one head; returns (status, W)."""
    q, k, u, theta = _f64(q), _f64(k), _f64(u), _f64(theta)
    n = u.shape[0]
    d = q.shape[1] if q.ndim == 2 else 0
    wr, wi = np.zeros((n, n)), np.zeros((n, n))
    st = _load().oracle_operator(_ptr(q), _ptr(k), _ptr(u), _ptr(theta), n, d, float(beta),
                                 float(qk), float(g), _ptr(wr), _ptr(wi))
    return st, wr + 1j * wi


def forward_rows(q, k, u, theta, v, beta, qk, g, rows, nthreads=None):
    """Readout rows of one head: q,k [n,d], v [n,dv], u,theta [n].

    Returns (status, O [len(rows), dv] complex)."""
    q, k, u, theta, v = _f64(q), _f64(k), _f64(u), _f64(theta), _f64(v)
    n = u.shape[0]
    d = q.shape[1] if q.ndim == 2 else 0
    dv = v.shape[1] if v.ndim == 2 else 0
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    nr = rows.shape[0]
    orr, oi = np.zeros((nr, dv)), np.zeros((nr, dv))
    st = _load().oracle_forward_rows(
        _ptr(q), _ptr(k), _ptr(u), _ptr(theta), _ptr(v), n, d, dv, float(beta), float(qk),
        float(g), rows.ctypes.data_as(_i64p), nr, _ptr(orr), _ptr(oi),
        int(nthreads or default_threads()))
    return st, orr + 1j * oi


def forward(q, k, u, theta, v, beta, qk, g, nthreads=None):
    """Full readout: q,k [B,H,n,d], v [B,H,n,dv], u,theta [B,H,n].

    Returns (status, O [B,H,n,dv] complex)."""
    q, k, u, theta, v = _f64(q), _f64(k), _f64(u), _f64(theta), _f64(v)
    B, H, n = u.shape
    d = q.shape[3]
    dv = v.shape[3]
    orr, oi = np.zeros((B, H, n, dv)), np.zeros((B, H, n, dv))
    st = _load().oracle_forward(
        _ptr(q), _ptr(k), _ptr(u), _ptr(theta), _ptr(v), B, H, n, d, dv, float(beta),
        float(qk), float(g), _ptr(orr), _ptr(oi), int(nthreads or default_threads()))
    return st, orr + 1j * oi
