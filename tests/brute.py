"""Brute-force evaluation of the resolvent head in 50-digit arithmetic (mpmath).

Test helper.  It writes the definition of the "Resolvent Operator" page
(section "Object") literally, with the dense normaliser Z_i^beta (no log
domain, no max shift) and the path product multiplied in ascending k order,
so it shares neither formulation nor code with the fp64 oracle it pins.
For n <= 8 only.
"""
import mpmath as mp

mp.mp.dps = 50


def weights(q, k, u, theta, beta, qk, g):
    """W [n][n] as mpmath complex numbers (0 above the diagonal)."""
    n = len(u)
    d = len(q[0]) if n else 0
    beta, qk, g = mp.mpf(beta), mp.mpf(qk), mp.mpf(g)
    m, a = [], []
    for x in range(n):
        lerp = (1 - g) + g * mp.mpf(u[x])
        mk = min(max(lerp, mp.mpf(0)), mp.mpf(1))
        th = g * mp.mpf(theta[x])
        m.append(mk)
        a.append(mk * mp.expj(th))
    s = [[mp.fsum(mp.mpf(q[i][e]) * mp.mpf(k[j][e]) for e in range(d)) / mp.sqrt(d)
          for j in range(n)] for i in range(n)]
    W = [[mp.mpc(0) for _ in range(n)] for _ in range(n)]
    for i in range(n):
        G, R = [], []
        for j in range(i + 1):
            gp, rp = mp.mpc(1), mp.mpf(1)
            for kk in range(j + 1, i + 1):
                gp *= a[kk]
                rp *= m[kk]
            G.append(gp)
            R.append(rp)
        Z = mp.fsum(R[j] * mp.exp(qk * s[i][j]) for j in range(i + 1))
        for j in range(i + 1):
            W[i][j] = G[j] * mp.exp(qk * s[i][j]) / mp.power(Z, beta)
    return W


def readout(W, v):
    n = len(W)
    dv = len(v[0]) if n else 0
    return [[mp.fsum(W[i][j] * mp.mpf(v[j][c]) for j in range(i + 1)) for c in range(dv)]
            for i in range(n)]
