"""Brute-force LeapQuant on tiny heads -- an independent second implementation.

Written differently from the oracle on purpose: one state at a time, the
transition as an explicit dense matrix A_t = D_t - k~_t b_t^T, and a
scalar-loop quantizer with a full sort.  Used only to pin the oracle.
"""
import numpy as np

f32 = np.float32


def brute_quantize(S, r, smooth=True):
    """One state (2-D array).  Returns (codes, a, s, idx, w) as Python lists."""
    S = [[f32(x) for x in row] for row in np.asarray(S, dtype=np.float32)]
    dk, dv = len(S), len(S[0])
    norms = []
    for i in range(dk):
        acc = 0.0
        for j in range(dv):
            acc += float(S[i][j]) * float(S[i][j])
        norms.append(acc)
    order = sorted(range(dk), key=lambda i: (-norms[i], i))
    idx = order[:r]
    w = [[S[i][j] for j in range(dv)] for i in idx]
    R = [[f32(0) if i in idx else S[i][j] for j in range(dv)] for i in range(dk)]
    s = []
    for j in range(dv):
        if smooth:
            mx = f32(0)
            for i in range(dk):
                if abs(R[i][j]) > mx:
                    mx = abs(R[i][j])
            s.append(mx if mx != 0 else f32(1))
        else:
            s.append(f32(1))
    a = []
    codes = []
    for i in range(dk):
        qrow = [R[i][j] * (f32(1) / s[j]) for j in range(dv)]
        m = f32(0)
        for x in qrow:
            if abs(x) > m:
                m = abs(x)
        if m == 0:
            a.append(f32(0))
            codes.append([0] * dv)
            continue
        a.append(m / f32(127))
        inv = f32(127) / m
        row = []
        for x in qrow:
            y = x * inv
            c = int(np.rint(y))
            row.append(max(-127, min(127, c)))
        codes.append(row)
    return codes, a, s, idx, w


def brute_dequant(codes, a, s, idx, w):
    dk, dv = len(codes), len(codes[0])
    B = np.zeros((dk, dv))
    for i in range(dk):
        for j in range(dv):
            B[i, j] = float(codes[i][j]) * float(a[i]) * float(s[j])
    for c, i in enumerate(idx):
        for j in range(dv):
            B[i, j] += float(w[c][j])
    return B


def brute_windowed(S_init, q, k, v, beta, alpha, p, r, kda, smooth=True):
    """One state; q,k [T,dk], v [T,dv], beta [T], alpha [T] or [T,dk].

    Returns (outputs [T,dv], list of boundary tuples at every window start,
    including the one after the last window).
    """
    T, dk = q.shape
    bnd = brute_quantize(S_init, r, smooth)
    bounds = [bnd]
    S = brute_dequant(*bnd)
    outs = np.zeros((T, v.shape[1]))
    for t in range(T):
        Dvec = np.array(alpha[t], dtype=np.float64) if kda else np.full(dk, float(alpha[t]))
        D = np.diag(Dvec)
        kt = float(beta[t]) * np.asarray(k[t], np.float64)
        b = Dvec * np.asarray(k[t], np.float64)
        A = D - np.outer(kt, b)
        S = A @ S + np.outer(kt, np.asarray(v[t], np.float64))
        outs[t] = S.T @ np.asarray(q[t], np.float64)
        if (t + 1) % p == 0 or t == T - 1:
            bnd = brute_quantize(S.astype(np.float32), r, smooth)
            bounds.append(bnd)
            S = brute_dequant(*bnd)
    return outs, bounds
