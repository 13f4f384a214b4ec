"""Quadratic ("dual") form of the SSD operator, by brute force (TEST INFRASTRUCTURE ONLY).

For one sequence and one head, unrolling the recurrence
h_t = exp(dt_t A) h_{t-1} + dt_t x_t (outer) B_t,  y_t = h_t . C_t + D x_t
gives, with decay(j -> i) = product over u = j+1 .. i of exp(dt_u A):

    y_i = sum_{j <= i} (C_i . B_j) * decay(j -> i) * dt_j * x_j
          + decay(-1 -> i) * (h_0 . C_i) + D x_i
    h_L = sum_{j < L} decay(j -> L-1) * dt_j * x_j (outer) B_j + decay(-1 -> L-1) * h_0

Decays are products of per-token factors, never differences of a cumulative
sum, so this shares no arithmetic route with either the recurrence or the
chunked steps. Plain Python loops: tiny inputs only.
"""
from __future__ import annotations

import math

import numpy as np

from . import f64


def dual_single(x, dt, A: float, B, C, D: float, h0=None):
    """x [L,P], dt [L], B/C [L,N], h0 [P,N] or None. Returns y [L,P], h_L [P,N]."""
    x, dt, B, C = f64(x), f64(dt), f64(B), f64(C)
    L, P = x.shape
    N = B.shape[1]
    h0 = np.zeros((P, N)) if h0 is None else f64(h0)
    f = [math.exp(float(dt[u]) * float(A)) for u in range(L)]

    def decay(j, i):          # product of f[u] for u in (j, i]
        prod = 1.0
        for u in range(j + 1, i + 1):
            prod *= f[u]
        return prod

    y = np.zeros((L, P))
    for i in range(L):
        for p in range(P):
            acc = 0.0
            for j in range(i + 1):
                cb = sum(float(C[i, n]) * float(B[j, n]) for n in range(N))
                acc += cb * decay(j, i) * float(dt[j]) * float(x[j, p])
            acc += decay(-1, i) * sum(float(h0[p, n]) * float(C[i, n]) for n in range(N))
            y[i, p] = acc + D * float(x[i, p])
    hL = np.zeros((P, N))
    for p in range(P):
        for n in range(N):
            acc = 0.0
            for j in range(L):
                acc += decay(j, L - 1) * float(dt[j]) * float(x[j, p]) * float(B[j, n])
            hL[p, n] = acc + decay(-1, L - 1) * float(h0[p, n])
    return y, hL


def dual(x, dt, A, B, C, D, cu_seqlens, init=None, has_init=None):
    """Packed batch: x [T,H,P], dt [T,H], B/C [T,G,N]. Returns y [T,H,P], final [S,H,P,N]."""
    x, dt, A, B, C = f64(x), f64(dt), f64(A), f64(B), f64(C)
    Dv = np.zeros(x.shape[1]) if D is None else f64(D)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    S = len(cu) - 1
    y = np.zeros((T, H, P))
    final = np.zeros((S, H, P, N))
    for s in range(S):
        a, b = int(cu[s]), int(cu[s + 1])
        for h in range(H):
            g = h // (H // G)
            h0 = None
            if init is not None and (has_init is None or has_init[s]):
                h0 = f64(init[s, h])
            if b > a:
                y[a:b, h], final[s, h] = dual_single(x[a:b, h], dt[a:b, h], A[h], B[a:b, g],
                                                     C[a:b, g], Dv[h], h0)
            else:
                final[s, h] = 0.0 if h0 is None else h0
    return y, final
