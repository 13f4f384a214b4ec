"""The chunked SSD scan, step by step, in float64 numpy (TEST INFRASTRUCTURE ONLY).

The pages split a Mamba2 prefill into five steps: chunk cumsum, chunk state,
state passing, bmm and chunk scan (vLLM PR #61501, section "Details"); in the
cache-indexed variant, state passing reads each sequence's initial state from
its cache slot and keeps every chunk's *entering* state in the workspace,
which chunk scan then consumes (vLLM PR #62922, sections "Overview" and
"Details"). Each function below is the plain definition of one step's output,
so a GPU step can be checked on its own. The chunking is exact algebra: the
steps composed equal the sequential recurrence, which the tests check for many
chunk sizes (Q = 1 is the recurrence itself; Q = L is the quadratic form).

Notation for chunk c of sequence s, tokens start_c .. start_c + len_c - 1,
head h, group g = h / (H / G), local token index i in [0, len_c):
    a_i     = dt_i * A_h
    cum_i   = a_0 + ... + a_i                  (inclusive)
    S_c     = sum_i exp(cum_{len-1} - cum_i) * dt_i * x_i (outer) B_i     [P x N]
    H_in(c) = state entering chunk c; H_in(first chunk) = initial state or 0
    H_in(c+1) = exp(cum_{len-1}) * H_in(c) + S_c
    CB[i,j] = C_i . B_j
    y_i     = sum_{j <= i} CB[i,j] * exp(cum_i - cum_j) * dt_j * x_j
              + exp(cum_i) * (H_in(c) . C_i) + D_h * x_i

Padding convention of the per-chunk arrays (rows of Q entries): local
positions i >= len_c behave as tokens with dt = 0 (cum stays flat, dt pads
with 0), so dA_cumsum[h, c, i] = cum_{len-1} and dt_pad[h, c, i] = 0 there.
"""
from __future__ import annotations

import numpy as np

from . import f64


def chunk_meta(cu_seqlens, Q: int):
    """Per-chunk (seq, start, len) and chunk_cu [S+1] from cu_seqlens."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    S = len(cu) - 1
    chunk_cu = np.zeros(S + 1, dtype=np.int64)
    seq, start, length = [], [], []
    for s in range(S):
        L = int(cu[s + 1] - cu[s])
        k = 0
        while k * Q < L:
            seq.append(s)
            start.append(int(cu[s]) + k * Q)
            length.append(min(Q, L - k * Q))
            k += 1
        chunk_cu[s + 1] = chunk_cu[s] + k
    return dict(chunk_cu=chunk_cu, seq=np.array(seq, dtype=np.int64),
                start=np.array(start, dtype=np.int64), len=np.array(length, dtype=np.int64))


def chunk_cumsum(dt, A, meta, Q: int):
    """dA_cumsum [H, nc, Q] and dt_pad [H, nc, Q] (float64)."""
    dt, A = f64(dt), f64(A)
    H = dt.shape[1]
    nc = len(meta["seq"])
    cum = np.zeros((H, nc, Q))
    dtp = np.zeros((H, nc, Q))
    for c in range(nc):
        st, ln = int(meta["start"][c]), int(meta["len"][c])
        d = np.zeros((Q, H))
        d[:ln] = dt[st:st + ln]
        dtp[:, c, :] = d.T
        cum[:, c, :] = np.cumsum(d * A[None, :], axis=0).T
    return cum, dtp


def chunk_state(x, B, cum, dtp, meta):
    """S_c [nc, H, P, N]: the state chunk c produces from a zero entering state."""
    x, B = f64(x), f64(B)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    nc = len(meta["seq"])
    out = np.zeros((nc, H, P, N))
    for c in range(nc):
        st, ln = int(meta["start"][c]), int(meta["len"][c])
        for h in range(H):
            g = h // (H // G)
            w = np.exp(cum[h, c, ln - 1] - cum[h, c, :ln]) * dtp[h, c, :ln]     # [len]
            out[c, h] = (x[st:st + ln, h, :] * w[:, None]).T @ B[st:st + ln, g, :]
    return out


def state_passing(states, cum, meta, init=None, has_init=None):
    """Entering state of every chunk, exit state of every chunk (the checkpoints)
    and the final state of every sequence. init [S,H,P,N] or None."""
    nc, H, P, N = states.shape
    S = len(meta["chunk_cu"]) - 1
    entering = np.zeros_like(states)
    exits = np.zeros_like(states)
    final = np.zeros((S, H, P, N))
    for s in range(S):
        if init is not None and (has_init is None or has_init[s]):
            h = f64(init[s]).copy()
        else:
            h = np.zeros((H, P, N))
        for c in range(int(meta["chunk_cu"][s]), int(meta["chunk_cu"][s + 1])):
            ln = int(meta["len"][c])
            entering[c] = h
            decay = np.exp(cum[:, c, ln - 1])                    # [H]
            h = decay[:, None, None] * h + states[c]
            exits[c] = h
        final[s] = h
    return entering, exits, final


def bmm(B, C, meta, Q: int):
    """CB [nc, G, Q, Q]: CB[i, j] = C_i . B_j inside each chunk (0 outside len)."""
    B, C = f64(B), f64(C)
    G = B.shape[1]
    nc = len(meta["seq"])
    out = np.zeros((nc, G, Q, Q))
    for c in range(nc):
        st, ln = int(meta["start"][c]), int(meta["len"][c])
        for g in range(G):
            out[c, g, :ln, :ln] = C[st:st + ln, g, :] @ B[st:st + ln, g, :].T
    return out


def chunk_scan(x, C, D, CB, cum, dtp, entering, meta):
    """y [T, H, P] from the chunk's inputs and its entering state."""
    x, C = f64(x), f64(C)
    T, H, P = x.shape
    G = C.shape[1]
    Dv = np.zeros(H) if D is None else f64(D)
    y = np.zeros((T, H, P))
    nc = len(meta["seq"])
    for c in range(nc):
        st, ln = int(meta["start"][c]), int(meta["len"][c])
        for h in range(H):
            g = h // (H // G)
            cm = cum[h, c, :ln]
            diff = cm[:, None] - cm[None, :]
            causal = np.tril(np.ones((ln, ln), dtype=bool))
            L = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0) * dtp[h, c, None, :ln]
            M = CB[c, g, :ln, :ln] * L
            xc = x[st:st + ln, h, :]
            inter = np.exp(cm)[:, None] * (C[st:st + ln, g, :] @ entering[c, h].T)
            y[st:st + ln, h, :] = M @ xc + inter + Dv[h] * xc
    return y


def scan(x, dt, A, B, C, D, cu_seqlens, Q: int, init=None, has_init=None):
    """All five steps composed. Returns a dict with every intermediate."""
    meta = chunk_meta(cu_seqlens, Q)
    cum, dtp = chunk_cumsum(dt, A, meta, Q)
    st = chunk_state(x, B, cum, dtp, meta)
    entering, exits, final = state_passing(st, cum, meta, init, has_init)
    CB = bmm(B, C, meta, Q)
    y = chunk_scan(x, C, D, CB, cum, dtp, entering, meta)
    return dict(meta=meta, dA_cumsum=cum, dt=dtp, chunk_states=st, entering=entering,
                ckpt=exits, final=final, CB=CB, y=y)
