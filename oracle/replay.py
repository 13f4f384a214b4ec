"""ReplaySSM decode as a plain state machine over one layer's storage (float64).

TEST INFRASTRUCTURE ONLY: imported by the test suite, never by the GPU library.

Source: vLLM PR #52928 "[Mamba] Add FlashInfer ReplaySSM support for MTP",
sections "Summary" and "Design": instead of a stored state per draft token,
each layer keeps a checkpoint state and a ring of the inputs; the accepted
length moves a shared cursor before the next forward, and the checkpoint is
rewritten only when the next verify window would overflow the ring. vLLM PR
#55688 (FlashInfer ReplaySSM prefix caching), "Summary": pending history is
materialised into a checkpoint before a state is published.

Readings (the pages give no formulas):

* Per slot: checkpoint (storage dtype), rings of x, dt, B with ring_len = W
  entries, cursor (start, n). The n accepted tokens since the checkpoint sit
  at ring positions (start + i) mod W. The slot's current state is the
  checkpoint followed by those tokens through the recurrence.
* The history holds at most L = W - T tokens, and one verify window of T
  tokens follows it (the pages' ring keeps the live window and the current
  verify window together). A verify step whose history could not take the
  next window after this one (n + T > L) rounds the rebuilt state into the
  checkpoint; the window still continues from the unrounded state.
* After sampling, a accepted drafts keep 1 + a window tokens: the cursor
  becomes (start, n + 1 + a), or ((start + n) mod W, 1 + a) when that verify
  step rewrote the checkpoint.
* Materialise: checkpoint = rounded current state, cursor ((start + n) mod W, 0).

Arithmetic is the per-token recurrence (no folding, no chunking):
h <- exp(dt A) h + dt x (x) B, y = C . h + D x, in float64 on the exact
values the GPU reads.
"""
from __future__ import annotations

import numpy as np
import torch

from . import f64, round_to


class ReplayLayer:
    """Checkpoints, input rings and cursors of one layer (CPU tensors)."""

    def __init__(self, ckpt: torch.Tensor, ring_len: int, ngroups: int, in_dtype: torch.dtype):
        S, H, P, N = ckpt.shape
        self.ckpt = ckpt.clone()
        self.W = int(ring_len)
        self.G = int(ngroups)
        self.ring_x = torch.zeros(S, self.W, H, P, dtype=in_dtype)
        self.ring_dt = torch.zeros(S, self.W, H, dtype=in_dtype)
        self.ring_B = torch.zeros(S, self.W, self.G, N, dtype=in_dtype)
        self.cursor = np.zeros((S, 2), dtype=np.int64)


def _token(h, x, dt, A, B, gmap):
    """One recurrence step for every head: h [H,P,N], x [H,P], dt [H], B [G,N]."""
    a = np.exp(dt * A)
    return a[:, None, None] * h + (dt[:, None] * x)[:, :, None] * B[gmap][:, None, :]


def _gmap(H: int, G: int) -> np.ndarray:
    return np.arange(H) // (H // G)


def _history_state(layer: ReplayLayer, s: int, A: np.ndarray) -> np.ndarray:
    """The slot's current state: its checkpoint, then its n history tokens in order."""
    start, n = (int(v) for v in layer.cursor[s])
    h = f64(layer.ckpt[s])
    gmap = _gmap(h.shape[0], layer.G)
    for i in range(n):
        pos = (start + i) % layer.W
        h = _token(h, f64(layer.ring_x[s, pos]), f64(layer.ring_dt[s, pos]), A,
                   f64(layer.ring_B[s, pos]), gmap)
    return h


def replay_update(layer: ReplayLayer, state_indices, x, dt, A, B, C, D) -> np.ndarray:
    """Verify step. x [R,T,H,P], dt [R,T,H], B/C [R,T,G,N] (torch, storage dtypes);
    A, D [H]. Returns y float64 [R,T,H,P]; updates checkpoints and rings in place."""
    A = f64(A)
    D = np.zeros_like(A) if D is None else f64(D)
    R, T, H, P = x.shape
    L = layer.W - T
    gmap = _gmap(H, layer.G)
    y = np.zeros((R, T, H, P))
    for r, s in enumerate(np.asarray(state_indices, dtype=np.int64)):
        s = int(s)
        start, n = (int(v) for v in layer.cursor[s])
        h = _history_state(layer, s, A)
        if n + T > L:
            layer.ckpt[s] = round_to(h, layer.ckpt.dtype)
        for t in range(T):
            xt = f64(x[r, t])
            h = _token(h, xt, f64(dt[r, t]), A, f64(B[r, t]), gmap)
            Ct = f64(C[r, t])[gmap]                       # [H,N]
            y[r, t] = np.einsum("hpn,hn->hp", h, Ct) + D[:, None] * xt
            pos = (start + n + t) % layer.W
            layer.ring_x[s, pos] = x[r, t]
            layer.ring_dt[s, pos] = dt[r, t]
            layer.ring_B[s, pos] = B[r, t]
    return y


def replay_advance(layer: ReplayLayer, state_indices, num_accepted, T: int) -> None:
    """Cursor move after sampling (1 + a tokens of the last window are kept)."""
    L = layer.W - T
    for s, a in zip(np.asarray(state_indices, dtype=np.int64), np.asarray(num_accepted)):
        start, n = (int(v) for v in layer.cursor[int(s)])
        if n + T > L:
            layer.cursor[int(s)] = ((start + n) % layer.W, 1 + int(a))
        else:
            layer.cursor[int(s)] = (start, n + 1 + int(a))


def replay_materialize(layer: ReplayLayer, state_indices, A) -> None:
    """Fold each slot's history into its checkpoint and empty the history."""
    A = f64(A)
    for s in np.asarray(state_indices, dtype=np.int64):
        s = int(s)
        h = _history_state(layer, s, A)
        layer.ckpt[s] = round_to(h, layer.ckpt.dtype)
        start, n = (int(v) for v in layer.cursor[s])
        layer.cursor[s] = ((start + n) % layer.W, 0)
