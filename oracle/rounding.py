"""Stochastic rounding of float32 states to an fp16 cache (numpy).

TEST INFRASTRUCTURE ONLY: imported by the test suite, never by the GPU library.

The pages run the SSM cache in float16 with stochastic rounding driven by a
Philox generator with a configurable number of rounds and one seed per step
read from a device buffer (vLLM PR #61501, section "Serve and client
commands": --mamba-ssm-cache-dtype float16, --enable-mamba-cache-stochastic-
rounding, --mamba-cache-philox-rounds 5; section "Details", its list of
changes: the per-step ReplaySSM seed).
They define neither the rounding nor the stream layout; the readings here:

* Stochastic rounding of x (float32) to fp16: with lo, hi the adjacent fp16
  values bracketing x (lo toward zero), the result is hi with probability
  (|x| - |lo|) / (|hi| - |lo|) and lo otherwise, so its expectation is x.
  The probability is exact in float32 (a difference of nearby floats over a
  power of two). Non-finite values and |x| > 65504 round to nearest even.
* The uniform draw is u = d / 2^16 from a 16-bit draw d; round up when
  u < probability. The probability is a multiple of 2^-13 wherever the fp16
  spacing is that of a normal number (|x - lo| is a multiple of the float32
  spacing, 2^-23 of the binade, and |hi - lo| is 2^-10 of it), and of at most
  2^-16 for |x| >= 2^-17, so there the draw is exactly unbiased; below 2^-17
  the chance of rounding up is the probability rounded up to a multiple of
  2^-16.
* Draws come from Philox4x32 with R rounds (Salmon, Moraes, Dror, Shaw,
  "Parallel random numbers: as easy as 1, 2, 3", SC 2011): a 128-bit counter,
  a 64-bit key, per round two 32x32 -> 64-bit products with the multipliers
  0xD2511F53 and 0xCD9E8D57, the key bumped by 0x9E3779B9 and 0xBB67AE85
  between rounds. Element e of a destination array of kind k (0 final states,
  1 checkpoints, 2 per-token states, 3 ReplaySSM checkpoints) takes the 16-bit
  half e mod 2 (the low half first) of word (e // 2) mod 4 of
  Philox(counter = (e // 8 low 32 bits, e // 8 high 32 bits, k, 0),
  key = (seed low 32 bits, seed high 32 bits)): one call serves 8 consecutive
  elements.
"""
from __future__ import annotations

import numpy as np

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK = 0xFFFFFFFF


def philox4x32(counter, key, rounds: int = 10):
    """Philox4x32-R on arrays: counter uint32 [..., 4], key uint32 [..., 2] (broadcast).
    Returns uint32 [..., 4]."""
    c = [np.asarray(counter[..., i], dtype=np.uint64) for i in range(4)]
    k0 = np.asarray(key[..., 0], dtype=np.uint64)
    k1 = np.asarray(key[..., 1], dtype=np.uint64)
    for r in range(rounds):
        if r:
            k0 = (k0 + W0) & MASK
            k1 = (k1 + W1) & MASK
        p0 = c[0] * M0                      # exact: both factors below 2^32
        p1 = c[2] * M1
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return np.stack([v.astype(np.uint32) for v in c], axis=-1)


def draws_for(n: int, seed: int, kind: int, rounds: int, first: int = 0) -> np.ndarray:
    """The 16-bit draws (as uint32 below 2^16) of elements first .. first + n - 1
    of a destination array."""
    e = np.arange(first, first + n, dtype=np.uint64)
    blk = e // np.uint64(8)
    ctr = np.stack([blk & MASK, blk >> np.uint64(32), np.full_like(blk, kind),
                    np.zeros_like(blk)], axis=-1).astype(np.uint32)
    key = np.array([seed & MASK, (seed >> 32) & MASK], dtype=np.uint32)
    out = philox4x32(ctr, key, rounds)
    word = out[np.arange(n), ((e // np.uint64(2)) % np.uint64(4)).astype(np.int64)]
    half = (e % np.uint64(2)).astype(np.uint32)
    return (word >> (np.uint32(16) * half)) & np.uint32(0xFFFF)


def _f16_neighbours(x32: np.ndarray):
    """(lo, hi): fp16 values bracketing float32 x, lo toward zero, hi one step away."""
    with np.errstate(over="ignore"):          # beyond 65504: infinity, as intended
        rne = x32.astype(np.float16)
    bits = rne.view(np.uint16).astype(np.int32)
    away = np.abs(rne.astype(np.float32)) > np.abs(x32)
    lo_bits = np.where(away, bits - 1, bits)             # magnitude one step down
    lo = lo_bits.astype(np.uint16).view(np.float16)
    hi = (lo_bits + 1).astype(np.uint16).view(np.float16)
    return lo, hi


def stochastic_round_f16(x, draws) -> np.ndarray:
    """Stochastic rounding of float32 values with the given 16-bit draws."""
    x32 = np.asarray(x, dtype=np.float32)
    draws = np.asarray(draws, dtype=np.uint32)
    lo, hi = _f16_neighbours(x32)
    a, l32, h32 = np.abs(x32), np.abs(lo.astype(np.float32)), np.abs(hi.astype(np.float32))
    with np.errstate(invalid="ignore", divide="ignore"):
        prob = (a - l32) / (h32 - l32)
    u = draws.astype(np.float32) * np.float32(2.0 ** -16)
    out = np.where(u < prob, hi, lo)
    plain = ~np.isfinite(x32) | (a > np.float32(65504.0)) | (a == l32)
    with np.errstate(over="ignore"):
        return np.where(plain, x32.astype(np.float16), out)
