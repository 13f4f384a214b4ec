"""Pins of the CPU oracle to things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle (the compiled
ssd_oracle.c passed as ``lib``; None = the default build) disagrees with a
closed form, a hand-worked case, brute force through the quadratic form, an
invariant of the recurrence, or a library routine. ``test_oracle_pins.py``
runs them on the real oracle; ``test_oracle_mutations.py`` runs them on copies
of the oracle with planted mistakes and requires each copy to fail at least
one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
from oracle import chunked, dual
from oracle import replay as oracle_replay
from oracle import rounding as oracle_rounding

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(seed, T, H, P, N, G, dt_range=(1e-3, 0.1), a_range=(1.0, 16.0)):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, H, P))
    dt = g.uniform(*dt_range, size=(T, H))
    A = -g.uniform(*a_range, size=H)
    B = g.standard_normal((T, G, N)) / math.sqrt(N)
    C = g.standard_normal((T, G, N)) / math.sqrt(N)
    D = g.standard_normal(H)
    return x, dt, A, B, C, D


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(1e-300, float(np.max(np.abs(b)))))


def pin_hand_worked(lib=None):
    """Two cases worked by hand with exact binary fractions (tests/golden)."""
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        cases = json.load(f)["cases"]
    for cs in cases:
        x = np.array(cs["x"], dtype=np.float64)
        dt = np.array(cs["dt"], dtype=np.float64)
        B = np.array(cs["B"], dtype=np.float64)
        C = np.array(cs["C"], dtype=np.float64)
        A = np.array(cs["A"]); D = np.array(cs["D"])
        T = x.shape[0]
        init = None if cs["h0"] is None else np.array(cs["h0"], dtype=np.float64)
        y, final, ckpt = oracle.recurrence(x, dt, A, B, C, D, [0, T], 1, init=init,
                                           checkpoints=True, lib=lib)
        np.testing.assert_allclose(y, np.array(cs["y"]), rtol=0, atol=1e-12, err_msg=cs["name"])
        np.testing.assert_allclose(final, np.array(cs["final"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(ckpt, np.array(cs["states_after_each_token"]), rtol=0,
                                   atol=1e-12)
        # the same case through the state update (one request, T tokens)
        h0 = np.zeros((1, cs["H"], cs["P"], cs["N"])) if init is None else init
        cache = torch.from_numpy(h0.copy())
        out = oracle.state_update(cache, [0], x[None], dt[None], A, B[None], C[None], D, True,
                                  lib=lib)
        np.testing.assert_allclose(out["y"][0], np.array(cs["y"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(out["states"][0], np.array(cs["states_after_each_token"]),
                                   rtol=0, atol=1e-12)


def pin_single_token_closed_form(lib=None):
    """L = 1: y_0 = exp(dt A)(h0 . C_0) + dt (C_0 . B_0) x_0 + D x_0."""
    x, dt, A, B, C, D = _rand(11, 1, 3, 4, 5, 1)
    h0 = np.random.default_rng(12).standard_normal((1, 3, 4, 5))
    for init in (None, h0):
        y, final, _ = oracle.recurrence(x, dt, A, B, C, D, [0, 1], 4, init=init, lib=lib)
        for h in range(3):
            z = np.zeros((4, 5)) if init is None else init[0, h]
            decay = math.exp(dt[0, h] * A[h])
            want_state = decay * z + dt[0, h] * np.outer(x[0, h], B[0, 0])
            want_y = decay * z @ C[0, 0] + dt[0, h] * (C[0, 0] @ B[0, 0]) * x[0, h] + D[h] * x[0, h]
            np.testing.assert_allclose(final[0, h], want_state, rtol=1e-13, atol=1e-15)
            np.testing.assert_allclose(y[0, h], want_y, rtol=1e-12, atol=1e-14)


def pin_cumsum_reduction(lib=None):
    """A = 0, dt = 1: h_t = sum_{j<=t} x_j (outer) B_j (numpy.cumsum); y_t = h_t . C_t + D x_t."""
    T, H, P, N, G = 9, 2, 3, 4, 2
    x, _, _, B, C, D = _rand(21, T, H, P, N, G)
    dt = np.ones((T, H))
    A = np.zeros(H)
    y, final, _ = oracle.recurrence(x, dt, A, B, C, D, [0, T], 4, lib=lib)
    for h in range(H):
        g = h // (H // G)
        outer = x[:, h, :, None] * B[:, g, None, :]             # [T,P,N]
        hs = np.cumsum(outer, axis=0)
        want_y = np.einsum("tpn,tn->tp", hs, C[:, g]) + D[h] * x[:, h]
        np.testing.assert_allclose(y[:, h], want_y, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(final[0, h], hs[-1], rtol=1e-12, atol=1e-12)


def pin_pure_decay(lib=None):
    """x = 0: h_t = exp(A sum_{u<=t} dt_u) h0 and y_t = that state . C_t."""
    T, H, P, N, G = 7, 2, 3, 4, 1
    _, dt, A, B, C, D = _rand(31, T, H, P, N, G)
    x = np.zeros((T, H, P))
    h0 = np.random.default_rng(32).standard_normal((1, H, P, N))
    y, final, ckpt = oracle.recurrence(x, dt, A, B, C, D, [0, T], 1, init=h0, checkpoints=True,
                                       lib=lib)
    for h in range(H):
        for t in range(T):
            f = math.exp(A[h] * float(np.sum(dt[: t + 1, h])))
            np.testing.assert_allclose(ckpt[t, h], f * h0[0, h], rtol=1e-12, atol=1e-300)
            np.testing.assert_allclose(y[t, h], f * h0[0, h] @ C[t, 0], rtol=1e-12, atol=1e-15)


def pin_skip_only(lib=None):
    """B = 0 or C = 0 (from a zero state): y = D x exactly."""
    T, H, P, N, G = 6, 2, 3, 4, 2
    x, dt, A, B, C, D = _rand(41, T, H, P, N, G)
    zero = np.zeros_like(B)
    for b, c in ((zero, C), (B, zero)):
        y, _, _ = oracle.recurrence(x, dt, A, b, c, D, [0, T], 4, lib=lib)
        np.testing.assert_array_equal(y, D[None, :, None] * x)


def pin_linearity(lib=None):
    """From a zero state the map x -> y is linear."""
    T, H, P, N, G = 10, 2, 3, 4, 1
    x1, dt, A, B, C, D = _rand(51, T, H, P, N, G)
    x2 = np.random.default_rng(52).standard_normal(x1.shape)
    y1, f1, _ = oracle.recurrence(x1, dt, A, B, C, D, [0, T], 4, lib=lib)
    y2, f2, _ = oracle.recurrence(x2, dt, A, B, C, D, [0, T], 4, lib=lib)
    y12, f12, _ = oracle.recurrence(x1 + x2, dt, A, B, C, D, [0, T], 4, lib=lib)
    ya, fa, _ = oracle.recurrence(2.5 * x1, dt, A, B, C, D, [0, T], 4, lib=lib)
    np.testing.assert_allclose(y12, y1 + y2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f12, f1 + f2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ya, 2.5 * y1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fa, 2.5 * f1, rtol=1e-12, atol=1e-12)


def pin_dual_form(lib=None):
    """Brute force: the quadratic form (decays as products) equals the recurrence to 1e-12."""
    for seed, lens, H, P, N, G, with_init in ((61, [7], 2, 2, 3, 1, False),
                                              (62, [5, 0, 9, 1], 4, 3, 2, 2, True),
                                              (63, [12, 3], 2, 3, 3, 2, True)):
        T = sum(lens)
        x, dt, A, B, C, D = _rand(seed, T, H, P, N, G, dt_range=(0.01, 0.5))
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        S = len(lens)
        init = hi = None
        if with_init:
            init = np.random.default_rng(seed + 100).standard_normal((S, H, P, N))
            hi = np.array([s % 2 for s in range(S)], dtype=np.uint8)
        y, final, _ = oracle.recurrence(x, dt, A, B, C, D, cu, 4, init=init, has_init=hi, lib=lib)
        yd, fd = dual.dual(x, dt, A, B, C, D, cu, init=init, has_init=hi)
        assert _rel(y, yd) < 1e-12, (seed, _rel(y, yd))
        assert _rel(final, fd) < 1e-12, (seed, _rel(final, fd))


def pin_continued_prefill(lib=None):
    """oracle(seq[:k]) -> state -> oracle(seq[k:]) equals oracle(seq), for every k."""
    T, H, P, N, G = 11, 2, 3, 4, 2
    x, dt, A, B, C, D = _rand(71, T, H, P, N, G)
    y, final, _ = oracle.recurrence(x, dt, A, B, C, D, [0, T], 4, lib=lib)
    for k in range(T + 1):
        ya, fa, _ = oracle.recurrence(x[:k], dt[:k], A, B[:k], C[:k], D, [0, k], 4, lib=lib)
        yb, fb, _ = oracle.recurrence(x[k:], dt[k:], A, B[k:], C[k:], D, [0, T - k], 4,
                                      init=fa, lib=lib)
        np.testing.assert_allclose(np.concatenate([ya, yb]), y, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(fb, final, rtol=1e-12, atol=1e-13)


def pin_varlen_packing(lib=None):
    """A packed batch equals each sequence run alone (bitwise: same operation order)."""
    lens = [5, 0, 13, 1, 8]
    T, H, P, N, G = sum(lens), 4, 3, 5, 2
    x, dt, A, B, C, D = _rand(81, T, H, P, N, G)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    S = len(lens)
    init = np.random.default_rng(82).standard_normal((S, H, P, N))
    hi = np.array([1, 0, 1, 1, 0], dtype=np.uint8)
    y, final, ckpt = oracle.recurrence(x, dt, A, B, C, D, cu, 4, init=init, has_init=hi,
                                       checkpoints=True, lib=lib)
    chunk_cu = oracle.chunk_counts(cu, 4)
    for s in range(S):
        a, b = cu[s], cu[s + 1]
        y1, f1, c1 = oracle.recurrence(x[a:b], dt[a:b], A, B[a:b], C[a:b], D, [0, b - a], 4,
                                       init=init[s:s + 1] if hi[s] else None, checkpoints=True,
                                       lib=lib)
        np.testing.assert_array_equal(y[a:b], y1)
        np.testing.assert_array_equal(final[s], f1[0])
        np.testing.assert_array_equal(ckpt[chunk_cu[s]:chunk_cu[s + 1]], c1)


def pin_checkpoints_are_truncated_finals(lib=None):
    """ckpt[k] equals the final state of the same prefill cut at min((k+1) Q, L)."""
    T, H, P, N, G, Q = 23, 2, 2, 3, 1, 5
    x, dt, A, B, C, D = _rand(91, T, H, P, N, G)
    h0 = np.random.default_rng(92).standard_normal((1, H, P, N))
    _, _, ckpt = oracle.recurrence(x, dt, A, B, C, D, [0, T], Q, init=h0, checkpoints=True,
                                   lib=lib)
    assert ckpt.shape[0] == math.ceil(T / Q)
    for k in range(ckpt.shape[0]):
        e = min((k + 1) * Q, T)
        _, fk, _ = oracle.recurrence(x[:e], dt[:e], A, B[:e], C[:e], D, [0, e], Q, init=h0,
                                     lib=lib)
        np.testing.assert_array_equal(ckpt[k], fk[0])


def pin_chunk_size_independence(lib=None):
    """The chunked steps (oracle.chunked) equal the recurrence for any chunk size:
    Q = 1 is the recurrence itself, Q = L the quadratic form."""
    lens = [19, 1, 0, 8]
    T, H, P, N, G = sum(lens), 4, 3, 4, 2
    x, dt, A, B, C, D = _rand(101, T, H, P, N, G)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    S = len(lens)
    init = np.random.default_rng(102).standard_normal((S, H, P, N))
    hi = np.array([1, 0, 1, 1], dtype=np.uint8)
    for Q in (1, 2, 3, 7, 16, 64, max(lens)):
        y, final, ckpt = oracle.recurrence(x, dt, A, B, C, D, cu, Q, init=init, has_init=hi,
                                           checkpoints=True, lib=lib)
        r = chunked.scan(x, dt, A, B, C, D, cu, Q, init=init, has_init=hi)
        assert _rel(r["y"], y) < 1e-12, (Q, _rel(r["y"], y))
        assert _rel(r["final"], final) < 1e-12, Q
        assert _rel(r["ckpt"], ckpt) < 1e-12, Q
        if Q == 1:   # entering state of chunk c == state after the previous token
            for s in range(S):
                a, b = int(cu[s]), int(cu[s + 1])
                c0 = int(r["meta"]["chunk_cu"][s])
                for k in range(1, b - a):
                    np.testing.assert_allclose(r["entering"][c0 + k], ckpt[c0 + k - 1],
                                               rtol=1e-12, atol=1e-14)


def pin_state_update_replay(lib=None):
    """replay[r, t] equals the prefill final state over tokens 0..t from the same start;
    T = 1 is plain decode; committing a accepted drafts equals a continued prefill
    over 1 + a tokens."""
    R, T, H, P, N, G = 3, 3, 4, 2, 3, 2
    x, dt, A, B, C, D = _rand(111, R * T, H, P, N, G)
    x4, dt4 = x.reshape(R, T, H, P), dt.reshape(R, T, H)
    B4, C4 = B.reshape(R, T, G, N), C.reshape(R, T, G, N)
    cache = torch.from_numpy(np.random.default_rng(112).standard_normal((5, H, P, N)))
    idx = np.array([3, 0, 4], dtype=np.int32)
    out = oracle.state_update(cache, idx, x4, dt4, A, B4, C4, D, True, lib=lib)
    assert torch.equal(out["cache"], cache)        # intermediate states kept: cache untouched
    for r in range(R):
        for t in range(T):
            y1, f1, _ = oracle.recurrence(x4[r, :t + 1], dt4[r, :t + 1], A, B4[r, :t + 1],
                                          C4[r, :t + 1], D, [0, t + 1], 8,
                                          init=cache[idx[r]].numpy()[None], lib=lib)
            np.testing.assert_allclose(out["states"][r, t], f1[0], rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(out["y"][r, :t + 1], y1, rtol=1e-12, atol=1e-14)
    # T = 1 decode writes the final state into the slot
    dec = oracle.state_update(cache, idx, x4[:, :1], dt4[:, :1], A, B4[:, :1], C4[:, :1], D,
                              False, lib=lib)
    for r in range(R):
        np.testing.assert_allclose(dec["cache"][idx[r]].numpy(), out["states"][r, 0],
                                   rtol=1e-12, atol=1e-14)
    untouched = [s for s in range(5) if s not in idx]
    assert torch.equal(dec["cache"][untouched], cache[untouched])
    # rollback to a accepted drafts
    acc = np.array([2, 0, 1], dtype=np.int32)
    replay = torch.from_numpy(out["states"])
    after = oracle.commit(cache, idx, replay, acc)
    for r in range(R):
        a = int(acc[r])
        _, fa, _ = oracle.recurrence(x4[r, :a + 1], dt4[r, :a + 1], A, B4[r, :a + 1],
                                     C4[r, :a + 1], D, [0, a + 1], 8,
                                     init=cache[idx[r]].numpy()[None], lib=lib)
        np.testing.assert_allclose(after[idx[r]].numpy(), fa[0], rtol=1e-12, atol=1e-14)


def pin_cache_semantics(lib=None):
    """Slots: snapshot reads, sequences without an initial state never read their
    (NaN) slot, untouched slots stay bit-identical, zero-length sequences write
    their initial state (or 0) back."""
    lens = [4, 0, 6, 0]
    T, H, P, N, G = sum(lens), 2, 2, 3, 1
    x, dt, A, B, C, D = _rand(121, T, H, P, N, G)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cache = torch.from_numpy(np.random.default_rng(122).standard_normal((8, H, P, N))).float()
    cache[5] = float("nan")
    cache[6] = float("nan")
    idx = np.array([2, 5, 7, 6], dtype=np.int32)
    hi = np.array([1, 0, 1, 0], dtype=np.uint8)
    out = oracle.prefill(x, dt, A, B, C, D, cu, idx, hi, cache, 4, lib=lib)
    assert np.all(np.isfinite(out["y"])) and np.all(np.isfinite(out["final"]))
    assert torch.equal(out["cache"][[0, 1, 3, 4]], cache[[0, 1, 3, 4]])
    assert torch.equal(out["cache"][5], torch.zeros_like(cache[5]))   # empty, no initial state
    assert torch.equal(out["cache"][6], torch.zeros_like(cache[6]))
    # sequence 0 continues from slot 2 as it was before the call
    y0, f0, _ = oracle.recurrence(x[:4], dt[:4], A, B[:4], C[:4], D, [0, 4], 4,
                                  init=cache[2].double().numpy()[None], lib=lib)
    np.testing.assert_allclose(out["y"][:4], y0, rtol=1e-12, atol=1e-14)
    # no initial state at all: identical to an all-zero cache
    z = oracle.prefill(x, dt, A, B, C, D, cu, idx, None, cache, 4, lib=lib)
    z2 = oracle.prefill(x, dt, A, B, C, D, cu, idx, np.zeros(4, np.uint8), torch.zeros_like(cache),
                        4, lib=lib)
    np.testing.assert_array_equal(z["y"], z2["y"])


def pin_bf16_rounding(lib=None):
    """Rounding to bf16 is round-to-nearest-even (checked on hand-picked ties)."""
    vals = np.array([1.0 + 2.0 ** -8,            # tie between 1 and 1+2^-7 -> 1 (even)
                     1.0 + 3 * 2.0 ** -8,        # tie between 1+2^-7 and 1+2^-6 -> 1+2^-6
                     1.0 + 2.0 ** -8 + 2.0 ** -20,  # above the tie -> 1+2^-7
                     -(2.0 + 2.0 ** -7)])        # tie at 2 (spacing 2^-6) -> -2
    want = np.array([1.0, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7, -2.0])
    got = oracle.round_to(vals, torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got, want)


def pin_replay_matches_recurrence(lib=None, replay=None):
    """ReplaySSM (checkpoint, input rings, cursor) against the plain recurrence over the
    kept tokens. Storage in float64, so nothing is rounded: every window's y and the
    materialised checkpoint must agree to 1e-12. The accepted pattern is fixed so the
    checkpoint schedule and cursors can be worked by hand: T = 3, W = 9 (history
    capacity L = 6), accepted drafts 2, 0, 1, 2, 2, 0, 1 give histories n = 0, 3, 4,
    2, 5, 3, 4 at the verify steps, checkpoints rewritten at steps 2, 4, 6 (n + T > L)
    and the cursor (4, 2) at the end, (6, 0) after materialising."""
    rp = replay or oracle_replay
    R, T, H, P, N, G, W = 3, 3, 4, 3, 5, 2, 9
    g = np.random.default_rng(131)
    idx = np.array([3, 0, 4], dtype=np.int64)
    init = g.standard_normal((5, H, P, N)) * 0.3
    layer = rp.ReplayLayer(torch.from_numpy(init), W, G, torch.float64)
    A = -g.uniform(1.0, 4.0, H)
    D = g.standard_normal(H)
    pattern = [2, 0, 1, 2, 2, 0, 1]
    want_ckpt_steps = {2, 4, 6}
    kept = [[] for _ in range(R)]            # (x, dt, B, C) of every kept token
    for step, a in enumerate(pattern):
        x = g.standard_normal((R, T, H, P))
        dt = g.uniform(1e-3, 0.4, (R, T, H))
        B = g.standard_normal((R, T, G, N)) / math.sqrt(N)
        C = g.standard_normal((R, T, G, N)) / math.sqrt(N)
        before = layer.ckpt.clone()
        y = rp.replay_update(layer, idx, *(torch.from_numpy(v) for v in (x, dt)),
                             torch.from_numpy(A), torch.from_numpy(B), torch.from_numpy(C),
                             torch.from_numpy(D))
        changed = not torch.equal(before[idx], layer.ckpt[idx])
        assert changed == (step in want_ckpt_steps), (step, changed)
        for r in range(R):
            seq = kept[r] + [(x[r, t], dt[r, t], B[r, t], C[r, t]) for t in range(T)]
            xs, dts, Bs, Cs = (np.stack([e[i] for e in seq]) for i in range(4))
            yr, _, _ = oracle.recurrence(xs, dts, A, Bs, Cs, D, [0, len(seq)], 8,
                                         init=init[idx[r]][None], lib=lib)
            np.testing.assert_allclose(y[r], yr[-T:], rtol=1e-12, atol=1e-13)
            kept[r] += seq[len(kept[r]):len(kept[r]) + 1 + a]
        rp.replay_advance(layer, idx, np.full(R, a), T)
    assert all(tuple(layer.cursor[s]) == (4, 2) for s in idx)
    rp.replay_materialize(layer, idx, torch.from_numpy(A))
    assert all(tuple(layer.cursor[s]) == (6, 0) for s in idx)
    for r in range(R):
        xs, dts, Bs, Cs = (np.stack([e[i] for e in kept[r]]) for i in range(4))
        _, fr, _ = oracle.recurrence(xs, dts, A, Bs, Cs, D, [0, len(kept[r])], 8,
                                     init=init[idx[r]][None], lib=lib)
        np.testing.assert_allclose(layer.ckpt[idx[r]].numpy(), fr[0], rtol=1e-12, atol=1e-13)
    untouched = [1, 2]
    np.testing.assert_array_equal(layer.ckpt[untouched].numpy(), init[untouched])


def pin_dt_preprocess(lib=None, dtp=None):
    """The step-size preprocessing: softplus(0) = log 2, softplus(v) - softplus(-v) = v,
    agreement with torch's float64 softplus (threshold 20), the clamp, and the bias
    taken per head (last axis)."""
    f = dtp or oracle.dt_preprocess
    big = 1e30
    np.testing.assert_allclose(f(np.zeros(3), None, 0.0, big), np.full(3, math.log(2.0)),
                               rtol=0, atol=1e-15)
    v = np.linspace(-19.0, 19.0, 77)
    np.testing.assert_allclose(f(v, None, 0.0, big) - f(-v, None, 0.0, big), v, rtol=0,
                               atol=1e-12)
    g = np.random.default_rng(141)
    raw = g.standard_normal((5, 4)) * 8.0
    bias = g.uniform(-3.0, 3.0, 4)
    want = torch.nn.functional.softplus(torch.from_numpy(raw + bias)).numpy()
    np.testing.assert_allclose(f(raw, bias, 0.0, big), want, rtol=1e-14, atol=1e-300)
    lo, hi = 1e-3, 0.1
    got = f(raw, bias, lo, hi)
    np.testing.assert_allclose(got, np.clip(want, lo, hi), rtol=1e-14, atol=0)
    assert got.min() >= lo and got.max() <= hi
    np.testing.assert_allclose(f(np.array([25.0]), None, 0.0, big), [25.0], rtol=0, atol=0)


def pin_varlen_update_is_prefill(lib=None):
    """The packed-varlen state update against the prefill recurrence over the same
    packed batch (every request starting from its slot): y equal; the state after
    every token equal to prefill checkpoints with chunk size 1; the written cache
    equal to prefill's write-back. Counts include an empty request."""
    counts = [3, 0, 1, 4, 2]
    R, H, P, N, G = len(counts), 4, 3, 5, 2
    Tt = sum(counts)
    x, dt, A, B, C, D = _rand(151, Tt, H, P, N, G)
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    cache = torch.from_numpy(np.random.default_rng(152).standard_normal((7, H, P, N)))
    idx = np.array([5, 1, 0, 6, 2], dtype=np.int32)
    keep = oracle.state_update_varlen(cache, idx, cu, x, dt, A, B, C, D, True, lib=lib)
    plain = oracle.state_update_varlen(cache, idx, cu, x, dt, A, B, C, D, False, lib=lib)
    init = cache[torch.from_numpy(idx.astype(np.int64))].numpy()
    yp, fp, ck = oracle.recurrence(x, dt, A, B, C, D, cu, 1, init=init,
                                   has_init=np.ones(R, np.uint8), checkpoints=True, lib=lib)
    np.testing.assert_allclose(keep["y"], yp, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(plain["y"], yp, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(keep["states"], ck, rtol=1e-12, atol=1e-14)
    assert torch.equal(keep["cache"], cache)
    for r in range(R):
        np.testing.assert_allclose(plain["cache"][idx[r]].numpy(), fp[r], rtol=1e-12, atol=1e-14)
    untouched = [3, 4]
    assert torch.equal(plain["cache"][untouched], cache[untouched])


def pin_aligned_checkpoints(lib=None):
    """Align mode: chunk cuts worked by hand; a prefix that is a multiple of Q gives
    the plain checkpoints; every aligned checkpoint equals the final state of the
    prefill truncated at that absolute position (separate recurrence calls); and a
    suffix prefill after a cached prefix reproduces the whole sequence's plain
    checkpoints at the same absolute positions."""
    assert oracle.aligned_chunks(10, 4, 6) == [(0, 2), (2, 4), (6, 4)]
    assert oracle.aligned_chunks(3, 4, 6) == [(0, 2), (2, 1)]
    assert oracle.aligned_chunks(1, 4, 7) == [(0, 1)]
    assert oracle.aligned_chunks(9, 4, 8) == [(0, 4), (4, 4), (8, 1)]
    assert oracle.aligned_chunks(0, 4, 3) == []
    assert oracle.aligned_chunks(10, 4, 5) == [(0, 3), (3, 4), (7, 3)]
    assert oracle.aligned_chunks(6, 8, 3) == [(0, 5), (5, 1)]
    assert oracle.aligned_chunks(5, 8, 21) == [(0, 3), (3, 2)]
    lens, Q = [10, 3, 0, 7], 4
    T, H, P, N, G = sum(lens), 2, 2, 3, 1
    x, dt, A, B, C, D = _rand(161, T, H, P, N, G)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cache = torch.from_numpy(np.random.default_rng(162).standard_normal((6, H, P, N)))
    idx = np.array([4, 0, 2, 5], dtype=np.int32)
    hi = np.array([1, 0, 1, 1], dtype=np.uint8)
    plain = oracle.prefill(x, dt, A, B, C, D, cu, idx, hi, cache, Q, checkpoints=True, lib=lib)
    same = oracle.prefill_aligned(x, dt, A, B, C, D, cu, idx, hi, cache, Q, [0, 8, 4, 12],
                                  lib=lib)
    np.testing.assert_allclose(same["ckpt"], plain["ckpt"], rtol=1e-12, atol=1e-14)
    prefix = [6, 1, 5, 13]
    al = oracle.prefill_aligned(x, dt, A, B, C, D, cu, idx, hi, cache, Q, prefix, lib=lib)
    np.testing.assert_allclose(al["y"], plain["y"], rtol=1e-12, atol=1e-14)
    row = 0
    for s in range(len(lens)):
        a = int(cu[s])
        init = cache[int(idx[s])].numpy()[None] if hi[s] else None
        for off, ln in oracle.aligned_chunks(lens[s], Q, prefix[s]):
            e = off + ln
            _, f, _ = oracle.recurrence(x[a:a + e], dt[a:a + e], A, B[a:a + e], C[a:a + e], D,
                                        [0, e], Q, init=init, lib=lib)
            np.testing.assert_allclose(al["ckpt"][row], f[0], rtol=1e-12, atol=1e-14)
            row += 1
    assert row == len(al["ckpt"])
    # a 16-token sequence cut after 6 cached tokens: the 10-token suffix's aligned
    # checkpoints are the whole sequence's plain ones at absolute positions 8, 12, 16
    x1, dt1, A1, B1, C1, D1 = _rand(163, 16, H, P, N, G)
    whole = oracle.recurrence(x1, dt1, A1, B1, C1, D1, [0, 16], Q, checkpoints=True, lib=lib)[2]
    _, f6, _ = oracle.recurrence(x1[:6], dt1[:6], A1, B1[:6], C1[:6], D1, [0, 6], Q, lib=lib)
    c1 = torch.from_numpy(f6)
    suf = oracle.prefill_aligned(x1[6:], dt1[6:], A1, B1[6:], C1[6:], D1, [0, 10], [0], [1], c1,
                                 Q, [6], lib=lib)
    np.testing.assert_allclose(suf["ckpt"], whole[1:], rtol=1e-12, atol=1e-14)


def pin_philox_known_answers(lib=None, rnd=None):
    """Philox4x32-10 against the generator's published known-answer vectors
    (tests/golden), and the per-element word layout of the state stores."""
    r = rnd or oracle_rounding
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        cases = json.load(f)["cases"]
    for cs in cases:
        ctr = np.array([int(v, 16) for v in cs["counter"]], dtype=np.uint32)
        key = np.array([int(v, 16) for v in cs["key"]], dtype=np.uint32)
        got = r.philox4x32(ctr, key, 10)
        assert [int(v) for v in got] == [int(v, 16) for v in cs["out"]], cs
    # element e of stream k takes the 16-bit half e % 2 (low first) of word
    # (e // 2) % 4 of the block e // 8
    seed, kind = 0x0123456789ABCDEF, 3
    d = r.draws_for(21, seed, kind, 7, first=(1 << 35) + 3)
    for j, e in enumerate(range((1 << 35) + 3, (1 << 35) + 24)):
        blk = e // 8
        ctr = np.array([blk & 0xFFFFFFFF, blk >> 32, kind, 0], dtype=np.uint32)
        key = np.array([seed & 0xFFFFFFFF, seed >> 32], dtype=np.uint32)
        word = int(r.philox4x32(ctr, key, 7)[(e // 2) % 4])
        assert int(d[j]) == (word >> (16 * (e % 2))) & 0xFFFF


def pin_stochastic_rounding(lib=None, rnd=None):
    """fp32 -> fp16 stochastic rounding: the two candidates are the fp16 values
    bracketing x (found by brute force over every finite fp16 value), the draw
    u = d / 2^16 goes up exactly when u < (|x| - |lo|) / (|hi| - |lo|), that
    probability has at most 16 fractional bits for |x| >= 2^-17 (so a 16-bit
    draw is exactly unbiased there), representable and special values pass
    unchanged or round to nearest, and the mean over random draws is x."""
    r = rnd or oracle_rounding
    allh = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    fin = np.unique(allh[np.isfinite(allh)].astype(np.float32))
    g = np.random.default_rng(171)
    x = np.concatenate([g.standard_normal(400) * 0.03, g.standard_normal(200) * 30.0,
                        g.uniform(-6e-5, 6e-5, 200), g.uniform(-3e-7, 3e-7, 50)]
                       ).astype(np.float32)
    exact = np.isin(x, fin)
    i = np.searchsorted(fin, np.abs(x), side="right") - 1      # largest magnitude <= |x|
    lo_mag, hi_mag = fin[i], fin[np.minimum(i + 1, len(fin) - 1)]
    sign = np.where(x < 0, -1.0, 1.0).astype(np.float32)
    up = r.stochastic_round_f16(x, np.zeros(len(x), np.uint32)).astype(np.float32)
    down = r.stochastic_round_f16(x, np.full(len(x), 0xFFFF, np.uint32)).astype(np.float32)
    np.testing.assert_array_equal(down, sign * lo_mag)
    np.testing.assert_array_equal(up[~exact], (sign * hi_mag)[~exact])
    np.testing.assert_array_equal(up[exact], x[exact])
    # the probability's fractional bits, measured in float64 from the bracket
    big = np.abs(x) >= 2.0 ** -17
    prob = ((np.abs(x).astype(np.float64) - lo_mag) / (hi_mag - lo_mag))[big & ~exact]
    assert np.all(prob * 2.0 ** 16 == np.floor(prob * 2.0 ** 16))
    # the threshold: x half way between neighbours goes up for u just below 1/2 only
    half = np.float32(1.0 + 2.0 ** -11)                          # fp16 ulp at 1 is 2^-10
    w_lo = np.array([2 ** 15 - 1], np.uint32)
    w_hi = np.array([2 ** 15], np.uint32)
    assert float(r.stochastic_round_f16(np.array([half]), w_lo)[0]) == 1.0 + 2.0 ** -10
    assert float(r.stochastic_round_f16(np.array([half]), w_hi)[0]) == 1.0
    assert float(r.stochastic_round_f16(np.array([-half]), w_lo)[0]) == -(1.0 + 2.0 ** -10)
    # specials: nearest even
    sp = np.array([np.inf, -np.inf, 70000.0, 65510.0, 0.0], np.float32)
    got = r.stochastic_round_f16(sp, np.zeros(5, np.uint32)).astype(np.float32)
    np.testing.assert_array_equal(got, [np.inf, -np.inf, np.inf, 65504.0, 0.0])
    assert np.isnan(r.stochastic_round_f16(np.array([np.nan], np.float32), [0])[0])
    # unbiased: 4096 random words per value
    xs = np.repeat(x[:64], 4096)
    ws = g.integers(0, 2 ** 16, size=len(xs), dtype=np.uint64).astype(np.uint32)
    mean = r.stochastic_round_f16(xs, ws).astype(np.float64).reshape(64, 4096).mean(axis=1)
    ulp = (hi_mag - lo_mag)[:64].astype(np.float64)
    assert np.all(np.abs(mean - x[:64]) <= 6 * 0.5 * ulp / 64.0 + 1e-12)


ALL_PINS = [pin_hand_worked, pin_single_token_closed_form, pin_cumsum_reduction, pin_pure_decay,
            pin_skip_only, pin_linearity, pin_dual_form, pin_continued_prefill,
            pin_varlen_packing, pin_checkpoints_are_truncated_finals,
            pin_chunk_size_independence, pin_state_update_replay, pin_cache_semantics,
            pin_bf16_rounding, pin_replay_matches_recurrence, pin_dt_preprocess,
            pin_varlen_update_is_prefill, pin_aligned_checkpoints, pin_philox_known_answers,
            pin_stochastic_rounding]
