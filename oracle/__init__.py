"""CPU oracle for the Mamba2 SSD varlen scan and the MTP selective state update.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke entry point and the
benchmark's CPU-baseline leg are the only code that may import this package.
The GPU library (``state_space_model_varlen_amd``) never imports it, and it
imports nothing from the GPU library.

Three independent references live here:

* ``ssd_oracle.c`` (float64, OpenMP over (sequence, head) pairs): the
  sequential per-token recurrence. ``prefill`` and ``state_update`` below wrap
  it and add the state-cache semantics (slot gather as a snapshot, write-back,
  rounding to the storage dtype).
* ``oracle.chunked`` (numpy float64): the five steps of the chunked scan,
  each as its plain definition, for step-by-step checks of the GPU steps.
* ``oracle.dual`` (pure Python, tiny inputs only): the quadratic form of the
  same operator with decays taken as products of per-token factors.

Where each piece is pinned (closed forms, brute force, invariants) is in
``tests/test_oracle_pins.py``. Absolute values are not printed on the pages:
no worked example exists, so there is no page-printed fixture to pin to
("parity unpinned by the pages"; the pins are mathematical).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile ``ssd_oracle.c`` with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
                               "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def load_lib(path: str):
    """Load a compiled copy of ssd_oracle.c (the default build, or a copy a test built)."""
    lib = ctypes.CDLL(path)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    lib.ssd_oracle_prefill.argtypes = [i64] * 7 + [vp] * 12 + [i32]
    lib.ssd_oracle_prefill.restype = i32
    lib.ssd_oracle_state_update.argtypes = [i64] * 6 + [vp] * 10 + [i32]
    lib.ssd_oracle_state_update.restype = i32
    lib.ssd_oracle_max_threads.restype = i32
    return lib


def _load(lib=None):
    global _lib
    if lib is not None:
        return lib
    if _lib is None:
        build()
        _lib = load_lib(_LIB_PATH)
    return _lib


def max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def f64(a) -> np.ndarray:
    """Exact widening of a torch tensor (any float dtype) or array to float64."""
    if isinstance(a, torch.Tensor):
        return np.ascontiguousarray(a.detach().cpu().to(torch.float64).numpy())
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def round_to(a, dtype: torch.dtype) -> torch.Tensor:
    """Round float64 values to a storage dtype (round to nearest even, via torch)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    return t.to(dtype)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def chunk_counts(cu_seqlens, Q: int) -> np.ndarray:
    """chunk_cu: exclusive prefix sum of ceil(L_s / Q), length S + 1."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    lens = np.diff(cu)
    out = np.zeros(len(cu), dtype=np.int64)
    out[1:] = np.cumsum((lens + Q - 1) // Q)
    return out


def recurrence(x, dt, A, B, C, D, cu_seqlens, chunk_size: int, init=None, has_init=None,
               checkpoints: bool = False, nthreads: int = 0, lib=None):
    """The sequential recurrence over a packed batch (float64).

    x [T,H,P], dt [T,H], A [H], B/C [T,G,N], D [H] or None, cu_seqlens [S+1],
    init [S,H,P,N] or None, has_init [S] or None.
    Returns y [T,H,P], final [S,H,P,N], ckpt [nc,H,P,N] or None.
    """
    x, dt, A, B, C = f64(x), f64(dt), f64(A), f64(B), f64(C)
    D = None if D is None else f64(D)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    S = len(cu) - 1
    init64 = None if init is None else f64(init)
    hi = None if has_init is None else np.ascontiguousarray(np.asarray(has_init, dtype=np.uint8))
    y = np.zeros((T, H, P))
    final = np.zeros((S, H, P, N))
    nc = int(chunk_counts(cu, chunk_size)[-1])
    ckpt = np.zeros((nc, H, P, N)) if checkpoints else None
    rc = _load(lib).ssd_oracle_prefill(T, S, H, P, N, G, int(chunk_size), _ptr(x), _ptr(dt), _ptr(A),
                                    _ptr(B), _ptr(C), _ptr(D), _ptr(cu), _ptr(init64), _ptr(hi),
                                    _ptr(y), _ptr(final), _ptr(ckpt), int(nthreads))
    if rc != 0:
        raise ValueError("ssd_oracle_prefill rejected its arguments")
    return y, final, ckpt


def prefill(x, dt, A, B, C, D, cu_seqlens, state_indices, has_initial, cache: torch.Tensor,
            chunk_size: int, checkpoints: bool = False, nthreads: int = 0, lib=None):
    """One varlen prefill against a slot-indexed state cache.

    Every initial state is read from the cache as it was before the call
    (a snapshot; vLLM PR #62922, section "Details"); sequences whose
    has_initial flag is 0, or all of them when ``has_initial`` is None, start
    from zero and never read their slot (vLLM PR #61501, section "Details":
    gather only when some sequence has an initial state, otherwise start from a
    zero state). Each final state is rounded to the cache dtype and scattered
    into the sequence's slot; the other slots keep their contents.

    Returns dict(y=float64, final=float64, ckpt=float64 or None,
    cache=torch tensor after the call, in the cache dtype).
    """
    idx = np.asarray(state_indices, dtype=np.int64)
    S = len(idx)
    init = None
    hi = None
    if has_initial is not None:
        hi = np.asarray(has_initial, dtype=np.uint8)
        init = f64(cache[torch.from_numpy(idx)]) if S else np.zeros((0,) + tuple(cache.shape[1:]))
        # a sequence without an initial state does not read its slot: zero it here
        init[hi == 0] = 0.0
    y, final, ckpt = recurrence(x, dt, A, B, C, D, cu_seqlens, chunk_size, init, hi,
                                checkpoints, nthreads, lib)
    after = cache.clone()
    if S:
        after[torch.from_numpy(idx)] = round_to(final, cache.dtype)
    return dict(y=y, final=final, ckpt=ckpt, cache=after)


def aligned_chunks(L: int, Q: int, prefix_len: int):
    """(offset, length) of each chunk of an L-token sequence that follows
    prefix_len cached tokens, cut at absolute token positions that are multiples
    of Q (align mode, vLLM PR #55688 "Summary"): the first chunk runs to the next
    multiple of Q, the others are Q long, the last may be partial."""
    o = prefix_len % Q if prefix_len > 0 else 0
    first = Q - o if o else Q
    out, pos = [], 0
    while pos < L:
        ln = min(first if pos == 0 else Q, L - pos)
        out.append((pos, ln))
        pos += ln
    return out


def prefill_aligned(x, dt, A, B, C, D, cu_seqlens, state_indices, has_initial,
                    cache: torch.Tensor, chunk_size: int, prefix_lens, lib=None):
    """Align-mode prefill: as ``prefill``, with the checkpoint of every chunk cut by
    ``aligned_chunks`` (the state after the chunk's last token), in packed chunk
    order. The states come from the recurrence run with a checkpoint after every
    token (chunk size 1)."""
    out = prefill(x, dt, A, B, C, D, cu_seqlens, state_indices, has_initial, cache,
                  chunk_size, lib=lib)
    per_token = prefill(x, dt, A, B, C, D, cu_seqlens, state_indices, has_initial, cache, 1,
                        checkpoints=True, lib=lib)["ckpt"]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    rows, base = [], 0
    for s in range(len(cu) - 1):
        L = max(int(cu[s + 1] - cu[s]), 0)
        for off, ln in aligned_chunks(L, chunk_size, int(prefix_lens[s])):
            rows.append(per_token[base + off + ln - 1])
        base += L
    shape = (0,) + tuple(per_token.shape[1:])
    out["ckpt"] = np.stack(rows) if rows else np.zeros(shape)
    return out


def state_update(cache: torch.Tensor, state_indices, x, dt, A, B, C, D, keep_states: bool,
                 nthreads: int = 0, lib=None):
    """Decode / MTP verify: per request, continue from cache[state_indices[r]].

    x [R,T,H,P], dt [R,T,H], B/C [R,T,G,N]. With ``keep_states`` the state after
    every token is returned (the intermediate states a rollback reads) and the
    cache is not written; without it the state after the last token is rounded
    to the cache dtype and written to the request's slot.

    Returns dict(y=float64 [R,T,H,P], states=float64 [R,T,H,P,N] or None,
    final=float64 [R,H,P,N], cache=torch tensor after the call).
    """
    idx = np.asarray(state_indices, dtype=np.int64)
    x, dt, A, B, C = f64(x), f64(dt), f64(A), f64(B), f64(C)
    D = None if D is None else f64(D)
    R, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    init = f64(cache[torch.from_numpy(idx)]) if R else np.zeros((0, H, P, N))
    y = np.zeros((R, T, H, P))
    states = np.zeros((R, T, H, P, N)) if keep_states else None
    final = np.zeros((R, H, P, N))
    rc = _load(lib).ssd_oracle_state_update(R, T, H, P, N, G, _ptr(init), _ptr(x), _ptr(dt),
                                         _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(y),
                                         _ptr(states), _ptr(final), int(nthreads))
    if rc != 0:
        raise ValueError("ssd_oracle_state_update rejected its arguments")
    after = cache.clone()
    if not keep_states and R:
        after[torch.from_numpy(idx)] = round_to(final, cache.dtype)
    return dict(y=y, states=states, final=final, cache=after)


def dt_preprocess(dt_raw, dt_bias, dt_min: float, dt_max: float) -> np.ndarray:
    """The layer's step-size preprocessing in float64 (the step size of the pages'
    workload, vLLM PR #52928 "Summary"): clamp(softplus(dt_raw + dt_bias_h),
    dt_min, dt_max), softplus(v) = log(1 + exp(v)), taken as v itself above 20
    (the kernels' convention). dt_raw [..., H]; dt_bias [H] or None."""
    v = f64(dt_raw)
    if dt_bias is not None:
        v = v + f64(dt_bias)
    sp = np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))
    return np.minimum(np.maximum(sp, float(dt_min)), float(dt_max))


def state_update_varlen(cache: torch.Tensor, state_indices, cu_seqlens, x, dt, A, B, C, D,
                        keep_states: bool, lib=None):
    """Packed-varlen verify: request r owns packed tokens cu[r] .. cu[r+1]-1 and
    continues from cache[state_indices[r]]; each request is the state update above
    over its own tokens (a request with no token changes nothing).

    x [Tt,H,P], dt [Tt,H], B/C [Tt,G,N]. Returns dict(y [Tt,H,P], states
    [Tt,H,P,N] or None, cache after the call)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    x, dt, B, C = f64(x), f64(dt), f64(B), f64(C)
    Tt, H, P = x.shape
    N = B.shape[2]
    y = np.zeros((Tt, H, P))
    states = np.zeros((Tt, H, P, N)) if keep_states else None
    after = cache.clone()
    for r, slot in enumerate(np.asarray(state_indices, dtype=np.int64)):
        a, b = int(cu[r]), int(cu[r + 1])
        if b <= a:
            continue
        out = state_update(cache, [slot], x[None, a:b], dt[None, a:b], A, B[None, a:b],
                           C[None, a:b], D, keep_states, lib=lib)
        y[a:b] = out["y"][0]
        if keep_states:
            states[a:b] = out["states"][0]
        else:
            after[int(slot)] = out["cache"][int(slot)]
    return dict(y=y, states=states, cache=after)


def commit(cache: torch.Tensor, state_indices, replay: torch.Tensor, num_accepted) -> torch.Tensor:
    """Rollback to the accepted count: cache[idx[r]] = replay[r, a_r] (a copy)."""
    after = cache.clone()
    for r, (slot, a) in enumerate(zip(np.asarray(state_indices), np.asarray(num_accepted))):
        after[int(slot)] = replay[r, int(a)]
    return after
