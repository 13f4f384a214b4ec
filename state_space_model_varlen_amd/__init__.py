"""Python binding of the MI355X SSD library (``libssd_mi355x.so``, C ABI in
``include/ssd_mi355x.h``).

Argument marshalling only: every function checks the torch tensors it is
given against the problem sizes (device, dtype, shape, contiguity), passes
their device pointers and the current HIP stream to the C entry point of the
same name, and raises on a non-zero status. All arithmetic runs in the HIP
kernels; there is no CPU or PyTorch fallback - importing this package fails
loudly when the library has not been built.

Layouts (row-major): x, y [T,H,P]; dt [T,H]; A, D [H] float32; B, C [T,G,N];
cu_seqlens [S+1] int32; state_indices [S] int32; has_initial_state [S] uint8;
state cache [num_slots,H,P,N]; checkpoints [max_chunks,H,P,N].
Decode: x, y [R,T,H,P]; dt [R,T,H]; B, C [R,T,G,N]; intermediate states
[R,T,H,P,N]; num_accepted [R] int32.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssd_mi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python state_space_model_varlen_amd/_build.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

SSD_OK = 0
F32, BF16, F16 = 0, 1, 2
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
_TORCH = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}


class ssd_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "total_tokens", "num_seqs", "nheads", "headdim", "d_state", "ngroups", "chunk_size",
        "num_slots", "in_dtype", "state_dtype")]


class ssu_problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_reqs", "tokens_per_req", "nheads", "headdim", "d_state", "ngroups", "num_slots",
        "in_dtype", "state_dtype")]


class ssd_dt_transform(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("dt_min", ctypes.c_float),
                ("dt_max", ctypes.c_float)]


TRACE_MAX_LAUNCHES = 16


class ssd_launch_trace(ctypes.Structure):
    _fields_ = [("events", ctypes.POINTER(ctypes.c_void_p)), ("capacity", ctypes.c_int32),
                ("count", ctypes.c_int32), ("names", ctypes.c_char_p * TRACE_MAX_LAUNCHES)]


class ssd_options(ctypes.Structure):
    _fields_ = [("dt_transform", ctypes.c_void_p), ("prefix_lens", ctypes.c_void_p),
                ("sr_seed", ctypes.c_void_p), ("sr_rounds", ctypes.c_int32),
                ("trace", ctypes.POINTER(ssd_launch_trace))]


_vp = ctypes.c_void_p
_pp = ctypes.POINTER(ssd_problem)
_up = ctypes.POINTER(ssu_problem)
_tp = ctypes.POINTER(ssd_dt_transform)
_SIGS = {
    "ssd_abi_version": ([], ctypes.c_int),
    "ssd_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "ssd_max_chunks": ([_pp], ctypes.c_int64),
    "ssd_chunk_meta_count": ([_pp], ctypes.c_int64),
    "ssd_workspace_bytes": ([_pp], ctypes.c_size_t),
    "ssd_chunk_cumsum": ([_pp] + [_vp] * 7, ctypes.c_int),
    "ssd_chunk_state": ([_pp] + [_vp] * 7, ctypes.c_int),
    "ssd_state_passing": ([_pp] + [_vp] * 9, ctypes.c_int),
    "ssd_chunk_state_passing": ([_pp] + [_vp] * 11, ctypes.c_int),
    "ssd_bmm_chunk": ([_pp] + [_vp] * 5, ctypes.c_int),
    "ssd_chunk_scan": ([_pp] + [_vp] * 10, ctypes.c_int),
    "ssd_combined_varlen": ([_pp] + [_vp] * 13 + [ctypes.c_size_t, _vp], ctypes.c_int),
    "selective_state_update": ([_up] + [_vp] * 11, ctypes.c_int),
    "ssd_state_commit": ([_up] + [_vp] * 5, ctypes.c_int),
    "ssd_max_chunks_aligned": ([_pp], ctypes.c_int64),
    "ssd_workspace_bytes_aligned": ([_pp], ctypes.c_size_t),
    "ssd_combined_varlen_aligned": ([_pp] + [_vp] * 14 + [ctypes.c_size_t, _vp], ctypes.c_int),
    "ssd_chunk_cumsum_dt": ([_pp, _tp] + [_vp] * 7, ctypes.c_int),
    "ssd_combined_varlen_ex": ([_pp, ctypes.POINTER(ssd_options)] + [_vp] * 13
                               + [ctypes.c_size_t, _vp], ctypes.c_int),
    "selective_state_update_ex": ([_up, ctypes.POINTER(ssd_options), ctypes.c_int32]
                                  + [_vp] * 12, ctypes.c_int),
    "ssd_round_f16": ([_vp, _vp, ctypes.c_int64, _vp, ctypes.c_int32, ctypes.c_int32, _vp],
                      ctypes.c_int),
    "ssd_replay_update_ex": ([_up, ctypes.POINTER(ssd_options), ctypes.c_int32] + [_vp] * 14,
                             ctypes.c_int),
    "ssd_replay_materialize_ex": ([_up, ctypes.POINTER(ssd_options), ctypes.c_int32] + [_vp] * 8,
                                  ctypes.c_int),
    "ssd_combined_varlen_dt": ([_pp, _tp] + [_vp] * 13 + [ctypes.c_size_t, _vp], ctypes.c_int),
    "selective_state_update_varlen": ([_up, ctypes.c_int32, _vp, _tp] + [_vp] * 11, ctypes.c_int),
    "ssd_state_commit_varlen": ([_up, ctypes.c_int32] + [_vp] * 6, ctypes.c_int),
    "ssd_replay_update": ([_up, ctypes.c_int32] + [_vp] * 14, ctypes.c_int),
    "ssd_replay_advance": ([_up, ctypes.c_int32] + [_vp] * 4, ctypes.c_int),
    "ssd_replay_materialize": ([_up, ctypes.c_int32] + [_vp] * 8, ctypes.c_int),
    "ssd_noalloc_scratch_bytes": ([], ctypes.c_size_t),
    "ssd_combined_varlen_noalloc": ([_pp] + [_vp] * 13, ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_SIGS)


class SSDError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} (status {status})")
        self.status = status


def abi_version() -> int:
    return int(_lib.ssd_abi_version())


def status_string(status: int) -> str:
    return _lib.ssd_status_string(int(status)).decode()


# ---------------------------------------------------------------------------
# problem descriptors

def make_problem(total_tokens: int, num_seqs: int, nheads: int, headdim: int, d_state: int,
                 ngroups: int, chunk_size: int, num_slots: int, in_dtype: torch.dtype,
                 state_dtype: torch.dtype) -> ssd_problem:
    return ssd_problem(int(total_tokens), int(num_seqs), int(nheads), int(headdim), int(d_state),
                       int(ngroups), int(chunk_size), int(num_slots), _DT[in_dtype],
                       _DT[state_dtype])


def make_ssu_problem(num_reqs: int, tokens_per_req: int, nheads: int, headdim: int, d_state: int,
                     ngroups: int, num_slots: int, in_dtype: torch.dtype,
                     state_dtype: torch.dtype) -> ssu_problem:
    return ssu_problem(int(num_reqs), int(tokens_per_req), int(nheads), int(headdim),
                       int(d_state), int(ngroups), int(num_slots), _DT[in_dtype],
                       _DT[state_dtype])


def max_chunks(p: ssd_problem) -> int:
    return int(_lib.ssd_max_chunks(ctypes.byref(p)))


def chunk_meta_count(p: ssd_problem) -> int:
    return int(_lib.ssd_chunk_meta_count(ctypes.byref(p)))


def workspace_bytes(p: ssd_problem) -> int:
    return int(_lib.ssd_workspace_bytes(ctypes.byref(p)))


# ---------------------------------------------------------------------------
# marshalling helpers

def _stream(stream) -> _vp:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return _vp(stream.cuda_stream)
    return _vp(int(stream))


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, shape=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _vp(t.data_ptr()) if t.numel() else _vp(t.data_ptr() or 16)


def _check(fn: str, rc: int):
    if rc != SSD_OK:
        raise SSDError(fn, rc)


def _dims(p: ssd_problem):
    return (p.total_tokens, p.num_seqs, p.nheads, p.headdim, p.d_state, p.ngroups, p.chunk_size,
            max_chunks(p))


# ---------------------------------------------------------------------------
# prefill steps

def ssd_chunk_cumsum(p: ssd_problem, dt, A, cu_seqlens, chunk_meta, dA_cumsum, dt_chunk,
                     stream=None):
    T, S, H, P, N, G, Q, mc = _dims(p)
    ti = _TORCH[p.in_dtype]
    rc = _lib.ssd_chunk_cumsum(
        ctypes.byref(p), _ptr(dt, "dt", ti, (T, H)), _ptr(A, "A", torch.float32, (H,)),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32, (S + 1,)),
        _ptr(chunk_meta, "chunk_meta", torch.int32, (chunk_meta_count(p),)),
        _ptr(dA_cumsum, "dA_cumsum", torch.float32, (H, mc, Q)),
        _ptr(dt_chunk, "dt_chunk", torch.float32, (H, mc, Q)), _stream(stream))
    _check("ssd_chunk_cumsum", rc)


def ssd_chunk_state(p: ssd_problem, x, B, chunk_meta, dA_cumsum, dt_chunk, chunk_states,
                    stream=None):
    T, S, H, P, N, G, Q, mc = _dims(p)
    ti = _TORCH[p.in_dtype]
    rc = _lib.ssd_chunk_state(
        ctypes.byref(p), _ptr(x, "x", ti, (T, H, P)), _ptr(B, "B", ti, (T, G, N)),
        _ptr(chunk_meta, "chunk_meta", torch.int32, (chunk_meta_count(p),)),
        _ptr(dA_cumsum, "dA_cumsum", torch.float32, (H, mc, Q)),
        _ptr(dt_chunk, "dt_chunk", torch.float32, (H, mc, Q)),
        _ptr(chunk_states, "chunk_states", torch.float32, (mc, H, P, N)), _stream(stream))
    _check("ssd_chunk_state", rc)


def ssd_state_passing(p: ssd_problem, chunk_states, dA_cumsum, chunk_meta, state_cache,
                      state_indices, has_initial_state, entering_states, checkpoints=None,
                      stream=None):
    T, S, H, P, N, G, Q, mc = _dims(p)
    ts = _TORCH[p.state_dtype]
    rc = _lib.ssd_state_passing(
        ctypes.byref(p), _ptr(chunk_states, "chunk_states", torch.float32, (mc, H, P, N)),
        _ptr(dA_cumsum, "dA_cumsum", torch.float32, (H, mc, Q)),
        _ptr(chunk_meta, "chunk_meta", torch.int32, (chunk_meta_count(p),)),
        _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (S,)),
        _ptr(has_initial_state, "has_initial_state", torch.uint8, (S,), optional=True),
        _ptr(entering_states, "entering_states", _TORCH[p.in_dtype], (mc, H, P, N)),
        _ptr(checkpoints, "checkpoints", ts, (mc, H, P, N), optional=True), _stream(stream))
    _check("ssd_state_passing", rc)


def ssd_chunk_state_passing(p: ssd_problem, x, B, chunk_meta, dA_cumsum, dt_chunk,
                            state_cache, state_indices, has_initial_state, entering_states,
                            checkpoints=None, stream=None):
    T, S, H, P, N, G, Q, mc = _dims(p)
    ti, ts = _TORCH[p.in_dtype], _TORCH[p.state_dtype]
    rc = _lib.ssd_chunk_state_passing(
        ctypes.byref(p), _ptr(x, "x", ti, (T, H, P)), _ptr(B, "B", ti, (T, G, N)),
        _ptr(chunk_meta, "chunk_meta", torch.int32, (chunk_meta_count(p),)),
        _ptr(dA_cumsum, "dA_cumsum", torch.float32, (H, mc, Q)),
        _ptr(dt_chunk, "dt_chunk", torch.float32, (H, mc, Q)),
        _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (S,)),
        _ptr(has_initial_state, "has_initial_state", torch.uint8, (S,), optional=True),
        _ptr(entering_states, "entering_states", ti, (mc, H, P, N)),
        _ptr(checkpoints, "checkpoints", ts, (mc, H, P, N), optional=True), _stream(stream))
    _check("ssd_chunk_state_passing", rc)


def ssd_bmm_chunk(p: ssd_problem, B, C, chunk_meta, CB, stream=None):
    T, S, H, P, N, G, Q, mc = _dims(p)
    ti = _TORCH[p.in_dtype]
    rc = _lib.ssd_bmm_chunk(
        ctypes.byref(p), _ptr(B, "B", ti, (T, G, N)), _ptr(C, "C", ti, (T, G, N)),
        _ptr(chunk_meta, "chunk_meta", torch.int32, (chunk_meta_count(p),)),
        _ptr(CB, "CB", ti, (mc, G, Q, Q)), _stream(stream))
    _check("ssd_bmm_chunk", rc)


def ssd_chunk_scan(p: ssd_problem, x, C, D, chunk_meta, dA_cumsum, dt_chunk, CB,
                   entering_states, y, stream=None):
    T, S, H, P, N, G, Q, mc = _dims(p)
    ti = _TORCH[p.in_dtype]
    rc = _lib.ssd_chunk_scan(
        ctypes.byref(p), _ptr(x, "x", ti, (T, H, P)), _ptr(C, "C", ti, (T, G, N)),
        _ptr(D, "D", torch.float32, (H,), optional=True),
        _ptr(chunk_meta, "chunk_meta", torch.int32, (chunk_meta_count(p),)),
        _ptr(dA_cumsum, "dA_cumsum", torch.float32, (H, mc, Q)),
        _ptr(dt_chunk, "dt_chunk", torch.float32, (H, mc, Q)),
        _ptr(CB, "CB", ti, (mc, G, Q, Q)),
        _ptr(entering_states, "entering_states", ti, (mc, H, P, N)),
        _ptr(y, "y", ti, (T, H, P)), _stream(stream))
    _check("ssd_chunk_scan", rc)


def ssd_combined_varlen(p: ssd_problem, x, dt, A, B, C, D, cu_seqlens, state_cache,
                        state_indices, has_initial_state, y, checkpoints, workspace,
                        stream=None):
    T, S, H, P, N, G, Q, mc = _dims(p)
    ti, ts = _TORCH[p.in_dtype], _TORCH[p.state_dtype]
    if workspace is None or workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 GPU tensor")
    rc = _lib.ssd_combined_varlen(
        ctypes.byref(p), _ptr(x, "x", ti, (T, H, P)), _ptr(dt, "dt", ti, (T, H)),
        _ptr(A, "A", torch.float32, (H,)), _ptr(B, "B", ti, (T, G, N)),
        _ptr(C, "C", ti, (T, G, N)), _ptr(D, "D", torch.float32, (H,), optional=True),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32, (S + 1,)),
        _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (S,)),
        _ptr(has_initial_state, "has_initial_state", torch.uint8, (S,), optional=True),
        _ptr(y, "y", ti, (T, H, P)),
        _ptr(checkpoints, "checkpoints", ts, (mc, H, P, N), optional=True),
        _ptr(workspace, "workspace", torch.uint8), ctypes.c_size_t(workspace.numel()),
        _stream(stream))
    _check("ssd_combined_varlen", rc)


def noalloc_scratch_bytes() -> int:
    """Bytes of the static scratch array of ssd_combined_varlen_noalloc."""
    return int(_lib.ssd_noalloc_scratch_bytes())


def ssd_combined_varlen_noalloc(p: ssd_problem, x, dt, A, B, C, D, cu_seqlens, state_cache,
                                state_indices, has_initial_state, y, checkpoints, stream=None):
    """ssd_combined_varlen with the library's static scratch array as its workspace
    (no allocation; problems needing more than noalloc_scratch_bytes() are rejected)."""
    T, S, H, P, N, G, Q, mc = _dims(p)
    ti, ts = _TORCH[p.in_dtype], _TORCH[p.state_dtype]
    rc = _lib.ssd_combined_varlen_noalloc(
        ctypes.byref(p), _ptr(x, "x", ti, (T, H, P)), _ptr(dt, "dt", ti, (T, H)),
        _ptr(A, "A", torch.float32, (H,)), _ptr(B, "B", ti, (T, G, N)),
        _ptr(C, "C", ti, (T, G, N)), _ptr(D, "D", torch.float32, (H,), optional=True),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32, (S + 1,)),
        _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (S,)),
        _ptr(has_initial_state, "has_initial_state", torch.uint8, (S,), optional=True),
        _ptr(y, "y", ti, (T, H, P)),
        _ptr(checkpoints, "checkpoints", ts, (mc, H, P, N), optional=True),
        _stream(stream))
    _check("ssd_combined_varlen_noalloc", rc)


# ---------------------------------------------------------------------------
# decode / MTP

def selective_state_update(p: ssu_problem, state_cache, state_indices, x, dt, A, B, C, D, y,
                           intermediate_states=None, stream=None):
    R, T, H, P, N, G = (p.num_reqs, p.tokens_per_req, p.nheads, p.headdim, p.d_state, p.ngroups)
    ti, ts = _TORCH[p.in_dtype], _TORCH[p.state_dtype]
    rc = _lib.selective_state_update(
        ctypes.byref(p), _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (R,)),
        _ptr(x, "x", ti, (R, T, H, P)), _ptr(dt, "dt", ti, (R, T, H)),
        _ptr(A, "A", torch.float32, (H,)), _ptr(B, "B", ti, (R, T, G, N)),
        _ptr(C, "C", ti, (R, T, G, N)), _ptr(D, "D", torch.float32, (H,), optional=True),
        _ptr(y, "y", ti, (R, T, H, P)),
        _ptr(intermediate_states, "intermediate_states", ts, (R, T, H, P, N), optional=True),
        _stream(stream))
    _check("selective_state_update", rc)


def ssd_state_commit(p: ssu_problem, state_cache, state_indices, intermediate_states,
                     num_accepted, stream=None):
    R, T, H, P, N = p.num_reqs, p.tokens_per_req, p.nheads, p.headdim, p.d_state
    ts = _TORCH[p.state_dtype]
    rc = _lib.ssd_state_commit(
        ctypes.byref(p), _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (R,)),
        _ptr(intermediate_states, "intermediate_states", ts, (R, T, H, P, N)),
        _ptr(num_accepted, "num_accepted", torch.int32, (R,)), _stream(stream))
    _check("ssd_state_commit", rc)


# ---------------------------------------------------------------------------
# align-mode prefill: chunk boundaries at absolute multiples of the chunk size

def max_chunks_aligned(p: ssd_problem) -> int:
    return int(_lib.ssd_max_chunks_aligned(ctypes.byref(p)))


def workspace_bytes_aligned(p: ssd_problem) -> int:
    return int(_lib.ssd_workspace_bytes_aligned(ctypes.byref(p)))


def alloc_workspace_aligned(p: ssd_problem, device="cuda") -> torch.Tensor:
    n = workspace_bytes_aligned(p)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def ssd_combined_varlen_aligned(p: ssd_problem, prefix_lens, x, dt, A, B, C, D, cu_seqlens,
                                state_cache, state_indices, has_initial_state, y, checkpoints,
                                workspace, stream=None):
    T, S, H, P, N, G, Q, _ = _dims(p)
    mc = max_chunks_aligned(p)
    ti, ts = _TORCH[p.in_dtype], _TORCH[p.state_dtype]
    if workspace is None or workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 GPU tensor")
    rc = _lib.ssd_combined_varlen_aligned(
        ctypes.byref(p), _ptr(prefix_lens, "prefix_lens", torch.int32, (S,)),
        _ptr(x, "x", ti, (T, H, P)), _ptr(dt, "dt", ti, (T, H)),
        _ptr(A, "A", torch.float32, (H,)), _ptr(B, "B", ti, (T, G, N)),
        _ptr(C, "C", ti, (T, G, N)), _ptr(D, "D", torch.float32, (H,), optional=True),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32, (S + 1,)),
        _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (S,)),
        _ptr(has_initial_state, "has_initial_state", torch.uint8, (S,), optional=True),
        _ptr(y, "y", ti, (T, H, P)),
        _ptr(checkpoints, "checkpoints", ts, (mc, H, P, N), optional=True),
        _ptr(workspace, "workspace", torch.uint8), ctypes.c_size_t(workspace.numel()),
        _stream(stream))
    _check("ssd_combined_varlen_aligned", rc)


# ---------------------------------------------------------------------------
# dt preprocessing fused into the kernels, packed-varlen MTP verify

def make_dt_transform(dt_bias, dt_min: float, dt_max: float) -> ssd_dt_transform:
    """dt = clamp(softplus(dt_raw + dt_bias[h]), dt_min, dt_max). dt_bias: [H] float32
    GPU tensor or None; the returned struct holds a reference to it, so the device
    memory stays valid as long as the struct is alive."""
    t = ssd_dt_transform()
    t.dt_bias = None if dt_bias is None else _ptr(dt_bias, "dt_bias", torch.float32)
    t.dt_min, t.dt_max = float(dt_min), float(dt_max)
    t._dt_bias_tensor = dt_bias
    return t


def ssd_chunk_cumsum_dt(p: ssd_problem, dt_transform: ssd_dt_transform, dt_raw, A, cu_seqlens,
                        chunk_meta, dA_cumsum, dt_chunk, stream=None):
    T, S, H, P, N, G, Q, mc = _dims(p)
    ti = _TORCH[p.in_dtype]
    rc = _lib.ssd_chunk_cumsum_dt(
        ctypes.byref(p), ctypes.byref(dt_transform), _ptr(dt_raw, "dt_raw", ti, (T, H)),
        _ptr(A, "A", torch.float32, (H,)), _ptr(cu_seqlens, "cu_seqlens", torch.int32, (S + 1,)),
        _ptr(chunk_meta, "chunk_meta", torch.int32, (chunk_meta_count(p),)),
        _ptr(dA_cumsum, "dA_cumsum", torch.float32, (H, mc, Q)),
        _ptr(dt_chunk, "dt_chunk", torch.float32, (H, mc, Q)), _stream(stream))
    _check("ssd_chunk_cumsum_dt", rc)


def ssd_combined_varlen_dt(p: ssd_problem, dt_transform: ssd_dt_transform, x, dt_raw, A, B, C, D,
                           cu_seqlens, state_cache, state_indices, has_initial_state, y,
                           checkpoints, workspace, stream=None):
    T, S, H, P, N, G, Q, mc = _dims(p)
    ti, ts = _TORCH[p.in_dtype], _TORCH[p.state_dtype]
    if workspace is None or workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 GPU tensor")
    rc = _lib.ssd_combined_varlen_dt(
        ctypes.byref(p), ctypes.byref(dt_transform), _ptr(x, "x", ti, (T, H, P)),
        _ptr(dt_raw, "dt_raw", ti, (T, H)), _ptr(A, "A", torch.float32, (H,)),
        _ptr(B, "B", ti, (T, G, N)), _ptr(C, "C", ti, (T, G, N)),
        _ptr(D, "D", torch.float32, (H,), optional=True),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32, (S + 1,)),
        _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (S,)),
        _ptr(has_initial_state, "has_initial_state", torch.uint8, (S,), optional=True),
        _ptr(y, "y", ti, (T, H, P)),
        _ptr(checkpoints, "checkpoints", ts, (mc, H, P, N), optional=True),
        _ptr(workspace, "workspace", torch.uint8), ctypes.c_size_t(workspace.numel()),
        _stream(stream))
    _check("ssd_combined_varlen_dt", rc)


def selective_state_update_varlen(p: ssu_problem, cu_seqlens, state_cache, state_indices, x, dt,
                                  A, B, C, D, y, intermediate_states=None, dt_transform=None,
                                  stream=None):
    """Packed-varlen verify: x [T_tot,H,P] etc., request r owning rows cu[r] .. cu[r+1]-1."""
    R, H, P, N, G = p.num_reqs, p.nheads, p.headdim, p.d_state, p.ngroups
    ti, ts = _TORCH[p.in_dtype], _TORCH[p.state_dtype]
    Tt = int(x.shape[0])
    rc = _lib.selective_state_update_varlen(
        ctypes.byref(p), Tt, _ptr(cu_seqlens, "cu_seqlens", torch.int32, (R + 1,)),
        None if dt_transform is None else ctypes.byref(dt_transform),
        _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (R,)),
        _ptr(x, "x", ti, (Tt, H, P)), _ptr(dt, "dt", ti, (Tt, H)),
        _ptr(A, "A", torch.float32, (H,)), _ptr(B, "B", ti, (Tt, G, N)),
        _ptr(C, "C", ti, (Tt, G, N)), _ptr(D, "D", torch.float32, (H,), optional=True),
        _ptr(y, "y", ti, (Tt, H, P)),
        _ptr(intermediate_states, "intermediate_states", ts, (Tt, H, P, N), optional=True),
        _stream(stream))
    _check("selective_state_update_varlen", rc)


def ssd_state_commit_varlen(p: ssu_problem, cu_seqlens, state_cache, state_indices,
                            intermediate_states, num_accepted, stream=None):
    R, H, P, N = p.num_reqs, p.nheads, p.headdim, p.d_state
    ts = _TORCH[p.state_dtype]
    Tt = int(intermediate_states.shape[0])
    rc = _lib.ssd_state_commit_varlen(
        ctypes.byref(p), Tt, _ptr(cu_seqlens, "cu_seqlens", torch.int32, (R + 1,)),
        _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (R,)),
        _ptr(intermediate_states, "intermediate_states", ts, (Tt, H, P, N)),
        _ptr(num_accepted, "num_accepted", torch.int32, (R,)), _stream(stream))
    _check("ssd_state_commit_varlen", rc)


# ---------------------------------------------------------------------------
# options: dt preprocessing, align mode, stochastic rounding of fp16 states

def make_options(dt_transform=None, prefix_lens=None, sr_seed=None, sr_rounds: int = 10,
                 trace=None):
    """ssd_options; sr_seed: a 1-element int64 GPU tensor (read by the kernels, so it can
    be refreshed per step); trace: a LaunchTrace. The struct keeps references to the
    objects it points at."""
    o = ssd_options()
    o.dt_transform = None if dt_transform is None else ctypes.addressof(dt_transform)
    o.prefix_lens = None if prefix_lens is None else _ptr(prefix_lens, "prefix_lens", torch.int32)
    o.sr_seed = None if sr_seed is None else _ptr(sr_seed, "sr_seed", torch.int64, (1,))
    o.sr_rounds = int(sr_rounds) if sr_seed is not None else 0
    o.trace = None if trace is None else ctypes.pointer(trace.struct)
    o._refs = (dt_transform, prefix_lens, sr_seed, trace)
    return o


class LaunchTrace:
    """Per-launch timing of a prefill call (ssd_launch_trace): two HIP events per
    kernel launch, on which the launch records its own start and end. The events
    are created without the system-scope fence that HIP events carry by default
    (hipEventDisableSystemFence), so recording them does not write back the caches
    between the launches and the intervals are the kernels' own. After the call
    and a synchronisation, ``durations_us()`` gives (name, us) per launch."""

    _DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence

    def __init__(self, capacity: int = 2 * TRACE_MAX_LAUNCHES):
        # the HIP runtime torch and this library already share (by its soname)
        self._hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        self._handles = (ctypes.c_void_p * capacity)()
        for k in range(capacity):
            rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self._handles, k * 8),
                                                   ctypes.c_uint(self._DISABLE_SYSTEM_FENCE))
            if rc != 0:
                raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.struct = ssd_launch_trace()
        self.struct.events = ctypes.cast(self._handles, ctypes.POINTER(ctypes.c_void_p))
        self.struct.capacity = capacity
        self.struct.count = 0

    def _elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self._handles[a]),
                                           ctypes.c_void_p(self._handles[b]))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def durations_us(self):
        n = min(int(self.struct.count), len(self._handles) // 2, TRACE_MAX_LAUNCHES)
        return [(self.struct.names[k].decode(), self._elapsed_ms(2 * k, 2 * k + 1) * 1e3)
                for k in range(n)]

    def __del__(self):
        hip = getattr(self, "_hip", None)
        if hip is not None:
            for h in self._handles:
                if h:
                    hip.hipEventDestroy(ctypes.c_void_p(h))


def ssd_combined_varlen_ex(p: ssd_problem, options: ssd_options, x, dt, A, B, C, D, cu_seqlens,
                           state_cache, state_indices, has_initial_state, y, checkpoints,
                           workspace, stream=None):
    T, S, H, P, N, G, Q, mc = _dims(p)
    if options.prefix_lens:
        mc = max_chunks_aligned(p)
    ti, ts = _TORCH[p.in_dtype], _TORCH[p.state_dtype]
    if workspace is None or workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 GPU tensor")
    rc = _lib.ssd_combined_varlen_ex(
        ctypes.byref(p), ctypes.byref(options), _ptr(x, "x", ti, (T, H, P)),
        _ptr(dt, "dt", ti, (T, H)), _ptr(A, "A", torch.float32, (H,)),
        _ptr(B, "B", ti, (T, G, N)), _ptr(C, "C", ti, (T, G, N)),
        _ptr(D, "D", torch.float32, (H,), optional=True),
        _ptr(cu_seqlens, "cu_seqlens", torch.int32, (S + 1,)),
        _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (S,)),
        _ptr(has_initial_state, "has_initial_state", torch.uint8, (S,), optional=True),
        _ptr(y, "y", ti, (T, H, P)),
        _ptr(checkpoints, "checkpoints", ts, (mc, H, P, N), optional=True),
        _ptr(workspace, "workspace", torch.uint8), ctypes.c_size_t(workspace.numel()),
        _stream(stream))
    _check("ssd_combined_varlen_ex", rc)


def selective_state_update_ex(p: ssu_problem, options: ssd_options, state_cache, state_indices,
                              x, dt, A, B, C, D, y, intermediate_states=None, cu_seqlens=None,
                              stream=None):
    """Uniform (x [R,T,H,P] ...) or, with cu_seqlens, packed-varlen (x [T_tot,H,P] ...)."""
    R, T, H, P, N, G = (p.num_reqs, p.tokens_per_req, p.nheads, p.headdim, p.d_state, p.ngroups)
    ti, ts = _TORCH[p.in_dtype], _TORCH[p.state_dtype]
    lead = (R, T) if cu_seqlens is None else (int(x.shape[0]),)
    Tt = R * T if cu_seqlens is None else int(x.shape[0])
    rc = _lib.selective_state_update_ex(
        ctypes.byref(p), ctypes.byref(options), Tt,
        None if cu_seqlens is None else _ptr(cu_seqlens, "cu_seqlens", torch.int32, (R + 1,)),
        _ptr(state_cache, "state_cache", ts, (p.num_slots, H, P, N)),
        _ptr(state_indices, "state_indices", torch.int32, (R,)),
        _ptr(x, "x", ti, lead + (H, P)), _ptr(dt, "dt", ti, lead + (H,)),
        _ptr(A, "A", torch.float32, (H,)), _ptr(B, "B", ti, lead + (G, N)),
        _ptr(C, "C", ti, lead + (G, N)), _ptr(D, "D", torch.float32, (H,), optional=True),
        _ptr(y, "y", ti, lead + (H, P)),
        _ptr(intermediate_states, "intermediate_states", ts, lead + (H, P, N), optional=True),
        _stream(stream))
    _check("selective_state_update_ex", rc)


def ssd_round_f16(x, out, sr_seed=None, sr_rounds: int = 10, kind: int = 0, stream=None):
    """out (float16) = x (float32) rounded as the fp16 state stores are."""
    if x.numel() != out.numel() or out.dtype != torch.float16:
        raise ValueError("out must be a float16 tensor with as many elements as x")
    rc = _lib.ssd_round_f16(_ptr(x, "x", torch.float32), _ptr(out, "out", torch.float16),
                            int(x.numel()),
                            None if sr_seed is None else _ptr(sr_seed, "sr_seed", torch.int64, (1,)),
                            int(sr_rounds), int(kind), _stream(stream))
    _check("ssd_round_f16", rc)


def ssd_replay_update_ex(p: ssu_problem, options: ssd_options, ring_len: int, ckpt, ring_x,
                         ring_dt, ring_B, cursor, state_indices, x, dt, A, B, C, D, y,
                         stream=None):
    R, T, H, P, N, G = (p.num_reqs, p.tokens_per_req, p.nheads, p.headdim, p.d_state, p.ngroups)
    ti, ts = _TORCH[p.in_dtype], _TORCH[p.state_dtype]
    rc = _lib.ssd_replay_update_ex(
        ctypes.byref(p), ctypes.byref(options), int(ring_len),
        _ptr(ckpt, "ckpt", ts, (p.num_slots, H, P, N)),
        *_ring_ptrs(p, ring_len, ring_x, ring_dt, ring_B),
        _ptr(cursor, "cursor", torch.int32, (p.num_slots, 2)),
        _ptr(state_indices, "state_indices", torch.int32, (R,)),
        _ptr(x, "x", ti, (R, T, H, P)), _ptr(dt, "dt", ti, (R, T, H)),
        _ptr(A, "A", torch.float32, (H,)), _ptr(B, "B", ti, (R, T, G, N)),
        _ptr(C, "C", ti, (R, T, G, N)), _ptr(D, "D", torch.float32, (H,), optional=True),
        _ptr(y, "y", ti, (R, T, H, P)), _stream(stream))
    _check("ssd_replay_update_ex", rc)


def ssd_replay_materialize_ex(p: ssu_problem, options: ssd_options, ring_len: int, ckpt, ring_x,
                              ring_dt, ring_B, cursor, state_indices, A, stream=None):
    H, P, N = p.nheads, p.headdim, p.d_state
    ts = _TORCH[p.state_dtype]
    rc = _lib.ssd_replay_materialize_ex(
        ctypes.byref(p), ctypes.byref(options), int(ring_len),
        _ptr(ckpt, "ckpt", ts, (p.num_slots, H, P, N)),
        *_ring_ptrs(p, ring_len, ring_x, ring_dt, ring_B),
        _ptr(cursor, "cursor", torch.int32, (p.num_slots, 2)),
        _ptr(state_indices, "state_indices", torch.int32, (p.num_reqs,)),
        _ptr(A, "A", torch.float32, (H,)), _stream(stream))
    _check("ssd_replay_materialize_ex", rc)


# ---------------------------------------------------------------------------
# ReplaySSM decode: checkpoint + input rings per slot (see include/ssd_mi355x.h)

def _ring_ptrs(p: ssu_problem, W: int, ring_x, ring_dt, ring_B):
    H, P, N, G = p.nheads, p.headdim, p.d_state, p.ngroups
    ti = _TORCH[p.in_dtype]
    return (_ptr(ring_x, "ring_x", ti, (p.num_slots, W, H, P)),
            _ptr(ring_dt, "ring_dt", ti, (p.num_slots, W, H)),
            _ptr(ring_B, "ring_B", ti, (p.num_slots, W, G, N)))


def ssd_replay_update(p: ssu_problem, ring_len: int, ckpt, ring_x, ring_dt, ring_B, cursor,
                      state_indices, x, dt, A, B, C, D, y, stream=None):
    R, T, H, P, N, G = (p.num_reqs, p.tokens_per_req, p.nheads, p.headdim, p.d_state, p.ngroups)
    ti, ts = _TORCH[p.in_dtype], _TORCH[p.state_dtype]
    rc = _lib.ssd_replay_update(
        ctypes.byref(p), int(ring_len), _ptr(ckpt, "ckpt", ts, (p.num_slots, H, P, N)),
        *_ring_ptrs(p, ring_len, ring_x, ring_dt, ring_B),
        _ptr(cursor, "cursor", torch.int32, (p.num_slots, 2)),
        _ptr(state_indices, "state_indices", torch.int32, (R,)),
        _ptr(x, "x", ti, (R, T, H, P)), _ptr(dt, "dt", ti, (R, T, H)),
        _ptr(A, "A", torch.float32, (H,)), _ptr(B, "B", ti, (R, T, G, N)),
        _ptr(C, "C", ti, (R, T, G, N)), _ptr(D, "D", torch.float32, (H,), optional=True),
        _ptr(y, "y", ti, (R, T, H, P)), _stream(stream))
    _check("ssd_replay_update", rc)


def ssd_replay_advance(p: ssu_problem, ring_len: int, cursor, state_indices, num_accepted,
                       stream=None):
    rc = _lib.ssd_replay_advance(
        ctypes.byref(p), int(ring_len), _ptr(cursor, "cursor", torch.int32, (p.num_slots, 2)),
        _ptr(state_indices, "state_indices", torch.int32, (p.num_reqs,)),
        _ptr(num_accepted, "num_accepted", torch.int32, (p.num_reqs,)), _stream(stream))
    _check("ssd_replay_advance", rc)


def ssd_replay_materialize(p: ssu_problem, ring_len: int, ckpt, ring_x, ring_dt, ring_B, cursor,
                           state_indices, A, stream=None):
    H, P, N = p.nheads, p.headdim, p.d_state
    ts = _TORCH[p.state_dtype]
    rc = _lib.ssd_replay_materialize(
        ctypes.byref(p), int(ring_len), _ptr(ckpt, "ckpt", ts, (p.num_slots, H, P, N)),
        *_ring_ptrs(p, ring_len, ring_x, ring_dt, ring_B),
        _ptr(cursor, "cursor", torch.int32, (p.num_slots, 2)),
        _ptr(state_indices, "state_indices", torch.int32, (p.num_reqs,)),
        _ptr(A, "A", torch.float32, (H,)), _stream(stream))
    _check("ssd_replay_materialize", rc)


# ---------------------------------------------------------------------------
# allocation helpers (torch plumbing; no arithmetic)

def alloc_workspace(p: ssd_problem, device="cuda") -> torch.Tensor:
    return torch.empty(max(workspace_bytes(p), 256), dtype=torch.uint8, device=device)


def alloc_step_buffers(p: ssd_problem, device="cuda") -> dict:
    """Buffers the five prefill steps exchange when called one by one."""
    T, S, H, P, N, G, Q, mc = _dims(p)
    f = dict(dtype=torch.float32, device=device)
    return dict(
        chunk_meta=torch.empty(chunk_meta_count(p), dtype=torch.int32, device=device),
        dA_cumsum=torch.empty((H, mc, Q), **f), dt_chunk=torch.empty((H, mc, Q), **f),
        chunk_states=torch.empty((mc, H, P, N), **f),
        entering=torch.empty((mc, H, P, N), dtype=_TORCH[p.in_dtype], device=device),
        CB=torch.empty((mc, G, Q, Q), dtype=_TORCH[p.in_dtype], device=device))


def alloc_replay_rings(p: ssu_problem, ring_len: int, device="cuda") -> dict:
    """Input rings and cursors of a ReplaySSM layer, zeroed (every history empty)."""
    H, P, N, G, S = p.nheads, p.headdim, p.d_state, p.ngroups, p.num_slots
    ti = _TORCH[p.in_dtype]
    return dict(ring_x=torch.zeros((S, ring_len, H, P), dtype=ti, device=device),
                ring_dt=torch.zeros((S, ring_len, H), dtype=ti, device=device),
                ring_B=torch.zeros((S, ring_len, G, N), dtype=ti, device=device),
                cursor=torch.zeros((S, 2), dtype=torch.int32, device=device))
