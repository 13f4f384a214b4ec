"""Seeded synthetic inputs for the Mamba2 SSD varlen scan and the MTP state update.

This module only draws numbers: it holds none of the scan's arithmetic and is
shared by the CPU oracle's tests, the GPU parity tests and the benchmark.

Workload shapes follow the pages' workloads: the single-sequence layer prefill;
the cached short continuation (4,224-token prefix + 32-token suffix, 32
sequences) and the mixed varlen prefill (suffix lengths
[32, 600, 1600, 128, 32, 600, 1600, 128]) of vLLM PR #62922 (initial states
read from the cache in state passing), section "Serving performance"; and the
MTP verify batch (one target token plus draft tokens) of vLLM PR #52928
"[Mamba] Add FlashInfer ReplaySSM support for MTP", section "Summary".
The pages' own datasets and models are not used: these seeded draws stand in.

Generator: numpy PCG64 seeded with ``[cfg, stream, ...]``.
  stream 0 -> layer parameters, drawn in the order A, dt_bias, D
  stream 1 -> tokens, drawn in the order x, z (dt pre-activation), B, C
  stream 2 -> state_indices (a random permutation of the cache slots)
  stream [3, s] -> the prefix tokens of sequence / request s (drawn on demand)
  stream 4 -> accepted-draft counts of the MTP verify batch
Values are drawn in float64 and then cast to the input dtype (round to nearest
even, through torch).

Value distributions: x ~ N(0,1); B, C ~ N(0,1)/sqrt(d_state);
A_h = -exp(U(log 1, log 16)); D_h ~ N(0,1);
dt = clip(softplus(z + dt_bias_h), 1e-3, 0.1), z ~ N(0,1),
dt_bias_h = softplus^-1(u_h), u_h log-uniform in [1e-3, 1e-1].
The kernels take the post-activation dt; the softplus here is part of drawing
inputs, not of the scan.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

DT_MIN = 1e-3
DT_MAX = 1e-1


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    """One packed varlen prefill problem."""
    name: str
    seqlens: tuple
    nheads: int
    headdim: int
    d_state: int
    ngroups: int
    chunk_size: int
    in_dtype: torch.dtype
    state_dtype: torch.dtype
    num_slots: int
    # per-sequence flag: start from a cached state (True) or from zero (False)
    has_initial: tuple
    prefix_len: int          # length of the seeded prefix that makes an initial state
    checkpoints: bool
    seed: int

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seqlens))

    @property
    def num_seqs(self) -> int:
        return len(self.seqlens)

    @property
    def any_initial(self) -> bool:
        return any(self.has_initial)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """One MTP verify / decode state-update problem."""
    name: str
    num_reqs: int
    tokens_per_req: int
    nheads: int
    headdim: int
    d_state: int
    ngroups: int
    in_dtype: torch.dtype
    state_dtype: torch.dtype
    num_slots: int
    prefix_len: int
    seed: int


# The five workloads.
C0 = PrefillConfig("c0_tiny_fp32", (256,), 4, 16, 16, 1, 64, torch.float32, torch.float32,
                   1, (False,), 0, False, 0)
C1 = PrefillConfig("c1_layer_prefill_L4096", (4096,), 80, 64, 128, 1, 256, torch.bfloat16,
                   torch.float32, 1, (False,), 0, False, 1)
C2 = PrefillConfig("c2_cached_short_continuation", (32,) * 32, 64, 64, 128, 8, 256,
                   torch.bfloat16, torch.bfloat16, 256, (True,) * 32, 4224, False, 2)
C3 = PrefillConfig("c3_mixed_varlen", (32, 600, 1600, 128, 32, 600, 1600, 128), 64, 64, 128, 8,
                   256, torch.bfloat16, torch.float32, 256,
                   tuple(i % 2 == 1 for i in range(8)), 4224, True, 3)
C4 = DecodeConfig("c4_mtp_verify", 128, 3, 128, 64, 128, 8, torch.bfloat16, torch.bfloat16,
                  512, 256, 4)

PREFILL_CONFIGS = {c.name: c for c in (C0, C1, C2, C3)}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def _softplus(v):
    return np.logaddexp(0.0, v)


def _softplus_inv(v):
    return v + np.log(-np.expm1(-v))


def to_dtype(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """float64 numpy -> torch CPU tensor of ``dtype`` (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(dtype)


def layer_params(seed: int, nheads: int):
    """A [H] (float64, negative), dt_bias [H], D [H]."""
    g = _rng(seed, 0)
    A = -np.exp(g.uniform(math.log(1.0), math.log(16.0), size=nheads))
    u = np.exp(g.uniform(math.log(DT_MIN), math.log(DT_MAX), size=nheads))
    dt_bias = _softplus_inv(u)
    D = g.standard_normal(nheads)
    return A, dt_bias, D


def token_block(g: np.random.Generator, ntok: int, nheads: int, headdim: int, ngroups: int,
                d_state: int, dt_bias: np.ndarray, with_raw: bool = False):
    """x [T,H,P], dt [T,H], B [T,G,N], C [T,G,N] in float64, drawn in this order;
    with_raw also returns z [T,H], the pre-activation draw behind dt."""
    x = g.standard_normal((ntok, nheads, headdim))
    z = g.standard_normal((ntok, nheads))
    dt = np.clip(_softplus(z + dt_bias[None, :]), DT_MIN, DT_MAX)
    scale = 1.0 / math.sqrt(d_state)
    B = g.standard_normal((ntok, ngroups, d_state)) * scale
    C = g.standard_normal((ntok, ngroups, d_state)) * scale
    return (x, dt, B, C, z) if with_raw else (x, dt, B, C)


@dataclasses.dataclass
class PrefillInputs:
    cfg: PrefillConfig
    x: torch.Tensor          # [T,H,P]  in_dtype
    dt: torch.Tensor         # [T,H]    in_dtype (post-activation)
    A: torch.Tensor          # [H] float32
    B: torch.Tensor          # [T,G,N]  in_dtype
    C: torch.Tensor          # [T,G,N]  in_dtype
    D: torch.Tensor          # [H] float32
    cu_seqlens: torch.Tensor  # [S+1] int32
    state_indices: torch.Tensor  # [S] int32
    has_initial: Optional[torch.Tensor]  # [S] uint8 or None
    dt_bias: np.ndarray = None
    dt_raw: torch.Tensor = None  # [T,H] in_dtype: z, the pre-activation draw behind dt

    def prefix_tokens(self, s: int):
        """(x, dt, B, C) of sequence s's seeded prefix (in_dtype), or None when the
        sequence starts from zero. Drawn on demand from stream [seed, 3, s]."""
        if self.has_initial is None or not int(self.has_initial[s]):
            return None
        c = self.cfg
        px, pdt, pB, pC = token_block(_rng(c.seed, 3, s), c.prefix_len, c.nheads, c.headdim,
                                      c.ngroups, c.d_state, self.dt_bias)
        return tuple(to_dtype(v, c.in_dtype) for v in (px, pdt, pB, pC))


def make_prefill(cfg: PrefillConfig, seqlens: Optional[Sequence[int]] = None) -> PrefillInputs:
    """Draw the inputs of a prefill workload. ``seqlens`` overrides the config's lengths
    (same generator streams), which tests use for small variants."""
    lens = tuple(int(v) for v in (cfg.seqlens if seqlens is None else seqlens))
    H, P, N, G = cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups
    T = int(sum(lens))
    A, dt_bias, D = layer_params(cfg.seed, H)
    x, dt, B, C, z = token_block(_rng(cfg.seed, 1), T, H, P, G, N, dt_bias, with_raw=True)
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    perm = _rng(cfg.seed, 2).permutation(cfg.num_slots).astype(np.int32)
    idx = perm[: len(lens)]
    has_init = None
    if cfg.any_initial:
        flags = [bool(cfg.has_initial[i % len(cfg.has_initial)]) for i in range(len(lens))]
        has_init = torch.tensor([1 if f else 0 for f in flags], dtype=torch.uint8)
    return PrefillInputs(
        cfg=cfg,
        x=to_dtype(x, cfg.in_dtype), dt=to_dtype(dt, cfg.in_dtype),
        A=to_dtype(A, torch.float32), B=to_dtype(B, cfg.in_dtype), C=to_dtype(C, cfg.in_dtype),
        D=to_dtype(D, torch.float32),
        cu_seqlens=torch.from_numpy(cu), state_indices=torch.from_numpy(idx.copy()),
        has_initial=has_init, dt_bias=dt_bias, dt_raw=to_dtype(z, cfg.in_dtype))


@dataclasses.dataclass
class DecodeInputs:
    cfg: DecodeConfig
    x: torch.Tensor    # [R,T,H,P]
    dt: torch.Tensor   # [R,T,H]
    A: torch.Tensor    # [H] float32
    B: torch.Tensor    # [R,T,G,N]
    C: torch.Tensor    # [R,T,G,N]
    D: torch.Tensor    # [H] float32
    state_indices: torch.Tensor  # [R] int32
    num_accepted: torch.Tensor   # [R] int32 in [0, T)
    dt_bias: np.ndarray = None
    dt_raw: torch.Tensor = None  # [R,T,H] in_dtype: z, the pre-activation draw behind dt

    def prefix_tokens(self, r: int):
        """(x [L,H,P], dt [L,H], B [L,G,N], C [L,G,N]) of request r's seeded prefix."""
        c = self.cfg
        px, pdt, pB, pC = token_block(_rng(c.seed, 3, r), c.prefix_len, c.nheads, c.headdim,
                                      c.ngroups, c.d_state, self.dt_bias)
        return tuple(to_dtype(v, c.in_dtype) for v in (px, pdt, pB, pC))


def make_decode(cfg: DecodeConfig, num_reqs: Optional[int] = None) -> DecodeInputs:
    R = cfg.num_reqs if num_reqs is None else int(num_reqs)
    T, H, P, N, G = cfg.tokens_per_req, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups
    A, dt_bias, D = layer_params(cfg.seed, H)
    x, dt, B, C, z = token_block(_rng(cfg.seed, 1), R * T, H, P, G, N, dt_bias, with_raw=True)
    perm = _rng(cfg.seed, 2).permutation(cfg.num_slots).astype(np.int32)
    acc = _rng(cfg.seed, 4).integers(0, T, size=R).astype(np.int32)
    return DecodeInputs(
        cfg=cfg,
        x=to_dtype(x.reshape(R, T, H, P), cfg.in_dtype),
        dt=to_dtype(dt.reshape(R, T, H), cfg.in_dtype),
        A=to_dtype(A, torch.float32),
        B=to_dtype(B.reshape(R, T, G, N), cfg.in_dtype),
        C=to_dtype(C.reshape(R, T, G, N), cfg.in_dtype),
        D=to_dtype(D, torch.float32),
        state_indices=torch.from_numpy(perm[:R].copy()),
        num_accepted=torch.from_numpy(acc), dt_bias=dt_bias,
        dt_raw=to_dtype(z.reshape(R, T, H), cfg.in_dtype))


def random_problem(seed: int, seqlens: Sequence[int], nheads: int, headdim: int, d_state: int,
                   ngroups: int, chunk_size: int, in_dtype=torch.float32,
                   state_dtype=torch.float32, num_slots: Optional[int] = None,
                   has_initial: Optional[Sequence[bool]] = None, prefix_len: int = 0,
                   checkpoints: bool = False) -> PrefillInputs:
    """A small prefill problem of any shape, same distributions (tests)."""
    S = len(seqlens)
    cfg = PrefillConfig(f"rand{seed}", tuple(int(v) for v in seqlens), nheads, headdim, d_state,
                        ngroups, chunk_size, in_dtype, state_dtype,
                        num_slots if num_slots is not None else max(S, 1),
                        tuple(has_initial) if has_initial is not None else (False,) * max(S, 1),
                        prefix_len, checkpoints, 1000 + seed)
    return make_prefill(cfg)


def nan_cache(num_slots: int, H: int, P: int, N: int, dtype: torch.dtype) -> torch.Tensor:
    """A state cache whose every slot is NaN: slots a call must not read stay NaN."""
    return torch.full((num_slots, H, P, N), float("nan"), dtype=dtype)


@dataclasses.dataclass
class LongPrefillInputs:
    x: torch.Tensor          # [T,H,P]  bf16, on the given device
    dt: torch.Tensor         # [T,H]    bf16 (post-activation)
    A: torch.Tensor          # [H] float32
    B: torch.Tensor          # [T,G,N]  bf16
    C: torch.Tensor          # [T,G,N]  bf16
    D: torch.Tensor          # [H] float32
    cu_seqlens: torch.Tensor  # [S+1] int32
    state_indices: torch.Tensor  # [S] int32


def long_prefill(seed: int, seqlens: Sequence[int], nheads: int, headdim: int, d_state: int,
                 ngroups: int, device) -> LongPrefillInputs:
    """A prefill too large to draw on the host in float64 (tests of the largest
    tensors): the same distributions as token_block, drawn by torch's seeded
    generator on ``device`` in float32 and rounded to bf16 there. Slot s for
    sequence s; layer parameters from layer_params."""
    lens = tuple(int(v) for v in seqlens)
    T, S = int(sum(lens)), len(lens)
    A, dt_bias, D = layer_params(seed, nheads)
    g = torch.Generator(device=device).manual_seed(seed)
    bf = torch.bfloat16
    x = torch.randn(T, nheads, headdim, generator=g, device=device).to(bf)
    z = torch.randn(T, nheads, generator=g, device=device)
    bias = torch.tensor(dt_bias, dtype=torch.float32, device=device)
    dt = torch.clamp(torch.nn.functional.softplus(z + bias[None, :]), DT_MIN, DT_MAX).to(bf)
    scale = 1.0 / math.sqrt(d_state)
    B = (torch.randn(T, ngroups, d_state, generator=g, device=device) * scale).to(bf)
    C = (torch.randn(T, ngroups, d_state, generator=g, device=device) * scale).to(bf)
    cu = np.zeros(S + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    return LongPrefillInputs(
        x=x, dt=dt, A=to_dtype(A, torch.float32).to(device), B=B, C=C,
        D=to_dtype(D, torch.float32).to(device), cu_seqlens=torch.from_numpy(cu).to(device),
        state_indices=torch.arange(S, dtype=torch.int32, device=device))
