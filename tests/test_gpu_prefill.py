"""GPU parity of the SSD varlen prefill against the CPU oracle.

Step by step (each of the five steps vs oracle.chunked) and end to end
(ssd_combined_varlen vs the sequential recurrence with cache semantics), on
small problems that still span several chunks, 16-row tiles and ragged tails,
and on the full-size workloads, every (sequence, head) of each.
"""
import numpy as np
import pytest
import torch

import oracle
import ssd_synth as sy
from gpu_helpers import (DEV, assert_close, assert_normalised, cb_fragment_to_dense, gpu_prefill,
                         looser, to64, workload_cache)
from oracle import chunked

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def _ssd():
    import state_space_model_varlen_amd as ssd
    return ssd


def _cache_with_states(inp, num_slots, dtype, scale=0.05, seed=0, nan_unused=True):
    """A cache whose used slots of sequences with an initial state hold random
    states (rounded to the cache dtype) and whose other slots are NaN."""
    H, P, N = inp.x.shape[1], inp.x.shape[2], inp.B.shape[2]
    cache = sy.nan_cache(num_slots, H, P, N, dtype) if nan_unused else \
        torch.zeros(num_slots, H, P, N, dtype=dtype)
    g = torch.Generator().manual_seed(seed)
    if inp.has_initial is not None:
        for s in range(len(inp.state_indices)):
            if int(inp.has_initial[s]):
                cache[int(inp.state_indices[s])] = (torch.randn(H, P, N, generator=g) * scale
                                                    ).to(dtype)
    return cache


# --------------------------------------------------------------------------------------
# step by step

STEP_CASES = [
    # seqlens, H, P, N, G, Q, in_dtype, state_dtype
    ((100, 156), 4, 16, 16, 1, 64, F32, F32),
    ((1, 17, 0, 255, 64, 31), 4, 16, 16, 2, 32, F32, F32),
    ((300, 5, 513), 4, 64, 128, 2, 128, BF16, F32),
    ((256, 1, 700, 16), 4, 64, 128, 1, 256, BF16, BF16),
    ((129, 64), 2, 16, 128, 1, 64, BF16, F32),
    ((77, 200), 2, 64, 16, 2, 64, BF16, BF16),
    ((90, 33), 2, 64, 128, 2, 64, F32, F32),
    # 23 chunk slots x 8 groups: CB with one block per (chunk, group) pair
    ((300, 5, 213, 0, 64), 8, 64, 128, 8, 32, BF16, BF16),
    # 64 sequences x 8 heads: state passing with four element groups per thread
    (tuple((7 * i) % 70 + 1 for i in range(63)) + (130,), 8, 64, 128, 2, 64, BF16, F32),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: f"L{sum(c[0])}_P{c[2]}N{c[3]}Q{c[5]}_"
                         f"{str(c[6])[6:]}_{str(c[7])[6:]}")
def test_steps_match_chunked_oracle(case):
    lens, H, P, N, G, Q, ti, ts = case
    S = len(lens)
    inp = sy.random_problem(STEP_CASES.index(case), lens, H, P, N, G, Q, ti, ts, num_slots=S + 3,
                            has_initial=[s % 2 == 0 for s in range(S)])
    cache = _cache_with_states(inp, S + 3, ts)
    ssd = _ssd()
    T = sum(lens)
    p = ssd.make_problem(T, S, H, P, N, G, Q, S + 3, ti, ts)
    buf = ssd.alloc_step_buffers(p, DEV)
    mc = ssd.max_chunks(p)
    x, dt, A, B, C, D = (t.to(DEV) for t in (inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D))
    cu, idx, hi = inp.cu_seqlens.to(DEV), inp.state_indices.to(DEV), inp.has_initial.to(DEV)
    g_cache = cache.to(DEV)
    ckpt = torch.empty(mc, H, P, N, dtype=ts, device=DEV)
    y = torch.empty(T, H, P, dtype=ti, device=DEV)

    ssd.ssd_chunk_cumsum(p, dt, A, cu, buf["chunk_meta"], buf["dA_cumsum"], buf["dt_chunk"])
    ssd.ssd_chunk_state(p, x, B, buf["chunk_meta"], buf["dA_cumsum"], buf["dt_chunk"],
                        buf["chunk_states"])
    ssd.ssd_bmm_chunk(p, B, C, buf["chunk_meta"], buf["CB"])
    ssd.ssd_state_passing(p, buf["chunk_states"], buf["dA_cumsum"], buf["chunk_meta"], g_cache,
                          idx, hi, buf["entering"], ckpt)
    ssd.ssd_chunk_scan(p, x, C, D, buf["chunk_meta"], buf["dA_cumsum"], buf["dt_chunk"],
                       buf["CB"], buf["entering"], y)
    torch.cuda.synchronize()

    # oracle steps on the same (exactly widened) inputs
    init = oracle.f64(cache[inp.state_indices.long()])
    hin = inp.has_initial.numpy()
    init[hin == 0] = 0.0
    r = chunked.scan(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens.numpy(), Q,
                     init=init, has_init=hin)
    meta = r["meta"]
    nc = len(meta["seq"])

    # 1. chunk metadata: exact
    gm = buf["chunk_meta"].cpu().numpy()
    assert gm[: S + 1].tolist() == meta["chunk_cu"].tolist()
    trip = gm[S + 1: S + 1 + 3 * mc].reshape(mc, 3)
    assert gm[S + 1 + 3 * mc: 2 * S + 2 + 3 * mc].tolist() == \
        np.clip(inp.cu_seqlens.numpy(), 0, T).tolist()
    assert (gm[2 * S + 2 + 3 * mc:] == Q).all()   # first chunks are whole outside align mode
    assert trip[:nc, 0].tolist() == meta["seq"].tolist()
    assert trip[:nc, 1].tolist() == meta["start"].tolist()
    assert trip[:nc, 2].tolist() == meta["len"].tolist()
    assert (trip[nc:, 2] == 0).all() and (trip[nc:, 0] == -1).all()

    # 1. cumsum over each chunk's tokens: within summation rounding; dt per chunk
    # position: exact copy
    gcum = to64(buf["dA_cumsum"][:, :nc])
    gdt = to64(buf["dt_chunk"][:, :nc])
    valid = np.arange(Q)[None, :] < meta["len"][:, None]          # [nc, Q]
    scale = np.abs(r["dA_cumsum"]).max() + 1.0
    assert np.abs(gcum - r["dA_cumsum"])[:, valid].max() <= Q * 1.2e-7 * scale
    assert np.array_equal(gdt[:, valid], r["dt"][:, valid])
    # positions past a chunk's end follow the step's layout contract (header,
    # ssd_chunk_cumsum): the chunk's total again (the wave prefix sum adds the same
    # terms in another order there, so equal within summation rounding), dt 0
    last = gcum[:, np.arange(nc), meta["len"] - 1]                 # [H, nc]
    pad_err = np.abs(np.where(valid, gcum, last[:, :, None]) - gcum).max()
    assert pad_err <= Q * 1.2e-7 * scale
    assert np.all(gdt[:, ~valid] == 0)

    # 4. bmm: causal part inside each chunk; fp32 accumulation, stored in the input
    # dtype (bf16 rounding: relative 2^-8 bound per element)
    gcb = to64(buf["CB"][:nc])
    if ti == BF16:
        gcb = cb_fragment_to_dense(gcb, Q)
    for c in range(nc):
        ln = int(meta["len"][c])
        low = np.tril(np.ones((ln, ln), dtype=bool))
        want = r["CB"][c][:, :ln, :ln][:, low]
        diff = np.abs(gcb[c][:, :ln, :ln][:, low] - want)
        scale = 1 + np.abs(r["CB"][c]).max()
        bound = 1e-5 * scale if ti == F32 else 2.0 ** -8 * np.abs(want) + 1e-5 * scale
        assert np.all(diff <= bound), c

    # 2, 3, 5
    assert_close(buf["chunk_states"][:nc], r["chunk_states"], ti, "chunk_states")
    assert_close(buf["entering"][:nc], r["entering"], ti, "entering states")
    assert_close(ckpt[:nc], r["ckpt"], looser(ti, ts), "checkpoints")
    assert_close(y, r["y"], ti, "y")


MULTI_CASES = [
    # seqlens, state dtype, checkpoints: 64 short sequences x 8 heads x 2 column
    # slices = 1024 items, on average under half a chunk: ssd_chunk_state_passing
    # runs its persistent multi-item kernel (item boundaries after one or two
    # chunks, empty sequences)
    ((1, 0, 200, 5, 64, 17, 0, 129) * 8, F32, True),
    ((3, 40, 0, 9, 130, 1, 22, 31) * 8, BF16, False),
]


@pytest.mark.parametrize("case", MULTI_CASES, ids=lambda c: f"{str(c[1])[6:]}_"
                         f"{'ckpt' if c[2] else 'nockpt'}")
def test_step_state_passing_on_short_batches(case):
    lens, ts, ck = case
    H, P, N, G, Q = 8, 64, 128, 2, 128
    S, T = len(lens), sum(lens)
    assert 2 * T <= S * Q and S * H * 2 >= 1024
    inp = sy.random_problem(990 + MULTI_CASES.index(case), lens, H, P, N, G, Q, BF16, ts,
                            num_slots=S + 3, has_initial=[s % 2 == 0 for s in range(S)])
    cache = _cache_with_states(inp, S + 3, ts)
    ssd = _ssd()
    p = ssd.make_problem(T, S, H, P, N, G, Q, S + 3, BF16, ts)
    buf = ssd.alloc_step_buffers(p, DEV)
    mc = ssd.max_chunks(p)
    g_cache = cache.to(DEV)
    ckpt = torch.empty(mc, H, P, N, dtype=ts, device=DEV) if ck else None
    ssd.ssd_chunk_cumsum(p, inp.dt.to(DEV), inp.A.to(DEV), inp.cu_seqlens.to(DEV),
                         buf["chunk_meta"], buf["dA_cumsum"], buf["dt_chunk"])
    ssd.ssd_chunk_state_passing(p, inp.x.to(DEV), inp.B.to(DEV), buf["chunk_meta"],
                                buf["dA_cumsum"], buf["dt_chunk"], g_cache,
                                inp.state_indices.to(DEV), inp.has_initial.to(DEV),
                                buf["entering"], ckpt)
    torch.cuda.synchronize()
    init = oracle.f64(cache[inp.state_indices.long()])
    hin = inp.has_initial.numpy()
    init[hin == 0] = 0.0
    r = chunked.scan(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens.numpy(), Q,
                     init=init, has_init=hin)
    nc = len(r["meta"]["seq"])
    assert_close(buf["entering"][:nc], r["entering"], BF16, "entering states")
    if ck:
        assert_close(ckpt[:nc], r["ckpt"], looser(BF16, ts), "checkpoints")
    used = inp.state_indices.long()
    after = g_cache.cpu()
    assert_close(after[used], r["final"], looser(BF16, ts), "final states")
    others = [k for k in range(S + 3) if k not in set(used.tolist())]
    bits = torch.int16 if ts == BF16 else torch.int32
    assert torch.equal(after[others].view(bits), cache[others].view(bits))


# --------------------------------------------------------------------------------------
# end to end vs the sequential recurrence

E2E_CASES = [
    ((256,), 4, 16, 16, 1, 64, F32, F32, False),
    ((5, 0, 300, 1, 64, 129), 4, 16, 16, 2, 64, F32, F32, True),
    ((600, 32, 1, 0, 257), 8, 64, 128, 2, 256, BF16, F32, True),
    ((33, 32, 31, 200), 8, 64, 128, 8, 128, BF16, BF16, True),
    ((1000,), 2, 64, 128, 1, 256, BF16, F32, False),
    ((150, 90), 4, 16, 128, 2, 32, BF16, BF16, True),
    ((90, 150), 4, 64, 16, 4, 64, F32, BF16, True),
    # at least 128 (chunk, group) pairs: CB one block per pair, chunk scan dealing
    # pairs over the XCDs (one head per group)
    ((400, 77, 130), 16, 64, 128, 16, 64, BF16, F32, True),
    ((700, 260, 5, 90), 16, 64, 128, 16, 128, BF16, BF16, False),
    # 64 mostly short sequences x 8 heads (on average under half a chunk): the
    # one-launch short-sequence kernel, sequences of one or two chunks and empty ones
    ((1, 0, 200, 5, 64, 17, 0, 129) * 8, 8, 64, 128, 2, 128, BF16, F32, True),
    ((3, 40, 0, 9, 130, 1, 22, 31) * 8, 8, 64, 128, 2, 128, BF16, BF16, False),
    # more than 256 sequences: the cumsum, CB and state launches of their own
    (tuple(40 + (13 * i) % 90 for i in range(300)), 2, 64, 128, 1, 64, BF16, F32, True),
]


def _e2e(case, D=True):
    lens, H, P, N, G, Q, ti, ts, ck = case
    S = len(lens)
    slots = 2 * S + 2
    inp = sy.random_problem(100 + E2E_CASES.index(case), lens, H, P, N, G, Q, ti, ts, num_slots=slots,
                            has_initial=[s % 3 != 1 for s in range(S)])
    cache = _cache_with_states(inp, slots, ts)
    y, cache_after, ckpt = gpu_prefill(inp, cache, Q, checkpoints=ck, D=D)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D if D else None,
                         inp.cu_seqlens, inp.state_indices, inp.has_initial, cache, Q,
                         checkpoints=ck)
    return inp, cache, y, cache_after, ckpt, ref


@pytest.mark.parametrize("case", E2E_CASES, ids=lambda c: f"S{len(c[0])}_P{c[2]}N{c[3]}Q{c[5]}_"
                         f"{str(c[6])[6:]}_{str(c[7])[6:]}")
def test_combined_matches_recurrence(case):
    lens, H, P, N, G, Q, ti, ts, ck = case
    inp, cache, y, cache_after, ckpt, ref = _e2e(case)
    assert_close(y, ref["y"], ti, "y", normalised=False)
    used = inp.state_indices.long()
    assert_close(cache_after[used], ref["final"], looser(ti, ts), "final states")
    # slots that are not in state_indices keep their exact bits (NaN included)
    others = [s for s in range(cache.shape[0]) if s not in set(used.tolist())]
    assert torch.equal(cache_after[others].view(torch.int16 if ts == BF16 else torch.int32),
                       cache[others].view(torch.int16 if ts == BF16 else torch.int32))
    if ck:
        nc = int(oracle.chunk_counts(inp.cu_seqlens.numpy(), Q)[-1])
        assert_close(ckpt[:nc], ref["ckpt"], looser(ti, ts), "checkpoints")


@pytest.mark.parametrize("case", [c for c in E2E_CASES if c[6] == BF16],
                         ids=lambda c: f"S{len(c[0])}_Q{c[5]}")
def test_ssm_part_normalised_error(case):
    """With D = 0, y is the SSM part alone: its normalised error must be small."""
    inp, cache, y, cache_after, ckpt, ref = _e2e(case, D=False)
    assert_close(y, ref["y"], case[6], "y (D = 0)")


def test_deterministic_and_inputs_untouched():
    case = E2E_CASES[2]
    lens, H, P, N, G, Q, ti, ts, ck = case
    S = len(lens)
    inp = sy.random_problem(5, lens, H, P, N, G, Q, ti, ts, num_slots=2 * S,
                            has_initial=[True] * S)
    cache = _cache_with_states(inp, 2 * S, ts)
    keep = [t.clone() for t in (inp.x, inp.dt, inp.B, inp.C, inp.A, inp.D)]
    y1, c1, k1 = gpu_prefill(inp, cache, Q, checkpoints=True)
    y2, c2, k2 = gpu_prefill(inp, cache, Q, checkpoints=True)
    bits = lambda t: t.view(torch.int16) if t.dtype == BF16 else t.view(torch.int32)
    nc = int(oracle.chunk_counts(inp.cu_seqlens.numpy(), Q)[-1])
    assert torch.equal(bits(y1), bits(y2))
    assert torch.equal(bits(c1), bits(c2))          # NaN slots compared by their bits
    assert torch.equal(bits(k1[:nc]), bits(k2[:nc]))
    for a, b in zip(keep, (inp.x, inp.dt, inp.B, inp.C, inp.A, inp.D)):
        assert torch.equal(a, b)


def test_packing_is_bitwise_invariant():
    """A packed batch gives the same bits as each sequence run alone: chunks
    start at every sequence's first token, so the work per sequence is identical.
    (A sequence's chain is cut into min(segment limit, its chunks) segments; here
    no sequence has more chunks than the limit of either run, so the cuts agree.
    Every sequence holds more than half a chunk, so no run takes the one-launch
    path for short sequences, whose sub-chunks round differently.)"""
    lens, H, P, N, G, Q = (300, 70, 513, 65), 4, 64, 128, 2, 128
    S = len(lens)
    inp = sy.random_problem(9, lens, H, P, N, G, Q, BF16, F32, num_slots=S,
                            has_initial=[True, False, True, True])
    cache = _cache_with_states(inp, S, F32)
    y, c_after, _ = gpu_prefill(inp, cache, Q)
    cu = inp.cu_seqlens.tolist()
    for s in range(S):
        a, b = cu[s], cu[s + 1]
        one = sy.PrefillInputs(cfg=inp.cfg, x=inp.x[a:b].contiguous(), dt=inp.dt[a:b].contiguous(),
                               A=inp.A, B=inp.B[a:b].contiguous(), C=inp.C[a:b].contiguous(),
                               D=inp.D, cu_seqlens=torch.tensor([0, b - a], dtype=torch.int32),
                               state_indices=inp.state_indices[s:s + 1].clone(),
                               has_initial=inp.has_initial[s:s + 1].clone())
        y1, c1, _ = gpu_prefill(one, cache, Q)
        assert torch.equal(y1, y[a:b]), s
        slot = int(inp.state_indices[s])
        assert torch.equal(c1[slot], c_after[slot]), s


def test_chunk_size_invariance():
    """Q = 64, 128, 256 each match the oracle; their results agree with each other."""
    lens = (700, 130, 1)
    inp = sy.random_problem(11, lens, 4, 64, 128, 2, 64, BF16, F32, num_slots=3,
                            has_initial=[True, True, False])
    cache = _cache_with_states(inp, 3, F32)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, 64)
    outs = []
    for Q in (32, 64, 128, 256):
        y, c, _ = gpu_prefill(inp, cache, Q)
        assert_close(y, ref["y"], BF16, f"y Q={Q}", normalised=False)
        assert_close(c[inp.state_indices.long()], ref["final"], BF16, f"final Q={Q}")
        outs.append(y)
    for o in outs[1:]:
        assert_close(o, to64(outs[0]), BF16, "y across chunk sizes", normalised=False)


def test_empty_batch_and_zero_length_sequences():
    ssd = _ssd()
    # S = 0, T = 0: nothing to do
    p = ssd.make_problem(0, 0, 4, 16, 16, 1, 64, 1, F32, F32)
    cache = torch.zeros(1, 4, 16, 16, device=DEV)
    ssd.ssd_combined_varlen(p, torch.empty(0, 4, 16, device=DEV), torch.empty(0, 4, device=DEV),
                            torch.ones(4, device=DEV), torch.empty(0, 1, 16, device=DEV),
                            torch.empty(0, 1, 16, device=DEV), None,
                            torch.zeros(1, dtype=torch.int32, device=DEV), cache,
                            torch.empty(0, dtype=torch.int32, device=DEV), None,
                            torch.empty(0, 4, 16, dtype=F32, device=DEV), None,
                            ssd.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    assert (cache == 0).all()
    # only zero-length sequences: each writes its initial state (or zeros) back
    inp = sy.random_problem(13, (0, 0, 0), 4, 16, 16, 1, 64, F32, F32, num_slots=5,
                            has_initial=[True, False, True])
    c = _cache_with_states(inp, 5, F32)
    y, after, _ = gpu_prefill(inp, c, 64)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, c, 64)
    assert torch.equal(after.view(torch.int32), ref["cache"].view(torch.int32))


@pytest.mark.parametrize("ti,ts", [(F32, F32), (BF16, BF16), (BF16, F32)])
def test_zero_length_sequences_between_others(ti, ts):
    """Empty sequences among non-empty ones (bf16 inputs with headdim 64 and
    d_state 128 take the fused chunk state + state passing kernel): each empty
    one writes its initial state (or zeros) back unchanged."""
    P, N = (64, 128) if ti == BF16 else (16, 16)
    lens = (0, 70, 0, 0, 300, 0)
    S = len(lens)
    inp = sy.random_problem(14, lens, 4, P, N, 2, 64, ti, ts, num_slots=S + 2,
                            has_initial=[True, True, False, True, False, True])
    cache = _cache_with_states(inp, S + 2, ts)
    y, after, ckpt = gpu_prefill(inp, cache, 64, checkpoints=True)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, 64, checkpoints=True)
    assert_close(y, ref["y"], ti, "y", normalised=False)
    used = inp.state_indices.long()
    assert_close(after[used], ref["final"], looser(ti, ts), "final states")
    nc = int(oracle.chunk_counts(inp.cu_seqlens.numpy(), 64)[-1])
    assert_close(ckpt[:nc], ref["ckpt"], looser(ti, ts), "checkpoints")
    bits = torch.int16 if ts == BF16 else torch.int32
    for s in (0, 3, 5):      # empty with an initial state: bits unchanged
        slot = int(inp.state_indices[s])
        assert torch.equal(after[slot].view(bits), cache[slot].view(bits)), s
    assert (after[int(inp.state_indices[2])] == 0).all()   # empty, no initial state


@pytest.mark.parametrize("ti,P,N", [(F32, 16, 16), (BF16, 64, 128)])
def test_bad_device_indices_do_not_fault(ti, P, N):
    """Slot indices outside [0, num_slots) are skipped on the device: the
    sequence starts from zero and nothing is written."""
    lens = (40, 70)
    inp = sy.random_problem(15, lens, 4, P, N, 1, 64, ti, F32, num_slots=2,
                            has_initial=[True, True])
    cache = _cache_with_states(inp, 2, F32, nan_unused=False)
    inp.state_indices[:] = torch.tensor([7, -3], dtype=torch.int32)
    y, after, _ = gpu_prefill(inp, cache, 64)
    assert torch.equal(after, cache)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         torch.tensor([0, 1]), None, cache, 64)
    assert_close(y, ref["y"], ti, "y from zero", normalised=False)


# --------------------------------------------------------------------------------------
# full-size workloads

def test_c0_tiny_fp32_full():
    inp = sy.make_prefill(sy.C0)
    cache = torch.full((1, 4, 16, 16), float("nan"))
    y, after, _ = gpu_prefill(inp, cache, 64)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, None, cache, 64)
    err_y = assert_close(y, ref["y"], F32, "c0 y")
    err_s = assert_close(after[0], ref["final"][0], F32, "c0 final state")
    assert err_y <= 1e-4 and err_s <= 1e-4


def test_c1_layer_prefill_full():
    inp = sy.make_prefill(sy.C1)
    cache = torch.full((1, 80, 64, 128), float("nan"))
    y, after, _ = gpu_prefill(inp, cache, 256)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, None, cache, 256)
    assert_close(y, ref["y"], BF16, "c1 y", normalised=False)
    assert_close(after[0], ref["final"][0], BF16, "c1 final state")
    yd, _, _ = gpu_prefill(inp, cache, 256, D=False)
    assert_close(yd, ref["y"] - to64(inp.D)[None, :, None] * to64(inp.x), BF16, "c1 y (D = 0)")


def test_launch_trace_names_and_times_every_launch():
    """ssd_options.trace on the layer call: an event before each kernel launch and
    one after the last. The launches are named in order, every interval is
    positive, and y and the final state are bit for bit those of the untraced
    call."""
    ssd = _ssd()
    cfg = sy.C1
    inp = sy.make_prefill(cfg)
    H, P, N, Q = cfg.nheads, cfg.headdim, cfg.d_state, cfg.chunk_size
    p = ssd.make_problem(cfg.total_tokens, 1, H, P, N, cfg.ngroups, Q, 1, BF16, F32)
    args = [t.to(DEV) for t in (inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens)]
    outs = []
    tr = ssd.LaunchTrace()
    for opt in (None, ssd.make_options(trace=tr)):
        cache = torch.zeros(1, H, P, N, device=DEV)
        y = torch.empty(cfg.total_tokens, H, P, dtype=BF16, device=DEV)
        ws = ssd.alloc_workspace(p, DEV)
        if opt is None:
            ssd.ssd_combined_varlen(p, *args, cache, inp.state_indices.to(DEV), None, y, None, ws)
        else:
            ssd.ssd_combined_varlen_ex(p, opt, *args, cache, inp.state_indices.to(DEV), None, y,
                                       None, ws)
        torch.cuda.synchronize()
        outs.append((y.cpu(), cache.cpu()))
    d = tr.durations_us()
    assert [n for n, _ in d] == ["chunk_state_passing_segmented_prep", "state_carry",
                                 "chunk_scan_segmented"]
    assert all(us > 0 for _, us in d), d
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1], outs[1][1])


OWN_CASES = [
    # seqlens, H, G, Q, state dtype, checkpoints: segmented or not, longest chain
    # first (S <= 64, H a multiple of 8) or not, sequences counted in several waves
    # of 64 (S > 64), empty sequences, a 1-token chunk
    ((40, 300, 700, 5), 16, 2, 128, F32, True),
    ((600, 32, 1600), 8, 1, 256, BF16, True),
    # more state blocks than one round (5 x 64 x 2 = 640): the CB blocks go out
    # after the first 512, their 30 padded to 32
    ((300, 900, 40, 1200, 130), 64, 2, 256, F32, True),
    ((100, 900, 0, 20, 400), 64, 8, 256, F32, False),
    ((1500,), 8, 1, 128, F32, False),
    ((257, 0, 3, 129), 6, 3, 64, BF16, False),
    (tuple(20 + (37 * i) % 280 for i in range(70)), 8, 2, 64, F32, True),
    # chunk 32: one wave scans, half of its lanes past the chunk
    ((100, 37, 260), 8, 2, 32, BF16, True),
    ((300, 45), 4, 1, 32, F32, False),
]


@pytest.mark.parametrize("case", OWN_CASES, ids=lambda c: f"S{len(c[0])}_H{c[1]}_Q{c[3]}_"
                         f"{str(c[4])[6:]}_{'ckpt' if c[5] else 'nockpt'}")
def test_state_launch_with_own_prep_matches_steps_bitwise(case):
    """The combined call (few sequences) runs the cumsum and CB inside its state
    launch. What that launch publishes (chunk metadata, cumsum and dt rows, CB)
    equals, bit for bit, what ssd_chunk_cumsum and ssd_bmm_chunk write; unsegmented,
    so do y, the final states, the checkpoints and the entering states of the
    step-by-step chain (the same kernels and arithmetic after the cumsum)."""
    lens, H, G, Q, ts, ckpt = case
    P, N = 64, 128
    S, T = len(lens), sum(lens)
    inp = sy.random_problem(970 + OWN_CASES.index(case), lens, H, P, N, G, Q, BF16, ts,
                            num_slots=S + 2, has_initial=[s % 3 != 1 for s in range(S)])
    cache = _cache_with_states(inp, S + 2, ts)
    ssd = _ssd()
    p = ssd.make_problem(T, S, H, P, N, G, Q, S + 2, BF16, ts)
    mc = ssd.max_chunks(p)
    x, dt, A, B, C, D = (t.to(DEV) for t in (inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D))
    cu, idx, hi = inp.cu_seqlens.to(DEV), inp.state_indices.to(DEV), inp.has_initial.to(DEV)

    # (both sides' buffers cleared: CB tiles past a chunk's rows are never written)
    ws = ssd.alloc_workspace(p, DEV).zero_()
    c1 = cache.to(DEV)
    y1 = torch.empty(T, H, P, dtype=BF16, device=DEV)
    k1 = torch.empty(mc, H, P, N, dtype=ts, device=DEV) if ckpt else None
    tr = ssd.LaunchTrace(8)
    ssd.ssd_combined_varlen_ex(p, ssd.make_options(trace=tr), x, dt, A, B, C, D, cu, c1, idx, hi,
                               y1, k1, ws)
    torch.cuda.synchronize()
    names = [n for n, _ in tr.durations_us()]
    segmented = names[0] == "chunk_state_passing_segmented_prep"
    assert names == (["chunk_state_passing_segmented_prep", "state_carry",
                      "chunk_scan_segmented"] if segmented
                     else ["chunk_state_passing_prep_bmm", "chunk_scan"]), names
    assert segmented == (not ckpt and len(lens) * H * 2 < 512 and mc > 1)

    buf = {k: v.zero_() for k, v in ssd.alloc_step_buffers(p, DEV).items()}
    c2 = cache.to(DEV)
    y2 = torch.empty(T, H, P, dtype=BF16, device=DEV)
    k2 = torch.empty(mc, H, P, N, dtype=ts, device=DEV) if ckpt else None
    ssd.ssd_chunk_cumsum(p, dt, A, cu, buf["chunk_meta"], buf["dA_cumsum"], buf["dt_chunk"])
    ssd.ssd_bmm_chunk(p, B, C, buf["chunk_meta"], buf["CB"])
    ssd.ssd_chunk_state_passing(p, x, B, buf["chunk_meta"], buf["dA_cumsum"], buf["dt_chunk"],
                                c2, idx, hi, buf["entering"], k2)
    ssd.ssd_chunk_scan(p, x, C, D, buf["chunk_meta"], buf["dA_cumsum"], buf["dt_chunk"],
                       buf["CB"], buf["entering"], y2)
    torch.cuda.synchronize()

    # the workspace as the combined call lays it out: metadata, cumsum, dt, CB,
    # entering states (the fused state path keeps no chunk states)
    r = lambda v: (v + 255) // 256 * 256
    nm = ssd.chunk_meta_count(p)
    o_cum = r(4 * nm)
    o_dt = o_cum + r(4 * H * mc * Q)
    o_cb = o_dt + r(4 * H * mc * Q)
    o_ent = o_cb + r(2 * mc * G * Q * Q)
    wsc = ws.cpu()
    view = lambda o, n, dt_: wsc[o:o + n * torch.tensor([], dtype=dt_).element_size()].view(dt_)
    meta1 = view(0, nm, torch.int32)
    meta2 = buf["chunk_meta"].cpu()
    assert torch.equal(meta1, meta2)
    nc = int(meta2[S])
    cum1 = view(o_cum, H * mc * Q, torch.int32).view(H, mc, Q)[:, :nc]
    dt1 = view(o_dt, H * mc * Q, torch.int32).view(H, mc, Q)[:, :nc]
    assert torch.equal(cum1, buf["dA_cumsum"].cpu().view(torch.int32)[:, :nc])
    assert torch.equal(dt1, buf["dt_chunk"].cpu().view(torch.int32)[:, :nc])
    cb1 = view(o_cb, mc * G * Q * Q, torch.int16).view(mc, G, Q, Q)[:nc]
    assert torch.equal(cb1, buf["CB"].cpu().view(torch.int16)[:nc])
    if segmented:
        return
    ent1 = view(o_ent, mc * H * P * N, torch.int16).view(mc, H, P, N)[:nc]
    assert torch.equal(ent1, buf["entering"].cpu().view(torch.int16)[:nc])
    assert torch.equal(y1.cpu().view(torch.int16), y2.cpu().view(torch.int16))
    bits = torch.int16 if ts == BF16 else torch.int32
    assert torch.equal(c1.cpu().view(bits), c2.cpu().view(bits))
    if ckpt:
        assert torch.equal(k1.cpu()[:nc].view(bits), k2.cpu()[:nc].view(bits))


def _full_continuation(cfg, checkpoints):
    """Full-size prefill from cached states: every sequence with an initial state
    starts from the oracle's state after its own seeded prefix (rounded to the
    cache dtype), all other slots are NaN. The oracle checks every (sequence,
    head): y, the final states read back from their slots and the checkpoints;
    then, with D = 0, y's SSM part alone under the normalised bound."""
    inp = sy.make_prefill(cfg)
    Q = cfg.chunk_size
    cache = workload_cache(inp)
    y, after, ckpt = gpu_prefill(inp, cache, Q, checkpoints=checkpoints)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, Q, checkpoints=checkpoints)
    ti, ts = cfg.in_dtype, cfg.state_dtype
    assert_close(y, ref["y"], ti, f"{cfg.name} y", normalised=False)
    used = inp.state_indices.long()
    assert_close(after[used], ref["final"], looser(ti, ts), f"{cfg.name} final states")
    if checkpoints:
        nc = len(ref["ckpt"])
        assert_close(ckpt[:nc], ref["ckpt"], looser(ti, ts), f"{cfg.name} checkpoints")
    # slots no sequence uses are untouched (NaN bits)
    others = [k for k in range(cfg.num_slots) if k not in set(used.tolist())]
    assert torch.isnan(after[others].float()).all()
    yd, afterd, _ = gpu_prefill(inp, cache, Q, D=False)
    refd = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, None, inp.cu_seqlens,
                          inp.state_indices, inp.has_initial, cache, Q)
    assert_close(yd, refd["y"], ti, f"{cfg.name} y (D = 0)")
    assert_close(afterd[used], refd["final"], looser(ti, ts), f"{cfg.name} final (D = 0 run)")


def test_c2_cached_short_continuation_full():
    _full_continuation(sy.C2, checkpoints=False)


def test_c3_mixed_varlen_full():
    _full_continuation(sy.C3, checkpoints=True)


@pytest.mark.parametrize("dt_scale", [1.0, 12.0, 40.0], ids=["whole_chunk", "per_block", "exact"])
def test_decay_span_modes(dt_scale):
    """The bf16 chunk scan picks its decay reference by span: the whole chunk (span
    <= 60 over the chunk), 32-token blocks (span <= 60 per block) or per element.
    The workload's dt reaches only the first two; scaled step sizes reach all
    three (every sequence here has full chunks, ragged tails and a cached state).
    (Far larger steps make a chunk's cumulative decay so large in magnitude that
    differences of its float32 prefix sums lose accuracy, as in any chunked scan
    built on cumsum differences; dt x 40 keeps it below about 3e4.)"""
    lens, H, P, N, G, Q = (600, 257, 31), 8, 64, 128, 2, 256
    S = len(lens)
    inp = sy.random_problem(900 + int(dt_scale), lens, H, P, N, G, Q, BF16, F32,
                            num_slots=2 * S, has_initial=[True] * S)
    inp.dt = (inp.dt.float() * dt_scale).to(BF16)
    cache = _cache_with_states(inp, 2 * S, F32)
    y, after, ckpt = gpu_prefill(inp, cache, Q, checkpoints=True)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, Q, checkpoints=True)
    assert_close(y, ref["y"], BF16, f"y (dt x {dt_scale})", normalised=False)
    used = inp.state_indices.long()
    assert_close(after[used], ref["final"], BF16, "final states")
    nc = len(ref["ckpt"])
    assert_close(ckpt[:nc], ref["ckpt"], BF16, "checkpoints")
    yd, _, _ = gpu_prefill(inp, cache, Q, D=False)
    refd = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, None, inp.cu_seqlens,
                          inp.state_indices, inp.has_initial, cache, Q)
    assert_close(yd, refd["y"], BF16, f"y without D (dt x {dt_scale})")


@pytest.mark.parametrize("growth", ["mild", "strong"])
def test_growing_state_positive_A(growth):
    """A_h > 0 on half the heads (a growing state: A_h dt > 0 at every step). The
    bf16 chunk scan's factored decay modes need a cumsum that never increases, so
    chunks of those heads take its exact mode.
    "mild": A = +0.05 with the workload's step sizes over several chunks (states
    stay of order one): the element-wise and normalised bounds.
    "strong": single-chunk sequences with A = +1 and step sizes of mean 0.25, so the
    cumsum rises by more than 60 nats inside a full chunk (values up to about 1e30,
    where the factored modes would overflow). The bf16 MFMA operands round the
    state term relative to the state's size, and single elements of y come from
    cancellation between terms of that size, so here the normalised bound applies
    (with every value finite)."""
    H, P, N, G, Q = 8, 64, 128, 2, 256
    lens = (600, 257, 31) if growth == "mild" else (230, 256, 31, 200)
    S = len(lens)
    inp = sy.random_problem(960 + len(lens), lens, H, P, N, G, Q, BF16, F32, num_slots=2 * S,
                            has_initial=[True] * S)
    if growth == "mild":
        inp.A[::2] = 0.05
    else:
        inp.A[::2] = 1.0
        d = inp.dt.float()
        inp.dt = (d * (0.25 / d.mean(0, keepdim=True))).to(BF16)   # every head: mean 0.25
    cache = _cache_with_states(inp, 2 * S, F32)
    for D in (True, False):
        y, after, ckpt = gpu_prefill(inp, cache, Q, checkpoints=True, D=D)
        ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D if D else None,
                             inp.cu_seqlens, inp.state_indices, inp.has_initial, cache, Q,
                             checkpoints=True)
        tag = f"({growth} growth{'' if D else ', D = 0'})"
        used = inp.state_indices.long()
        got = [(y, ref["y"], "y"), (after[used], ref["final"], "final states"),
               (ckpt[:len(ref["ckpt"])], ref["ckpt"], "checkpoints")]
        for g_, w_, what in got:
            if growth == "mild":
                assert_close(g_, w_, BF16, f"{what} {tag}", normalised=not (D and what == "y"))
            else:
                assert_normalised(g_, w_, BF16, f"{what} {tag}")


SHORT_CASES = [
    # seqlens, H, G, Q, state dtype, checkpoints: batches whose sequences hold on
    # average at most half a chunk (2 T <= S Q) run in one launch, one block per
    # (sequence, head) walking sub-chunks of at most 64 tokens
    ((32,) * 16, 16, 2, 256, BF16, False),
    ((1, 0, 63, 64, 65, 127, 128, 129, 0, 200, 2, 3) + (1,) * 12, 8, 2, 128, F32, True),
    ((5, 300, 0, 17, 31, 32, 33, 1) * 4, 8, 8, 256, BF16, True),
    ((40, 9, 0, 100, 20, 1) * 3, 8, 4, 64, F32, True),
    ((7, 40, 1, 2, 0) * 4, 4, 1, 32, BF16, True),
]


@pytest.mark.parametrize("case", SHORT_CASES, ids=lambda c: f"S{len(c[0])}_H{c[1]}_Q{c[3]}_"
                         f"{str(c[4])[6:]}_{'ckpt' if c[5] else 'nockpt'}")
def test_short_sequence_path(case):
    """The one-launch path for short sequences against the oracle: sequences of 0,
    1, 63-65, 127-129 and 200-300 tokens (several sub-chunks and chunks), cached
    and zero starts, checkpoints, NaN in every slot no sequence may read; y with D
    and without (normalised), final states, checkpoints, untouched slots."""
    lens, H, G, Q, ts, ck = case
    S = len(lens)
    assert 2 * sum(lens) <= S * Q
    inp = sy.random_problem(980 + SHORT_CASES.index(case), lens, H, 64, 128, G, Q, BF16, ts,
                            num_slots=2 * S + 3, has_initial=[s % 3 != 2 for s in range(S)])
    cache = _cache_with_states(inp, 2 * S + 3, ts)
    y, after, ckpt = gpu_prefill(inp, cache, Q, checkpoints=ck)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, Q, checkpoints=ck)
    assert_close(y, ref["y"], BF16, "y", normalised=False)
    used = inp.state_indices.long()
    assert_close(after[used], ref["final"], looser(BF16, ts), "final states")
    if ck:
        assert_close(ckpt[:len(ref["ckpt"])], ref["ckpt"], looser(BF16, ts), "checkpoints")
    others = [k for k in range(cache.shape[0]) if k not in set(used.tolist())]
    bits = torch.int16 if ts == BF16 else torch.int32
    assert torch.equal(after[others].view(bits), cache[others].view(bits))
    yd, _, _ = gpu_prefill(inp, cache, Q, D=False)
    refd = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, None, inp.cu_seqlens,
                          inp.state_indices, inp.has_initial, cache, Q)
    assert_close(yd, refd["y"], BF16, "y without D")


def test_short_sequence_path_bad_slots_and_launch_count():
    """Slot indices outside [0, num_slots) on the short path: the sequence starts
    from zero and nothing is written. The call is one launch."""
    ssd = _ssd()
    lens = (30, 2, 41, 0)
    inp = sy.random_problem(990, lens, 8, 64, 128, 2, 256, BF16, F32, num_slots=5,
                            has_initial=[True] * 4)
    cache = _cache_with_states(inp, 5, F32, nan_unused=False)
    inp.state_indices[:] = torch.tensor([7, -3, 1, 99], dtype=torch.int32)
    y, after, _ = gpu_prefill(inp, cache, 256)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         torch.tensor([0, 0, 1, 0]), torch.tensor([0, 0, 1, 0], dtype=torch.uint8),
                         cache, 256)
    assert_close(y, ref["y"], BF16, "y", normalised=False)
    assert torch.equal(after[[0, 2, 3, 4]], cache[[0, 2, 3, 4]])
    assert_close(after[1], ref["cache"][1], BF16, "slot 1 final state")
    T = sum(lens)
    p = ssd.make_problem(T, 4, 8, 64, 128, 2, 256, 5, BF16, F32)
    tr = ssd.LaunchTrace()
    g_cache = cache.to(DEV)
    ssd.ssd_combined_varlen_ex(p, ssd.make_options(trace=tr), inp.x.to(DEV), inp.dt.to(DEV),
                               inp.A.to(DEV), inp.B.to(DEV), inp.C.to(DEV), inp.D.to(DEV),
                               inp.cu_seqlens.to(DEV), g_cache, inp.state_indices.to(DEV),
                               inp.has_initial.to(DEV), torch.empty_like(y, device=DEV), None,
                               ssd.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    assert [n for n, _ in tr.durations_us()] == ["short_scan"]


SEG_CASES = [
    # seqlens, H, Q, state dtype, has_initial: short batches of long sequences, where
    # the state kernel cuts each chunk chain into segments chained by the carry step
    ((2000, 0, 700, 64, 1), 8, 64, F32, [True, True, False, True, True]),
    ((4096,), 2, 256, BF16, [True]),
    ((300, 5000), 4, 128, F32, [False, True]),
    ((1537, 2049), 8, 32, BF16, [True, False]),
    # one 65536-token sequence: 256 chunks in eight segments of 32
    ((65536,), 2, 256, BF16, [True]),
]


@pytest.mark.parametrize("case", SEG_CASES, ids=lambda c: f"S{len(c[0])}_H{c[1]}_Q{c[2]}_"
                         f"{str(c[3])[6:]}")
def test_segmented_state_passing(case):
    """Few (sequence, head) pairs: the combined call runs each sequence's chunk chain
    as up to eight parallel segments and chains their states afterwards. Sequences
    with more chunks than segments, fewer chunks than segments, one chunk, one
    token and none; with and without cached states. The step-wise state kernel
    (one block walks the whole chain) gives the same final states."""
    lens, H, Q, ts, hi = case
    P, N, G = 64, 128, 2
    S = len(lens)
    inp = sy.random_problem(950 + SEG_CASES.index(case), lens, H, P, N, G, Q, BF16, ts,
                            num_slots=2 * S + 1, has_initial=hi)
    cache = _cache_with_states(inp, 2 * S + 1, ts)
    ssd = _ssd()
    T = sum(lens)
    p = ssd.make_problem(T, S, H, P, N, G, Q, 2 * S + 1, BF16, ts)
    # the workspace holds segment buffers exactly when segments are used
    mc = ssd.max_chunks(p)
    r = lambda v: (v + 255) // 256 * 256
    plain = (r(4 * (3 * S + 2 + 3 * mc)) + 2 * r(4 * H * mc * Q) + r(2 * mc * G * Q * Q)
             + r(2 * mc * H * P * N))
    assert ssd.workspace_bytes(p) > plain
    y, after, _ = gpu_prefill(inp, cache, Q)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, Q)
    assert_close(y, ref["y"], BF16, "y", normalised=False)
    used = inp.state_indices.long()
    assert_close(after[used], ref["final"], looser(BF16, ts), "final states")
    others = [k for k in range(cache.shape[0]) if k not in set(used.tolist())]
    bits = torch.int16 if ts == BF16 else torch.int32
    assert torch.equal(after[others].view(bits), cache[others].view(bits))
    yd, _, _ = gpu_prefill(inp, cache, Q, D=False)
    refd = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, None, inp.cu_seqlens,
                          inp.state_indices, inp.has_initial, cache, Q)
    assert_close(yd, refd["y"], BF16, "y without D")
    # step-wise: cumsum, then the unsegmented state kernel
    buf = ssd.alloc_step_buffers(p, DEV)
    g_cache = cache.to(DEV)
    ssd.ssd_chunk_cumsum(p, inp.dt.to(DEV), inp.A.to(DEV), inp.cu_seqlens.to(DEV),
                         buf["chunk_meta"], buf["dA_cumsum"], buf["dt_chunk"])
    ssd.ssd_chunk_state_passing(p, inp.x.to(DEV), inp.B.to(DEV), buf["chunk_meta"],
                                buf["dA_cumsum"], buf["dt_chunk"], g_cache,
                                inp.state_indices.to(DEV), inp.has_initial.to(DEV),
                                buf["entering"], None)
    torch.cuda.synchronize()
    assert_close(g_cache.cpu()[used], to64(after[used]), looser(BF16, ts),
                 "segmented vs unsegmented final states")


@pytest.mark.parametrize("nseq", [1, 4], ids=["one_sequence_segmented", "four_sequences_ranked"])
def test_long_prefill_2gb_tensors_sampled_heads(nseq):
    """The largest tensors: 262144 tokens x 64 heads x headdim 64, so x and y hold
    2.1 GB of bf16 each (byte offsets past 2^31) and the entering states 1.07 GB
    (1025 chunk slots). One sequence takes the segmented state pass (4 segments of
    256 chunks), four take the longest-chain-first pass (chains of 256 chunks).
    Heads 0 and 41 of y and of every final state against the oracle's recurrence
    over the same inputs (the heads are independent; B and C are shared, G = 1)."""
    ssd = _ssd()
    T, H, P, N, G, Q = 262144, 64, 64, 128, 1, 256
    inp = sy.long_prefill(7, [T // nseq] * nseq, H, P, N, G, DEV)
    p = ssd.make_problem(T, nseq, H, P, N, G, Q, nseq, BF16, F32)
    cache = torch.full((nseq, H, P, N), float("nan"), device=DEV)
    y = torch.empty(T, H, P, dtype=BF16, device=DEV)
    ssd.ssd_combined_varlen(p, inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens, cache,
                            inp.state_indices, None, y, None, ssd.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    heads = [0, 41]
    ref_y, ref_fin, _ = oracle.recurrence(
        inp.x[:, heads].cpu(), inp.dt[:, heads].cpu(), inp.A[heads].cpu(), inp.B.cpu(),
        inp.C.cpu(), inp.D[heads].cpu(), inp.cu_seqlens.cpu(), Q)
    assert_close(y[:, heads].cpu(), ref_y, BF16, "long prefill y")
    assert_close(cache[:, heads].cpu(), ref_fin, BF16, "long prefill final states")
