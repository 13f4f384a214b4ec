"""GPU parity of the packed-varlen MTP verify / commit and of the fused step-size
preprocessing (dt = clamp(softplus(dt_raw + dt_bias), dt_min, dt_max)) in the
prefill and the decode update, against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import ssd_synth as sy
from gpu_helpers import DEV, assert_close, looser

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def _ssd():
    import state_space_model_varlen_amd as ssd
    return ssd


def _packed_decode(counts, H, P, N, G, ti, ts, seed):
    """Packed tokens of len(counts) requests (seeded), their slots and a cache whose
    used slots hold small random states (unused slots NaN)."""
    R, Tt = len(counts), int(sum(counts))
    cfg = sy.DecodeConfig(f"varlen{seed}", 1, max(Tt, 1), H, P, N, G, ti, ts, 2 * R + 1, 8, seed)
    d = sy.make_decode(cfg)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(counts)]), dtype=torch.int32)
    flat = lambda t: t.reshape(-1, *t.shape[2:])[:Tt].contiguous()
    idx = torch.from_numpy(np.random.default_rng(seed).permutation(2 * R + 1)[:R].astype(np.int32))
    cache = sy.nan_cache(2 * R + 1, H, P, N, ts)
    g = torch.Generator().manual_seed(seed)
    for s in idx:
        cache[int(s)] = (torch.randn(H, P, N, generator=g) * 0.05).to(ts)
    return (d, cu, idx, cache, flat(d.x), flat(d.dt), flat(d.dt_raw), flat(d.B), flat(d.C))


VARLEN_CASES = [
    # counts, H, P, N, G, in, state, dt preprocessing
    ((3, 0, 1, 4, 2, 3), 8, 64, 128, 2, BF16, BF16, False),
    ((2, 5, 0, 0, 1), 4, 16, 16, 1, F32, F32, True),
    ((1, 1, 4, 3), 4, 64, 16, 2, BF16, F32, True),
    ((6, 2, 3), 6, 16, 128, 3, F32, BF16, False),
]


@pytest.mark.parametrize("case", VARLEN_CASES,
                         ids=lambda c: f"R{len(c[0])}P{c[2]}N{c[3]}_{str(c[5])[6:]}_"
                                       f"{str(c[6])[6:]}{'_dt' if c[7] else ''}")
def test_varlen_update_matches_oracle(case):
    counts, H, P, N, G, ti, ts, use_tf = case
    ssd = _ssd()
    seed = 500 + VARLEN_CASES.index(case)
    d, cu, idx, cache, x, dt, dt_raw, B, C = _packed_decode(counts, H, P, N, G, ti, ts, seed)
    R, Tt = len(counts), int(sum(counts))
    up = ssd.make_ssu_problem(R, max(counts), H, P, N, G, cache.shape[0], ti, ts)
    bias = torch.from_numpy(d.dt_bias).float()
    tf = ssd.make_dt_transform(bias.to(DEV), sy.DT_MIN, sy.DT_MAX) if use_tf else None
    dt_in = dt_raw if use_tf else dt
    dt_ref = oracle.dt_preprocess(dt_raw, bias, sy.DT_MIN, sy.DT_MAX) if use_tf else dt
    for keep in (True, False):
        g_cache = cache.to(DEV)
        y = torch.empty(Tt, H, P, dtype=ti, device=DEV)
        inter = torch.empty(Tt, H, P, N, dtype=ts, device=DEV) if keep else None
        ssd.selective_state_update_varlen(up, cu.to(DEV), g_cache, idx.to(DEV), x.to(DEV),
                                          dt_in.to(DEV), d.A.to(DEV), B.to(DEV), C.to(DEV),
                                          d.D.to(DEV), y, inter, dt_transform=tf)
        torch.cuda.synchronize()
        ref = oracle.state_update_varlen(cache, idx, cu, x, dt_ref, d.A, B, C, d.D, keep)
        assert_close(y, ref["y"], ti, f"y (keep={keep})", normalised=False)
        if keep:
            assert_close(inter, ref["states"], looser(ti, ts), "intermediate states")
            assert torch.equal(g_cache.cpu().view(torch.uint8), cache.view(torch.uint8))
        else:
            used = [int(s) for s, c in zip(idx, counts) if c > 0]
            assert_close(g_cache.cpu()[used], ref["cache"][used], looser(ti, ts), "written states")
            # requests with no token and unused slots keep their exact bits
            kept = [k for k in range(cache.shape[0]) if k not in used]
            assert torch.equal(g_cache.cpu()[kept].view(torch.uint8), cache[kept].view(torch.uint8))


def test_varlen_commit():
    ssd = _ssd()
    counts = (3, 0, 1, 4, 2)
    H, P, N, G = 4, 64, 128, 2
    d, cu, idx, cache, x, dt, _, B, C = _packed_decode(counts, H, P, N, G, BF16, BF16, 77)
    R, Tt = len(counts), sum(counts)
    up = ssd.make_ssu_problem(R, max(counts), H, P, N, G, cache.shape[0], BF16, BF16)
    g_cache = cache.to(DEV)
    y = torch.empty(Tt, H, P, dtype=BF16, device=DEV)
    inter = torch.empty(Tt, H, P, N, dtype=BF16, device=DEV)
    ssd.selective_state_update_varlen(up, cu.to(DEV), g_cache, idx.to(DEV), x.to(DEV), dt.to(DEV),
                                      d.A.to(DEV), B.to(DEV), C.to(DEV), d.D.to(DEV), y, inter)
    acc = torch.tensor([2, 0, 0, 3, 2], dtype=torch.int32)   # request 1 has no token, 4 is out of range
    ssd.ssd_state_commit_varlen(up, cu.to(DEV), g_cache, idx.to(DEV), inter, acc.to(DEV))
    torch.cuda.synchronize()
    after, ic = g_cache.cpu(), inter.cpu()
    for r in range(R):
        slot, a = int(idx[r]), int(acc[r])
        if 0 <= a < counts[r]:
            assert torch.equal(after[slot].view(torch.int16), ic[int(cu[r]) + a].view(torch.int16))
        else:
            assert torch.equal(after[slot].view(torch.int16), cache[slot].view(torch.int16))


PREFILL_DT_CASES = [
    ((256,), 4, 16, 16, 1, 64, F32, F32, False),
    ((600, 32, 1, 0, 257), 8, 64, 128, 2, 256, BF16, F32, True),
    ((33, 32, 200), 8, 64, 128, 8, 128, BF16, BF16, True),
]


@pytest.mark.parametrize("case", PREFILL_DT_CASES,
                         ids=lambda c: f"S{len(c[0])}_P{c[2]}N{c[3]}Q{c[5]}_{str(c[6])[6:]}")
def test_prefill_with_fused_dt(case):
    lens, H, P, N, G, Q, ti, ts, ck = case
    ssd = _ssd()
    S = len(lens)
    slots = 2 * S + 2
    inp = sy.random_problem(600 + PREFILL_DT_CASES.index(case), lens, H, P, N, G, Q, ti, ts,
                            num_slots=slots, has_initial=[s % 2 == 0 for s in range(S)])
    cache = sy.nan_cache(slots, H, P, N, ts)
    g = torch.Generator().manual_seed(3)
    for s in range(S):
        if int(inp.has_initial[s]):
            cache[int(inp.state_indices[s])] = (torch.randn(H, P, N, generator=g) * 0.05).to(ts)
    T = sum(lens)
    bias = torch.from_numpy(inp.dt_bias).float()
    dt_ref = oracle.dt_preprocess(inp.dt_raw, bias, sy.DT_MIN, sy.DT_MAX)
    p = ssd.make_problem(T, S, H, P, N, G, Q, slots, ti, ts)
    tf = ssd.make_dt_transform(bias.to(DEV), sy.DT_MIN, sy.DT_MAX)
    # step 1 alone: the preprocessed step sizes land in dt_chunk (float32)
    buf = ssd.alloc_step_buffers(p, DEV)
    ssd.ssd_chunk_cumsum_dt(p, tf, inp.dt_raw.to(DEV), inp.A.to(DEV), inp.cu_seqlens.to(DEV),
                            buf["chunk_meta"], buf["dA_cumsum"], buf["dt_chunk"])
    torch.cuda.synchronize()
    meta = oracle.chunk_counts(inp.cu_seqlens.numpy(), Q)
    dtc = buf["dt_chunk"].cpu().numpy()
    cu = inp.cu_seqlens.tolist()
    for s in range(S):
        for k in range(int(meta[s + 1] - meta[s])):
            a = cu[s] + k * Q
            ln = min(Q, cu[s + 1] - a)
            got = dtc[:, int(meta[s]) + k, :ln].T
            np.testing.assert_allclose(got, dt_ref[a:a + ln], rtol=2e-6, atol=1e-9)
    # the whole prefill
    g_cache = cache.to(DEV)
    y = torch.empty(T, H, P, dtype=ti, device=DEV)
    ckpt = torch.empty(ssd.max_chunks(p), H, P, N, dtype=ts, device=DEV) if ck else None
    ssd.ssd_combined_varlen_dt(p, tf, inp.x.to(DEV), inp.dt_raw.to(DEV), inp.A.to(DEV),
                               inp.B.to(DEV), inp.C.to(DEV), inp.D.to(DEV),
                               inp.cu_seqlens.to(DEV), g_cache, inp.state_indices.to(DEV),
                               inp.has_initial.to(DEV), y, ckpt, ssd.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    ref = oracle.prefill(inp.x, dt_ref, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, Q, checkpoints=ck)
    assert_close(y, ref["y"], ti, "y", normalised=False)
    used = inp.state_indices.long()
    assert_close(g_cache.cpu()[used], ref["final"], looser(ti, ts), "final states")
    if ck:
        nc = int(meta[-1])
        assert_close(ckpt.cpu()[:nc], ref["ckpt"], looser(ti, ts), "checkpoints")


def test_c1_layer_prefill_fused_dt_full():
    """The 4096-token, 80-head layer with the step-size preprocessing fused in; the
    oracle checks every head (y, the final state, and y's SSM part with D = 0)."""
    ssd = _ssd()
    cfg = sy.C1
    inp = sy.make_prefill(cfg)
    T, H, P, N, G, Q = 4096, cfg.nheads, cfg.headdim, cfg.d_state, cfg.ngroups, cfg.chunk_size
    bias = torch.from_numpy(inp.dt_bias).float()
    p = ssd.make_problem(T, 1, H, P, N, G, Q, 1, cfg.in_dtype, cfg.state_dtype)
    tf = ssd.make_dt_transform(bias.to(DEV), sy.DT_MIN, sy.DT_MAX)
    dt_ref = torch.from_numpy(oracle.dt_preprocess(inp.dt_raw, bias, sy.DT_MIN, sy.DT_MAX))
    for with_d in (True, False):
        cache = torch.zeros(1, H, P, N, device=DEV)
        y = torch.empty(T, H, P, dtype=BF16, device=DEV)
        ssd.ssd_combined_varlen_dt(p, tf, inp.x.to(DEV), inp.dt_raw.to(DEV), inp.A.to(DEV),
                                   inp.B.to(DEV), inp.C.to(DEV),
                                   inp.D.to(DEV) if with_d else None, inp.cu_seqlens.to(DEV),
                                   cache, inp.state_indices.to(DEV), None, y, None,
                                   ssd.alloc_workspace(p, DEV))
        torch.cuda.synchronize()
        ry, rf, _ = oracle.recurrence(inp.x, dt_ref, inp.A, inp.B, inp.C,
                                      inp.D if with_d else None, [0, T], Q)
        tag = "" if with_d else " (D = 0)"
        assert_close(y.cpu(), ry, BF16, "c1 y (fused dt)" + tag, normalised=not with_d)
        assert_close(cache.cpu()[0], rf[0], BF16, "c1 final state (fused dt)" + tag)
