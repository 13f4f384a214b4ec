"""GPU parity of the decode / MTP verify selective state update and of the
rollback commit against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import ssd_synth as sy
from gpu_helpers import DEV, assert_close, looser, workload_cache

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def _ssd():
    import state_space_model_varlen_amd as ssd
    return ssd


def _run(d, cache, keep, D=True):
    ssd = _ssd()
    R, T, H, P = d.x.shape
    G, N = d.B.shape[2], d.B.shape[3]
    up = ssd.make_ssu_problem(R, T, H, P, N, G, cache.shape[0], d.x.dtype, cache.dtype)
    g_cache = cache.to(DEV)
    y = torch.empty(R, T, H, P, dtype=d.x.dtype, device=DEV)
    inter = torch.empty(R, T, H, P, N, dtype=cache.dtype, device=DEV) if keep else None
    ssd.selective_state_update(up, g_cache, d.state_indices.to(DEV), d.x.to(DEV), d.dt.to(DEV),
                               d.A.to(DEV), d.B.to(DEV), d.C.to(DEV),
                               d.D.to(DEV) if D else None, y, inter)
    torch.cuda.synchronize()
    return up, g_cache, y, inter


def _inputs(R, T, H, P, N, G, ti, ts, slots, seed):
    cfg = sy.DecodeConfig(f"dec{seed}", R, T, H, P, N, G, ti, ts, slots, 8, 200 + seed)
    d = sy.make_decode(cfg)
    g = torch.Generator().manual_seed(seed)
    cache = sy.nan_cache(slots, H, P, N, ts)
    for r in range(R):
        cache[int(d.state_indices[r])] = (torch.randn(H, P, N, generator=g) * 0.05).to(ts)
    return d, cache


CASES = [
    # R, T, H, P, N, G, in, state
    (4, 3, 8, 64, 128, 2, BF16, BF16),
    (3, 1, 4, 64, 128, 4, BF16, F32),
    (5, 4, 4, 16, 16, 1, F32, F32),
    (2, 3, 6, 16, 128, 3, F32, BF16),
    (3, 2, 4, 64, 16, 2, BF16, BF16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"R{c[0]}T{c[1]}P{c[3]}N{c[4]}_"
                         f"{str(c[6])[6:]}_{str(c[7])[6:]}")
def test_state_update_with_intermediate_states(case):
    R, T, H, P, N, G, ti, ts = case
    d, cache = _inputs(R, T, H, P, N, G, ti, ts, 2 * R + 1, CASES.index(case))
    up, g_cache, y, inter = _run(d, cache, keep=True)
    ref = oracle.state_update(cache, d.state_indices, d.x, d.dt, d.A, d.B, d.C, d.D, True)
    assert_close(y, ref["y"], ti, "y", normalised=False)
    assert_close(inter, ref["states"], looser(ti, ts), "intermediate states")
    # with intermediate states kept, the cache is not written
    assert torch.equal(g_cache.cpu().view(torch.uint8), cache.view(torch.uint8))
    # y of the D = 0 run: the SSM part alone, normalised
    _, _, y0, _ = _run(d, cache, keep=True, D=False)
    ref0 = oracle.state_update(cache, d.state_indices, d.x, d.dt, d.A, d.B, d.C, None, True)
    assert_close(y0, ref0["y"], ti, "y (D = 0)")


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"R{c[0]}T{c[1]}P{c[3]}N{c[4]}")
def test_plain_update_writes_the_cache(case):
    R, T, H, P, N, G, ti, ts = case
    d, cache = _inputs(R, T, H, P, N, G, ti, ts, 2 * R + 1, 10 + CASES.index(case))
    up, g_cache, y, _ = _run(d, cache, keep=False)
    ref = oracle.state_update(cache, d.state_indices, d.x, d.dt, d.A, d.B, d.C, d.D, False)
    assert_close(y, ref["y"], ti, "y", normalised=False)
    after = g_cache.cpu()
    idx = d.state_indices.long()
    assert_close(after[idx], ref["final"], looser(ti, ts), "final states")
    others = [s for s in range(cache.shape[0]) if s not in set(idx.tolist())]
    assert torch.isnan(after[others].float()).all()


def test_commit_rolls_back_to_accepted_count():
    ssd = _ssd()
    R, T, H, P, N, G = 6, 3, 4, 64, 128, 2
    d, cache = _inputs(R, T, H, P, N, G, BF16, BF16, 16, 21)
    up, g_cache, y, inter = _run(d, cache, keep=True)
    acc = torch.tensor([0, 1, 2, 2, 3, -1], dtype=torch.int32)   # last two are out of range
    ssd.ssd_state_commit(up, g_cache, d.state_indices.to(DEV), inter, acc.to(DEV))
    torch.cuda.synchronize()
    after = g_cache.cpu()
    ic = inter.cpu()
    for r in range(R):
        slot = int(d.state_indices[r])
        a = int(acc[r])
        if 0 <= a < T:
            assert torch.equal(after[slot].view(torch.int16), ic[r, a].view(torch.int16))
        else:
            assert torch.equal(after[slot].view(torch.int16), cache[slot].view(torch.int16))
    # committing a accepted drafts == a plain update over the first 1 + a tokens
    for r in range(4):
        a = int(acc[r])
        sub = sy.DecodeInputs(cfg=d.cfg, x=d.x[r:r + 1, :a + 1].contiguous(),
                              dt=d.dt[r:r + 1, :a + 1].contiguous(), A=d.A,
                              B=d.B[r:r + 1, :a + 1].contiguous(), C=d.C[r:r + 1, :a + 1].contiguous(),
                              D=d.D, state_indices=d.state_indices[r:r + 1].clone(),
                              num_accepted=acc[r:r + 1].clone())
        _, c2, _, _ = _run(sub, cache, keep=False)
        slot = int(d.state_indices[r])
        assert torch.equal(c2.cpu()[slot].view(torch.int16), after[slot].view(torch.int16)), r


def test_c4_mtp_verify_full():
    """128 requests x 3 tokens, bf16 cache of 512 slots. Every request starts from
    the oracle's state after its own seeded 256-token prefix; the oracle checks
    every (request, head): y, the intermediate state after each token, the
    rollback to the accepted counts, and with D = 0 y's SSM part under the
    normalised bound. Compared 16 requests at a time to bound host memory."""
    cfg = sy.C4
    d = sy.make_decode(cfg)
    cache = workload_cache(d)
    up, g_cache, y, inter = _run(d, cache, keep=True)
    _, _, yd, _ = _run(d, cache, keep=True, D=False)
    ssd = _ssd()
    ssd.ssd_state_commit(up, g_cache, d.state_indices.to(DEV), inter, d.num_accepted.to(DEV))
    torch.cuda.synchronize()
    y, yd, inter, after = y.cpu(), yd.cpu(), inter.cpu(), g_cache.cpu()
    for r0 in range(0, cfg.num_reqs, 16):
        rs = list(range(r0, min(r0 + 16, cfg.num_reqs)))
        sidx = d.state_indices[rs]
        ref = oracle.state_update(cache, sidx, d.x[rs], d.dt[rs], d.A, d.B[rs], d.C[rs], d.D,
                                  True)
        assert_close(y[rs], ref["y"], BF16, f"c4 y r{r0}", normalised=False)
        assert_close(inter[rs], ref["states"], BF16, f"c4 intermediate states r{r0}")
        refd = oracle.state_update(cache, sidx, d.x[rs], d.dt[rs], d.A, d.B[rs], d.C[rs], None,
                                   False)
        assert_close(yd[rs], refd["y"], BF16, f"c4 y (D = 0) r{r0}")
        acc = d.num_accepted[rs].long()
        assert_close(after[sidx.long()], ref["states"][np.arange(len(rs)), acc.numpy()], BF16,
                     f"c4 committed states r{r0}")
    used = set(d.state_indices.tolist())
    others = [k for k in range(cfg.num_slots) if k not in used]
    assert torch.isnan(after[others].float()).all()


@pytest.mark.parametrize("keep", [True, False], ids=["per_token_states", "cache_written"])
def test_state_update_cache_past_4gb(keep):
    """A bf16 cache of 2560 slots x 128 heads x 64 x 128 (5.4 GB): the requests'
    slots lie past 2^31 and 2^32 bytes. y, the per-token states and the written
    slots against the oracle (run on a cache holding only those slots, renumbered);
    a NaN slot next to a written one stays NaN."""
    ssd = _ssd()
    R, T, H, P, N, G, slots = 4, 3, 128, 64, 128, 8, 2560
    cfg = sy.DecodeConfig("dec_big", R, T, H, P, N, G, BF16, BF16, slots, 8, 321)
    d = sy.make_decode(cfg)
    sidx = torch.tensor([slots - 1, 2100, 1, 2400], dtype=torch.int32)
    g = torch.Generator().manual_seed(5)
    small = (torch.randn(R, H, P, N, generator=g) * 0.05).to(BF16)
    g_cache = torch.full((slots, H, P, N), float("nan"), dtype=BF16, device=DEV)
    g_cache[sidx.long().to(DEV)] = small.to(DEV)
    up = ssd.make_ssu_problem(R, T, H, P, N, G, slots, BF16, BF16)
    y = torch.empty(R, T, H, P, dtype=BF16, device=DEV)
    inter = torch.empty(R, T, H, P, N, dtype=BF16, device=DEV) if keep else None
    ssd.selective_state_update(up, g_cache, sidx.to(DEV), d.x.to(DEV), d.dt.to(DEV),
                               d.A.to(DEV), d.B.to(DEV), d.C.to(DEV), d.D.to(DEV), y, inter)
    torch.cuda.synchronize()
    ref = oracle.state_update(small, torch.arange(R, dtype=torch.int32), d.x, d.dt, d.A, d.B,
                              d.C, d.D, keep)
    assert_close(y.cpu(), ref["y"], BF16, "y", normalised=False)
    after = g_cache[sidx.long().to(DEV)].cpu()
    if keep:
        assert_close(inter.cpu(), ref["states"], BF16, "per-token states")
        assert torch.equal(after.view(torch.int16), small.view(torch.int16))
    else:
        assert_close(after, ref["final"], BF16, "final states")
    assert torch.isnan(g_cache[slots - 2].float()).all()
