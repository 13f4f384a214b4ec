"""GPU parity of the ReplaySSM decode path (checkpoint + input rings + cursor)
against the oracle's state machine over several verify / accept steps."""
import dataclasses

import numpy as np
import pytest
import torch

import ssd_synth as sy
from gpu_helpers import DEV, assert_close, looser, workload_cache
from oracle import replay as oracle_replay

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def _ssd():
    import state_space_model_varlen_amd as ssd
    return ssd


def _step_inputs(cfg, step, idx):
    """Seeded tokens of one verify step; the requests keep their slots and the layer
    its A and D across steps."""
    base = sy.make_decode(cfg)
    d = sy.make_decode(dataclasses.replace(cfg, seed=cfg.seed + 1000 * step))
    return dataclasses.replace(d, state_indices=idx.clone(), A=base.A, D=base.D)


def _run_steps(cfg, W, cache, steps, sample=None):
    """Runs `steps` verify + advance steps on the GPU and in the oracle, then
    materialises; compares y, rings, cursors and checkpoints after every step.
    `sample` restricts the oracle to some requests (the GPU runs them all)."""
    ssd = _ssd()
    R, T, H, P, N, G = (cfg.num_reqs, cfg.tokens_per_req, cfg.nheads, cfg.headdim, cfg.d_state,
                        cfg.ngroups)
    ti, ts = cfg.in_dtype, cfg.state_dtype
    up = ssd.make_ssu_problem(R, T, H, P, N, G, cfg.num_slots, ti, ts)
    rings = ssd.alloc_replay_rings(up, W, DEV)
    g_ckpt = cache.to(DEV)
    idx = sy.make_decode(cfg).state_indices
    rs = list(range(R)) if sample is None else list(sample)
    sidx = idx[rs]
    slots = [int(s) for s in sidx]
    layer = oracle_replay.ReplayLayer(cache, W, G, ti)
    for step in range(steps):
        d = _step_inputs(cfg, step, idx)
        y = torch.empty(R, T, H, P, dtype=ti, device=DEV)
        ssd.ssd_replay_update(up, W, g_ckpt, rings["ring_x"], rings["ring_dt"], rings["ring_B"],
                              rings["cursor"], idx.to(DEV), d.x.to(DEV), d.dt.to(DEV),
                              d.A.to(DEV), d.B.to(DEV), d.C.to(DEV), d.D.to(DEV), y)
        yref = oracle_replay.replay_update(layer, sidx, d.x[rs], d.dt[rs], d.A, d.B[rs], d.C[rs],
                                           d.D)
        torch.cuda.synchronize()
        assert_close(y[rs], yref, ti, f"step {step} y", normalised=False)
        # the rings hold copies of the inputs: bit-exact
        for name, ref in (("ring_x", layer.ring_x), ("ring_dt", layer.ring_dt),
                          ("ring_B", layer.ring_B)):
            got = rings[name].cpu()[slots]
            assert torch.equal(got.view(torch.uint8), ref[slots].view(torch.uint8)), \
                f"step {step}: {name}"
        assert_close(g_ckpt[slots], layer.ckpt[slots], looser(ti, ts), f"step {step} checkpoints")
        acc = d.num_accepted
        ssd.ssd_replay_advance(up, W, rings["cursor"], idx.to(DEV), acc.to(DEV))
        oracle_replay.replay_advance(layer, sidx, acc[rs].numpy(), T)
        torch.cuda.synchronize()
        assert np.array_equal(rings["cursor"].cpu().numpy()[slots], layer.cursor[slots]), step
    ssd.ssd_replay_materialize(up, W, g_ckpt, rings["ring_x"], rings["ring_dt"], rings["ring_B"],
                               rings["cursor"], idx.to(DEV), cfg_A(cfg).to(DEV))
    oracle_replay.replay_materialize(layer, sidx, cfg_A(cfg))
    torch.cuda.synchronize()
    assert_close(g_ckpt[slots], layer.ckpt[slots], looser(ti, ts), "materialised checkpoints")
    assert np.array_equal(rings["cursor"].cpu().numpy()[slots], layer.cursor[slots])
    assert (rings["cursor"].cpu().numpy()[slots][:, 1] == 0).all()
    return g_ckpt, idx


def cfg_A(cfg):
    return sy.make_decode(cfg).A


CASES = [
    # R, T, H, P, N, G, W, in, state
    (4, 3, 8, 64, 128, 2, 9, BF16, BF16),
    (3, 2, 4, 16, 16, 1, 5, F32, F32),
    (5, 4, 4, 64, 16, 2, 8, BF16, F32),     # W = 2 T: a checkpoint at every other step
    (2, 1, 6, 16, 128, 3, 4, F32, BF16),    # plain decode (no drafts)
    (3, 4, 8, 64, 128, 2, 20, BF16, BF16),  # bf16 fast path with 32 token slots
    (4, 4, 4, 64, 128, 4, 8, BF16, BF16),   # bf16 fast path, W = 2 T
    (3, 2, 8, 64, 128, 8, 40, BF16, BF16),  # bf16, ring longer than the fast path takes
    (3, 3, 12, 64, 128, 2, 12, BF16, BF16),  # bf16 fast path, 6 heads per group (2 per block)
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"R{c[0]}T{c[1]}P{c[3]}N{c[4]}W{c[6]}_"
                         f"{str(c[7])[6:]}_{str(c[8])[6:]}")
def test_replay_steps_match_oracle(case):
    R, T, H, P, N, G, W, ti, ts = case
    slots = 2 * R + 1
    cfg = sy.DecodeConfig(f"replay{CASES.index(case)}", R, T, H, P, N, G, ti, ts, slots, 8,
                          300 + CASES.index(case))
    idx = sy.make_decode(cfg).state_indices
    cache = sy.nan_cache(slots, H, P, N, ts)
    g = torch.Generator().manual_seed(CASES.index(case))
    for s in idx:
        cache[int(s)] = (torch.randn(H, P, N, generator=g) * 0.05).to(ts)
    g_ckpt, _ = _run_steps(cfg, W, cache, steps=8)
    # slots no request uses were never read or written (still NaN)
    other = [s for s in range(slots) if s not in set(int(v) for v in idx)]
    assert torch.isnan(g_ckpt.cpu()[other].float()).all()


def test_replay_agrees_with_stored_states_path():
    """Against the other decode path on the GPU: after accepting tokens step by step,
    the materialised checkpoint equals committing the stored intermediate states
    (float32 storage, so the two differ only by summation order)."""
    ssd = _ssd()
    R, T, H, P, N, G, W = 3, 3, 4, 64, 128, 2, 8
    cfg = sy.DecodeConfig("replay_vs_commit", R, T, H, P, N, G, F32, F32, 7, 8, 400)
    idx = sy.make_decode(cfg).state_indices
    g = torch.Generator().manual_seed(5)
    cache = torch.randn(7, H, P, N, generator=g) * 0.05
    up = ssd.make_ssu_problem(R, T, H, P, N, G, 7, F32, F32)
    rings = ssd.alloc_replay_rings(up, W, DEV)
    c_replay, c_plain = cache.to(DEV), cache.to(DEV)
    y1 = torch.empty(R, T, H, P, device=DEV)
    y2 = torch.empty_like(y1)
    inter = torch.empty(R, T, H, P, N, device=DEV)
    for step in range(5):
        d = _step_inputs(cfg, step, idx)
        args = [t.to(DEV) for t in (d.x, d.dt, d.A, d.B, d.C, d.D)]
        ssd.ssd_replay_update(up, W, c_replay, rings["ring_x"], rings["ring_dt"],
                              rings["ring_B"], rings["cursor"], idx.to(DEV), *args, y1)
        ssd.selective_state_update(up, c_plain, idx.to(DEV), *args, y2, inter)
        ssd.ssd_replay_advance(up, W, rings["cursor"], idx.to(DEV), d.num_accepted.to(DEV))
        ssd.ssd_state_commit(up, c_plain, idx.to(DEV), inter, d.num_accepted.to(DEV))
        torch.cuda.synchronize()
        assert_close(y1, y2, F32, f"step {step}: y of the two paths")
    ssd.ssd_replay_materialize(up, W, c_replay, rings["ring_x"], rings["ring_dt"],
                               rings["ring_B"], rings["cursor"], idx.to(DEV), cfg_A(cfg).to(DEV))
    torch.cuda.synchronize()
    assert_close(c_replay, c_plain, F32, "states of the two paths")


def test_c4_replay_full():
    """The MTP verify workload (128 requests x 3 tokens, 128 heads, bf16 cache of 512
    slots) through ReplaySSM with a 16-entry ring, 6 steps; every request starts from
    the oracle's state after its own seeded prefix, and the oracle follows every
    request (all heads): y, rings, cursors and checkpoints after each step."""
    cfg = sy.C4
    cache = workload_cache(sy.make_decode(cfg))
    _run_steps(cfg, 16, cache, steps=6)


def test_replay_slots_past_4gb():
    """Checkpoints of 2560 slots x 128 heads x 64 x 128 in bf16 (5.4 GB) and input
    rings of 32 tokens: the requests' slots lie past 2^31 and 2^32 bytes of the
    checkpoints. Three verify + advance steps and the materialisation against the
    oracle's state machine on a layer holding only those slots (renumbered): y,
    the rings bit for bit, the cursors and the checkpoints after every step."""
    ssd = _ssd()
    R, T, H, P, N, G, W, slots = 4, 3, 128, 64, 128, 8, 32, 2560
    cfg = sy.DecodeConfig("replay_big", R, T, H, P, N, G, BF16, BF16, slots, 8, 654)
    sidx = torch.tensor([slots - 1, 2100, 1, 2400], dtype=torch.int32)
    g = torch.Generator().manual_seed(9)
    small = (torch.randn(R, H, P, N, generator=g) * 0.05).to(BF16)
    g_ckpt = torch.full((slots, H, P, N), float("nan"), dtype=BF16, device=DEV)
    g_ckpt[sidx.long().to(DEV)] = small.to(DEV)
    up = ssd.make_ssu_problem(R, T, H, P, N, G, slots, BF16, BF16)
    rings = ssd.alloc_replay_rings(up, W, DEV)
    layer = oracle_replay.ReplayLayer(small, W, G, BF16)
    oidx = torch.arange(R, dtype=torch.int32)
    at = sidx.long().to(DEV)
    A = cfg_A(cfg)
    for step in range(3):
        d = _step_inputs(cfg, step, sidx)
        y = torch.empty(R, T, H, P, dtype=BF16, device=DEV)
        ssd.ssd_replay_update(up, W, g_ckpt, rings["ring_x"], rings["ring_dt"], rings["ring_B"],
                              rings["cursor"], sidx.to(DEV), d.x.to(DEV), d.dt.to(DEV),
                              A.to(DEV), d.B.to(DEV), d.C.to(DEV), d.D.to(DEV), y)
        yref = oracle_replay.replay_update(layer, oidx, d.x, d.dt, A, d.B, d.C, d.D)
        torch.cuda.synchronize()
        assert_close(y.cpu(), yref, BF16, f"step {step} y", normalised=False)
        for name, ref in (("ring_x", layer.ring_x), ("ring_dt", layer.ring_dt),
                          ("ring_B", layer.ring_B)):
            got = rings[name][at].cpu()
            assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8)), f"step {step}: {name}"
        assert_close(g_ckpt[at].cpu(), layer.ckpt, BF16, f"step {step} checkpoints")
        acc = d.num_accepted
        ssd.ssd_replay_advance(up, W, rings["cursor"], sidx.to(DEV), acc.to(DEV))
        oracle_replay.replay_advance(layer, oidx, acc.numpy(), T)
        torch.cuda.synchronize()
        assert np.array_equal(rings["cursor"][at].cpu().numpy(), layer.cursor), step
    ssd.ssd_replay_materialize(up, W, g_ckpt, rings["ring_x"], rings["ring_dt"], rings["ring_B"],
                               rings["cursor"], sidx.to(DEV), A.to(DEV))
    oracle_replay.replay_materialize(layer, oidx, A)
    torch.cuda.synchronize()
    assert_close(g_ckpt[at].cpu(), layer.ckpt, BF16, "materialised checkpoints")
    assert np.array_equal(rings["cursor"][at].cpu().numpy(), layer.cursor)
    assert torch.isnan(g_ckpt[slots - 2].float()).all()
