"""GPU checks of the fp16 state cache with stochastic rounding: the rounding
itself bit for bit against the oracle's definition (same float32 inputs, same
Philox words), and the prefill / decode / ReplaySSM paths against the float64
oracle within one fp16 step, deterministic for a seed and unbiased over seeds."""
import numpy as np
import pytest
import torch

import oracle
import ssd_synth as sy
from gpu_helpers import DEV, assert_close
from oracle import replay as oracle_replay
from oracle import rounding as rnd

pytestmark = pytest.mark.gpu

F32, BF16, F16 = torch.float32, torch.bfloat16, torch.float16


def _ssd():
    import state_space_model_varlen_amd as ssd
    return ssd


def _seed(v):
    return torch.tensor([v], dtype=torch.int64, device=DEV)


def _u64(v):
    return v & 0xFFFFFFFFFFFFFFFF


@pytest.mark.parametrize("seed,rounds,kind", [(0x0123456789ABCDEF, 10, 0), (7, 5, 3),
                                              (-2, 1, 2)])
def test_round_f16_bit_exact(seed, rounds, kind):
    ssd = _ssd()
    g = np.random.default_rng(181)
    x = np.concatenate([g.standard_normal(3000) * 0.03, g.standard_normal(500) * 300.0,
                        g.uniform(-6e-5, 6e-5, 400), g.uniform(-3e-7, 3e-7, 60),
                        np.arange(-8, 8, dtype=np.float32) / 8,       # exact fp16 values
                        # across the subnormal / normal boundary 2^-14, fp32 subnormals,
                        # multiples of the subnormal spacing 2^-24, the top binade
                        np.float32(2.0 ** -14) * (1 + g.uniform(-3e-3, 3e-3, 200)),
                        g.standard_normal(40) * 1e-40, np.arange(-5, 6) * 2.0 ** -25,
                        g.uniform(65400.0, 65504.0, 60), [65504.0, -65504.0, 65519.0, 65520.0],
                        [np.inf, -np.inf, np.nan, 70000.0, 65510.0, 0.0, -0.0]]).astype(np.float32)
    n = len(x) - 1                       # a ragged tail (not a multiple of 4)
    xg = torch.from_numpy(x[:n]).to(DEV)
    out = torch.empty(n, dtype=F16, device=DEV)
    ssd.ssd_round_f16(xg, out, sr_seed=_seed(seed), sr_rounds=rounds, kind=kind)
    torch.cuda.synchronize()
    want = rnd.stochastic_round_f16(x[:n], rnd.draws_for(n, _u64(seed), kind, rounds))
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), \
        int(np.sum(got.view(np.uint16) != want.view(np.uint16)))
    # without a seed: round to nearest even, as torch converts
    ssd.ssd_round_f16(xg, out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), xg.cpu().half().view(torch.int16))


@pytest.mark.parametrize("seed,rounds,kind", [(0xFEEDFACE, 5, 2), (-9, 10, 1)])
def test_round_f16_normal_range_bit_exact(seed, rounds, kind):
    """Only values in the fp16 normal range (2^-14 .. 65504, both signs, every
    binade, the end points included), so every wave takes the carry-step path
    and none the general rule."""
    ssd = _ssd()
    g = np.random.default_rng(182)
    n = 64 * 256 * 4 + 13                # many waves and a ragged tail
    mag = np.exp2(g.uniform(-14.0, 16.0, n)).clip(2.0 ** -14, 65504.0)
    mag[:4] = [2.0 ** -14, 65504.0, 1.0, 2.0 ** -14 * (1 + 2.0 ** -12)]
    x = (mag * np.where(g.random(n) < 0.5, -1.0, 1.0)).astype(np.float32)
    out = torch.empty(n, dtype=F16, device=DEV)
    ssd.ssd_round_f16(torch.from_numpy(x).to(DEV), out, sr_seed=_seed(seed), sr_rounds=rounds,
                      kind=kind)
    torch.cuda.synchronize()
    want = rnd.stochastic_round_f16(x, rnd.draws_for(n, _u64(seed), kind, rounds))
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16)), \
        int(np.sum(got.view(np.uint16) != want.view(np.uint16)))


def test_round_f16_one_off_range_slot_per_wave():
    """Normal-range values everywhere except one value per 512 (one wave of
    ssd_round_f16, 8 consecutive values per lane): in wave k, lane 7 k mod 64 holds
    an fp16 subnormal, a zero, an overflow or a non-finite value in value slot
    k mod 8. Every wave then mixes slots that take the general rule with slots that
    do not; every 9th wave is left all normal."""
    ssd = _ssd()
    g = np.random.default_rng(183)
    waves = 72
    n = 512 * waves + 5
    mag = np.exp2(g.uniform(-14.0, 16.0, n)).clip(2.0 ** -14, 65504.0)
    x = (mag * np.where(g.random(n) < 0.5, -1.0, 1.0)).astype(np.float32)
    odd = np.array([3e-6, -4.5e-7, 0.0, -0.0, 6.0e-5, 2.0 ** -24, 65519.0, -70000.0, np.inf,
                    np.nan, 1e-40, 2.0 ** -14 * (1 - 2.0 ** -20)], dtype=np.float32)
    for k in range(waves):
        if k % 9 == 8:
            continue
        x[512 * k + 8 * ((7 * k) % 64) + k % 8] = odd[k % len(odd)]
    out = torch.empty(n, dtype=F16, device=DEV)
    ssd.ssd_round_f16(torch.from_numpy(x).to(DEV), out, sr_seed=_seed(0x51075107), sr_rounds=5,
                      kind=3)
    torch.cuda.synchronize()
    want = rnd.stochastic_round_f16(x, rnd.draws_for(n, _u64(0x51075107), 3, 5))
    got = out.cpu().numpy().view(np.uint16)
    want = want.view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan]), int(np.sum(got[~nan] != want[~nan]))
    assert np.all(np.isnan(out.cpu().numpy()[nan]))

def _f16_step_bound(ref):
    """One fp16 step at the value (the spacing of the bracketing fp16 values)."""
    a = np.abs(np.asarray(ref, dtype=np.float64)).astype(np.float32)
    lo, hi = rnd._f16_neighbours(a)
    return np.abs(hi.astype(np.float64) - lo.astype(np.float64))


def _prefill(inp, cache, Q, seed, rounds=10, ck=True):
    ssd = _ssd()
    T, S = int(inp.cu_seqlens[-1]), len(inp.cu_seqlens) - 1
    H, P, N, G = inp.x.shape[1], inp.x.shape[2], inp.B.shape[2], inp.B.shape[1]
    p = ssd.make_problem(T, S, H, P, N, G, Q, cache.shape[0], inp.x.dtype, F16)
    sd = None if seed is None else _seed(seed)
    opt = ssd.make_options(sr_seed=sd, sr_rounds=rounds)
    g_cache = cache.to(DEV)
    y = torch.empty(T, H, P, dtype=inp.x.dtype, device=DEV)
    ckpt = torch.empty(ssd.max_chunks(p), H, P, N, dtype=F16, device=DEV) if ck else None
    ssd.ssd_combined_varlen_ex(p, opt, inp.x.to(DEV), inp.dt.to(DEV), inp.A.to(DEV),
                               inp.B.to(DEV), inp.C.to(DEV), inp.D.to(DEV),
                               inp.cu_seqlens.to(DEV), g_cache, inp.state_indices.to(DEV),
                               inp.has_initial.to(DEV), y, ckpt, ssd.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    return y.cpu(), g_cache.cpu(), None if ckpt is None else ckpt.cpu()


def _problem(lens, H, P, N, G, Q, ti, seed):
    S = len(lens)
    inp = sy.random_problem(seed, lens, H, P, N, G, Q, ti, F16, num_slots=2 * S + 1,
                            has_initial=[s % 2 == 0 for s in range(S)])
    cache = sy.nan_cache(2 * S + 1, H, P, N, F16)
    g = torch.Generator().manual_seed(seed)
    for s in range(S):
        if int(inp.has_initial[s]):
            cache[int(inp.state_indices[s])] = (torch.randn(H, P, N, generator=g) * 0.05).half()
    return inp, cache


def test_prefill_fp32_inputs_fp16_cache_within_one_step():
    """float32 inputs: the float32 state is within ~1e-6 of the float64 one, so every
    stored fp16 state is one of the two fp16 values around the exact state."""
    Q = 64
    inp, cache = _problem((150, 0, 37, 260), 4, 16, 16, 2, Q, F32, 811)
    y, after, ck = _prefill(inp, cache, Q, seed=12345)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, Q, checkpoints=True)
    assert_close(y, ref["y"], F32, "y", normalised=False)
    used = inp.state_indices.long()
    for got, want, what in ((after[used], ref["final"], "final states"),
                            (ck[:len(ref["ckpt"])], ref["ckpt"], "checkpoints")):
        g64 = got.double().numpy()
        err = np.abs(g64 - want)
        assert np.all(err <= _f16_step_bound(want) * (1 + 1e-3) + 1e-7), what
    # deterministic for a seed, different for another
    _, after2, ck2 = _prefill(inp, cache, Q, seed=12345)
    assert torch.equal(after2.view(torch.int16), after.view(torch.int16))
    nck = len(ref["ckpt"])            # rows past the last checkpoint are never written
    assert torch.equal(ck2[:nck].view(torch.int16), ck[:nck].view(torch.int16))
    _, after3, _ = _prefill(inp, cache, Q, seed=54321)
    assert not torch.equal(after3[used].view(torch.int16), after[used].view(torch.int16))


def test_prefill_stochastic_rounding_is_unbiased():
    """Averaged over 32 seeds the fp16 final states approach the exact ones far closer
    than rounding to nearest does."""
    Q = 64
    inp, cache = _problem((200, 90), 4, 16, 16, 2, Q, F32, 812)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, Q)
    used = inp.state_indices.long()
    acc = np.zeros(ref["final"].shape)
    for k in range(32):
        _, after, _ = _prefill(inp, cache, Q, seed=1000 + k, ck=False)
        acc += after[used].double().numpy()
    mean_err = np.mean(np.abs(acc / 32 - ref["final"]))
    rne_err = np.mean(np.abs(ref["final"].astype(np.float16).astype(np.float64) - ref["final"]))
    assert mean_err < 0.5 * rne_err, (mean_err, rne_err)


def test_prefill_bf16_fused_path_fp16_cache():
    """The fused bf16 state kernel with an fp16 cache and checkpoints (bf16
    tolerance: its chunk states carry bf16-rounded operands)."""
    Q = 256
    inp, cache = _problem((600, 32, 1, 257), 8, 64, 128, 2, Q, BF16, 813)
    y, after, ck = _prefill(inp, cache, Q, seed=99, rounds=5)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, Q, checkpoints=True)
    assert_close(y, ref["y"], BF16, "y", normalised=False)
    used = inp.state_indices.long()
    assert_close(after[used], ref["final"], BF16, "final states")
    assert_close(ck[:len(ref["ckpt"])], ref["ckpt"], BF16, "checkpoints")
    _, after2, ck2 = _prefill(inp, cache, Q, seed=99, rounds=5)
    assert torch.equal(after2.view(torch.int16), after.view(torch.int16))
    nck = len(ref["ckpt"])            # rows past the last checkpoint are never written
    assert torch.equal(ck2[:nck].view(torch.int16), ck[:nck].view(torch.int16))


def test_prefill_bf16_segmented_fp16_cache():
    """Without checkpoints a short batch takes the segmented state path: the final
    fp16 states are written (stochastically rounded) by the carry step."""
    Q = 128
    inp, cache = _problem((1500, 3, 900), 4, 64, 128, 2, Q, BF16, 814)
    y, after, _ = _prefill(inp, cache, Q, seed=7, rounds=5, ck=False)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, Q)
    assert_close(y, ref["y"], BF16, "y", normalised=False)
    used = inp.state_indices.long()
    assert_close(after[used], ref["final"], BF16, "final states")
    _, after2, _ = _prefill(inp, cache, Q, seed=7, rounds=5, ck=False)
    assert torch.equal(after2.view(torch.int16), after.view(torch.int16))


def test_prefill_bf16_short_path_fp16_cache():
    """A batch of short sequences (the one-launch path) with an fp16 cache,
    checkpoints and Philox-5 stochastic rounding: within the bf16 tolerance of the
    oracle, the same bits for the same seed, other bits for another seed."""
    Q = 256
    inp, cache = _problem((20, 1, 0, 90, 33, 64) * 4, 8, 64, 128, 2, Q, BF16, 815)
    y, after, ck = _prefill(inp, cache, Q, seed=31, rounds=5)
    ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                         inp.state_indices, inp.has_initial, cache, Q, checkpoints=True)
    assert_close(y, ref["y"], BF16, "y", normalised=False)
    used = inp.state_indices.long()
    assert_close(after[used], ref["final"], BF16, "final states")
    assert_close(ck[:len(ref["ckpt"])], ref["ckpt"], BF16, "checkpoints")
    _, after2, ck2 = _prefill(inp, cache, Q, seed=31, rounds=5)
    assert torch.equal(after2.view(torch.int16), after.view(torch.int16))
    nck = len(ref["ckpt"])            # rows past the last checkpoint are never written
    assert torch.equal(ck2[:nck].view(torch.int16), ck[:nck].view(torch.int16))
    _, after3, _ = _prefill(inp, cache, Q, seed=32, rounds=5)
    assert not torch.equal(after3[used].view(torch.int16), after[used].view(torch.int16))


@pytest.mark.parametrize("keep", [True, False])
def test_decode_fp16_states(keep):
    ssd = _ssd()
    R, T, H, P, N, G = 4, 3, 4, 16, 16, 2
    cfg = sy.DecodeConfig("sr_dec", R, T, H, P, N, G, F32, F16, 9, 8, 820)
    d = sy.make_decode(cfg)
    cache = sy.nan_cache(9, H, P, N, F16)
    g = torch.Generator().manual_seed(3)
    for s in d.state_indices:
        cache[int(s)] = (torch.randn(H, P, N, generator=g) * 0.05).half()
    up = ssd.make_ssu_problem(R, T, H, P, N, G, 9, F32, F16)

    def run(seed):
        opt = ssd.make_options(sr_seed=_seed(seed), sr_rounds=10)
        g_cache = cache.to(DEV)
        y = torch.empty(R, T, H, P, device=DEV)
        inter = torch.empty(R, T, H, P, N, dtype=F16, device=DEV) if keep else None
        ssd.selective_state_update_ex(up, opt, g_cache, d.state_indices.to(DEV), d.x.to(DEV),
                                      d.dt.to(DEV), d.A.to(DEV), d.B.to(DEV), d.C.to(DEV),
                                      d.D.to(DEV), y, inter)
        torch.cuda.synchronize()
        return y.cpu(), g_cache.cpu(), None if inter is None else inter.cpu()

    y, after, inter = run(4242)
    ref = oracle.state_update(cache, d.state_indices, d.x, d.dt, d.A, d.B, d.C, d.D, keep)
    assert_close(y, ref["y"], F32, "y", normalised=False)
    if keep:
        got, want = inter.double().numpy(), ref["states"]
    else:
        got, want = after[d.state_indices.long()].double().numpy(), ref["final"]
    assert np.all(np.abs(got - want) <= _f16_step_bound(want) * (1 + 1e-3) + 1e-7)
    y2, after2, inter2 = run(4242)
    assert torch.equal(after2.view(torch.int16), after.view(torch.int16))
    if keep:
        assert torch.equal(inter2.view(torch.int16), inter.view(torch.int16))


def test_replay_fp16_checkpoints():
    """ReplaySSM with an fp16 checkpoint and stochastic rounding over several steps:
    y and the materialised checkpoints stay within the fp16 storage error of the
    oracle's state machine, and a repeated seed repeats every bit."""
    ssd = _ssd()
    R, T, H, P, N, G, W = 3, 2, 4, 16, 16, 1, 5
    cfg = sy.DecodeConfig("sr_replay", R, T, H, P, N, G, F32, F16, 7, 8, 830)
    base = sy.make_decode(cfg)
    idx = base.state_indices
    cache = sy.nan_cache(7, H, P, N, F16)
    g = torch.Generator().manual_seed(8)
    for s in idx:
        cache[int(s)] = (torch.randn(H, P, N, generator=g) * 0.05).half()
    up = ssd.make_ssu_problem(R, T, H, P, N, G, 7, F32, F16)
    steps = []
    for k in range(6):
        d = sy.make_decode(sy.DecodeConfig("sr_replay", R, T, H, P, N, G, F32, F16, 7, 8,
                                           830 + 1000 * (k + 1)))
        steps.append((d.x, d.dt, d.B, d.C, d.num_accepted))

    def run(seed):
        opt = ssd.make_options(sr_seed=_seed(seed), sr_rounds=5)
        rings = ssd.alloc_replay_rings(up, W, DEV)
        ck = cache.to(DEV)
        ys = []
        for x, dt, B, C, acc in steps:
            y = torch.empty(R, T, H, P, device=DEV)
            ssd.ssd_replay_update_ex(up, opt, W, ck, rings["ring_x"], rings["ring_dt"],
                                     rings["ring_B"], rings["cursor"], idx.to(DEV), x.to(DEV),
                                     dt.to(DEV), base.A.to(DEV), B.to(DEV), C.to(DEV),
                                     base.D.to(DEV), y)
            ssd.ssd_replay_advance(up, W, rings["cursor"], idx.to(DEV), acc.to(DEV))
            ys.append(y.cpu())
        ssd.ssd_replay_materialize_ex(up, opt, W, ck, rings["ring_x"], rings["ring_dt"],
                                      rings["ring_B"], rings["cursor"], idx.to(DEV),
                                      base.A.to(DEV))
        torch.cuda.synchronize()
        return ys, ck.cpu()

    ys, ck = run(77)
    layer = oracle_replay.ReplayLayer(cache, W, G, F32)
    # fp16 storage: each checkpoint write moves a state by up to one fp16 step
    # (~5e-4 of its size, states ~0.05 here); y sees that through C (N = 16)
    atol = 2e-4
    for (x, dt, B, C, acc), y in zip(steps, ys):
        yref = oracle_replay.replay_update(layer, idx, x, dt, base.A, B, C, base.D)
        oracle_replay.replay_advance(layer, idx, acc.numpy(), T)
        assert np.max(np.abs(y.double().numpy() - yref)) <= atol
    oracle_replay.replay_materialize(layer, idx, base.A)
    slots = [int(s) for s in idx]
    got, want = ck[slots].double().numpy(), layer.ckpt[slots].double().numpy()
    assert np.max(np.abs(got - want)) <= 4 * np.max(_f16_step_bound(want))
    ys2, ck2 = run(77)
    assert torch.equal(ck2.view(torch.int16), ck.view(torch.int16))
    assert all(torch.equal(a, b) for a, b in zip(ys, ys2))


# ---------------------------------------------------------------------------
# Every store path of the fp16 cache against the rounding's definition, bit for
# bit: the same problem with a float32 cache gives the exact values that the
# fp16 run rounds (the state arithmetic is float32 whatever the cache dtype, and
# no initial state is read, or an fp16-exact one), so the fp16 bits must equal
# the oracle's stochastic rounding of those values with the draws of their flat
# indices in the destination array (stream 0 final states, 1 checkpoints, 2
# per-token states).

def _combined_ts(inp, nslots, Q, ts, seed=None, rounds=5, ck=True):
    ssd = _ssd()
    T, S = int(inp.cu_seqlens[-1]), len(inp.cu_seqlens) - 1
    H, P, N, G = inp.x.shape[1], inp.x.shape[2], inp.B.shape[2], inp.B.shape[1]
    p = ssd.make_problem(T, S, H, P, N, G, Q, nslots, inp.x.dtype, ts)
    opt = ssd.make_options(sr_seed=None if seed is None else _seed(seed), sr_rounds=rounds)
    cache = torch.zeros(nslots, H, P, N, dtype=ts, device=DEV)
    y = torch.empty(T, H, P, dtype=inp.x.dtype, device=DEV)
    ckpt = torch.zeros(ssd.max_chunks(p), H, P, N, dtype=ts, device=DEV) if ck else None
    ssd.ssd_combined_varlen_ex(p, opt, inp.x.to(DEV), inp.dt.to(DEV), inp.A.to(DEV),
                               inp.B.to(DEV), inp.C.to(DEV), inp.D.to(DEV),
                               inp.cu_seqlens.to(DEV), cache, inp.state_indices.to(DEV),
                               torch.zeros(S, dtype=torch.uint8, device=DEV), y, ckpt,
                               ssd.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    return cache.cpu(), None if ckpt is None else ckpt.cpu()


def _rounded(exact, seed, kind, rounds):
    flat = exact.numpy().reshape(-1)
    return rnd.stochastic_round_f16(flat, rnd.draws_for(flat.size, _u64(seed), kind, rounds)
                                    ).reshape(exact.shape).view(np.uint16)


@pytest.mark.parametrize("lens,H,Q,ck,path", [
    ((1500,), 4, 128, False, "segmented state pass: carry stores"),
    ((600, 32, 1, 257), 8, 256, True, "fused state kernel: checkpoints and finals"),
    ((20, 1, 0, 90, 33, 64) * 4, 8, 256, True, "short-sequence kernel"),
])
def test_prefill_fp16_stores_bit_exact(lens, H, Q, ck, path):
    S, seed, rounds = len(lens), 0x5EED5EED1234, 5
    inp = sy.random_problem(816, lens, H, 64, 128, 2, Q, BF16, F16, num_slots=2 * S + 1,
                            has_initial=[False] * S)
    c32, k32 = _combined_ts(inp, 2 * S + 1, Q, F32, ck=ck)
    c16, k16 = _combined_ts(inp, 2 * S + 1, Q, F16, seed=seed, rounds=rounds, ck=ck)
    used = inp.state_indices.long().numpy()
    want = _rounded(c32, seed, 0, rounds)
    got = c16.numpy().view(np.uint16)
    assert np.array_equal(got[used], want[used]), (path, int(np.sum(got[used] != want[used])))
    if ck:
        # (rows past the last checkpoint stay zero in both runs, and zero rounds to zero)
        wk, gk = _rounded(k32, seed, 1, rounds), k16.numpy().view(np.uint16)
        assert np.array_equal(gk, wk), (path, int(np.sum(gk != wk)))


@pytest.mark.parametrize("keep", [True, False])
def test_decode_fp16_stores_bit_exact(keep):
    ssd = _ssd()
    R, T, H, P, N, G, ns, seed, rounds = 6, 3, 8, 64, 128, 2, 13, 0xABCDEF0123, 5
    cfg = sy.DecodeConfig("sr_bits", R, T, H, P, N, G, BF16, F16, ns, 8, 840)
    d = sy.make_decode(cfg)
    g = torch.Generator().manual_seed(5)
    c16 = torch.zeros(ns, H, P, N, dtype=F16)
    for s in d.state_indices:
        c16[int(s)] = (torch.randn(H, P, N, generator=g) * 0.05).half()
    args = [t.to(DEV) for t in (d.x, d.dt, d.A, d.B, d.C, d.D)]

    def run(ts, sd):
        up = ssd.make_ssu_problem(R, T, H, P, N, G, ns, BF16, ts)
        opt = ssd.make_options(sr_seed=None if sd is None else _seed(sd), sr_rounds=rounds)
        cache = c16.to(ts).to(DEV)
        y = torch.empty(R, T, H, P, dtype=BF16, device=DEV)
        inter = torch.empty(R, T, H, P, N, dtype=ts, device=DEV) if keep else None
        ssd.selective_state_update_ex(up, opt, cache, d.state_indices.to(DEV), *args, y, inter)
        torch.cuda.synchronize()
        return cache.cpu(), None if inter is None else inter.cpu()

    a32, i32 = run(F32, None)
    a16, i16 = run(F16, seed)
    if keep:
        want, got = _rounded(i32, seed, 2, rounds), i16.numpy().view(np.uint16)
        assert np.array_equal(got, want), int(np.sum(got != want))
    else:
        used = d.state_indices.long().numpy()
        want, got = _rounded(a32, seed, 0, rounds), a16.numpy().view(np.uint16)
        assert np.array_equal(got[used], want[used]), int(np.sum(got[used] != want[used]))


def test_replay_fp16_store_bit_exact():
    """The ReplaySSM checkpoint store (stream 3): two verify steps that leave the
    checkpoint alone (the history stays below the ring's capacity), then a
    materialisation, once with float32 checkpoints and once with fp16 ones holding
    the same (fp16-exact) values; the fp16 bits are the oracle's rounding of the
    float32 result."""
    ssd = _ssd()
    R, T, H, P, N, G, W, ns, seed, rounds = 4, 2, 4, 64, 128, 2, 16, 9, 0x1234567, 5
    cfg = sy.DecodeConfig("sr_replay_bits", R, T, H, P, N, G, BF16, F16, ns, 8, 850)
    base = sy.make_decode(cfg)
    idx = base.state_indices
    g = torch.Generator().manual_seed(9)
    c16 = torch.zeros(ns, H, P, N, dtype=F16)
    for s in idx:
        c16[int(s)] = (torch.randn(H, P, N, generator=g) * 0.05).half()
    steps = []
    for k in range(2):
        d = sy.make_decode(sy.DecodeConfig("sr_replay_bits", R, T, H, P, N, G, BF16, F16, ns, 8,
                                           850 + 1000 * (k + 1)))
        steps.append((d.x, d.dt, d.B, d.C, d.num_accepted))

    def run(ts, sd):
        up = ssd.make_ssu_problem(R, T, H, P, N, G, ns, BF16, ts)
        opt = ssd.make_options(sr_seed=None if sd is None else _seed(sd), sr_rounds=rounds)
        rings = ssd.alloc_replay_rings(up, W, DEV)
        ck = c16.to(ts).to(DEV)
        for x, dt, B, C, acc in steps:
            y = torch.empty(R, T, H, P, dtype=BF16, device=DEV)
            ssd.ssd_replay_update_ex(up, opt, W, ck, rings["ring_x"], rings["ring_dt"],
                                     rings["ring_B"], rings["cursor"], idx.to(DEV), x.to(DEV),
                                     dt.to(DEV), base.A.to(DEV), B.to(DEV), C.to(DEV),
                                     base.D.to(DEV), y)
            ssd.ssd_replay_advance(up, W, rings["cursor"], idx.to(DEV), acc.to(DEV))
        assert int(rings["cursor"].cpu()[:, 1].max()) + T <= W - T   # (no rewrite so far)
        ssd.ssd_replay_materialize_ex(up, opt, W, ck, rings["ring_x"], rings["ring_dt"],
                                      rings["ring_B"], rings["cursor"], idx.to(DEV),
                                      base.A.to(DEV))
        torch.cuda.synchronize()
        return ck.cpu()

    k32 = run(F32, None)
    k16 = run(F16, seed)
    used = idx.long().numpy()
    want, got = _rounded(k32, seed, 3, rounds), k16.numpy().view(np.uint16)
    assert np.array_equal(got[used], want[used]), int(np.sum(got[used] != want[used]))
