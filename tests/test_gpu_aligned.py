"""GPU parity of the align-mode prefill (chunk boundaries at absolute multiples
of the chunk size after each sequence's cached prefix) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import ssd_synth as sy
from gpu_helpers import DEV, assert_close, looser, select_heads, workload_cache

pytestmark = pytest.mark.gpu

F32, BF16 = torch.float32, torch.bfloat16


def _ssd():
    import state_space_model_varlen_amd as ssd
    return ssd


def _gpu_aligned(inp, cache, Q, prefix):
    ssd = _ssd()
    T, S = int(inp.cu_seqlens[-1]), len(inp.cu_seqlens) - 1
    H, P, N, G = inp.x.shape[1], inp.x.shape[2], inp.B.shape[2], inp.B.shape[1]
    p = ssd.make_problem(T, S, H, P, N, G, Q, cache.shape[0], inp.x.dtype, cache.dtype)
    g_cache = cache.to(DEV)
    y = torch.empty(T, H, P, dtype=inp.x.dtype, device=DEV)
    ck = torch.full((ssd.max_chunks_aligned(p), H, P, N), float("nan"), dtype=cache.dtype,
                    device=DEV)
    ssd.ssd_combined_varlen_aligned(p, torch.tensor(prefix, dtype=torch.int32, device=DEV),
                                    inp.x.to(DEV), inp.dt.to(DEV), inp.A.to(DEV), inp.B.to(DEV),
                                    inp.C.to(DEV), inp.D.to(DEV), inp.cu_seqlens.to(DEV), g_cache,
                                    inp.state_indices.to(DEV),
                                    None if inp.has_initial is None else inp.has_initial.to(DEV),
                                    y, ck, ssd.alloc_workspace_aligned(p, DEV))
    torch.cuda.synchronize()
    return y.cpu(), g_cache.cpu(), ck.cpu()


CASES = [
    # lens, cached prefix lengths, H, P, N, G, Q, in, state
    ((10, 300, 0, 129, 64), (6, 100, 3, 0, 64), 4, 16, 16, 2, 64, F32, F32),
    ((600, 32, 1, 257), (4224, 0, 255, 1), 8, 64, 128, 2, 256, BF16, F32),
    ((33, 200, 500), (100, 128, 7), 8, 64, 128, 8, 128, BF16, BF16),
    ((70, 5), (-3, 2 ** 30), 4, 64, 16, 4, 32, F32, BF16),
    # 64 mostly short sequences x 8 heads: the multi-item state pass in align mode
    ((3, 70, 0, 9, 130, 1, 22, 31) * 8, (5, 100, 0, 127, 1, 64, 300, 2) * 8, 8, 64, 128, 2, 128,
     BF16, BF16),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"S{len(c[0])}_P{c[3]}N{c[4]}Q{c[6]}_"
                         f"{str(c[7])[6:]}_{str(c[8])[6:]}")
def test_aligned_prefill_matches_oracle(case):
    lens, prefix, H, P, N, G, Q, ti, ts = case
    S = len(lens)
    slots = 2 * S + 1
    inp = sy.random_problem(700 + CASES.index(case), lens, H, P, N, G, Q, ti, ts,
                            num_slots=slots, has_initial=[s % 2 == 0 for s in range(S)])
    cache = sy.nan_cache(slots, H, P, N, ts)
    g = torch.Generator().manual_seed(7)
    for s in range(S):
        if int(inp.has_initial[s]):
            cache[int(inp.state_indices[s])] = (torch.randn(H, P, N, generator=g) * 0.05).to(ts)
    y, after, ck = _gpu_aligned(inp, cache, Q, prefix)
    ref = oracle.prefill_aligned(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                                 inp.state_indices, inp.has_initial, cache, Q,
                                 [max(v, 0) for v in prefix])
    assert_close(y, ref["y"], ti, "y", normalised=False)
    used = inp.state_indices.long()
    assert_close(after[used], ref["final"], looser(ti, ts), "final states")
    nc = len(ref["ckpt"])
    assert_close(ck[:nc], ref["ckpt"], looser(ti, ts), "aligned checkpoints")
    assert torch.isnan(ck[nc:].float()).all()        # rows past the chunks stay unwritten


def test_c3_mixed_varlen_aligned_full():
    """The 8-sequence mixed batch with checkpoints in align mode: odd sequences
    continue after 4224 cached tokens (first chunk 128 tokens) from the oracle's
    state after their own seeded prefix, even ones start fresh. The oracle checks
    every (sequence, head), one B/C group (8 heads) at a time to bound the host
    memory of its per-token states."""
    cfg = sy.C3
    inp = sy.make_prefill(cfg)
    H, G, Q = cfg.nheads, cfg.ngroups, cfg.chunk_size
    cache = workload_cache(inp)
    prefix = [cfg.prefix_len if int(inp.has_initial[s]) else 0 for s in range(cfg.num_seqs)]
    y, after, ck = _gpu_aligned(inp, cache, Q, prefix)
    used = inp.state_indices.long()
    hpg = H // G
    for g in range(G):
        heads = list(range(g * hpg, (g + 1) * hpg))
        x, dt, A, B, C, D = select_heads(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, heads, G)
        ref = oracle.prefill_aligned(x, dt, A, B, C, D, inp.cu_seqlens, inp.state_indices,
                                     inp.has_initial, cache[:, heads], Q, prefix)
        assert_close(y[:, heads], ref["y"], BF16, f"c3 aligned y, group {g}", normalised=False)
        assert_close(after[used][:, heads], ref["final"], BF16,
                     f"c3 aligned final states, group {g}")
        nc = len(ref["ckpt"])
        # chunks: 1, 7 for the fresh 32- and 1600-token sequences; after 4224 cached
        # tokens the 600-token ones cut as 128 + 256 + 216 and the 128-token ones as
        # one chunk
        assert nc == 24
        assert_close(ck[:nc][:, heads], ref["ckpt"], BF16, f"c3 aligned checkpoints, group {g}")
    assert torch.isnan(ck[24:].float()).all()
