"""ssd_combined_varlen_noalloc (the entry point that allocates nothing, for
callers that cannot allocate): the same results as ssd_combined_varlen with a
caller's workspace, bit for bit, on two calls in a row (the second smaller, so
the static scratch array holds the first call's leftovers), and the oracle's
results within the tolerances; a problem too large for the array is rejected."""
import ctypes

import pytest
import torch

import oracle
import ssd_synth as sy
from gpu_helpers import DEV, assert_close, looser

pytestmark = pytest.mark.gpu

BF16, F32 = torch.bfloat16, torch.float32


def _run(ssd, inp, cache, Q, noalloc, checkpoints):
    T, S = int(inp.cu_seqlens[-1]), len(inp.cu_seqlens) - 1
    H, P, N, G = inp.x.shape[1], inp.x.shape[2], inp.B.shape[2], inp.B.shape[1]
    p = ssd.make_problem(T, S, H, P, N, G, Q, cache.shape[0], inp.x.dtype, cache.dtype)
    g_cache = cache.to(DEV)
    y = torch.empty(T, H, P, dtype=inp.x.dtype, device=DEV)
    ck = torch.empty(ssd.max_chunks(p), H, P, N, dtype=cache.dtype, device=DEV) \
        if checkpoints else None
    args = (p, inp.x.to(DEV), inp.dt.to(DEV), inp.A.to(DEV), inp.B.to(DEV), inp.C.to(DEV),
            inp.D.to(DEV), inp.cu_seqlens.to(DEV), g_cache, inp.state_indices.to(DEV),
            None if inp.has_initial is None else inp.has_initial.to(DEV), y, ck)
    if noalloc:
        ssd.ssd_combined_varlen_noalloc(*args)
    else:
        ssd.ssd_combined_varlen(*args, ssd.alloc_workspace(p, DEV))
    torch.cuda.synchronize()
    return y.cpu(), g_cache.cpu(), None if ck is None else ck.cpu()


def _bits(t):
    return t.view(torch.int16) if t.dtype == BF16 else t.view(torch.int32)


CASES = [
    # the 4096-token, 80-head layer (segmented state pass), then a smaller mixed batch
    # with cached states and checkpoints
    ("c1", sy.C1, None, False),
    ("mixed", None, (600, 32, 1, 0, 257), True),
]


def test_noalloc_matches_workspace_entry_point_twice():
    import state_space_model_varlen_amd as ssd
    assert ssd.noalloc_scratch_bytes() == 128 << 20
    for name, cfg, lens, ck in CASES:
        if cfg is not None:
            inp, Q = sy.make_prefill(cfg), cfg.chunk_size
            cache = torch.full((1, cfg.nheads, cfg.headdim, cfg.d_state), float("nan"))
        else:
            Q = 256
            inp = sy.random_problem(31, lens, 8, 64, 128, 2, Q, BF16, F32, num_slots=12,
                                    has_initial=[True, False, True, True, False])
            g = torch.Generator().manual_seed(2)
            cache = torch.full((12, 8, 64, 128), float("nan"))
            for s in range(len(lens)):
                if int(inp.has_initial[s]):
                    cache[int(inp.state_indices[s])] = torch.randn(8, 64, 128, generator=g) * 0.05
        print(f"no-alloc case {name}: T={int(inp.cu_seqlens[-1])}", flush=True)
        y0, c0, k0 = _run(ssd, inp, cache, Q, False, ck)
        y1, c1, k1 = _run(ssd, inp, cache, Q, True, ck)
        assert torch.equal(_bits(y0), _bits(y1)), name
        assert torch.equal(_bits(c0), _bits(c1)), name      # NaN slots by their bits
        if ck:
            nc = int(oracle.chunk_counts(inp.cu_seqlens.numpy(), Q)[-1])
            assert torch.equal(_bits(k0[:nc]), _bits(k1[:nc])), name
        ref = oracle.prefill(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.cu_seqlens,
                             inp.state_indices, inp.has_initial, cache, Q, checkpoints=ck)
        assert_close(y1, ref["y"], BF16, f"{name} y", normalised=False)
        used = inp.state_indices.long()
        assert_close(c1[used], ref["final"], looser(BF16, cache.dtype), f"{name} final states")
        if ck:
            assert_close(k1[:nc], ref["ckpt"], BF16, f"{name} checkpoints")


def test_noalloc_rejects_problems_beyond_its_scratch():
    import state_space_model_varlen_amd as ssd
    # 64 heads x 16384 tokens x 64 sequences: far more workspace than 128 MiB
    p = ssd.make_problem(16384, 64, 64, 64, 128, 8, 256, 64, BF16, BF16)
    assert ssd.workspace_bytes(p) > ssd.noalloc_scratch_bytes()
    fake = ctypes.c_void_p(256)
    rc = ssd._lib.ssd_combined_varlen_noalloc(ctypes.byref(p), *([fake] * 12), None)
    assert rc == 8 and "scratch" in ssd.status_string(rc)
