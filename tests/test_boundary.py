"""The C-ABI library loads, exports every function include/ssd_mi355x.h declares,
and rejects bad arguments on the host before anything reaches the GPU."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd_mi355x.h")

ssd = pytest.importorskip("state_space_model_varlen_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_functions_are_exported():
    names = declared_functions()
    assert len(names) >= 13, names
    lib = ctypes.CDLL(ssd.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert set(names) == set(ssd.EXPORTED)


def test_version_and_status_strings():
    assert ssd.abi_version() == 3
    for s in range(9):
        assert ssd.status_string(s) != "unknown status"
    assert ssd.status_string(99) == "unknown status"


def P(**kw):
    base = dict(total_tokens=256, num_seqs=1, nheads=4, headdim=16, d_state=16, ngroups=1,
                chunk_size=64, num_slots=1, in_dtype=torch.float32, state_dtype=torch.float32)
    base.update(kw)
    return ssd.make_problem(**base)


def test_sizes():
    p = P()
    assert ssd.max_chunks(p) == 256 // 64 + 1
    # chunk_cu, chunk triples, clamped cu, first-chunk lengths
    assert ssd.chunk_meta_count(p) == 2 + 3 * 5 + 2 + 1
    ws = ssd.workspace_bytes(p)
    # meta, cumsum, dt, CB and chunk states, each rounded up to 256 bytes
    r = lambda v: (v + 255) // 256 * 256
    want = (r(4 * 20) + 2 * r(4 * 4 * 5 * 64) + r(4 * 5 * 1 * 64 * 64) + r(4 * 5 * 4 * 16 * 16)
            + r(4 * 5 * 4 * 16 * 16))   # fp32 inputs: CB and entering states in fp32
    assert ws == want
    big = P(total_tokens=4096, nheads=80, headdim=64, d_state=128, chunk_size=256,
            in_dtype=torch.bfloat16)
    assert ssd.max_chunks(big) == 17
    # bf16 inputs, headdim 64, d_state 128: the fused state kernel needs no chunk states
    mc, H, Q = 17, 80, 256
    # one sequence over 80 heads x 2 column slices: 160 state blocks, so the chunk
    # chain is cut into 512 // 160 = 3 segments with their own buffers (final
    # states fp32, starting states bf16, decays, per-chunk decay and segment index)
    ns = 3
    want_big = (r(4 * (5 + 3 * mc)) + 2 * r(4 * H * mc * Q) + r(2 * mc * 1 * Q * Q)
                + r(2 * mc * H * 64 * 128)
                + r(4 * ns * H * 64 * 128) + r(2 * ns * H * 64 * 128) + r(4 * ns * H)
                + r(4 * mc * H) + r(4 * mc))
    assert ssd.workspace_bytes(big) == want_big
    # 32 sequences x 64 heads fill the chip: no segments
    many = P(total_tokens=1024, num_seqs=32, nheads=64, headdim=64, d_state=128,
             chunk_size=256, ngroups=8, in_dtype=torch.bfloat16)
    mc = 1024 // 256 + 32
    assert ssd.workspace_bytes(many) == (r(4 * (3 * 32 + 2 + 3 * mc)) + 2 * r(4 * 64 * mc * 256)
                                         + r(2 * mc * 8 * 256 * 256) + r(2 * mc * 64 * 64 * 128))


@pytest.mark.parametrize("kw,status", [
    (dict(nheads=0), 2), (dict(total_tokens=-1), 2), (dict(nheads=6, ngroups=4), 2),
    (dict(num_slots=0), 2), (dict(headdim=32), 4), (dict(d_state=64), 4),
    (dict(chunk_size=48), 4), (dict(chunk_size=512), 4),
])
def test_invalid_problems_rejected(kw, status):
    p = P(**kw)
    assert ssd.workspace_bytes(p) == 0
    assert ssd.max_chunks(p) == 0
    lib = ssd._lib
    fake = ctypes.c_void_p(256)
    rc = lib.ssd_combined_varlen(ctypes.byref(p), *([fake] * 13), ctypes.c_size_t(1 << 30), None)
    assert rc == status


def test_align_mode_chunk_bound_checked_before_launch():
    """Align mode bounds the chunks by T / Q + 2 S, which sizes its grids: a batch
    within the plain bound (T / Q + S <= 65535) but past the align-mode one is
    rejected before anything is enqueued."""
    p = P(total_tokens=64 * 40000, num_seqs=20000, num_slots=20000)
    assert ssd.max_chunks(p) == 40000 + 20000
    assert ssd.max_chunks_aligned(p) == 0 and ssd.workspace_bytes_aligned(p) == 0
    fake = ctypes.c_void_p(256)
    rc = ssd._lib.ssd_combined_varlen_aligned(ctypes.byref(p), *([fake] * 14),
                                              ctypes.c_size_t(1 << 40), None)
    assert rc == 4


def test_noalloc_rejects_problems_beyond_its_scratch_on_the_host():
    """The no-alloc entry point checks the problem's workspace against its static
    array before looking anything up on a device or enqueueing."""
    p = P(total_tokens=16384, num_seqs=64, nheads=64, headdim=64, d_state=128, ngroups=8,
          chunk_size=256, num_slots=64, in_dtype=torch.bfloat16, state_dtype=torch.bfloat16)
    assert ssd.workspace_bytes(p) > ssd.noalloc_scratch_bytes() == 128 << 20
    fake = ctypes.c_void_p(256)
    assert ssd._lib.ssd_combined_varlen_noalloc(ctypes.byref(p), *([fake] * 12), None) == 8
    # an invalid problem gets the status of ssd_combined_varlen
    assert ssd._lib.ssd_combined_varlen_noalloc(ctypes.byref(P(nheads=0)), *([fake] * 12),
                                                None) == 2


def test_bad_dtype_code():
    p = P()
    p.in_dtype = 7
    rc = ssd._lib.ssd_chunk_cumsum(ctypes.byref(p), *([ctypes.c_void_p(256)] * 6), None)
    assert rc == 3


def test_null_and_alignment_and_workspace():
    p = P()
    lib = ssd._lib
    ok = ctypes.c_void_p(256)
    args = [ok] * 13
    # NULL x
    a = list(args)
    a[0] = None
    assert lib.ssd_combined_varlen(ctypes.byref(p), *a, ctypes.c_size_t(1 << 30), None) == 1
    # misaligned x
    a = list(args)
    a[0] = ctypes.c_void_p(258)
    assert lib.ssd_combined_varlen(ctypes.byref(p), *a, ctypes.c_size_t(1 << 30), None) == 7
    # workspace not 256-byte aligned
    a = list(args)
    a[12] = ctypes.c_void_p(272)
    assert lib.ssd_combined_varlen(ctypes.byref(p), *a, ctypes.c_size_t(1 << 30), None) == 7
    # workspace too small
    assert lib.ssd_combined_varlen(ctypes.byref(p), *args,
                                   ctypes.c_size_t(ssd.workspace_bytes(p) - 1), None) == 5
    # the step entry points check their pointers too
    assert lib.ssd_chunk_scan(ctypes.byref(p), *([ok] * 6), None, ok, ok, None) == 1
    assert lib.ssd_state_passing(ctypes.byref(p), ok, ok, ok, None, ok, None, ok, None, None) == 1


def test_fused_state_entry_point_shapes():
    """ssd_chunk_state_passing serves bf16 inputs with headdim 64, d_state 128 only."""
    lib = ssd._lib
    ok = ctypes.c_void_p(256)
    args = [ok] * 7 + [None, ok, None, None]
    assert lib.ssd_chunk_state_passing(ctypes.byref(P()), *args) == 4
    assert lib.ssd_chunk_state_passing(ctypes.byref(P(in_dtype=torch.bfloat16)), *args) == 4
    fast = P(headdim=64, d_state=128, in_dtype=torch.bfloat16)
    a = list(args)
    a[0] = None
    assert lib.ssd_chunk_state_passing(ctypes.byref(fast), *a) == 1
    a = list(args)
    a[8] = ctypes.c_void_p(264)
    assert lib.ssd_chunk_state_passing(ctypes.byref(fast), *a) == 7


def test_decode_validation():
    lib = ssd._lib
    ok = ctypes.c_void_p(256)
    up = ssd.make_ssu_problem(2, 3, 8, 64, 128, 2, 4, torch.bfloat16, torch.bfloat16)
    assert lib.selective_state_update(ctypes.byref(up), ok, ok, ok, ok, ok, ok, None, None, ok,
                                      None, None) == 1
    bad = ssd.make_ssu_problem(2, 3, 8, 64, 128, 3, 4, torch.bfloat16, torch.bfloat16)
    assert lib.selective_state_update(ctypes.byref(bad), *([ok] * 10), None, None) == 2
    un = ssd.make_ssu_problem(2, 3, 8, 32, 128, 2, 4, torch.bfloat16, torch.bfloat16)
    assert lib.ssd_state_commit(ctypes.byref(un), ok, ok, ok, ok, None) == 4
    assert lib.ssd_state_commit(ctypes.byref(up), ok, ok, ctypes.c_void_p(264), ok, None) == 7


def test_binding_checks_shapes_before_the_library():
    p = P()
    x = torch.empty(10, 4, 16)   # CPU tensor: rejected by the binding
    with pytest.raises(ValueError):
        ssd.ssd_chunk_state(p, x, x, x, x, x, x)


def test_replay_validation():
    """ReplaySSM entry points: ring length at least two windows, NULL and alignment
    checks on the host (nothing is launched in these cases)."""
    lib = ssd._lib
    ok = ctypes.c_void_p(256)
    up = ssd.make_ssu_problem(2, 3, 8, 64, 128, 2, 4, torch.bfloat16, torch.bfloat16)
    args = [ok] * 11 + [None, ok, None]  # ckpt .. C, D = NULL, y, stream
    assert lib.ssd_replay_update(ctypes.byref(up), 5, *args) == 2   # W < 2 T
    assert lib.ssd_replay_update(ctypes.byref(up), 0, *args) == 2
    a = list(args)
    a[0] = None                                                     # ckpt
    assert lib.ssd_replay_update(ctypes.byref(up), 6, *a) == 1
    a = list(args)
    a[3] = None                                                     # ring_B
    assert lib.ssd_replay_update(ctypes.byref(up), 6, *a) == 1
    a = list(args)
    a[1] = ctypes.c_void_p(264)                                     # ring_x misaligned
    assert lib.ssd_replay_update(ctypes.byref(up), 6, *a) == 7
    assert lib.ssd_replay_advance(ctypes.byref(up), 5, ok, ok, ok, None) == 2
    assert lib.ssd_replay_advance(ctypes.byref(up), 6, ok, ok, None, None) == 1
    assert lib.ssd_replay_materialize(ctypes.byref(up), 6, ok, ok, ok, ok, ok, ok, None,
                                      None) == 1
    assert lib.ssd_replay_materialize(ctypes.byref(up), 6, ctypes.c_void_p(8), ok, ok, ok, ok,
                                      ok, ok, None) == 7
    un = ssd.make_ssu_problem(2, 3, 8, 32, 128, 2, 4, torch.bfloat16, torch.bfloat16)
    assert lib.ssd_replay_advance(ctypes.byref(un), 6, ok, ok, ok, None) == 4


def test_dt_transform_and_varlen_validation():
    """NULL transform, inverted clamp, bad token counts and NULL arrays are refused
    on the host."""
    lib = ssd._lib
    ok = ctypes.c_void_p(256)
    p = P()
    good = ssd.ssd_dt_transform(None, 1e-3, 0.1)
    bad = ssd.ssd_dt_transform(None, 0.5, 0.1)
    assert lib.ssd_chunk_cumsum_dt(ctypes.byref(p), None, *([ok] * 6), None) == 1
    assert lib.ssd_chunk_cumsum_dt(ctypes.byref(p), ctypes.byref(bad), *([ok] * 6), None) == 2
    assert lib.ssd_chunk_cumsum_dt(ctypes.byref(p), ctypes.byref(good), None, *([ok] * 5),
                                   None) == 1
    assert lib.ssd_combined_varlen_dt(ctypes.byref(p), None, *([ok] * 13),
                                      ctypes.c_size_t(1 << 30), None) == 1
    up = ssd.make_ssu_problem(2, 3, 8, 64, 128, 2, 4, torch.bfloat16, torch.bfloat16)
    args = [ok] * 7 + [None, ok, None]     # cache .. C, D = NULL, y, inter = NULL
    f = lib.selective_state_update_varlen
    assert f(ctypes.byref(up), -1, ok, None, *args, None) == 2
    assert f(ctypes.byref(up), 6, None, None, *args, None) == 1
    assert f(ctypes.byref(up), 6, ok, ctypes.byref(bad), *args, None) == 2
    zero = ssd.make_ssu_problem(2, 0, 8, 64, 128, 2, 4, torch.bfloat16, torch.bfloat16)
    assert f(ctypes.byref(zero), 6, ok, None, *args, None) == 2
    g = lib.ssd_state_commit_varlen
    assert g(ctypes.byref(up), 6, None, ok, ok, ok, ok, None) == 1
    assert g(ctypes.byref(up), 6, ok, ok, ok, ctypes.c_void_p(264), ok, None) == 7


def test_fp16_state_and_options_validation():
    """fp16 is a state dtype only; stochastic rounding needs an fp16 state and 1..16
    Philox rounds; NULL arrays are refused (nothing is launched in these cases)."""
    lib = ssd._lib
    ok = ctypes.c_void_p(256)
    seed = ctypes.c_void_p(512)
    p16 = P(state_dtype=torch.float16)
    assert ssd.workspace_bytes(p16) > 0
    bad_in = P()
    bad_in.in_dtype = 2
    assert ssd.workspace_bytes(bad_in) == 0
    opt = ssd.ssd_options(None, None, seed.value, 10)
    pf32 = P()
    assert lib.ssd_combined_varlen_ex(ctypes.byref(pf32), ctypes.byref(opt), *([ok] * 13),
                                      ctypes.c_size_t(1 << 30), None) == 4
    opt0 = ssd.ssd_options(None, None, seed.value, 0)
    assert lib.ssd_combined_varlen_ex(ctypes.byref(p16), ctypes.byref(opt0), *([ok] * 13),
                                      ctypes.c_size_t(1 << 30), None) == 2
    a = [ok] * 13
    a[0] = None
    assert lib.ssd_combined_varlen_ex(ctypes.byref(p16), ctypes.byref(opt), *a,
                                      ctypes.c_size_t(1 << 30), None) == 1
    up = ssd.make_ssu_problem(2, 3, 8, 64, 128, 2, 4, torch.bfloat16, torch.float16)
    args = [ok] * 7 + [None, None, None]     # cache .. C, D, y = NULL, inter
    assert lib.selective_state_update_ex(ctypes.byref(up), ctypes.byref(opt), 6, None, *args,
                                         None) == 1
    assert lib.ssd_round_f16(None, ok, 8, None, 10, 0, None) == 1
    assert lib.ssd_round_f16(ok, ok, -1, None, 10, 0, None) == 2
    assert lib.ssd_round_f16(ok, ok, 8, seed, 17, 0, None) == 2
    assert lib.ssd_round_f16(ok, ok, 0, None, 10, 0, None) == 0     # nothing to do
    ub = ssd.make_ssu_problem(2, 3, 8, 64, 128, 2, 4, torch.bfloat16, torch.bfloat16)
    assert lib.ssd_replay_update_ex(ctypes.byref(ub), ctypes.byref(opt), 6,
                                    *([ok] * 11), None, ok, None) == 4
