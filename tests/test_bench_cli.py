"""Host-side checks of bench.py: the one-GPU contract and the algorithmic bytes
the roofline divides by (no GPU work)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_launch_bytes_and_flops_of_the_layer_prefill():
    """4096 tokens, 80 heads, headdim 64, d_state 128, one group, chunk 256, bf16
    inputs, float32 state, no cached state: 16 chunks, the state pass cut into 3
    segments. Each figure is the sum of the tensors the launch must read or write
    once, counted by hand here."""
    import ssd_synth as sy
    T, S, H, P, N, G, Q, nc = 4096, 1, 80, 64, 128, 1, 256, 16
    assert bench.segments(sy.C1) == 3
    w = bench.layer_work(sy.C1, 3)
    assert (w.T, w.S, w.nc, w.ex, w.es, w.s_init) == (T, S, nc, 2, 4, 0)
    x = T * H * P * 2                      # x (and y): 41.9 MB each
    bc = T * G * N * 2                     # B or C
    per_chunk = 2 * H * nc * Q * 4         # cumsum and dt, float32
    entering = nc * H * P * N * 2          # entering states, bf16
    final = S * H * P * N * 4              # the final state, float32
    cb = nc * G * (16 * 17 // 2) * 256 * 2   # causal 16 x 16 tiles of CB, bf16
    fins = 3 * H * P * N * 4                 # segment final states, float32
    assert bench.launch_bytes("chunk_cumsum", w) == T * H * 2 + per_chunk
    assert bench.launch_bytes("chunk_scan", w) == 2 * x + bc + per_chunk + cb + entering
    assert round(bench.launch_bytes("chunk_scan", w) / 1e6, 1) == 109.6
    # the scope document's per-kernel table counts entering states in float32: 130.5 MB
    # there (CB's causal half element by element), 130.6 MB here (whole 16 x 16 tiles)
    assert round(bench.launch_bytes("chunk_scan", w, entering_bytes=4) / 1e6, 1) == 130.6
    assert bench.launch_bytes("chunk_scan_segmented", w) == \
        2 * x + bc + per_chunk + cb + entering + 2 * H * P * N * 2
    assert bench.launch_bytes("chunk_state_passing_segmented", w) == \
        x + bc + per_chunk + entering + fins
    assert bench.launch_bytes("state_carry", w) == fins + 3 * H * P * N * 2 + final
    # the state launch doing the cumsum and CB itself: dt and C read, cumsum and dt
    # rows and CB written
    assert bench.launch_bytes("chunk_state_passing_segmented_prep", w) == \
        x + 2 * bc + T * H * 2 + per_chunk + entering + fins + cb
    # flops: causal intra-chunk 80 * 64 * 256 * 257 per chunk plus the state term
    # 2 * 80 * 64 * 128 * 256 per chunk: 10.76 GFLOP
    assert bench.launch_flops("chunk_scan_segmented", w) == \
        16 * (H * P * 256 * 257 + 2 * H * P * N * 256)
    assert round(bench.launch_flops("chunk_scan", w) / 1e9, 2) == 10.76
    assert bench.launch_flops("chunk_state_passing_segmented", w) == 16 * 2 * H * P * N * 256


def test_kernel_names_map_to_launches():
    n = lambda k: bench.launch_name(k)[0]
    assert n("_ZN3ssd22chunk_scan_fast_kernelILi256ELb1ELb1EEEviii") == "chunk_scan_segmented"
    assert n("_ZN3ssd22chunk_scan_fast_kernelILi256ELb0ELb1EEEviii") == "chunk_scan"
    assert n("_ZN3ssd22chunk_scan_fast_kernelILi128ELb0ELb0EEEviii") == "chunk_scan"
    assert n("void ssd::chunk_scan_fast_kernel<256, true, false>(int") == "chunk_scan_segmented"
    assert n("void ssd::chunk_scan_fast_kernel<256, false, true>(int") == "chunk_scan"
    assert n("_ZN3ssd22state_scan_fast_kernelILi256ELb0ELb1ELb0EfEEvii") == \
        "chunk_state_passing_segmented"
    assert n("_ZN3ssd22state_scan_fast_kernelILi256ELb1ELb0ELb0EfEEvii") == "chunk_state_passing"
    assert n("_ZN3ssd22state_scan_fast_kernelILi256ELb0ELb1ELb1EfEEvii") == \
        "chunk_state_passing_segmented_prep"
    assert n("_ZN3ssd22state_scan_fast_kernelILi256ELb1ELb0ELb1EfEEvii") == \
        "chunk_state_passing_prep_bmm"
    assert n("void ssd::state_scan_fast_kernel<256, true, false, true, float>(int") == \
        "chunk_state_passing_prep_bmm"
    assert n("void ssd::state_scan_fast_kernel<128, false, true, false, bf16>(int") == \
        "chunk_state_passing_segmented"
    assert n("void ssd::state_carry_kernel<float>(int, int") == "state_carry"
    assert n("_ZN3ssd19chunk_cumsum_kernelIDF16bEEvii") == "chunk_cumsum"
    assert n("_ZN3ssd15bmm_pair_kernelILi256EEEvii") == "bmm_chunk_pairs"
    assert n("void ssd::short_scan_kernel<32, float>(int, int") == "short_scan"
    assert n("at::native::vectorized_elementwise_kernel") is None
