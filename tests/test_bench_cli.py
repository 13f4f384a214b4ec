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


def test_prefill_bytes_of_the_layer_prefill():
    """4096 tokens, 80 heads, headdim 64, d_state 128, one group, chunk 256, bf16
    inputs: 16 chunks. Each figure is the sum of the tensors the kernel must read
    or write once, counted by hand here."""
    T, S, H, P, N, G, Q, nc = 4096, 1, 80, 64, 128, 1, 256, 16
    b = bench.prefill_bytes(T, S, H, P, N, G, Q, nc, 2, 4, 0, False)
    x = T * H * P * 2                      # x (and y): 41.9 MB each
    bc = T * G * N * 2                     # B or C
    per_chunk = 2 * H * nc * Q * 4         # cumsum and dt, float32
    entering = nc * H * P * N * 2          # entering states, bf16
    final = S * H * P * N * 4              # the final state, float32
    cb = nc * G * (16 * 17 // 2) * 256 * 2   # causal 16 x 16 tiles of CB, bf16
    assert b["chunk_cumsum"] == T * H * 2 + per_chunk
    assert b["chunk_state_passing"] == x + bc + per_chunk + entering + final
    assert b["chunk_scan"] == 2 * x + bc + per_chunk + cb + entering
    assert round(b["chunk_scan"] / 1e6, 1) == 109.6
    assert round(b["chunk_state_passing"] / 1e6, 1) == 69.2
