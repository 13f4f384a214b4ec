"""The seeded input generator: determinism, shapes, dtypes and value ranges."""
import numpy as np
import torch

import ssd_synth as sy


def test_prefill_shapes_and_determinism():
    a = sy.make_prefill(sy.C3)
    b = sy.make_prefill(sy.C3)
    cfg = sy.C3
    T = cfg.total_tokens
    assert T == 4720
    assert a.x.shape == (T, 64, 64) and a.x.dtype == torch.bfloat16
    assert a.dt.shape == (T, 64) and a.B.shape == (T, 8, 128) and a.C.shape == (T, 8, 128)
    assert torch.equal(a.x, b.x) and torch.equal(a.dt, b.dt) and torch.equal(a.B, b.B)
    assert a.cu_seqlens.tolist() == [0, 32, 632, 2232, 2360, 2392, 2992, 4592, 4720]
    assert a.has_initial.tolist() == [0, 1, 0, 1, 0, 1, 0, 1]
    assert len(set(a.state_indices.tolist())) == 8
    assert all(0 <= i < 256 for i in a.state_indices.tolist())
    assert a.prefix_tokens(0) is None and a.prefix_tokens(1)[0].shape == (4224, 64, 64)
    assert torch.equal(a.prefix_tokens(1)[2], b.prefix_tokens(1)[2])


def test_value_ranges():
    a = sy.make_prefill(sy.C0)
    dt = a.dt.double()
    assert float(dt.min()) >= 1e-3 * (1 - 1e-6) and float(dt.max()) <= 0.1 * (1 + 1e-6)
    assert float(a.A.max()) <= -1.0 and float(a.A.min()) >= -16.0
    assert a.x.dtype == torch.float32


def test_decode_inputs():
    d = sy.make_decode(sy.C4, num_reqs=4)
    assert d.x.shape == (4, 3, 128, 64) and d.B.shape == (4, 3, 8, 128)
    assert d.num_accepted.min() >= 0 and d.num_accepted.max() <= 2
    full_idx = sy.make_decode(sy.C4, num_reqs=4).state_indices
    assert torch.equal(d.state_indices, full_idx)


def test_small_variant_uses_same_streams():
    a = sy.make_prefill(sy.C1, seqlens=[64])
    b = sy.make_prefill(sy.C1, seqlens=[128])
    # same layer parameters, and token draws are a prefix of the longer draw only per stream order
    assert torch.equal(a.A, b.A) and torch.equal(a.D, b.D)
    assert np.isfinite(a.x.float().numpy()).all()
