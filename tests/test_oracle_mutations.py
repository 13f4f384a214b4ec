"""Negative controls: copies of the oracle with a planted mistake must fail a pin.

Each mutation edits one line of a copy of oracle/ssd_oracle.c (in a temporary
directory; the oracle itself is untouched), compiles it, and runs every pin.
A mutation that no pin catches would mean the pins cannot tell that mistake
from the correct recurrence.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

# (name, exact text in the oracle, replacement)
MUTATIONS = [
    ("input_term_dropped", "hp[n] = decay * hp[n] + u * Bt[n];", "hp[n] = decay * hp[n];"),
    ("decay_dropped", "hp[n] = decay * hp[n] + u * Bt[n];", "hp[n] = hp[n] + u * Bt[n];"),
    ("decay_applied_to_own_input", "hp[n] = decay * hp[n] + u * Bt[n];",
     "hp[n] = decay * (hp[n] + u * Bt[n]);"),
    ("decay_sign_flipped", "const double decay = exp(dtt * Ah);",
     "const double decay = exp(-dtt * Ah);"),
    ("skip_term_dropped", "yt[p] = acc + Dh * xt[p];", "yt[p] = acc;"),
    ("output_reads_B_not_C", "acc += Ct[n] * hp[n];", "acc += Bt[n] * hp[n];"),
    ("wrong_group_map", "g = hd / heads_per_group;", "g = hd % G;"),
    ("checkpoint_row_shifted", "const int64_t row = chunk_cu[s] + k / Q;",
     "const int64_t row = chunk_cu[s] + (k / Q == 0 ? 0 : k / Q - 1);"),
    ("initial_state_ignored", "if (use_init)\n                memcpy", "if (0)\n                memcpy"),
    ("dt_not_applied_to_input", "const double u = dtt * xt[p];", "const double u = xt[p];"),
]


def _build_mutant(tmp, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation {name}: text not found in the oracle"
    mutated = src.replace(old, new, 1)
    path_c = os.path.join(tmp, f"{name}.c")
    path_so = os.path.join(tmp, f"lib{name}.so")
    with open(path_c, "w") as f:
        f.write(mutated)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o",
                           path_so, path_c, "-lm"])
    return oracle.load_lib(path_so)


@pytest.mark.parametrize("mut", MUTATIONS, ids=lambda m: m[0])
def test_mutation_is_caught(mut):
    name, old, new = mut
    with tempfile.TemporaryDirectory() as tmp:
        lib = _build_mutant(tmp, name, old, new)
        caught = []
        for pin in oracle_pins.ALL_PINS:
            try:
                pin(lib=lib)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin.__name__)
        assert caught, f"no pin catches the planted mistake '{name}'"


# Planted mistakes in the chunked steps (oracle.chunked), swapped in with monkeypatch.
import numpy as np  # noqa: E402

from oracle import chunked  # noqa: E402


def _bad_chunk_state_sign(x, B, cum, dtp, meta):
    flipped = cum.copy()
    for c in range(len(meta["seq"])):
        ln = int(meta["len"][c])
        flipped[:, c, :ln] = 2 * cum[:, c, ln - 1][:, None] - cum[:, c, :ln]
    return _orig["chunk_state"](x, B, flipped, dtp, meta)


def _bad_state_passing_no_decay(states, cum, meta, init=None, has_init=None):
    return _orig["state_passing"](states, np.zeros_like(cum), meta, init, has_init)


def _bad_bmm_transposed(B, C, meta, Q):
    return np.swapaxes(_orig["bmm"](B, C, meta, Q), 2, 3)


def _bad_chunk_scan_no_inter(x, C, D, CB, cum, dtp, entering, meta):
    return _orig["chunk_scan"](x, C, D, CB, cum, dtp, np.zeros_like(entering), meta)


def _bad_cumsum_exclusive(dt, A, meta, Q):
    cum, dtp = _orig["chunk_cumsum"](dt, A, meta, Q)
    shifted = np.zeros_like(cum)
    shifted[:, :, 1:] = cum[:, :, :-1]
    return shifted, dtp


_orig = {k: getattr(chunked, k) for k in ("chunk_state", "state_passing", "bmm", "chunk_scan",
                                            "chunk_cumsum")}

CHUNKED_MUTATIONS = [("chunk_state", _bad_chunk_state_sign),
                     ("state_passing", _bad_state_passing_no_decay),
                     ("bmm", _bad_bmm_transposed),
                     ("chunk_scan", _bad_chunk_scan_no_inter),
                     ("chunk_cumsum", _bad_cumsum_exclusive)]


@pytest.mark.parametrize("mut", CHUNKED_MUTATIONS, ids=lambda m: m[1].__name__)
def test_chunked_mutation_is_caught(mut, monkeypatch):
    name, bad = mut
    monkeypatch.setattr(chunked, name, bad)
    with pytest.raises(AssertionError):
        oracle_pins.pin_chunk_size_independence()


# Planted mistakes in the ReplaySSM state machine (oracle/replay.py): each edits one
# line of a copy of the module, loaded under another name; the ReplaySSM pin must fail.
import importlib.util  # noqa: E402

REPLAY_SRC = os.path.join(os.path.dirname(oracle.__file__), "replay.py")
REPLAY_MUTATIONS = [
    ("target_token_not_kept", "layer.cursor[int(s)] = (start, n + 1 + int(a))",
     "layer.cursor[int(s)] = (start, n + int(a))"),
    ("window_overwrites_history", "pos = (start + n + t) % layer.W", "pos = (start + t) % layer.W"),
    ("last_history_token_skipped", "    for i in range(n):\n", "    for i in range(n - 1):\n"),
    ("checkpoint_one_step_late", "        if n + T > L:\n            layer.ckpt[s]",
     "        if n + T > L + 1:\n            layer.ckpt[s]"),
    ("cursor_not_moved_on_checkpoint", "layer.cursor[int(s)] = ((start + n) % layer.W, 1 + int(a))",
     "layer.cursor[int(s)] = (start, n + 1 + int(a))"),
]


@pytest.mark.parametrize("mut", REPLAY_MUTATIONS, ids=lambda m: m[0])
def test_replay_mutation_is_caught(mut, tmp_path):
    name, old, new = mut
    src = open(REPLAY_SRC).read()
    assert src.count(old) == 1, f"mutation {name}: text not found once in oracle/replay.py"
    src = src.replace(old, new).replace("from . import f64, round_to", "from oracle import f64, round_to")
    path = tmp_path / f"replay_{name}.py"
    path.write_text(src)
    spec = importlib.util.spec_from_file_location(f"replay_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with pytest.raises((AssertionError, IndexError)):
        oracle_pins.pin_replay_matches_recurrence(replay=mod)


# Planted mistakes in the step-size preprocessing, passed to its pin directly.
def _dtp_no_bias(dt_raw, dt_bias, lo, hi):
    return oracle.dt_preprocess(dt_raw, None, lo, hi)


def _dtp_exp_not_softplus(dt_raw, dt_bias, lo, hi):
    v = oracle.f64(dt_raw) + (0.0 if dt_bias is None else oracle.f64(dt_bias))
    return np.clip(np.exp(np.minimum(v, 20.0)), lo, hi)


def _dtp_clamp_before_softplus(dt_raw, dt_bias, lo, hi):
    v = oracle.f64(dt_raw) + (0.0 if dt_bias is None else oracle.f64(dt_bias))
    return np.log1p(np.exp(np.clip(v, lo, hi)))


@pytest.mark.parametrize("bad", [_dtp_no_bias, _dtp_exp_not_softplus, _dtp_clamp_before_softplus],
                         ids=lambda f: f.__name__)
def test_dt_preprocess_mutation_is_caught(bad):
    with pytest.raises(AssertionError):
        oracle_pins.pin_dt_preprocess(dtp=bad)


# Planted mistakes in the align-mode chunk cuts, swapped in with monkeypatch.
def _cuts_first_is_remainder(L, Q, prefix_len):
    o = prefix_len % Q if prefix_len > 0 else 0
    first = o if o else Q
    out, pos = [], 0
    while pos < L:
        ln = min(first if pos == 0 else Q, L - pos)
        out.append((pos, ln))
        pos += ln
    return out


def _cuts_ignore_prefix(L, Q, prefix_len):
    return [(pos, min(Q, L - pos)) for pos in range(0, L, Q)]


@pytest.mark.parametrize("bad", [_cuts_first_is_remainder, _cuts_ignore_prefix],
                         ids=lambda f: f.__name__)
def test_aligned_cut_mutation_is_caught(bad, monkeypatch):
    monkeypatch.setattr(oracle, "aligned_chunks", bad)
    with pytest.raises(AssertionError):
        oracle_pins.pin_aligned_checkpoints()


# Planted mistakes in the generator and the rounding (copies of oracle/rounding.py).
ROUNDING_SRC = os.path.join(os.path.dirname(oracle.__file__), "rounding.py")
ROUNDING_MUTATIONS = [
    ("wrong_multiplier", "M0, M1 = 0xD2511F53, 0xCD9E8D57", "M0, M1 = 0xD2511F55, 0xCD9E8D57"),
    ("key_not_bumped", "            k0 = (k0 + W0) & MASK\n", "            k0 = k0\n"),
    ("words_swapped", "c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]",
     "c = [hi0 ^ c[1] ^ k0, lo1, hi1 ^ c[3] ^ k1, lo0]"),
    ("rounds_up_at_equality", "out = np.where(u < prob, hi, lo)", "out = np.where(u <= prob, hi, lo)"),
    ("rounds_toward_the_nearer", "out = np.where(u < prob, hi, lo)",
     "out = np.where(u < 1 - prob, hi, lo)"),
    ("stream_ignored", "np.full_like(blk, kind)", "np.zeros_like(blk)"),
    ("halves_swapped", "(word >> (np.uint32(16) * half))", "(word >> (np.uint32(16) * (1 - half)))"),
    ("four_per_call", "blk = e // np.uint64(8)", "blk = e // np.uint64(4)"),
]


@pytest.mark.parametrize("mut", ROUNDING_MUTATIONS, ids=lambda m: m[0])
def test_rounding_mutation_is_caught(mut, tmp_path):
    name, old, new = mut
    src = open(ROUNDING_SRC).read()
    assert src.count(old) == 1, f"mutation {name}: text not found once in oracle/rounding.py"
    path = tmp_path / f"rounding_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"rounding_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    caught = False
    for pin in (oracle_pins.pin_philox_known_answers, oracle_pins.pin_stochastic_rounding):
        try:
            pin(rnd=mod)
        except AssertionError:
            caught = True
    assert caught, f"no pin catches the planted mistake '{name}'"
