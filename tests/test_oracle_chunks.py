"""Pins for the oracle's chunk-descriptor builder (CPU only).

Rule (page "perf(gdn): dispatch exact causal-conv chunks", section "What
changed"): one program per exact (sequence, 8-token chunk) pair, sequences in
order.  The pins below use an independent formulation -- map every packed
token to the chunk that holds it and keep the distinct pairs in order -- so
a ceil/floor slip or a reordering in the oracle fails them.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth


def chunks_by_token(qsl):
    """Distinct (seq, (t - start) // 8) over all tokens, in token order."""
    out = []
    for s in range(len(qsl) - 1):
        for t in range(qsl[s], qsl[s + 1]):
            pair = (s, (t - qsl[s]) // 8)
            if not out or out[-1] != pair:
                out.append(pair)
    return out


def test_tiny_lengths_5_and_13():
    # lengths 5 and 13: one chunk for sequence 0, chunks 0 and 1 (8 + 5) for 1
    got = oracle.build_conv_chunks([0, 5, 18])
    assert [tuple(p) for p in got] == [(0, 0), (1, 0), (1, 1)]


def test_step_budget_two_sequences_gives_256():
    # 2 x 1024 tokens -> 2 x 128 chunks
    got = oracle.build_conv_chunks([0, 1024, 2048])
    assert got.shape == (256, 2)
    assert np.array_equal(got[:128, 0], np.zeros(128)) and np.array_equal(got[128:, 0], np.ones(128))
    assert np.array_equal(got[:128, 1], np.arange(128)) and np.array_equal(got[128:, 1], np.arange(128))


def test_closed_form_count_mixed_step():
    d = synth.mixed_step(0)
    got = oracle.build_conv_chunks(d["qsl"])
    assert len(got) == sum((L + 7) // 8 for L in d["lens"])


def test_exhaustive_small():
    for S in range(0, 4):
        for lens in itertools.product(range(0, 21), repeat=S) if S < 3 else \
                itertools.product([0, 1, 7, 8, 9, 15, 16, 17, 20], repeat=S):
            qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            got = [tuple(p) for p in oracle.build_conv_chunks(qsl)]
            assert got == chunks_by_token(list(qsl)), lens


def test_capacity_reports_needed_count():
    import ctypes
    lib = oracle._load()
    qsl = np.array([0, 9, 9, 30], np.int32)        # 2 + 0 + 3 chunks
    out = np.zeros((2, 2), np.int32)
    n = ctypes.c_int32(-1)
    rc = lib.oracle_build_conv_chunks(qsl.ctypes.data, 3, out.ctypes.data, 2, ctypes.byref(n))
    assert rc == -3 and n.value == 5
    assert [tuple(p) for p in out] == [(0, 0), (0, 1)]


def test_decreasing_qsl_rejected():
    with pytest.raises(ValueError):
        oracle.build_conv_chunks([0, 5, 3])
