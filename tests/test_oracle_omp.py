"""The oracle compiled with OpenMP (used only for the benchmark's multi-core
CPU baseline) gives bit-identical results to the serial build: its pragmas
only spread independent iterations (conv channels, recurrence (sequence,
v-head) pairs) over threads."""
import ctypes

import numpy as np

import oracle
import synth


def _omp_lib(threads=4):
    lib = oracle.bind(oracle.build_omp())
    ctypes.CDLL("libgomp.so.1").omp_set_num_threads(threads)
    return lib


def _with(lib, fn, *a, **kw):
    saved = oracle._lib
    oracle._lib = lib
    try:
        return fn(*a, **kw)
    finally:
        oracle._lib = saved


def test_omp_build_matches_serial_bit_for_bit():
    omp = _omp_lib()
    d = synth.random_conv(11, 80, [37, 0, 64, 5], C=64, num_slots=6, has_init=[1, 0, 1, 1])
    args = (d["x"], d["weight"], d["bias"], d["conv_state"], d["qsl"], d["state_indices"], d["has_init"])
    y1, s1 = oracle.causal_conv1d_varlen(*args)
    y2, s2 = _with(omp, oracle.causal_conv1d_varlen, *args)
    assert np.array_equal(y1, y2, equal_nan=True) and np.array_equal(s1, s2)
    xd = synth.normal_bf16(synth.rng(11, 81, synth.T_X), (4, 64))
    u1 = oracle.causal_conv1d_update(xd, d["weight"], d["bias"], s1, [3, 0, -1, 5])
    u2 = _with(omp, oracle.causal_conv1d_update, xd, d["weight"], d["bias"], s1, [3, 0, -1, 5])
    assert np.array_equal(u1[0], u2[0], equal_nan=True) and np.array_equal(u1[1], u2[1])
    g = synth.random_gdn(11, 82, [9, 1, 20, 0, 7], 2, 6, 32, 16, num_slots=8, has_init=[1, 0, 1, 1, 0])
    idx = g["state_indices"].copy()
    idx[1] = -1
    a = (g["q"], g["k"], g["v"], g["g"], g["beta"], g["state"], idx, g["qsl"], g["has_init"], 0.5, True)
    o1, st1 = oracle.gated_delta_rule(*a)
    o2, st2 = _with(omp, oracle.gated_delta_rule, *a)
    assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(st1, st2)
