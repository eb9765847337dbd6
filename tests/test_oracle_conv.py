"""Pins for the oracle's causal conv (CPU only).

The conv is a depthwise cross-correlation of width K over the window
[carried state || inputs] with bias and optional SiLU (width 4: page "RTX
5070 Ti: close Qwen3.5-4B TTFT, TPOT, and VRAM gaps vs vLLM", section
"Existing evidence").  Pins: numpy ``correlate`` per channel and torch's
grouped ``conv1d`` (textbook routines with their own tap conventions),
impulse/shift weights that fix the tap order and the state carry, the
split-versus-whole invariant and update == varlen with one token.
"""
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
import synth


def f64(b):
    return synth.from_bf16(b).astype(np.float64)


def silu(z):
    return z / (1.0 + np.exp(-z))


def brute_numpy(x, w, bias, init, silu_on=True):
    """Per-channel np.correlate of [init || x] with the taps (valid mode)."""
    L, C = x.shape
    K = w.shape[1]
    e = np.concatenate([f64(init), f64(x)], axis=0)      # (K-1+L, C)
    y = np.empty((L, C))
    for c in range(C):
        y[:, c] = np.correlate(e[:, c], f64(w[c]), mode="valid") + f64(bias[c])
    return silu(y) if silu_on else y


def test_matches_numpy_correlate_with_state():
    d = synth.tiny(0)
    y, st = oracle.causal_conv1d_varlen(d["x"], d["weight"], d["bias"], d["conv_state"],
                                         d["qsl"], d["state_indices"], d["has_init"])
    K = d["K"]
    # seq 0: no initial state; seq 1: slot 0 carried in
    ref0 = brute_numpy(d["x"][0:5], d["weight"], d["bias"], np.zeros((K - 1, 64), np.uint16))
    ref1 = brute_numpy(d["x"][5:18], d["weight"], d["bias"], d["conv_state"][0])
    np.testing.assert_allclose(y[0:5], ref0, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y[5:18], ref1, rtol=1e-13, atol=1e-13)
    # new slots hold the last K-1 inputs of each sequence (bit copies)
    assert np.array_equal(st[2], d["x"][2:5])
    assert np.array_equal(st[0], d["x"][15:18])
    # untouched slots
    assert np.array_equal(st[1], d["conv_state"][1]) and np.array_equal(st[3], d["conv_state"][3])


def test_matches_torch_conv1d_zero_state():
    d = synth.random_conv(3, 90, [37], C=24, num_slots=2, has_init=[0])
    y, _ = oracle.causal_conv1d_varlen(d["x"], d["weight"], d["bias"], d["conv_state"],
                                        d["qsl"], d["state_indices"], d["has_init"], silu=False)
    xt = torch.from_numpy(f64(d["x"]).T.copy()).unsqueeze(0)            # (1, C, L)
    wt = torch.from_numpy(f64(d["weight"])).unsqueeze(1)                # (C, 1, K)
    bt = torch.from_numpy(f64(d["bias"]))
    ref = torch.nn.functional.conv1d(xt, wt, bt, padding=3, groups=24)[0, :, :37].T.numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def _one(x, w, bias, state, has_init, silu_on, slot=0):
    qsl = np.array([0, x.shape[0]], np.int32)
    return oracle.causal_conv1d_varlen(x, w, bias, state, qsl, np.array([slot], np.int32),
                                       np.array([has_init], np.uint8), silu=silu_on)


def test_identity_tap_gives_input_plus_bias():
    d = synth.random_conv(1, 91, [19], C=16, num_slots=1)
    w = np.zeros_like(d["weight"]); w[:, 3] = synth.to_bf16(np.ones(16, np.float32))
    y, _ = _one(d["x"], w, d["bias"], d["conv_state"], 1, False)
    assert np.array_equal(y, f64(d["x"]) + f64(d["bias"])[None, :])


def test_oldest_tap_shifts_by_three_and_reads_state():
    d = synth.random_conv(2, 92, [11], C=8, num_slots=1)
    w = np.zeros_like(d["weight"]); w[:, 0] = synth.to_bf16(np.ones(8, np.float32))
    y, _ = _one(d["x"], w, None, d["conv_state"], 1, False)
    expect = np.concatenate([f64(d["conv_state"][0]), f64(d["x"])[:-3]], axis=0)
    assert np.array_equal(y, expect)
    # without an initial state the first three outputs see zeros
    y0, _ = _one(d["x"], w, None, d["conv_state"], 0, False)
    assert np.array_equal(y0[:3], np.zeros((3, 8))) and np.array_equal(y0[3:], f64(d["x"])[:-3])


def test_zero_weights_give_silu_of_bias():
    d = synth.random_conv(3, 93, [6], C=8, num_slots=1)
    w = np.zeros_like(d["weight"])
    y, _ = _one(d["x"], w, d["bias"], d["conv_state"], 1, True)
    assert np.array_equal(y, np.broadcast_to(silu(f64(d["bias"])), y.shape))


@pytest.mark.parametrize("L", list(range(0, 21)))
def test_short_sequences_state_carry(L):
    """Lengths around K-1: the new slot mixes old state and new inputs."""
    d = synth.random_conv(4, 94, [L], C=8, num_slots=3, state_indices=[1])
    y, st = _one(d["x"], d["weight"], d["bias"], d["conv_state"], 1, True, slot=1)
    e = np.concatenate([d["conv_state"][1], d["x"]], axis=0)
    assert np.array_equal(st[1], e[L:L + 3])
    assert np.array_equal(st[0], d["conv_state"][0]) and np.array_equal(st[2], d["conv_state"][2])
    if L:
        ref = brute_numpy(d["x"], d["weight"], d["bias"], d["conv_state"][1])
        np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def _split_run(x, w, bias, state, cuts, slot=0):
    """Run a single sequence as consecutive calls, carrying the slot."""
    ys = []
    st = state
    bounds = [0] + list(cuts) + [x.shape[0]]
    for i in range(len(bounds) - 1):
        a, b = bounds[i], bounds[i + 1]
        y, st = _one(x[a:b], w, bias, st, int(i > 0), True, slot)
        ys.append(y)
    return np.concatenate(ys, axis=0), st


@settings(max_examples=60, deadline=None)
@given(L=st.integers(1, 40), data=st.data())
def test_split_vs_whole_bit_identical(L, data):
    d = synth.random_conv(5, 95, [L], C=8, num_slots=1)
    cuts = sorted(set(data.draw(st.lists(st.integers(1, max(1, L - 1)), max_size=5)))) if L > 1 else []
    y_whole, st_whole = _split_run(d["x"], d["weight"], d["bias"], d["conv_state"], [])
    y_split, st_split = _split_run(d["x"], d["weight"], d["bias"], d["conv_state"], cuts)
    assert np.array_equal(y_whole, y_split)
    assert np.array_equal(st_whole, st_split)


def test_update_equals_varlen_single_token():
    d = synth.fused_decode(0)
    C = 256
    x = d["x"][:, :C].copy()
    cs = d["conv_state"][:, :, :C].copy()
    w, b = d["weight"][:C], d["bias"][:C]
    idx = d["state_indices"]
    y_u, st_u = oracle.causal_conv1d_update(x, w, b, cs, idx)
    qsl = np.arange(x.shape[0] + 1, dtype=np.int32)
    y_v, st_v = oracle.causal_conv1d_varlen(x, w, b, cs, qsl, idx, np.ones(len(idx), np.uint8))
    assert np.array_equal(y_u, y_v)
    assert np.array_equal(st_u, st_v)


def test_update_window_shift():
    d = synth.fused_decode(1)
    C = 64
    x, cs = d["x"][:4, :C].copy(), d["conv_state"][:, :, :C].copy()
    idx = np.array([5, -1, 7, 9], np.int32)
    y, st = oracle.causal_conv1d_update(x, d["weight"][:C], d["bias"][:C], cs, idx)
    assert np.array_equal(st[5], np.stack([cs[5, 1], cs[5, 2], x[0]]))
    assert np.isnan(y[1]).all()                     # padding row untouched
    ref = brute_numpy(x[2:3], d["weight"][:C], d["bias"][:C], cs[7])
    np.testing.assert_allclose(y[2:3], ref, rtol=1e-13, atol=1e-13)
    others = [s for s in range(64) if s not in (5, 7, 9)]
    assert np.array_equal(st[others], cs[others])


def test_padding_and_empty_sequences_untouched():
    d = synth.random_conv(6, 96, [4, 0, 9], C=16, num_slots=4, state_indices=[0, 1, -1])
    y, st = oracle.causal_conv1d_varlen(d["x"], d["weight"], d["bias"], d["conv_state"],
                                         d["qsl"], d["state_indices"], d["has_init"])
    assert not np.isnan(y[:4]).any()
    assert np.isnan(y[4:]).all()                    # slot -1: nothing written
    assert np.array_equal(st[1:], d["conv_state"][1:])  # empty seq and padding keep slots


def test_strided_rows_match_packed():
    d = synth.random_conv(7, 97, [10, 7], C=16, num_slots=4)
    wide = np.zeros((17, 40), np.uint16)
    wide[:, 8:24] = d["x"]
    y1, s1 = oracle.causal_conv1d_varlen(wide[:, 8:24], d["weight"], d["bias"], d["conv_state"],
                                          d["qsl"], d["state_indices"], d["has_init"])
    y2, s2 = oracle.causal_conv1d_varlen(d["x"], d["weight"], d["bias"], d["conv_state"],
                                          d["qsl"], d["state_indices"], d["has_init"])
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_round_bf16_rounds_doubles_once():
    """Doubles just off a bf16 tie, closer to it than float32 can resolve:
    the nearest bf16 is fixed by the side of the tie the value lies on.
    Rounding through float32 first would land on the tie itself and then
    round to even, picking the wrong neighbour for half of these values.
    Expected values come from the construction (the two bf16 neighbours
    around each tie), not from any rounding routine."""
    r = np.random.default_rng(3)
    n = 20000
    # random finite, normal bf16 values and the next bf16 away from zero
    exp_bits = r.integers(1, 254, n).astype(np.uint32) << 7
    man = r.integers(0, 127, n).astype(np.uint32)        # 127 excluded: the neighbour keeps the exponent
    sign = r.integers(0, 2, n).astype(np.uint32) << 15
    lo_bits = (sign | exp_bits | man).astype(np.uint16)
    hi_bits = (lo_bits + 1).astype(np.uint16)            # one ulp further from zero
    lo = synth.from_bf16(lo_bits).astype(np.float64)
    hi = synth.from_bf16(hi_bits).astype(np.float64)
    tie = (lo + hi) / 2                                   # exact in float64
    # offsets well below half a float32 ulp of the tie, yet nonzero in float64
    off = np.abs(tie) * 2.0 ** -40
    above, below = tie + np.sign(tie) * off, tie - np.sign(tie) * off
    assert np.all(above.astype(np.float32).astype(np.float64) == tie)    # float32 cannot tell them apart
    assert np.array_equal(oracle.round_bf16(above), hi_bits)
    assert np.array_equal(oracle.round_bf16(below), lo_bits)
    # and exactly on the tie: to the neighbour with the even last bit
    even = np.where(lo_bits % 2 == 0, lo_bits, hi_bits)
    assert np.array_equal(oracle.round_bf16(tie), even)


def test_round_bf16_matches_input_rounding():
    """The oracle's own fp64 -> bf16 rounding agrees with round-to-nearest-even
    done on the float32 bit pattern for values that are exactly float32."""
    r = np.random.default_rng(0)
    a = (r.standard_normal(100000) * np.exp(r.uniform(-20, 20, 100000))).astype(np.float32)
    a[:4] = [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]     # ties: to even
    assert np.array_equal(oracle.round_bf16(a.astype(np.float64)), synth.to_bf16(a))
