"""Pins for the oracle's gated delta rule (CPU only).

The rule (Yang, Kautz, Hatamizadeh, "Gated Delta Networks", ICLR 2025,
recurrent form; the fused decode is named on page "RTX 5070 Ti: close
Qwen3.5-4B TTFT, TPOT, and VRAM gaps vs vLLM", section "Existing evidence"):
S <- a S (I - b k k^T) + b v k^T, o = scale S q, with a = exp(g) and q, k
optionally L2-normalised.  Pins: a dense brute force with the explicit dk x dk
transition matrix, the one-token closed form from a zero state, the
delta-rule retrieval identity, orthonormal keys, identity/decay special
cases, split-versus-whole, slot permutation and the GQA head map.
"""
import numpy as np
import pytest

import oracle
import synth


def f64(b):
    return synth.from_bf16(b).astype(np.float64)


def l2n(x):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + 1e-6)


def dense_reference(q, k, v, g, beta, S0, scale, norm):
    """Single sequence, single head pair: matrices written out in full."""
    S = S0.copy()
    dk = S.shape[1]
    out = []
    for t in range(q.shape[0]):
        qt, kt = (l2n(q[t]), l2n(k[t])) if norm else (q[t], k[t])
        a, b = np.exp(g[t]), beta[t]
        M = np.eye(dk) - b * np.outer(kt, kt)
        S = a * (S @ M) + b * np.outer(v[t], kt)
        out.append(scale * (S @ qt))
    return np.array(out), S


@pytest.mark.parametrize("norm", [True, False])
@pytest.mark.parametrize("HK,HV", [(2, 2), (2, 4), (1, 3)])
def test_dense_brute_force(norm, HK, HV):
    lens = [5, 1, 9]
    d = synth.random_gdn(11, 80, lens, HK, HV, 16, 8, num_slots=5, has_init=[1, 0, 1])
    scale = 0.37
    o, st = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                    d["state_indices"], d["qsl"], d["has_init"], scale, norm)
    grp = HV // HK
    for s in range(len(lens)):
        a, b = d["qsl"][s], d["qsl"][s + 1]
        slot = d["state_indices"][s]
        for h in range(HV):
            S0 = d["state"][slot, h].astype(np.float64) if d["has_init"][s] else np.zeros((8, 16))
            ref_o, ref_S = dense_reference(f64(d["q"][a:b, h // grp]), f64(d["k"][a:b, h // grp]),
                                           f64(d["v"][a:b, h]), d["g"][a:b, h].astype(np.float64),
                                           d["beta"][a:b, h].astype(np.float64), S0, scale, norm)
            np.testing.assert_allclose(o[a:b, h], ref_o, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(st[slot, h], ref_S, rtol=1e-11, atol=1e-12)


def test_single_token_from_zero_closed_form():
    """From S = 0, one token: S = b v k^T and o = scale b (k.q) v."""
    d = synth.tiny(0)
    o, st = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                    d["state_indices"], None, None, 0.5, True)
    for s in range(2):
        slot = d["state_indices"][s]
        for h in range(2):
            q, k, v = l2n(f64(d["q"][s, h])), l2n(f64(d["k"][s, h])), f64(d["v"][s, h])
            b = float(d["beta"][s, h])
            np.testing.assert_allclose(st[slot, h], b * np.outer(v, k), rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(o[s, h], 0.5 * b * (k @ q) * v, rtol=1e-13, atol=1e-15)


def _single(q, k, v, g, beta, S0, norm=False, scale=1.0):
    """One sequence, one head, everything given as float arrays."""
    T, dk = q.shape
    dv = v.shape[1]
    qb = synth.to_bf16(q.astype(np.float32)).reshape(T, 1, dk)
    kb = synth.to_bf16(k.astype(np.float32)).reshape(T, 1, dk)
    vb = synth.to_bf16(v.astype(np.float32)).reshape(T, 1, dv)
    o, st = oracle.gated_delta_rule(qb, kb, vb, np.asarray(g, np.float32).reshape(T, 1),
                                    np.asarray(beta, np.float32).reshape(T, 1),
                                    S0.reshape(1, 1, dv, dk), np.array([0], np.int32),
                                    np.array([0, T], np.int32), None, scale, norm)
    return o[:, 0], st[0, 0]


def test_identity_when_beta_zero_alpha_one():
    r = np.random.default_rng(1)
    S0 = r.standard_normal((8, 16))
    q, k, v = r.standard_normal((3, 16)), r.standard_normal((3, 16)), r.standard_normal((3, 8))
    o, S = _single(q, k, v, np.zeros(3), np.zeros(3), S0)
    assert np.array_equal(S, S0)
    np.testing.assert_allclose(o[-1], S0 @ f64(synth.to_bf16(q[-1].astype(np.float32))), rtol=1e-13)


def test_zero_key_only_decays():
    r = np.random.default_rng(2)
    S0 = r.standard_normal((8, 16))
    q, v = r.standard_normal((1, 16)), r.standard_normal((1, 8))
    g = np.array([-0.3])
    o, S = _single(q, np.zeros((1, 16)), v, g, np.array([0.7]), S0)
    np.testing.assert_allclose(S, np.exp(np.float64(np.float32(-0.3))) * S0, rtol=1e-15)


def test_delta_rule_retrieval():
    """a = b = 1 and a unit key: the new state maps the key to v exactly."""
    r = np.random.default_rng(3)
    S0 = r.standard_normal((8, 16))
    k = np.zeros((1, 16)); k[0, 5] = 1.0                      # unit, exact in bf16
    v = r.standard_normal((1, 8))
    o, S = _single(r.standard_normal((1, 16)), k, v, np.zeros(1), np.ones(1), S0)
    np.testing.assert_allclose(S @ k[0], f64(synth.to_bf16(v[0].astype(np.float32))), rtol=0, atol=1e-14)
    # directions orthogonal to k are untouched
    np.testing.assert_array_equal(np.delete(S, 5, axis=1), np.delete(S0, 5, axis=1))


def test_orthonormal_keys_accumulate_outer_products():
    """a = b = 1, zero start, keys = distinct basis vectors: S = sum v_i k_i^T."""
    r = np.random.default_rng(4)
    n = 6
    k = np.eye(16)[[3, 0, 9, 12, 7, 1]]
    v = synth.from_bf16(synth.to_bf16(r.standard_normal((n, 8)).astype(np.float32))).astype(np.float64)
    o, S = _single(r.standard_normal((n, 16)), k, v, np.zeros(n), np.ones(n), np.zeros((8, 16)))
    np.testing.assert_allclose(S, v.T @ k, rtol=0, atol=1e-15)


def test_split_vs_whole_bit_identical():
    d = synth.random_gdn(12, 81, [23], 2, 4, 16, 16, num_slots=2, state_indices=[1])
    args = (d["g"], d["beta"])
    o_w, st_w = oracle.gated_delta_rule(d["q"], d["k"], d["v"], *args, d["state"],
                                        d["state_indices"], d["qsl"], None, 1.0, True)
    st = d["state"].astype(np.float64)
    outs = []
    for a, b in [(0, 7), (7, 8), (8, 20), (20, 23)]:
        o, st = oracle.gated_delta_rule(d["q"][a:b], d["k"][a:b], d["v"][a:b], d["g"][a:b],
                                        d["beta"][a:b], st, d["state_indices"],
                                        np.array([0, b - a], np.int32), None, 1.0, True)
        outs.append(o)
    assert np.array_equal(np.concatenate(outs), o_w)
    assert np.array_equal(st, st_w)


def test_slot_permutation_equivariance_and_untouched_slots():
    d = synth.random_gdn(13, 82, [3, 4, 2], 1, 2, 8, 8, num_slots=6, state_indices=[4, 0, 2])
    o1, st1 = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                      d["state_indices"], d["qsl"], None, 1.0, True)
    perm = np.array([3, 5, 1, 0, 4, 2])                      # slot i -> perm[i]
    st_p = np.empty_like(d["state"]); st_p[perm] = d["state"]
    o2, st2 = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], st_p,
                                      perm[d["state_indices"]].astype(np.int32), d["qsl"], None, 1.0, True)
    assert np.array_equal(o1, o2)
    assert np.array_equal(st2[perm], st1)
    for s in (1, 3, 5):
        assert np.array_equal(st1[s], d["state"][s].astype(np.float64))


def test_padding_slot_and_no_initial_state():
    d = synth.random_gdn(14, 83, [2, 3], 1, 1, 8, 8, num_slots=3, state_indices=[-1, 2],
                         has_init=[1, 0])
    o, st = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                    d["state_indices"], d["qsl"], d["has_init"], 1.0, True)
    assert np.isnan(o[:2]).all() and not np.isnan(o[2:]).any()
    d2 = dict(d); junk = d["state"].copy(); junk[2] = 1e3
    o2, _ = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], junk,
                                    d["state_indices"], d["qsl"], d["has_init"], 1.0, True)
    assert np.array_equal(o[2:], o2[2:])                     # has_init = 0 ignores the slot


def test_gqa_head_map():
    """HV = 2 HK: v-heads 2j and 2j+1 read q/k head j."""
    d = synth.random_gdn(15, 84, [4], 2, 4, 8, 8, num_slots=1, state_indices=[0])
    o, st = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                    d["state_indices"], d["qsl"], None, 1.0, True)
    for h in range(4):
        oh, sh = _single(f64(d["q"][:, h // 2]), f64(d["k"][:, h // 2]), f64(d["v"][:, h]),
                         d["g"][:, h], d["beta"][:, h], d["state"][0, h].astype(np.float64), True)
        assert np.array_equal(oh, o[:, h])
        assert np.array_equal(sh, st[0, h])


def test_l2norm_scale_invariance_and_scale_linearity():
    d = synth.random_gdn(16, 85, [5], 1, 1, 16, 8, num_slots=1, state_indices=[0])
    base = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                   d["state_indices"], d["qsl"], None, 1.0, True)[0]
    q4 = synth.to_bf16(4.0 * synth.from_bf16(d["q"]))       # exact: power of two
    o4 = oracle.gated_delta_rule(q4, d["k"], d["v"], d["g"], d["beta"], d["state"],
                                 d["state_indices"], d["qsl"], None, 1.0, True)[0]
    np.testing.assert_allclose(o4, base, rtol=1e-7, atol=1e-9)
    o3 = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                 d["state_indices"], d["qsl"], None, 3.0, True)[0]
    np.testing.assert_allclose(o3, 3.0 * base, rtol=1e-15, atol=0)
