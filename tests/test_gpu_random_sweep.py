"""Seeded random sweep of the library's entry points against the fp64 oracle.

The fixed-case tests pin the workload shapes and the edges one by one; this
file draws shapes at random (from one seeded generator, so every run draws the
same cases) over the ranges each entry point accepts, to catch a combination
that no fixed case covers: sequence counts and lengths around the 8- and
64-token chunk boundaries (empty sequences included), padded slots, a mix of
has_initial_state flags, channel counts that leave a partial channel tile,
GQA ratios, head_v_dim values, output scales and strided views.  Every result
is held to the bars in ``parity.py``; conv_state is bit-exact.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_token_amd as gdn
import oracle
import synth
from parity import SENTINEL, bits, check_bf16, check_state, dev, sentinel_like

pytestmark = pytest.mark.gpu

_R = np.random.default_rng(20261202)


def _lens(r, n_max, t_max):
    """1..n_max sequence lengths: a mix of empty, short, near-chunk-boundary
    and longer sequences, at most t_max tokens in all."""
    pool = [0, 1, 2, 3, 7, 8, 9, 15, 17, 31, 33, 63, 64, 65, 127, 128, 129, 191, 200, 257]
    out = []
    for _ in range(int(r.integers(1, n_max + 1))):
        n = int(r.choice(pool)) if r.random() < 0.7 else int(r.integers(1, 300))
        if sum(out) + n > t_max:
            n = max(0, t_max - sum(out))
        out.append(n)
    if sum(out) == 0:                  # (calls without tokens are covered by the boundary tests)
        out[-1] = 1
    return out


def _flags(r, n, p):
    return [int(r.random() < p) for _ in range(n)]


CONV_CASES = []
for _ in range(48):
    lens = _lens(_R, 6, 400)
    C = 8 * int(_R.integers(1, 700))               # 8 .. 5592 channels: partial last tile
    CONV_CASES.append(dict(lens=lens, C=C, hi=_flags(_R, len(lens), 0.6), pad=_flags(_R, len(lens), 0.2),
                           silu=bool(_R.random() < 0.7), bias=bool(_R.random() < 0.8),
                           xpad=8 * int(_R.integers(0, 4)), seed=int(_R.integers(1 << 30))))

CHUNK_CASES = []
for _ in range(48):
    lens = _lens(_R, 5, 450)
    HK = int(_R.choice([1, 2, 4]))
    HV = HK * int(_R.choice([1, 2, 3, 4]))
    CHUNK_CASES.append(dict(lens=lens, HK=HK, HV=HV, dv=int(_R.choice([32, 64, 96, 128, 160, 256])),
                            hi=_flags(_R, len(lens), 0.6), pad=_flags(_R, len(lens), 0.2),
                            scale=float(_R.choice([1.0, 0.0884, 0.5])), seed=int(_R.integers(1 << 30))))

DECODE_CASES = []
for _ in range(32):
    HK = int(_R.choice([1, 2, 4, 8]))
    HV = HK * int(_R.choice([1, 2, 4]))
    B = int(_R.integers(1, 41))
    DECODE_CASES.append(dict(B=B, HK=HK, HV=HV, dk=int(_R.choice([16, 32, 64, 128])),
                             dv=8 * int(_R.integers(2, 33)), pad=_flags(_R, B, 0.15),
                             scale=float(_R.choice([1.0, 0.25])), seed=int(_R.integers(1 << 30))))

MIXED_CASES = []
for _ in range(24):
    lens = _lens(_R, 4, 450)
    HK = int(_R.choice([1, 2, 4]))
    HV = HK * int(_R.choice([1, 2, 4]))
    B = int(_R.integers(0, 33))
    MIXED_CASES.append(dict(lens=lens, B=B, HK=HK, HV=HV, dv=int(_R.choice([32, 64, 128, 256])),
                            hi=_flags(_R, len(lens), 0.6), pad_pre=_flags(_R, len(lens), 0.2),
                            pad_dec=_flags(_R, B, 0.15), scale=float(_R.choice([1.0, 0.0884])),
                            seed=int(_R.integers(1 << 30))))


@pytest.mark.parametrize("case", range(len(CONV_CASES)))
def test_random_conv_varlen(case):
    c = CONV_CASES[case]
    lens, C, S = c["lens"], c["C"], len(c["lens"])
    d = synth.random_conv(c["seed"], 80, lens, C, num_slots=S + 2, has_init=c["hi"])
    idx = d["state_indices"].copy()
    idx[np.array(c["pad"], bool)] = -1
    T = int(sum(lens))
    bias = d["bias"] if c["bias"] else None
    y_ref, cs_ref = oracle.causal_conv1d_varlen(d["x"], d["weight"], bias, d["conv_state"], d["qsl"], idx,
                                                 d["has_init"], c["silu"])
    ch = gdn.gdn_build_conv_chunks(d["qsl"])
    outs = []
    for dpp in (1, 2):
        xp = c["xpad"]
        xw = np.zeros((max(T, 1), C + xp), np.uint16)
        xw[:T, xp:] = d["x"]
        xt = dev(xw)[:T, xp:]
        yw = sentinel_like((max(T, 1), C + 16))
        yt = yw[:T, 8:8 + C]
        cst = dev(d["conv_state"])
        gdn.gdn_causal_conv1d_varlen(xt, dev(d["weight"]), None if bias is None else dev(bias), cst,
                                     dev(d["qsl"]), dev(idx), dev(d["has_init"]), dev(ch) if len(ch) else None,
                                     yt, silu=c["silu"], descriptors_per_program=dpp)
        torch.cuda.synchronize()
        if T:
            check_bf16(yt, y_ref, "random conv y (%d descriptors per program)" % dpp)
        assert np.array_equal(bits(cst), cs_ref)
        b = bits(yw)
        assert np.all(b[:, :8] == SENTINEL) and np.all(b[:, 8 + C:] == SENTINEL)
        outs.append((bits(yw), bits(cst)))
    # the 8- and 16-token programs give the same bits
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("case", range(len(CHUNK_CASES)))
def test_random_chunk_rule(case):
    c = CHUNK_CASES[case]
    lens, S = c["lens"], len(c["lens"])
    d = synth.random_gdn(c["seed"], 81, lens, c["HK"], c["HV"], 128, c["dv"], num_slots=S + 3, has_init=c["hi"])
    idx = d["state_indices"].copy()
    idx[np.array(c["pad"], bool)] = -1
    T = int(sum(lens))
    HV, dv = c["HV"], c["dv"]
    o_ref, st_ref = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], idx, d["qsl"],
                                            d["has_init"], c["scale"], True)

    def rows(a):
        return dev(a if a.shape[0] else np.zeros((1,) + a.shape[1:], a.dtype))[:T]

    o = sentinel_like((max(T, 1), HV, dv))[:T]
    st = dev(d["state"])
    gdn.gdn_chunk_gated_delta_rule(rows(d["q"]), rows(d["k"]), rows(d["v"]), rows(d["g"]), rows(d["beta"]), st,
                                   dev(idx), o, dev(d["qsl"]), dev(d["has_init"]), c["scale"], True)
    torch.cuda.synchronize()
    if T:
        check_bf16(o, o_ref, "random chunk o")
    used = [int(idx[s]) for s in range(S) if lens[s] > 0 and idx[s] >= 0]
    check_state(st, st_ref, d["state"], used)          # and every other slot bit-identical


@pytest.mark.parametrize("case", range(len(DECODE_CASES)))
def test_random_fused_decode(case):
    c = DECODE_CASES[case]
    B, HK, HV, dk, dv = c["B"], c["HK"], c["HV"], c["dk"], c["dv"]
    C = 2 * HK * dk + HV * dv
    slots = B + 2
    r = synth.rng
    s = c["seed"]
    idx = r(s, 82, synth.T_PERM).permutation(slots)[:B].astype(np.int32)
    idx[np.array(c["pad"], bool)] = -1
    x = synth.normal_bf16(r(s, 82, synth.T_X), (B, C))
    w = synth.normal_bf16(r(s, 82, synth.T_W), (C, 4), 0.5)
    b = synth.normal_bf16(r(s, 82, synth.T_BIAS), (C,), 0.1)
    cs = synth.normal_bf16(r(s, 82, synth.T_CSTATE), (slots, 3, C))
    g = synth.neg_softplus_normal(r(s, 82, synth.T_G), (B, HV))
    beta = synth.sigmoid_normal(r(s, 82, synth.T_BETA), (B, HV))
    st0 = r(s, 82, synth.T_STATE).standard_normal((slots, HV, dv, dk), dtype=np.float32) / np.float32(np.sqrt(dk))

    cst, stt = dev(cs), dev(st0)
    y = sentinel_like((B, C))
    o = sentinel_like((B, HV, dv))
    gdn.gdn_fused_conv_decode(dev(x), dev(w), dev(b), cst, dev(g), dev(beta), stt, dev(idx), o, HK, dk, y=y,
                              scale=c["scale"])
    torch.cuda.synchronize()
    y_ref, cs_ref = oracle.causal_conv1d_update(x, w, b, cs, idx)
    check_bf16(y, y_ref, "random fused conv y")
    assert np.array_equal(bits(cst), cs_ref)
    yb = oracle.round_bf16(y_ref)
    o_ref, st_ref = oracle.gated_delta_rule(yb[:, :HK * dk].reshape(B, HK, dk),
                                            yb[:, HK * dk:2 * HK * dk].reshape(B, HK, dk),
                                            yb[:, 2 * HK * dk:].reshape(B, HV, dv), g, beta, st0, idx, None, None,
                                            c["scale"], True)
    check_bf16(o, o_ref, "random fused o")
    used = [int(i) for i in idx if i >= 0]
    # the recurrence runs on the GPU's own bf16 conv outputs (chained comparison)
    check_state(stt, st_ref, st0, used, name="random fused state", tol=1e-3)


@pytest.mark.parametrize("case", range(len(MIXED_CASES)))
def test_random_mixed_step(case):
    """The one-grid mixed-step call: its prefill half against the oracle's
    rule, its decode half against the oracle's conv update + rule chain."""
    c = MIXED_CASES[case]
    lens, B, HK, HV, dv = c["lens"], c["B"], c["HK"], c["HV"], c["dv"]
    dk, S = 128, len(lens)
    slots = S + B + 2
    d = synth.random_gdn(c["seed"], 83, lens, HK, HV, dk, dv, num_slots=slots, has_init=c["hi"])
    r, s = synth.rng, c["seed"]
    perm = r(s, 84, synth.T_PERM).permutation(slots).astype(np.int32)
    idx, didx = perm[:S].copy(), perm[S:S + B].copy()
    idx[np.array(c["pad_pre"], bool)] = -1
    didx[np.array(c["pad_dec"], bool)] = -1
    C = 2 * HK * dk + HV * dv
    x = synth.normal_bf16(r(s, 84, synth.T_X), (B, C))
    w = synth.normal_bf16(r(s, 84, synth.T_W), (C, 4), 0.5)
    b = synth.normal_bf16(r(s, 84, synth.T_BIAS), (C,), 0.1)
    cs = synth.normal_bf16(r(s, 84, synth.T_CSTATE), (slots, 3, C))
    dg = synth.neg_softplus_normal(r(s, 84, synth.T_G), (B, HV))
    dbeta = synth.sigmoid_normal(r(s, 84, synth.T_BETA), (B, HV))
    T = int(sum(lens))

    def rows(a, n):
        return dev(a if a.shape[0] else np.zeros((1,) + a.shape[1:], a.dtype))[:n]

    st, cst = dev(d["state"]), dev(cs)
    o = sentinel_like((max(T, 1), HV, dv))[:T]
    do = sentinel_like((max(B, 1), HV, dv))[:B]
    y = sentinel_like((max(B, 1), C))[:B]
    gdn.gdn_chunk_rule_and_fused_decode(rows(d["q"], T), rows(d["k"], T), rows(d["v"], T), rows(d["g"], T),
                                        rows(d["beta"], T), dev(idx), o, dev(d["qsl"]), dev(d["has_init"]),
                                        rows(x, B), dev(w), dev(b), cst, rows(dg, B), rows(dbeta, B), rows(didx, B),
                                        do, st, HK, dec_y=y, scale=c["scale"])
    torch.cuda.synchronize()

    o_ref, st_pre = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], idx, d["qsl"],
                                            d["has_init"], c["scale"], True)
    check_bf16(o, o_ref, "random mixed prefill o")
    st_ref = np.asarray(st_pre, np.float64).copy()
    dec_used = []
    if B:
        y_ref, cs_ref = oracle.causal_conv1d_update(x, w, b, cs, didx)
        check_bf16(y, y_ref, "random mixed decode y")
        assert np.array_equal(bits(cst), cs_ref)
        yb = oracle.round_bf16(y_ref)
        do_ref, st_dec = oracle.gated_delta_rule(yb[:, :HK * dk].reshape(B, HK, dk),
                                                 yb[:, HK * dk:2 * HK * dk].reshape(B, HK, dk),
                                                 yb[:, 2 * HK * dk:].reshape(B, HV, dv), dg, dbeta, d["state"], didx,
                                                 None, None, c["scale"], True)
        check_bf16(do, do_ref, "random mixed decode o")
        dec_used = [int(i) for i in didx if i >= 0]
        st_ref[dec_used] = st_dec[dec_used]
    else:
        assert np.array_equal(bits(cst), cs)
    pre_used = [int(idx[i]) for i in range(S) if lens[i] > 0 and idx[i] >= 0]
    # prefill slots at the state bar, decode slots at the chained bar, every other slot untouched
    check_state(st, st_ref, d["state"], pre_used + dec_used, name="random mixed state", tol=1e-3)
    if pre_used:
        check_state(st[pre_used], st_ref[pre_used], d["state"][pre_used], range(len(pre_used)),
                    name="random mixed prefill state")
