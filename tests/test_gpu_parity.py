"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle on
identical seeded inputs, element by element, at the workload sizes and on
ragged/edge cases.  Bars are defined in ``parity.py``."""
import numpy as np
import pytest
import torch

import gated_deltanet_token_amd as gdn
import oracle
import synth
from parity import (SENTINEL, bits, check_bf16, check_state, dev, f64, sentinel_like)

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# runners: one call each, inputs as numpy, results back as tensors
# ---------------------------------------------------------------------------

def gpu_varlen(x, w, b, cs, qsl, idx, hi, y=None, silu=True):
    xt = x if torch.is_tensor(x) else dev(x)
    yt = sentinel_like(tuple(xt.shape)) if y is None else y
    cst = dev(cs)
    ch = gdn.gdn_build_conv_chunks(qsl)
    cht = dev(ch) if len(ch) else None
    gdn.gdn_causal_conv1d_varlen(xt, dev(w), None if b is None else dev(b), cst, dev(qsl), dev(idx),
                                 None if hi is None else dev(hi), cht, yt, silu=silu)
    _sync()
    return yt, cst


def gpu_update(x, w, b, cs, idx, silu=True):
    xt = dev(x)
    yt = sentinel_like(tuple(xt.shape))
    cst = dev(cs)
    gdn.gdn_causal_conv1d_update(xt, dev(w), None if b is None else dev(b), cst, dev(idx), yt, silu=silu)
    _sync()
    return yt, cst


def gpu_rec(q, k, v, g, beta, state, idx, qsl=None, hi=None, scale=1.0, norm=True, o=None,
            state_t=None):
    qt, kt, vt = (a if torch.is_tensor(a) else dev(a) for a in (q, k, v))
    T, HV, dv_ = vt.shape
    ot = sentinel_like((T, HV, dv_)) if o is None else o
    st = dev(state) if state_t is None else state_t
    gdn.gdn_fused_recurrent_decode(qt, kt, vt, dev(g), dev(beta), st, dev(idx), ot,
                                   None if qsl is None else dev(qsl), None if hi is None else dev(hi),
                                   scale, norm)
    _sync()
    return ot, st


# ---------------------------------------------------------------------------
# the tiny case
# ---------------------------------------------------------------------------

def test_tiny_conv_varlen_and_update():
    d = synth.tiny(0)
    y, cs = gpu_varlen(d["x"], d["weight"], d["bias"], d["conv_state"], d["qsl"], d["state_indices"],
                       d["has_init"])
    y_ref, cs_ref = oracle.causal_conv1d_varlen(d["x"], d["weight"], d["bias"], d["conv_state"],
                                                 d["qsl"], d["state_indices"], d["has_init"])
    check_bf16(y, y_ref, "tiny conv y")
    assert np.array_equal(bits(cs), cs_ref)
    yu, cs2 = gpu_update(d["x_dec"], d["weight"], d["bias"], cs_ref, d["state_indices"])
    yu_ref, cs2_ref = oracle.causal_conv1d_update(d["x_dec"], d["weight"], d["bias"], cs_ref,
                                                  d["state_indices"])
    check_bf16(yu, yu_ref, "tiny update y")
    assert np.array_equal(bits(cs2), cs2_ref)


@pytest.mark.parametrize("scale,norm", [(1.0, True), (0.25, True), (1.0, False)])
def test_tiny_decode(scale, norm):
    d = synth.tiny(0)
    q, k = d["q"], d["k"]
    if not norm:   # unit-scale inputs when the kernel does not normalise (exact /4)
        q = synth.to_bf16(synth.from_bf16(q) * 0.25)
        k = synth.to_bf16(synth.from_bf16(k) * 0.25)
    o, st = gpu_rec(q, k, d["v"], d["g"], d["beta"], d["state"], d["state_indices"], scale=scale, norm=norm)
    o_ref, st_ref = oracle.gated_delta_rule(q, k, d["v"], d["g"], d["beta"], d["state"],
                                            d["state_indices"], None, None, scale, norm)
    check_bf16(o, o_ref, "tiny o")
    check_state(st, st_ref, d["state"], d["state_indices"])


# ---------------------------------------------------------------------------
# workload-size cases
# ---------------------------------------------------------------------------

def test_varlen_prefill_2x1024_8192ch():
    d = synth.varlen_prefill(0)
    y, cs = gpu_varlen(d["x"], d["weight"], d["bias"], d["conv_state"], d["qsl"], d["state_indices"],
                       d["has_init"])
    y_ref, cs_ref = oracle.causal_conv1d_varlen(d["x"], d["weight"], d["bias"], d["conv_state"],
                                                 d["qsl"], d["state_indices"], d["has_init"])
    check_bf16(y, y_ref, "prefill conv y")
    assert np.array_equal(bits(cs), cs_ref)      # new slots and 62 untouched slots


def test_mixed_step_conv_and_recurrence():
    d = synth.mixed_step(0, with_recurrence=True)
    nd = d["n_dec"]
    x_all = dev(d["x_all"])
    y_all = sentinel_like(tuple(x_all.shape))
    # prefill rows follow the decode rows: column-aligned views into one buffer
    y_pre, cs = gpu_varlen(x_all[nd:], d["weight"], d["bias"], d["conv_state"], d["qsl"],
                           d["state_indices"], d["has_init"], y=y_all[nd:])
    cs_np = bits(cs)
    gdn.gdn_causal_conv1d_update(x_all[:nd], dev(d["weight"]), dev(d["bias"]), cs, dev(d["dec_indices"]),
                                 y_all[:nd])
    _sync()
    y_ref = np.full(d["x_all"].shape, np.nan)
    y_ref[nd:], cs_ref = oracle.causal_conv1d_varlen(d["x_all"][nd:], d["weight"], d["bias"],
                                                     d["conv_state"], d["qsl"], d["state_indices"],
                                                     d["has_init"])
    assert np.array_equal(cs_np, cs_ref)
    y_ref[:nd], cs_ref = oracle.causal_conv1d_update(d["x_all"][:nd], d["weight"], d["bias"], cs_ref,
                                                     d["dec_indices"])
    check_bf16(y_all, y_ref, "mixed step conv y")
    assert np.array_equal(bits(cs), cs_ref)

    # recurrence: decodes (one token each) then the three prefill chunks
    st = dev(d["state"])
    o = sentinel_like((d["x_all"].shape[0], d["HV"], d["dv"]))
    gpu_rec(d["q"][:nd], d["k"][:nd], d["v"][:nd], d["g"][:nd], d["beta"][:nd], None, d["dec_indices"],
            o=o[:nd], state_t=st)
    gpu_rec(d["q"][nd:], d["k"][nd:], d["v"][nd:], d["g"][nd:], d["beta"][nd:], None,
            d["state_indices"], qsl=d["qsl"], hi=d["has_init"], o=o[nd:], state_t=st)
    o_ref = np.full((d["x_all"].shape[0], d["HV"], d["dv"]), np.nan)
    o_ref[:nd], s_ref = oracle.gated_delta_rule(d["q"][:nd], d["k"][:nd], d["v"][:nd], d["g"][:nd],
                                                d["beta"][:nd], d["state"], d["dec_indices"], None, None,
                                                1.0, True)
    o_ref[nd:], s_ref = oracle.gated_delta_rule(d["q"][nd:], d["k"][nd:], d["v"][nd:], d["g"][nd:],
                                                d["beta"][nd:], s_ref, d["state_indices"], d["qsl"],
                                                d["has_init"], 1.0, True)
    check_bf16(o, o_ref, "mixed step o")
    check_state(st, s_ref, d["state"], np.concatenate([d["dec_indices"], d["state_indices"]]))


def test_fused_decode_32seqs_gqa():
    d = synth.fused_decode(0)
    y, cs = gpu_update(d["x"], d["weight"], d["bias"], d["conv_state"], d["state_indices"])
    y_ref, cs_ref = oracle.causal_conv1d_update(d["x"], d["weight"], d["bias"], d["conv_state"],
                                                d["state_indices"])
    check_bf16(y, y_ref, "decode update y")
    assert np.array_equal(bits(cs), cs_ref)
    o, st = gpu_rec(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["state_indices"])
    o_ref, st_ref = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                            d["state_indices"], None, None, 1.0, True)
    check_bf16(o, o_ref, "decode o")
    check_state(st, st_ref, d["state"], d["state_indices"])


# ---------------------------------------------------------------------------
# ragged and edge cases
# ---------------------------------------------------------------------------

CONV_EDGES = [
    # lens, channels, has_init, padding mask
    ([1], 8, [1], None),
    ([5, 13], 64, [0, 1], None),
    ([0, 1, 2, 3, 4, 7, 8, 9, 15, 16, 17, 31], 2056, None, None),
    ([33, 0, 21, 9], 4104, [1, 0, 1, 1], [False, False, True, False]),
    ([64, 3], 8192, [0, 1], None),
    ([2], 6144, [1], [True]),
]


@pytest.mark.parametrize("lens,C,hi,pad", CONV_EDGES)
@pytest.mark.parametrize("silu", [True, False])
def test_conv_varlen_edges(lens, C, hi, pad, silu):
    S = len(lens)
    d = synth.random_conv(21, 60 + len(lens), lens, C, num_slots=S + 3, has_init=hi)
    idx = d["state_indices"].copy()
    if pad is not None:
        idx[np.array(pad)] = -1
    # strided rows: x and y live in wider buffers
    T = int(sum(lens))
    xw = np.zeros((T, C + 24), np.uint16)
    xw[:, 16:16 + C] = d["x"]
    xt = dev(xw)[:, 16:16 + C]
    yw = sentinel_like((T, C + 40))
    bias = None if C == 6144 else d["bias"]
    y, cs = gpu_varlen(xt, d["weight"], bias, d["conv_state"], d["qsl"], idx, d["has_init"] if hi else None,
                       y=yw[:, 8:8 + C], silu=silu)
    y_ref, cs_ref = oracle.causal_conv1d_varlen(d["x"], d["weight"], bias, d["conv_state"], d["qsl"], idx,
                                                 d["has_init"] if hi else None, silu)
    check_bf16(y, y_ref, "conv edge y")
    b = bits(yw)
    assert np.all(b[:, :8] == SENTINEL) and np.all(b[:, 8 + C:] == SENTINEL)
    assert np.array_equal(bits(cs), cs_ref)


def test_conv_update_padding_and_strides():
    d = synth.random_conv(22, 70, [7], 2056, num_slots=9)
    x = synth.normal_bf16(synth.rng(22, 70, 99), (6, 2056))
    idx = np.array([3, -1, 0, 8, -1, 5], np.int32)
    xw = np.zeros((6, 2056 + 8), np.uint16)
    xw[:, 8:] = x
    yw = sentinel_like((6, 2056 + 16))
    cst = dev(d["conv_state"])
    gdn.gdn_causal_conv1d_update(dev(xw)[:, 8:], dev(d["weight"]), dev(d["bias"]), cst, dev(idx),
                                 yw[:, 16:])
    _sync()
    y_ref, cs_ref = oracle.causal_conv1d_update(x, d["weight"], d["bias"], d["conv_state"], idx)
    check_bf16(yw[:, 16:], y_ref, "update edge y")
    assert np.all(bits(yw)[:, :16] == SENTINEL)
    assert np.array_equal(bits(cst), cs_ref)


REC_EDGES = [
    # lens, HK, HV, dk, dv, has_init, padding
    ([1, 1, 1], 2, 2, 16, 16, None, None),
    ([3, 0, 5, 1], 1, 4, 32, 8, [1, 1, 0, 1], None),
    ([7, 2], 2, 4, 64, 72, [0, 1], [False, True]),
    ([9, 1, 17], 4, 8, 128, 128, [1, 0, 1], None),
    ([4, 6], 2, 2, 128, 256, None, [True, False]),
    ([25], 1, 3, 128, 40, [1], None),
]


@pytest.mark.parametrize("lens,HK,HV,dk,dv_,hi,pad", REC_EDGES)
@pytest.mark.parametrize("scale,norm", [(1.0, True), (0.125, True)])
def test_recurrent_varlen_edges(lens, HK, HV, dk, dv_, hi, pad, scale, norm):
    S = len(lens)
    d = synth.random_gdn(23, 40 + S, lens, HK, HV, dk, dv_, num_slots=S + 2, has_init=hi)
    idx = d["state_indices"].copy()
    if pad is not None:
        idx[np.array(pad)] = -1
    T = int(sum(lens))
    # q, k and v as column views of one activation row, like a conv output
    wq, wv = HK * dk, HV * dv_
    row = np.zeros((T, 2 * wq + wv + 16), np.uint16)
    row[:, 0:wq] = d["q"].reshape(T, wq)
    row[:, wq:2 * wq] = d["k"].reshape(T, wq)
    row[:, 2 * wq + 8:2 * wq + 8 + wv] = d["v"].reshape(T, wv)
    rt = dev(row)
    qt = rt[:, 0:wq].view(T, HK, dk)
    kt = rt[:, wq:2 * wq].view(T, HK, dk)
    vt = rt[:, 2 * wq + 8:2 * wq + 8 + wv].view(T, HV, dv_)
    o, st = gpu_rec(qt, kt, vt, d["g"], d["beta"], d["state"], idx, qsl=d["qsl"],
                    hi=d["has_init"] if hi else None, scale=scale, norm=norm)
    o_ref, st_ref = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], idx,
                                            d["qsl"], d["has_init"] if hi else None, scale, norm)
    check_bf16(o, o_ref, "recurrent edge o")
    used = [int(idx[s]) for s in range(S) if lens[s] > 0 and idx[s] >= 0]
    check_state(st, st_ref, d["state"], used)


def test_recurrent_decode_matches_oracle_small_dims():
    for dk, dv_ in ((16, 8), (32, 32), (64, 128)):
        d = synth.random_gdn(24, 50, [1] * 5, 1, 2, dk, dv_, num_slots=7)
        o, st = gpu_rec(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["state_indices"])
        o_ref, st_ref = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                                d["state_indices"], None, None, 1.0, True)
        check_bf16(o, o_ref, "decode dims o")
        check_state(st, st_ref, d["state"], d["state_indices"])


DECODE_EDGES = [
    # S, HK, HV, dk, dv, has_init, padding
    (5, 1, 4, 128, 128, [1, 0, 1, 1, 0], [False, False, True, False, False]),   # 512 rows: two passes
    (3, 1, 3, 128, 40, None, None),                                            # 120 rows: ragged pass
    (4, 2, 4, 16, 24, [0, 1, 1, 0], None),                                     # 4 lanes per row
    (2, 4, 8, 64, 72, [1, 1], [True, False]),
    (6, 2, 2, 32, 8, None, None),                                              # one v head per q/k head
]


@pytest.mark.parametrize("S,HK,HV,dk,dv_,hi,pad", DECODE_EDGES)
def test_decode_edges_and_varlen_launch_bit_exact(S, HK, HV, dk, dv_, hi, pad):
    """One token per sequence without query_start_loc (the decode launch)
    against the oracle, and bit for bit against the same tokens given with
    query_start_loc (the token-loop launch): the per-row arithmetic is the
    same, only the work split differs."""
    d = synth.random_gdn(27, 80 + S, [1] * S, HK, HV, dk, dv_, num_slots=S + 3, has_init=hi)
    idx = d["state_indices"].copy()
    if pad is not None:
        idx[np.array(pad)] = -1
    wq, wv = HK * dk, HV * dv_
    row = np.zeros((S, 2 * wq + wv + 24), np.uint16)
    row[:, 0:wq] = d["q"].reshape(S, wq)
    row[:, wq:2 * wq] = d["k"].reshape(S, wq)
    row[:, 2 * wq + 16:2 * wq + 16 + wv] = d["v"].reshape(S, wv)
    rt = dev(row)
    qt = rt[:, 0:wq].view(S, HK, dk)
    kt = rt[:, wq:2 * wq].view(S, HK, dk)
    vt = rt[:, 2 * wq + 16:2 * wq + 16 + wv].view(S, HV, dv_)
    hi_arr = d["has_init"] if hi else None
    o, st = gpu_rec(qt, kt, vt, d["g"], d["beta"], d["state"], idx, hi=hi_arr)
    o_ref, st_ref = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], idx,
                                            None, hi_arr, 1.0, True)
    check_bf16(o, o_ref, "decode edge o")
    used = [int(i) for i in idx if i >= 0]
    check_state(st, st_ref, d["state"], used)
    o2, st2 = gpu_rec(qt, kt, vt, d["g"], d["beta"], d["state"], idx, qsl=np.arange(S + 1, dtype=np.int32),
                      hi=hi_arr)
    assert np.array_equal(bits(o), bits(o2))
    assert torch.equal(st, st2)


# ---------------------------------------------------------------------------
# split-vs-whole on the GPU: bit-exact (identical per-token arithmetic)
# ---------------------------------------------------------------------------

def test_gpu_conv_split_vs_whole_bit_exact():
    L, C = 45, 2056
    d = synth.random_conv(25, 75, [L], C, num_slots=2, has_init=[1])
    y_w, cs_w = gpu_varlen(d["x"], d["weight"], d["bias"], d["conv_state"], d["qsl"], d["state_indices"],
                           d["has_init"])
    # pieces: 11 tokens (from the slot), 2 single-token updates, 20, then updates
    cst = dev(d["conv_state"])
    xt = dev(d["x"])
    y = sentinel_like((L, C))
    w, b, idx = dev(d["weight"]), dev(d["bias"]), dev(d["state_indices"])
    pos = 0
    for n in (11, 1, 1, 20, 1, 3, 1, 7):
        if n == 1:
            gdn.gdn_causal_conv1d_update(xt[pos:pos + 1], w, b, cst, idx, y[pos:pos + 1])
        else:
            qsl = np.array([0, n], np.int32)
            ch = dev(gdn.gdn_build_conv_chunks(qsl))
            gdn.gdn_causal_conv1d_varlen(xt[pos:pos + n], w, b, cst, dev(qsl), idx, dev(np.array([1], np.uint8)),
                                         ch, y[pos:pos + n])
        pos += n
    assert pos == L
    _sync()
    assert np.array_equal(bits(y), bits(y_w))
    assert np.array_equal(bits(cst), bits(cs_w))


def test_gpu_recurrent_split_vs_whole_bit_exact():
    L = 40
    d = synth.random_gdn(26, 76, [L], 16, 32, 128, 128, num_slots=3, state_indices=[2], has_init=[1])
    o_w, st_w = gpu_rec(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["state_indices"],
                        qsl=d["qsl"], hi=d["has_init"])
    st = dev(d["state"])
    o = sentinel_like((L, 32, 128))
    qt, kt, vt = dev(d["q"]), dev(d["k"]), dev(d["v"])
    gt, bt = dev(d["g"]), dev(d["beta"])
    idx = dev(d["state_indices"])
    pos = 0
    for n in (13, 1, 1, 17, 1, 7):
        sl = slice(pos, pos + n)
        if n == 1:   # the decode launch shape
            gdn.gdn_fused_recurrent_decode(qt[sl], kt[sl], vt[sl], gt[sl], bt[sl], st, idx, o[sl])
        else:
            gdn.gdn_fused_recurrent_decode(qt[sl], kt[sl], vt[sl], gt[sl].contiguous(), bt[sl].contiguous(),
                                           st, idx, o[sl], query_start_loc=dev(np.array([0, n], np.int32)))
        pos += n
    assert pos == L
    _sync()
    assert np.array_equal(bits(o), bits(o_w))
    assert np.array_equal(st.cpu().numpy().view(np.uint32), st_w.cpu().numpy().view(np.uint32))
