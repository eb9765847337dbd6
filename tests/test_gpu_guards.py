"""GPU checks of the kernels' own index guards: a state index at or past the
pool size is skipped exactly like a padding index (-1), and a descriptor
naming no sequence of the call (or a chunk past its sequence's end) is
skipped.  Expected results come from the oracle with the offending index
replaced by -1; nothing outside the valid sequences may be written."""
import numpy as np
import pytest
import torch

import gated_deltanet_token_amd as gdn
import oracle
import synth
from parity import bits, check_bf16, check_state, dev, sentinel_like

pytestmark = pytest.mark.gpu


def _padded(idx, num_slots):
    idx = np.asarray(idx, np.int32).copy()
    idx[idx >= num_slots] = -1
    return idx


def test_conv_varlen_out_of_pool_slot_and_stray_descriptors():
    d = synth.random_conv(5, 70, [20, 13, 9], C=64, num_slots=4, has_init=[1, 0, 1])
    idx = np.array([7, 1, 2], np.int32)                 # sequence 0: past the 4-slot pool
    ch = gdn.gdn_build_conv_chunks(d["qsl"])
    stray = np.array([[3, 0], [5, 1], [-1, 0], [1, 99], [0, -2]], np.int32)
    cht = dev(np.concatenate([ch, stray]))
    x, cs = dev(d["x"]), dev(d["conv_state"])
    y = sentinel_like(tuple(x.shape))
    gdn.gdn_causal_conv1d_varlen(x, dev(d["weight"]), dev(d["bias"]), cs, dev(d["qsl"]), dev(idx),
                                 dev(d["has_init"]), cht, y)
    torch.cuda.synchronize()
    y_ref, cs_ref = oracle.causal_conv1d_varlen(d["x"], d["weight"], d["bias"], d["conv_state"], d["qsl"],
                                                _padded(idx, 4), d["has_init"])
    check_bf16(y, y_ref, "guarded conv y")
    assert np.array_equal(bits(cs), cs_ref)


def test_conv_update_out_of_pool_slot():
    d = synth.random_conv(6, 71, [1, 1, 1], C=64, num_slots=4)
    idx = np.array([0, 9, 2], np.int32)
    x, cs = dev(d["x"]), dev(d["conv_state"])
    y = sentinel_like(tuple(x.shape))
    gdn.gdn_causal_conv1d_update(x, dev(d["weight"]), dev(d["bias"]), cs, dev(idx), y)
    torch.cuda.synchronize()
    y_ref, cs_ref = oracle.causal_conv1d_update(d["x"], d["weight"], d["bias"], d["conv_state"], _padded(idx, 4))
    check_bf16(y, y_ref, "guarded update y")
    assert np.array_equal(bits(cs), cs_ref)


@pytest.mark.parametrize("form", ["decode", "token_loop", "chunk"])
def test_recurrence_out_of_pool_slot(form):
    lens = [1, 1, 1, 1] if form == "decode" else [70, 3, 129, 64]
    d = synth.random_gdn(7, 72, lens, 2, 4, 128, 64, num_slots=6)
    idx = np.array([4, 6, 1, 1000], np.int32)          # 6 and 1000: past the 6-slot pool
    q, k, v, g, b = (dev(d[n]) for n in ("q", "k", "v", "g", "beta"))
    T = q.shape[0]
    o, st = sentinel_like((T, 4, 64)), dev(d["state"])
    if form == "decode":
        gdn.gdn_fused_recurrent_decode(q, k, v, g, b, st, dev(idx), o)
        qsl = None
    elif form == "token_loop":
        gdn.gdn_fused_recurrent_decode(q, k, v, g, b, st, dev(idx), o, dev(d["qsl"]), dev(d["has_init"]))
        qsl = d["qsl"]
    else:
        gdn.gdn_chunk_gated_delta_rule(q, k, v, g, b, st, dev(idx), o, dev(d["qsl"]), dev(d["has_init"]))
        qsl = d["qsl"]
    torch.cuda.synchronize()
    pidx = _padded(idx, 6)
    o_ref, st_ref = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], pidx,
                                            qsl if qsl is not None else np.arange(T + 1, dtype=np.int32),
                                            d["has_init"] if qsl is not None else None, 1.0, True)
    check_bf16(o, o_ref, "guarded %s o" % form)
    check_state(st, st_ref, d["state"], pidx, name="guarded %s state" % form)


def test_fused_decode_slot_outside_either_pool():
    """The decode row uses one index in the conv_state pool (4 slots) and the
    state pool (8 slots): index 5 fits the second only, 9 neither; both rows
    are skipped."""
    HK, HV, dk, dv, B = 1, 2, 16, 16, 4
    C = 2 * HK * dk + HV * dv
    r = synth.rng
    x = synth.normal_bf16(r(8, 73, synth.T_X), (B, C))
    w = synth.normal_bf16(r(8, 73, synth.T_W), (C, 4), 0.5)
    bias = synth.normal_bf16(r(8, 73, synth.T_BIAS), (C,), 0.1)
    cs0 = synth.normal_bf16(r(8, 73, synth.T_CSTATE), (4, 3, C))
    g = synth.neg_softplus_normal(r(8, 73, synth.T_G), (B, HV))
    beta = synth.sigmoid_normal(r(8, 73, synth.T_BETA), (B, HV))
    st0 = (r(8, 73, synth.T_STATE).standard_normal((8, HV, dv, dk)) / np.sqrt(dk)).astype(np.float32)
    idx = np.array([3, 5, 0, 9], np.int32)
    cs, st, o = dev(cs0), dev(st0), sentinel_like((B, HV, dv))
    y = sentinel_like((B, C))
    gdn.gdn_fused_conv_decode(dev(x), dev(w), dev(bias), cs, dev(g), dev(beta), st, dev(idx), o, HK, dk, y=y)
    torch.cuda.synchronize()
    pidx = _padded(idx, 4)
    y_ref, cs_ref = oracle.causal_conv1d_update(x, w, bias, cs0, pidx)
    check_bf16(y, y_ref, "guarded fused y")
    assert np.array_equal(bits(cs), cs_ref)
    yb = oracle.round_bf16(np.nan_to_num(y_ref))
    o_ref, st_ref = oracle.gated_delta_rule(yb[:, :HK * dk].reshape(B, HK, dk),
                                            yb[:, HK * dk:2 * HK * dk].reshape(B, HK, dk),
                                            yb[:, 2 * HK * dk:].reshape(B, HV, dv), g, beta, st0, pidx,
                                            np.arange(B + 1, dtype=np.int32), None, 1.0, True)
    check_bf16(o, o_ref, "guarded fused o")
    check_state(st, st_ref, st0, pidx, name="guarded fused state")
