"""GPU checks of gdn_fused_conv_decode: bit-identical to
gdn_causal_conv1d_update followed by gdn_fused_recurrent_decode on the
conv output (columns q | k | v), and, end to end, within the parity bars of
the oracle's own chain (fp64 conv update -> bf16 -> fp64 recurrence)."""
import numpy as np
import pytest
import torch

import gated_deltanet_token_amd as gdn
import oracle
import synth
from parity import bits, check_bf16, check_state, dev, sentinel_like

pytestmark = pytest.mark.gpu


def make_case(seed, B, HK, HV, dk, dv, slots, pad=()):
    C = 2 * HK * dk + HV * dv
    r = synth.rng
    d = dict(B=B, HK=HK, HV=HV, dk=dk, dv=dv, C=C)
    perm = r(seed, 70, synth.T_PERM).permutation(slots)[:B].astype(np.int32)
    perm[list(pad)] = -1
    d["idx"] = perm
    d["x"] = synth.normal_bf16(r(seed, 70, synth.T_X), (B, C))
    d["w"] = synth.normal_bf16(r(seed, 70, synth.T_W), (C, 4), 0.5)
    d["b"] = synth.normal_bf16(r(seed, 70, synth.T_BIAS), (C,), 0.1)
    d["cs"] = synth.normal_bf16(r(seed, 70, synth.T_CSTATE), (slots, 3, C))
    d["g"] = synth.neg_softplus_normal(r(seed, 70, synth.T_G), (B, HV))
    d["beta"] = synth.sigmoid_normal(r(seed, 70, synth.T_BETA), (B, HV))
    d["st"] = (r(seed, 70, synth.T_STATE).standard_normal((slots, HV, dv, dk), dtype=np.float32)
               / np.float32(np.sqrt(dk)))
    return d


def run_two_call(d):
    B, C, HK, HV, dk, dv = d["B"], d["C"], d["HK"], d["HV"], d["dk"], d["dv"]
    cs, st = dev(d["cs"]), dev(d["st"])
    y = sentinel_like((B, C))
    gdn.gdn_causal_conv1d_update(dev(d["x"]), dev(d["w"]), dev(d["b"]), cs, dev(d["idx"]), y)
    o = sentinel_like((B, HV, dv))
    gdn.gdn_fused_recurrent_decode(y[:, :HK * dk].view(B, HK, dk), y[:, HK * dk:2 * HK * dk].view(B, HK, dk),
                                   y[:, 2 * HK * dk:].view(B, HV, dv), dev(d["g"]), dev(d["beta"]), st,
                                   dev(d["idx"]), o)
    torch.cuda.synchronize()
    return y, cs, st, o


def run_fused(d, with_y=True):
    B, C, HK, HV, dk, dv = d["B"], d["C"], d["HK"], d["HV"], d["dk"], d["dv"]
    cs, st = dev(d["cs"]), dev(d["st"])
    y = sentinel_like((B, C)) if with_y else None
    o = sentinel_like((B, HV, dv))
    gdn.gdn_fused_conv_decode(dev(d["x"]), dev(d["w"]), dev(d["b"]), cs, dev(d["g"]), dev(d["beta"]), st,
                              dev(d["idx"]), o, HK, dk, y=y)
    torch.cuda.synchronize()
    return y, cs, st, o


CASES = [
    # B, HK, HV, dk, dv, slots, padded rows
    (32, 16, 32, 128, 128, 64, ()),          # the decode workload
    (5, 2, 2, 16, 16, 8, (3,)),              # tiny chained geometry: 96 channels
    (7, 1, 4, 64, 72, 9, (0, 6)),            # GQA 1:4, ragged dv
    (3, 4, 8, 32, 256, 4, ()),
    (64, 16, 32, 128, 128, 64, ()),          # every slot of the 64-slot pool
]


@pytest.mark.parametrize("B,HK,HV,dk,dv,slots,pad", CASES)
def test_fused_equals_two_calls_bit_for_bit(B, HK, HV, dk, dv, slots, pad):
    d = make_case(41, B, HK, HV, dk, dv, slots, pad)
    y2, cs2, st2, o2 = run_two_call(d)
    y1, cs1, st1, o1 = run_fused(d)
    assert np.array_equal(bits(y1), bits(y2))
    assert np.array_equal(bits(cs1), bits(cs2))
    assert np.array_equal(bits(o1), bits(o2))
    assert np.array_equal(st1.cpu().numpy().view(np.uint32), st2.cpu().numpy().view(np.uint32))
    _, cs0, st0, o0 = run_fused(d, with_y=False)          # y is optional
    assert np.array_equal(bits(o0), bits(o2)) and np.array_equal(bits(cs0), bits(cs2))


def test_fused_against_oracle_chain():
    d = make_case(42, 32, 16, 32, 128, 128, 64)
    B, C, HK, HV, dk, dv = d["B"], d["C"], d["HK"], d["HV"], d["dk"], d["dv"]
    y, cs, st, o = run_fused(d)
    y_ref, cs_ref = oracle.causal_conv1d_update(d["x"], d["w"], d["b"], d["cs"], d["idx"])
    check_bf16(y, y_ref, "fused conv y")
    assert np.array_equal(bits(cs), cs_ref)
    yb = oracle.round_bf16(y_ref)
    o_ref, st_ref = oracle.gated_delta_rule(yb[:, :HK * dk].reshape(B, HK, dk),
                                            yb[:, HK * dk:2 * HK * dk].reshape(B, HK, dk),
                                            yb[:, 2 * HK * dk:].reshape(B, HV, dv), d["g"], d["beta"], d["st"],
                                            d["idx"], None, None, 1.0, True)
    check_bf16(o, o_ref, "fused o")
    # inputs of the recurrence: the GPU's bf16 conv outputs vs the oracle's own
    # rounding of its fp64 conv (chained comparison)
    check_state(st, st_ref, d["st"], d["idx"], name="fused state", tol=1e-3)
