"""GPU checks of gdn_chunk_rule_and_fused_decode (the chunkwise rule on a
step's prefill tokens and the fused decode of its decode rows in one grid):
bit-identical to gdn_chunk_gated_delta_rule followed by gdn_fused_conv_decode
on the same state pool, and, at the c32 mixed-step shape, within the parity
bars of the oracle for both halves."""
import numpy as np
import pytest
import torch

import gated_deltanet_token_amd as gdn
import oracle
import synth
from parity import bits, check_bf16, check_state, dev, sentinel_like

pytestmark = pytest.mark.gpu

DK = 128


def make_case(seed, lens, B, HK, HV, dv, slots, hi=None, pad_pre=(), pad_dec=()):
    """Prefill sequences `lens` and B decode rows on one state pool of
    `slots` slots; the two halves take disjoint slots of one permutation."""
    S = len(lens)
    d = synth.random_gdn(seed, 60, lens, HK, HV, DK, dv, num_slots=slots, has_init=hi)
    perm = synth.rng(seed, 61, synth.T_PERM).permutation(slots).astype(np.int32)
    d["state_indices"] = perm[:S].copy()
    d["state_indices"][list(pad_pre)] = -1
    C = 2 * HK * DK + HV * dv
    r = synth.rng
    d.update(B=B, C=C, didx=perm[S:S + B].copy())
    d["didx"][list(pad_dec)] = -1
    d["x"] = synth.normal_bf16(r(seed, 62, synth.T_X), (B, C))
    d["w"] = synth.normal_bf16(r(seed, 62, synth.T_W), (C, 4), 0.5)
    d["b"] = synth.normal_bf16(r(seed, 62, synth.T_BIAS), (C,), 0.1)
    d["cs"] = synth.normal_bf16(r(seed, 62, synth.T_CSTATE), (slots, 3, C))
    d["dg"] = synth.neg_softplus_normal(r(seed, 62, synth.T_G), (B, HV))
    d["dbeta"] = synth.sigmoid_normal(r(seed, 62, synth.T_BETA), (B, HV))
    return d


def rows(a, n):
    """Device copy of a with at least one row, viewed as its first n rows
    (a non-NULL pointer even when n is 0)."""
    if a.shape[0] == 0:
        a = np.zeros((1,) + a.shape[1:], a.dtype)
    return dev(a)[:n]


def operands(d):
    T = d["q"].shape[0]
    HV, dv, B, C = d["HV"], d["dv"], d["B"], d["C"]
    return dict(q=rows(d["q"], T), k=rows(d["k"], T), v=rows(d["v"], T), g=rows(d["g"], T),
                beta=rows(d["beta"], T), idx=rows(d["state_indices"], len(d["state_indices"])),
                qsl=dev(d["qsl"]), hi=rows(d["has_init"], len(d["has_init"])),
                o=sentinel_like((max(T, 1), HV, dv))[:T], x=rows(d["x"], B), w=dev(d["w"]), b=dev(d["b"]),
                cs=dev(d["cs"]), dg=rows(d["dg"], B), dbeta=rows(d["dbeta"], B),
                didx=rows(d["didx"], B),
                do=sentinel_like((max(B, 1), HV, dv))[:B], y=sentinel_like((max(B, 1), C))[:B],
                st=dev(d["state"]))


def run_mixed(d, scale=1.0, norm=True, hi=True):
    t = operands(d)
    gdn.gdn_chunk_rule_and_fused_decode(t["q"], t["k"], t["v"], t["g"], t["beta"], t["idx"], t["o"], t["qsl"],
                                        t["hi"] if hi else None, t["x"], t["w"], t["b"], t["cs"], t["dg"],
                                        t["dbeta"], t["didx"], t["do"], t["st"], d["HK"], dec_y=t["y"],
                                        scale=scale, qk_l2norm=norm)
    torch.cuda.synchronize()
    return t


def run_two_calls(d, scale=1.0, norm=True, hi=True):
    t = operands(d)
    if d["q"].shape[0]:
        gdn.gdn_chunk_gated_delta_rule(t["q"], t["k"], t["v"], t["g"], t["beta"], t["st"], t["idx"], t["o"],
                                       t["qsl"], t["hi"] if hi else None, scale=scale, qk_l2norm=norm)
    if d["B"]:
        gdn.gdn_fused_conv_decode(t["x"], t["w"], t["b"], t["cs"], t["dg"], t["dbeta"], t["st"], t["didx"], t["do"],
                                  d["HK"], DK, y=t["y"], scale=scale, qk_l2norm=norm)
    torch.cuda.synchronize()
    return t


def assert_same(t1, t2):
    for n in ("o", "do", "y", "cs"):
        assert np.array_equal(bits(t1[n]), bits(t2[n])), n
    assert np.array_equal(t1["st"].cpu().numpy().view(np.uint32), t2["st"].cpu().numpy().view(np.uint32))


CASES = [
    # lens, B, HK, HV, dv, slots, has_init, padded prefill seqs, padded decode rows
    # the c32 mixed step: 192 scan workgroups, 464 decode units
    ([635, 637, 747], 29, 16, 32, 128, 64, [1, 0, 1], (), ()),
    # 6 scan workgroups padded to 8, an empty and a padded sequence, padded decode rows
    ([70, 0, 129], 5, 2, 2, 64, 12, [1, 1, 0], (2,), (1, 4)),
    # three v heads per q/k head (one v head per prep workgroup)
    ([90, 40], 7, 2, 6, 64, 12, [0, 1], (), (6,)),
    # 256-row heads: four scan workgroups per head; 512 state rows per decode unit (two passes)
    ([100, 65], 3, 2, 4, 256, 8, [1, 1], (), ()),
    # more decode units (960) than CUs left by the scan: they wait for scan CUs
    ([300, 64], 60, 16, 32, 128, 64, [1, 0], (), (7,)),
    # head_v_dim 96: the two operations as consecutive launches
    ([65, 64], 4, 2, 4, 96, 8, [1, 0], (), ()),
    # an empty half: decode only, prefill only
    ([], 6, 2, 4, 128, 8, [], (), ()),
    ([64, 1], 0, 2, 4, 128, 8, [0, 1], (), ()),
]


@pytest.mark.parametrize("lens,B,HK,HV,dv,slots,hi,pad_pre,pad_dec", CASES)
def test_mixed_call_equals_two_calls_bit_for_bit(lens, B, HK, HV, dv, slots, hi, pad_pre, pad_dec):
    d = make_case(71, lens, B, HK, HV, dv, slots, hi, pad_pre, pad_dec)
    print("mixed call case", lens, B, HK, HV, dv, flush=True)
    t2 = run_two_calls(d)
    t1 = run_mixed(d)
    assert_same(t1, t2)
    # the prefill's padded sequences and empty halves leave o, dec_o and y unwritten
    # where the separate calls do, and slots outside both halves untouched
    used = [int(s) for s in d["state_indices"] if s >= 0] + [int(s) for s in d["didx"] if s >= 0]
    untouched = np.setdiff1d(np.arange(slots), used)
    assert np.array_equal(t1["st"].cpu().numpy()[untouched], d["state"][untouched])


def test_mixed_call_scale_and_initial_state_reach_both_halves():
    """scale is shared by the two halves; without has_initial_state every
    prefill sequence starts from its slot."""
    d = make_case(73, [129, 64], 9, 2, 4, 128, 16, [1, 1])
    t2 = run_two_calls(d, scale=0.0884, hi=False)
    t1 = run_mixed(d, scale=0.0884, hi=False)
    assert_same(t1, t2)
    HK, HV, dv, B = d["HK"], d["HV"], d["dv"], d["B"]
    o_ref, st_ref = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                            d["state_indices"], d["qsl"], None, 0.0884, True)
    check_bf16(t1["o"], o_ref, "scaled prefill o")
    y_ref, _ = oracle.causal_conv1d_update(d["x"], d["w"], d["b"], d["cs"], d["didx"])
    yb = oracle.round_bf16(y_ref)
    do_ref, _ = oracle.gated_delta_rule(yb[:, :HK * DK].reshape(B, HK, DK), yb[:, HK * DK:2 * HK * DK].reshape(B, HK, DK),
                                        yb[:, 2 * HK * DK:].reshape(B, HV, dv), d["dg"], d["dbeta"], d["state"],
                                        d["didx"], None, None, 0.0884, True)
    check_bf16(t1["do"], do_ref, "scaled decode o")


def test_mixed_call_against_oracle_c32_step():
    d = make_case(72, [635, 637, 747], 29, 16, 32, 128, 64, [1, 0, 1])
    t = run_mixed(d)
    HK, HV, dv, B = d["HK"], d["HV"], d["dv"], d["B"]
    # prefill half
    o_ref, st_ref = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                                            d["state_indices"], d["qsl"], d["has_init"], 1.0, True)
    check_bf16(t["o"], o_ref, "mixed prefill o")
    got = t["st"].cpu().numpy()
    pre, dec = list(d["state_indices"]), list(d["didx"])
    # each half's check takes the other half's slots as the GPU left them
    before = d["state"].copy()
    before[dec] = got[dec]
    check_state(t["st"], st_ref, before, pre, name="mixed prefill state")
    # decode half: fp64 conv update -> bf16 -> fp64 rule
    y_ref, cs_ref = oracle.causal_conv1d_update(d["x"], d["w"], d["b"], d["cs"], d["didx"])
    check_bf16(t["y"], y_ref, "mixed decode y")
    assert np.array_equal(bits(t["cs"]), cs_ref)
    yb = oracle.round_bf16(y_ref)
    do_ref, dst_ref = oracle.gated_delta_rule(yb[:, :HK * DK].reshape(B, HK, DK),
                                              yb[:, HK * DK:2 * HK * DK].reshape(B, HK, DK),
                                              yb[:, 2 * HK * DK:].reshape(B, HV, dv), d["dg"], d["dbeta"],
                                              d["state"], d["didx"], None, None, 1.0, True)
    check_bf16(t["do"], do_ref, "mixed decode o")
    before = d["state"].copy()
    before[pre] = got[pre]
    check_state(t["st"], dst_ref, before, dec, name="mixed decode state", tol=1e-3)
