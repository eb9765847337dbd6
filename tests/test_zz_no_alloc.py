"""The no-allocation entry point (gdn_chunk_rule_and_fused_decode_noalloc,
through the C ABI) against the entry point it varies
(gdn_chunk_rule_and_fused_decode with a caller workspace): bit-identical
results on calls in a row -- the second with a smaller input, so it finds the
first call's records still in the static scratch -- and no device memory
allocated by the call."""
import numpy as np
import pytest
import torch

import gated_deltanet_token_amd as gdn
from parity import bits
from test_gpu_mixed_call import make_case, operands

pytestmark = pytest.mark.gpu


def _call(d, noalloc):
    t = operands(d)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"], t["idx"], t["o"], t["qsl"], t["hi"], t["x"], t["w"], t["b"],
            t["cs"], t["dg"], t["dbeta"], t["didx"], t["do"], t["st"], d["HK"])
    torch.cuda.synchronize()
    if noalloc:
        before = torch.cuda.memory_allocated()
        gdn.gdn_chunk_rule_and_fused_decode_noalloc(*args, dec_y=t["y"])
        assert torch.cuda.memory_allocated() == before
    else:
        gdn.gdn_chunk_rule_and_fused_decode(*args, dec_y=t["y"])
    torch.cuda.synchronize()
    return t


def _same(ref, got, what):
    for n in ("o", "do", "y", "cs"):
        assert np.array_equal(bits(ref[n]), bits(got[n])), "%s: %s differs" % (what, n)
    assert torch.equal(ref["st"].view(torch.int32), got["st"].view(torch.int32)), "%s: state differs" % what


def test_calls_in_a_row_match_the_workspace_call():
    """The c32 mixed step (3 prefill chunks of 2019 tokens, 29 decode rows),
    then a smaller step on the same head shape, then a prefill-only and a
    decode-only step."""
    cases = [("c32 mixed step", make_case(0, [635, 637, 747], 29, 16, 32, 128, 64, [1, 0, 1])),
             ("smaller step", make_case(1, [300, 65], 7, 16, 32, 128, 64, [0, 1])),
             ("prefill only", make_case(2, [130, 1], 0, 16, 32, 128, 64, [1, 1])),
             ("decode only", make_case(3, [], 12, 16, 32, 128, 64, []))]
    for what, d in cases:
        _same(_call(d, False), _call(d, True), what)


def test_refuses_a_prefill_half_larger_than_the_scratch():
    """Three sequences at 16 q/k and 32 v heads with just more tokens than
    the scratch's chunk records cover: refused before anything is enqueued."""
    T = 64
    while gdn.gdn_chunk_workspace_size(3, T, 16, 32) <= gdn.NOALLOC_SCRATCH_BYTES:
        T += 64
    d = make_case(4, [T // 3, T // 3, T - 2 * (T // 3)], 2, 16, 32, 128, 64, [0, 0, 0])
    t = operands(d)
    with pytest.raises(gdn.GDNError) as e:
        gdn.gdn_chunk_rule_and_fused_decode_noalloc(t["q"], t["k"], t["v"], t["g"], t["beta"], t["idx"], t["o"],
                                                    t["qsl"], t["hi"], t["x"], t["w"], t["b"], t["cs"], t["dg"],
                                                    t["dbeta"], t["didx"], t["do"], t["st"], d["HK"])
    assert e.value.code == gdn.GDN_ERR_CAPACITY
    torch.cuda.synchronize()
    assert np.all(bits(t["o"]) == bits(operands(d)["o"]))      # nothing was written
