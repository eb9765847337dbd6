"""GPU parity on the rule's degenerate values, for the chunkwise form, the
token loop and the one-token decode: gates of 0 (no decay) and of -30 and
-100 (the decay factor underflows), beta of 0 (no update) and 1, k rows of
zeros (the normalized key is zero, so only the decay acts) and q rows of
zeros (o is exactly zero).  Same bars as every recurrence test (bf16
outputs; fp32 state within 1e-4 per (slot, head) against the fp64 oracle)."""
import numpy as np
import pytest
import torch

import gated_deltanet_token_amd as gdn
import oracle
import synth
from parity import check_bf16, check_state, dev, sentinel_like

pytestmark = pytest.mark.gpu


def degenerate(d, seed):
    """Plant degenerate values at seeded token positions (per token and head
    for the gates and betas).  A sequence's last token never pairs a gate of
    -100 with no update (beta 0 or a zero key): the exact state would then be
    e^-100 times the old one, below fp32's normal range, where a relative
    state bar means nothing; it gets -30 there instead."""
    r = np.random.default_rng([seed, 7])
    T = d["q"].shape[0]
    g, beta = d["g"].copy(), d["beta"].copy()
    q, k = d["q"].copy(), d["k"].copy()
    for vals, arr in (((0.0, -30.0, -100.0), g), ((0.0, 1.0), beta)):
        for val in vals:
            pick = r.random(arr.shape) < 0.08
            arr[pick] = val
    k[r.random(T) < 0.06] = 0
    q[r.random(T) < 0.06] = 0
    # the first 20 tokens: no decay and no update (the identity step)
    g[: min(T, 20)] = 0.0
    beta[: min(T, 20)] = 0.0
    for t in d["qsl"][1:] - 1:
        frozen = (beta[t] == 0) | (not k[t].any())
        g[t][(g[t] == -100.0) & frozen] = -30.0
    out = dict(d)
    out.update(g=g, beta=beta, q=q, k=k)
    return out


def reference(d, qsl, hi):
    return oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["state_indices"],
                                   qsl, hi, 1.0, True)


def check(o, st, o_ref, st_ref, d, used, name):
    check_bf16(o, o_ref, name + " o")
    check_state(st, st_ref, d["state"], used, name=name + " state")


@pytest.mark.parametrize("path", ["chunk", "token_loop"])
def test_degenerate_values_prefill(path):
    lens = [150, 70, 1]
    d = degenerate(synth.random_gdn(51, 40, lens, 2, 4, 128, 64, num_slots=5, has_init=[1, 0, 1]), 1)
    T = sum(lens)
    o, st = sentinel_like((T, 4, 64)), dev(d["state"])
    args = (dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), dev(d["beta"]), st, dev(d["state_indices"]), o)
    if path == "chunk":
        gdn.gdn_chunk_gated_delta_rule(*args, dev(d["qsl"]), dev(d["has_init"]))
    else:
        gdn.gdn_fused_recurrent_decode(*args, query_start_loc=dev(d["qsl"]), has_initial_state=dev(d["has_init"]))
    torch.cuda.synchronize()
    o_ref, st_ref = reference(d, d["qsl"], d["has_init"])
    check(o, st, o_ref, st_ref, d, [int(s) for s in d["state_indices"]], path)
    # a zero q row gives an exactly zero output
    zq = np.flatnonzero(~d["q"].any(axis=(1, 2)))
    assert zq.size and not o[torch.as_tensor(zq)].float().abs().sum().item()


def test_degenerate_values_decode():
    B = 24
    d = degenerate(synth.random_gdn(52, 41, [1] * B, 4, 8, 128, 128, num_slots=B + 3), 2)
    o, st = sentinel_like((B, 8, 128)), dev(d["state"])
    gdn.gdn_fused_recurrent_decode(dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), dev(d["beta"]), st,
                                   dev(d["state_indices"]), o)
    torch.cuda.synchronize()
    o_ref, st_ref = reference(d, None, None)
    check(o, st, o_ref, st_ref, d, [int(s) for s in d["state_indices"]], "decode")
