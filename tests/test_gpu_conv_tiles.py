"""GPU checks of the 16-token conv programs (gdn_causal_conv1d_varlen_tiles
with two descriptors per program): bit-identical to the 8-token programs of
gdn_causal_conv1d_varlen on every case -- contiguous pairs (the second
descriptor's halo taken from the first's rows), pairs that straddle two
sequences, a last unpaired descriptor, padding, stray descriptors, mixed
initial states, strided rows -- and against the oracle on two of them."""
import numpy as np
import pytest
import torch

import gated_deltanet_token_amd as gdn
import oracle
import synth
from parity import SENTINEL, bits, check_bf16, dev, sentinel_like

pytestmark = pytest.mark.gpu


def _run(d, x, idx, hi, bias, silu, dpp, chunks=None, y_pad=0):
    T, C = x.shape
    yw = sentinel_like((T, C + 2 * y_pad))
    y = yw[:, y_pad:y_pad + C] if y_pad else yw
    cs = dev(d["conv_state"])
    ch = gdn.gdn_build_conv_chunks(d["qsl"]) if chunks is None else chunks
    gdn.gdn_causal_conv1d_varlen(x, dev(d["weight"]), None if bias is None else dev(bias), cs, dev(d["qsl"]),
                                 dev(idx), None if hi is None else dev(hi), dev(ch), y, silu=silu,
                                 descriptors_per_program=dpp)
    torch.cuda.synchronize()
    return yw, cs


CASES = [
    # lens, channels, has_init, padding mask, silu
    ([1], 8, [1], None, True),
    ([5, 13], 64, [0, 1], None, True),                    # 3 descriptors: one pair straddles, one alone
    ([16, 8, 24, 9, 7], 2056, [1, 0, 1, 1, 0], None, False),
    ([0, 1, 2, 3, 4, 7, 8, 9, 15, 16, 17, 31], 2056, None, None, True),
    ([33, 0, 21, 9], 4104, [1, 0, 1, 1], [False, False, True, False], True),
    ([1024, 1024], 8192, [0, 0], None, True),            # the c32 prefill shape
    ([635, 637, 747], 8192, [0, 0, 1], None, True),      # the c32 mixed step's prefill rows
]


@pytest.mark.parametrize("lens,C,hi,pad,silu", CASES)
def test_tiles_bit_identical_to_8_token_programs(lens, C, hi, pad, silu):
    d = synth.random_conv(31, 40 + len(lens), lens, C, num_slots=len(lens) + 2, has_init=hi)
    idx = d["state_indices"].copy()
    if pad is not None:
        idx[np.array(pad)] = -1
    x = dev(d["x"])
    hi_arr = d["has_init"] if hi is not None else None
    y1, cs1 = _run(d, x, idx, hi_arr, d["bias"], silu, 1, y_pad=8)
    y2, cs2 = _run(d, x, idx, hi_arr, d["bias"], silu, 2, y_pad=8)
    assert np.array_equal(bits(y1), bits(y2)), "16-token programs differ from 8-token programs"
    assert np.array_equal(bits(cs1), bits(cs2))
    b = bits(y2)
    assert np.all(b[:, :8] == SENTINEL) and np.all(b[:, 8 + C:] == SENTINEL)


@pytest.mark.parametrize("lens,C", [([5, 13, 64, 3], 2056), ([635, 637, 747], 8192)])
def test_tiles_against_oracle(lens, C):
    d = synth.random_conv(32, 50, lens, C, num_slots=len(lens) + 1, has_init=[(i + 1) % 2 for i in range(len(lens))])
    y, cs = _run(d, dev(d["x"]), d["state_indices"], d["has_init"], d["bias"], True, 2)
    y_ref, cs_ref = oracle.causal_conv1d_varlen(d["x"], d["weight"], d["bias"], d["conv_state"], d["qsl"],
                                                d["state_indices"], d["has_init"])
    check_bf16(y, y_ref, "16-token conv y")
    assert np.array_equal(bits(cs), cs_ref)


def test_tiles_stray_descriptors_and_out_of_pool_slot():
    """Descriptors naming no sequence, or chunks past a sequence's end, are
    skipped in either position of a pair; a slot past the pool too."""
    d = synth.random_conv(33, 51, [20, 13, 9], C=64, num_slots=4, has_init=[1, 0, 1])
    idx = np.array([7, 1, 2], np.int32)                 # sequence 0: past the 4-slot pool
    ch = gdn.gdn_build_conv_chunks(d["qsl"])
    stray = np.array([[3, 0], [5, 1], [-1, 0], [1, 99], [0, -2]], np.int32)
    chs = np.concatenate([ch[:2], stray, ch[2:]])
    x = dev(d["x"])
    y1, cs1 = _run(d, x, idx, d["has_init"], d["bias"], True, 1, chunks=chs)
    y2, cs2 = _run(d, x, idx, d["has_init"], d["bias"], True, 2, chunks=chs)
    assert np.array_equal(bits(y1), bits(y2))
    assert np.array_equal(bits(cs1), bits(cs2))
    pidx = idx.copy()
    pidx[pidx >= 4] = -1
    y_ref, cs_ref = oracle.causal_conv1d_varlen(d["x"], d["weight"], d["bias"], d["conv_state"], d["qsl"], pidx,
                                                d["has_init"])
    check_bf16(y2, y_ref, "16-token guarded conv y")
    assert np.array_equal(bits(cs2), cs_ref)
