"""GPU parity of the chunkwise gated delta rule (gdn_chunk_gated_delta_rule)
against the fp64 oracle: the same bars as the per-token kernel (bf16
outputs, fp32 state within 1e-4 per (slot, head)), on the mixed-step prefill
chunks, full c32 requests, and ragged lengths around the 64-token chunk."""
import numpy as np
import pytest
import torch

import gated_deltanet_token_amd as gdn
import oracle
import synth
from parity import bits, check_bf16, check_state, dev, sentinel_like

pytestmark = pytest.mark.gpu


def run_chunk(d, idx=None, hi="default", scale=1.0, norm=True, views=False):
    idx = d["state_indices"] if idx is None else idx
    hi = d["has_init"] if isinstance(hi, str) else hi
    T = d["q"].shape[0]
    HK, HV, dk, dv_ = d["HK"], d["HV"], d["dk"], d["dv"]
    if views:
        wq, wv = HK * dk, HV * dv_
        row = np.zeros((T, 2 * wq + wv + 8), np.uint16)
        row[:, :wq] = d["q"].reshape(T, wq)
        row[:, wq:2 * wq] = d["k"].reshape(T, wq)
        row[:, 2 * wq + 8:] = d["v"].reshape(T, wv)
        rt = dev(row)
        q, k = rt[:, :wq].view(T, HK, dk), rt[:, wq:2 * wq].view(T, HK, dk)
        v = rt[:, 2 * wq + 8:].view(T, HV, dv_)
    else:
        q, k, v = dev(d["q"]), dev(d["k"]), dev(d["v"])
    o = sentinel_like((T, HV, dv_))
    st = dev(d["state"])
    gdn.gdn_chunk_gated_delta_rule(q, k, v, dev(d["g"]), dev(d["beta"]), st, dev(idx), o, dev(d["qsl"]),
                                   None if hi is None else dev(hi), scale, norm)
    torch.cuda.synchronize()
    o_ref, st_ref = oracle.gated_delta_rule(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], idx,
                                            d["qsl"], hi, scale, norm)
    return o, st, o_ref, st_ref


def test_mixed_step_prefill_chunks():
    d = synth.mixed_step(0, with_recurrence=True)
    nd = d["n_dec"]
    sub = dict(HK=d["HK"], HV=d["HV"], dk=d["dk"], dv=d["dv"], qsl=d["qsl"], state_indices=d["state_indices"],
               has_init=d["has_init"], q=d["q"][nd:], k=d["k"][nd:], v=d["v"][nd:], g=d["g"][nd:],
               beta=d["beta"][nd:], state=d["state"])
    o, st, o_ref, st_ref = run_chunk(sub)
    check_bf16(o, o_ref, "chunk mixed-step o")
    check_state(st, st_ref, d["state"], d["state_indices"])


@pytest.mark.parametrize("lens,HK,HV,dv_,hi,pad", [
    ([1], 1, 1, 32, [1], None),
    ([63, 64, 65], 2, 4, 128, [1, 0, 1], None),
    ([127, 0, 128, 129], 2, 2, 64, [0, 1, 1, 0], [False, False, True, False]),
    ([200, 5], 1, 2, 256, None, None),
    ([70, 33], 4, 8, 96, [1, 1], [True, False]),
    # three v-heads per q/k head: one v-head per prep workgroup, K^T written
    # by the first of each three
    ([90, 40, 64], 2, 6, 64, [0, 1, 1], None),
    # four v-heads per q/k head: two pair workgroups per q/k head, K^T written
    # by the first
    ([129, 64, 3], 2, 8, 64, [1, 0, 1], [False, True, False]),
])
@pytest.mark.parametrize("scale,norm,views", [(1.0, True, False), (0.0884, True, True)])
def test_chunk_edges(lens, HK, HV, dv_, hi, pad, scale, norm, views):
    S = len(lens)
    d = synth.random_gdn(31, 90 + S, lens, HK, HV, 128, dv_, num_slots=S + 2, has_init=hi)
    idx = d["state_indices"].copy()
    if pad is not None:
        idx[np.array(pad)] = -1
    o, st, o_ref, st_ref = run_chunk(d, idx=idx, hi=d["has_init"] if hi else None, scale=scale, norm=norm,
                                     views=views)
    check_bf16(o, o_ref, "chunk edge o")
    used = [int(idx[s]) for s in range(S) if lens[s] > 0 and idx[s] >= 0]
    check_state(st, st_ref, d["state"], used)


def test_full_requests_from_zero_state():
    """Two c32 requests end to end (1151 tokens each, q/k/v drawn directly),
    state from zero, 16 q/k and 32 v heads of 128."""
    d = synth.random_gdn(32, 99, [1151, 1151], 16, 32, 128, 128, num_slots=4, has_init=[0, 0])
    o, st, o_ref, st_ref = run_chunk(d)
    check_bf16(o, o_ref, "chunk full-request o")
    check_state(st, st_ref, d["state"], d["state_indices"])


def test_chunk_agrees_with_token_by_token_kernel():
    d = synth.random_gdn(33, 98, [300, 77], 16, 32, 128, 128, num_slots=3, has_init=[1, 0])
    o_c, st_c, o_ref, st_ref = run_chunk(d)
    o_f = sentinel_like(o_c.shape)
    st_f = dev(d["state"])
    gdn.gdn_fused_recurrent_decode(dev(d["q"]), dev(d["k"]), dev(d["v"]), dev(d["g"]), dev(d["beta"]), st_f,
                                   dev(d["state_indices"]), o_f, dev(d["qsl"]), dev(d["has_init"]))
    torch.cuda.synchronize()
    check_bf16(o_c, o_ref, "chunk o")
    check_bf16(o_f, o_ref, "token-by-token o")
    check_state(st_c, st_ref, d["state"], d["state_indices"])
    check_state(st_f, st_ref, d["state"], d["state_indices"])


def test_chunk_split_vs_whole_within_rounding():
    """Splitting a sequence across calls moves the chunk boundaries: the
    results agree with one pass (and with the oracle) to fp32 rounding."""
    L = 400
    d = synth.random_gdn(34, 97, [L], 16, 32, 128, 128, num_slots=2, state_indices=[1], has_init=[1])
    o_w, st_w, o_ref, st_ref = run_chunk(d)
    st = dev(d["state"])
    o = sentinel_like((L, 32, 128))
    q, k, v, g, b = (dev(d[n]) for n in ("q", "k", "v", "g", "beta"))
    pos = 0
    for n in (100, 1, 64, 170, 65):
        sl = slice(pos, pos + n)
        gdn.gdn_chunk_gated_delta_rule(q[sl], k[sl], v[sl], g[sl].contiguous(), b[sl].contiguous(), st,
                                       dev(d["state_indices"]), o[sl], dev(np.array([0, n], np.int32)))
        pos += n
    assert pos == L
    torch.cuda.synchronize()
    check_bf16(o, o_ref, "chunk split o")
    check_state(st, st_ref, d["state"], d["state_indices"])
    diff = np.abs(o.float().cpu().numpy() - o_w.float().cpu().numpy()).max()
    assert diff <= 2e-2, diff


@pytest.mark.parametrize("lens,HK,HV,dv_,hi,pad", [
    # 64-row workgroups (head_v_dim a multiple of 64): one per (sequence, head)
    # at dv 64, four per head at dv 256; dv 32 and 96 elsewhere take the
    # 32-row form
    ([0, 1, 63, 64, 65, 100, 17, 128, 30], 16, 32, 64, [1, 0, 1, 1, 0, 1, 0, 1, 1],
     [False] * 7 + [True, False]),
    # 3 sequences with 256-row heads: four 64-row workgroups per head
    ([70, 65, 129], 16, 32, 256, [0, 1, 1], None),
])
def test_chunk_wide_workgroups(lens, HK, HV, dv_, hi, pad):
    S = len(lens)
    d = synth.random_gdn(35, 80 + S, lens, HK, HV, 128, dv_, num_slots=S + 2, has_init=hi)
    idx = d["state_indices"].copy()
    if pad is not None:
        idx[np.array(pad)] = -1
    o, st, o_ref, st_ref = run_chunk(d, idx=idx)
    check_bf16(o, o_ref, "chunk wide o")
    used = [int(idx[s]) for s in range(S) if lens[s] > 0 and idx[s] >= 0]
    check_state(st, st_ref, d["state"], used)


def test_chunk_many_sequences():
    """More than 64 sequences (empty ones and a padded one among them): the
    chunk -> sequence lookup and the first-chunk offset walk the sequences 64
    at a time."""
    lens = [(i * 37) % 45 for i in range(70)]
    lens[5] = 130
    S = len(lens)
    hi = [i % 3 != 0 for i in range(S)]
    d = synth.random_gdn(36, 77, lens, 2, 4, 128, 64, num_slots=S + 2, has_init=hi)
    idx = d["state_indices"].copy()
    idx[66] = -1
    o, st, o_ref, st_ref = run_chunk(d, idx=idx)
    check_bf16(o, o_ref, "chunk many-sequence o")
    used = [int(idx[s]) for s in range(S) if lens[s] > 0 and idx[s] >= 0]
    check_state(st, st_ref, d["state"], used)


def test_chunk_long_sequence():
    """One 8,001-token sequence (126 chunks in series, the last holding one
    token) next to a short one: the state is carried through every chunk
    boundary, and chunk indices run past a hundred."""
    lens = [8001, 37]
    d = synth.random_gdn(37, 78, lens, 2, 4, 128, 64, num_slots=4, has_init=[1, 0])
    o, st, o_ref, st_ref = run_chunk(d)
    check_bf16(o, o_ref, "chunk long-sequence o")
    check_state(st, st_ref, d["state"], [int(s) for s in d["state_indices"]])


def test_chunk_many_short_sequences_several_rounds():
    """32 sequences of 64 tokens at the c32 head shape (2,048 tokens): 2,048
    scan workgroups, several rounds on 256 CUs, and 1,024 prep workgroups."""
    lens = [64] * 32
    hi = [i % 2 == 0 for i in range(32)]
    d = synth.random_gdn(38, 79, lens, 16, 32, 128, 128, num_slots=64, has_init=hi)
    o, st, o_ref, st_ref = run_chunk(d)
    check_bf16(o, o_ref, "chunk 32 x 64 o")
    check_state(st, st_ref, d["state"], [int(s) for s in d["state_indices"]])


def test_side_stream_without_workspace():
    """The call on a side stream, its workspace allocated by the binding: the
    block must stay reserved for that stream's kernels.  The current stream
    meanwhile allocates a same-size buffer and overwrites it again and again
    while the side stream's kernels run (they start behind a sleep); if the
    workspace's memory had been handed out again, the scan would read the
    overwritten records.  Outputs must equal a call on the current stream
    bit for bit."""
    d = synth.mixed_step(0, with_recurrence=True)
    nd = d["n_dec"]
    q, k, v = dev(d["q"][nd:]), dev(d["k"][nd:]), dev(d["v"][nd:])
    g, b = dev(d["g"][nd:]), dev(d["beta"][nd:])
    idx, qsl, hi = dev(d["state_indices"]), dev(d["qsl"]), dev(d["has_init"])
    T, HV, dv_ = q.shape[0], d["HV"], d["dv"]
    o_ref, st_ref = sentinel_like((T, HV, dv_)), dev(d["state"])
    gdn.gdn_chunk_gated_delta_rule(q, k, v, g, b, st_ref, idx, o_ref, qsl, hi)
    torch.cuda.synchronize()
    need = gdn.gdn_chunk_workspace_size(len(d["state_indices"]), T, d["HK"], HV)
    o, st = sentinel_like((T, HV, dv_)), dev(d["state"])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        torch.cuda._sleep(20_000_000)
    gdn.gdn_chunk_gated_delta_rule(q, k, v, g, b, st, idx, o, qsl, hi, stream=side)
    junk = torch.empty(need, dtype=torch.uint8, device="cuda")
    for i in range(300):
        junk.fill_(i & 255)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), bits(o_ref))
    assert torch.equal(st.view(torch.int32), st_ref.view(torch.int32))
