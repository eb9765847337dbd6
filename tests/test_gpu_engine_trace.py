"""The c32 engine-step trace at full size, in the launch configuration the
benchmark times: 128 requests x (1024 prompt + 127 decode forwards), at
most 32 running, 2048-token chunked-prefill budget (529 engine steps,
147,328 tokens), 8192 conv channels, 16 q/k and 32 v heads of 128, through
two GDN layers.  Per step: the descriptors are built on the host and
uploaded once, and both layers' varlen convs use that one upload (page
"perf(gdn): dispatch exact causal-conv chunks", section "What changed":
built once per engine step, reused by every layer); then, per layer, the
fused conv update + recurrence for a decode-only step, the chunkwise
recurrence for a prefill-only step, and both in one call
(gdn_chunk_rule_and_fused_decode) for a step with both; each layer carries
its own conv_state and recurrent-state pools (64 slots) and its own
weights and activations.

Checks (the oracle is too slow for the whole trace; it checks sampled
requests end to end):
  * split vs whole on the GPU, per layer: the same requests pushed through
    as whole sequences give bit-identical conv outputs and final
    conv_states, and recurrence outputs / final states within the parity
    bars (the chunkwise form's chunk boundaries move with the split);
  * sampled requests against the oracle's own chain (fp64 conv, bf16
    rounding, fp64 recurrence): in layer 0 the first and the last request
    (the last reuses a freed slot) and two whose prompt is split across two
    engine steps (1022 + 2 and 798 + 226 tokens), and in layer 1 a split
    one and the last one.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_token_amd as gdn
import oracle
import synth
from parity import bits, check_bf16, check_state, dev

pytestmark = pytest.mark.gpu

C, HK, HV, D = synth.C_FULL, synth.HK_FULL, synth.HV_FULL, synth.D_FULL
LAYERS = (0, 1)
# (layer, request): r = 3 and r = 31 prefill across two steps (1022 + 2 and
# 798 + 226 tokens); r = 127 reuses a slot a finished request freed
SAMPLED = ((0, 0), (0, 3), (0, 31), (0, 127), (1, 31), (1, 127))


def _split_requests(tr):
    pieces = {}
    for st in tr.steps:
        for (r, _p0, n, _s, _h) in st.prefills:
            pieces.setdefault(r, []).append(n)
    return {r: v for r, v in pieces.items() if len(v) > 1}


@pytest.fixture(scope="module")
def trace_run():
    torch.cuda.synchronize()
    tr = synth.engine_trace_schedule(0)
    L = tr.seq_len
    rows, offs = synth.trace_step_rows(tr)
    allrows = np.concatenate(rows)
    flat = allrows[:, 0] * L + allrows[:, 1]
    T = len(flat)
    lay = {}
    for li in LAYERS:
        x_req, g_req, b_req = synth.trace_all_inputs(0, li, tr)
        w, b = synth.trace_layer_weights(0, li)
        lay[li] = dict(
            x_req=x_req, g_req=g_req, b_req=b_req, w=w, b=b,
            # step-packed activations (inputs resident on the device)
            X=dev(x_req.reshape(-1, C)[flat]), G=dev(g_req.reshape(-1, HV)[flat]), B=dev(b_req.reshape(-1, HV)[flat]),
            wt=dev(w), bt=dev(b),
            cs=torch.zeros(synth.POOL_SLOTS, 3, C, dtype=torch.bfloat16, device="cuda"),
            st=torch.zeros(synth.POOL_SLOTS, HV, D, D, dtype=torch.float32, device="cuda"),
            Y=torch.empty(T, C, dtype=torch.bfloat16, device="cuda"),
            O=torch.empty(T, HV, D, dtype=torch.bfloat16, device="cuda"),
            final_cs={}, final_st={})
    ws = torch.empty(gdn.gdn_chunk_workspace_size(32, 2048, HK, HV), dtype=torch.uint8, device="cuda")
    uploads = 0
    for si, step in enumerate(tr.steps):
        off, nd = int(offs[si]), len(step.decodes)
        Tn = step.n_tokens
        if nd:
            di = dev(np.array([s for (_r, _p, s) in step.decodes], np.int32))
        if step.prefills:
            lens = [n for (_r, _p, n, _s, _h) in step.prefills]
            qsl = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            qsl_d = dev(qsl)
            pi = dev(np.array([s for (_r, _p, _n, s, _h) in step.prefills], np.int32))
            ph = dev(np.array([h for (_r, _p, _n, _s, h) in step.prefills], np.uint8))
            ch = dev(gdn.gdn_build_conv_chunks(qsl))       # built and uploaded once per step
            uploads += 1
        for li in LAYERS:
            d = lay[li]
            X, G, B, Y, O, cs, st = d["X"], d["G"], d["B"], d["Y"], d["O"], d["cs"], d["st"]
            y = Y[off:off + Tn]
            if step.prefills:
                gdn.gdn_causal_conv1d_varlen(X[off + nd:off + Tn], d["wt"], d["bt"], cs, qsl_d, pi, ph, ch, y[nd:])
            q = y[:, :HK * D].view(Tn, HK, D)
            k = y[:, HK * D:2 * HK * D].view(Tn, HK, D)
            v = y[:, 2 * HK * D:].view(Tn, HV, D)
            if nd and step.prefills:
                gdn.gdn_chunk_rule_and_fused_decode(q[nd:], k[nd:], v[nd:], G[off + nd:off + Tn],
                                                    B[off + nd:off + Tn], pi, O[off + nd:off + Tn], qsl_d, ph,
                                                    X[off:off + nd], d["wt"], d["bt"], cs, G[off:off + nd],
                                                    B[off:off + nd], di, O[off:off + nd], st, HK, dec_y=y[:nd],
                                                    workspace=ws)
            elif nd:
                gdn.gdn_fused_conv_decode(X[off:off + nd], d["wt"], d["bt"], cs, G[off:off + nd], B[off:off + nd],
                                          st, di, O[off:off + nd], HK, D, y=y[:nd])
            else:
                gdn.gdn_chunk_gated_delta_rule(q[nd:], k[nd:], v[nd:], G[off + nd:off + Tn], B[off + nd:off + Tn],
                                               st, pi, O[off + nd:off + Tn], qsl_d, ph, workspace=ws)
            for r in range(tr.n_requests):
                if tr.finish_step[r] == si:
                    slot = tr.slot_of[r]
                    d["final_cs"][r] = cs[slot].clone()
                    d["final_st"][r] = st[slot].clone()
    torch.cuda.synchronize()

    # the same requests as whole sequences (slot r for request r), per layer
    qsl_w = np.arange(tr.n_requests + 1, dtype=np.int32) * L
    idx_w = np.arange(tr.n_requests, dtype=np.int32)
    hi_w = np.zeros(tr.n_requests, np.uint8)
    Tw = tr.n_requests * L
    ch_w = dev(gdn.gdn_build_conv_chunks(qsl_w))
    for li in LAYERS:
        d = lay[li]
        xr = dev(d["x_req"].reshape(-1, C))
        d["cs_w"] = torch.zeros(tr.n_requests, 3, C, dtype=torch.bfloat16, device="cuda")
        d["Yw"] = Yw = torch.empty_like(xr)
        gdn.gdn_causal_conv1d_varlen(xr, d["wt"], d["bt"], d["cs_w"], dev(qsl_w), dev(idx_w), dev(hi_w), ch_w, Yw)
        del xr
        d["st_w"] = torch.zeros(tr.n_requests, HV, D, D, dtype=torch.float32, device="cuda")
        d["Ow"] = torch.empty(Tw, HV, D, dtype=torch.bfloat16, device="cuda")
        gdn.gdn_chunk_gated_delta_rule(Yw[:, :HK * D].view(Tw, HK, D), Yw[:, HK * D:2 * HK * D].view(Tw, HK, D),
                                       Yw[:, 2 * HK * D:].view(Tw, HV, D), dev(d["g_req"].reshape(-1, HV)),
                                       dev(d["b_req"].reshape(-1, HV)), d["st_w"], dev(idx_w), d["Ow"], dev(qsl_w),
                                       dev(hi_w))
        for n in ("X", "G", "B"):
            del d[n]
    torch.cuda.synchronize()
    return dict(tr=tr, lay=lay, flat=torch.from_numpy(flat).cuda(), uploads=uploads)


def test_trace_shape(trace_run):
    tr = trace_run["tr"]
    assert len(tr.steps) == 529 and tr.n_tokens == 147328
    assert max(s.n_tokens for s in tr.steps) == 2048
    assert all(len(s.decodes) + len(s.prefills) <= 32 for s in tr.steps)
    # one descriptor upload per step with prefill rows, shared by both layers
    assert trace_run["uploads"] == sum(1 for s in tr.steps if s.prefills)
    split = _split_requests(tr)
    assert split[3] == [1022, 2] and split[31] == [798, 226]


@pytest.mark.parametrize("li", LAYERS)
def test_conv_split_vs_whole_bit_exact(trace_run, li):
    """Chunked prefill + decode updates give exactly the whole-sequence conv."""
    d = trace_run["lay"][li]
    assert torch.equal(d["Y"].view(torch.int16), d["Yw"][trace_run["flat"]].view(torch.int16))
    for r, cs in d["final_cs"].items():
        assert torch.equal(cs.view(torch.int16), d["cs_w"][r].view(torch.int16)), r
    # the carried window is the last three inputs of the request
    for (l2, r) in SAMPLED:
        if l2 == li:
            assert np.array_equal(bits(d["final_cs"][r]), d["x_req"][r, -3:])


@pytest.mark.parametrize("li", LAYERS)
def test_recurrence_split_vs_whole(trace_run, li):
    d = trace_run["lay"][li]
    o_step = d["O"].float()
    o_whole = d["Ow"][trace_run["flat"]].float()
    diff = (o_step - o_whole).abs()
    rel = float(torch.linalg.vector_norm(o_step - o_whole) / torch.linalg.vector_norm(o_whole))
    assert float(diff.max()) <= 2e-2 and rel < 5e-3, (float(diff.max()), rel)
    print("\n[margin] layer %d trace o step vs whole: max abs %.3g rel L2 %.3g" % (li, float(diff.max()), rel))
    worst = 0.0
    for r, st in d["final_st"].items():
        ref = d["st_w"][r].double()
        num = torch.linalg.vector_norm((st.double() - ref).reshape(HV, -1), dim=1)
        den = torch.linalg.vector_norm(ref.reshape(HV, -1), dim=1)
        worst = max(worst, float((num / den).max()))
    assert worst <= 1e-4, worst
    print("[margin] layer %d trace final state step vs whole: worst rel F %.3g" % (li, worst))


@pytest.mark.parametrize("li,r", SAMPLED)
def test_sampled_request_against_oracle_chain(trace_run, li, r):
    """Request r of layer li end to end through the oracle's own chain: fp64
    conv -> bf16 rounding -> fp64 gated delta rule, from a zero state."""
    d = trace_run["lay"][li]
    tr = trace_run["tr"]
    L = tr.seq_len
    x = d["x_req"][r]
    y_ref, cs_ref = oracle.causal_conv1d_varlen(x, d["w"], d["b"], np.zeros((1, 3, C), np.uint16), [0, L], [0],
                                                 [0])
    yb = oracle.round_bf16(y_ref)
    o_ref, st_ref = oracle.gated_delta_rule(yb[:, :HK * D].reshape(L, HK, D), yb[:, HK * D:2 * HK * D].reshape(L, HK, D),
                                            yb[:, 2 * HK * D:].reshape(L, HV, D), d["g_req"][r], d["b_req"][r],
                                            np.zeros((1, HV, D, D)), [0], [0, L], [0], 1.0, True)
    # this request's rows in the step-packed outputs, in position order
    flat = trace_run["flat"].cpu().numpy()
    pos = np.nonzero(flat // L == r)[0]
    pos = pos[np.argsort(flat[pos] % L)]
    ey = check_bf16(d["Y"][torch.from_numpy(pos).cuda()], y_ref, "layer %d trace conv y, request %d" % (li, r))
    eo = check_bf16(d["O"][torch.from_numpy(pos).cuda()], o_ref, "layer %d trace o, request %d" % (li, r))
    assert np.array_equal(bits(d["final_cs"][r]), cs_ref[0])
    # the recurrence consumes the GPU's own bf16 conv outputs while the oracle
    # consumes its own rounding of the fp64 conv: where the two roundings
    # differ by one bf16 ulp the inputs differ, so the state bar here is the
    # chained one (1e-3), not the 1e-4 of identical inputs
    es = check_state(d["final_st"][r].unsqueeze(0), st_ref, np.zeros((1, HV, D, D), np.float32), [0],
                     name="layer %d trace final state, request %d" % (li, r), tol=1e-3)
    print("\n[margin] layer %d request %d vs oracle chain: y max %.3g rel %.3g; o max %.3g rel %.3g; "
          "state rel F %.3g" % (li, r, ey[0], ey[1], eo[0], eo[1], es))
