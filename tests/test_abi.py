"""CPU checks of the C-ABI library: it loads, exports every call declared
in include/gdn.h, builds chunk descriptors bit-exactly like the oracle, and
rejects each invalid argument with its documented status before touching
the GPU (no compute call is made here)."""
import ctypes
import os
import re

import numpy as np
import pytest

import gated_deltanet_token_amd as gdn
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INV, UNS, CAP = gdn.GDN_ERR_INVALID, gdn.GDN_ERR_UNSUPPORTED, gdn.GDN_ERR_CAPACITY


def declared_calls():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_call():
    names = declared_calls()
    assert set(names) == set(gdn.EXPORTS)
    for n in names:
        assert hasattr(gdn.lib, n), n


def _chunks_lib(qsl, capacity):
    qsl = np.ascontiguousarray(qsl, np.int32)
    out = (gdn_conv_chunk * max(capacity, 1))()
    n = ctypes.c_int32(-1)
    rc = gdn.lib.gdn_build_conv_chunks(qsl.ctypes.data, qsl.size - 1, out, capacity, ctypes.byref(n))
    return rc, n.value, np.array([(c.seq, c.chunk) for c in out[:min(capacity, max(n.value, 0))]],
                                 np.int32).reshape(-1, 2)


class gdn_conv_chunk(ctypes.Structure):
    _fields_ = [("seq", ctypes.c_int32), ("chunk", ctypes.c_int32)]


def test_chunks_bit_exact_vs_oracle_random_and_edges():
    r = np.random.default_rng(7)
    cases = [[0], [0, 0], [0, 5, 18], [0, 1024, 2048], [0, 8, 16, 24], [0, 7, 7, 15, 16, 17]]
    for _ in range(300):
        S = int(r.integers(1, 40))
        lens = r.integers(0, 40, S) * (r.random(S) < 0.9)
        cases.append(np.concatenate([[0], np.cumsum(lens)]).tolist())
    for qsl in cases:
        ref = oracle.build_conv_chunks(qsl)
        got = gdn.gdn_build_conv_chunks(qsl)
        assert got.dtype == np.int32 and np.array_equal(got, ref), qsl


def test_chunks_capacity_and_errors():
    rc, n, got = _chunks_lib([0, 9, 9, 30], 2)
    assert rc == CAP and n == 5 and np.array_equal(got, [[0, 0], [0, 1]])
    rc, n, _ = _chunks_lib([0, 9, 9, 30], 0)
    assert rc == CAP and n == 5
    rc, n, got = _chunks_lib([0, 9, 9, 30], 5)
    assert rc == 0 and n == 5
    rc, _, _ = _chunks_lib([0, 5, 3], 10)
    assert rc == INV and b"decreases" in gdn.lib.gdn_last_error()
    n = ctypes.c_int32()
    assert gdn.lib.gdn_build_conv_chunks(None, 1, None, 0, ctypes.byref(n)) == INV
    q = np.array([0, 1], np.int32)
    assert gdn.lib.gdn_build_conv_chunks(q.ctypes.data, -1, None, 0, ctypes.byref(n)) == INV
    assert gdn.lib.gdn_build_conv_chunks(q.ctypes.data, 1, None, 4, ctypes.byref(n)) == INV


# fake, well-aligned device addresses: validation never dereferences them and
# every case below fails validation, so nothing is launched
A = 0x10000000
X, W, B, CS, QSL, IDX, HI, CH, Y = (A + i * 0x1000000 for i in range(9))


def varlen(**kw):
    a = dict(x=X, xs=8192, w=W, b=B, cs=CS, slots=64, qsl=QSL, idx=IDX, hi=HI, ch=CH, nch=256,
             y=Y, ys=8192, S=2, T=2048, C=8192, K=4, silu=1)
    a.update(kw)
    return gdn.lib.gdn_causal_conv1d_varlen(a["x"], a["xs"], a["w"], a["b"], a["cs"], a["slots"], a["qsl"],
                                            a["idx"], a["hi"], a["ch"], a["nch"], a["y"], a["ys"], a["S"],
                                            a["T"], a["C"], a["K"], a["silu"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), INV), (dict(w=None), INV), (dict(cs=None), INV), (dict(y=None), INV),
    (dict(qsl=None), INV), (dict(idx=None), INV),
    (dict(ch=None), INV),                        # pair mismatch: count without buffer
    (dict(nch=0), INV),                          # pair mismatch: buffer without count
    (dict(nch=-1), INV), (dict(S=-1), INV), (dict(T=-1), INV), (dict(slots=0), INV),
    (dict(xs=8000), INV), (dict(ys=100), INV), (dict(y=X), INV), (dict(y=X + 2 * 8192), INV),
    (dict(y=CS), INV), (dict(y=W, x=Y), INV), (dict(y=B), INV),     # y over conv_state, weight, bias
    (dict(nch=3000), INV), (dict(S=0), INV),
    (dict(ch=None, nch=0), INV),                 # tokens but no descriptors: nothing would run
    (dict(nch=255), INV),                        # 255 descriptors cannot cover 2048 tokens
    (dict(nch=1, T=9, S=1), INV),                # nor one descriptor 9 tokens
    (dict(K=3), UNS), (dict(K=5), UNS), (dict(C=8190, xs=8190, ys=8190), UNS),
    (dict(xs=8196), UNS), (dict(x=X + 2), UNS), (dict(b=B + 8), UNS), (dict(cs=CS + 4), UNS),
])
def test_conv_varlen_validation(kw, code):
    assert varlen(**kw) == code, gdn.lib.gdn_last_error()
    assert gdn.lib.gdn_last_error()


def test_conv_varlen_without_tokens_or_descriptors_is_a_no_op():
    """No tokens and no descriptors: valid, and nothing is enqueued (the
    fake device addresses are never touched)."""
    assert varlen(ch=None, nch=0, T=0) == gdn.GDN_OK, gdn.lib.gdn_last_error()
    assert varlen(ch=None, nch=0, T=0, S=0) == gdn.GDN_OK


def varlen_tiles(dpp, **kw):
    a = dict(x=X, xs=8192, w=W, b=B, cs=CS, slots=64, qsl=QSL, idx=IDX, hi=HI, ch=CH, nch=256,
             y=Y, ys=8192, S=2, T=2048, C=8192, K=4, silu=1)
    a.update(kw)
    return gdn.lib.gdn_causal_conv1d_varlen_tiles(a["x"], a["xs"], a["w"], a["b"], a["cs"], a["slots"], a["qsl"],
                                                  a["idx"], a["hi"], a["ch"], a["nch"], a["y"], a["ys"], a["S"],
                                                  a["T"], a["C"], a["K"], a["silu"], dpp, None)


@pytest.mark.parametrize("dpp,kw,code", [
    (0, {}, UNS), (3, {}, UNS), (-1, {}, UNS),
    (2, dict(x=None), INV), (2, dict(nch=255), INV), (1, dict(ch=None, nch=0), INV),
    # strides past 2^26 (x or y placed far apart, so they do not overlap)
    (2, dict(xs=(1 << 26) + 8, y=1 << 44), UNS), (2, dict(ys=(1 << 26) + 8, y=1 << 44), UNS),
])
def test_conv_varlen_tiles_validation(dpp, kw, code):
    assert varlen_tiles(dpp, **kw) == code, gdn.lib.gdn_last_error()
    assert gdn.lib.gdn_last_error()


def test_conv_varlen_tiles_without_tokens_is_a_no_op():
    assert varlen_tiles(2, ch=None, nch=0, T=0) == gdn.GDN_OK, gdn.lib.gdn_last_error()


def update(**kw):
    a = dict(x=X, xs=8192, w=W, b=B, cs=CS, slots=64, idx=IDX, y=Y, ys=8192, B=32, C=8192, K=4, silu=1)
    a.update(kw)
    return gdn.lib.gdn_causal_conv1d_update(a["x"], a["xs"], a["w"], a["b"], a["cs"], a["slots"], a["idx"],
                                            a["y"], a["ys"], a["B"], a["C"], a["K"], a["silu"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), INV), (dict(idx=None), INV), (dict(B=-1), INV), (dict(y=X), INV), (dict(y=CS), INV),
    (dict(slots=0), INV), (dict(K=2), UNS), (dict(C=12, xs=16, ys=16), UNS), (dict(y=Y + 6), UNS),
])
def test_conv_update_validation(kw, code):
    assert update(**kw) == code, gdn.lib.gdn_last_error()


# 256 MiB apart, after the conv buffers: the 64-slot state pool alone spans 128 MiB
Q, K_, V, G, BE, ST, O = (A + (i + 1) * 0x10000000 for i in range(7))


def rec(**kw):
    a = dict(q=Q, qs=2048, k=K_, ks=2048, v=V, vs=4096, g=G, b=BE, st=ST, slots=64, qsl=None, idx=IDX,
             hi=None, o=O, os=4096, S=32, T=32, HK=16, HV=32, dk=128, dv=128, scale=1.0, norm=1)
    a.update(kw)
    return gdn.lib.gdn_fused_recurrent_decode(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"],
                                              a["b"], a["st"], a["slots"], a["qsl"], a["idx"], a["hi"],
                                              a["o"], a["os"], a["S"], a["T"], a["HK"], a["HV"], a["dk"],
                                              a["dv"], a["scale"], a["norm"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INV), (dict(k=None), INV), (dict(v=None), INV), (dict(g=None), INV),
    (dict(b=None), INV), (dict(st=None), INV), (dict(idx=None), INV), (dict(o=None), INV),
    (dict(S=-1), INV), (dict(T=-2), INV), (dict(slots=0), INV), (dict(HV=24), INV), (dict(HK=0), INV),
    (dict(qs=2000), INV), (dict(vs=4000), INV), (dict(os=1024), INV),
    (dict(T=33), INV),                           # one token per sequence without qsl
    (dict(o=V), INV),                            # o overlaps v
    (dict(o=ST + 0x10000), INV), (dict(o=G), INV), (dict(o=BE), INV),   # o over the state, g, beta
    (dict(dk=96), UNS), (dict(dk=256), UNS), (dict(dv=100), UNS), (dict(dv=512), UNS),
    (dict(qs=2052), UNS), (dict(q=Q + 8), UNS), (dict(st=ST + 4), UNS),
])
def test_recurrent_validation(kw, code):
    assert rec(**kw) == code, gdn.lib.gdn_last_error()


def test_error_text_cleared_on_success():
    varlen(K=3)
    assert gdn.lib.gdn_last_error()
    gdn.gdn_build_conv_chunks([0, 4])
    assert gdn.lib.gdn_last_error() == b""


WS = A + 0x80000000
WS_NEED = gdn.gdn_chunk_workspace_size(3, 2019, 16, 32)


def chunk(**kw):
    a = dict(q=Q, qs=2048, k=K_, ks=2048, v=V, vs=4096, g=G, b=BE, st=ST, slots=64, qsl=QSL, idx=IDX,
             hi=None, o=O, os=4096, S=3, T=2019, HK=16, HV=32, dk=128, dv=128, ws=WS, wsb=WS_NEED,
             scale=1.0, norm=1)
    a.update(kw)
    return gdn.lib.gdn_chunk_gated_delta_rule(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"],
                                              a["b"], a["st"], a["slots"], a["qsl"], a["idx"], a["hi"],
                                              a["o"], a["os"], a["S"], a["T"], a["HK"], a["HV"], a["dk"],
                                              a["dv"], a["ws"], a["wsb"], a["scale"], a["norm"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(qsl=None), INV), (dict(q=None), INV), (dict(HV=24), INV), (dict(o=V), INV),
    (dict(dk=64), UNS), (dict(dk=16), UNS), (dict(dv=48), UNS), (dict(dv=512), UNS), (dict(q=Q + 8), UNS),
    (dict(ws=None), INV), (dict(ws=WS + 128), UNS), (dict(wsb=WS_NEED - 1), CAP),
    (dict(os=1 << 24), UNS),     # 32-bit byte offsets within a 64-token chunk
    # a workspace over an operand: o, the state pool, q
    (dict(ws=O), INV), (dict(ws=ST + 0x100000), INV), (dict(ws=Q), INV),
])
def test_chunk_validation(kw, code):
    assert chunk(**kw) == code, gdn.lib.gdn_last_error()


def test_chunk_workspace_size_formula():
    # per (64-token chunk, v-head): T and P as hi/lo bf16, the ten 16 x 16
    # blocks of each lower-triangular 64 x 64 matrix (4 x 10 x 512 B), + 5 x 64
    # fp32 factors; chunks bounded by ceil(T / 64) + S
    for S, T, HK, HV in ((3, 2019, 16, 32), (1, 1, 1, 1), (2, 2048, 16, 32), (0, 0, 16, 32)):
        mc = (T + 63) // 64 + S
        assert gdn.gdn_chunk_workspace_size(S, T, HK, HV) == mc * HV * (4 * 10 * 512 + 5 * 256)


def fused(**kw):
    a = dict(x=X, xs=8192, w=W, b=B, cs=CS, cslots=64, g=G, be=BE, st=ST, slots=64, idx=IDX, o=O, os=4096,
             y=None, ys=0, B=32, HK=16, HV=32, dk=128, dv=128, silu=1, scale=1.0, norm=1)
    a.update(kw)
    return gdn.lib.gdn_fused_conv_decode(a["x"], a["xs"], a["w"], a["b"], a["cs"], a["cslots"], a["g"], a["be"],
                                         a["st"], a["slots"], a["idx"], a["o"], a["os"], a["y"], a["ys"], a["B"],
                                         a["HK"], a["HV"], a["dk"], a["dv"], a["silu"], a["scale"], a["norm"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), INV), (dict(w=None), INV), (dict(cs=None), INV), (dict(g=None), INV), (dict(st=None), INV),
    (dict(idx=None), INV), (dict(o=None), INV), (dict(B=-1), INV), (dict(cslots=0), INV), (dict(slots=0), INV),
    (dict(HV=24), INV), (dict(xs=8000), INV), (dict(os=1000), INV), (dict(o=X), INV),
    (dict(y=Y, ys=100), INV), (dict(y=X, ys=8192), INV),
    (dict(o=ST), INV), (dict(o=CS), INV), (dict(o=G), INV), (dict(o=BE), INV),
    (dict(y=CS, ys=8192), INV), (dict(y=ST, ys=8192), INV),
    (dict(dk=96), UNS), (dict(dv=12), UNS), (dict(xs=8196), UNS), (dict(x=X + 4), UNS), (dict(y=Y + 2, ys=8192), UNS),
    (dict(HK=1, HV=64, dk=128, dv=128, xs=8448), UNS),   # one q/k group reads > 8192 channels
])
def test_fused_validation(kw, code):
    assert fused(**kw) == code, gdn.lib.gdn_last_error()


# the decode half's own g, beta, o and slots, past the workspace
DG, DBE, DO, DIDX = (A + 0x90000000 + i * 0x1000000 for i in range(4))


def mixed(**kw):
    a = dict(q=Q, qs=2048, k=K_, ks=2048, v=V, vs=4096, g=G, b=BE, qsl=QSL, idx=IDX, hi=None, o=O, os=4096,
             S=3, T=2019, ws=WS, wsb=WS_NEED,
             x=X, xs=8192, w=W, bias=B, cs=CS, cslots=64, dg=DG, dbe=DBE, didx=DIDX, do=DO, dos=4096,
             y=None, ys=0, B=32, silu=1,
             st=ST, slots=64, HK=16, HV=32, dk=128, dv=128, scale=1.0, norm=1)
    a.update(kw)
    return gdn.lib.gdn_chunk_rule_and_fused_decode(
        a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"], a["b"], a["qsl"], a["idx"], a["hi"], a["o"],
        a["os"], a["S"], a["T"], a["ws"], a["wsb"],
        a["x"], a["xs"], a["w"], a["bias"], a["cs"], a["cslots"], a["dg"], a["dbe"], a["didx"], a["do"], a["dos"],
        a["y"], a["ys"], a["B"], a["silu"],
        a["st"], a["slots"], a["HK"], a["HV"], a["dk"], a["dv"], a["scale"], a["norm"], None)


@pytest.mark.parametrize("kw,code", [
    # each half's own checks
    (dict(qsl=None), INV), (dict(q=None), INV), (dict(o=V), INV), (dict(wsb=WS_NEED - 1), CAP),
    (dict(ws=WS + 128), UNS), (dict(dk=64), UNS), (dict(dv=48), UNS),
    (dict(x=None), INV), (dict(cslots=0), INV), (dict(B=-1), INV), (dict(do=ST), INV), (dict(do=CS), INV),
    (dict(xs=8196), UNS),
    # what one half writes over the other half's operands
    (dict(o=X), INV), (dict(o=W), INV), (dict(o=DG), INV), (dict(o=DBE), INV), (dict(o=DO), INV),
    (dict(o=CS + 0x1000), INV),
    (dict(ws=X), INV), (dict(ws=CS), INV), (dict(ws=DBE), INV), (dict(ws=DO), INV),
    (dict(do=Q), INV), (dict(do=V + 0x100), INV), (dict(do=G), INV), (dict(do=O), INV),
    (dict(y=BE, ys=8192), INV), (dict(y=K_, ys=8192), INV),
    (dict(cs=V), INV), (dict(cs=Q), INV), (dict(cs=G), INV),
])
def test_mixed_validation(kw, code):
    assert mixed(**kw) == code, gdn.lib.gdn_last_error()


def test_mixed_both_halves_empty_enqueue_nothing():
    # nothing to launch: returns GDN_OK without touching a device, and an
    # empty half's operands overlap nothing
    assert mixed(S=0, T=0, B=0) == gdn.GDN_OK
    assert gdn.lib.gdn_last_error() == b""
    assert mixed(S=0, T=0, B=0, do=Q, o=X) == gdn.GDN_OK
    assert mixed(S=0, T=0, B=0, q=None, o=None, ws=None, x=None, do=None, st=None) == gdn.GDN_OK
    assert mixed(S=0, T=-1, B=0) == INV and mixed(S=3, T=2019, B=-1) == INV


def noalloc(**kw):
    a = dict(q=Q, qs=2048, k=K_, ks=2048, v=V, vs=4096, g=G, b=BE, qsl=QSL, idx=IDX, hi=None, o=O, os=4096,
             S=3, T=2019, x=X, xs=8192, w=W, bias=B, cs=CS, cslots=64, dg=DG, dbe=DBE, didx=DIDX, do=DO, dos=4096,
             y=None, ys=0, B=32, silu=1, st=ST, slots=64, HK=16, HV=32, dk=128, dv=128, scale=1.0, norm=1)
    a.update(kw)
    return gdn.lib.gdn_chunk_rule_and_fused_decode_noalloc(
        a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["g"], a["b"], a["qsl"], a["idx"], a["hi"], a["o"],
        a["os"], a["S"], a["T"],
        a["x"], a["xs"], a["w"], a["bias"], a["cs"], a["cslots"], a["dg"], a["dbe"], a["didx"], a["do"], a["dos"],
        a["y"], a["ys"], a["B"], a["silu"],
        a["st"], a["slots"], a["HK"], a["HV"], a["dk"], a["dv"], a["scale"], a["norm"], None)


def test_noalloc_scratch_size_matches_the_header():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == gdn.NOALLOC_SCRATCH_BYTES


def test_noalloc_refuses_a_prefill_half_larger_than_its_scratch():
    """Refused on the host, before the scratch is looked up or anything is
    enqueued (fake device addresses; no GPU needed)."""
    T = 64
    while gdn.gdn_chunk_workspace_size(3, T, 16, 32) <= gdn.NOALLOC_SCRATCH_BYTES:
        T += 64
    assert noalloc(T=T) == CAP
    assert b"static scratch" in gdn.lib.gdn_last_error()
    assert gdn.gdn_chunk_workspace_size(3, 2019, 16, 32) <= gdn.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw,code", [
    (dict(S=0, T=0, B=0), gdn.GDN_OK),              # both halves empty: nothing to do
    (dict(S=0, T=0, x=None), INV),                  # the decode half's own checks
    (dict(S=0, T=0, B=-1), INV),
    (dict(S=0, T=-1, B=0), INV),
])
def test_noalloc_without_a_prefill_half(kw, code):
    """With no prefill tokens the scratch is not needed and never looked up,
    so these run on the host alone."""
    assert noalloc(**kw) == code, gdn.lib.gdn_last_error()
