"""CPU checks of the Python binding's argument checks: wrong shapes, wrong
dtypes, host tensors and short workspaces are rejected before anything
reaches the library (a recording stub stands in for it, and must see no
call)."""
import pytest
import torch

import gated_deltanet_token_amd as gdn

BF, F32, I32, U8 = torch.bfloat16, torch.float32, torch.int32, torch.uint8
C, HK, HV, D, SLOTS = 64, 1, 2, 16, 4          # conv rows q | k | v = 16 + 16 + 32 channels


class _Recorder:
    """Stands in for the library: records every call instead of making it."""

    def __init__(self, real):
        self.real, self.calls = real, []

    def __getattr__(self, name):
        if name in ("gdn_last_error", "gdn_build_conv_chunks", "gdn_chunk_workspace_size"):
            return getattr(self.real, name)
        return lambda *a: self.calls.append(name) or 0


@pytest.fixture
def rec(monkeypatch):
    r = _Recorder(gdn.lib)
    monkeypatch.setattr(gdn, "lib", r)
    yield r
    assert r.calls == [], "the library was called: %s" % r.calls


def conv_args(T=10, S=2):
    return dict(x=torch.zeros(T, C, dtype=BF), weight=torch.zeros(C, 4, dtype=BF), bias=torch.zeros(C, dtype=BF),
                conv_state=torch.zeros(SLOTS, 3, C, dtype=BF),
                query_start_loc=torch.tensor([0, 4, T][:S + 1], dtype=I32),
                state_indices=torch.arange(S, dtype=I32), has_initial_state=torch.zeros(S, dtype=U8),
                chunks=torch.zeros(2, 2, dtype=I32), y=torch.zeros(T, C, dtype=BF))


@pytest.mark.parametrize("change,msg", [
    (dict(), "GPU tensor"),                                           # right shapes, host memory
    (dict(conv_state=torch.zeros(SLOTS, 3, C + 8, dtype=BF)), "conv_state"),
    (dict(conv_state=torch.zeros(SLOTS, 4, C, dtype=BF)), "conv_state"),
    (dict(weight=torch.zeros(C - 8, 4, dtype=BF)), "weight"),
    (dict(bias=torch.zeros(C - 8, dtype=BF)), "bias"),
    (dict(y=torch.zeros(9, C, dtype=BF)), "y"),
    (dict(query_start_loc=torch.tensor([0, 10], dtype=I32)), "query_start_loc"),
    (dict(has_initial_state=torch.zeros(3, dtype=U8)), "has_initial_state"),
    (dict(chunks=torch.zeros(2, 3, dtype=I32)), "chunks"),
    (dict(x=torch.zeros(10, C, dtype=F32)), "x"),
    (dict(state_indices=torch.arange(2, dtype=torch.int64)), "state_indices"),
])
def test_conv_varlen_rejects(rec, change, msg):
    a = conv_args()
    a.update(change)
    with pytest.raises((ValueError, TypeError), match=msg):
        gdn.gdn_causal_conv1d_varlen(**a)


@pytest.mark.parametrize("change,msg", [
    (dict(), "GPU tensor"),
    (dict(state_indices=torch.arange(3, dtype=I32)), "state_indices"),
    (dict(y=torch.zeros(2, C + 8, dtype=BF)), "y"),
    (dict(conv_state=torch.zeros(SLOTS, 3, 32, dtype=BF)), "conv_state"),
])
def test_conv_update_rejects(rec, change, msg):
    a = dict(x=torch.zeros(2, C, dtype=BF), weight=torch.zeros(C, 4, dtype=BF), bias=None,
             conv_state=torch.zeros(SLOTS, 3, C, dtype=BF), state_indices=torch.arange(2, dtype=I32),
             y=torch.zeros(2, C, dtype=BF))
    a.update(change)
    with pytest.raises((ValueError, TypeError), match=msg):
        gdn.gdn_causal_conv1d_update(**a)


def rule_args(T=3, S=3, dk=D, dv=D):
    return dict(q=torch.zeros(T, HK, dk, dtype=BF), k=torch.zeros(T, HK, dk, dtype=BF),
                v=torch.zeros(T, HV, dv, dtype=BF), g=torch.zeros(T, HV), beta=torch.zeros(T, HV),
                state=torch.zeros(SLOTS, HV, dv, dk), state_indices=torch.arange(S, dtype=I32),
                o=torch.zeros(T, HV, dv, dtype=BF))


@pytest.mark.parametrize("change,msg", [
    (dict(), "GPU tensor"),
    (dict(state=torch.zeros(SLOTS, HV + 1, D, D)), "state"),
    (dict(state=torch.zeros(SLOTS, HV, D, D + 16)), "state"),
    (dict(g=torch.zeros(3, HV + 1)), "g"),
    (dict(beta=torch.zeros(2, HV)), "beta"),
    (dict(o=torch.zeros(3, HV, D + 8, dtype=BF)), "o"),
    (dict(k=torch.zeros(3, HK + 1, D, dtype=BF)), "k"),
    (dict(state_indices=torch.arange(2, dtype=I32)), "one token per sequence"),
    (dict(state=torch.zeros(SLOTS, HV, D, D).transpose(2, 3)), "contiguous"),
    (dict(query_start_loc=torch.tensor([0, 1, 3], dtype=I32)), "query_start_loc"),
])
def test_recurrent_decode_rejects(rec, change, msg):
    a = rule_args()
    a.update(change)
    with pytest.raises((ValueError, TypeError), match=msg):
        gdn.gdn_fused_recurrent_decode(**a)


def test_chunk_rule_needs_query_start_loc(rec):
    with pytest.raises(ValueError, match="query_start_loc"):
        gdn.gdn_chunk_gated_delta_rule(**rule_args(T=64, S=1, dk=128, dv=64), query_start_loc=None)


def test_chunk_rule_rejects_short_workspace(rec, monkeypatch):
    """A caller's workspace below gdn_chunk_workspace_size is refused in
    Python (device checks stubbed out: host tensors stand in)."""
    monkeypatch.setattr(gdn, "_on_gpu", lambda named: None)
    a = rule_args(T=64, S=1, dk=128, dv=64)
    need = gdn.gdn_chunk_workspace_size(1, 64, HK, HV)
    for ws, msg in ((torch.zeros(need - 1, dtype=U8), "needed"), (torch.zeros(need, dtype=F32), "workspace")):
        with pytest.raises((ValueError, TypeError), match=msg):
            gdn.gdn_chunk_gated_delta_rule(**a, query_start_loc=torch.tensor([0, 64], dtype=I32), workspace=ws)


def fused_args(B=2):
    return dict(x=torch.zeros(B, C, dtype=BF), conv_weight=torch.zeros(C, 4, dtype=BF), conv_bias=None,
                conv_state=torch.zeros(SLOTS, 3, C, dtype=BF), g=torch.zeros(B, HV), beta=torch.zeros(B, HV),
                state=torch.zeros(SLOTS, HV, D, D), state_indices=torch.arange(B, dtype=I32),
                o=torch.zeros(B, HV, D, dtype=BF), num_k_heads=HK, head_k_dim=D)


@pytest.mark.parametrize("change,msg", [
    (dict(), "GPU tensor"),
    (dict(x=torch.zeros(2, C - 8, dtype=BF)), "x"),
    (dict(conv_weight=torch.zeros(C, 3, dtype=BF)), "conv_weight"),
    (dict(num_k_heads=2), "x"),                       # q | k | v would be 96 channels
    (dict(state=torch.zeros(SLOTS, HV, D, 32)), "state"),
    (dict(y=torch.zeros(3, C, dtype=BF)), "y"),
    (dict(state_indices=torch.arange(1, dtype=I32)), "state_indices"),
])
def test_fused_decode_rejects(rec, change, msg):
    a = fused_args()
    a.update(change)
    with pytest.raises((ValueError, TypeError), match=msg):
        gdn.gdn_fused_conv_decode(**a)


def test_mixed_call_rejects(rec):
    """Each half checked as its own call, and the halves' head shapes must
    agree."""
    r = rule_args(T=64, S=1, dk=D, dv=D)
    f = fused_args()
    common = dict(q=r["q"], k=r["k"], v=r["v"], g=r["g"], beta=r["beta"], state_indices=r["state_indices"],
                  o=r["o"], query_start_loc=torch.tensor([0, 64], dtype=I32), has_initial_state=None,
                  dec_x=f["x"], conv_weight=f["conv_weight"], conv_bias=None, conv_state=f["conv_state"],
                  dec_g=f["g"], dec_beta=f["beta"], dec_state_indices=f["state_indices"], dec_o=f["o"],
                  state=f["state"], num_k_heads=HK)
    with pytest.raises(ValueError, match="GPU tensor"):
        gdn.gdn_chunk_rule_and_fused_decode(**common)
    bad = dict(common, dec_x=torch.zeros(2, C + 8, dtype=BF))
    with pytest.raises(ValueError, match="dec_x"):
        gdn.gdn_chunk_rule_and_fused_decode(**bad)
    bad = dict(common, dec_g=torch.zeros(3, HV))
    with pytest.raises(ValueError, match="dec_g"):
        gdn.gdn_chunk_rule_and_fused_decode(**bad)
    bad = dict(common, num_k_heads=2)
    with pytest.raises(ValueError, match="num_k_heads"):
        gdn.gdn_chunk_rule_and_fused_decode(**bad)
