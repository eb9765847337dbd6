"""Seeded synthetic inputs for the GDN token-mixer hot path.

This module is shared by the tests, the benchmark and the smoke check.  It
holds input generation and workload structure only -- no step of the
method's arithmetic: both the oracle and the HIP library receive exactly the
arrays built here.

Conventions
-----------
* bf16 tensors are numpy ``uint16`` arrays of raw bf16 bits, made by drawing
  float32 values and rounding them to nearest-even.
* Every tensor comes from ``np.random.default_rng([seed, config_id,
  tensor_id, ...])`` so tensors are independent and reproducible.
* Distributions: x ~ N(0,1); conv weight ~ N(0, 0.5) and bias ~ N(0, 0.1)
  (second parameter = standard deviation); carried conv state ~ N(0,1);
  beta = sigmoid(N(0,1)); the log-decay g = -softplus(N(0,1)) (the tiny case
  draws alpha ~ U(0.9, 1) and passes g = ln alpha); recurrent state
  ~ N(0,1)/sqrt(dk) where it is carried in.

The c32 workload the pages measure (page "RTX 5070 Ti: close Qwen3.5-4B TTFT,
TPOT, and VRAM gaps vs vLLM", section "Problem": 128 requests, 1,024 input and
128 output tokens, concurrency 32, 2048-token step budget) is reproduced by
:func:`engine_trace_schedule`; its prompts are replaced by seeded activations
(a GDN layer sees only the lengths).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

# model geometry of the c32 workload: q/k 16 heads x 128, v 32 heads x 128
C_FULL = 8192
HK_FULL, HV_FULL, D_FULL = 16, 32, 128
K_CONV = 4
POOL_SLOTS = 64
STEP_BUDGET = 2048

# tensor ids (the third element of every rng key)
T_X, T_W, T_BIAS, T_CSTATE, T_XDEC, T_Q, T_K, T_V, T_G, T_BETA, T_STATE, T_PERM, \
    T_LEN, T_FREE = range(14)


def rng(*key) -> np.random.Generator:
    return np.random.default_rng([int(k) for k in key])


# ----------------------------------------------------------------------------
# bf16 bits <-> float32
# ----------------------------------------------------------------------------

def to_bf16(a) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (inputs are finite)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).copy()
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    u += np.uint32(0x7FFF)
    u += lsb
    u >>= np.uint32(16)
    return u.astype(np.uint16)


def from_bf16(b) -> np.ndarray:
    """bf16 bits -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(r: np.random.Generator, shape, std=1.0) -> np.ndarray:
    a = r.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return to_bf16(a)


def sigmoid_normal(r, shape) -> np.ndarray:
    z = r.standard_normal(shape)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def neg_softplus_normal(r, shape) -> np.ndarray:
    z = r.standard_normal(shape)
    return (-np.logaddexp(0.0, z)).astype(np.float32)


# ----------------------------------------------------------------------------
# per-op configurations
# ----------------------------------------------------------------------------

def tiny(seed: int = 0) -> dict:
    """2 sequences of lengths 5 and 13, 64 channels, then one decode token
    per sequence; an independent decode with 2 q/k heads, 2 v heads, d=16."""
    cid = 1
    C, T = 64, 18
    d = dict(C=C, K=K_CONV, num_slots=4)
    d["qsl"] = np.array([0, 5, 18], np.int32)
    d["x"] = normal_bf16(rng(seed, cid, T_X), (T, C))
    d["weight"] = normal_bf16(rng(seed, cid, T_W), (C, K_CONV), 0.5)
    d["bias"] = normal_bf16(rng(seed, cid, T_BIAS), (C,), 0.1)
    d["has_init"] = np.array([0, 1], np.uint8)
    d["state_indices"] = np.array([2, 0], np.int32)
    d["conv_state"] = normal_bf16(rng(seed, cid, T_CSTATE), (4, K_CONV - 1, C))
    d["x_dec"] = normal_bf16(rng(seed, cid, T_XDEC), (2, C))
    # decode through the gated delta rule
    HK = HV = 2
    D = 16
    d.update(HK=HK, HV=HV, dk=D, dv=D)
    d["q"] = normal_bf16(rng(seed, cid, T_Q), (2, HK, D))
    d["k"] = normal_bf16(rng(seed, cid, T_K), (2, HK, D))
    d["v"] = normal_bf16(rng(seed, cid, T_V), (2, HV, D))
    alpha = rng(seed, cid, T_G).uniform(0.9, 1.0, (2, HV))
    d["g"] = np.log(alpha).astype(np.float32)
    d["beta"] = sigmoid_normal(rng(seed, cid, T_BETA), (2, HV))
    d["state"] = np.zeros((4, HV, D, D), np.float32)
    return d


def varlen_prefill(seed: int = 0) -> dict:
    """2 sequences x 1024 tokens packed, 8192 channels, zero initial state."""
    cid = 2
    C, T = C_FULL, 2048
    d = dict(C=C, K=K_CONV, num_slots=POOL_SLOTS)
    d["qsl"] = np.array([0, 1024, 2048], np.int32)
    d["x"] = normal_bf16(rng(seed, cid, T_X), (T, C))
    d["weight"] = normal_bf16(rng(seed, cid, T_W), (C, K_CONV), 0.5)
    d["bias"] = normal_bf16(rng(seed, cid, T_BIAS), (C,), 0.1)
    d["has_init"] = np.array([0, 0], np.uint8)
    perm = rng(seed, cid, T_PERM).permutation(POOL_SLOTS).astype(np.int32)
    d["state_indices"] = perm[:2].copy()
    # every slot holds junk: has_init = 0 must ignore it, other slots must survive
    d["conv_state"] = normal_bf16(rng(seed, cid, T_CSTATE), (POOL_SLOTS, K_CONV - 1, C))
    return d


def _mixed_lengths(r, total=STEP_BUDGET - 29, lo=100, hi=1500):
    while True:
        a, b = (int(v) for v in r.integers(lo, hi + 1, size=2))
        c = total - a - b
        if lo <= c <= hi:
            return [a, b, c]


def mixed_step(seed: int = 0, with_recurrence: bool = False) -> dict:
    """One chunked-prefill engine step: 29 single-token decodes (batch rows
    first) then 3 prefill chunks of random lengths summing to 2019; the third
    continues from a carried state.  Slots: the first 32 of a random
    permutation of the 64-slot pool."""
    cid = 3
    C = C_FULL
    nd = 29
    lens = _mixed_lengths(rng(seed, cid, T_LEN))
    T = nd + sum(lens)
    d = dict(C=C, K=K_CONV, num_slots=POOL_SLOTS, n_dec=nd, lens=lens)
    perm = rng(seed, cid, T_PERM).permutation(POOL_SLOTS).astype(np.int32)
    d["dec_indices"] = perm[:nd].copy()
    d["state_indices"] = perm[nd:nd + 3].copy()
    d["x_all"] = normal_bf16(rng(seed, cid, T_X), (T, C))
    d["qsl"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)  # relative to prefill rows
    d["has_init"] = np.array([0, 0, 1], np.uint8)
    d["weight"] = normal_bf16(rng(seed, cid, T_W), (C, K_CONV), 0.5)
    d["bias"] = normal_bf16(rng(seed, cid, T_BIAS), (C,), 0.1)
    d["conv_state"] = normal_bf16(rng(seed, cid, T_CSTATE), (POOL_SLOTS, K_CONV - 1, C))
    if with_recurrence:
        HK, HV, D = HK_FULL, HV_FULL, D_FULL
        d.update(HK=HK, HV=HV, dk=D, dv=D)
        d["q"] = normal_bf16(rng(seed, cid, T_Q), (T, HK, D))
        d["k"] = normal_bf16(rng(seed, cid, T_K), (T, HK, D))
        d["v"] = normal_bf16(rng(seed, cid, T_V), (T, HV, D))
        d["g"] = neg_softplus_normal(rng(seed, cid, T_G), (T, HV))
        d["beta"] = sigmoid_normal(rng(seed, cid, T_BETA), (T, HV))
        d["state"] = (rng(seed, cid, T_STATE).standard_normal(
            (POOL_SLOTS, HV, D, D), dtype=np.float32) / np.float32(np.sqrt(D)))
    return d


def fused_decode(seed: int = 0) -> dict:
    """32 sequences x 1 token: conv update on 8192 channels, then the gated
    delta rule with 16 q/k heads, 32 v heads, head dim 128, fp32 state in a
    64-slot pool."""
    cid = 4
    C, B = C_FULL, 32
    HK, HV, D = HK_FULL, HV_FULL, D_FULL
    d = dict(C=C, K=K_CONV, num_slots=POOL_SLOTS, B=B, HK=HK, HV=HV, dk=D, dv=D)
    perm = rng(seed, cid, T_PERM).permutation(POOL_SLOTS).astype(np.int32)
    d["state_indices"] = perm[:B].copy()
    d["x"] = normal_bf16(rng(seed, cid, T_X), (B, C))
    d["weight"] = normal_bf16(rng(seed, cid, T_W), (C, K_CONV), 0.5)
    d["bias"] = normal_bf16(rng(seed, cid, T_BIAS), (C,), 0.1)
    d["conv_state"] = normal_bf16(rng(seed, cid, T_CSTATE), (POOL_SLOTS, K_CONV - 1, C))
    d["q"] = normal_bf16(rng(seed, cid, T_Q), (B, HK, D))
    d["k"] = normal_bf16(rng(seed, cid, T_K), (B, HK, D))
    d["v"] = normal_bf16(rng(seed, cid, T_V), (B, HV, D))
    d["g"] = neg_softplus_normal(rng(seed, cid, T_G), (B, HV))
    d["beta"] = sigmoid_normal(rng(seed, cid, T_BETA), (B, HV))
    d["state"] = (rng(seed, cid, T_STATE).standard_normal(
        (POOL_SLOTS, HV, D, D), dtype=np.float32) / np.float32(np.sqrt(D)))
    return d


def random_gdn(seed, cid, lens, HK, HV, dk, dv, num_slots, has_init=None,
               state_indices=None):
    """Generic varlen recurrence inputs (for parity sweeps)."""
    T = int(sum(lens))
    d = dict(HK=HK, HV=HV, dk=dk, dv=dv, num_slots=num_slots)
    d["qsl"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    S = len(lens)
    if state_indices is None:
        state_indices = rng(seed, cid, T_PERM).permutation(num_slots)[:S]
    d["state_indices"] = np.asarray(state_indices, np.int32)
    d["has_init"] = (np.ones(S, np.uint8) if has_init is None
                     else np.asarray(has_init, np.uint8))
    d["q"] = normal_bf16(rng(seed, cid, T_Q), (T, HK, dk))
    d["k"] = normal_bf16(rng(seed, cid, T_K), (T, HK, dk))
    d["v"] = normal_bf16(rng(seed, cid, T_V), (T, HV, dv))
    d["g"] = neg_softplus_normal(rng(seed, cid, T_G), (T, HV))
    d["beta"] = sigmoid_normal(rng(seed, cid, T_BETA), (T, HV))
    d["state"] = (rng(seed, cid, T_STATE).standard_normal(
        (num_slots, HV, dv, dk), dtype=np.float32) / np.float32(np.sqrt(dk)))
    return d


def random_conv(seed, cid, lens, C, num_slots, has_init=None, state_indices=None):
    """Generic varlen conv inputs (for parity sweeps)."""
    T = int(sum(lens))
    S = len(lens)
    d = dict(C=C, K=K_CONV, num_slots=num_slots)
    d["qsl"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    if state_indices is None:
        state_indices = rng(seed, cid, T_PERM).permutation(num_slots)[:S]
    d["state_indices"] = np.asarray(state_indices, np.int32)
    d["has_init"] = (np.ones(S, np.uint8) if has_init is None
                     else np.asarray(has_init, np.uint8))
    d["x"] = normal_bf16(rng(seed, cid, T_X), (T, C))
    d["weight"] = normal_bf16(rng(seed, cid, T_W), (C, K_CONV), 0.5)
    d["bias"] = normal_bf16(rng(seed, cid, T_BIAS), (C,), 0.1)
    d["conv_state"] = normal_bf16(rng(seed, cid, T_CSTATE), (num_slots, K_CONV - 1, C))
    return d


# ----------------------------------------------------------------------------
# the c32 engine-step trace
# ----------------------------------------------------------------------------

@dataclass
class TraceStep:
    # decodes: (request, position, slot); batch rows come first, in this order
    decodes: list = field(default_factory=list)
    # prefill chunks: (request, first position, n tokens, slot, has_init)
    prefills: list = field(default_factory=list)

    @property
    def n_tokens(self):
        return len(self.decodes) + sum(p[2] for p in self.prefills)


@dataclass
class Trace:
    steps: list
    n_requests: int
    prompt: int
    decode_forwards: int
    slot_of: list          # slot held by each request
    finish_step: list      # step index at which each request's last token ran

    @property
    def seq_len(self):
        return self.prompt + self.decode_forwards

    @property
    def n_tokens(self):
        return sum(s.n_tokens for s in self.steps)


def engine_trace_schedule(seed: int = 0, n_requests: int = 128, prompt: int = 1024,
                          output_tokens: int = 128, max_running: int = 32,
                          budget: int = STEP_BUDGET, n_slots: int = POOL_SLOTS) -> Trace:
    """Chunked-prefill FIFO schedule of the c32 workload for one GDN layer.

    Each step first gives one token to every decoding request, then continues
    unfinished prefills in arrival order, then admits waiting requests in
    arrival order (while fewer than ``max_running`` run), chunking prompts to
    fill ``budget`` tokens.  The last prefill chunk yields the first output
    token, so each request then runs ``output_tokens - 1`` decode forwards.
    Slots come from a seeded free list and return to its tail on finish.
    """
    cid = 5
    decode_forwards = output_tokens - 1
    free = list(rng(seed, cid, T_FREE).permutation(n_slots).astype(int))
    waiting = list(range(n_requests))
    prefilling = []          # [request, next position]
    decoding = []            # [request, decodes done]
    slot_of = [-1] * n_requests
    finish = [-1] * n_requests
    steps = []
    while waiting or prefilling or decoding:
        st = TraceStep()
        left = budget
        for rd in decoding:
            r, done = rd
            st.decodes.append((r, prompt + done, slot_of[r]))
            rd[1] += 1
            left -= 1
        for pf in prefilling:
            if left == 0:
                break
            r, p0 = pf
            n = min(prompt - p0, left)
            st.prefills.append((r, p0, n, slot_of[r], int(p0 > 0)))
            pf[1] += n
            left -= n
        while waiting and left > 0 and len(prefilling) + len(decoding) < max_running:
            r = waiting.pop(0)
            slot_of[r] = free.pop(0)
            n = min(prompt, left)
            st.prefills.append((r, 0, n, slot_of[r], 0))
            prefilling.append([r, n])
            left -= n
        steps.append(st)
        si = len(steps) - 1
        still = []
        for rd in decoding:
            if rd[1] == decode_forwards:
                finish[rd[0]] = si
                free.append(slot_of[rd[0]])
            else:
                still.append(rd)
        decoding = still
        still = []
        for pf in prefilling:
            if pf[1] == prompt:
                if decode_forwards == 0:
                    finish[pf[0]] = si
                    free.append(slot_of[pf[0]])
                else:
                    decoding.append([pf[0], 0])
            else:
                still.append(pf)
        prefilling = still
    return Trace(steps, n_requests, prompt, decode_forwards, slot_of, finish)


def trace_request_inputs(seed: int, layer: int, r: int, seq_len: int,
                         C: int = C_FULL, HV: int = HV_FULL):
    """Activations of request r at every position 0..seq_len-1 for one layer:
    x bf16 [seq_len][C], g and beta float32 [seq_len][HV].  A pure function
    of (seed, layer, r), so chunking cannot change the inputs."""
    cid = 5
    x = normal_bf16(rng(seed, cid, T_X, layer, r), (seq_len, C))
    g = neg_softplus_normal(rng(seed, cid, T_G, layer, r), (seq_len, HV))
    beta = sigmoid_normal(rng(seed, cid, T_BETA, layer, r), (seq_len, HV))
    return x, g, beta


def trace_layer_weights(seed: int, layer: int, C: int = C_FULL):
    cid = 5
    w = normal_bf16(rng(seed, cid, T_W, layer), (C, K_CONV), 0.5)
    b = normal_bf16(rng(seed, cid, T_BIAS, layer), (C,), 0.1)
    return w, b


def trace_all_inputs(seed: int, layer: int, trace: Trace, C: int = C_FULL,
                     HV: int = HV_FULL, workers: int | None = None):
    """All requests' activations, [n_requests][seq_len][...], generated in
    parallel threads (numpy releases the GIL while drawing)."""
    L = trace.seq_len
    R = trace.n_requests
    x = np.empty((R, L, C), np.uint16)
    g = np.empty((R, L, HV), np.float32)
    beta = np.empty((R, L, HV), np.float32)

    def one(r):
        x[r], g[r], beta[r] = trace_request_inputs(seed, layer, r, L, C, HV)

    workers = workers or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, range(R)))
    return x, g, beta


def trace_step_rows(trace: Trace):
    """For every step, the (request, position) of each packed token row,
    decodes first, then prefill chunks in order; and the packed offset of
    each step."""
    rows = []
    offs = [0]
    for st in trace.steps:
        rr = [(r, p) for (r, p, _s) in st.decodes]
        for (r, p0, n, _s, _h) in st.prefills:
            rr.extend((r, p0 + i) for i in range(n))
        rows.append(np.array(rr, np.int64).reshape(-1, 2))
        offs.append(offs[-1] + len(rr))
    return rows, np.array(offs, np.int64)
