#!/usr/bin/env python3
"""Benchmark of the GDN token-mixer hot path on one MI355X.

Workload (one bench "step"): the c32 engine-step trace -- 128 requests of
1,024 prompt tokens and 128 output tokens, at most 32 running, 2,048-token
chunked-prefill budget per engine step, FIFO admission (529 engine steps,
147,328 tokens) -- pushed through ``--layers`` GDN layers.  Each layer has its
own conv weights, conv_state pool and recurrent-state pool (64 slots each)
and its own activations, so consecutive layers do not find each other's state
in the 256 MB Infinity Cache, as in a model with several GDN layers.

Per engine step: the host builds the exact (sequence, 8-token chunk)
descriptors once (gdn_build_conv_chunks) and uploads them once; then for every
layer: the varlen conv for the prefill rows, and the recurrence -- the
chunkwise (matrix-core) form of the rule for the prefill chunks (q, k, v are
column views of the conv output) and, for the decode rows, the conv update
fused with the rule.  A step with only decode rows makes one
gdn_fused_conv_decode call per layer, a step with only prefill rows a
gdn_chunk_gated_delta_rule call, a step with both one
gdn_chunk_rule_and_fused_decode call (the chunkwise scan and the decode in
one grid).  Inputs are resident in HBM before the timed region; every call
goes through the C ABI on torch's current stream.

Output: one JSON line.  ``value`` is GDN-layer tokens per second (tokens x
layers / wall time).  ``roofline`` is for the kernel with the largest share
of GPU time; its average launch duration comes from HIP events recorded on
the launch stream inside the timed region: one pair around every run of
several consecutive launches of that kernel and around every seventh
one-launch run, the latter weighted, which estimates the kernel's total time.
Each recorded event idles the stream for a few microseconds on this GPU; that
cost is measured in the same process (fixed-length spin kernels with and
without an event pair around each) and subtracted from every bracketed span,
here and in the per-kernel figures (``kernels``).  ``isolated`` times each
call alone at its c32 shape with HBM-resident operands, beside a plain copy
(conv) and an in-place read-modify-write (decode) of the same bytes as
measured ceilings.  ``cpu_baseline`` is the fp64 oracle timed on this host on
a bounded sample of the same workload, serial on one core and (``multicore``)
the same source built with OpenMP on every core, each sample taken half
before and half after the GPU's timed region.  ``context`` carries the pages'
own figures (another GPU, a whole engine): context only.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN layer tokens/s + achieved HBM GB/s (% peak), c32 prefill & decode"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak

C, HK, HV, D, K = 8192, 16, 32, 128, 4
ROOFLINE_STRIDE = 7             # every 7th one-launch run of the dominant kernel is timed with events
SLOTS = 64
BUDGET = 2048

# The pages' own figures for this path, carried beside the results as
# context only: a different GPU and a whole serving engine, not a target.
PAGES_CONTEXT = {
    "hardware": "RTX 5070 Ti (sm_120), whole Qwen3.5-4B BF16 engine, c32 workload (128 requests, 1024 in / 128 out, "
                "concurrency 32, 2048-token budget)",
    "causal_conv_gpu_time_ms": {"whole_sequence_dispatch": 720.2, "exact_8_token_chunks": 234.4,
                                "vllm_triton_kernel": 145.4,
                                "source": 'page "perf(gdn): dispatch exact causal-conv chunks", section "Speed '
                                          'claims"; vLLM figure: page "RTX 5070 Ti: close Qwen3.5-4B TTFT, TPOT, '
                                          'and VRAM gaps vs vLLM", section "Existing evidence"'},
    "end_to_end_tokens_per_s": {"before": 6587.66, "after": 6727.35,
                                "source": 'page "perf(gdn): dispatch exact causal-conv chunks", section "Speed '
                                          'claims" (whole model, input + output tokens, profiled run)'},
    "note": "sums over a whole served run on another GPU; no per-kernel time or bandwidth is given on the pages",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-sample-requests", type=int, default=14,
                    help="requests timed through the serial oracle (one core)")
    ap.add_argument("--cpu-multicore-requests", type=int, default=48,
                    help="requests timed through the OpenMP build of the oracle (every core)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-isolated", action="store_true",
                    help="skip the per-call measurements at the c32 shapes with HBM-only operands")
    ap.add_argument("--out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times) and exit: the "
                         "reference kernel for scaling memory-traffic counters")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work per launch (what the method must move / compute)
# ---------------------------------------------------------------------------

def bytes_conv_varlen(tokens, seqs, seqs_with_init, n_chunks):
    return (2 * tokens * C * 2                       # x read, y write
            + seqs * 3 * C * 2 + seqs_with_init * 3 * C * 2   # slot write / read
            + C * K * 2 + C * 2                      # weights, bias
            + n_chunks * 8 + (seqs + 1) * 4 + seqs * 5)


def bytes_conv_update(batch):
    return batch * (2 * C * 2 + 2 * 3 * C * 2 + 4) + C * K * 2 + C * 2


def bytes_fused_decode(batch):
    state = D * D * 4 * HV
    return (batch * (C * 2 + 2 * 3 * C * 2 + 4)        # x, conv_state read + write, slot index
            + C * K * 2 + C * 2                         # conv weights, bias
            + batch * 2 * state                         # recurrent state read + write
            + batch * (HV * D * 2 + HV * 8))            # o, g, beta


def bytes_recurrent(tokens, seqs_with_state_read, seqs):
    state = D * D * 4 * HV
    return (seqs_with_state_read * state + seqs * state          # state read, write
            + tokens * ((2 * HK * D + HV * D) * 2 + HV * D * 2 + HV * 8))


def flops_recurrent(tokens):
    # per token and v-head: S k (2 d^2), the rank-1 update a S + c k^T (2 d^2),
    # S q (2 d^2)
    return 6.0 * tokens * HV * D * D


# ---------------------------------------------------------------------------
# memory traffic per launch, from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# ---------------------------------------------------------------------------
# The counter figures live in a committed profile summary, one "traffic-record"
# line per kernel, together with a digest of the kernel's source files at the
# time the counters were taken.  A figure is used only while the sources still
# match: after any change to the kernel it is reported as null until measured
# again.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_c32_trace_4layers.md")
_CSRC = os.path.join(ROOT, "gated_deltanet_token_amd", "csrc")
KERNEL_SOURCES = {
    "fused_decode": ["fused.hip", "fused_unit.h", "conv_math.h", "gdr_math.h", "gdn_device.h", "gdn_internal.h"],
    "conv_varlen": ["conv.hip", "conv_math.h", "gdn_device.h", "gdn_internal.h"],
    "recurrent_chunk": ["chunk.hip", "fused_unit.h", "conv_math.h", "gdr_math.h", "gdn_device.h",
                        "gdn_internal.h"],
    "chunk_and_decode": ["chunk.hip", "fused_unit.h", "conv_math.h", "gdr_math.h", "gdn_device.h",
                         "gdn_internal.h"],
}


def sources_digest(kind):
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read() + b"\0")
    return h.hexdigest()[:16]


def traffic_per_launch(kind):
    """Measured HBM bytes (fetch + write) per launch of ``kind`` in the trace,
    or None if there is no record for the current sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = [ln.split() for ln in f if ln.startswith("traffic-record ")]
    except OSError:
        return None
    for parts in lines:
        rec = dict(p.split("=", 1) for p in parts[1:])
        if rec.get("kernel") == kind and rec.get("sources") == sources_digest(kind):
            return int(rec["fetch_bytes"]) + int(rec["write_bytes"])
    return None


# ---------------------------------------------------------------------------
# every call of the path alone at its c32 shape, from HBM
# ---------------------------------------------------------------------------

def isolated(seed, reps=64):
    """Each hot-path call alone at its c32 shape with its operands in HBM.

    The operands rotate over buffer sets that together exceed the 256 MB
    Infinity Cache several times, so no launch finds its inputs in a cache.
    A sleep kernel at the head of the stream lets the host queue every timed
    launch before the first one starts, so host-side launch cost does not
    open gaps between kernels.  Returns {call: {...}} with the average launch
    time from HIP events on the launch stream."""
    import torch
    import gated_deltanet_token_amd as gdn
    import synth
    lib = gdn.lib
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)
    gen = torch.Generator(device=dev)
    gen.manual_seed(7919 + seed)

    def bf(*shape, std=1.0):
        return (std * torch.randn(*shape, generator=gen, device=dev)).to(torch.bfloat16)

    def i32(a):
        return torch.as_tensor(np.asarray(a, np.int32), device=dev)

    def u8(a):
        return torch.as_tensor(np.asarray(a, np.uint8), device=dev)

    def check(rc, what):
        if rc != 0:
            raise RuntimeError("%s: %s" % (what, lib.gdn_last_error().decode()))

    # the reference copy kernels for the ceilings (their own library)
    ceil = ctypes.CDLL(os.path.join(ROOT, "gated_deltanet_token_amd", "ceiling", "libgdn_ceiling.so"))
    ceil.ceiling_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_void_p]
    ceil.ceiling_stream_rmw.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]

    def timed(calls, reps=reps):
        for c in calls:
            c()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(2_000_000)
        e0.record(stream)
        for i in range(reps):
            calls[i % len(calls)]()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    def entry(us, nbytes, nflops=None, **extra):
        d = {"avg_launch_us": us, "algorithmic_bytes": nbytes, "gb_per_s": nbytes / us / 1e3,
             "hbm_frac": nbytes / us / 1e3 / HBM_PEAK_GBS}
        if nflops:
            d["tflop_per_s"] = nflops / us / 1e6
        d.update(extra)
        return d

    out = {}
    w, b = bf(C, K, std=0.5), bf(C, std=0.1)

    # A1: varlen conv, 2 sequences x 1024 tokens, 256 descriptors, zero initial state
    T2 = 2048
    qsl2 = np.array([0, 1024, 2048], np.int32)
    ch2 = gdn.gdn_build_conv_chunks(qsl2)
    ch2_d, qsl2_d = i32(ch2.reshape(-1)), i32(qsl2)
    idx2, hi2 = i32([17, 42]), u8([0, 0])
    cs = torch.zeros(SLOTS, 3, C, dtype=torch.bfloat16, device=dev)
    sets = [(bf(T2, C), torch.empty(T2, C, dtype=torch.bfloat16, device=dev)) for _ in range(10)]
    calls = [lambda x=x, y=y: check(lib.gdn_causal_conv1d_varlen(
        x.data_ptr(), C, w.data_ptr(), b.data_ptr(), cs.data_ptr(), SLOTS, qsl2_d.data_ptr(), idx2.data_ptr(),
        hi2.data_ptr(), ch2_d.data_ptr(), len(ch2), y.data_ptr(), C, 2, T2, C, K, 1, sptr), "conv_varlen")
        for x, y in sets]
    out["conv_varlen"] = entry(timed(calls), bytes_conv_varlen(T2, 2, 0, len(ch2)),
                               shape="2 x 1024 tokens, 8192 channels, 256 descriptors", buffer_sets=len(sets))
    # what HBM allows for these bytes: a plain streaming copy of x into y
    # (the same buffers, the same rotation)
    nb_copy = 2 * T2 * C * 2
    us_copy, u_copy = min((timed([lambda x=x, y=y: check(ceil.ceiling_stream_copy(
        x.data_ptr(), y.data_ptr(), nb_copy // 2, u, sptr), "ceiling copy") for x, y in sets]), u) for u in (1, 4, 16))
    out["conv_varlen"]["ceiling"] = {
        "kind": "streaming device copy of the same bytes (%.1f MB in + %.1f MB out, 16-byte nontemporal loads and "
                "stores, %d per lane: the fastest of 1, 4, 16)" % (nb_copy / 2e6, nb_copy / 2e6, u_copy),
        "avg_launch_us": us_copy, "gb_per_s": nb_copy / us_copy / 1e3, "hbm_frac": nb_copy / us_copy / 1e3 / HBM_PEAK_GBS}
    out["conv_varlen"]["frac_of_ceiling"] = out["conv_varlen"]["gb_per_s"] / out["conv_varlen"]["ceiling"]["gb_per_s"]
    # the same call with 16-token programs (two descriptors per program,
    # gdn_causal_conv1d_varlen_tiles): same results, 19 rows read per 16 tokens
    calls = [lambda x=x, y=y: check(lib.gdn_causal_conv1d_varlen_tiles(
        x.data_ptr(), C, w.data_ptr(), b.data_ptr(), cs.data_ptr(), SLOTS, qsl2_d.data_ptr(), idx2.data_ptr(),
        hi2.data_ptr(), ch2_d.data_ptr(), len(ch2), y.data_ptr(), C, 2, T2, C, K, 1, 2, sptr), "conv_varlen_tiles")
        for x, y in sets]
    out["conv_varlen_16token_programs"] = entry(timed(calls), bytes_conv_varlen(T2, 2, 0, len(ch2)),
                                                shape="the same in 16-token programs: 128 descriptor pairs x 4 channel tiles",
                                                buffer_sets=len(sets))
    del sets, calls

    # A2 + A3 at the decode shape: 32 sequences, 16 q/k heads, 32 v heads, d = 128
    B = 32
    idx_d = i32(np.random.default_rng(seed).permutation(SLOTS)[:B])
    pools = []
    for _ in range(6):
        st = (torch.randn(SLOTS, HV, D, D, generator=gen, device=dev) / np.sqrt(D)).contiguous()
        pools.append(dict(state=st, cs=bf(SLOTS, 3, C), x=bf(B, C), q=bf(B, HK, D), k=bf(B, HK, D),
                          v=bf(B, HV, D), o=torch.empty(B, HV, D, dtype=torch.bfloat16, device=dev),
                          y=torch.empty(B, C, dtype=torch.bfloat16, device=dev)))
    g = -torch.nn.functional.softplus(torch.randn(B, HV, generator=gen, device=dev)).contiguous()
    beta = torch.sigmoid(torch.randn(B, HV, generator=gen, device=dev)).contiguous()
    f1 = ctypes.c_float(1.0)
    calls = [lambda p=p: check(lib.gdn_fused_conv_decode(
        p["x"].data_ptr(), C, w.data_ptr(), b.data_ptr(), p["cs"].data_ptr(), SLOTS, g.data_ptr(), beta.data_ptr(),
        p["state"].data_ptr(), SLOTS, idx_d.data_ptr(), p["o"].data_ptr(), HV * D, None, 0, B, HK, HV, D, D, 1,
        f1, 1, sptr), "fused_decode") for p in pools]
    out["fused_decode"] = entry(timed(calls), bytes_fused_decode(B), flops_recurrent(B),
                                shape="32 sequences x 1 token: conv update on 8192 channels + gated delta rule, "
                                      "16 q/k heads, 32 v heads, d 128", buffer_sets=len(pools))
    # what HBM allows for the state traffic: a streaming in-place
    # read-modify-write of 32 slots' worth of fp32 state, in the same pools
    n_rmw = B * HV * D * D
    nb_rmw = 2 * n_rmw * 4
    us_rmw, u_rmw = min((timed([lambda p=p: check(ceil.ceiling_stream_rmw(p["state"].data_ptr(), nb_rmw // 2, u, sptr),
                                                  "ceiling rmw") for p in pools]), u) for u in (1, 4, 16))
    out["fused_decode"]["ceiling"] = {
        "kind": "streaming in-place read-modify-write of %.1f MB of fp32 (read and written once, %d 16-byte "
                "accesses per lane: the fastest of 1, 4, 16)" % (nb_rmw / 2e6, u_rmw),
        "avg_launch_us": us_rmw, "gb_per_s": nb_rmw / us_rmw / 1e3, "hbm_frac": nb_rmw / us_rmw / 1e3 / HBM_PEAK_GBS}
    out["fused_decode"]["frac_of_ceiling"] = out["fused_decode"]["gb_per_s"] / out["fused_decode"]["ceiling"]["gb_per_s"]
    calls = [lambda p=p: check(lib.gdn_fused_recurrent_decode(
        p["q"].data_ptr(), HK * D, p["k"].data_ptr(), HK * D, p["v"].data_ptr(), HV * D, g.data_ptr(),
        beta.data_ptr(), p["state"].data_ptr(), SLOTS, None, idx_d.data_ptr(), None, p["o"].data_ptr(), HV * D,
        B, B, HK, HV, D, D, f1, 1, sptr), "recurrent_decode") for p in pools]
    out["recurrent_decode"] = entry(timed(calls), bytes_recurrent(B, B, B), flops_recurrent(B),
                                    shape="32 sequences x 1 token, 16 q/k heads, 32 v heads, d 128",
                                    buffer_sets=len(pools))
    calls = [lambda p=p: check(lib.gdn_causal_conv1d_update(
        p["x"].data_ptr(), C, w.data_ptr(), b.data_ptr(), p["cs"].data_ptr(), SLOTS, idx_d.data_ptr(),
        p["y"].data_ptr(), C, B, C, K, 1, sptr), "conv_update") for p in pools]
    out["conv_update"] = entry(timed(calls), bytes_conv_update(B), shape="32 rows x 8192 channels",
                               buffer_sets=len(pools), note="launch-bound")
    del calls

    # A4: chunkwise recurrence at the mixed-step shape (3 prefill chunks summing to 2019 tokens)
    lens = synth._mixed_lengths(synth.rng(seed, 3, synth.T_LEN))
    T3 = int(sum(lens))
    qsl3 = i32(np.concatenate([[0], np.cumsum(lens)]))
    idx3, hi3 = i32([5, 33, 60]), u8([0, 0, 1])
    ws_bytes = gdn.gdn_chunk_workspace_size(3, T3, HK, HV)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    g3 = -torch.nn.functional.softplus(torch.randn(T3, HV, generator=gen, device=dev)).contiguous()
    b3 = torch.sigmoid(torch.randn(T3, HV, generator=gen, device=dev)).contiguous()
    sets = []
    for p in pools[:4]:
        sets.append((bf(T3, C), p["state"], torch.empty(T3, HV, D, dtype=torch.bfloat16, device=dev)))
    calls = [lambda y=y, st=st, o=o: check(lib.gdn_chunk_gated_delta_rule(
        y.data_ptr(), C, y.data_ptr() + HK * D * 2, C, y.data_ptr() + 2 * HK * D * 2, C, g3.data_ptr(),
        b3.data_ptr(), st.data_ptr(), SLOTS, qsl3.data_ptr(), idx3.data_ptr(), hi3.data_ptr(), o.data_ptr(), HV * D,
        3, T3, HK, HV, D, D, ws.data_ptr(), ws_bytes, f1, 1, sptr), "recurrent_chunk") for y, st, o in sets]
    us = timed(calls)
    out["recurrent_chunk"] = entry(us, bytes_recurrent(T3, 1, 3), flops_recurrent(T3),
                                   shape="3 prefill chunks of %s tokens, 16 q/k heads, 32 v heads, d 128"
                                         % "+".join(str(x) for x in lens),
                                   buffer_sets=len(sets), tokens_per_s=T3 / us * 1e6,
                                   bound="latency (serial over 64-token chunks)")
    # the same tokens through the token-by-token form (gdn_fused_recurrent_decode
    # with query_start_loc): the state stays in registers across a sequence's
    # tokens, each token a serial step
    calls = [lambda y=y, st=st, o=o: check(lib.gdn_fused_recurrent_decode(
        y.data_ptr(), C, y.data_ptr() + HK * D * 2, C, y.data_ptr() + 2 * HK * D * 2, C, g3.data_ptr(),
        b3.data_ptr(), st.data_ptr(), SLOTS, qsl3.data_ptr(), idx3.data_ptr(), hi3.data_ptr(), o.data_ptr(), HV * D,
        3, T3, HK, HV, D, D, f1, 1, sptr), "recurrent_token_loop") for y, st, o in sets]
    us_tl = timed(calls, reps=20)
    out["recurrent_token_loop"] = entry(us_tl, bytes_recurrent(T3, 1, 3), flops_recurrent(T3),
                                        shape="the same 3 prefill chunks, token by token", buffer_sets=len(sets),
                                        tokens_per_s=T3 / us_tl * 1e6, bound="latency (serial over tokens)")

    # the mixed step's recurrence as one call (gdn_chunk_rule_and_fused_decode):
    # the same prefill chunks and 29 decode rows on other slots of the same pool,
    # against the chunkwise call followed by the fused decode
    nd = 29
    didx = i32(np.random.default_rng(seed + 1).permutation(np.setdiff1d(np.arange(SLOTS), [5, 33, 60]))[:nd])
    gd, bd = g[:nd].contiguous(), beta[:nd].contiguous()
    msets = [(y, st, o, p) for (y, st, o), p in zip(sets, pools[:4])]
    mixed = [lambda y=y, st=st, o=o, p=p: check(lib.gdn_chunk_rule_and_fused_decode(
        y.data_ptr(), C, y.data_ptr() + HK * D * 2, C, y.data_ptr() + 2 * HK * D * 2, C, g3.data_ptr(),
        b3.data_ptr(), qsl3.data_ptr(), idx3.data_ptr(), hi3.data_ptr(), o.data_ptr(), HV * D, 3, T3,
        ws.data_ptr(), ws_bytes, p["x"].data_ptr(), C, w.data_ptr(), b.data_ptr(), p["cs"].data_ptr(), SLOTS,
        gd.data_ptr(), bd.data_ptr(), didx.data_ptr(), p["o"].data_ptr(), HV * D, None, 0, nd, 1,
        st.data_ptr(), SLOTS, HK, HV, D, D, f1, 1, sptr), "chunk_and_decode") for y, st, o, p in msets]

    def two(y, st, o, p):
        check(lib.gdn_chunk_gated_delta_rule(
            y.data_ptr(), C, y.data_ptr() + HK * D * 2, C, y.data_ptr() + 2 * HK * D * 2, C, g3.data_ptr(),
            b3.data_ptr(), st.data_ptr(), SLOTS, qsl3.data_ptr(), idx3.data_ptr(), hi3.data_ptr(), o.data_ptr(),
            HV * D, 3, T3, HK, HV, D, D, ws.data_ptr(), ws_bytes, f1, 1, sptr), "recurrent_chunk")
        check(lib.gdn_fused_conv_decode(
            p["x"].data_ptr(), C, w.data_ptr(), b.data_ptr(), p["cs"].data_ptr(), SLOTS, gd.data_ptr(),
            bd.data_ptr(), st.data_ptr(), SLOTS, didx.data_ptr(), p["o"].data_ptr(), HV * D, None, 0, nd, HK, HV,
            D, D, 1, f1, 1, sptr), "fused_decode")
    us_two = timed([lambda m=m: two(*m) for m in msets])
    us = timed(mixed)
    out["chunk_and_decode"] = entry(us, bytes_recurrent(T3, 1, 3) + bytes_fused_decode(nd),
                                    flops_recurrent(T3) + flops_recurrent(nd),
                                    shape="the mixed step's recurrence: 3 prefill chunks of %s tokens and %d "
                                          "decode rows (conv update + rule)" % ("+".join(str(x) for x in lens), nd),
                                    buffer_sets=len(msets), two_calls_us=us_two)
    del sets, msets, calls, mixed, pools
    torch.cuda.synchronize()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class CpuBaseline:
    """The fp64 oracle timed on this host over whole requests of the trace
    (one GDN layer: conv, bf16 rounding, gated delta rule per request).  Two
    legs: the serial oracle on one core, and the same source built with
    OpenMP on every core in sched_getaffinity (independent conv channels and
    (sequence, v-head) pairs on separate threads, identical results).  Each
    leg's sample is taken in two halves, one before and one after the GPU's
    timed region (the pages' order-alternated A/B practice)."""

    def __init__(self, seed, seq_len, n_serial, n_multi):
        import ctypes as ct
        import oracle
        self.oracle, self.seed, self.seq_len = oracle, seed, seq_len
        self.w, self.b = None, None
        self.serial = oracle._load()
        self.cores = len(os.sched_getaffinity(0))
        self.omp = oracle.bind(oracle.build_omp())
        ct.CDLL("libgomp.so.1").omp_set_num_threads(self.cores)
        self.reqs = {"serial": list(range(n_serial)), "multi": list(range(n_serial, n_serial + n_multi))}
        self.time = {"serial": 0.0, "multi": 0.0}
        self.done = {"serial": 0, "multi": 0}

    def _one(self, lib, r):
        import synth
        o = self.oracle
        if self.w is None:
            self.w, self.b = synth.trace_layer_weights(self.seed, 0)
        L = self.seq_len
        x, g, beta = synth.trace_request_inputs(self.seed, 0, r, L)
        saved = o._lib
        o._lib = lib
        try:
            t0 = time.perf_counter()
            y, _ = o.causal_conv1d_varlen(x, self.w, self.b, np.zeros((1, 3, C), np.uint16), [0, L], [0], [0])
            yb = o.round_bf16(y)
            o.gated_delta_rule(yb[:, :HK * D].reshape(L, HK, D), yb[:, HK * D:2 * HK * D].reshape(L, HK, D),
                               yb[:, 2 * HK * D:].reshape(L, HV, D), g, beta, np.zeros((1, HV, D, D)), [0], [0, L],
                               [0], 1.0, True)
            return time.perf_counter() - t0
        finally:
            o._lib = saved

    def half(self, which):
        """Time the first (which=0) or second half of each leg's sample."""
        for leg, lib in (("serial", self.serial), ("multi", self.omp)):
            rs = self.reqs[leg]
            part = rs[:len(rs) // 2] if which == 0 else rs[len(rs) // 2:]
            for r in part:
                self.time[leg] += self._one(lib, r)
                self.done[leg] += 1

    def result(self):
        L = self.seq_len
        model = cpu_model()

        def leg(name, cores, kind):
            n, t = self.done[name], self.time[name]
            return {"value": n * L / t, "unit": "tokens/s", "cores": cores, "kind": kind,
                    "sample": "%d of the 128 requests, %d tokens each (1024 prompt + 127 decode forwards), one GDN "
                              "layer, whole-sequence oracle passes (conv, bf16 rounding, gated delta rule) in fp64; "
                              "%.1f s, half before and half after the GPU timed region" % (n, L, t),
                    "cpu_model": model}
        out = leg("serial", 1, "oracle")
        out["multicore"] = leg("multi", self.cores, "oracle (the same source built with OpenMP: independent conv "
                                                    "channels and (sequence, v-head) pairs on separate threads)")
        return out


def step_call_kinds(n_decodes, n_prefills, layers):
    """The calls of one engine step in launch order: per layer, the varlen
    conv for prefill rows, then the recurrence -- the fused decode for a
    decode-only step, the chunkwise call for a prefill-only step, the
    one-grid call for a step with both."""
    per_layer = ["conv_varlen"] if n_prefills else []
    if n_decodes and n_prefills:
        per_layer.append("chunk_and_decode")
    elif n_decodes:
        per_layer.append("fused_decode")
    elif n_prefills:
        per_layer.append("recurrent_chunk")
    return per_layer * layers


def bracket_runs(kinds, kind, single_stride=1):
    """Events that bracket maximal runs of consecutive ``kind`` launches in
    ``kinds`` (the kind of every launch of a pass, as (step, call) -> kind
    lists, in launch order): every run of several launches, and every
    ``single_stride``-th run of one launch.  Returns the bracket map
    ((step, call) -> "open" / "close" / "both"), the number of events, each
    bracketed run's weight (1 for a long run; for the others, the number of
    one-launch runs per bracketed one, so the weighted sum of the spans
    estimates the kind's total time) and the number of launches inside the
    bracketed runs.  Kernels on one stream run back to back, so a run's span
    is the sum of its kernels' durations plus the (sub-microsecond) dispatch
    gaps between them."""
    runs, cur = [], None
    for si, step in enumerate(kinds):
        for ci, k in enumerate(step):
            if k == kind:
                if cur is None:
                    cur = []
                    runs.append(cur)
                cur.append((si, ci))
            else:
                cur = None
    singles = [r for r in runs if len(r) == 1]
    picked_singles = singles[::single_stride]
    w_single = len(singles) / max(len(picked_singles), 1)
    keep = {id(r) for r in picked_singles}
    picked = [r for r in runs if len(r) > 1 or id(r) in keep]
    br = {}
    for run in picked:
        if len(run) == 1:
            br[run[0]] = "both"
        else:
            br[run[0]], br[run[-1]] = "open", "close"
    weights = [1.0 if len(r) > 1 else w_single for r in picked]
    return br, 2 * len(picked), weights, sum(len(r) for r in picked)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (the GDN mixer shards by sequence or head "
              "group with no exchange inside the path); --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_token_amd as gdn
    import synth

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}))
        return

    lib = gdn.lib
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    trace = synth.engine_trace_schedule(args.seed)
    steps = trace.steps
    _, offs = synth.trace_step_rows(trace)
    T_all = int(offs[-1])
    L = args.layers

    # ---- per-step metadata (host and device), built before the timed region
    dec_idx, pf_qsl, pf_idx, pf_hi, n_chunks = [], [], [], [], []
    for st in steps:
        dec_idx.append(np.array([s for (_r, _p, s) in st.decodes], np.int32))
        lens = [n for (_r, _p0, n, _s, _h) in st.prefills]
        pf_qsl.append(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32))
        pf_idx.append(np.array([s for (_r, _p0, _n, s, _h) in st.prefills], np.int32))
        pf_hi.append(np.array([h for (_r, _p0, _n, _s, h) in st.prefills], np.uint8))
        n_chunks.append(sum((n + 7) // 8 for n in lens))

    def pack(arrs, dtype):
        offs_ = np.concatenate([[0], np.cumsum([len(a) for a in arrs])]).astype(np.int64)
        flat = np.concatenate(arrs).astype(dtype) if offs_[-1] else np.zeros(1, dtype)
        t = torch.from_numpy(flat).to(dev)
        return t, offs_

    dec_idx_d, dec_off = pack(dec_idx, np.int32)
    qsl_d, qsl_off = pack(pf_qsl, np.int32)
    pidx_d, pidx_off = pack(pf_idx, np.int32)
    phi_d, phi_off = pack(pf_hi, np.uint8)
    ch_off = np.concatenate([[0], np.cumsum(n_chunks)]).astype(np.int64)
    ch_host = torch.zeros(int(ch_off[-1]) * 2, dtype=torch.int32, pin_memory=True)
    ch_dev = torch.zeros(int(ch_off[-1]) * 2, dtype=torch.int32, device=dev)
    qsl_host = [np.ascontiguousarray(q) for q in pf_qsl]

    # ---- per-layer weights, pools and activations (seeded, on the device)
    layers = []
    for li in range(L):
        gen = torch.Generator(device=dev)
        gen.manual_seed(1000 * args.seed + li)
        x = torch.empty(T_all, C, dtype=torch.bfloat16, device=dev)
        for a in range(0, T_all, 16384):
            e = min(T_all, a + 16384)
            x[a:e] = torch.randn(e - a, C, generator=gen, device=dev).to(torch.bfloat16)
        g = -torch.nn.functional.softplus(torch.randn(T_all, HV, generator=gen, device=dev))
        beta = torch.sigmoid(torch.randn(T_all, HV, generator=gen, device=dev))
        w = (0.5 * torch.randn(C, K, generator=gen, device=dev)).to(torch.bfloat16)
        b = (0.1 * torch.randn(C, generator=gen, device=dev)).to(torch.bfloat16)
        layers.append(dict(
            x=x, g=g.contiguous(), beta=beta.contiguous(), w=w, b=b,
            cs=torch.zeros(SLOTS, 3, C, dtype=torch.bfloat16, device=dev),
            state=torch.zeros(SLOTS, HV, D, D, dtype=torch.float32, device=dev),
            y=torch.empty(BUDGET, C, dtype=torch.bfloat16, device=dev),
            o=torch.empty(T_all, HV, D, dtype=torch.bfloat16, device=dev)))
    torch.cuda.synchronize()

    # scratch of the chunkwise recurrence, sized for the largest prefill step
    # and shared by every call (they are ordered on one stream)
    ws_bytes = max(gdn.gdn_chunk_workspace_size(len(pf_idx[i]), steps[i].n_tokens - len(steps[i].decodes), HK, HV)
                   for i in range(len(steps)))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    # ---- launch lists: (kind, fn, args, bytes, flops) per engine step
    i32 = np.dtype(np.int32).itemsize
    plans = []
    for si, st in enumerate(steps):
        nd, npf = len(st.decodes), len(st.prefills)
        tp = st.n_tokens - nd
        off = int(offs[si])
        calls = []
        for ly in layers:
            X, Y, O = ly["x"].data_ptr(), ly["y"].data_ptr(), ly["o"].data_ptr()
            G, B = ly["g"].data_ptr(), ly["beta"].data_ptr()
            yq, yk, yv = Y, Y + HK * D * 2, Y + 2 * HK * D * 2
            di = dec_idx_d.data_ptr() + int(dec_off[si]) * i32
            if nd and not npf:
                # decode rows: conv update fused with the recurrence (one launch)
                calls.append(("fused_decode", lib.gdn_fused_conv_decode,
                              (X + off * C * 2, C, ly["w"].data_ptr(), ly["b"].data_ptr(), ly["cs"].data_ptr(),
                               SLOTS, G + off * HV * 4, B + off * HV * 4, ly["state"].data_ptr(), SLOTS, di,
                               O + off * HV * D * 2, HV * D, None, 0, nd, HK, HV, D, D, 1, ctypes.c_float(1.0),
                               1, sptr),
                              bytes_fused_decode(nd), flops_recurrent(nd)))
            if npf:
                qd = qsl_d.data_ptr() + int(qsl_off[si]) * i32
                pi = pidx_d.data_ptr() + int(pidx_off[si]) * i32
                ph = phi_d.data_ptr() + int(phi_off[si])
                cd = ch_dev.data_ptr() + int(ch_off[si]) * 2 * i32
                n_init = int(pf_hi[si].sum())
                calls.append(("conv_varlen", lib.gdn_causal_conv1d_varlen,
                              (X + (off + nd) * C * 2, C, ly["w"].data_ptr(), ly["b"].data_ptr(),
                               ly["cs"].data_ptr(), SLOTS, qd, pi, ph, cd, n_chunks[si], Y + nd * C * 2, C,
                               npf, tp, C, K, 1, sptr),
                              bytes_conv_varlen(tp, npf, n_init, n_chunks[si]), 0.0))
            if npf and nd:
                # the prefill chunks' recurrence and the decode rows (conv update
                # + recurrence) in one call, after the prefill conv
                po = off + nd
                calls.append(("chunk_and_decode", lib.gdn_chunk_rule_and_fused_decode,
                              (yq + nd * C * 2, C, yk + nd * C * 2, C, yv + nd * C * 2, C, G + po * HV * 4,
                               B + po * HV * 4, qd, pi, ph, O + po * HV * D * 2, HV * D, npf, tp, ws.data_ptr(),
                               ws_bytes, X + off * C * 2, C, ly["w"].data_ptr(), ly["b"].data_ptr(),
                               ly["cs"].data_ptr(), SLOTS, G + off * HV * 4, B + off * HV * 4, di,
                               O + off * HV * D * 2, HV * D, None, 0, nd, 1, ly["state"].data_ptr(), SLOTS,
                               HK, HV, D, D, ctypes.c_float(1.0), 1, sptr),
                              bytes_recurrent(tp, n_init, npf) + bytes_fused_decode(nd),
                              flops_recurrent(tp) + flops_recurrent(nd)))
            elif npf:
                po = off + nd
                calls.append(("recurrent_chunk", lib.gdn_chunk_gated_delta_rule,
                              (yq + nd * C * 2, C, yk + nd * C * 2, C, yv + nd * C * 2, C, G + po * HV * 4,
                               B + po * HV * 4, ly["state"].data_ptr(), SLOTS, qd, pi, ph,
                               O + po * HV * D * 2, HV * D, npf, tp, HK, HV, D, D, ws.data_ptr(), ws_bytes,
                               ctypes.c_float(1.0), 1, sptr),
                              bytes_recurrent(tp, n_init, npf), flops_recurrent(tp)))
        assert [c[0] for c in calls] == step_call_kinds(nd, npf, L)
        plans.append(calls)

    ch_host_ptr = ch_host.data_ptr()
    n_out = ctypes.c_int32()

    def run_pass(timing=None):
        """One pass of the whole trace through every layer.

        ``timing`` (optional) is ``(brackets, events)``: ``brackets`` maps a
        (step, call) position to "open", "close" or "both", and an event from
        the pre-created list ``events`` is recorded on the launch stream
        before an opening and after a closing launch."""
        brackets, events = timing if timing is not None else ({}, None)
        ev = 0
        for si, calls in enumerate(plans):
            if n_chunks[si]:
                # the step's chunk descriptors: built once on the host, uploaded once
                a = int(ch_off[si])
                rc = lib.gdn_build_conv_chunks(qsl_host[si].ctypes.data, len(pf_idx[si]),
                                               ctypes.c_void_p(ch_host_ptr + a * 2 * i32), n_chunks[si],
                                               ctypes.byref(n_out))
                if rc != 0:
                    raise RuntimeError("gdn_build_conv_chunks: " + lib.gdn_last_error().decode())
                ch_dev[2 * a:2 * (a + n_chunks[si])].copy_(ch_host[2 * a:2 * (a + n_chunks[si])],
                                                            non_blocking=True)
            for ci, (kind, fn, fargs, _nb, _nf) in enumerate(calls):
                br = brackets.get((si, ci))
                if br in ("open", "both"):
                    events[ev].record(stream)
                    ev += 1
                rc = fn(*fargs)
                if rc != 0:
                    raise RuntimeError("%s: %s" % (kind, lib.gdn_last_error().decode()))
                if br in ("close", "both"):
                    events[ev].record(stream)
                    ev += 1
        return ev

    plan_kinds = [[c[0] for c in calls] for calls in plans]

    def span_ms(events, weights):
        return sum(w * events[2 * i].elapsed_time(events[2 * i + 1]) for i, w in enumerate(weights))

    def totals(kind):
        calls_of = [c for calls in plans for c in calls if c[0] == kind]
        return len(calls_of), sum(c[3] for c in calls_of), sum(c[4] for c in calls_of)

    kinds = [k for k in ("conv_varlen", "fused_decode", "recurrent_chunk", "chunk_and_decode")
             if any(k in ks for ks in plan_kinds)]

    # ---- what one recorded event costs: each idles the stream for a few us
    # on this GPU, and a bracketed run's span includes that idle time.  N
    # fixed-length spin kernels timed as one run, then each inside its own
    # event pair: the difference per pair is subtracted from every bracketed
    # span below.
    def event_cost_us(n=40, cycles=20000):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            torch.cuda._sleep(cycles)
        e1.record(stream)
        pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a_, b_ in pairs:
            a_.record(stream)
            torch.cuda._sleep(cycles)
            b_.record(stream)
        torch.cuda.synchronize()
        whole = e0.elapsed_time(e1) / n
        each = sum(a_.elapsed_time(b_) for a_, b_ in pairs) / n
        return max(0.0, 1e3 * (each - whole))

    # ---- warm-up, then one instrumented pass (untimed) per call kind for the
    # per-kernel figures
    for _ in range(args.warmup):
        run_pass()
    torch.cuda.synchronize()
    ev_cost = sorted(event_cost_us() for _ in range(5))[2]
    kern = {}
    for k in kinds:
        br, n_ev, wts, _ = bracket_runs(plan_kinds, k)
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        run_pass((br, evs))
        torch.cuda.synchronize()
        raw = span_ms(evs, wts)
        ms = raw - 1e-3 * ev_cost * sum(wts)
        n, nb, nf = totals(k)
        kern[k] = {"launches_per_step": n, "ms_per_step": ms, "avg_us": 1e3 * ms / max(n, 1),
                   "avg_us_events_raw": 1e3 * raw / max(n, 1), "bracketed_runs": n_ev // 2,
                   "gb_per_s": nb / (ms * 1e-3) / 1e9 if ms else 0.0,
                   "hbm_frac": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS if ms else 0.0}
        if nf:
            kern[k]["tflop_per_s"] = nf / (ms * 1e-3) / 1e12
    dominant = max(kinds, key=lambda k: kern[k]["ms_per_step"])

    cpu = None
    if not args.no_cpu_baseline:
        # first half of the oracle's sample before the GPU's timed region
        cpu = CpuBaseline(args.seed, trace.seq_len, args.cpu_sample_requests, args.cpu_multicore_requests)
        cpu.half(0)

    # ---- timed region: the dominant kernel's runs bracketed by pre-created
    # events -- every long run, and every ROOFLINE_STRIDE-th one-launch run
    # (weighted), a stratified estimate of its total time.  Each recorded
    # event idles the stream for ~5 us on this GPU: bracketing all ~280 runs
    # of a pass cost ~2% of the measured throughput.
    br, n_ev, wts, n_timed = bracket_runs(plan_kinds, dominant, ROOFLINE_STRIDE)
    live = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_pass((br, live[i]))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    if cpu is not None:
        cpu.half(1)

    ms_dom = sum(span_ms(evs, wts) for evs in live) / args.steps - 1e-3 * ev_cost * sum(wts)
    n, nb, nf = totals(dominant)
    avg_us = 1e3 * ms_dom / n
    sample_note = ("events around every run of several consecutive launches and every %dth one-launch run "
                   "(weighted): estimated total time of all %d launches per step, less the measured cost of "
                   "each event pair (%.2f us)" % (ROOFLINE_STRIDE, n, ev_cost))
    if dominant == "recurrent_chunk":
        # matrix-core kernel (bf16 MFMA, fp32 operands split hi+lo); algorithmic
        # flops of the rule against the dense bf16 MFMA peak
        achieved = nf / (ms_dom * 1e-3) / 1e12
        roof = {"kernel": dominant, "bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS, "traffic": None,
                "avg_launch_us": avg_us, "algorithmic_per_launch": nf / n, "timed_runs_per_step": n_ev // 2,
                "timed_launches_per_step": n_timed, "launches_per_step": n, "timing_sample": sample_note}
    else:
        achieved = nb / (ms_dom * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_per_launch(dominant),
                "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "avg_launch_us": avg_us, "algorithmic_per_launch": nb / n, "timed_runs_per_step": n_ev // 2,
                "timed_launches_per_step": n_timed, "launches_per_step": n, "timing_sample": sample_note}

    ms_per_step = 1e3 * wall / args.steps
    value = T_all * L * args.steps / wall
    out = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp32", "io_dtype": "bf16",
        "dtype_detail": "bf16 activations and outputs (RNE); fp32 recurrent state and vector arithmetic "
                        "(conv, decode); the chunkwise prefill's matrix products on bf16 MFMA with every fp32 "
                        "operand split into hi + lo bf16 parts (16 significant bits) and fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": "c32 engine-step trace: 128 requests x (1024 prompt + 128 output tokens), "
                               "concurrency 32, 2048-token chunked-prefill budget, %d engine steps, "
                               "%d tokens per layer, %d GDN layers" % (len(steps), T_all, L),
                   "engine_steps": len(steps), "tokens_per_layer": T_all, "gdn_layers": L,
                   "conv_channels": C, "conv_width": K, "qk_heads": HK, "v_heads": HV, "head_dim": D,
                   "state_slots": SLOTS, "value_is": "tokens x layers / wall seconds"},
        "roofline": roof,
        "kernels": kern,
        "event_pair_cost_us": ev_cost,
        "context": PAGES_CONTEXT,
    }
    if not args.no_isolated:
        out["isolated"] = isolated(args.seed)
        ceil = out["isolated"].get(dominant, {}).get("ceiling")
        if ceil and roof["unit"] == "GB/s":
            roof["ceiling"] = dict(ceil, frac_of_ceiling=roof["achieved"] / ceil["gb_per_s"])
    if cpu is not None:
        out["cpu_baseline"] = cpu.result()
    line = json.dumps(out)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
