"""Host-side logic of bench.py (no GPU): algorithmic byte counts, the
traffic records tied to kernel sources, and the one-GPU contract."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_bytes_at_the_c32_shapes(bench):
    # 2 x 1024 prefill: x read + y write, two slots written, weights, bias, descriptors, qsl, indices, flags
    assert bench.bytes_conv_varlen(2048, 2, 0, 256) == 67_291_158
    # 32-sequence decode: fp32 state read + written (2 x 32 x 2 MiB), q/k/v, o, g, beta
    assert bench.bytes_recurrent(32, 32, 32) == 135_012_352
    # fused decode adds the conv update's x, conv_state read + write, weights
    assert bench.bytes_fused_decode(32) == bench.bytes_recurrent(32, 32, 32) - 32 * (2 * 16 * 128 + 32 * 128) * 2 \
        + 32 * (8192 * 2 + 2 * 3 * 8192 * 2 + 4) + 8192 * 4 * 2 + 8192 * 2
    assert bench.flops_recurrent(1) == 6 * 32 * 128 * 128


def test_traffic_record_follows_the_sources(bench, tmp_path, monkeypatch):
    digest = bench.sources_digest("fused_decode")
    rec = tmp_path / "traffic.md"
    rec.write_text("text\ntraffic-record kernel=fused_decode fetch_bytes=10 write_bytes=5 sources=%s\n"
                   "traffic-record kernel=conv_varlen fetch_bytes=1 write_bytes=1 sources=0000000000000000\n"
                   % digest)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.traffic_per_launch("fused_decode") == 15
    assert bench.traffic_per_launch("conv_varlen") is None          # measured on other sources
    assert bench.traffic_per_launch("recurrent_chunk") is None      # never measured
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.traffic_per_launch("fused_decode") is None


def test_sources_digest_changes_with_a_kernel_file(bench, tmp_path, monkeypatch):
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    for name in bench.KERNEL_SOURCES["conv_varlen"]:
        (csrc / name).write_text("// " + name)
    monkeypatch.setattr(bench, "_CSRC", str(csrc))
    d0 = bench.sources_digest("conv_varlen")
    (csrc / "conv.hip").write_text("// conv.hip changed")
    assert bench.sources_digest("conv_varlen") != d0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_bracket_runs_stratified_sample(bench):
    # a pass: a run of three F launches, ten one-launch runs of F (each
    # followed by another kind), then another run of three
    kinds = [["F", "F"], ["F", "C"]] + [["F", "R"] for _ in range(10)] + [["C", "F", "F", "F"]]
    br, n_ev, w, n_timed = bench.bracket_runs(kinds, "F", 1)
    assert n_ev == 2 * 12 and w == [1.0] * 12 and n_timed == 3 + 10 + 3
    assert br[(0, 0)] == "open" and br[(1, 0)] == "close"
    assert br[(12, 1)] == "open" and br[(12, 3)] == "close"
    assert all(br[(s, 0)] == "both" for s in range(2, 12))
    br, n_ev, w, n_timed = bench.bracket_runs(kinds, "F", 3)
    # both long runs, and one-launch runs 0, 3, 6 and 9 of the ten (steps 2, 5, 8, 11)
    assert n_ev == 2 * 6 and n_timed == 3 + 4 + 3
    assert sorted(k for k, v in br.items() if v == "both") == [(2, 0), (5, 0), (8, 0), (11, 0)]
    assert w == [1.0, 2.5, 2.5, 2.5, 2.5, 1.0]
    # with equal launch durations the weighted spans give the exact total
    d = 7.0
    spans = [3 * d, d, d, d, d, 3 * d]
    assert sum(x * y for x, y in zip(w, spans)) == pytest.approx(16 * d)
    # events come in launch order: opens and closes alternate
    flat = [e for k in sorted(br) for e in (("open", "close") if br[k] == "both" else (br[k],))]
    assert flat == ["open", "close"] * 6


def test_plan_of_the_c32_trace(bench):
    """The calls the bench makes over the c32 trace: one fused decode per
    layer of a decode-only step, the conv and the one-grid call per layer of
    a step with both kinds of rows.  The fused decode's launches then form
    only runs of several launches (the decode-only stretches), so the
    timed region brackets every one of them, each run with weight 1."""
    import synth
    tr = synth.engine_trace_schedule(0)
    L = 4
    kinds = [bench.step_call_kinds(len(st.decodes), len(st.prefills), L) for st in tr.steps]
    flat = [k for ks in kinds for k in ks]
    n_dec_only = sum(1 for st in tr.steps if st.decodes and not st.prefills)
    n_mixed = sum(1 for st in tr.steps if st.decodes and st.prefills)
    n_pre_only = sum(1 for st in tr.steps if st.prefills and not st.decodes)
    assert n_dec_only + n_mixed + n_pre_only == len(tr.steps) == 529
    assert flat.count("fused_decode") == L * n_dec_only
    assert flat.count("chunk_and_decode") == L * n_mixed
    assert flat.count("recurrent_chunk") == L * n_pre_only
    assert flat.count("conv_varlen") == L * (n_mixed + n_pre_only)
    br, n_ev, wts, n_timed = bench.bracket_runs(kinds, "fused_decode", bench.ROOFLINE_STRIDE)
    assert n_timed == flat.count("fused_decode")
    assert wts and all(w == 1.0 for w in wts)
    assert n_ev == 2 * len(wts) == 8          # four decode-only stretches
