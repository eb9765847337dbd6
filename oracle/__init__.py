"""Plain serial double-precision CPU oracle for the GDN token-mixer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this package:
only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` call it.  The arithmetic lives in ``gdn_oracle.c`` (plain C,
fp64, serial); this module only marshals numpy arrays through ctypes.

Sources (restated in ``gdn_oracle.c``): chunk descriptors from page
"perf(gdn): dispatch exact causal-conv chunks", section "What changed"; the
width-4 conv from page "RTX 5070 Ti: close Qwen3.5-4B TTFT, TPOT, and VRAM
gaps vs vLLM", section "Existing evidence"; the gated delta rule from Yang,
Kautz, Hatamizadeh, "Gated Delta Networks: Improving Mamba2 with Delta Rule"
(ICLR 2025), recurrent form.

bf16 tensors are numpy ``uint16`` arrays of raw bf16 bits.  Outputs are
float64 and unrounded.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
# the same source built with OpenMP: only the benchmark's multi-core CPU
# baseline loads it (same results; independent iterations on several threads)
_LIB_OMP = os.path.join(_HERE, "libgdn_oracle_omp.so")
_FLAGS = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall",
          "-Wextra"]

_lib = None


def _compile(lib, extra, force):
    if force or not os.path.exists(lib) or os.path.getmtime(lib) < os.path.getmtime(_SRC):
        tmp = lib + ".tmp%d" % os.getpid()
        subprocess.check_call(_FLAGS + extra + ["-o", tmp, _SRC, "-lm"])
        os.replace(tmp, lib)
    return lib


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE double, no FMA contraction), serial:
    its OpenMP pragmas are ignored."""
    return _compile(_LIB, ["-Wno-unknown-pragmas"], force)


def build_omp(force: bool = False) -> str:
    """The same oracle compiled with OpenMP (for the multi-core CPU baseline)."""
    return _compile(_LIB_OMP, ["-fopenmp"], force)


def bind(path: str):
    """Load an oracle shared library from ``path`` and declare its signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_build_conv_chunks.argtypes = [P, i32, P, i32, P]
    lib.oracle_build_conv_chunks.restype = ctypes.c_int
    lib.oracle_causal_conv1d_varlen.argtypes = [
        P, i64, P, P, P, i32, P, P, P, P, i64, i32, i32, i32, i32]
    lib.oracle_causal_conv1d_varlen.restype = None
    lib.oracle_causal_conv1d_update.argtypes = [
        P, i64, P, P, P, i32, P, P, i64, i32, i32, i32, i32]
    lib.oracle_causal_conv1d_update.restype = None
    lib.oracle_gated_delta_rule.argtypes = [
        P, i64, P, i64, P, i64, P, P, P, i32, P, P, P, P, i64,
        i32, i32, i32, i32, i32, dbl, i32]
    lib.oracle_gated_delta_rule.restype = None
    lib.oracle_round_bf16.argtypes = [P, P, i64]
    lib.oracle_round_bf16.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = bind(build())
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a), dtype=dtype)


def _rows(a, name):
    """A 2-D array whose rows may be strided but whose elements are packed."""
    if a.ndim == 2 and a.shape[0] <= 1:
        return a.shape[1]
    if a.ndim != 2 or a.strides[1] != a.itemsize or a.strides[0] % a.itemsize:
        raise ValueError("%s must be 2-D with contiguous rows" % name)
    return a.strides[0] // a.itemsize


def build_conv_chunks(qsl, capacity=None):
    """Return the (sequence, chunk) descriptor list as an int32 [n, 2] array."""
    lib = _load()
    qsl = _c(qsl, np.int32)
    ns = qsl.size - 1
    n = ctypes.c_int32(0)
    rc = lib.oracle_build_conv_chunks(_ptr(qsl), ns, None, 0, ctypes.byref(n))
    if rc not in (0, -3):
        raise ValueError("oracle_build_conv_chunks: invalid query_start_loc")
    cap = n.value if capacity is None else capacity
    out = np.zeros((max(cap, 1), 2), np.int32)
    rc = lib.oracle_build_conv_chunks(_ptr(qsl), ns, _ptr(out), cap, ctypes.byref(n))
    if rc != 0:
        raise ValueError("oracle_build_conv_chunks failed: %d" % rc)
    return out[: n.value].copy()


def causal_conv1d_varlen(x, weight, bias, conv_state, qsl, state_indices,
                         has_initial_state=None, silu=True):
    """Varlen causal conv.  Returns (y float64 [T][C] with NaN where nothing
    was written, new conv_state uint16 [slots][K-1][C])."""
    lib = _load()
    x = np.asarray(x, np.uint16)
    xs = _rows(x, "x")
    T, C = x.shape
    w = _c(weight, np.uint16)
    K = w.shape[1]
    b = _c(bias, np.uint16)
    st = np.array(conv_state, np.uint16, copy=True, order="C")
    qsl = _c(qsl, np.int32)
    idx = _c(state_indices, np.int32)
    hi = _c(has_initial_state, np.uint8)
    y = np.full((T, C), np.nan)
    lib.oracle_causal_conv1d_varlen(_ptr(x), xs, _ptr(w), _ptr(b), _ptr(st), st.shape[0],
                                    _ptr(qsl), _ptr(idx), _ptr(hi), _ptr(y), C,
                                    qsl.size - 1, C, K, int(bool(silu)))
    return y, st


def causal_conv1d_update(x, weight, bias, conv_state, state_indices, silu=True):
    """Single-token conv update.  Returns (y float64 [B][C], new conv_state)."""
    lib = _load()
    x = np.asarray(x, np.uint16)
    xs = _rows(x, "x")
    B, C = x.shape
    w = _c(weight, np.uint16)
    K = w.shape[1]
    b = _c(bias, np.uint16)
    st = np.array(conv_state, np.uint16, copy=True, order="C")
    idx = _c(state_indices, np.int32)
    y = np.full((B, C), np.nan)
    lib.oracle_causal_conv1d_update(_ptr(x), xs, _ptr(w), _ptr(b), _ptr(st), st.shape[0],
                                    _ptr(idx), _ptr(y), C, B, C, K, int(bool(silu)))
    return y, st


def _heads(a, name):
    """[T][H][d] array with packed heads; returns the token stride (elements)."""
    if a.ndim == 3 and a.shape[0] <= 1 and a.flags.c_contiguous:
        return a.shape[1] * a.shape[2]
    if a.ndim != 3 or a.strides[2] != 2 or a.strides[1] != 2 * a.shape[2] or a.strides[0] % 2:
        raise ValueError("%s must be [T][H][d] with packed heads" % name)
    return a.strides[0] // 2


def gated_delta_rule(q, k, v, g, beta, state, state_indices, qsl=None,
                     has_initial_state=None, scale=1.0, qk_l2norm=True):
    """Gated delta rule over packed tokens.

    q, k: uint16 [T][HK][dk]; v: uint16 [T][HV][dv] (token rows may be strided
    views of a wider activation); g, beta: float32 [T][HV]; state: float
    [slots][HV][dv][dk] (copied to float64).  Returns (o float64 [T][HV][dv]
    with NaN where nothing was written, new state float64).
    """
    lib = _load()
    q = np.asarray(q, np.uint16)
    k = np.asarray(k, np.uint16)
    v = np.asarray(v, np.uint16)
    qs, ks, vs = _heads(q, "q"), _heads(k, "k"), _heads(v, "v")
    T, HK, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    g = _c(g, np.float32)
    beta = _c(beta, np.float32)
    st = np.array(state, np.float64, copy=True, order="C")
    idx = _c(state_indices, np.int32)
    qsl_c = _c(qsl, np.int32)
    hi = _c(has_initial_state, np.uint8)
    ns = idx.size
    o = np.full((T, HV, dv), np.nan)
    lib.oracle_gated_delta_rule(_ptr(q), qs, _ptr(k), ks, _ptr(v), vs, _ptr(g), _ptr(beta),
                                _ptr(st), st.shape[0], _ptr(qsl_c), _ptr(idx), _ptr(hi),
                                _ptr(o), HV * dv, ns, HK, HV, dk, dv, float(scale),
                                int(bool(qk_l2norm)))
    return o, st


def round_bf16(a):
    """float64 -> bf16 bits, round to nearest even."""
    lib = _load()
    a = np.ascontiguousarray(a, np.float64)
    out = np.empty(a.shape, np.uint16)
    lib.oracle_round_bf16(_ptr(a), _ptr(out), a.size)
    return out
