"""Python binding of libgdn, the MI355X (gfx950) GDN token-mixer library.

Argument marshalling only: every step of the path runs in the HIP kernels of
``libgdn.so`` (built in-tree by ``gated_deltanet_token_amd/build.py``), reached
through its C ABI (``include/gdn.h``).  PyTorch supplies device memory and
streams.  There is no fallback: importing this package without the built
library raises ``ImportError``.

bf16 tensors are ``torch.bfloat16``; token rows may be strided views (the
last dimension must be contiguous).  Calls are asynchronous on the current
torch stream unless ``stream`` is given.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_OK, GDN_ERR_INVALID, GDN_ERR_UNSUPPORTED, GDN_ERR_CAPACITY, GDN_ERR_HIP = 0, -1, -2, -3, -4
CONV_CHUNK_TOKENS = 8
CONV_WIDTH = 4

# every entry point declared in include/gdn.h
EXPORTS = ("gdn_last_error", "gdn_build_conv_chunks", "gdn_causal_conv1d_varlen", "gdn_causal_conv1d_varlen_tiles",
           "gdn_causal_conv1d_update", "gdn_fused_recurrent_decode", "gdn_chunk_gated_delta_rule",
           "gdn_fused_conv_decode", "gdn_chunk_workspace_size", "gdn_chunk_rule_and_fused_decode",
           "gdn_chunk_rule_and_fused_decode_noalloc")
# bytes of the static device scratch gdn_chunk_rule_and_fused_decode_noalloc uses (gdn.h)
NOALLOC_SCRATCH_BYTES = 64 << 20


class GDNError(RuntimeError):
    def __init__(self, code, func, message):
        super().__init__("%s failed (%d): %s" % (func, code, message))
        self.code = code


def _bind(path):
    lib = ctypes.CDLL(path)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_build_conv_chunks.argtypes = [P, i32, P, i32, P]
    lib.gdn_causal_conv1d_varlen.argtypes = [P, i64, P, P, P, i32, P, P, P, P, i32, P, i64,
                                             i32, i32, i32, i32, i32, P]
    lib.gdn_causal_conv1d_varlen_tiles.argtypes = [P, i64, P, P, P, i32, P, P, P, P, i32, P, i64,
                                                   i32, i32, i32, i32, i32, i32, P]
    lib.gdn_causal_conv1d_update.argtypes = [P, i64, P, P, P, i32, P, P, i64, i32, i32, i32, i32, P]
    lib.gdn_fused_recurrent_decode.argtypes = [P, i64, P, i64, P, i64, P, P, P, i32, P, P, P, P, i64,
                                               i32, i32, i32, i32, i32, i32, f32, i32, P]
    lib.gdn_chunk_gated_delta_rule.argtypes = [P, i64, P, i64, P, i64, P, P, P, i32, P, P, P, P, i64,
                                               i32, i32, i32, i32, i32, i32, P, ctypes.c_size_t, f32, i32, P]
    for name in EXPORTS[1:]:
        if name != "gdn_chunk_workspace_size":
            getattr(lib, name).restype = ctypes.c_int
    lib.gdn_fused_conv_decode.argtypes = [P, i64, P, P, P, i32, P, P, P, i32, P, P, i64, P, i64,
                                          i32, i32, i32, i32, i32, i32, f32, i32, P]
    lib.gdn_chunk_rule_and_fused_decode.argtypes = [
        P, i64, P, i64, P, i64, P, P, P, P, P, P, i64, i32, i32, P, ctypes.c_size_t,   # prefill tokens
        P, i64, P, P, P, i32, P, P, P, P, i64, P, i64, i32, i32,                       # decode rows
        P, i32, i32, i32, i32, i32, f32, i32, P]                                       # shared
    lib.gdn_chunk_rule_and_fused_decode_noalloc.argtypes = [
        P, i64, P, i64, P, i64, P, P, P, P, P, P, i64, i32, i32,                        # prefill tokens
        P, i64, P, P, P, i32, P, P, P, P, i64, P, i64, i32, i32,                       # decode rows
        P, i32, i32, i32, i32, i32, f32, i32, P]                                       # shared
    lib.gdn_chunk_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.gdn_chunk_workspace_size.restype = ctypes.c_size_t
    return lib


def _hip_runtimes():
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln})
    except OSError:
        return []


if not os.path.exists(LIB_PATH):
    raise ImportError("libgdn.so is not built (%s); run python gated_deltanet_token_amd/build.py"
                      % LIB_PATH)
# torch's HIP runtime must be the process's only one: load it first so that
# libgdn's libamdhip64.so.7 dependency resolves to it (by soname)
import torch  # noqa: E402,F401

lib = _bind(LIB_PATH)
if len(_hip_runtimes()) > 1:
    raise ImportError("two HIP runtimes are loaded (%s); libgdn must share torch's"
                      % ", ".join(_hip_runtimes()))


def _check(rc, func):
    if rc != GDN_OK:
        raise GDNError(rc, func, lib.gdn_last_error().decode())


# ---------------------------------------------------------------------------
# host call
# ---------------------------------------------------------------------------

def gdn_build_conv_chunks(query_start_loc_host) -> np.ndarray:
    """Exact (sequence, 8-token chunk) descriptors as an int32 [n, 2] array
    (layout of ``gdn_conv_chunk``), built on the host."""
    qsl = np.ascontiguousarray(np.asarray(query_start_loc_host), dtype=np.int32)
    ns = qsl.size - 1
    n = ctypes.c_int32(0)
    rc = lib.gdn_build_conv_chunks(qsl.ctypes.data, ns, None, 0, ctypes.byref(n))
    if rc not in (GDN_OK, GDN_ERR_CAPACITY):
        _check(rc, "gdn_build_conv_chunks")
    out = np.empty((max(n.value, 1), 2), np.int32)
    _check(lib.gdn_build_conv_chunks(qsl.ctypes.data, ns, out.ctypes.data, n.value, ctypes.byref(n)),
           "gdn_build_conv_chunks")
    return out[: n.value]


# ---------------------------------------------------------------------------
# GPU calls (torch tensors on the current HIP device)
# ---------------------------------------------------------------------------
# Every wrapper checks, before anything reaches the library: dtypes, the
# shapes the head arguments imply, contiguity where the ABI assumes packed
# data, and -- last, so that the shape checks can run without a GPU -- that
# every tensor lives on the current GPU.  A host tensor or an undersized
# buffer would otherwise reach the kernels as a wrong or short device range.

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _rows(t, name):
    """Token stride (elements) of a 2-D tensor with a contiguous last dim."""
    if t.dim() != 2 or (t.size(1) > 1 and t.stride(1) != 1):
        raise ValueError("%s must be 2-D with contiguous rows" % name)
    return t.stride(0) if t.size(0) > 1 else max(t.stride(0), t.size(1))


def _heads(t, name):
    """Token stride of a [T][H][d] tensor whose heads are packed."""
    if t.dim() != 3 or t.stride(2) != 1 or (t.size(1) > 1 and t.stride(1) != t.size(2)):
        raise ValueError("%s must be [T][H][d] with packed heads" % name)
    return t.stride(0) if t.size(0) > 1 else max(t.stride(0), t.size(1) * t.size(2))


def _dtype(t, dt, name):
    if t is not None and t.dtype != dt:
        raise TypeError("%s must be %s, got %s" % (name, dt, t.dtype))


def _shape(t, shape, name):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _dims(t, n, name):
    if t is not None and t.dim() != n:
        raise ValueError("%s must be %d-D, got shape %s" % (name, n, tuple(t.shape)))


def _contig(named):
    for name, t in named:
        if t is not None and not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


def _on_gpu(named):
    """Every tensor on the current HIP device (the library's calls address
    the current device's memory)."""
    torch = _torch()
    dev = None
    for name, t in named:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError("%s must be a GPU tensor, got one on %s" % (name, t.device))
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, the other operands on %s" % (name, t.device, dev))
    if dev is not None and dev.index is not None and dev.index != torch.cuda.current_device():
        raise ValueError("operands are on %s but the current device is cuda:%d"
                         % (dev, torch.cuda.current_device()))


def _workspace(workspace, need, device, stream):
    """The caller's workspace (checked), or one allocated for this call.  An
    allocated one is marked as used on ``stream`` so that the caching
    allocator does not hand its memory out again before the call's kernels
    on that stream are done with it."""
    torch = _torch()
    if workspace is not None:
        _dtype(workspace, torch.uint8, "workspace")
        _contig([("workspace", workspace)])
        if workspace.numel() < need:
            raise ValueError("workspace of %d bytes, %d needed" % (workspace.numel(), need))
        return workspace
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    if stream is not None:
        ws.record_stream(stream)
    return ws


def _check_conv(x, weight, bias, conv_state, y, rows_name="x"):
    torch = _torch()
    for t, n in ((x, "x"), (weight, "weight"), (bias, "bias"), (conv_state, "conv_state"), (y, "y")):
        _dtype(t, torch.bfloat16, n)
    _dims(x, 2, rows_name)
    T, C = x.shape
    _shape(y, (T, C), "y")
    _dims(weight, 2, "weight")
    if weight.shape[0] != C:
        raise ValueError("weight must have shape (%d, width), got %s" % (C, tuple(weight.shape)))
    _shape(bias, (C,), "bias")
    _dims(conv_state, 3, "conv_state")
    if tuple(conv_state.shape[1:]) != (CONV_WIDTH - 1, C):
        raise ValueError("conv_state must have shape (slots, %d, %d), got %s"
                         % (CONV_WIDTH - 1, C, tuple(conv_state.shape)))
    _contig([("weight", weight), ("bias", bias), ("conv_state", conv_state)])
    return T, C


def _check_index(t, n, name, dt):
    _dtype(t, dt, name)
    if t is not None:
        _dims(t, 1, name)
        if t.numel() != n:
            raise ValueError("%s must have %d entries, got %d" % (name, n, t.numel()))
        _contig([(name, t)])


def gdn_causal_conv1d_varlen(x, weight, bias, conv_state, query_start_loc, state_indices,
                             has_initial_state, chunks, y, silu=True, stream=None, descriptors_per_program=1):
    """Varlen causal conv (width 4) over packed tokens; see gdn.h.

    x, y: bf16 [T][C] (strided rows allowed); weight bf16 [C][4]; bias bf16
    [C] or None; conv_state bf16 [slots][3][C]; query_start_loc int32 [S+1];
    state_indices int32 [S]; has_initial_state uint8 [S] or None; chunks
    int32 [n][2] device tensor from gdn_build_conv_chunks (required when T > 0).
    descriptors_per_program: 1 (8-token programs, gdn_causal_conv1d_varlen)
    or 2 (16-token programs, gdn_causal_conv1d_varlen_tiles); same results.
    """
    torch = _torch()
    T, C = _check_conv(x, weight, bias, conv_state, y)
    _dims(state_indices, 1, "state_indices")
    S = state_indices.numel()
    _check_index(state_indices, S, "state_indices", torch.int32)
    _check_index(query_start_loc, S + 1, "query_start_loc", torch.int32)
    _check_index(has_initial_state, S, "has_initial_state", torch.uint8)
    _dtype(chunks, torch.int32, "chunks")
    if chunks is not None and (chunks.dim() != 2 or chunks.shape[1] != 2 or not chunks.is_contiguous()):
        raise ValueError("chunks must be a contiguous int32 [n][2] tensor, got shape %s" % (tuple(chunks.shape),))
    _on_gpu([("x", x), ("weight", weight), ("bias", bias), ("conv_state", conv_state),
             ("query_start_loc", query_start_loc), ("state_indices", state_indices),
             ("has_initial_state", has_initial_state), ("chunks", chunks), ("y", y)])
    n_chunks = 0 if chunks is None else chunks.shape[0]
    args = (_ptr(x), _rows(x, "x"), _ptr(weight), _ptr(bias), _ptr(conv_state), conv_state.shape[0],
            _ptr(query_start_loc), _ptr(state_indices), _ptr(has_initial_state),
            _ptr(chunks) if n_chunks else None, n_chunks, _ptr(y), _rows(y, "y"),
            S, T, C, weight.shape[1], int(bool(silu)))
    if descriptors_per_program == 1:
        _check(lib.gdn_causal_conv1d_varlen(*args, _stream(stream)), "gdn_causal_conv1d_varlen")
    else:
        _check(lib.gdn_causal_conv1d_varlen_tiles(*args, int(descriptors_per_program), _stream(stream)),
               "gdn_causal_conv1d_varlen_tiles")


def gdn_causal_conv1d_update(x, weight, bias, conv_state, state_indices, y, silu=True, stream=None):
    """Single-token conv update (decode); see gdn.h."""
    torch = _torch()
    B, C = _check_conv(x, weight, bias, conv_state, y)
    _check_index(state_indices, B, "state_indices", torch.int32)
    _on_gpu([("x", x), ("weight", weight), ("bias", bias), ("conv_state", conv_state),
             ("state_indices", state_indices), ("y", y)])
    rc = lib.gdn_causal_conv1d_update(
        _ptr(x), _rows(x, "x"), _ptr(weight), _ptr(bias), _ptr(conv_state), conv_state.shape[0],
        _ptr(state_indices), _ptr(y), _rows(y, "y"), B, C, weight.shape[1], int(bool(silu)),
        _stream(stream))
    _check(rc, "gdn_causal_conv1d_update")


def _check_rule(q, k, v, g, beta, state, o):
    """dtypes and shapes of a recurrence call's token tensors; returns
    (T, HK, dk, HV, dv)."""
    torch = _torch()
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _dtype(t, torch.bfloat16, n)
    for t, n in ((g, "g"), (beta, "beta"), (state, "state")):
        _dtype(t, torch.float32, n)
    _dims(q, 3, "q")
    _dims(v, 3, "v")
    T, HK, dk = q.shape
    HV, dv = v.shape[1], v.shape[2]
    _shape(k, (T, HK, dk), "k")
    _shape(v, (T, HV, dv), "v")
    _shape(o, (T, HV, dv), "o")
    _shape(g, (T, HV), "g")
    _shape(beta, (T, HV), "beta")
    _dims(state, 4, "state")
    if tuple(state.shape[1:]) != (HV, dv, dk):
        raise ValueError("state must have shape (slots, %d, %d, %d), got %s" % (HV, dv, dk, tuple(state.shape)))
    _contig([("g", g), ("beta", beta), ("state", state)])
    return T, HK, dk, HV, dv


def _recurrent(func, q, k, v, g, beta, state, state_indices, o, query_start_loc, has_initial_state, scale,
               qk_l2norm, stream, workspace=None):
    torch = _torch()
    T, HK, dk, HV, dv = _check_rule(q, k, v, g, beta, state, o)
    _dims(state_indices, 1, "state_indices")
    S = state_indices.numel()
    _check_index(state_indices, S, "state_indices", torch.int32)
    _check_index(query_start_loc, S + 1, "query_start_loc", torch.int32)
    _check_index(has_initial_state, S, "has_initial_state", torch.uint8)
    if query_start_loc is None and S != T:
        raise ValueError("without query_start_loc there is one token per sequence: %d tokens, %d sequences"
                         % (T, S))
    _on_gpu([("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state),
             ("state_indices", state_indices), ("o", o), ("query_start_loc", query_start_loc),
             ("has_initial_state", has_initial_state), ("workspace", workspace)])
    args = [_ptr(q), _heads(q, "q"), _ptr(k), _heads(k, "k"), _ptr(v), _heads(v, "v"), _ptr(g),
            _ptr(beta), _ptr(state), state.shape[0], _ptr(query_start_loc), _ptr(state_indices),
            _ptr(has_initial_state), _ptr(o), _heads(o, "o"), S, T, HK, HV, dk, dv]
    if func == "gdn_chunk_gated_delta_rule":
        workspace = _workspace(workspace, gdn_chunk_workspace_size(S, T, HK, HV), q.device, stream)
        args += [_ptr(workspace), workspace.numel()]
    args += [float(scale), int(bool(qk_l2norm)), _stream(stream)]
    _check(getattr(lib, func)(*args), func)


def gdn_fused_recurrent_decode(q, k, v, g, beta, state, state_indices, o, query_start_loc=None,
                               has_initial_state=None, scale=1.0, qk_l2norm=True, stream=None):
    """Gated delta rule over packed tokens, token by token; see gdn.h.

    q, k: bf16 [T][HK][dk]; v: bf16 [T][HV][dv] (token rows may be strided
    views of one wider activation); g, beta: fp32 [T][HV]; state: fp32
    [slots][HV][dv][dk] (in place); o: bf16 [T][HV][dv]; query_start_loc
    int32 [S+1] or None (one token per sequence, S = T).
    """
    _recurrent("gdn_fused_recurrent_decode", q, k, v, g, beta, state, state_indices, o, query_start_loc,
               has_initial_state, scale, qk_l2norm, stream)


def gdn_chunk_workspace_size(num_seqs, num_tokens, num_k_heads, num_v_heads) -> int:
    """Bytes of device scratch gdn_chunk_gated_delta_rule needs."""
    return int(lib.gdn_chunk_workspace_size(num_seqs, num_tokens, num_k_heads, num_v_heads))


def gdn_chunk_gated_delta_rule(q, k, v, g, beta, state, state_indices, o, query_start_loc,
                               has_initial_state=None, scale=1.0, qk_l2norm=True, stream=None,
                               workspace=None):
    """The same rule over packed prefill tokens, chunkwise on the matrix
    cores (dk = 128, dv a multiple of 32); see gdn.h.  ``workspace`` is a
    contiguous uint8 device tensor of at least gdn_chunk_workspace_size(...)
    bytes; when omitted, torch allocates one for the call."""
    if query_start_loc is None:
        raise ValueError("the chunkwise call needs query_start_loc")
    _recurrent("gdn_chunk_gated_delta_rule", q, k, v, g, beta, state, state_indices, o, query_start_loc,
               has_initial_state, scale, qk_l2norm, stream, workspace)


def _check_fused(x, conv_weight, conv_bias, conv_state, g, beta, state, state_indices, o, num_k_heads,
                 head_k_dim, y, prefix=""):
    """dtypes and shapes of the fused decode's operands; returns (B, HV, dv)."""
    torch = _torch()
    for t, n in ((x, "x"), (conv_weight, "conv_weight"), (conv_bias, "conv_bias"),
                 (conv_state, "conv_state"), (o, "o"), (y, "y")):
        _dtype(t, torch.bfloat16, prefix + n if n in ("x", "o", "y") else n)
    for t, n in ((g, "g"), (beta, "beta"), (state, "state")):
        _dtype(t, torch.float32, prefix + n if n != "state" else n)
    _dims(o, 3, prefix + "o")
    _dims(x, 2, prefix + "x")
    B, HV, dv = o.shape
    HK, dk = int(num_k_heads), int(head_k_dim)
    C = 2 * HK * dk + HV * dv
    _shape(x, (B, C), prefix + "x")
    _shape(y, (B, C), prefix + "y")
    _shape(conv_weight, (C, CONV_WIDTH), "conv_weight")
    _shape(conv_bias, (C,), "conv_bias")
    _dims(conv_state, 3, "conv_state")
    if tuple(conv_state.shape[1:]) != (CONV_WIDTH - 1, C):
        raise ValueError("conv_state must have shape (slots, %d, %d), got %s"
                         % (CONV_WIDTH - 1, C, tuple(conv_state.shape)))
    _shape(g, (B, HV), prefix + "g")
    _shape(beta, (B, HV), prefix + "beta")
    _dims(state, 4, "state")
    if tuple(state.shape[1:]) != (HV, dv, dk):
        raise ValueError("state must have shape (slots, %d, %d, %d), got %s" % (HV, dv, dk, tuple(state.shape)))
    _check_index(state_indices, B, prefix + "state_indices", torch.int32)
    _contig([("conv_weight", conv_weight), ("conv_bias", conv_bias), ("conv_state", conv_state),
             (prefix + "g", g), (prefix + "beta", beta), ("state", state)])
    return B, HV, dv


def gdn_fused_conv_decode(x, conv_weight, conv_bias, conv_state, g, beta, state, state_indices, o,
                          num_k_heads, head_k_dim, y=None, silu=True, scale=1.0, qk_l2norm=True,
                          stream=None):
    """Decode step: conv update of x (q | k | v channels) fused with the gated
    delta rule on its output; see gdn.h.  x: bf16 [B][2 HK dk + HV dv];
    o: bf16 [B][HV][dv]; y optional, shaped like x."""
    B, HV, dv = _check_fused(x, conv_weight, conv_bias, conv_state, g, beta, state, state_indices, o,
                             num_k_heads, head_k_dim, y)
    _on_gpu([("x", x), ("conv_weight", conv_weight), ("conv_bias", conv_bias), ("conv_state", conv_state),
             ("g", g), ("beta", beta), ("state", state), ("state_indices", state_indices), ("o", o), ("y", y)])
    rc = lib.gdn_fused_conv_decode(
        _ptr(x), _rows(x, "x"), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state), conv_state.shape[0],
        _ptr(g), _ptr(beta), _ptr(state), state.shape[0], _ptr(state_indices), _ptr(o), _heads(o, "o"),
        _ptr(y), 0 if y is None else _rows(y, "y"), B, num_k_heads, HV, head_k_dim, dv, int(bool(silu)),
        float(scale), int(bool(qk_l2norm)), _stream(stream))
    _check(rc, "gdn_fused_conv_decode")


def _mixed_operands(q, k, v, g, beta, state_indices, o, query_start_loc, has_initial_state, dec_x, conv_weight,
                    conv_bias, conv_state, dec_g, dec_beta, dec_state_indices, dec_o, state, num_k_heads, dec_y):
    """Checks of gdn_chunk_rule_and_fused_decode's operands; returns
    (T, S, B, HK, dk, HV, dv)."""
    torch = _torch()
    T, HK, dk, HV, dv = _check_rule(q, k, v, g, beta, state, o)
    if HK != int(num_k_heads):
        raise ValueError("q has %d heads, num_k_heads is %d" % (HK, num_k_heads))
    _dims(state_indices, 1, "state_indices")
    S = state_indices.numel()
    _check_index(state_indices, S, "state_indices", torch.int32)
    _check_index(query_start_loc, S + 1, "query_start_loc", torch.int32)
    _check_index(has_initial_state, S, "has_initial_state", torch.uint8)
    B, HVd, dvd = _check_fused(dec_x, conv_weight, conv_bias, conv_state, dec_g, dec_beta, state, dec_state_indices,
                               dec_o, num_k_heads, dk, dec_y, prefix="dec_")
    if (HVd, dvd) != (HV, dv):
        raise ValueError("dec_o has %d heads of %d, v has %d of %d" % (HVd, dvd, HV, dv))
    return T, S, B, HK, dk, HV, dv


def _mixed_args(q, k, v, g, beta, state_indices, o, query_start_loc, has_initial_state, dec_x, conv_weight,
                conv_bias, conv_state, dec_g, dec_beta, dec_state_indices, dec_o, state, num_k_heads, dec_y, silu,
                S, T, B, HV, dk, dv):
    """The ABI arguments of the one-grid mixed call before the workspace,
    and those after it up to (not including) the stream."""
    pre = [_ptr(q), _heads(q, "q"), _ptr(k), _heads(k, "k"), _ptr(v), _heads(v, "v"), _ptr(g), _ptr(beta),
           _ptr(query_start_loc), _ptr(state_indices), _ptr(has_initial_state), _ptr(o), _heads(o, "o"), S, T]
    post = [_ptr(dec_x), _rows(dec_x, "dec_x"), _ptr(conv_weight), _ptr(conv_bias), _ptr(conv_state),
            conv_state.shape[0], _ptr(dec_g), _ptr(dec_beta), _ptr(dec_state_indices), _ptr(dec_o),
            _heads(dec_o, "dec_o"), _ptr(dec_y), 0 if dec_y is None else _rows(dec_y, "dec_y"), B, int(bool(silu)),
            _ptr(state), state.shape[0], num_k_heads, HV, dk, dv]
    return pre, post


def gdn_chunk_rule_and_fused_decode(q, k, v, g, beta, state_indices, o, query_start_loc, has_initial_state,
                                    dec_x, conv_weight, conv_bias, conv_state, dec_g, dec_beta,
                                    dec_state_indices, dec_o, state, num_k_heads, dec_y=None, silu=True,
                                    scale=1.0, qk_l2norm=True, stream=None, workspace=None):
    """One engine step's recurrence on both kinds of rows: the chunkwise rule
    over the prefill tokens (q, k, v, g, beta, o, query_start_loc, ...; as
    gdn_chunk_gated_delta_rule) and the fused conv update + rule on the
    decode rows (dec_*; as gdn_fused_conv_decode), sharing the state pool
    ``state`` on distinct slots; see gdn.h."""
    named = [("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state_indices", state_indices), ("o", o),
             ("query_start_loc", query_start_loc), ("has_initial_state", has_initial_state), ("dec_x", dec_x),
             ("conv_weight", conv_weight), ("conv_bias", conv_bias), ("conv_state", conv_state), ("dec_g", dec_g),
             ("dec_beta", dec_beta), ("dec_state_indices", dec_state_indices), ("dec_o", dec_o), ("state", state),
             ("dec_y", dec_y), ("workspace", workspace)]
    T, S, B, HK, dk, HV, dv = _mixed_operands(*[t for _n, t in named[:18]], num_k_heads, dec_y)
    _on_gpu(named)
    workspace = _workspace(workspace, gdn_chunk_workspace_size(S, T, HK, HV), q.device, stream)
    pre, post = _mixed_args(q, k, v, g, beta, state_indices, o, query_start_loc, has_initial_state, dec_x,
                            conv_weight, conv_bias, conv_state, dec_g, dec_beta, dec_state_indices, dec_o, state,
                            num_k_heads, dec_y, silu, S, T, B, HV, dk, dv)
    rc = lib.gdn_chunk_rule_and_fused_decode(*pre, _ptr(workspace), workspace.numel(), *post,
                                             float(scale), int(bool(qk_l2norm)), _stream(stream))
    _check(rc, "gdn_chunk_rule_and_fused_decode")


def gdn_chunk_rule_and_fused_decode_noalloc(q, k, v, g, beta, state_indices, o, query_start_loc,
                                            has_initial_state, dec_x, conv_weight, conv_bias, conv_state, dec_g,
                                            dec_beta, dec_state_indices, dec_o, state, num_k_heads, dec_y=None,
                                            silu=True, scale=1.0, qk_l2norm=True, stream=None):
    """gdn_chunk_rule_and_fused_decode with the library's static device
    scratch (NOALLOC_SCRATCH_BYTES per GPU) as the chunk workspace: neither
    the library nor this wrapper allocates device memory.  Calls that
    overlap in time on one GPU race on that scratch; see gdn.h."""
    named = [("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state_indices", state_indices), ("o", o),
             ("query_start_loc", query_start_loc), ("has_initial_state", has_initial_state), ("dec_x", dec_x),
             ("conv_weight", conv_weight), ("conv_bias", conv_bias), ("conv_state", conv_state), ("dec_g", dec_g),
             ("dec_beta", dec_beta), ("dec_state_indices", dec_state_indices), ("dec_o", dec_o), ("state", state),
             ("dec_y", dec_y)]
    T, S, B, HK, dk, HV, dv = _mixed_operands(*[t for _n, t in named[:18]], num_k_heads, dec_y)
    _on_gpu(named)
    pre, post = _mixed_args(q, k, v, g, beta, state_indices, o, query_start_loc, has_initial_state, dec_x,
                            conv_weight, conv_bias, conv_state, dec_g, dec_beta, dec_state_indices, dec_o, state,
                            num_k_heads, dec_y, silu, S, T, B, HV, dk, dv)
    rc = lib.gdn_chunk_rule_and_fused_decode_noalloc(*pre, *post, float(scale), int(bool(qk_l2norm)),
                                                     _stream(stream))
    _check(rc, "gdn_chunk_rule_and_fused_decode_noalloc")
