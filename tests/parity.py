"""Helpers for the GPU parity tests: move seeded numpy inputs to the device,
read results back, and apply the parity bars.

Bars (written here once, used by every GPU test):
  * bf16 outputs, GPU vs the unrounded fp64 oracle: ||diff||_2 / ||ref||_2
    < 5e-3 over each output tensor, and per element |diff| <= 2e-2 -- or,
    where |ref| >= 8, half a bf16 ulp at |ref| (times 1 + 2^-6 for the fp32
    arithmetic before the rounding): above 8 the bf16 format cannot hold any
    value within 2e-2 of every real number, so no bf16 result could meet the
    flat bound there;
  * fp32 recurrent state: ||dS||_F / ||S_ref||_F <= 1e-4 for every
    (slot, head) a call touched;
  * conv_state, chunk descriptors and anything a call must not touch:
    bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3
STATE_REL_F = 1e-4
SENTINEL = 0x7FE5          # a quiet-NaN bf16 pattern (quiet bit 0x0040 set): "never written"


def bf16_half_ulp(ref):
    """Half the spacing of bf16 numbers at |ref| (8 significant bits)."""
    a = np.maximum(np.abs(ref), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 8)


def dev(a, device="cuda"):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a)
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to(device)


def bits(t):
    """bf16 tensor -> numpy uint16 bit patterns."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def sentinel_like(shape, device="cuda"):
    return torch.full(shape, SENTINEL, dtype=torch.int16, device=device).view(torch.bfloat16)


def check_bf16(got_t, ref, name, written=None):
    """got_t: bf16 tensor; ref: float64 array with NaN where the oracle wrote
    nothing.  Entries the oracle did not write must still hold SENTINEL when
    ``written`` is None and the tensor was sentinel-filled."""
    g_bits = bits(got_t)
    mask = ~np.isnan(ref) if written is None else written
    if written is None and (~mask).any():
        assert np.all(g_bits[~mask] == SENTINEL), "%s: wrote outside its tokens" % name
    got = f64(got_t)[mask]
    r = ref[mask]
    if r.size == 0:
        return 0.0, 0.0
    assert np.isfinite(got).all(), "%s: non-finite output" % name
    diff = np.abs(got - r)
    bound = np.maximum(BF16_MAX_ABS, bf16_half_ulp(r) * (1.0 + 2.0 ** -6))
    worst = int(np.argmax(diff / bound))
    err = float(diff.max())
    rel = float(np.linalg.norm(got - r) / max(np.linalg.norm(r), 1e-30))
    assert diff[worst] <= bound[worst], "%s: |diff| %.4g at ref %.4g exceeds %.4g" % (
        name, diff[worst], r[worst], bound[worst])
    assert rel < BF16_REL_L2, "%s: rel L2 %.3g" % (name, rel)
    return err, rel


def check_state(got_t, ref, before, slots, name="state", tol=STATE_REL_F):
    """Touched slots within the Frobenius bar per (slot, head); every other
    slot bit-identical to ``before``."""
    got = got_t.cpu().numpy()
    slots = sorted(set(int(s) for s in np.asarray(slots).ravel() if s >= 0))
    worst = 0.0
    for s in slots:
        for h in range(got.shape[1]):
            d = np.linalg.norm(got[s, h].astype(np.float64) - ref[s, h])
            n = np.linalg.norm(ref[s, h])
            rel = d / n if n > 0 else d
            worst = max(worst, rel)
            assert rel <= tol, "%s: slot %d head %d rel %.3g" % (name, s, h, rel)
    others = [s for s in range(got.shape[0]) if s not in slots]
    if others:
        assert np.array_equal(got[others].view(np.uint32), np.asarray(before)[others].view(np.uint32)), \
            "%s: untouched slots changed" % name
    return worst
