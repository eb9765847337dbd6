"""CPU check of the parity helpers' bf16 spacing rule."""
import numpy as np

import synth
from parity import bf16_half_ulp


def test_half_ulp_is_half_the_bf16_spacing():
    r = np.random.default_rng(0)
    a = (r.standard_normal(20000) * np.exp(r.uniform(-10, 10, 20000))).astype(np.float32)
    b = synth.from_bf16(synth.to_bf16(a)).astype(np.float64)
    up = synth.from_bf16(synth.to_bf16(a).astype(np.uint32).__add__(1).astype(np.uint16)).astype(np.float64)
    spacing = np.abs(up - b)
    # away from binade edges the spacing at |a| equals the spacing at |b|
    inner = np.abs(np.log2(np.abs(b)) - np.round(np.log2(np.abs(b)))) > 0.01
    np.testing.assert_array_equal(bf16_half_ulp(b)[inner] * 2, spacing[inner])
    # rounding to bf16 never moves a value by more than the half spacing
    assert np.all(np.abs(b - a) <= bf16_half_ulp(a))
