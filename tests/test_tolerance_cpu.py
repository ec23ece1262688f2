"""The rounding model behind the few-key lse bound of head-partitioned reuse
(gpu_util.relocated_rope_rounding), checked on the CPU against an emulation
of the relocation kernel's arithmetic: fp32 cos/sin of fp64 angles, one fp32
product, one fused multiply-add, round to bf16 (nearest even)."""
import numpy as np
import pytest

import mla_inputs as mi
from oracle import mla_oracle as orc

from gpu_util import relocated_rope_rounding


def _kernel_emulation(q, delta, base=10000.0):
    # angles -delta * base^(-2k/64) in fp64, cos/sin rounded to fp32
    k = np.arange(32)
    phi = -float(delta) * base ** (-2.0 * k / 64.0)
    c = np.cos(phi).astype(np.float32).astype(np.float64)
    s = np.sin(phi).astype(np.float32).astype(np.float64)
    x0, x1 = q[:, 0::2], q[:, 1::2]
    # fma(a, b, d) = round32(a*b + d): a*b of fp32 values is exact in fp64,
    # and the fp64 sum's own rounding is far below fp32's
    t0 = (x1 * s).astype(np.float32).astype(np.float64)
    t1 = (x1 * c).astype(np.float32).astype(np.float64)
    y0 = (x0 * c - t0).astype(np.float32)
    y1 = (x0 * s + t1).astype(np.float32)
    y = np.empty((q.shape[0], 64), np.float32)
    y[:, 0::2], y[:, 1::2] = y0, y1
    return orc.bf16_to_f64(mi.f32_to_bf16_bits(y))


@pytest.mark.parametrize("delta", [1, 4096, 2 ** 18 + 3])
def test_relocation_rounding_model_covers_the_kernel(delta):
    rng = np.random.default_rng(delta)
    q = orc.bf16_to_f64(mi.f32_to_bf16_bits(rng.standard_normal((4000, 64)).astype(np.float32)))
    got = _kernel_emulation(q, delta)
    exact = orc.relocate_q(q, delta)
    err, err_max = relocated_rope_rounding(q, delta)
    det = err_max == 0
    # determined elements: the emulated kernel lands exactly on the predicted value
    assert np.array_equal(got[det], (exact + err)[det])
    # the others: within the larger of the two possible roundings
    assert np.all(np.abs(got - exact)[~det] <= err_max[~det])
    # almost every element is determined, so the bound is essentially exact
    assert det.mean() > 0.999
