"""GPU parity of the two-level (NVFP-style) quantization, Eqs. (4)-(6) of the
MicroQonv paper (FP32 tensor scale, E4M3 block scales, 8 x 8 square blocks):
codes, block scales and tensor scale bit for bit against the oracle; and the
per-element error of the format against the E8M0 (MX) format at the same
element bits (the finer scales of the two-level format, §II-D)."""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_mxq_amd as mq
import oracle
from microscaling_quantized_convolution_mxq_amd.workloads import WORKLOADS, draw_inputs
from gpu_common import dev, host, say

pytestmark = pytest.mark.gpu


def _gpu_nvfp(x, role, fmt):
    d = x.shape
    codes = torch.full((mq.mqconv_codes_bytes(role, fmt, *d),), 0xAB, dtype=torch.uint8, device="cuda")
    bs = torch.full((mq.mqconv_nvfp_scales_bytes(role, *d),), 0xAB, dtype=torch.uint8, device="cuda")
    ts = torch.full((1,), float("nan"), device="cuda")
    ws = torch.empty(mq.mqconv_nvfp_workspace_bytes(), dtype=torch.uint8, device="cuda")
    mq.mqconv_nvfp_quantize(dev(x), role, fmt, d, codes, bs, ts, ws)
    return host(codes), host(bs), float(host(ts)[0])


def _check(x, role, fmt, label):
    say(f"nvfp {label} role={role} fmt={fmt} shape={x.shape}")
    gc, gb, gt = _gpu_nvfp(x, role, fmt)
    oc, ob, ot = oracle.nvfp_quantize(role, fmt, x)
    assert np.float32(gt) == np.float32(ot), f"tensor scale {label}: gpu {gt!r} oracle {ot!r}"
    np.testing.assert_array_equal(gb, ob.reshape(-1), err_msg=f"block scales {label}")
    np.testing.assert_array_equal(gc, oracle.pack(fmt, oc).reshape(-1), err_msg=f"codes {label}")
    return oc, ob, ot


SHAPES = [(3, 2, 33, 45), (2, 3, 1, 3), (1, 2, 40, 70), (2, 2, 16, 64), (4, 1, 8, 13)]


@pytest.mark.parametrize("fmt", range(5))
@pytest.mark.parametrize("role", [mq.ROLE_ACT, mq.ROLE_GRAD, mq.ROLE_WEIGHT])
def test_nvfp_small_ragged(fmt, role):
    rng = np.random.default_rng(700 + 10 * fmt + role)
    for shp in SHAPES:
        if role == mq.ROLE_WEIGHT:
            shp = (shp[2], 3, shp[0], shp[3])
        x = (rng.standard_normal(shp) * np.exp(rng.uniform(-6, 6, size=shp[:-1] + (1,)))).astype(np.float32)
        _check(x, role, fmt, f"random{shp}")


@pytest.mark.parametrize("fmt", range(5))
def test_nvfp_special_values(fmt):
    """Zeros and signed zeros, an all-zero tensor, a block whose scale rounds
    to 0, non-finite blocks, ties."""
    rng = np.random.default_rng(71 + fmt)
    x = rng.standard_normal((4, 4, 16, 48)).astype(np.float32)
    x[0, 0] = 0.0
    x[0, 1] = -0.0
    x[0, 2, :8, :8] = 1e-12  # scale below the smallest E4M3 subnormal relative to the tensor maximum
    x[1, 0] = rng.choice([-1.0, 1.0], (16, 48)) * rng.integers(0, 64, (16, 48)) / 8.0
    x[2, 1, 3, 5] = np.inf
    x[2, 2, 9, 40] = np.nan
    x[3, 3, 0, 0] = 1000.0
    _check(x, mq.ROLE_GRAD, fmt, "special")
    _check(np.zeros((2, 2, 8, 32), np.float32), mq.ROLE_ACT, fmt, "zeros")


@pytest.mark.parametrize("key,fmt", [("c4", 4), ("c5", 3), ("c2", 0)])
def test_nvfp_full_activation_and_error_against_mx(key, fmt):
    """The workload's activation in the two-level format, bit for bit; its
    mean squared error against fp32 is below that of the E8M0 format with
    32 x bp square blocks at the same element bits (here measured on the
    oracle's dequantization of the same codes the GPU wrote)."""
    wl = WORKLOADS[key]
    x, _, _ = draw_inputs(wl)
    oc, ob, ot = _check(x, mq.ROLE_ACT, fmt, key)
    nv = oracle.nvfp_dequantize(oracle.ROLE_ACT, fmt, oc, ob, ot)
    mc, ms, _ = oracle.quantize(oracle.ROLE_ACT, fmt, wl.bp, x)
    mx = oracle.dequantize(oracle.ROLE_ACT, fmt, wl.bp, mc, ms)
    xf = x.astype(np.float64)
    e_nv, e_mx = float(np.mean((nv - xf) ** 2)), float(np.mean((mx - xf) ** 2))
    say(f"  {key} fmt={fmt}: MSE two-level {e_nv:.4e}, E8M0 {e_mx:.4e}, ratio {e_nv / e_mx:.3f}")
    assert e_nv < e_mx
