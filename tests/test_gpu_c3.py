"""Every convolution of the YOLOv8n-shaped backbone workload (27 layers, batch
16, MXFP8 activations and weights, E5M2 gradients): each tensor quantized once
and the CBF im2col compared bit for bit with the oracle, and the forward,
backward-data and backward-weight GEMMs compared element by element with the
oracle's direct convolutions on the dequantized operands."""
import pytest

import microscaling_quantized_convolution_mxq_amd as mq
from microscaling_quantized_convolution_mxq_amd.workloads import C3_LAYERS, c3_workload, draw_inputs
from gpu_common import check_im2col, check_quant, compare_gemms

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("layer", range(len(C3_LAYERS)))
def test_c3_layer(layer):
    wl = c3_workload(layer)
    x, w, dy = draw_inputs(wl)
    tag = f"c3 L{layer:02d}"
    check_quant(x, mq.ROLE_ACT, wl.fx, wl.bp, tag + " X")
    check_quant(w, mq.ROLE_WEIGHT, wl.fw, wl.bp, tag + " W")
    check_quant(dy, mq.ROLE_GRAD, wl.fdy, wl.bp, tag + " dY")
    check_im2col(wl.shape, x, wl.fx, wl.bp, tag)
    compare_gemms(wl.shape, x, w, dy, wl.fx, wl.fw, wl.fdy, wl.bp, wl.passes, tag)
