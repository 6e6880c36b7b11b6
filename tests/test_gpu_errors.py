"""Error paths on the GPU: a launch failure injected at any kernel of an
entry point (mqconv_inject_launch_failure, checked from the host after each
launch; no kernel is made to fail) makes that call return MQ_ERR_HIP, and
the library then runs normally: the next calls give exactly the results of
calls made before the failure."""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_mxq_amd as mq
from gpu_common import dev, gpu_quantize, host, say
from microscaling_quantized_convolution_mxq_amd.workloads import ConvShape

pytestmark = pytest.mark.gpu
MQ_ERR_HIP = -7


@pytest.fixture(autouse=True)
def _no_pending_injection():
    yield
    mq.mqconv_inject_launch_failure(0)


def _fails(call):
    with pytest.raises(mq.MqConvError) as e:
        call()
    torch.cuda.synchronize()
    assert e.value.status == MQ_ERR_HIP, str(e.value)


def test_quantize_fails_then_recovers():
    say("errors: quantize, injected failure at its one launch")
    rng = np.random.default_rng(71)
    x = rng.standard_normal((3, 4, 32, 72)).astype(np.float32)
    ref = gpu_quantize(x, mq.ROLE_ACT, 0, 32)
    t = mq.MxTensor.empty(mq.ROLE_ACT, 0, 32, x.shape)
    mq.mqconv_inject_launch_failure(1)
    _fails(lambda: mq.mqconv_quantize(dev(x), t))
    mq.mqconv_quantize(dev(x), t)
    np.testing.assert_array_equal(host(t.codes), host(ref.codes))
    np.testing.assert_array_equal(host(t.scales), host(ref.scales))


@pytest.mark.parametrize("noalloc", [False, True])
def test_backward_weight_fails_at_each_launch_then_recovers(noalloc):
    # 6-bit dY and X: both re-laid, then the split-K GEMM and the fixed-order
    # reduction (four launches)
    s = ConvShape(32, 64, 18, 14, 96)
    say(f"errors: backward_weight noalloc={noalloc} shape={s.as_tuple()}")
    rng = np.random.default_rng(72)
    x = rng.standard_normal((s.h, s.w, s.n, s.cin)).astype(np.float32)
    dy = rng.standard_normal((s.ho, s.wo, s.n, s.cout)).astype(np.float32)
    xq = gpu_quantize(x, mq.ROLE_ACT, 3, 32)
    gq = gpu_quantize(dy, mq.ROLE_GRAD, 3, 32)
    ws = torch.empty(max(1, mq.mqconv_workspace_bytes(s, mq.OP_WGRAD, 3, 3)), dtype=torch.uint8, device="cuda")

    def call(dw):
        if noalloc:
            mq.mqconv_backward_weight_noalloc(s, gq, xq, dw)
        else:
            mq.mqconv_backward_weight(s, gq, xq, dw, ws)

    ref = torch.empty((s.cout, s.kh, s.kw, s.cin), device="cuda")
    call(ref)
    ref_h = host(ref)
    failed = 0
    for n in range(1, 8):
        dw = torch.full_like(ref, float("nan"))
        mq.mqconv_inject_launch_failure(n)
        try:
            call(dw)
        except mq.MqConvError as e:
            assert e.status == MQ_ERR_HIP, str(e)
            failed += 1
            continue
        # fewer launches than n: this call ran whole, and the countdown is
        # left for the next check, which is cancelled
        mq.mqconv_inject_launch_failure(0)
        np.testing.assert_array_equal(host(dw), ref_h)
        break
    # the two re-layings, the GEMM and the reduction each failed once
    assert failed == 4, failed
    dw = torch.full_like(ref, float("nan"))
    call(dw)
    np.testing.assert_array_equal(host(dw), ref_h)
