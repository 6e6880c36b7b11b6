"""The whole path captured in one HIP graph and replayed several times, with
eager work of the program in between: every replay must reproduce the eager
results bit for bit (the kernels are deterministic and the entry points
record no memset nodes)."""
import numpy as np
import pytest
import torch

import microscaling_quantized_convolution_mxq_amd as mq
from microscaling_quantized_convolution_mxq_amd.workloads import WORKLOADS, ConvShape, draw_inputs

from gpu_common import dev, say, workspace

pytestmark = pytest.mark.gpu

CASES = [
    ("c2", ConvShape(8, 64, 20, 20, 64, 3, 3, 1, 1)),
    ("c5", ConvShape(32, 96, 18, 18, 64, 3, 3, 2, 1)),
    ("c4", ConvShape(40, 64, 9, 11, 96, 3, 3, 1, 1)),
]


@pytest.mark.parametrize("name,shape", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_match_eager(name, shape):
    say(f"graph replay {name} {shape.as_tuple()}")
    wl = WORKLOADS[name]
    x, w, dy = draw_inputs(wl, shape)
    s = shape
    X, Wt, DY = dev(x), dev(w), dev(dy)
    xq = mq.MxTensor.empty(mq.ROLE_ACT, wl.fx, 32, x.shape)
    wq = mq.MxTensor.empty(mq.ROLE_WEIGHT, wl.fw, 32, w.shape)
    gq = mq.MxTensor.empty(mq.ROLE_GRAD, wl.fdy, 32, dy.shape)
    cc = torch.empty(mq.mqconv_im2col_codes_bytes(s, wl.fx), dtype=torch.uint8, device="cuda")
    cs = torch.empty(mq.mqconv_im2col_scales_bytes(s, 32), dtype=torch.uint8, device="cuda")
    y = torch.empty((s.ho, s.wo, s.n, s.cout), device="cuda")
    dx = torch.empty(x.shape, device="cuda")
    dw = torch.empty(w.shape, device="cuda")
    ws1 = workspace(mq.mqconv_workspace_bytes(s, 1, wl.fdy, wl.fw))
    ws2 = workspace(mq.mqconv_workspace_bytes(s, 2, wl.fdy, wl.fx))
    ybp = 32 if (s.n % 32 == 0 or 32 % s.n == 0) else 1
    yq = mq.MxTensor.empty(mq.ROLE_ACT, wl.fx, ybp, (s.ho, s.wo, s.n, s.cout))
    dxq = mq.MxTensor.empty(mq.ROLE_GRAD, wl.fdy, ybp, x.shape)
    outs = [xq.codes, xq.scales, wq.codes, wq.scales, gq.codes, gq.scales, cc, cs, y, dx, dw, yq.codes, yq.scales,
            dxq.codes, dxq.scales]

    def path():
        mq.mqconv_quantize_group([(X, xq), (Wt, wq)])
        mq.mqconv_quantize(DY, gq)
        mq.mqconv_cbf_im2col(s, xq, cc, cs)
        mq.mqconv_forward(s, xq, wq, y)
        mq.mqconv_forward_mx(s, xq, wq, yq)
        mq.mqconv_backward_data(s, gq, wq, dx, ws1)
        mq.mqconv_backward_data_mx(s, gq, wq, dxq, ws1)
        mq.mqconv_backward_weight(s, gq, xq, dw, ws2)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        path()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        path()  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            path()
    torch.cuda.synchronize()

    for rep in range(4):
        for t in outs:  # clobber every output, then replay
            t.fill_(0x5A if t.dtype == torch.uint8 else float("nan"))
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        for i, (t, e) in enumerate(zip(outs, eager)):
            assert torch.equal(t.view(torch.uint8) if t.dtype != torch.uint8 else t,
                               e.view(torch.uint8) if e.dtype != torch.uint8 else e), f"replay {rep}: output {i} differs"
        # eager work of the program between replays
        with torch.cuda.stream(stream):
            path()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t.view(torch.uint8) if t.dtype != torch.uint8 else t,
                               e.view(torch.uint8) if e.dtype != torch.uint8 else e)
