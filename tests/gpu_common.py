"""Helpers shared by the GPU parity tests: run the library through its C ABI
and run the oracle on the same host arrays."""
import json
import os
import sys

import numpy as np
import torch

import microscaling_quantized_convolution_mxq_amd as mq
import oracle

# max |gpu - oracle| / max |oracle| for fp32-accumulated block-scaled GEMMs
REL_TOL = 1e-3
# per element: |gpu - oracle| <= ELEM_TOL * (sum of the absolute products that
# make up that output). Summing n products in fp32 in any order errs by at most
# about n * 2^-24 of that sum, and far less for blocked sums; the hardware's
# block-scaled accumulation measured about 1e-4 of it.
ELEM_TOL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def gpu_quantize(x, role, fmt, bp):
    """Quantize host array x (role layout) on the GPU; returns the MxTensor."""
    t = mq.MxTensor.empty(role, fmt, bp, x.shape)
    t.codes.fill_(0xAB)  # poison: every byte must be overwritten
    t.scales.fill_(0xAB)
    mq.mqconv_quantize(dev(x.astype(np.float32)), t)
    return t


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def oracle_packed(x, role, fmt, bp):
    codes, scales, _ = oracle.quantize(role, fmt, bp, x)
    return oracle.pack(fmt, codes), scales


def check_quant(x, role, fmt, bp, label):
    say(f"quantize {label} role={role} fmt={fmt} bp={bp} shape={x.shape}")
    t = gpu_quantize(x, role, fmt, bp)
    gc, gs = host(t.codes), host(t.scales)
    oc, os_ = oracle_packed(x, role, fmt, bp)
    np.testing.assert_array_equal(gs, os_.reshape(-1), err_msg=f"scales {label}")
    if not np.array_equal(gc, oc.reshape(-1)):
        C = x.shape[-1]
        gl = oracle.unpack(fmt, gc.reshape(oc.shape), C)
        ol = oracle.unpack(fmt, oc, C)
        bad = np.argwhere(gl != ol)
        i = tuple(bad[0])
        raise AssertionError(f"codes {label}: {len(bad)} mismatches, first at {i}: gpu {gl[i]:#x} "
                             f"oracle {ol[i]:#x} x={x[i]!r}")


def check_im2col(shape, x, fmt, bp, label):
    say(f"im2col {label} shape={shape.as_tuple()} fmt={fmt} bp={bp}")
    t = gpu_quantize(x, mq.ROLE_ACT, fmt, bp)
    nc = mq.mqconv_im2col_codes_bytes(shape, fmt)
    ns = mq.mqconv_im2col_scales_bytes(shape, bp)
    cc = torch.full((nc,), 0xAB, dtype=torch.uint8, device="cuda")
    cs = torch.full((ns,), 0xAB, dtype=torch.uint8, device="cuda")
    mq.mqconv_cbf_im2col(shape, t, cc, cs)
    gc, gs = host(cc), host(cs)
    xc, xs, _ = oracle.quantize(oracle.ROLE_ACT, fmt, bp, x)
    oc, os_ = oracle.cbf_im2col_codes(shape, bp, xc, xs)
    np.testing.assert_array_equal(gs, os_.reshape(-1), err_msg=f"im2col scales {label}")
    rb = oracle.row_bytes(fmt, shape.cin)
    opk = oracle.pack(fmt, oc).reshape(-1, rb)
    gpk = gc.reshape(-1, rb)
    np.testing.assert_array_equal(gpk, opk, err_msg=f"im2col codes {label}")


def rel_err(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    den = np.abs(r).max()
    if den == 0:
        return float(np.abs(g).max())
    return float(np.abs(g - r).max() / den)


def workspace(nbytes):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device="cuda")


def _t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def abs_sums(shape, op, a, b):
    """Sum of |products| behind every output of one GEMM: the same
    convolution applied to the absolute values of the dequantized operands
    (torch float64 on the CPU; it only scales the element-wise tolerance).
    op "fwd": a = X, b = W; "dgrad": a = dY, b = W; "wgrad": a = dY, b = X,
    all in the library's orders ([H][W][N][C], [Cout][Kh][Kw][Cin])."""
    import torch.nn.functional as F
    from torch.nn import grad as G
    nchw = lambda t: _t64(np.abs(t)).permute(2, 3, 0, 1).contiguous()
    oihw = lambda t: _t64(np.abs(t)).permute(0, 3, 1, 2).contiguous()
    s, p = shape.stride, shape.pad
    if op == "fwd":
        out = F.conv2d(nchw(a), oihw(b), stride=s, padding=p)
        return out.permute(2, 3, 0, 1).numpy()
    if op == "dgrad":
        out = G.conv2d_input((shape.n, shape.cin, shape.h, shape.w), oihw(b), nchw(a), stride=s, padding=p)
        return out.permute(2, 3, 0, 1).numpy()
    out = G.conv2d_weight(nchw(b), (shape.cout, shape.cin, shape.kh, shape.kw), nchw(a), stride=s, padding=p)
    return out.permute(0, 2, 3, 1).numpy()


def conv_errors(g, r, sabs):
    """(max-normalised error, element-wise error against the absolute-product
    sums, element-wise relative error over |r| >= 1e-3 max|r|) on the finite
    reference entries."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    d = np.abs(g - r)
    den = np.abs(r).max()
    e_max = float(d.max() / den) if den > 0 else float(np.abs(g).max())
    zero = sabs == 0
    if zero.any() and np.any(g[zero] != 0):
        e_elem = float("inf")  # an output with no nonzero product must be exactly 0
    else:
        e_elem = float((d[~zero] / sabs[~zero]).max()) if (~zero).any() else 0.0
    big = np.abs(r) >= 1e-3 * den
    e_rel = float((d[big] / np.abs(r[big])).max()) if big.any() else 0.0
    return e_max, e_elem, e_rel


def assert_conv_close(name, g, r, sabs, label):
    """R15's max-normalised bound plus the element-wise bound; NaN positions
    (non-finite input blocks) must coincide."""
    g = np.asarray(g)
    nan_r = np.isnan(r)
    assert np.array_equal(np.isnan(g), nan_r), f"{name} {label}: NaN positions differ"
    ok = ~nan_r
    assert np.isfinite(g[ok]).all(), f"{name} {label}: non-finite output"
    e_max, e_elem, e_rel = conv_errors(g[ok], r[ok], sabs[ok])
    say(f"  {name} {label}: max-normalised {e_max:.2e}, vs |products| {e_elem:.2e}, "
        f"element-wise relative (|r| >= 1e-3 max) {e_rel:.2e}")
    log = os.environ.get("MQCONV_ERROR_LOG")
    if log:  # one JSON line per compared output, for the record of achieved errors
        with open(log, "a") as fh:
            fh.write(json.dumps({"out": name, "case": label, "max_normalised": e_max, "vs_abs_products": e_elem,
                                 "elementwise_rel": e_rel, "n": int(ok.sum())}) + "\n")
    assert e_max <= REL_TOL, f"{name} {label}: max-normalised error {e_max:.3e}"
    assert e_elem <= ELEM_TOL, f"{name} {label}: element-wise error {e_elem:.3e} of the |products| sum"
    return e_max, e_elem, e_rel


def run_gpu(shape, x, w, dy, fx, fw, fdy, bp, passes=("fwd", "dgrad", "wgrad"), bpw=None):
    """Quantize on the GPU and run the requested GEMMs; returns host arrays."""
    bpw = bp if bpw is None else bpw
    out = {}
    xq = gpu_quantize(x, mq.ROLE_ACT, fx, bp)
    wq = gpu_quantize(w, mq.ROLE_WEIGHT, fw, bpw)
    if "fwd" in passes:
        y = torch.full((shape.ho, shape.wo, shape.n, shape.cout), float("nan"), device="cuda")
        mq.mqconv_forward(shape, xq, wq, y, workspace(mq.mqconv_workspace_bytes(shape, 0, fx, fw)))
        out["y"] = host(y)
    if dy is not None and ("dgrad" in passes or "wgrad" in passes):
        gq = gpu_quantize(dy, mq.ROLE_GRAD, fdy, bp)
        if "dgrad" in passes:
            dx = torch.full((shape.h, shape.w, shape.n, shape.cin), float("nan"), device="cuda")
            mq.mqconv_backward_data(shape, gq, wq, dx, workspace(mq.mqconv_workspace_bytes(shape, 1, fdy, fw)))
            out["dx"] = host(dx)
        if "wgrad" in passes:
            dw = torch.full((shape.cout, shape.kh, shape.kw, shape.cin), float("nan"), device="cuda")
            mq.mqconv_backward_weight(shape, gq, xq, dw, workspace(mq.mqconv_workspace_bytes(shape, 2, fdy, fx)))
            out["dw"] = host(dw)
    return out


def compare_gemms(shape, x, w, dy, fx, fw, fdy, bp, passes, label, bpw=None):
    """Every output element against the oracle's direct convolution on its own
    quantization of the same host arrays (max-normalised and element-wise)."""
    say(f"gemm {label} shape={shape.as_tuple()} fmts=({fx},{fw},{fdy}) bp={bp} passes={passes}")
    g = run_gpu(shape, x, w, dy, fx, fw, fdy, bp, passes, bpw)
    bpw = bp if bpw is None else bpw
    xc, xs, _ = oracle.quantize(oracle.ROLE_ACT, fx, bp, x)
    wc, ws, _ = oracle.quantize(oracle.ROLE_WEIGHT, fw, bpw, w)
    xh = oracle.dequantize(oracle.ROLE_ACT, fx, bp, xc, xs)
    wh = oracle.dequantize(oracle.ROLE_WEIGHT, fw, bpw, wc, ws)
    del xc
    errs = {}
    if "fwd" in passes:
        errs["y"] = assert_conv_close("y", g["y"], oracle.conv_fwd(shape, xh, wh), abs_sums(shape, "fwd", xh, wh), label)
    if dy is not None and ("dgrad" in passes or "wgrad" in passes):
        gc, gs, _ = oracle.quantize(oracle.ROLE_GRAD, fdy, bp, dy)
        gh = oracle.dequantize(oracle.ROLE_GRAD, fdy, bp, gc, gs)
        del gc
        if "dgrad" in passes:
            errs["dx"] = assert_conv_close("dx", g["dx"], oracle.conv_dgrad(shape, gh, wh),
                                           abs_sums(shape, "dgrad", gh, wh), label)
        if "wgrad" in passes:
            errs["dw"] = assert_conv_close("dw", g["dw"], oracle.conv_wgrad(shape, gh, xh),
                                           abs_sums(shape, "wgrad", gh, xh), label)
    return g, errs
