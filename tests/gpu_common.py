"""Helpers shared by the GPU parity tests: run the library through its C ABI
and run the oracle on the same host arrays."""
import sys

import numpy as np
import torch

import microscaling_quantized_convolution_mxq_amd as mq
import oracle

# max |gpu - oracle| / max |oracle| for fp32-accumulated block-scaled GEMMs
REL_TOL = 1e-3


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


def rel_err(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    den = np.abs(r).max()
    if den == 0:
        return float(np.abs(g).max())
    return float(np.abs(g - r).max() / den)


def workspace(nbytes):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device="cuda")
