"""Closed-form quantization counts and memory-movement models.

TEST INFRASTRUCTURE (part of the oracle). Source: "MicroQonv: Reshaping
Convolution Tensors for Efficient Microscaling in Training and Inference",
§IV-C Table I (per-element quantization count and backward memory movement
for Dacapo, the Cuyckens et al. extrapolation and MicroQonv), §V Fig. 4 (the
transfers counted: quantized weights loaded, activations saved in the
forward pass and loaded in the backward pass) and the bits-per-element
figures of §IV-D, §VI-A and §VII-B.

Each method is described by what it quantizes and what it stores:
  microqonv  quantizes X, W and G_Y once each (X before CBF im2col) and saves
             the quantized X for the backward pass;
  dacapo     quantizes the im2col-expanded X' along the forward direction and
             again along the backward direction, W and G_Y along both of
             their GEMM directions, and saves the fp32 X (and loads fp32 W);
  cuyckens   square-quantizes the im2col-expanded X' once and saves it; W and
             G_Y once each.
"""
from __future__ import annotations


def _sizes(shape):
    ho = (shape.h + 2 * shape.pad - shape.kh) // shape.stride + 1
    wo = (shape.w + 2 * shape.pad - shape.kw) // shape.stride + 1
    x = shape.n * shape.cin * shape.h * shape.w
    w = shape.cout * shape.cin * shape.kh * shape.kw
    g = shape.n * shape.cout * ho * wo
    xcol = shape.n * ho * wo * shape.cin * shape.kh * shape.kw  # padding positions included
    return x, w, g, xcol


def quantization_counts(method: str, shape) -> dict:
    """Element quantizations per training step, per tensor (A, W, G)."""
    x, w, g, xcol = _sizes(shape)
    if method == "microqonv":
        return {"A": x, "W": w, "G": g}
    if method == "dacapo":
        return {"A": 2 * xcol, "W": 2 * w, "G": 2 * g}
    if method == "cuyckens":
        return {"A": xcol, "W": w, "G": g}
    raise ValueError(method)


def bits_per_element(elem_bits: float, block_elems: int, scale_bits: int = 8) -> float:
    """Storage bits per element of a microscaled tensor: the element plus its
    share of one block scale."""
    return elem_bits + scale_bits / block_elems


def backward_bytes(method: str, shape, elem_bits: float, block_elems: int) -> dict:
    """Bytes stored in the forward pass and brought back for the backward
    pass (Table I 'Backward Mem. Move.'): activations (A) and weights (W)."""
    x, w, g, xcol = _sizes(shape)
    q = bits_per_element(elem_bits, block_elems) / 8.0
    if method == "microqonv":
        return {"A": q * x, "W": q * w}
    if method == "dacapo":
        return {"A": 4.0 * x, "W": 4.0 * w}
    if method == "cuyckens":
        return {"A": q * xcol, "W": q * w}
    raise ValueError(method)
