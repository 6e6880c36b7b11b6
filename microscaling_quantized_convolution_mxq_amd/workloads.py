"""Seeded synthetic workloads shaped like the MicroQonv paper's experiments.

This module only draws random inputs and describes shapes. It holds none of
the method's arithmetic, so both the GPU library's callers and the CPU oracle
can take their inputs from it.

Shapes follow the paper's workloads ("MicroQonv: Reshaping Convolution
Tensors for Efficient Microscaling in Training and Inference"):
  - YOLOv8-nano convolutions (§V-A, §VI: YOLOv8n on PascalVOC), a 3x3
    stride-1 layer and the whole backbone at width 0.25;
  - 4-bit quantized latent replay (§VII): activations stored as MXFP4 and
    read back by channel-batch-first im2col;
  - a stride-2 stress layer with FP6 activations (§IV-D "MicroQonv+").
No dataset is read; every tensor is drawn from numpy's PCG64 generator in
fp64 and cast to fp32, directly in the channel-batch-first order
[H][W][N][C] (activations, gradients) or [Cout][Kh][Kw][Cin] (weights).
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Tuple

import numpy as np

E4M3, E5M2, E2M3, E3M2, E2M1 = 0, 1, 2, 3, 4
FORMAT_NAMES = {E4M3: "e4m3", E5M2: "e5m2", E2M3: "e2m3", E3M2: "e3m2", E2M1: "e2m1"}
ROLE_ACT, ROLE_WEIGHT, ROLE_GRAD = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class ConvShape:
    n: int
    cin: int
    h: int
    w: int
    cout: int
    kh: int = 3
    kw: int = 3
    stride: int = 1
    pad: int = 1

    @property
    def ho(self) -> int:
        return (self.h + 2 * self.pad - self.kh) // self.stride + 1

    @property
    def wo(self) -> int:
        return (self.w + 2 * self.pad - self.kw) // self.stride + 1

    def as_tuple(self) -> Tuple[int, ...]:
        """(n, cin, h, w, cout, kh, kw, sh, sw, ph, pw): the library's mq_conv order."""
        return (self.n, self.cin, self.h, self.w, self.cout, self.kh, self.kw,
                self.stride, self.stride, self.pad, self.pad)

    def flops(self) -> int:
        """Multiply-adds x2 of one of the three GEMMs (all three are equal)."""
        return 2 * self.n * self.ho * self.wo * self.cout * self.cin * self.kh * self.kw


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    shape: ConvShape
    seed: int
    x_dist: str            # "normal" | "silu" | "relu"
    dy_dist: Optional[str]  # None (forward only) | "normal_outliers" | "normal" | "student_t3"
    fx: int
    fw: int
    fdy: int
    bp: int
    passes: Tuple[str, ...]


def _c3_backbone() -> List[ConvShape]:
    """Convolutions of a YOLOv8n-shaped backbone (width 0.25, depth 0.33),
    input 640x640x3, batch 16: stride-2 3x3 downsamplers, C2f blocks of 1x1
    and 3x3 convolutions, and the SPPF 1x1 convolutions (pooling is not a
    convolution). The paper notes 40% of YOLOv8n layers are 1x1 (§V-B)."""
    N = 16
    L: List[ConvShape] = []

    def conv(cin, cout, hw, k, s):
        p = k // 2
        L.append(ConvShape(N, cin, hw, hw, cout, k, k, s, p))

    def c2f(c, n_bottleneck, hw):
        conv(c, c, hw, 1, 1)                       # cv1
        for _ in range(n_bottleneck):              # bottlenecks on half the channels
            conv(c // 2, c // 2, hw, 3, 1)
            conv(c // 2, c // 2, hw, 3, 1)
        conv(c // 2 * (2 + n_bottleneck), c, hw, 1, 1)  # cv2 on the concatenation

    conv(3, 16, 640, 3, 2)
    conv(16, 32, 320, 3, 2)
    c2f(32, 1, 160)
    conv(32, 64, 160, 3, 2)
    c2f(64, 2, 80)
    conv(64, 128, 80, 3, 2)
    c2f(128, 2, 40)
    conv(128, 256, 40, 3, 2)
    c2f(256, 1, 20)
    conv(256, 128, 20, 1, 1)   # SPPF cv1
    conv(512, 256, 20, 1, 1)   # SPPF cv2 on the 4-way concatenation
    return L


C3_LAYERS = _c3_backbone()

WORKLOADS = {
    "c1": Workload("c1_conv3x3_n2_c32_16x16", ConvShape(2, 32, 16, 16, 32), 1,
                   "normal", None, E4M3, E4M3, E5M2, 1, ("fwd",)),
    "c2": Workload("c2_yolov8n_conv3x3_n16_c64_80x80", ConvShape(16, 64, 80, 80, 64), 2,
                   "silu", "normal_outliers", E4M3, E4M3, E5M2, 32, ("fwd", "dgrad", "wgrad")),
    "c4": Workload("c4_latent_replay_conv3x3_n128_c256_20x20", ConvShape(128, 256, 20, 20, 256), 4,
                   "relu", "normal", E2M1, E4M3, E5M2, 32, ("fwd", "dgrad", "wgrad")),
    "c5": Workload("c5_stress_conv3x3s2_n32_c128to256_160x160", ConvShape(32, 128, 160, 160, 256, 3, 3, 2, 1), 5,
                   "silu", "student_t3", E3M2, E4M3, E5M2, 32, ("fwd", "dgrad", "wgrad")),
}


def c3_workload(layer: int) -> Workload:
    s = C3_LAYERS[layer]
    return Workload(f"c3_yolov8n_backbone_layer{layer:02d}", s, 300 + layer, "silu",
                    "normal_outliers", E4M3, E4M3, E5M2, 32, ("fwd", "dgrad", "wgrad"))


def _silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def draw_inputs(wl: Workload, shape: Optional[ConvShape] = None, seed: Optional[int] = None):
    """Return (x, w, dy) as fp32 numpy arrays:
    x [H][W][N][Cin], w [Cout][Kh][Kw][Cin], dy [Ho][Wo][N][Cout] (None for
    forward-only workloads). `shape`/`seed` override the workload's own, so a
    reduced problem keeps the workload's value distributions."""
    s = shape or wl.shape
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    z = rng.standard_normal((s.h, s.w, s.n, s.cin))
    if wl.x_dist == "silu":
        z = _silu(z)
    elif wl.x_dist == "relu":
        z = np.maximum(z, 0.0)
    x = z.astype(np.float32)
    sigma = np.sqrt(2.0 / (s.cin * s.kh * s.kw))  # Kaiming-normal, fan-in
    w = (rng.standard_normal((s.cout, s.kh, s.kw, s.cin)) * sigma).astype(np.float32)
    dy = None
    if wl.dy_dist is not None:
        shp = (s.ho, s.wo, s.n, s.cout)
        if wl.dy_dist == "student_t3":
            g = 1e-3 * rng.standard_t(3.0, size=shp)
        else:
            g = 1e-3 * rng.standard_normal(shp)
            if wl.dy_dist == "normal_outliers":
                k = int(round(0.001 * g.size))  # 0.1% of the entries, scaled by 100
                idx = rng.choice(g.size, size=k, replace=False)
                g.reshape(-1)[idx] *= 100.0
        dy = g.astype(np.float32)
    return x, w, dy
