"""Benchmark of the MicroQonv training hot path on one MI355X.

One step = one pass of every step of the path over one batch of synthetic
input: quantize X and W (one grouped call, as before a layer's forward
pass; one launch for up to two element formats) and G_Y once (MX, E8M0
scales, round-to-nearest), channel-batch-first
im2col of the quantized activation, then the forward, backward-data and
backward-weight block-scaled GEMMs. Inputs are resident in HBM before the
timed region; R copies of every buffer are rotated so the live set exceeds
the 256 MB Infinity Cache.

Each step is one HIP graph (captured once per buffer set) so the timed
region measures the GPU, not Python launch overhead. `value` is fwd+bwd
TFLOP/s of the whole step (algorithmic FLOPs of the three GEMMs / step
time). Every entry point is also timed on its own (a graph of repeated
calls on rotating buffer sets, HIP events on the stream the kernels run
on); `roofline` covers the entry point that takes the most time per step,
with its algorithmic bytes or FLOPs per call. The forward whose epilogue
writes Y as MX codes (`mqconv_forward_mx`), the backward-data whose
epilogue writes dX as MX codes (`mqconv_backward_data_mx`), the gradient
quantized with stochastic rounding (`mqconv_quantize_sr`) and the
backward-weight without allocation (`mqconv_backward_weight_noalloc`) are
timed the same way and listed with `in_step: false`. `roofline.traffic` is
taken from the committed counter summary of that entry point when its
source hash matches the kernels. `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload. The default workload is the stride-2
MXFP6 layer (N=32, 128 -> 256 channels, 160x160), the largest one.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# dense MFMA peaks of MI355X (TFLOP/s); mixed 6/4-bit x 8-bit products run at the 8-bit rate
MFMA_PEAK_TFLOPS = {"fp8": 5000.0, "fp6fp4": 10100.0}
CSRC = os.path.join(ROOT, "microscaling_quantized_convolution_mxq_amd", "csrc")
CALLS = ["quantize_xw", "quantize_dy", "cbf_im2col", "forward", "backward_data", "backward_weight"]
# timed on their own too, but not part of the step: the forward whose epilogue
# writes Y as MX codes and scales (the next layer's activation) instead of fp32,
# the backward-data that writes dX the same way (the previous layer's gradient),
# the gradient quantized with stochastic rounding, and the backward-weight
# variant that takes its scratch from the library's fixed array
EXTRA = ["forward_mx", "backward_data_mx", "quantize_dy_sr", "backward_weight_noalloc"]
# kernels each entry point launches (see the launchers in csrc/)
CALL_KERNELS = {
    # X and W share one launch (the grouped quantizer takes up to two formats)
    "quantize_xw": ["mxq_quantize_group_kernel (X and W in one launch, of one or two element formats)"],
    "quantize_dy": ["mxq_quantize_kernel"], "cbf_im2col": ["cbf_im2col_kernel"],
    "quantize_dy_sr": ["mxq_quantize_kernel (stochastic rounding)"],
    "backward_weight_noalloc": ["as backward_weight, scratch in the library's fixed array"],
    "forward": ["mx_gemm_kernel<FwdProb>"], "forward_mx": ["mx_gemm_kernel<MxOutProb<FwdProb>>"],
    "backward_data_mx": ["mx_gemm_kernel<MxOutProb<DgradNatProb>> (8-bit W; else transpose_codes_kernel + "
                         "mx_gemm_kernel<MxOutProb<DgradProb>>)"],
    # 8-bit codes are read in place; other formats are first re-laid by transpose_codes_kernel
    "backward_data": ["mx_gemm_kernel<DgradNatProb> (8-bit W; else transpose_codes_kernel + mx_gemm_kernel<DgradProb>)"],
    "backward_weight": ["mx_gemm_kernel<WgradNatProb> (8-bit dY and X) or mx_gemm_kernel<WgradNatSubProb> (8-bit "
                        "dY, 6/4-bit X), both read in place when Cin % 16 == 0; else transpose_codes_kernel (X) + "
                        "mx_gemm_kernel<WgradMixProb> (8-bit dY), or 2 x transpose_codes_kernel + "
                        "mx_gemm_kernel<WgradProb>",
                        "splitk_reduce_kernel (when split)"],
}


def source_sha() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c5")
    ap.add_argument("--rotate-mb", type=float, default=640.0, help="minimum live set across rotated buffers")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-naive", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch the step call by call instead of as a graph")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the per-GPU kernels are what it measures). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import microscaling_quantized_convolution_mxq_amd as mq
    from microscaling_quantized_convolution_mxq_amd.workloads import WORKLOADS, FORMAT_NAMES, draw_inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mq.lib()  # fails loudly if the HIP library is missing
    wl = WORKLOADS[args.workload]
    s = wl.shape
    x, w, dy = draw_inputs(wl)
    bp = wl.bp

    # ---- per-set buffers ---------------------------------------------------
    def make_set():
        d = {}
        d["x"] = torch.from_numpy(x).cuda()
        d["w"] = torch.from_numpy(w).cuda()
        d["dy"] = torch.from_numpy(dy).cuda()
        d["xq"] = mq.MxTensor.empty(mq.ROLE_ACT, wl.fx, bp, x.shape)
        d["wq"] = mq.MxTensor.empty(mq.ROLE_WEIGHT, wl.fw, bp, w.shape)
        d["gq"] = mq.MxTensor.empty(mq.ROLE_GRAD, wl.fdy, bp, dy.shape)
        d["cc"] = torch.empty(mq.mqconv_im2col_codes_bytes(s, wl.fx), dtype=torch.uint8, device="cuda")
        d["cs"] = torch.empty(mq.mqconv_im2col_scales_bytes(s, bp), dtype=torch.uint8, device="cuda")
        d["y"] = torch.empty((s.ho, s.wo, s.n, s.cout), device="cuda")
        d["yq"] = mq.MxTensor.empty(mq.ROLE_ACT, wl.fx, bp, (s.ho, s.wo, s.n, s.cout))
        d["dx"] = torch.empty(x.shape, device="cuda")
        d["dxq"] = mq.MxTensor.empty(mq.ROLE_GRAD, wl.fdy, bp, x.shape)
        d["dw"] = torch.empty(w.shape, device="cuda")
        d["ws1"] = torch.empty(max(1, mq.mqconv_workspace_bytes(s, 1, wl.fdy, wl.fw)), dtype=torch.uint8, device="cuda")
        d["ws2"] = torch.empty(max(1, mq.mqconv_workspace_bytes(s, 2, wl.fdy, wl.fx)), dtype=torch.uint8, device="cuda")
        return d

    first = make_set()
    set_bytes = sum((t.codes.numel() + t.scales.numel()) if isinstance(t, mq.MxTensor) else t.numel() * t.element_size()
                    for t in first.values())
    R = int(min(8, max(2, np.ceil(args.rotate_mb * 1e6 / set_bytes))))
    sets = [first] + [make_set() for _ in range(R - 1)]

    def run(d, name):
        if name == "quantize_xw":
            mq.mqconv_quantize_group([(d["x"], d["xq"]), (d["w"], d["wq"])])
        elif name == "quantize_dy":
            mq.mqconv_quantize(d["dy"], d["gq"])
        elif name == "quantize_dy_sr":
            mq.mqconv_quantize_sr(d["dy"], d["gq"], 0x5EED)
        elif name == "cbf_im2col":
            mq.mqconv_cbf_im2col(s, d["xq"], d["cc"], d["cs"])
        elif name == "forward":
            mq.mqconv_forward(s, d["xq"], d["wq"], d["y"])
        elif name == "forward_mx":
            mq.mqconv_forward_mx(s, d["xq"], d["wq"], d["yq"])
        elif name == "backward_data":
            mq.mqconv_backward_data(s, d["gq"], d["wq"], d["dx"], d["ws1"])
        elif name == "backward_data_mx":
            mq.mqconv_backward_data_mx(s, d["gq"], d["wq"], d["dxq"], d["ws1"])
        elif name == "backward_weight":
            mq.mqconv_backward_weight(s, d["gq"], d["xq"], d["dw"], d["ws2"])
        elif name == "backward_weight_noalloc":
            mq.mqconv_backward_weight_noalloc(s, d["gq"], d["xq"], d["dw"])

    def step(d):
        for c in CALLS:
            run(d, c)

    stream = torch.cuda.Stream()  # kernels, graphs and events all live on this stream
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for d in sets:  # eager warm-up of every set
            step(d)
    torch.cuda.synchronize()

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                fn()
        torch.cuda.synchronize()
        return g

    # One graph runs G = 4R steps, cycling over the buffer sets (a graph
    # launch costs ~8 us, so it is amortized over G steps); single-step graphs
    # make up a count that is not a multiple of G.
    G = 4 * R
    if args.eager:
        step_graphs = multi_graph = None
    else:
        step_graphs = [capture(lambda d=d: step(d)) for d in sets]
        multi_graph = capture(lambda: [step(sets[i % R]) for i in range(G)])

    def launch_steps(n):
        """Exactly n steps, cycling over the buffer sets."""
        if multi_graph is None:
            for i in range(n):
                step(sets[i % R])
            return
        for _ in range(n // G):
            multi_graph.replay()
        for i in range(n % G):
            step_graphs[i % R].replay()

    # ---- warm-up, then exactly K timed steps -----------------------------------
    with torch.cuda.stream(stream):
        launch_steps(args.warmup)
    torch.cuda.synchronize()
    K = args.steps
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    with torch.cuda.stream(stream):
        t_start.record(stream)
        launch_steps(K)
        t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / K

    # ---- every entry point on its own --------------------------------------
    # A graph of 2 x Rc calls rotating over Rc copies of just the buffers the
    # call touches, with Rc chosen so that those copies exceed the 256 MB
    # Infinity Cache as the step's sets do (no call reads cache-resident inputs).
    NEED = {"quantize_xw": ("x", "xq", "w", "wq"), "quantize_dy": ("dy", "gq"), "quantize_dy_sr": ("dy", "gq"),
            "backward_weight_noalloc": ("gq", "xq", "dw"),
            "cbf_im2col": ("xq", "cc", "cs"), "forward": ("xq", "wq", "y"), "forward_mx": ("xq", "wq", "yq"),
            "backward_data": ("gq", "wq", "dx", "ws1"), "backward_data_mx": ("gq", "wq", "dxq", "ws1"),
            "backward_weight": ("gq", "xq", "dw", "ws2")}

    def nbytes(v):
        return (v.codes.numel() + v.scales.numel()) if isinstance(v, mq.MxTensor) else v.numel() * v.element_size()

    def clone(v):
        if isinstance(v, mq.MxTensor):
            return mq.MxTensor(v.codes.clone(), v.scales.clone(), v.fmt, v.bp, v.role, v.dims)
        return v.clone()

    per_call = {}
    for c in CALLS + EXTRA:
        call_bytes = sum(nbytes(sets[0][k]) for k in NEED[c])
        Rc = int(min(64, max(2, np.ceil(args.rotate_mb * 1e6 / call_bytes))))
        csets = [{k: clone(sets[0][k]) for k in NEED[c]} for _ in range(Rc)]
        g = capture(lambda c=c: [run(csets[i % Rc], c) for i in range(2 * Rc)])
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nrep = 10
        with torch.cuda.stream(stream):
            a.record(stream)
            for _ in range(nrep):
                g.replay()
            b.record(stream)
        torch.cuda.synchronize()
        per_call[c] = a.elapsed_time(b) / (nrep * 2 * Rc)
        del g, csets

    # ---- algorithmic work -----------------------------------------------------
    flop = s.flops()
    nx, nw, ng = x.size, w.size, dy.size
    xq_b = mq.mqconv_codes_bytes(mq.ROLE_ACT, wl.fx, *x.shape) + mq.mqconv_scales_bytes(mq.ROLE_ACT, bp, *x.shape)
    wq_b = mq.mqconv_codes_bytes(mq.ROLE_WEIGHT, wl.fw, *w.shape) + mq.mqconv_scales_bytes(mq.ROLE_WEIGHT, bp, *w.shape)
    gq_b = mq.mqconv_codes_bytes(mq.ROLE_GRAD, wl.fdy, *dy.shape) + mq.mqconv_scales_bytes(mq.ROLE_GRAD, bp, *dy.shape)
    col_b = mq.mqconv_im2col_codes_bytes(s, wl.fx) + mq.mqconv_im2col_scales_bytes(s, bp)
    yq_dims = (s.ho, s.wo, s.n, s.cout)
    yq_b = mq.mqconv_codes_bytes(mq.ROLE_ACT, wl.fx, *yq_dims) + mq.mqconv_scales_bytes(mq.ROLE_ACT, bp, *yq_dims)
    dxq_b = mq.mqconv_codes_bytes(mq.ROLE_GRAD, wl.fdy, *x.shape) + mq.mqconv_scales_bytes(mq.ROLE_GRAD, bp, *x.shape)
    # bytes each call must move at least once (inputs read, outputs written)
    alg_bytes = {
        "quantize_xw": 4 * nx + xq_b + 4 * nw + wq_b, "quantize_dy": 4 * ng + gq_b, "quantize_dy_sr": 4 * ng + gq_b,
        "backward_weight_noalloc": gq_b + xq_b + 4 * nw,
        "cbf_im2col": xq_b + col_b,
        "forward": xq_b + wq_b + 4 * ng, "backward_data": gq_b + wq_b + 4 * nx, "backward_weight": gq_b + xq_b + 4 * nw,
        "forward_mx": xq_b + wq_b + yq_b, "backward_data_mx": gq_b + wq_b + dxq_b,
    }
    alg_flop = {"forward": flop, "backward_data": flop, "backward_weight": flop, "forward_mx": flop,
                "backward_data_mx": flop, "backward_weight_noalloc": flop}
    step_gemms = ("forward", "backward_data", "backward_weight")

    def mfma_peak(fa, fb):
        return MFMA_PEAK_TFLOPS["fp6fp4"] if (fa >= 2 and fb >= 2) else MFMA_PEAK_TFLOPS["fp8"]

    call_peak = {"forward": mfma_peak(wl.fx, wl.fw), "forward_mx": mfma_peak(wl.fx, wl.fw),
                 "backward_data": mfma_peak(wl.fdy, wl.fw), "backward_data_mx": mfma_peak(wl.fdy, wl.fw),
                 "backward_weight": mfma_peak(wl.fdy, wl.fx), "backward_weight_noalloc": mfma_peak(wl.fdy, wl.fx)}
    kernels = {}
    for c in CALLS + EXTRA:
        t = per_call[c] * 1e-3
        k = {"ms": round(per_call[c], 5), "GB/s": round(alg_bytes[c] / t / 1e9, 1),
             "hbm_frac": round(alg_bytes[c] / t / 1e9 / HBM_PEAK_GBS, 4), "launches": CALL_KERNELS[c]}
        if c in alg_flop:
            peak = call_peak[c]
            ai = alg_flop[c] / alg_bytes[c]
            attainable = min(peak, ai * HBM_PEAK_GBS / 1e3)
            k.update({"TFLOP/s": round(alg_flop[c] / t / 1e12, 2), "mfma_frac": round(alg_flop[c] / t / 1e12 / peak, 4),
                      "attainable_TFLOP/s": round(attainable, 1),
                      "attainable_frac": round(alg_flop[c] / t / 1e12 / attainable, 4)})
        k["in_step"] = c in CALLS
        kernels[c] = k

    dominant = max(CALLS, key=lambda c: per_call[c])
    t_dom = per_call[dominant] * 1e-3
    if dominant in alg_flop and alg_flop[dominant] / alg_bytes[dominant] > call_peak[dominant] * 1e3 / HBM_PEAK_GBS:
        roof = {"bound": "mfma", "achieved": round(alg_flop[dominant] / t_dom / 1e12, 2),
                "peak": call_peak[dominant], "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(alg_bytes[dominant] / t_dom / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = dominant
    roof["launches"] = CALL_KERNELS[dominant]
    roof["ms_per_call"] = round(per_call[dominant], 5)
    tf = os.path.join(ROOT, "profiles", f"traffic_{wl.name}_{dominant}.json")
    if os.path.exists(tf):
        rec = json.load(open(tf))
        if rec.get("source_sha") == source_sha():
            roof["traffic"] = rec.get("traffic_bytes")

    q_im_bytes = sum(alg_bytes[c] for c in ("quantize_xw", "quantize_dy", "cbf_im2col"))
    q_im_ms = sum(per_call[c] for c in ("quantize_xw", "quantize_dy", "cbf_im2col"))
    gemm_ms = sum(per_call[c] for c in step_gemms)

    # ---- naive comparison path (not part of the step) ------------------------
    naive = None
    if not args.no_naive:
        d = sets[0]
        wsn = [torch.empty(max(1, mq.mqconv_naive_workspace_bytes(s, op, a, b)), dtype=torch.uint8, device="cuda")
               for op, a, b in ((0, wl.fx, wl.fw), (1, wl.fdy, wl.fw), (2, wl.fdy, wl.fx))]

        def naive_step():
            mq.mqconv_naive_forward(s, d["x"], d["w"], wl.fx, wl.fw, d["y"], wsn[0])
            mq.mqconv_naive_backward_data(s, d["dy"], d["w"], wl.fdy, wl.fw, d["dx"], wsn[1])
            mq.mqconv_naive_backward_weight(s, d["dy"], d["x"], wl.fdy, wl.fx, d["dw"], wsn[2])

        with torch.cuda.stream(stream):
            for _ in range(3):
                naive_step()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            nrep = 10
            for _ in range(nrep):
                naive_step()
            b.record(stream)
        torch.cuda.synchronize()
        naive = {"ms_per_step": round(a.elapsed_time(b) / nrep, 4), "launch": "eager"}
        del wsn

    # ---- CPU baseline: the oracle on a bounded sample of the same workload ----
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        t0 = time.perf_counter()
        ref = oracle.microqonv_step(s, x, w, dy, wl.fx, wl.fw, wl.fdy, bp)
        oracle.cbf_im2col_codes(s, bp, ref["xcodes"], ref["xscales"])
        tc = time.perf_counter() - t0
        cpu = {"value": round(3 * flop / tc / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.threads(),
               "kind": "oracle", "ms_per_step": round(tc * 1e3, 1),
               "sample": f"one full {wl.name} step (quantize X, W, dY; CBF im2col of the codes; fp64 direct "
                         "fwd, dgrad and wgrad on the dequantized operands)"}

    value = 3 * flop / (ms_step * 1e-3) / 1e12
    out = {
        "metric": "MX conv fwd+bwd TFLOP/s and quantize+im2col HBM GB/s (% of roofline), 1 GPU",
        "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"mx{FORMAT_NAMES[wl.fx]}x{FORMAT_NAMES[wl.fw]}/{FORMAT_NAMES[wl.fdy]} fp32-accumulate",
        "data": "synthetic",
        "config": {"workload": wl.name, "n": s.n, "cin": s.cin, "cout": s.cout, "h": s.h, "w": s.w,
                   "kernel": f"{s.kh}x{s.kw}", "stride": s.stride, "pad": s.pad, "block": f"32 ch x {bp} batch",
                   "rotated_sets": R, "launch": "eager" if args.eager else "hip_graph",
                   "steps_per_graph": 1 if args.eager else G},
        "roofline": roof,
        "cpu_baseline": cpu,
        "quantize_im2col_GB/s": round(q_im_bytes / (q_im_ms * 1e-3) / 1e9, 1),
        "quantize_im2col_hbm_frac": round(q_im_bytes / (q_im_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "gemm_TFLOP/s": round(3 * flop / (gemm_ms * 1e-3) / 1e12, 2),
        "kernels": kernels,
        "naive_path": naive,
        "wall_s": round(wall, 3),
        "source_sha": source_sha(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
