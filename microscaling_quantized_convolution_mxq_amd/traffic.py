"""HBM traffic of the quantize-once path and of the naive path, from rocprofv3
counters.

Modes:
  step       run one training step of a workload (every layer for the YOLOv8n
             backbone) through one path, so that rocprofv3 --pmc can count it
  call       quantize the inputs, then run one entry point once (its own
             kernels are the dispatches that are not quantize kernels)
  copy       run a plain device-to-device copy of known size (calibration)
  summarize  read the counter CSVs of the step runs and write a summary
  summarize-call
             read the counter CSVs of a call run and write the HBM bytes of
             one call of that entry point (profiles/traffic_<workload>_<call>.json)
  kernels    read the kernel statistics of a rocprofv3 --kernel-trace --stats
             run of bench.py and its JSON line, and write both side by side
             (profiles/kernels_<workload>.txt)
  mfma       read the counter CSV of a step run with the matrix-core counters
             and write, per GEMM kernel, the fraction of SIMD cycles the MFMA
             unit was busy and the matrix operations it executed
             (profiles/mfma_<workload>.txt)

Counter passes (one counter group per run, as rocprofv3 requires), e.g. for
the 3x3 YOLOv8n-style layer:
  rocprofv3 --pmc FETCH_SIZE -d D -o mq_fetch -- python -m microscaling_quantized_convolution_mxq_amd.traffic step --workload c2 --path microqonv
  rocprofv3 --pmc WRITE_SIZE -d D -o mq_write -- ... --path microqonv
  (the same with --path naive -> naive_fetch / naive_write, and copy -> copy_fetch / copy_write)
  python -m microscaling_quantized_convolution_mxq_amd.traffic summarize --dir D --workload c2

FETCH_SIZE and WRITE_SIZE are KiB per dispatch. Each is divided by what the
same counter reads per byte of the copy, so the result is in bytes of the
copy's own accounting.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "microscaling_quantized_convolution_mxq_amd", "csrc")
COPY_MB = 512


def _workloads(name):
    from microscaling_quantized_convolution_mxq_amd.workloads import WORKLOADS, C3_LAYERS, c3_workload
    if name == "c3":
        return [c3_workload(i) for i in range(len(C3_LAYERS))]
    return [WORKLOADS[name]]


def run_step(workload: str, path: str) -> None:
    import torch
    import microscaling_quantized_convolution_mxq_amd as mq
    from microscaling_quantized_convolution_mxq_amd.workloads import draw_inputs

    for wl in _workloads(workload):
        s = wl.shape
        x, w, dy = draw_inputs(wl)
        X, Wt, DY = (torch.from_numpy(a).cuda() for a in (x, w, dy))
        y = torch.empty((s.ho, s.wo, s.n, s.cout), device="cuda")
        dx = torch.empty(x.shape, device="cuda")
        dw = torch.empty(w.shape, device="cuda")
        if path == "microqonv":
            xq = mq.MxTensor.empty(mq.ROLE_ACT, wl.fx, wl.bp, x.shape)
            wq = mq.MxTensor.empty(mq.ROLE_WEIGHT, wl.fw, wl.bp, w.shape)
            gq = mq.MxTensor.empty(mq.ROLE_GRAD, wl.fdy, wl.bp, dy.shape)
            ws1 = torch.empty(max(1, mq.mqconv_workspace_bytes(s, 1, wl.fdy, wl.fw)), dtype=torch.uint8, device="cuda")
            ws2 = torch.empty(max(1, mq.mqconv_workspace_bytes(s, 2, wl.fdy, wl.fx)), dtype=torch.uint8, device="cuda")
            torch.cuda.synchronize()
            mq.mqconv_quantize_group([(X, xq), (Wt, wq)])
            mq.mqconv_quantize(DY, gq)
            mq.mqconv_forward(s, xq, wq, y)
            mq.mqconv_backward_data(s, gq, wq, dx, ws1)
            mq.mqconv_backward_weight(s, gq, xq, dw, ws2)
        else:
            ws = [torch.empty(max(1, mq.mqconv_naive_workspace_bytes(s, op, a, b)), dtype=torch.uint8, device="cuda")
                  for op, a, b in ((0, wl.fx, wl.fw), (1, wl.fdy, wl.fw), (2, wl.fdy, wl.fx))]
            torch.cuda.synchronize()
            mq.mqconv_naive_forward(s, X, Wt, wl.fx, wl.fw, y, ws[0])
            mq.mqconv_naive_backward_data(s, DY, Wt, wl.fdy, wl.fw, dx, ws[1])
            mq.mqconv_naive_backward_weight(s, DY, X, wl.fdy, wl.fx, dw, ws[2])
        torch.cuda.synchronize()
        print(f"step {path} {wl.name}", flush=True)


CALL_NAMES = ("cbf_im2col", "forward", "backward_data", "backward_weight")


def run_call(workload: str, call: str) -> None:
    import torch
    import microscaling_quantized_convolution_mxq_amd as mq
    from microscaling_quantized_convolution_mxq_amd.workloads import draw_inputs

    wl = WORKLOADS_ONE(workload)
    s = wl.shape
    x, w, dy = draw_inputs(wl)
    X, Wt, DY = (torch.from_numpy(a).cuda() for a in (x, w, dy))
    xq = mq.MxTensor.empty(mq.ROLE_ACT, wl.fx, wl.bp, x.shape)
    wq = mq.MxTensor.empty(mq.ROLE_WEIGHT, wl.fw, wl.bp, w.shape)
    gq = mq.MxTensor.empty(mq.ROLE_GRAD, wl.fdy, wl.bp, dy.shape)
    mq.mqconv_quantize(X, xq)
    mq.mqconv_quantize(Wt, wq)
    mq.mqconv_quantize(DY, gq)
    torch.cuda.synchronize()
    if call == "cbf_im2col":
        cc = torch.empty(mq.mqconv_im2col_codes_bytes(s, wl.fx), dtype=torch.uint8, device="cuda")
        cs = torch.empty(mq.mqconv_im2col_scales_bytes(s, wl.bp), dtype=torch.uint8, device="cuda")
        mq.mqconv_cbf_im2col(s, xq, cc, cs)
    elif call == "forward":
        mq.mqconv_forward(s, xq, wq, torch.empty((s.ho, s.wo, s.n, s.cout), device="cuda"))
    elif call == "backward_data":
        ws = torch.empty(max(1, mq.mqconv_workspace_bytes(s, 1, wl.fdy, wl.fw)), dtype=torch.uint8, device="cuda")
        mq.mqconv_backward_data(s, gq, wq, torch.empty(x.shape, device="cuda"), ws)
    else:
        ws = torch.empty(max(1, mq.mqconv_workspace_bytes(s, 2, wl.fdy, wl.fx)), dtype=torch.uint8, device="cuda")
        mq.mqconv_backward_weight(s, gq, xq, torch.empty(w.shape, device="cuda"), ws)
    torch.cuda.synchronize()
    print(f"call {call} {wl.name}", flush=True)


def WORKLOADS_ONE(name):
    from microscaling_quantized_convolution_mxq_amd.workloads import WORKLOADS
    return WORKLOADS[name]


def run_copy() -> None:
    import torch
    n = COPY_MB * (1 << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(f"copy {COPY_MB} MiB", flush=True)


def _read(d: str, stem: str, counter: str):
    """Per-dispatch (kernel name, value in bytes) of one counter run."""
    files = glob.glob(os.path.join(d, "**", f"{stem}_counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no {stem}_counter_collection.csv under {d}")
    out = []
    for r in csv.DictReader(open(files[0])):
        if r["Counter_Name"] != counter:
            continue
        out.append((r["Kernel_Name"], float(r["Counter_Value"]) * 1024.0))
    return out


def _source_sha() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def _run_bytes(fmt: int) -> int:
    return 32 if fmt <= 1 else (24 if fmt <= 3 else 16)


def model_bytes(wl) -> dict:
    """Full-kernel byte model of one training step of one layer: every kernel
    reads each of its inputs once and writes each output once (fp32: 4 B per
    element; MX: packed codes of whole 32-channel runs plus one scale byte per
    block), no re-reads, no split-K partial sums, no caches.
      quantize-once: quantize X, W, dY (fp32 in, codes out); forward (X_q,
        W_q in, fp32 Y out); backward-data (dY_q, W_q in, fp32 dX out);
        backward-weight (dY_q, X_q in, fp32 dW out).
      naive: per GEMM, its fp32 operands are laid out along that GEMM's
        contraction (classic im2col of X, flattening or transposing W and
        dY: fp32 in, fp32 out), then quantized in line blocks along it;
        the GEMM reads both and writes fp32 (backward-data: G_X', then
        col2im folds it into dX)."""
    s = wl.shape
    ho, wo = s.ho, s.wo
    X, Wn, G = s.h * s.w * s.n * s.cin, s.cout * s.kh * s.kw * s.cin, ho * wo * s.n * s.cout
    M, K = ho * wo * s.n, s.cin * s.kh * s.kw
    cdiv = lambda a, b: -(-a // b)

    def mx(rows, chans, partner_rows, fmt, bp):  # CBF tensor: rows x chans codes, blocks over partner_rows
        nb = cdiv(chans, 32)
        return rows * nb * _run_bytes(fmt) + cdiv(partner_rows, bp) * (rows // partner_rows) * nb

    def lines(R, L, fmt):  # R rows quantized in line blocks of 32 along L
        nb = cdiv(L, 32)
        return R * nb * _run_bytes(fmt) + R * nb

    xq = mx(s.h * s.w * s.n, s.cin, s.n, wl.fx, wl.bp)
    wq = mx(s.cout * s.kh * s.kw, s.cin, s.cout, wl.fw, wl.bp)
    gq = mx(ho * wo * s.n, s.cout, s.n, wl.fdy, wl.bp)
    once = (4 * (X + Wn + G) + xq + wq + gq) + (xq + wq + 4 * G) + (gq + wq + 4 * X) + (gq + xq + 4 * Wn)
    fwd = (4 * X + 4 * M * K) + (4 * M * K + lines(M, K, wl.fx)) + 8 * Wn + (4 * Wn + lines(s.cout, K, wl.fw)) \
        + (lines(M, K, wl.fx) + lines(s.cout, K, wl.fw) + 4 * G)
    dgrad = (4 * G + lines(M, s.cout, wl.fdy)) + 8 * Wn + (4 * Wn + lines(K, s.cout, wl.fw)) \
        + (lines(M, s.cout, wl.fdy) + lines(K, s.cout, wl.fw) + 4 * M * K) + (4 * M * K + 4 * X)
    wgrad = 8 * G + (4 * G + lines(s.cout, M, wl.fdy)) + (4 * X + 4 * M * K) + (4 * M * K + lines(K, M, wl.fx)) \
        + (lines(s.cout, M, wl.fdy) + lines(K, M, wl.fx) + 4 * Wn)
    return {"microqonv": float(once), "naive": float(fwd + dgrad + wgrad)}


def summarize(d: str, workload: str, out_dir: str) -> dict:
    copy_bytes = COPY_MB * (1 << 20)
    cf = [v for k, v in _read(d, "copy_fetch", "FETCH_SIZE") if "mq::" not in k]
    cw = [v for k, v in _read(d, "copy_write", "WRITE_SIZE") if "mq::" not in k]
    # the copy is the largest dispatch of its run (the fill before it writes only)
    f_fetch = max(cf) / copy_bytes
    f_write = max(cw) / copy_bytes
    res = {"workload": workload, "copy_MiB": COPY_MB, "fetch_factor": round(f_fetch, 4),
           "write_factor": round(f_write, 4), "source_sha": _source_sha(), "paths": {}}
    lines = []
    for path, stem in (("microqonv", "mq"), ("naive", "naive")):
        fe = [(k, v / f_fetch) for k, v in _read(d, f"{stem}_fetch", "FETCH_SIZE") if "mq::" in k]
        wr = [(k, v / f_write) for k, v in _read(d, f"{stem}_write", "WRITE_SIZE") if "mq::" in k]
        per_kernel = {}
        for k, v in fe:
            key = k.split("(")[0].replace("void ", "")
            per_kernel.setdefault(key, [0.0, 0.0, 0])
            per_kernel[key][0] += v
            per_kernel[key][2] += 1
        for k, v in wr:
            key = k.split("(")[0].replace("void ", "")
            per_kernel.setdefault(key, [0.0, 0.0, 0])
            per_kernel[key][1] += v
        tot_f, tot_w = sum(v for _, v in fe), sum(v for _, v in wr)
        res["paths"][path] = {"fetch_bytes": tot_f, "write_bytes": tot_w, "total_bytes": tot_f + tot_w,
                              "dispatches": len(fe),
                              "kernels": {k: {"fetch": v[0], "write": v[1], "dispatches": v[2]}
                                          for k, v in per_kernel.items()}}
        lines.append(f"{path}: {len(fe)} dispatches, read {tot_f / 1e6:.1f} MB, write {tot_w / 1e6:.1f} MB, "
                     f"total {(tot_f + tot_w) / 1e6:.1f} MB")
        for k, v in sorted(per_kernel.items(), key=lambda kv: -(kv[1][0] + kv[1][1])):
            lines.append(f"    {k[:70]:70s} x{v[2]:3d}  read {v[0] / 1e6:9.2f} MB  write {v[1] / 1e6:9.2f} MB")
    m, n = res["paths"]["microqonv"]["total_bytes"], res["paths"]["naive"]["total_bytes"]
    res["naive_over_microqonv"] = round(n / m, 3)
    lines.append(f"naive / quantize-once bytes: x{n / m:.2f}")
    mod = {"microqonv": 0.0, "naive": 0.0}
    for wl in _workloads(workload):
        for k, v in model_bytes(wl).items():
            mod[k] += v
    res["model_bytes"] = mod
    res["model_naive_over_microqonv"] = round(mod["naive"] / mod["microqonv"], 3)
    lines.append("full-kernel model (each kernel's inputs read once, outputs written once): "
                 f"quantize-once {mod['microqonv'] / 1e6:.1f} MB, naive {mod['naive'] / 1e6:.1f} MB, "
                 f"x{mod['naive'] / mod['microqonv']:.2f}")
    lines.append(f"measured / model: quantize-once x{m / mod['microqonv']:.2f}, naive x{n / mod['naive']:.2f}")
    text = "\n".join(lines)
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"bytes_{workload}.json"), "w") as fh:
        json.dump(res, fh, indent=1)
    print(text)
    return res


def summarize_call(d: str, workload: str, call: str, out_dir: str, command: str) -> dict:
    """HBM bytes of one call: FETCH_SIZE and WRITE_SIZE of its own dispatches
    (every mq:: dispatch of the call run except the quantize kernels of the
    prelude), each divided by the copy's factor."""
    copy_bytes = COPY_MB * (1 << 20)
    f_fetch = max(v for k, v in _read(d, "copy_fetch", "FETCH_SIZE") if "mq::" not in k) / copy_bytes
    f_write = max(v for k, v in _read(d, "copy_write", "WRITE_SIZE") if "mq::" not in k) / copy_bytes
    own = lambda k: "mq::" in k and "mxq_quantize_kernel" not in k
    fe = [(k, v / f_fetch) for k, v in _read(d, "call_fetch", "FETCH_SIZE") if own(k)]
    wr = [(k, v / f_write) for k, v in _read(d, "call_write", "WRITE_SIZE") if own(k)]
    per = {}
    for k, v in fe:
        per.setdefault(k.split("(")[0].replace("void ", ""), [0.0, 0.0])[0] += v
    for k, v in wr:
        per.setdefault(k.split("(")[0].replace("void ", ""), [0.0, 0.0])[1] += v
    tf, tw = sum(v for _, v in fe), sum(v for _, v in wr)
    wl = WORKLOADS_ONE(workload)
    rec = {"workload": wl.name, "call": call, "dispatches": len(fe), "fetch_bytes": tf, "write_bytes": tw,
           "traffic_bytes": tf + tw, "fetch_factor": round(f_fetch, 4), "write_factor": round(f_write, 4),
           "copy_MiB": COPY_MB, "kernels": {k: {"fetch": v[0], "write": v[1]} for k, v in per.items()},
           "source_sha": _source_sha(), "command": command}
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"traffic_{wl.name}_{call}.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
    print(json.dumps(rec, indent=1))
    return rec


MFMA_COUNTERS = ("GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_F8",
                 "SQ_INSTS_VALU_MFMA_MOPS_F6F4")
N_XCC, N_SIMD = 8, 1024  # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def summarize_mfma(d: str, stem: str, workload: str, out_dir: str, command: str) -> str:
    """Per GEMM dispatch of a step run (one counter pass with MFMA_COUNTERS):
      MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES (summed over all SIMDs) divided by
                  the kernel's cycles (GRBM_GUI_ACTIVE summed over the 8 XCDs,
                  / 8) times the 1024 SIMDs;
      executed  = (MOPS_F8 + MOPS_F6F4) x 512 matrix operations (adds and
                  multiplies, zero padding of short K-blocks included), against
                  the GEMM's algorithmic 2 N Ho Wo Cout Cin Kh Kw."""
    files = glob.glob(os.path.join(d, "**", f"{stem}_counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no {stem}_counter_collection.csv under {d}")
    per = {}
    for r in csv.DictReader(open(files[0])):
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Kernel_Name"])
        per.setdefault(key, {})[r["Counter_Name"]] = per.get(key, {}).get(r["Counter_Name"], 0.0) + float(
            r["Counter_Value"])
    wls = _workloads(workload)
    flops = sum(wl.shape.flops() for wl in wls)
    lines = [f"MFMA counters of one training step, workload {workload} ({len(wls)} layer(s)); "
             f"algorithmic FLOP per GEMM kind {flops / 1e9:.2f} G", "", "Command (run from the repository root on one MI355X):",
             "  " + command, f"Library source hash: {_source_sha()}", "",
             f"{'kernel':74s} {'calls':>5s} {'cycles':>9s} {'MFMA busy':>9s} {'exec GFLOP':>10s}"]
    agg = {}
    for (_, name), c in per.items():
        if "mx_gemm_kernel" not in name:
            continue
        k = name.split("(")[0].replace("void ", "")
        a = agg.setdefault(k, [0, 0.0, 0.0, 0.0])
        a[0] += 1
        a[1] += c.get("GRBM_GUI_ACTIVE", 0.0) / N_XCC
        a[2] += c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        a[3] += (c.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0.0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0)) * 512
    for k, (n, cyc, busy, ops) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        frac = busy / (cyc * N_SIMD) if cyc else 0.0
        lines.append(f"{k[:74]:74s} {n:5d} {cyc / n:9.0f} {frac:9.3f} {ops / n / 1e9:10.2f}")
    text = "\n".join(lines) + "\n"
    os.makedirs(out_dir, exist_ok=True)
    wl_name = wls[0].name if len(wls) == 1 else "c3_yolov8n_backbone_27convs_n16"
    with open(os.path.join(out_dir, f"mfma_{wl_name}.txt"), "w") as fh:
        fh.write(text)
    print(text)
    return text


def summarize_kernels(d: str, stem: str, bench_log: str, workload: str, title: str, out_dir: str,
                      command: str) -> str:
    """Kernel statistics of a rocprofv3 --kernel-trace --stats run of bench.py
    (D/<stem>_kernel_stats.csv) next to bench.py's own per-call times of the
    same run (the JSON line of its log): profiles/kernels_<workload>.txt."""
    from microscaling_quantized_convolution_mxq_amd.workloads import WORKLOADS
    paths = glob.glob(os.path.join(d, "**", f"{stem}_kernel_stats.csv"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no {stem}_kernel_stats.csv under {d}")
    rows = list(csv.DictReader(open(paths[0])))

    def col(r, *keys):
        for k in r:
            if any(k.lower() == key.lower() for key in keys):
                return r[k]
        raise KeyError(keys)
    def short(name):  # without the return type and the parameter list
        name = name[5:] if name.startswith("void ") else name
        depth = 0
        for i, ch in enumerate(name):
            depth += ch == "<"
            depth -= ch == ">"
            if ch == "(" and depth == 0:
                return name[:i]
        return name
    stats = []
    for r in rows:
        stats.append((short(col(r, "Name", "KernelName", "Kernel_Name")), int(float(col(r, "Calls"))),
                      float(col(r, "AverageNs")) / 1e3, float(col(r, "MinNs")) / 1e3,
                      float(col(r, "MaxNs")) / 1e3, float(col(r, "Percentage"))))
    stats.sort(key=lambda t: -t[5])
    line = [x for x in open(bench_log) if x.startswith("{")][-1]
    b = json.loads(line)
    full = WORKLOADS[workload].name
    out = [title, "", "Command (run from the repository root on one MI355X):", f"  {command}",
           f"Library source hash: {_source_sha()}", "",
           "rocprofv3 kernel statistics (durations in microseconds; per launch):", "",
           f"{'kernel':88s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'share':>7s}"]
    for name, calls, avg, mn, mx, pct in stats:
        out.append(f"{name[:88]:88s} {calls:6d} {avg:9.2f} {mn:9.2f} {mx:9.2f} {pct:6.2f}%")
    out += ["", "bench.py per-call times of the same run (HIP events over graphs of calls, microseconds):"]
    for k, v in b["kernels"].items():
        out.append(f"  {k:24s} {v['ms'] * 1000:9.2f}   launches: {'; '.join(v['launches'])}")
    out += ["", f"Dominant entry point: {b['roofline']['kernel']}; roofline object of the same run: "
            f"{json.dumps(b['roofline'])}",
            f"Step: {b['value']:.3f} TFLOP/s, {b['ms_per_step']:.5f} ms per step (traced run)."]
    text = "\n".join(out) + "\n"
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"kernels_{full}.txt"), "w") as f:
        f.write(text)
    return text


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    a = sub.add_parser("step")
    a.add_argument("--workload", default="c2")
    a.add_argument("--path", choices=("microqonv", "naive"), default="microqonv")
    b = sub.add_parser("call")
    b.add_argument("--workload", default="c2")
    b.add_argument("--call", choices=CALL_NAMES, default="backward_weight")
    sub.add_parser("copy")
    e = sub.add_parser("summarize-call")
    e.add_argument("--dir", required=True)
    e.add_argument("--workload", default="c2")
    e.add_argument("--call", choices=CALL_NAMES, default="backward_weight")
    e.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    e.add_argument("--command", default="")
    f = sub.add_parser("mfma")
    f.add_argument("--dir", required=True)
    f.add_argument("--stem", default="mfma")
    f.add_argument("--workload", default="c2")
    f.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    f.add_argument("--command", default="")
    k = sub.add_parser("kernels")
    k.add_argument("--dir", required=True)
    k.add_argument("--stem", default="kt")
    k.add_argument("--bench-log", required=True)
    k.add_argument("--workload", default="c5")
    k.add_argument("--title", default="")
    k.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    k.add_argument("--command", default="")
    c = sub.add_parser("summarize")
    c.add_argument("--dir", required=True)
    c.add_argument("--workload", default="c2")
    c.add_argument("--out", default=os.path.join(ROOT, "gpurun_out"))
    args = ap.parse_args(argv)
    if args.mode == "step":
        run_step(args.workload, args.path)
    elif args.mode == "call":
        run_call(args.workload, args.call)
    elif args.mode == "copy":
        run_copy()
    elif args.mode == "mfma":
        summarize_mfma(args.dir, args.stem, args.workload, args.out, args.command)
    elif args.mode == "kernels":
        summarize_kernels(args.dir, args.stem, args.bench_log, args.workload, args.title, args.out, args.command)
    elif args.mode == "summarize-call":
        summarize_call(args.dir, args.workload, args.call, args.out, args.command)
    else:
        summarize(args.dir, args.workload, args.out)


if __name__ == "__main__":
    main()
