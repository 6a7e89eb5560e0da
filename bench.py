"""Benchmark of the S3R-EC quantized backward of one linear layer on one MI355X.

One step = the whole backward hot path on one batch of synthetic input: the
fused quantizer (fold, per-tensor step, S3R thresholds, codes, S3R-EC
statistics), dX (correction GEMV + INT8 GEMM with dequant/correction
epilogue) and dW (correction GEMV + INT8 GEMM with epilogue).  The forward
operand prep (RTNE codes of X and W with their scales and column sums) is
forward-pass work and runs once before timing.

Prints one JSON line.  ``value`` is the step's INT8 throughput in TOP/s:
2 GEMMs x 2*T*D*d_in ops over the measured step time (the quantizer and the
correction are inside the step).  Extra fields report the quantizer's GB/s
(algorithmic bytes: one read of G plus one write of Q) and each kernel's time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0     # MI355X dense INT8 MFMA, TOP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, GB/s

# HBM byte counts of the GEMM kernels, taken with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE and
# scaled by the same counters' reading for a plain copy of known size.  The file records the
# sha256 of the kernel source it was measured on; a stale record is not reported.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_down-8192x14336x4096.md")
GEMM_SOURCE = os.path.join(ROOT, "stochastic_rounding_quantization_amd", "csrc", "gemm.hip")

MODES = {
    "s3r-ec-two-way": (2, 2), "s3r-ec-dx-only": (2, 1), "s3r": (2, 0), "sr": (1, 0), "rtne": (0, 0),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(kernel_key, workload):
    """HBM bytes per launch of one GEMM kernel from the committed counter summary, or None."""
    import hashlib
    import re
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if not m or m.group(1) != src or f"workload: {workload}" not in text:
        return None
    m = re.search(rf"{kernel_key}_hbm_bytes_per_launch:\s*([0-9]+)", text)
    return int(m.group(1)) if m else None


def copy_calibration(device, nbytes=1 << 30, reps=4):
    """A plain device-to-device copy of ``nbytes`` (torch's copy kernel), run ``reps`` times.

    Under rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE per dispatch against the known ``nbytes``
    gives the factor that turns those counters into bytes."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.int32, device=device).fill_(7)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def cpu_baseline(inp, w, mode, ec, rows):
    """Time the CPU oracle on a bounded sample: the first ``rows`` tokens of the workload."""
    import numpy as np
    from oracle import backward, pipeline
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    S = min(w.rows_per_example, rows)
    sample = {"G": inp["G"][:rows], "X": inp["X"][:rows], "W": inp["W"], "dtype": inp["dtype"]}
    fx, fw = pipeline.forward_operands(sample["X"], sample["W"], inp["dtype"], S)
    t0 = time.perf_counter()
    q = pipeline.quantize_gradient(sample["G"], inp["dtype"], fx, fw, mode=mode, scale=0, seed=0, layer_id=0,
                                   rows_per_example=S)
    dx = backward.backward_dx(q["Q"], q["delta"], fw["Q"], fx["scale"], ec=ec, r_W=fw["code_colsum"][0],
                              eps=q["eps"], ebar=q["ebar"], mu=q["mu"], rows_per_example=S)
    dw = backward.backward_dw(q["Q"], q["delta"], fx["Q"], fw["scale"], ec=ec, xs=fx["code_colsum"],
                              eps=q["eps"], ebar=q["ebar"], mu=q["mu"], rows_per_example=S)
    dt = time.perf_counter() - t0
    assert np.isfinite(dx).all() and np.isfinite(dw).all()
    ops = 2 * 2.0 * rows * w.d_out * w.d_in
    return {"value": ops / dt / 1e12, "unit": "TOP/s", "cores": int(blas_threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": ("the whole workload: " if rows == w.tokens else f"first {rows} tokens of the workload: ") +
                      f"{rows} tokens ({rows // S} example(s) of {S}), "
                      f"D={w.d_out} and d_in={w.d_in}: numpy quantizer (1 thread) + dX + dW with float64 BLAS "
                      f"integer GEMMs ({blas_threads} BLAS threads); forward-operand prep untimed"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="down-8192x14336x4096-bf16")
    ap.add_argument("--mode", default="s3r-ec-two-way", choices=sorted(MODES))
    ap.add_argument("--cpu-rows", type=int, default=-1,
                    help="tokens in the CPU-oracle sample (-1: the whole workload, 0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (reference for HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU path is design-only)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from stochastic_rounding_quantization_amd import inputs, s3r

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(dev)
        return
    s3r.lib()   # fail loudly if the HIP library is missing
    mode, ec = MODES[args.mode]
    w = inputs.WORKLOADS[args.workload]
    T, D, K, S = w.tokens, w.d_out, w.d_in, w.rows_per_example
    log(f"workload {w.name}: T={T} D={D} d_in={K} S={S} mode={args.mode}; drawing inputs")
    inp = inputs.make_linear_inputs(w)

    def to_dev(a):
        if inp["dtype"] == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    G, X, W = to_dev(inp["G"]), to_dev(inp["X"]), to_dev(inp["W"])
    log("forward-operand prep (untimed)")
    fx = s3r.forward_operand(X, rows_per_example=S)
    fw = s3r.forward_operand(W, rows_per_example=D)
    del X, W
    desc = s3r.qdesc(T, D, S, mode, ec, s3r.PER_TENSOR, layer_id=0, seed=0)
    B = T // S
    Q = s3r.q_buffer(T, D, dev)
    delta = torch.empty(1, dtype=torch.float32, device=dev)
    e_r = torch.empty(T, dtype=torch.float32, device=dev) if ec else None
    e_c = torch.empty(B, D, dtype=torch.float32, device=dev) if ec else None
    e_m = torch.empty(B, dtype=torch.float32, device=dev) if ec else None
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    ws_q = torch.zeros(max(s3r.s3r_quantize_workspace(desc), 1), dtype=torch.uint8, device=dev)
    ws_b = torch.zeros(max(s3r.s3r_backward_workspace(desc, K), 1), dtype=torch.uint8, device=dev)
    dX = torch.empty(T, K, dtype=torch.float32, device=dev)
    dW = torch.empty(D, K, dtype=torch.float32, device=dev)
    s_x, s_w = fx.delta, fw.delta
    r_W, xs = fw.code_colsum[0], fx.code_colsum

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()          # creates the underlying HIP event
        return e

    def step(events=None):
        if events:
            events[0].record()
        s3r.s3r_quantize(desc, G, s_x, s_w, Q, delta, None, e_r, e_c, e_m, flags, ws_q)
        if events:
            events[1].record()
            s3r.s3r_time_next_gemm(events[2], events[3])
        s3r.s3r_backward_dx(desc, Q, delta, fw.Q, s_x, r_W, e_r, e_c, e_m, dX, ws_b)
        if events:
            s3r.s3r_time_next_gemm(events[4], events[5])
        s3r.s3r_backward_dw(desc, Q, delta, fx.Q, s_w, xs, e_r, e_c, e_m, dW, ws_b)
        if events:
            events[6].record()

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[ev() for _ in range(7)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    assert int(flags.item()) == 0

    def avg(a, b):
        return float(np.mean([e[a].elapsed_time(e[b]) for e in evs]))   # ms

    t_q = avg(0, 1)
    t_gx = avg(2, 3)
    t_gw = avg(4, 5)
    t_step_ev = avg(0, 6)
    gop = 2.0 * T * D * K / 1e9
    value = 2 * gop / (ms_step / 1e3) / 1e3          # TOP/s
    q_bytes = T * D * (2 if inp["dtype"] == "bf16" else 4) + T * D
    q_gbs = q_bytes / (t_q / 1e3) / 1e9
    dom_key, dom_name, t_dom = ("dw", "gemm dW (gemm_i8_kernel<false, EPI_DW>)", t_gw) if t_gw >= t_gx else \
        ("dx", "gemm dX (gemm_i8_kernel<true, EPI_DX>)", t_gx)
    achieved = gop / (t_dom / 1e3) / 1e3              # TOP/s
    out = {
        "metric": "S3R-EC backward TOPS (quant+INT8 dX/dW) & quantizer GB/s, % of MI355X peak",
        "value": round(value, 2), "unit": "TOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "d_in": K, "d_out": D, "rows_per_example": S,
                   "mode": args.mode, "step_scale": "per-tensor", "g_dtype": inp["dtype"]},
        "frac_of_int8_peak": round(value / PEAK_INT8_TOPS, 4),
        "quantizer": {"us": round(t_q * 1e3, 2), "GB_s": round(q_gbs, 1),
                      "frac_of_hbm_peak": round(q_gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": q_bytes},
        "kernels_us": {"quantize_call": round(t_q * 1e3, 2), "gemm_dx": round(t_gx * 1e3, 2),
                       "gemm_dw": round(t_gw * 1e3, 2), "step_events": round(t_step_ev * 1e3, 2)},
        "gemm_tops": {"dx": round(gop / (t_gx / 1e3) / 1e3, 1), "dw": round(gop / (t_gw / 1e3) / 1e3, 1)},
        "roofline": {"kernel": dom_name, "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_INT8_TOPS, "unit": "TOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4),
                     "traffic": measured_traffic(dom_key, w.name),
                     "algorithmic": f"2*T*D*d_in = {gop:.1f} GOP per launch (int8 multiply-adds x 2)"},
    }
    if args.cpu_rows != 0:
        rows = T if args.cpu_rows < 0 else min(args.cpu_rows, T)
        rows = max(S, rows // S * S)
        log(f"CPU oracle baseline on the first {rows} tokens")
        out["cpu_baseline"] = cpu_baseline(inp, w, mode, ec, rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
