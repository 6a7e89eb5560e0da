"""Benchmark of the S3R-EC quantized backward on one MI355X.

Default workload: the backward of one Llama-3-8B-shaped SwiGLU FFN block
(T = 8192 tokens in 4 examples of 2048, d_model 4096, d_ff 14336, bf16).  One
step = the whole backward on one batch of synthetic input:
  down projection: quantize G_out (fold, per-tensor step, S3R thresholds,
    codes, S3R-EC statistics) -> dH (correction GEMV + INT8 GEMM + epilogue)
    -> dW_down (correction GEMV + INT8 GEMM + epilogue);
  SwiGLU glue: dH, A_gate, A_up -> G_gate, G_up (bf16), and in the same pass
    the per-tensor amax of each as its projection's quantizer folds it;
  gate and up projections: quantize with that amax (one read of G), dX
    (added into one dX) and dW.
The forward-operand prep (RTNE codes of X, H and the three weights with their
scales and column sums) is forward-pass work and runs once before timing.
The step is timed on one stream and, with ``--streams 2`` (the default), with
each projection's dW (its correction GEMV and INT8 GEMM) on a second HIP stream
after that projection's dX, beside the next stage; the faster of the two is
reported.  The per-kernel fields come from a single-stream pass of the same step
with an event pair around each kernel.
``--workload down-8192x14336x4096-bf16`` (or another linear workload) times one
linear layer's backward instead.

Prints one JSON line.  ``value`` is the step's INT8 throughput in TOP/s: the
GEMMs' 2*M*N*K ops (6 GEMMs for the block, 2 for a linear layer) over the
measured step time, with everything else inside the step.  Extra fields report
the quantizer's GB/s (algorithmic bytes: one read of G plus one write of Q per
quantize call) and each stage's time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0     # MI355X dense INT8 MFMA, TOP/s
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, GB/s
PEAK_FP4_TFLOPS = 10100.0   # MI355X dense FP4 (MXFP4) MFMA, TFLOP/s

# Byte counts of the GEMM kernels, taken with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE and scaled by
# the same counters' reading for a plain copy of known size.  Those counters see the L2's requests to
# the fabric, last-level (MALL) hits included, so the figure bounds the HBM bytes from above.  The
# file records the sha256 of the kernel source it was measured on; a stale record is not reported.
TRAFFIC_FILES = {
    "down-8192x14336x4096-bf16": os.path.join(ROOT, "profiles", "traffic_gemm_down-8192x14336x4096.md"),
    "ffn-block-8192x4096x14336-bf16": os.path.join(ROOT, "profiles", "traffic_gemm_ffn-block-8192x4096x14336.md"),
}
GEMM_SOURCE = os.path.join(ROOT, "stochastic_rounding_quantization_amd", "csrc", "gemm.hip")

MODES = {
    "s3r-ec-two-way": (2, 2), "s3r-ec-dx-only": (2, 1), "s3r": (2, 0), "sr": (1, 0), "rtne": (0, 0),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(kernel_key, workload):
    """L2-to-fabric bytes (reads + writes) per launch of one GEMM kernel from the committed counter
    summary, or None."""
    import hashlib
    import re
    path = TRAFFIC_FILES.get(workload)
    if path is None or not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    if not m or m.group(1) != src or f"workload: {workload}" not in text:
        return None
    m = re.search(rf"{kernel_key}_l2_egress_bytes_per_launch:\s*([0-9]+)", text)
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


def cpu_baseline(inp, w, mode, ec, rows, repeats=1, single_thread=False):
    """Time the CPU oracle on a bounded sample: the first ``rows`` tokens of the workload.

    ``repeats`` runs are timed and the median reported; ``single_thread`` adds the same sample
    timed with every BLAS pool limited to one thread."""
    import numpy as np
    from oracle import backward, pipeline
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        blas_threads = 1
    S = min(w.rows_per_example, rows)
    sample = {"G": inp["G"][:rows], "X": inp["X"][:rows], "W": inp["W"], "dtype": inp["dtype"]}
    fx, fw = pipeline.forward_operands(sample["X"], sample["W"], inp["dtype"], S)

    def once():
        t0 = time.perf_counter()
        q = pipeline.quantize_gradient(sample["G"], inp["dtype"], fx, fw, mode=mode, scale=0, seed=0, layer_id=0,
                                       rows_per_example=S)
        dx = backward.backward_dx(q["Q"], q["delta"], fw["Q"], fx["scale"], ec=ec, r_W=fw["code_colsum"][0],
                                  eps=q["eps"], ebar=q["ebar"], mu=q["mu"], rows_per_example=S)
        dw = backward.backward_dw(q["Q"], q["delta"], fx["Q"], fw["scale"], ec=ec, xs=fx["code_colsum"],
                                  eps=q["eps"], ebar=q["ebar"], mu=q["mu"], rows_per_example=S)
        dt = time.perf_counter() - t0
        assert np.isfinite(dx).all() and np.isfinite(dw).all()
        return dt

    ops = 2 * 2.0 * rows * w.d_out * w.d_in
    runs = [once() for _ in range(repeats)]
    dt = float(np.median(runs))
    out = {"value": ops / dt / 1e12, "unit": "TOP/s", "cores": int(blas_threads), "kind": "oracle",
           "seconds": round(dt, 4), "runs_s": [round(r, 4) for r in runs],
           "sample": ("the whole workload: " if rows == w.tokens else f"first {rows} tokens of the workload: ") +
                     f"{rows} tokens ({rows // S} example(s) of {S}), "
                     f"D={w.d_out} and d_in={w.d_in}: numpy quantizer (1 thread) + dX + dW with float64 BLAS "
                     f"integer GEMMs ({blas_threads} BLAS threads); forward-operand prep untimed; "
                     f"median of {repeats} run(s)"}
    if single_thread and threadpool_limits is not None:
        with threadpool_limits(limits=1):
            runs1 = [once() for _ in range(repeats)]
        dt1 = float(np.median(runs1))
        out["single_thread"] = {"value": ops / dt1 / 1e12, "unit": "TOP/s", "cores": 1, "seconds": round(dt1, 4),
                                "runs_s": [round(r, 4) for r in runs1]}
    return out


def block_cpu_baseline(inp, b, mode, ec, rows):
    """Time the CPU oracle's FFN-block backward on the first ``rows`` tokens (whole examples)."""
    import numpy as np
    from oracle import pipeline
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    S = b.rows_per_example
    sample = {k: (v[:rows] if k in ("G", "X", "H", "A_gate", "A_up") else v) for k, v in inp.items()}
    t0 = time.perf_counter()
    r = pipeline.ffn_block_backward(sample, mode=mode, ec=ec, rows_per_example=S)
    dt = time.perf_counter() - t0
    assert np.isfinite(r["dX"]).all()
    ops = 6 * 2.0 * rows * b.d_model * b.d_ff
    return {"value": ops / dt / 1e12, "unit": "TOP/s", "cores": int(blas_threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"first {rows} tokens ({rows // S} example(s) of {S}) of the block, full d_model={b.d_model} "
                      f"and d_ff={b.d_ff}: three quantizers and the glue in numpy (1 thread), six float64 BLAS "
                      f"integer GEMMs ({blas_threads} BLAS threads), forward-operand prep inside the timing"}


class Timeline:
    """Named intervals of one step, timed with HIP events on the launch stream."""

    def __init__(self, torch, names, steps):
        self.torch, self.names = torch, names
        self.ev = []
        for _ in range(steps):
            d = {}
            for n in names:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(); b.record()          # creates the underlying HIP events
                d[n] = (a, b)
            self.ev.append(d)

    def avg_us(self, name):
        import numpy as np
        return float(np.mean([d[name][0].elapsed_time(d[name][1]) for d in self.ev])) * 1e3

    def spread(self):
        """[min, median, max] in us of every interval over the timed steps."""
        import numpy as np
        out = {}
        for n in self.names:
            v = np.array([d[n][0].elapsed_time(d[n][1]) for d in self.ev]) * 1e3
            out[n] = [round(float(v.min()), 2), round(float(np.median(v)), 2), round(float(v.max()), 2)]
        return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ffn-block-8192x4096x14336-bf16")
    ap.add_argument("--mode", default="s3r-ec-two-way", choices=sorted(MODES))
    ap.add_argument("--streams", type=int, default=2, choices=(1, 2, 3),
                    help="FFN block: 2 runs each dW product on a second stream after its dX, 3 after its quantize "
                         "call (beside the dX); a single linear or MoE layer: above 1 times its dW on a second "
                         "stream after the quantize call. Above 1 the step is also timed on one stream and the "
                         "faster schedule is reported. Per-kernel fields always come from a single-stream pass")
    ap.add_argument("--dw-pair", type=int, default=1, choices=(0, 1),
                    help="FFN block: the gate and up projections' dW as one launch (1) or two (0)")
    ap.add_argument("--fuse-glue", type=int, default=0, choices=(0, 1),
                    help="FFN block: 1 computes the SwiGLU glue inside the gate and up quantizers "
                         "(s3r_swiglu_quantize: G_gate and G_up are never written); 0 writes them in the glue pass")
    ap.add_argument("--cpu-rows", type=int, default=-1,
                    help="tokens in the CPU-oracle sample (-1: the default sample, 0: skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (reference for HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU path is design-only)", file=sys.stderr)
        sys.exit(2)

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
    if args.workload in inputs.BLOCKS:
        out = run_block(args, dev, torch, inputs, s3r)
    elif args.workload in inputs.MOE:
        out = run_moe(args, dev, torch, inputs, s3r)
    elif args.workload in inputs.MX_WORKLOADS:
        out = run_mx(args, dev, torch, inputs, s3r)
    else:
        out = run_linear(args, dev, torch, inputs, s3r)
    print(json.dumps(out), flush=True)


def _to_dev(torch, dev, a, dtype):
    import numpy as np
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def _timed_steps(torch, step, tl, steps, warmup):
    log(f"warmup {warmup}")
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    log(f"timing {steps} steps")
    t0 = time.perf_counter()
    for i in range(steps):
        step(tl.ev[i])
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def _pick_streams(torch, args, make_step, ms_single):
    """Single-layer step: with --streams above 1, time the step with its dW on a second stream too and
    report the faster schedule (a small, launch-bound layer loses the overlap to the cross-stream events).
    Returns (ms per step, streams used, two-stream ms or None)."""
    if args.streams <= 1:
        return ms_single, 1, None
    log("timing the step with 2 streams")
    stepn = make_step(2)
    ms_two = _timed_steps(torch, lambda ev: stepn(None), Timeline(torch, [], args.steps), args.steps, args.warmup)
    if ms_two < ms_single:
        return ms_two, 2, round(ms_two, 4)
    return ms_single, 1, round(ms_two, 4)


def _roofline(gemm_us, workload, gop):
    """The longest GEMM launch against the INT8 peak; gop: GOP per launch (a number, or one per key)."""
    key = max(gemm_us, key=lambda k: gemm_us[k])
    gop = gop[key] if isinstance(gop, dict) else gop
    achieved = gop / (gemm_us[key] / 1e6) / 1e3
    return {"kernel": f"gemm {key}", "bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_INT8_TOPS,
            "unit": "TOP/s", "frac": round(achieved / PEAK_INT8_TOPS, 4), "traffic": measured_traffic(key, workload),
            "traffic_counts": "FETCH_SIZE + WRITE_SIZE bytes per launch: L2-to-fabric traffic, MALL hits included",
            "algorithmic": f"2*M*N*K = {gop:.1f} GOP per launch (int8 multiply-adds x 2)"}


def run_block(args, dev, torch, inputs, s3r):
    mode, ec = MODES[args.mode]
    b = inputs.BLOCKS[args.workload]
    T, M, F, S = b.tokens, b.d_model, b.d_ff, b.rows_per_example
    B = T // S
    log(f"workload {b.name}: T={T} d_model={M} d_ff={F} S={S} mode={args.mode}; drawing inputs")
    inp = inputs.make_ffn_block_inputs(b)
    dv = {k: _to_dev(torch, dev, inp[k], "bf16") for k in ("G", "X", "H", "W_down", "W_gate", "W_up", "A_gate", "A_up")}
    log("forward-operand prep (untimed)")
    fx = s3r.forward_operand(dv["X"], rows_per_example=S)
    fh = s3r.forward_operand(dv["H"], rows_per_example=S)
    fwd = s3r.forward_operand(dv["W_down"], rows_per_example=M)
    fwg = s3r.forward_operand(dv["W_gate"], rows_per_example=F)
    fwu = s3r.forward_operand(dv["W_up"], rows_per_example=F)
    for k in ("X", "H", "W_down", "W_gate", "W_up"):
        del dv[k]
    proj = {  # name: (rows of G, cols of G = D, d_in, layer, forward operand of X, of W)
        "down": (M, F, 0, fh, fwd), "gate": (F, M, 1, fx, fwg), "up": (F, M, 2, fx, fwu)}
    dH = torch.empty(T, F, dtype=torch.float32, device=dev)
    Gg = torch.empty(T, F, dtype=torch.bfloat16, device=dev)
    Gu = torch.empty_like(Gg)
    dX = torch.empty(T, M, dtype=torch.float32, device=dev)
    dW = {"down": torch.empty(M, F, dtype=torch.float32, device=dev),
          "gate": torch.empty(F, M, dtype=torch.float32, device=dev),
          "up": torch.empty(F, M, dtype=torch.float32, device=dev)}
    G_in = {"down": dv["G"], "gate": Gg, "up": Gu}
    dX_out = {"down": dH, "gate": dX, "up": dX}
    dw_keys = ["dw_down", "dw_gate_up"] if args.dw_pair else [f"dw_{n}" for n in proj]
    names = ["step", "glue"] + [f"quantize_{n}" for n in proj] + [f"dx_{n}" for n in proj] + dw_keys

    def make_step(mode, ec, streams, pair=True, fused=False):
        """The block's backward step for one rounding mode / correction, with its own descriptors and workspaces.
        pair: the gate and up projections' dW as one launch (s3r_backward_dw_pair) after the up projection's dX.
        fused: the glue computed inside the gate and up quantizers (one s3r_swiglu_quantize call in place of the
        glue pass and the two quantize calls; its time is the "glue" interval)."""
        st = {}
        for name, (D, din, layer, fxx, fww) in proj.items():
            d = s3r.qdesc(T, D, S, mode, ec, s3r.PER_TENSOR, layer_id=layer, seed=0)
            st[name] = dict(desc=d, Q=s3r.q_buffer(T, D, dev), delta=torch.empty(1, dtype=torch.float32, device=dev),
                            er=torch.empty(T, dtype=torch.float32, device=dev) if ec else None,
                            ec=torch.empty(B, D, dtype=torch.float32, device=dev) if ec else None,
                            em=torch.empty(B, dtype=torch.float32, device=dev) if ec else None,
                            flags=torch.zeros(1, dtype=torch.int32, device=dev), din=din, fx=fxx, fw=fww)
        ws_q = torch.empty(max(s3r.s3r_quantize_workspace(st[n]["desc"]) for n in st), dtype=torch.uint8,
                           device=dev)
        ws_g = torch.empty(s3r.s3r_swiglu_quantize_workspace(st["gate"]["desc"]) if fused
                           else s3r.s3r_swiglu_amax_workspace(T, F), dtype=torch.uint8, device=dev)
        amax = torch.zeros(2, dtype=torch.int32, device=dev)     # gate, up: max|G'| bits from the glue
        ws_b = torch.empty(max(max(s3r.s3r_backward_workspace(st[n]["desc"], st[n]["din"]) for n in st), 1),
                           dtype=torch.uint8, device=dev)
        # streams 2: the dW products (each with its U GEMV) on a second stream (default priority), each
        # after its dX; streams 3: the same second stream, each dW waiting only for its quantize call,
        # so it runs beside that projection's v GEMV and dX GEMM
        s2 = torch.cuda.Stream() if streams >= 2 else None
        ws_b2 = torch.empty_like(ws_b) if s2 is not None else ws_b
        ws_p = torch.empty(max(s3r.s3r_backward_dw_pair_workspace(st["gate"]["desc"], M), 1), dtype=torch.uint8,
                           device=dev)

        def side(after_dx):
            # the second stream waits for the main stream's work so far (streams 2: after a dX; 3: after a quantize)
            if s2 is not None and streams == (2 if after_dx else 3):
                e = torch.cuda.Event()
                e.record()
                s2.wait_event(e)

        sid = None if s2 is None else s2.cuda_stream

        def quantize(name, ev):
            p = st[name]
            if ev:
                ev[f"quantize_{name}"][0].record()
            if name == "down":
                s3r.s3r_quantize(p["desc"], G_in[name], p["fx"].delta, p["fw"].delta, p["Q"], p["delta"], None,
                                 p["er"], p["ec"], p["em"], p["flags"], ws_q)
            else:   # the glue already found the step's amax: one read of G
                k = 0 if name == "gate" else 1
                s3r.s3r_quantize_with_amax(p["desc"], G_in[name], p["fx"].delta, p["fw"].delta, amax[k:k + 1],
                                           p["Q"], p["delta"], p["er"], p["ec"], p["em"], p["flags"], ws_q)
            if ev:
                ev[f"quantize_{name}"][1].record()

        def dx(name, ev):
            p = st[name]
            if ev:
                s3r.s3r_time_next_gemm(*ev[f"dx_{name}"])
            s3r.s3r_backward_dx(p["desc"], p["Q"], p["delta"], p["fw"].Q, p["fx"].delta, p["fw"].code_colsum[0],
                                p["er"], p["ec"], p["em"], dX_out[name], ws_b, accumulate=(name == "up"))

        def dw(name, ev):
            p = st[name]
            if ev:
                s3r.s3r_time_next_gemm(*ev[f"dw_{name}"])
            s3r.s3r_backward_dw(p["desc"], p["Q"], p["delta"], p["fx"].Q, p["fw"].delta, p["fx"].code_colsum,
                                p["er"], p["ec"], p["em"], dW[name], ws_b2, stream=sid)

        def dw_pair(ev):
            g, u = st["gate"], st["up"]
            if ev:
                s3r.s3r_time_next_gemm(*ev["dw_gate_up"])
            s3r.s3r_backward_dw_pair(g["desc"], g["Q"], u["Q"], g["delta"], u["delta"], fx.Q, g["fw"].delta,
                                     u["fw"].delta, fx.code_colsum, (g["er"], g["ec"], g["em"]),
                                     (u["er"], u["ec"], u["em"]), dW["gate"], dW["up"], ws_p, stream=sid)

        def step(ev):
            if ev:
                ev["step"][0].record()
            quantize("down", ev)
            side(after_dx=False)
            dx("down", ev)
            side(after_dx=True)
            dw("down", ev)
            if ev:
                ev["glue"][0].record()
            if fused:
                g, u = st["gate"], st["up"]
                s3r.s3r_swiglu_quantize(g["desc"], u["desc"], dH, dv["A_gate"], dv["A_up"], fx.delta, fwg.delta,
                                        fwu.delta, g["Q"], u["Q"], g["delta"], u["delta"], (g["er"], g["ec"], g["em"]),
                                        (u["er"], u["ec"], u["em"]), g["flags"], ws_g)
            else:
                s3r.s3r_swiglu_backward_amax(dH, dv["A_gate"], dv["A_up"], Gg, Gu, fx.delta, fwg.delta, fwu.delta,
                                             amax, ws_g)
            if ev:
                ev["glue"][1].record()
            if fused and ev:        # no separate quantize calls: empty intervals
                for n in ("quantize_gate", "quantize_up"):
                    ev[n][0].record()
                    ev[n][1].record()
            q_gate = (lambda ev_: None) if fused else (lambda ev_: quantize("gate", ev_))
            q_up = (lambda ev_: None) if fused else (lambda ev_: quantize("up", ev_))
            if pair and streams == 3:
                # both quantize calls first; the paired dW on the second stream beside both dX products
                q_gate(ev)
                q_up(ev)
                side(after_dx=False)
                dw_pair(ev)
                dx("gate", ev)
                dx("up", ev)
            elif pair:
                q_gate(ev)
                dx("gate", ev)
                q_up(ev)
                dx("up", ev)
                side(after_dx=True)
                dw_pair(ev)
            else:
                for name in ("gate", "up"):
                    (q_gate if name == "gate" else q_up)(ev)
                    side(after_dx=False)
                    dx(name, ev)
                    side(after_dx=True)
                    dw(name, ev)
            if s2 is not None:
                e = torch.cuda.Event()
                e.record(s2)
                torch.cuda.current_stream().wait_event(e)
            if ev:
                ev["step"][1].record()

        return step, st

    # per-kernel times from a single-stream pass (an event pair around a kernel that shares the GPU
    # with another stream's work would time both); the step itself in the configured schedule
    step, st = make_step(mode, ec, 1, args.dw_pair, bool(args.fuse_glue))
    tl = Timeline(torch, names, args.steps)
    ms_single = _timed_steps(torch, step, tl, args.steps, args.warmup)
    for n in st:
        assert int(st[n]["flags"].item()) == 0, n

    sched = {"streams": args.streams}

    def step_ms(m2, e2, pair=args.dw_pair, fused=bool(args.fuse_glue), streams=None):
        """Whole-step time (no per-kernel events); streams: the schedule (default: the one reported)."""
        stepn, _ = make_step(m2, e2, streams or sched["streams"], pair, fused)
        return _timed_steps(torch, lambda ev: stepn(None), Timeline(torch, [], args.steps), args.steps,
                            args.warmup)

    # the whole step on one stream and in the --streams schedule, both without per-kernel events; the faster
    # is reported (on a power-limited chip two GEMMs side by side need not beat one after the other)
    log("timing the step on one stream")
    ms_by_streams = {1: step_ms(mode, ec, streams=1)}
    if args.streams > 1:
        log(f"timing the step with {args.streams} streams")
        ms_by_streams[args.streams] = step_ms(mode, ec, streams=args.streams)
    sched["streams"] = min(ms_by_streams, key=ms_by_streams.get)
    ms_step = ms_by_streams[sched["streams"]]
    gop = 2.0 * T * M * F / 1e9                      # each of the six GEMMs
    value = 6 * gop / (ms_step / 1e3) / 1e3
    gemm_us = {k: tl.avg_us(k) for k in [f"dx_{n}" for n in st] + dw_keys}
    gemm_gop = {k: gop * (2 if k == "dw_gate_up" else 1) for k in gemm_us}
    q_us = sum(tl.avg_us(f"quantize_{n}") for n in st)
    q_bytes = (T * M + 2 * T * F) * 3                 # bf16 G read once + int8 Q written, three calls
    if args.fuse_glue:   # the gate and up quantizers are the fused call: two passes over dH, A_gate, A_up
        q_us += tl.avg_us("glue")
        q_bytes = T * M * 3 + T * F * (2 * 8 + 2)
    q_gbs = q_bytes / (q_us / 1e6) / 1e9
    out = {
        "metric": "S3R-EC backward TOPS (quant+INT8 dX/dW) & quantizer GB/s, % of MI355X peak",
        "value": round(value, 2), "unit": "TOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic",
        "config": {"workload": b.name, "tokens": T, "d_model": M, "d_ff": F, "rows_per_example": S,
                   "mode": args.mode, "step_scale": "per-tensor", "g_dtype": "bf16", "streams": sched["streams"],
                   "dw_pair": bool(args.dw_pair), "fuse_glue": bool(args.fuse_glue),
                   "stages": "down (quantize, dX=dH, dW), SwiGLU glue with the gate/up amax, gate and up "
                             "(quantize with that amax, dX added), the gate and up dW as one launch (dw_pair); "
                             "with 2 streams each dW launch (its U GEMVs and GEMM) runs on a second stream "
                             "after the dX before it"},
        "ms_per_step_by_streams": {str(k): round(v, 4) for k, v in ms_by_streams.items()},
        "ms_per_step_single_stream": round(ms_single, 4),
        "kernel_fields": "kernels_us, gemm_tops, roofline and quantizer come from a single-stream pass of the "
                         "same step, HIP events on the launch stream around each kernel",
        "frac_of_int8_peak": round(value / PEAK_INT8_TOPS, 4),
        "quantizer": {"us": round(q_us, 2), "GB_s": round(q_gbs, 1), "frac_of_hbm_peak": round(q_gbs / PEAK_HBM_GBS, 4),
                      "algorithmic_bytes": q_bytes, "calls": 3,
                      "note": ("gate and up: the fused call (glue amax pass, then glue and both code passes: "
                               "dH, A_gate, A_up read twice, G never written)" if args.fuse_glue else
                               "gate and up calls take their per-tensor amax from the glue pass (one read of G)")},
        "kernels_us": {**{f"quantize_{n}": round(tl.avg_us(f"quantize_{n}"), 2) for n in st},
                       **{f"gemm_{k}": round(v, 2) for k, v in gemm_us.items()},
                       "glue": round(tl.avg_us("glue"), 2), "step_events": round(tl.avg_us("step"), 2)},
        "kernels_us_min_median_max": tl.spread(),
        "gemm_tops": {k: round(gemm_gop[k] / (v / 1e6) / 1e3, 1) for k, v in gemm_us.items()},
        "roofline": _roofline(gemm_us, b.name, gemm_gop),
    }
    if (mode, ec) == MODES["s3r-ec-two-way"]:
        # the correction's cost, measured in this run: the same step without it, and dX-only
        ov = {"s3r_ec_two_way_ms": round(ms_step, 4)}
        for label, (m2, e2) in (("s3r", MODES["s3r"]), ("s3r_ec_dx_only", MODES["s3r-ec-dx-only"])):
            log(f"EC overhead: timing the {label} step")
            ov[f"{label}_ms"] = round(step_ms(m2, e2), 4)
        ov["two_way_over_s3r"] = round(ov["s3r_ec_two_way_ms"] / ov["s3r_ms"], 4)
        ov["dx_only_over_s3r"] = round(ov["s3r_ec_dx_only_ms"] / ov["s3r_ms"], 4)
        ov["note"] = ("whole-step times of the same block in the same stream schedule, in this run; ratio 1.0 = "
                      "free correction")
        out["ec_overhead"] = ov
    log("timing the step with the other dW launch arrangement")
    other = round(step_ms(mode, ec, pair=not args.dw_pair), 4)
    out["dw_pair_ablation"] = {"paired_ms": round(ms_step, 4) if args.dw_pair else other,
                               "separate_ms": other if args.dw_pair else round(ms_step, 4),
                               "note": "whole-step times in this run: the gate and up dW as one launch or two"}
    log("timing the step with the glue computed inside the gate and up quantizers" if not args.fuse_glue
        else "timing the step with the glue as its own pass")
    other = round(step_ms(mode, ec, fused=not args.fuse_glue), 4)
    out["glue_fusion_ablation"] = {
        "glue_pass_ms": other if args.fuse_glue else round(ms_step, 4),
        "glue_in_quantizers_ms": round(ms_step, 4) if args.fuse_glue else other,
        "note": "whole-step times in this run: G_gate and G_up written by the glue pass and read by the "
                "quantizers, or never written (s3r_swiglu_quantize: one glue pass for the maxima, the glue again "
                "in the code pass)"}
    del st, step, dv, dH, dX, Gg, Gu, dW
    out["bf16_context"] = bf16_gemm_context(torch, dev, T, M, F, sum(gemm_us.values()), ms_step, args.steps)
    if args.cpu_rows != 0:
        rows = S if args.cpu_rows < 0 else max(S, min(args.cpu_rows, T) // S * S)
        log(f"CPU oracle baseline on the first {rows} tokens")
        out["cpu_baseline"] = block_cpu_baseline(inp, b, mode, ec, rows)
    return out


def bf16_gemm_context(torch, dev, T, M, F, int8_gemm_us, int8_step_ms, steps):
    """Context for the pages' speedups over BF16 (not the method): the FFN block's six backward products as
    plain bf16 GEMMs (torch.matmul, hipBLASLt), fp32 accumulation and bf16 outputs, on random operands of the
    same shapes, timed like the step."""
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    r = lambda *s_: torch.randn(*s_, device=dev, generator=g).to(torch.bfloat16)
    Gd, Gg, Gu = r(T, M), r(T, F), r(T, F)
    Wd, Wg, Wu = r(M, F), r(F, M), r(F, M)
    H, X = r(T, F), r(T, M)
    Gdt, Ggt, Gut = Gd.t().contiguous(), Gg.t().contiguous(), Gu.t().contiguous()

    def six():
        torch.matmul(Gd, Wd)        # dH = G_down . W_down      [T x F]
        torch.matmul(Gdt, H)        # dW_down = G_down^T . H    [M x F]
        torch.matmul(Gg, Wg)        # dX (gate)                 [T x M]
        torch.matmul(Ggt, X)        # dW_gate                   [F x M]
        torch.matmul(Gu, Wu)        # dX (up)
        torch.matmul(Gut, X)        # dW_up

    for _ in range(3):
        six()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        six()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    return {"bf16_six_gemms_ms": round(ms, 4), "int8_six_gemms_ms": round(int8_gemm_us / 1e3, 4),
            "gemm_speedup_over_bf16": round(ms / (int8_gemm_us / 1e3), 3),
            "step_speedup_over_bf16_gemms_alone": round(ms / int8_step_ms, 3),
            "note": "torch.matmul bf16 on the same shapes; context for the pages' ratios, not a measured baseline "
                    "of the method"}


def moe_cpu_baseline(inp, m, mode, ec, experts):
    """Time the CPU oracle's grouped backward on a bounded sample: a few whole experts."""
    from oracle import moe
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    fx, fws, xs = moe.forward_operands(inp["X"], inp["W"], "bf16", inp["offsets"])
    t0 = time.perf_counter()
    moe.grouped_backward(inp, mode=mode, ec=ec, fx=fx, fws=fws, xs=xs, experts=experts)
    dt = time.perf_counter() - t0
    rows = int(sum(inp["counts"][e] for e in experts))
    ops = 2 * 2.0 * rows * m.d_model * m.d_ff
    return {"value": ops / dt / 1e12, "unit": "TOP/s", "cores": int(blas_threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{len(experts)} experts ({rows} of {m.rows} rows), full d_model={m.d_model} and d_ff={m.d_ff}: "
                      f"numpy quantizer (1 thread) + dX + dW with float64 BLAS integer GEMMs ({blas_threads} BLAS "
                      f"threads); forward-operand prep untimed"}


def run_moe(args, dev, torch, inputs, s3r):
    """The MoE expert path: 64 experts' down projections over 32768 expert-sorted rows."""
    mode, ec = MODES[args.mode]
    m = inputs.MOE[args.workload]
    R, E, M, F = m.rows, m.experts, m.d_model, m.d_ff
    log(f"workload {m.name}: rows={R} experts={E} d_model={M} d_ff={F} mode={args.mode}; drawing inputs")
    inp = inputs.make_moe_inputs(m)
    off = torch.from_numpy(inp["offsets"]).to(dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    log("forward-operand prep (untimed)")
    X = _to_dev(torch, dev, inp["X"], "bf16")
    xdesc = s3r.qdesc(R, F, 1, s3r.RTNE, s3r.EC_NONE, s3r.PER_TOKEN)
    Xq = s3r.q_buffer(R, F, dev)
    sx = torch.empty(R, device=dev)
    xs = torch.empty(E, F, dtype=torch.int32, device=dev)
    ws = torch.zeros(s3r.s3r_grouped_workspace(xdesc, E, F), dtype=torch.uint8, device=dev)
    s3r.s3r_grouped_quantize(xdesc, off, X, None, None, Xq, sx, xs, flags=flags, ws=ws)
    W = _to_dev(torch, dev, inp["W"].reshape(E * M, F), "bf16")
    ld = (F + 15) // 16 * 16
    wbuf = torch.empty(E * M, ld, dtype=torch.int8, device=dev)
    wdesc = s3r.qdesc(E * M, F, M, s3r.RTNE, s3r.EC_NONE, s3r.PER_TOKEN)
    sw = torch.empty(E * M, device=dev)
    rW = torch.empty(E, F, dtype=torch.int32, device=dev)
    wws = torch.zeros(max(s3r.s3r_quantize_workspace(wdesc), 1), dtype=torch.uint8, device=dev)
    s3r.s3r_quantize(wdesc, W, None, None, wbuf[:, :F], sw, rW, ws=wws)
    Wq = wbuf.view(E, M, ld)[:, :, :F]
    del X, W, wws
    G = _to_dev(torch, dev, inp["G"], "bf16")
    desc = s3r.qdesc(R, M, 1, mode, ec, s3r.PER_TENSOR, layer_id=0, seed=0)
    Q = s3r.q_buffer(R, M, dev)
    delta = torch.empty(E, device=dev)
    st = (torch.empty(R, device=dev), torch.empty(E, M, device=dev), torch.empty(E, device=dev)) if ec \
        else (None, None, None)
    ws = torch.zeros(s3r.s3r_grouped_workspace(desc, E, F), dtype=torch.uint8, device=dev)
    ws2 = torch.zeros_like(ws)
    dX = torch.empty(R, F, device=dev)
    dW = torch.empty(E, M, F, device=dev)
    tl = Timeline(torch, ["step", "quantize", "dx", "dw"], args.steps)

    def make_step(streams):
        # streams 2: the grouped dW (its U GEMV and GEMM) on a second stream after the quantize call,
        # beside the dX (its v GEMV and GEMM), with its own workspace
        s2 = torch.cuda.Stream() if streams >= 2 else None

        def step(ev):
            if ev:
                ev["step"][0].record()
                ev["quantize"][0].record()
            s3r.s3r_grouped_quantize(desc, off, G, sx, sw.view(E, M), Q, delta, None, *st, flags, ws)
            if ev:
                ev["quantize"][1].record()
            if s2 is not None:
                e = torch.cuda.Event()
                e.record()
                s2.wait_event(e)
            if ev:
                s3r.s3r_time_next_gemm(*ev["dx"])
            s3r.s3r_grouped_backward_dx(desc, off, Q, delta, Wq, sx, rW, *st, dX, flags, ws)
            if ev:
                s3r.s3r_time_next_gemm(*ev["dw"])
            s3r.s3r_grouped_backward_dw(desc, off, Q, delta, Xq, sw.view(E, M), xs, *st, dW, flags,
                                        ws if s2 is None else ws2, stream=None if s2 is None else s2.cuda_stream)
            if s2 is not None:
                e = torch.cuda.Event()
                e.record(s2)
                torch.cuda.current_stream().wait_event(e)
            if ev:
                ev["step"][1].record()
        return step

    ms_single = _timed_steps(torch, make_step(1), tl, args.steps, args.warmup)
    assert int(flags.item()) == 0
    ms_step, used, ms_two = _pick_streams(torch, args, make_step, ms_single)
    t_q, t_gx, t_gw = tl.avg_us("quantize"), tl.avg_us("dx"), tl.avg_us("dw")
    gop = 2.0 * R * M * F / 1e9                     # each of the two grouped GEMMs
    value = 2 * gop / (ms_step / 1e3) / 1e3
    q_bytes = R * M * 3
    counts = inp["counts"]
    out = {
        "metric": "S3R-EC backward TOPS (quant+INT8 dX/dW) & quantizer GB/s, % of MI355X peak",
        "value": round(value, 2), "unit": "TOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic",
        "config": {"workload": m.name, "rows": R, "experts": E, "top_k": m.top_k, "tokens": m.tokens,
                   "d_model": M, "d_ff": F, "expert_rows_max": int(counts.max()), "expert_rows_min": int(counts.min()),
                   "mode": args.mode, "step_scale": "per-tensor per expert", "g_dtype": "bf16",
                   "streams": used, "ms_per_step_two_streams": ms_two,
                   "stages": "experts' down projections: grouped quantize, grouped dX, grouped dW (with 2 streams "
                             "the grouped dW runs on a second stream after the quantize call)"},
        "ms_per_step_single_stream": round(ms_single, 4),
        "kernel_fields": "kernels_us, gemm_tops, roofline and quantizer come from a single-stream pass",
        "frac_of_int8_peak": round(value / PEAK_INT8_TOPS, 4),
        "quantizer": {"us": round(t_q, 2), "GB_s": round(q_bytes / (t_q / 1e6) / 1e9, 1),
                      "frac_of_hbm_peak": round(q_bytes / (t_q / 1e6) / 1e9 / PEAK_HBM_GBS, 4),
                      "algorithmic_bytes": q_bytes},
        "kernels_us": {"quantize_call": round(t_q, 2), "gemm_dx": round(t_gx, 2), "gemm_dw": round(t_gw, 2),
                       "step_events": round(tl.avg_us("step"), 2)},
        "kernels_us_min_median_max": tl.spread(),
        "gemm_tops": {"dx": round(gop / (t_gx / 1e6) / 1e3, 1), "dw": round(gop / (t_gw / 1e6) / 1e3, 1)},
        "roofline": _roofline({"dx": t_gx, "dw": t_gw}, m.name, gop),
    }
    if args.cpu_rows != 0:
        experts = list(range(E))
        log("CPU oracle baseline on every expert (the whole workload)")
        out["cpu_baseline"] = moe_cpu_baseline(inp, m, mode, ec, experts)
    return out


def run_linear(args, dev, torch, inputs, s3r):
    mode, ec = MODES[args.mode]
    w = inputs.WORKLOADS[args.workload]
    T, D, K, S = w.tokens, w.d_out, w.d_in, w.rows_per_example
    log(f"workload {w.name}: T={T} D={D} d_in={K} S={S} mode={args.mode}; drawing inputs")
    inp = inputs.make_linear_inputs(w)
    G, X, W = (_to_dev(torch, dev, inp[k], inp["dtype"]) for k in ("G", "X", "W"))
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
    ws_b2 = torch.zeros_like(ws_b)
    dX = torch.empty(T, K, dtype=torch.float32, device=dev)
    dW = torch.empty(D, K, dtype=torch.float32, device=dev)
    tl = Timeline(torch, ["step", "quantize", "dx", "dw"], args.steps)

    def make_step(streams):
        # streams 2: dW (its U GEMV and GEMM) on a second stream after the quantize call, beside the dX
        s2 = torch.cuda.Stream() if streams >= 2 else None

        def step(ev):
            if ev:
                ev["step"][0].record()
                ev["quantize"][0].record()
            s3r.s3r_quantize(desc, G, fx.delta, fw.delta, Q, delta, None, e_r, e_c, e_m, flags, ws_q)
            if ev:
                ev["quantize"][1].record()
            if s2 is not None:
                e = torch.cuda.Event()
                e.record()
                s2.wait_event(e)
            if ev:
                s3r.s3r_time_next_gemm(*ev["dx"])
            s3r.s3r_backward_dx(desc, Q, delta, fw.Q, fx.delta, fw.code_colsum[0], e_r, e_c, e_m, dX, ws_b)
            if ev:
                s3r.s3r_time_next_gemm(*ev["dw"])
            s3r.s3r_backward_dw(desc, Q, delta, fx.Q, fw.delta, fx.code_colsum, e_r, e_c, e_m, dW,
                                ws_b if s2 is None else ws_b2, stream=None if s2 is None else s2.cuda_stream)
            if s2 is not None:
                e = torch.cuda.Event()
                e.record(s2)
                torch.cuda.current_stream().wait_event(e)
            if ev:
                ev["step"][1].record()
        return step

    ms_single = _timed_steps(torch, make_step(1), tl, args.steps, args.warmup)
    assert int(flags.item()) == 0
    ms_step, used, ms_two = _pick_streams(torch, args, make_step, ms_single)
    t_q, t_gx, t_gw = tl.avg_us("quantize"), tl.avg_us("dx"), tl.avg_us("dw")
    gop = 2.0 * T * D * K / 1e9
    value = 2 * gop / (ms_step / 1e3) / 1e3
    q_bytes = T * D * (2 if inp["dtype"] == "bf16" else 4) + T * D
    q_gbs = q_bytes / (t_q / 1e6) / 1e9
    out = {
        "metric": "S3R-EC backward TOPS (quant+INT8 dX/dW) & quantizer GB/s, % of MI355X peak",
        "value": round(value, 2), "unit": "TOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "i8", "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "d_in": K, "d_out": D, "rows_per_example": S,
                   "mode": args.mode, "step_scale": "per-tensor", "g_dtype": inp["dtype"],
                   "streams": used, "ms_per_step_two_streams": ms_two},
        "ms_per_step_single_stream": round(ms_single, 4),
        "kernel_fields": "kernels_us, gemm_tops, roofline and quantizer come from a single-stream pass",
        "frac_of_int8_peak": round(value / PEAK_INT8_TOPS, 4),
        "quantizer": {"us": round(t_q, 2), "GB_s": round(q_gbs, 1),
                      "frac_of_hbm_peak": round(q_gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": q_bytes},
        "kernels_us": {"quantize_call": round(t_q, 2), "gemm_dx": round(t_gx, 2), "gemm_dw": round(t_gw, 2),
                       "step_events": round(tl.avg_us("step"), 2)},
        "kernels_us_min_median_max": tl.spread(),
        "gemm_tops": {"dx": round(gop / (t_gx / 1e6) / 1e3, 1), "dw": round(gop / (t_gw / 1e6) / 1e3, 1)},
        "roofline": _roofline({"dx": t_gx, "dw": t_gw}, w.name, gop),
    }
    if args.cpu_rows != 0:
        # a bounded sample: the whole of a small workload, else its first example (at least 1024
        # tokens); three timed runs below 2^38 multiply-adds, and for a small layer one thread as well
        small = T * D * K <= (1 << 28)
        rows = (T if small else min(T, max(1024, S))) if args.cpu_rows < 0 else min(args.cpu_rows, T)
        if rows >= S:
            rows = rows // S * S
        log(f"CPU oracle baseline on the first {rows} tokens")
        out["cpu_baseline"] = cpu_baseline(inp, w, mode, ec, rows, repeats=3 if T * D * K <= (1 << 38) else 1,
                                           single_thread=small)
    return out


def mx_cpu_baseline(inp, w, mode, ec, rows):
    """Time the CPU oracle's MXFP4 backward on the first ``rows`` tokens (whole examples)."""
    import numpy as np
    from oracle import mx
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    from stochastic_rounding_quantization_amd import inputs
    S = w.rows_per_example
    f32 = lambda a: inputs.bf16_bits_to_f32(a) if inp["dtype"] == "bf16" else np.asarray(a, np.float32)
    G, X, W = f32(inp["G"][:rows]), f32(inp["X"][:rows]), f32(inp["W"])
    t0 = time.perf_counter()
    r = mx.backward(G, X, W, mode=mode, ec=ec, rows_per_example=S, seed=0)
    dt = time.perf_counter() - t0
    assert np.isfinite(r["dX"]).all() and np.isfinite(r["dW"]).all()
    ops = 2 * 2.0 * rows * w.d_out * w.d_in
    return {"value": ops / dt / 1e12, "unit": "TOP/s", "cores": int(blas_threads), "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"first {rows} tokens ({rows // S} example(s) of {S}), D={w.d_out}, d_in={w.d_in}: numpy "
                      f"MXFP4 quantization of G (both blockings), X and W, statistics, and dX + dW as float64 "
                      f"BLAS products of the dequantized operands ({blas_threads} BLAS threads), all timed"}


def run_mx(args, dev, torch, inputs, s3r):
    mode, ec = MODES[args.mode]
    if mode == 3:
        raise SystemExit("the MXFP4 path has no per-example threshold mode")
    w = inputs.MX_WORKLOADS[args.workload]
    T, D, K, S = w.tokens, w.d_out, w.d_in, w.rows_per_example
    log(f"workload {w.name}: T={T} D={D} d_in={K} S={S} mode={args.mode}; drawing inputs")
    inp = inputs.make_linear_inputs(w)
    G, X, W = (_to_dev(torch, dev, inp[k], inp["dtype"]) for k in ("G", "X", "W"))
    log("forward-operand prep (untimed): RTNE MXFP4 of W and X, transposed, with column sums")
    Wt, Wts, rW = s3r.mx_operand(W, rows_per_example=D)
    Xt, Xts, xs = s3r.mx_operand(X, rows_per_example=S)
    del X, W
    desc = s3r.qdesc(T, D, S, mode, ec, s3r.PER_TENSOR, layer_id=0, seed=0)
    B = T // S
    u8 = dict(dtype=torch.uint8, device=dev)
    Qh, Qhs = s3r.mx_codes(T, D, dev), torch.empty(D // 128, 4 * T, **u8)
    Qt, Qts = s3r.mx_codes(D, T, dev), torch.empty(T // 128, 4 * D, **u8)
    f32 = dict(dtype=torch.float32, device=dev)
    st_h = (torch.empty(T, **f32), torch.empty(B, D, **f32), torch.empty(B, **f32)) if ec else (None,) * 3
    st_t = (torch.empty(T, **f32), torch.empty(B, D, **f32), torch.empty(B, **f32)) if ec else (None,) * 3
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.zeros(max(s3r.s3r_mx_workspace(desc, K), 1), **u8)
    dX = torch.empty(T, K, **f32)
    dW = torch.empty(D, K, **f32)
    tl = Timeline(torch, ["step", "quantize", "dx", "dw"], args.steps)

    def step(ev):
        if ev:
            ev["step"][0].record()
            ev["quantize"][0].record()
        s3r.s3r_mx_quantize(desc, G, Qh, Qhs, Qt, Qts, *st_h, *st_t, flags, ws)
        if ev:
            ev["quantize"][1].record()
            s3r.s3r_time_next_gemm(*ev["dx"])
        s3r.s3r_mx_backward_dx(desc, Qh, Qhs, Wt, Wts, rW[0], *st_h, dX, ws)
        if ev:
            s3r.s3r_time_next_gemm(*ev["dw"])
        s3r.s3r_mx_backward_dw(desc, Qt, Qts, Xt, Xts, xs, *st_t, dW, ws)
        if ev:
            ev["step"][1].record()

    ms_step = _timed_steps(torch, step, tl, args.steps, args.warmup)
    assert int(flags.item()) == 0
    t_q, t_gx, t_gw = tl.avg_us("quantize"), tl.avg_us("dx"), tl.avg_us("dw")
    gop = 2.0 * T * D * K / 1e9
    value = 2 * gop / (ms_step / 1e3) / 1e3
    el = 2 if inp["dtype"] == "bf16" else 4
    q_bytes = int(T * D * (el + 2 * (0.5 + 1 / 32)))
    q_gbs = q_bytes / (t_q / 1e6) / 1e9
    key = "dx" if t_gx >= t_gw else "dw"
    achieved = gop / (max(t_gx, t_gw) / 1e6) / 1e3
    out = {
        "metric": "S3R-EC backward TOPS (quant+INT8 dX/dW) & quantizer GB/s, % of MI355X peak",
        "value": round(value, 2), "unit": "TOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4", "data": "synthetic",
        "config": {"workload": w.name, "tokens": T, "d_in": K, "d_out": D, "rows_per_example": S,
                   "mode": args.mode, "format": "MXFP4 (E2M1, E8M0 per 32 along the contraction)",
                   "g_dtype": inp["dtype"]},
        "frac_of_fp4_peak": round(value / PEAK_FP4_TFLOPS, 4),
        "quantizer": {"us": round(t_q, 2), "GB_s": round(q_gbs, 1),
                      "frac_of_hbm_peak": round(q_gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": q_bytes},
        "kernels_us": {"quantize_call": round(t_q, 2), "gemm_dx": round(t_gx, 2), "gemm_dw": round(t_gw, 2),
                       "step_events": round(tl.avg_us("step"), 2)},
        "kernels_us_min_median_max": tl.spread(),
        "gemm_tops": {"dx": round(gop / (t_gx / 1e6) / 1e3, 1), "dw": round(gop / (t_gw / 1e6) / 1e3, 1)},
        "roofline": {"kernel": f"mx gemm {key}", "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP4_TFLOPS, 4),
                     "traffic": None, "algorithmic": f"2*M*N*K = {gop:.1f} GFLOP per launch (FP4 products)"},
    }
    if args.cpu_rows != 0:
        rows = S if args.cpu_rows < 0 else max(S, min(args.cpu_rows, T) // S * S)
        log(f"CPU oracle baseline on the first {rows} tokens")
        out["cpu_baseline"] = mx_cpu_baseline(inp, w, mode, ec, rows)
    return out


if __name__ == "__main__":
    main()
