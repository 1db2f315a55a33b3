"""Benchmark: fused linear cross-entropy forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one flce_fused_fwd_bwd call (forward logits + online LSE, loss,
recomputed softmax, dW and dX; grad_output = 1) over the whole synthetic batch,
with inputs already resident in HBM.  Prints one JSON line with tokens/s, the
fraction of the bf16 MFMA peak (against 8 N D V, and against 8 n_valid D V
since rows with ignore_index are skipped), peak allocated HBM bytes, the
roofline of the forward kernel (timed live with HIP events on the library's
stream) and the fp64 CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FLCE fwd+bwd tokens/sec, % bf16 MFMA peak, peak HBM bytes at N=65536 D=4096 V=128256"
PEAK_BF16_TFLOPS = 2516.6     # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_F32_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
# The pages' own figure for this shape (B200, CuTe-DSL FLCE, bf16, BT = 65 536,
# V = 128 256, H = 4096): 194 ms per fwd+bwd, i.e. 337.8 k tokens/s.
PAGES_TOKENS_PER_S = 65536 / 0.194
_CSRC = os.path.join(ROOT, "linear_cross_entropy_bf16_amd", "csrc")
# committed counter summaries, and the sources each measured kernel is built from
TRAFFIC = {
    "k_fwd": (os.path.join(ROOT, "profiles", "k_fwd_llama3_8b_batch8_traffic.json"),
              ("flce_gemm.hpp", "flce_kernels.hpp", "flce_launch.hpp", "flce_fwd.hip", "flce.hip")),
    "k_ce_fused": (os.path.join(ROOT, "profiles", "k_ce_fused_ce_logits_llama3_8b_seq_traffic.json"),
                   ("flce_kernels.hpp", "flce_ce.hpp", "flce_launch.hpp", "flce_ce.hip", "flce.hip")),
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def timed_steps(run, steps: int, stream):
    """Runs ``steps`` calls of ``run`` on ``stream`` between K + 1 events, one
    before each step and one after the last, and returns the mean over the
    whole timed region with the median and the fastest single step (ms)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(steps):
        run()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    mid = steps // 2
    p50 = per[mid] if steps % 2 else 0.5 * (per[mid - 1] + per[mid])
    return ev[0].elapsed_time(ev[steps]) / steps, p50, per[0]


def kernel_source_hash(kernel: str = "k_fwd") -> str:
    h = hashlib.sha256()
    for name in TRAFFIC[kernel][1]:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str = "k_fwd"):
    """Per-launch HBM bytes of ``kernel`` from the committed counter summary,
    or None when it is missing, for another workload, or stale (taken on other
    kernel sources)."""
    try:
        with open(TRAFFIC[kernel][0]) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("workload") != workload or t.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


def blas_threads() -> int:
    """Threads the BLAS behind numpy will use (what the oracle's products run on)."""
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        return max((i.get("num_threads") or 1) for i in info) if info else 1
    except Exception:  # pragma: no cover - threadpoolctl missing
        return os.cpu_count() or 1


def one_thread_rate(fn, rows: int):
    """tokens/s of fn() over `rows` rows with the BLAS held to one thread, or
    None where the thread count cannot be limited."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover - threadpoolctl missing
        return None
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        fn()
        dt = time.perf_counter() - t0
    return {"value": round(rows / dt, 3), "rows": rows, "seconds": round(dt, 2)}


def cpu_baseline(wl, inp, max_rows: int):
    """The fp64 oracle as it stands on a bounded row sample of the workload
    (full D and V, dW included), on all the threads its BLAS uses, and on a
    sixteenth of the sample with one thread.  Its cost is linear in the rows
    at fixed D and V, so tokens/s carries over to the whole batch."""
    import numpy as np
    from oracle import flce_oracle as O
    threads = blas_threads()
    rows = np.arange(min(max_rows, wl.n))
    o = O.LossOptions(wl.ignore_index, wl.label_smoothing, wl.lse_square_scale, wl.softcap,
                      wl.reduction)
    t0 = time.perf_counter()
    O.forward_backward(inp["x"][rows], inp["w"], inp["bias"], inp["targets"][rows], o)
    dt = time.perf_counter() - t0
    r1 = rows[:max(16, len(rows) // 16)]
    one = one_thread_rate(lambda: O.forward_backward(inp["x"][r1], inp["w"], inp["bias"],
                                                     inp["targets"][r1], o), len(r1))
    return {"value": round(len(rows) / dt, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "nproc": os.cpu_count(), "one_thread": one,
            "sample": f"first {len(rows)} of {wl.n} rows of {wl.name} (full D={wl.d}, V={wl.v}, dW "
                      f"included), fp64 numpy, {dt:.1f} s; tokens/s is per row, so it holds for "
                      f"the whole batch (cost linear in N)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_batch8")
    ap.add_argument("--vocab-slice", type=int, default=0)
    ap.add_argument("--token-chunk", type=int, default=0,
                    help="backward over this many packed rows at a time (0 = whole batch)")
    ap.add_argument("--dw-bf16", action="store_true", help="dW in bf16 instead of fp32")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the extra measurements (stored-logits schedule, token sweep, one-sequence "
                         "share, library GEMM floor)")
    ap.add_argument("--stored-logits", action="store_true",
                    help="three-contraction schedule: logits kept per token chunk, not recomputed "
                         "(6 N D V FLOPs; the MFMA fractions are then quoted against 6 N D V)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="rows of the workload the CPU oracle baseline runs on (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES bytes (the reference "
                         "for scaling FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        a = torch.ones(args.copy_calibration // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": a.numel() * 4}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the step is "
              f"data-parallel over tokens: each GPU would run this measurement on its share of "
              f"the batch, followed by an all-reduce of dW).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from linear_cross_entropy_bf16_amd import api, workloads as W

    if args.workload in W.CE_WORKLOADS:
        return bench_ce(args, W.CE_WORKLOADS[args.workload])
    wl = W.WORKLOADS[args.workload]
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a ROCm GPU")
    dev = torch.device("cuda:0")
    log(f"generating {wl}")
    inp = W.generate(wl)

    def put(a):
        t = torch.from_numpy(a)
        if wl.dtype == "bf16":
            t = t.view(torch.bfloat16)
        return t.to(dev)

    x, w = put(inp["x"]), put(inp["w"])
    b = put(inp["bias"]) if inp["bias"] is not None else None
    t = torch.from_numpy(inp["targets"]).to(dev)
    opts = dict(ignore_index=wl.ignore_index, label_smoothing=wl.label_smoothing,
                lse_square_scale=wl.lse_square_scale, softcap=wl.softcap, reduction=wl.reduction,
                vocab_slice=args.vocab_slice, token_chunk=args.token_chunk, dw_bf16=args.dw_bf16)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base_alloc = torch.cuda.memory_allocated(dev)

    # Outputs and workspace are allocated once and reused by every step.
    nbytes = api.workspace_bytes(wl.n, wl.d, wl.v, x.dtype, True, stored_logits=args.stored_logits,
                                 **opts)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = (torch.empty(1, dtype=torch.float32, device=dev),
           torch.empty(wl.n, dtype=torch.float32, device=dev),
           torch.empty((wl.n, wl.d), dtype=x.dtype, device=dev),
           torch.empty((wl.v, wl.d), dtype=torch.bfloat16 if args.dw_bf16 else torch.float32,
                       device=dev),
           torch.empty(wl.v, dtype=torch.float32, device=dev) if b is not None else None)

    def step():
        return api.fused_fwd_bwd(x, w, t, b, workspace=ws, out=out, stored_logits=args.stored_logits,
                                 **opts)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # one step captured in a HIP graph (the library only launches kernels
        # on the caller's stream), replayed as the timed step
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
        run()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms, ms_p50, ms_min = timed_steps(run, args.steps, stream)
    wall = time.perf_counter() - wall0
    peak_bytes = torch.cuda.max_memory_allocated(dev)
    loss = float(out[0].item())
    log(f"{ms:.3f} ms/step (wall {1e3 * wall / args.steps:.3f}), loss {loss:.6f}")

    # Forward kernel alone: flce_forward is k_fwd plus three launches that
    # each touch O(N) floats, timed on the same stream.
    fwd_ws = torch.empty(api.workspace_bytes(wl.n, wl.d, wl.v, x.dtype, False, **opts),
                         dtype=torch.uint8, device=dev)
    from linear_cross_entropy_bf16_amd import _lib
    p = api.make_params(wl.n, wl.d, wl.v, x.dtype, wl.ignore_index, wl.label_smoothing,
                        wl.lse_square_scale, wl.softcap, wl.reduction, args.vocab_slice)
    fwd_loss = torch.empty(1, dtype=torch.float32, device=dev)
    fwd_lse = torch.empty(wl.n, dtype=torch.float32, device=dev)

    def fwd():
        st = _lib.forward(p, x.data_ptr(), w.data_ptr(), None if b is None else b.data_ptr(),
                          t.data_ptr(), fwd_loss.data_ptr(), fwd_lse.data_ptr(), None,
                          fwd_ws.data_ptr(), fwd_ws.numel(), stream.cuda_stream)
        if st != 0:
            raise _lib.FLCEError(st, "flce_forward")

    fwd()
    torch.cuda.synchronize()
    reps = max(3, args.steps)
    ev0.record(stream)
    for _ in range(reps):
        fwd()
    ev1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = ev0.elapsed_time(ev1) / reps
    del fwd_ws

    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    # Rows whose target is ignore_index are dropped before the GEMMs, so the
    # MFMA work actually needed is 8 n_valid D V; the step fraction is also
    # quoted against 8 N D V as the benchmark defines it.
    n_valid = int((inp["targets"] != wl.ignore_index).sum())
    # FLOPs actually done per step: 8 N D V with recompute, 6 N D V when the
    # logits are kept (never credited with the recompute)
    contractions = 6.0 if args.stored_logits else 8.0
    step_tflops = contractions / 8.0 * wl.flops_fwd_bwd / (ms * 1e-3) / 1e12
    step_tflops_valid = contractions * n_valid * wl.d * wl.v / (ms * 1e-3) / 1e12
    fwd_flops = 2.0 * n_valid * wl.d * wl.v
    fwd_tflops = fwd_flops / (fwd_ms * 1e-3) / 1e12
    tokens_per_s = wl.n / (ms * 1e-3)
    traffic = measured_traffic(wl.name)

    variants = None
    if not args.no_variants and not args.stored_logits and wl.dtype == "bf16":
        variants = {"stored_logits": bench_stored_variant(args, wl, x, w, t, b, opts, dev, n_valid)}
        if wl.name == "llama3_8b_batch8" and not args.graph:
            variants["token_sweep"] = bench_token_sweep(args, wl, x, w, t, dev)
            variants["llama3_8b_seq"] = bench_workload_variant(args, W.WORKLOADS["llama3_8b_seq"], dev)
            variants["library_gemm_floor"] = bench_library_floor(args, wl, x, w, t, dev, ms)

    cpu = None
    if args.cpu_rows > 0:
        log(f"cpu oracle baseline on {args.cpu_rows} rows")
        cpu = cpu_baseline(wl, inp, args.cpu_rows)

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "ms_p50": round(ms_p50, 3),
        "ms_min": round(ms_min, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tokens_per_s / PAGES_TOKENS_PER_S, 4) if wl.name == "llama3_8b_batch8" else None,
        "baseline_note": "pages' CuTe-DSL FLCE on B200 at this shape, 194 ms per fwd+bwd (context, "
                         "other hardware)",
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "n": wl.n, "d": wl.d, "v": wl.v, "targets": wl.targets,
                   "ignore_frac": wl.ignore_frac, "reduction": wl.reduction, "bias": wl.bias,
                   "label_smoothing": wl.label_smoothing, "lse_square_scale": wl.lse_square_scale,
                   "softcap": wl.softcap, "vocab_slice": args.vocab_slice or "default",
                   "launch": "hip graph replay" if args.graph else "eager",
                   "token_chunk": args.token_chunk or ("8192 (default of the schedule)" if args.stored_logits else "whole batch"),
                   "dw_dtype": "bf16" if args.dw_bf16 else "fp32",
                   "schedule": "stored logits, 6NDV" if args.stored_logits else "recompute, 8NDV",
                   "parallelism": "single GPU"},
        "mfma_frac_step": round(step_tflops / peak, 4),
        "step_tflops": round(step_tflops, 1),
        "n_valid": n_valid,
        "mfma_frac_step_valid_rows": round(step_tflops_valid / peak, 4),
        "step_tflops_valid_rows": round(step_tflops_valid, 1),
        "peak_hbm_bytes": int(peak_bytes),
        "peak_hbm_bytes_above_inputs": int(peak_bytes - base_alloc),
        "workspace_bytes": int(nbytes),
        "loss": loss,
        "roofline": {
            "kernel": "k_fwd (forward logits GEMM + online-LSE epilogue, valid rows only)",
            "bound": "mfma",
            "achieved": round(fwd_tflops, 1),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(fwd_tflops / peak, 4),
            "traffic": traffic,
            "fwd_ms": round(fwd_ms, 3),
            "flops_per_launch": fwd_flops,
        },
        "cpu_baseline": cpu,
    }
    if variants:
        result["variants"] = variants
    print(json.dumps(result), flush=True)


def _time_fused(args, n, d, v, x, w, t, b, opts, dev, steps):
    """(mean, p50, min ms per fused step, peak bytes of the step's own
    buffers on top of the inputs, workspace bytes) of one configuration."""
    import torch
    from linear_cross_entropy_bf16_amd import api
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    nbytes = api.workspace_bytes(n, d, v, x.dtype, True, **opts)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = (torch.empty(1, dtype=torch.float32, device=dev), torch.empty(n, dtype=torch.float32, device=dev),
           torch.empty((n, d), dtype=x.dtype, device=dev), torch.empty((v, d), dtype=torch.float32, device=dev),
           torch.empty(v, dtype=torch.float32, device=dev) if b is not None else None)

    def step():
        api.fused_fwd_bwd(x, w, t, b, workspace=ws, out=out, **opts)

    for _ in range(max(1, min(args.warmup, 2))):
        step()
    ms, ms_p50, ms_min = timed_steps(step, steps, torch.cuda.current_stream(dev))
    extra = torch.cuda.max_memory_allocated(dev) - base
    loss = float(out[0].item())
    del ws, out
    return ms, ms_p50, ms_min, int(extra), int(nbytes), loss


def _fused_record(wl_name, n, d, v, n_valid, ms, ms_p50, ms_min, extra, nbytes, inputs, loss, steps):
    flops = 8.0 * n * d * v
    return {"workload": wl_name, "n": n, "d": d, "v": v, "steps": steps, "ms_per_step": round(ms, 3),
            "ms_p50": round(ms_p50, 3), "ms_min": round(ms_min, 3),
            "tokens_per_s": round(n / (ms * 1e-3), 1),
            "mfma_frac_8ndv": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "mfma_frac_8ndv_valid_rows": round(8.0 * n_valid * d * v / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "n_valid": int(n_valid), "peak_hbm_bytes": int(extra + inputs), "workspace_bytes": nbytes,
            "loss": loss}


def bench_token_sweep(args, wl, x, w, t, dev):
    """Tokens-per-step sweep at V = 128256, D = 4096 (the pages' BT sweep at
    this vocabulary): the fused step on the first N rows of the headline
    batch (same recipe, 10% ignored), N = 8192, 16384, 32768; the headline
    itself is N = 65536.  Reported beside the headline, never as it."""
    res = []
    ign = wl.ignore_index
    for n in (8192, 16384, 32768):
        steps = max(3, min(args.steps, 10))
        xs, ts = x[:n], t[:n]
        n_valid = int((ts != ign).sum().item())
        ms, p50, mn, extra, nbytes, loss = _time_fused(
            args, n, wl.d, wl.v, xs, w, ts, None,
            dict(ignore_index=ign, reduction=wl.reduction), dev, steps)
        inputs = xs.numel() * 2 + w.numel() * 2 + ts.numel() * 4
        log(f"token sweep N={n}: {ms:.3f} ms/step")
        res.append(_fused_record(f"first {n} rows of {wl.name}", n, wl.d, wl.v, n_valid, ms, p50, mn,
                                 extra, nbytes, inputs, loss, steps))
    return res


def bench_workload_variant(args, wl, dev):
    """Another workload's fused step (its own seeded inputs), reported beside
    the headline: one 8-way data-parallel share of the headline batch."""
    import torch
    from linear_cross_entropy_bf16_amd import workloads as W
    inp = W.generate(wl)
    x = torch.from_numpy(inp["x"]).view(torch.bfloat16).to(dev)
    w = torch.from_numpy(inp["w"]).view(torch.bfloat16).to(dev)
    t = torch.from_numpy(inp["targets"]).to(dev)
    n_valid = int((inp["targets"] != wl.ignore_index).sum())
    steps = max(3, min(args.steps, 10))
    ms, p50, mn, extra, nbytes, loss = _time_fused(
        args, wl.n, wl.d, wl.v, x, w, t, None, dict(ignore_index=wl.ignore_index, reduction=wl.reduction),
        dev, steps)
    log(f"{wl.name}: {ms:.3f} ms/step")
    inputs = x.numel() * 2 + w.numel() * 2 + t.numel() * 4
    rec = _fused_record(wl.name, wl.n, wl.d, wl.v, n_valid, ms, p50, mn, extra, nbytes, inputs, loss, steps)
    del x, w, t
    return rec


def bench_library_floor(args, wl, x, w, t, dev, fused_ms):
    """The same step's four contractions as plain library GEMMs (hipBLASLt
    through torch.matmul), no epilogues: logits of the valid rows per
    8192-wide vocabulary slice for the forward, then per slice the recomputed
    logits, dW of the slice (logits^T X) and dX += logits W.  Outputs in bf16
    (dW and the dX running sum included, so it moves fewer bytes than the
    fused step).  Timed on the same GPU right after the fused step, as the
    speed the vendor's GEMMs reach on the same 8 n_valid D V MFMA work under
    the same power limit; the ratio is the fused step over it."""
    import torch
    ign = wl.ignore_index
    xv = x[t != ign].contiguous()
    nv = xv.shape[0]
    width = 8192
    z = torch.empty((nv, width), dtype=x.dtype, device=dev)
    dw = torch.empty((wl.v, wl.d), dtype=x.dtype, device=dev)
    dx = torch.zeros((nv, wl.d), dtype=x.dtype, device=dev)
    slices = [(a, min(wl.v, a + width)) for a in range(0, wl.v, width)]

    def step():
        for a, b in slices:
            torch.matmul(xv, w[a:b].t(), out=z[:, :b - a])
        for a, b in slices:
            zs = z[:, :b - a]
            torch.matmul(xv, w[a:b].t(), out=zs)
            torch.matmul(zs.t(), xv, out=dw[a:b])
            dx.addmm_(zs, w[a:b])

    step()
    steps = max(3, min(args.steps, 5))
    ms, ms_p50, ms_min = timed_steps(step, steps, torch.cuda.current_stream(dev))
    log(f"library GEMM floor: {ms:.3f} ms/step (fused {fused_ms:.3f})")
    res = {"what": "hipBLASLt (torch.matmul) bf16 GEMMs of the same step on the valid rows: "
                   "forward logits and, per 8192-wide vocabulary slice, recomputed logits, "
                   "dW slice and dX running sum; no epilogues, bf16 outputs",
           "n_valid": int(nv), "steps": steps, "ms_per_step": round(ms, 3),
           "ms_p50": round(ms_p50, 3), "ms_min": round(ms_min, 3),
           "tflops_executed": round(8.0 * nv * wl.d * wl.v / (ms * 1e-3) / 1e12, 1),
           "fused_step_over_floor": round(fused_ms / ms, 4)}
    del xv, z, dw, dx
    return res


def bench_stored_variant(args, wl, x, w, t, b, opts, dev, n_valid):
    """The same workload through the three-contraction schedule (each token
    chunk's logits kept, not recomputed): reported beside the headline, never
    as it, with its own FLOP count (6 N D V) and peak memory."""
    import torch
    from linear_cross_entropy_bf16_amd import api
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    inputs = sum(a.numel() * a.element_size() for a in (x, w, t, b) if a is not None)
    nbytes = api.workspace_bytes(wl.n, wl.d, wl.v, x.dtype, True, stored_logits=True, **opts)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    out = (torch.empty(1, dtype=torch.float32, device=dev),
           torch.empty(wl.n, dtype=torch.float32, device=dev),
           torch.empty((wl.n, wl.d), dtype=x.dtype, device=dev),
           torch.empty((wl.v, wl.d), dtype=torch.bfloat16 if opts.get("dw_bf16") else torch.float32,
                       device=dev),
           torch.empty(wl.v, dtype=torch.float32, device=dev) if b is not None else None)

    def step():
        api.fused_fwd_bwd(x, w, t, b, workspace=ws, out=out, stored_logits=True, **opts)

    step()
    steps = max(3, args.steps // 2)
    stream = torch.cuda.current_stream(dev)
    ms, ms_p50, ms_min = timed_steps(step, steps, stream)
    peak = PEAK_BF16_TFLOPS
    tflops = 6.0 * wl.n * wl.d * wl.v / (ms * 1e-3) / 1e12
    tflops_valid = 6.0 * n_valid * wl.d * wl.v / (ms * 1e-3) / 1e12
    log(f"stored-logits schedule: {ms:.3f} ms/step")
    res = {"schedule": "stored logits (6 N D V: forward GEMM keeps each 8192-token chunk's logits, "
                       "no recompute)", "steps": steps, "ms_per_step": round(ms, 3),
           "ms_p50": round(ms_p50, 3), "ms_min": round(ms_min, 3),
           "tokens_per_s": round(wl.n / (ms * 1e-3), 1),
           "vs_baseline": round(wl.n / (ms * 1e-3) / PAGES_TOKENS_PER_S, 4)
           if wl.name == "llama3_8b_batch8" else None,
           "mfma_frac_6ndv": round(tflops / peak, 4), "mfma_frac_6ndv_valid_rows": round(tflops_valid / peak, 4),
           # this schedule's own peak: its buffers on top of the inputs
           "peak_hbm_bytes": int(torch.cuda.max_memory_allocated(dev) - base) + inputs,
           "workspace_bytes": int(nbytes), "loss": float(out[0].item())}
    del ws, out
    return res


def cpu_baseline_ce(wl, inp, max_rows: int):
    """The fp64 oracle on the first rows of a logits workload (full V)."""
    from oracle import flce_oracle as O
    threads = blas_threads()
    rows = min(max_rows, wl.n)
    o = O.LossOptions(wl.ignore_index, wl.label_smoothing, wl.lse_square_scale, wl.softcap,
                      wl.reduction)
    t0 = time.perf_counter()
    O.cross_entropy_on_logits(inp["logits"][:rows], inp["targets"][:rows], o)
    dt = time.perf_counter() - t0
    r1 = max(1, rows // 4)
    one = one_thread_rate(lambda: O.cross_entropy_on_logits(inp["logits"][:r1], inp["targets"][:r1], o), r1)
    return {"value": round(rows / dt, 3), "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "nproc": os.cpu_count(), "one_thread": one,
            "sample": f"first {rows} of {wl.n} rows of {wl.name} (full V={wl.v}, loss and "
                      f"dL/dlogits), fp64 numpy, {dt:.1f} s"}


def bench_ce(args, wl):
    """Cross-entropy on given logits: one step is one flce_ce_fused_fwd_bwd
    (row statistics, loss, dL/dlogits) over the whole synthetic batch, logits
    resident in HBM.  HBM-bound: the roofline is bytes moved against 8 TB/s."""
    import numpy as np
    import torch
    from linear_cross_entropy_bf16_amd import api, workloads as W
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a ROCm GPU")
    dev = torch.device("cuda:0")
    log(f"generating {wl}")
    inp = W.generate_logits(wl)
    r = torch.from_numpy(inp["logits"])
    if wl.dtype == "bf16":
        r = r.view(torch.bfloat16)
    r = r.to(dev)
    t = torch.from_numpy(inp["targets"]).to(dev)
    opts = dict(ignore_index=wl.ignore_index, label_smoothing=wl.label_smoothing,
                lse_square_scale=wl.lse_square_scale, softcap=wl.softcap, reduction=wl.reduction)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base_alloc = torch.cuda.memory_allocated(dev)
    elem = r.element_size()
    out = (torch.empty(1, dtype=torch.float32, device=dev),
           torch.empty(wl.n, dtype=torch.float32, device=dev), torch.empty_like(r))
    p = api._ce_params(r, **opts)
    from linear_cross_entropy_bf16_amd import _lib
    ws = torch.empty(_lib.ce_workspace_size(p), dtype=torch.uint8, device=dev)

    def step():
        return api.cross_entropy_fused_fwd_bwd(r, t, workspace=ws, out=out, **opts)

    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        torch.cuda.synchronize()
        ev0.record(stream)
        for _ in range(reps):
            fn()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps

    log(f"warmup {args.warmup}")
    for _ in range(max(1, args.warmup)):
        step()
    log(f"timing {args.steps} steps")
    wall0 = time.perf_counter()
    ms, ms_p50, ms_min = timed_steps(step, args.steps, stream)
    wall = time.perf_counter() - wall0
    peak_bytes = torch.cuda.max_memory_allocated(dev)
    loss = float(out[0].item())
    log(f"{ms:.3f} ms/step (wall {1e3 * wall / args.steps:.3f}), loss {loss:.6f}")

    # forward alone (flce_ce_forward): reads the valid rows once
    lse = torch.empty(wl.n, dtype=torch.float32, device=dev)
    loss1 = torch.empty(1, dtype=torch.float32, device=dev)

    def fwd():
        st = _lib.ce_forward(p, r.data_ptr(), t.data_ptr(), loss1.data_ptr(), lse.data_ptr(), None,
                             ws.data_ptr(), ws.numel(), stream.cuda_stream)
        if st != 0:
            raise _lib.FLCEError(st, "flce_ce_forward")

    fwd()
    fwd_ms = timed(fwd, max(3, args.steps))
    grad = out[2]

    def bwd():
        st = _lib.ce_backward(p, r.data_ptr(), t.data_ptr(), lse.data_ptr(), None, grad.data_ptr(),
                              ws.data_ptr(), ws.numel(), stream.cuda_stream)
        if st != 0:
            raise _lib.FLCEError(st, "flce_ce_backward")

    bwd()
    bwd_ms = timed(bwd, max(3, args.steps))

    # practical ceiling for context: a plain device copy (torch's copy kernel)
    # moving the same bytes, every row read and written once
    def copy():
        grad.copy_(r)

    copy()
    copy_ms = timed(copy, max(3, args.steps))

    n_valid = int((inp["targets"] != wl.ignore_index).sum())
    # must-move bytes: the valid rows read once, the gradient written once
    # (ignored rows are written as zeros, never read)
    step_bytes = (n_valid + wl.n) * wl.v * elem
    fwd_bytes = n_valid * wl.v * elem
    cpu = cpu_baseline_ce(wl, inp, args.cpu_rows // 8) if args.cpu_rows > 0 else None
    tokens_per_s = wl.n / (ms * 1e-3)
    achieved = step_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": f"CE on given logits fwd+bwd tokens/sec at N={wl.n} V={wl.v} ({wl.dtype} logits)",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_p50": round(ms_p50, 4),
        "ms_min": round(ms_min, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "n": wl.n, "v": wl.v, "targets": wl.targets,
                   "ignore_frac": wl.ignore_frac, "reduction": wl.reduction,
                   "label_smoothing": wl.label_smoothing, "lse_square_scale": wl.lse_square_scale,
                   "softcap": wl.softcap, "parallelism": "single GPU"},
        "n_valid": n_valid,
        "peak_hbm_bytes": int(peak_bytes),
        "peak_hbm_bytes_above_inputs": int(peak_bytes - base_alloc),
        "workspace_bytes": int(ws.numel()),
        "loss": loss,
        "roofline": {
            "kernel": "k_ce_fused (row statistics + dL/dlogits, one workgroup per row)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(wl.name, "k_ce_fused"),
            "bytes_per_launch": step_bytes,
            "timed": "whole flce_ce_fused_fwd_bwd call (k_prep, k_ce_fused, two O(N) reduction "
                     "launches)",
            "fwd_ms": round(fwd_ms, 4),
            "fwd_gbs": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9, 1),
            "separate_bwd_ms": round(bwd_ms, 4),
            "separate_bwd_gbs": round(step_bytes / (bwd_ms * 1e-3) / 1e9, 1),
            "copy_reference": {
                "what": "torch copy_ of all logits into the gradient buffer (every row read and "
                        "written once)",
                "ms": round(copy_ms, 4),
                "gbs": round(2 * wl.n * wl.v * elem / (copy_ms * 1e-3) / 1e9, 1),
            },
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
