"""Benchmark: fused linear + cross-entropy forward+backward on one MI355X.

One step = one flce_forward_backward call over the whole batch (label pre-pass, label logits, and per
BT chunk: row references, logits GEMM + epilogue, row statistics, per-row factors, grad_hidden GEMM,
grad_W GEMM; then the loss), with
inputs and outputs resident in HBM. Prints one JSON line.

Workload (default): the Llama-3-8B LM head, BT=8192, H=4096, V=128256, bf16, RMS-normalised hidden,
W ~ N(0, 0.02^2), Zipf(1.1) labels with 5% ignore_index, mean reduction, seed 0 (synthetic).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FLCE fwd+bwd tokens/sec at H=4096,V=128256 bf16; % bf16 MFMA peak; peak bytes"
METRIC_FWD = "FLCE forward-only tokens/sec (flce_forward, no gradients); % bf16 MFMA peak; peak bytes"
METRIC_RECOMPUTE = ("FLCE fwd+bwd tokens/sec, recompute mode (flce_forward_backward_recompute); "
                    "% bf16 MFMA peak of the 6*BT*H*V algorithmic flops; peak bytes")
PEAK_BF16 = 2.5e15          # dense bf16 MFMA, MI355X published
PEAK_HBM = 8.0e12


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_head")
    ap.add_argument("--chunk", type=int, default=0, help="chunk_rows_max (0 = library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows of the oracle's bounded sample (0 = about 15 TFLOP of float64 work, at most the "
                         "whole call)")
    ap.add_argument("--profile-only", action="store_true", help="warmup + steps, no extras (for rocprofv3)")
    ap.add_argument("--mode", choices=("fwd_bwd", "forward", "recompute", "hipblaslt"), default="fwd_bwd",
                    help="fwd_bwd: the fused forward + backward (default); forward: flce_forward only; "
                         "recompute: flce_forward_backward_recompute (logits formed twice, one vocabulary "
                         "slice kept); hipblaslt: torch.matmul (hipBLASLt) alone at the three GEMM shapes of "
                         "one chunk, for comparison (never part of the library)")
    ap.add_argument("--vslice", type=int, default=0, help="vocabulary slice of the recompute mode (0 = 8192)")
    ap.add_argument("--sequences", type=int, default=0,
                    help="B > 0: lay the BT rows out as B sequences of BT/B + 1 positions, hidden [B, T+1, H], "
                         "with the next-token label shift done by the library (the *_rows entry points)")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for the FETCH_SIZE/WRITE_SIZE scale)")
    ap.add_argument("--no-peak-calib", action="store_true",
                    help="skip the measured ceilings (MFMA-only loop, device copy) reported beside the result")
    return ap.parse_args()


def measured_peaks(dev) -> dict:
    """The ceilings this GPU sustains, from libflce_calib.so (after the timed steps): an MFMA-only loop
    (1024 blocks of 8 waves, 8 independent v_mfma_f32_32x32x16_bf16 chains per wave on random bf16
    operands that change from one MFMA to the next, 65536 iterations; best of 3 launches) and a 1 GiB
    device-to-device copy (best of 5). The loop's exactness on +-2^-10 operands (twice the iterations,
    exactly twice the output) and the copy's destination are checked."""
    import ctypes

    from linear_cross_entropy_07_amd import build_lib

    L = ctypes.CDLL(build_lib.CALIB_LIB)
    d = ctypes.c_double
    L.flce_calib_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint,
                                       ctypes.c_int, ctypes.POINTER(d), ctypes.POINTER(d), ctypes.POINTER(d)]
    L.flce_calib_copy.argtypes = [ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.POINTER(d),
                                  ctypes.POINTER(d), ctypes.POINTER(ctypes.c_int)]

    def mfma(blocks, iters, reps, full_random):
        tf, ms, chk = d(), d(), d()
        rc = L.flce_calib_mfma_bf16(dev.index, blocks, iters, reps, 1, full_random, ctypes.byref(tf),
                                    ctypes.byref(ms), ctypes.byref(chk))
        if rc != 0:
            raise SystemExit(f"MFMA calibration failed (rc {rc})")
        return tf.value, ms.value, chk.value

    blocks, iters = 1024, 65536  # ~80 ms per launch: the sustained rate (shorter runs read ~2% higher)
    a, b = mfma(1, 64, 1, 0)[2], mfma(1, 128, 1, 0)[2]
    if a == 0.0 or b != 2.0 * a:
        raise SystemExit(f"MFMA calibration not exact ({a}, {b})")
    tf, ms, _ = mfma(blocks, iters, 3, 1)
    gbs, cms, ok = d(), d(), ctypes.c_int()
    rc = L.flce_calib_copy(dev.index, 1 << 30, 5, ctypes.byref(gbs), ctypes.byref(cms), ctypes.byref(ok))
    if rc != 0 or ok.value != 1:
        raise SystemExit(f"copy calibration failed (rc {rc}, ok {ok.value})")
    return {"mfma_bf16_tflops": round(tf, 1), "mfma_loop_ms": round(ms, 3),
            "copy_gbs": round(gbs.value, 1), "copy_ms": round(cms.value, 3),
            "how": f"MFMA-only loop: {blocks} blocks x 8 waves x {iters} iterations x 8 chains of "
                   "v_mfma_f32_32x32x16_bf16 on random bf16 operands changing per MFMA, best of 3; copy: "
                   "1 GiB device to device, (read + write) / time, best of 5"}


def kernel_source_hash() -> str:
    p = os.path.join(ROOT, "linear_cross_entropy_07_amd", "csrc", "flce_kernels.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str, launches_bytes_key: str = "bytes_per_launch"):
    """HBM bytes per launch measured by rocprofv3 counters for this exact kernel source and workload,
    else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}_{kernel}.json")
    try:
        d = json.load(open(p))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != kernel_source_hash() or d.get("workload") != workload:
        return None
    return d.get(launches_bytes_key)


def cpu_rows_for(BT: int, H: int, V: int, forward_only: bool, rows: int = 0) -> int:
    """Rows of the oracle's bounded sample: about 15 TFLOP of float64 work (10-20 s on the host's
    cores), a multiple of 256, at most the whole call."""
    if rows > 0:
        return min(rows, BT)
    per_row = (2.0 if forward_only else 6.0) * H * V
    return max(1, min(BT, int(15e12 / per_row) // 256 * 256))


def cpu_baseline(w, X, W, y, rows: int, forward_only: bool = False, BT: int | None = None):
    """The oracle as it stands, timed on the first `rows` rows of the same workload (a bounded sample).
    Its BLAS runs on as many threads as the process may use: the cores it is pinned to, capped by
    OMP_NUM_THREADS when that is set (the host's share of cores); `cores` is that thread count."""
    import oracle

    affinity = len(os.sched_getaffinity(0))
    threads = affinity
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = max(1, min(threads, int(os.environ["OMP_NUM_THREADS"])))
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info()
                                 if i.get("user_api") == "blas"})) or blas
        limiter = threadpool_limits(limits=threads, user_api="blas")
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
                           or [threads])
    except Exception:  # pragma: no cover
        limiter, blas_threads = None, threads
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:  # pragma: no cover
        pass
    Xs, ys = X[:rows], y[:rows]
    t0 = time.perf_counter()
    if forward_only:
        oracle.flce_forward(Xs, W, ys, -100, w.softcap, w.reduction)
    else:
        oracle.flce_blocked(Xs, W, ys, -100, w.softcap, w.reduction, block_rows=1024)
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister()
    BT = w.BT if BT is None else BT
    return {"value": rows / dt, "unit": "tokens/s", "cores": blas_threads, "affinity_cores": affinity,
            "kind": "oracle", "cpu": cpu, "blas": blas,
            "sample": f"first {rows} of {BT} rows of {w.name} (full H={w.H}, V={w.V}), fp64 numpy/OpenBLAS "
                      f"{'forward' if forward_only else 'forward+backward (flce_blocked, 1024-row blocks)'} "
                      f"incl. widening inputs to fp64; {dt:.2f} s on {blas_threads} BLAS threads"}


def library_gemms(args, dev, w):
    """torch.matmul (hipBLASLt, bf16 in and out, fp32 accumulation) at the three GEMM shapes of one
    chunk of the workload, for comparison with the library's kernels under the same counters. The
    logits product is W [V,H] . X^T [H,C] (the library's orientation, M = V); grad_hidden dZ [C,V] .
    W [V,H]; grad_W dZ^T [V,C] . X [C,H]. Operands are random and contiguous (transposes made once,
    outside the timed region)."""
    import torch

    from linear_cross_entropy_07_amd import flce

    eng = flce.FLCE(dev, chunk_rows_max=args.chunk)
    H, V = w.H, w.V
    n, C = eng.chunk_plan(w.BT, H, V)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    Wm = (torch.randn(V, H, device=dev, generator=g) * 0.02).to(torch.bfloat16)
    X = torch.randn(C, H, device=dev, generator=g).to(torch.bfloat16)
    dZ = (torch.randn(C, V, device=dev, generator=g) * 1e-4).to(torch.bfloat16)
    Xt, dZt = X.t().contiguous(), dZ.t().contiguous()
    prods = {"fwd": lambda: torch.matmul(Wm, Xt), "dx": lambda: torch.matmul(dZ, Wm),
             "dw": lambda: torch.matmul(dZt, X)}
    flops = 2.0 * C * H * V
    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)  # the reference dispatch: reads and writes exactly 1 GiB
        torch.cuda.synchronize(dev)
        del src, dst
    out = {}
    for name, f in prods.items():
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize(dev)
        if args.profile_only:
            for _ in range(args.steps):
                f()
            torch.cuda.synchronize(dev)
            continue
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in ev:
            a.record()
            f()
            b.record()
        torch.cuda.synchronize(dev)
        ms = statistics.median(a.elapsed_time(b) for a, b in ev)
        out[name] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1), "frac": round(flops / ms * 1e3 / PEAK_BF16, 4)}
    if args.profile_only:
        print(f"# profiled {args.steps} calls of each product", file=sys.stderr, flush=True)
        return
    print(json.dumps({"metric": "torch.matmul (hipBLASLt) at the FLCE GEMM shapes of one chunk (comparison only)",
                      "config": {"workload": w.name, "chunk_rows": C, "H": H, "V": V}, "steps": args.steps,
                      "products": out}), flush=True)


def ragged_sweep(args, dev):
    """The ragged B*T protocol: one handle, one code object, calls whose B*T changes every time.
    Hidden rows and labels of every call are the first B*T rows of one draw of the largest call."""
    import torch

    from linear_cross_entropy_07_amd import flce, inputs

    w = inputs.WORKLOADS["ragged"]
    bts = inputs.ragged_bt_list(0, 20)
    print(f"# generating the ragged sweep: {len(bts)} calls, B*T {min(bts)}..{max(bts)}", file=sys.stderr,
          flush=True)
    X, W, y = inputs.make_ragged_call(max(bts), seed=100)
    eng = flce.FLCE(dev, chunk_rows_max=args.chunk)
    H, V = w.H, w.V
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    gh = torch.empty_like(Xd)
    gw = torch.empty((V, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(eng.workspace_size(bt, H, V) for bt in bts), dtype=torch.uint8, device=dev)
    reps = max(1, args.steps // 10)

    def call(bt):
        eng.forward_backward(Xd[:bt], Wd, yd[:bt], -100, 0.0, "mean", out=(loss, gh[:bt], gw), workspace=ws)

    for bt in bts[: args.warmup]:
        call(bt)
    stream = torch.cuda.current_stream(dev)
    per_call = []
    eng.profile_begin(max_launches=64 * reps * len(bts))
    for bt in bts:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(stream)
            call(bt)
            b.record(stream)
        torch.cuda.synchronize(dev)
        per_call.append((bt, statistics.median(a.elapsed_time(b) for a, b in ev)))
    kt = eng.profile_end(stream)
    tot_bt = sum(bt for bt, _ in per_call)
    tot_ms = sum(ms for _, ms in per_call)
    flops = sum(6.0 * bt * H * V for bt, _ in per_call)
    # roofline of the slowest GEMM kernel over the sweep: its flops (2*BT*H*V per call) / its time
    gemm = {k: kt[k][0] / reps for k in ("fwd", "dx", "dw")}
    dom = max(gemm, key=gemm.get)
    achieved = (flops / 3.0) / (gemm[dom] * 1e-3)
    out = {
        "metric": "FLCE fwd+bwd tokens/sec over the ragged B*T sweep (sum of B*T / sum of call times)",
        "value": round(tot_bt / (tot_ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": reps,
        "warmup": args.warmup, "ms_per_step": round(tot_ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "ragged", "H": H, "V": V, "calls": len(bts), "BT": [bt for bt, _ in per_call],
                   "parallelism": "single GPU", "layout": "plain [BT, H]"},
        "mfma_frac_sweep": round(flops / (tot_ms * 1e-3) / PEAK_BF16, 4),
        "ms_per_call": [round(ms, 3) for _, ms in per_call],
        "kernels_ms_per_sweep": {k: round(v[0] / reps, 3) for k, v in kt.items() if v[1]},
        "roofline": {"kernel": f"k_{dom}", "bound": "mfma", "achieved": round(achieved / 1e12, 2),
                     "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        rows = cpu_rows_for(max(bts), H, V, False, args.cpu_rows)
        print(f"# timing the oracle on {rows} rows", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, X, W, y, rows, BT=max(bts))
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only (the library is single-GPU); run with --gpus 1"}), flush=True)
        sys.exit(2)

    import torch

    from linear_cross_entropy_07_amd import build_lib, flce, inputs

    build_lib.ensure_built()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = inputs.WORKLOADS[args.workload]
    if w.name == "ragged":
        return ragged_sweep(args, dev)
    if args.mode == "hipblaslt":
        return library_gemms(args, dev, w)
    print(f"# generating {w.name}: BT={w.BT} H={w.H} V={w.V} {w.dtype}", file=sys.stderr, flush=True)
    BT, H, V = w.BT, w.H, w.V
    nseq = args.sequences
    if nseq:
        if BT % nseq:
            raise SystemExit("--sequences must divide BT")
        X, W, y = inputs.make_inputs(w, seed=0, BT=BT + nseq)  # B sequences of BT/B + 1 positions
    else:
        X, W, y = inputs.make_inputs(w, seed=0)
    eng = flce.FLCE(dev, chunk_rows_max=args.chunk)
    n_chunks, chunk_rows = eng.chunk_plan(BT, H, V, X.dtype)
    if args.mode == "recompute":  # one pass over all rows, vocabulary slices outermost
        n_chunks, chunk_rows = 1, -(-BT // 256) * 256

    base_alloc = torch.cuda.memory_allocated(dev)
    Xd, Wd, yd = X.to(dev), W.to(dev), y.to(dev)
    if nseq:
        Xd, yd = Xd.reshape(nseq, BT // nseq + 1, H), yd.reshape(nseq, BT // nseq + 1)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    gh = torch.empty_like(Xd)
    gw = torch.empty((V, H), dtype=torch.float32, device=dev)
    fwd_only = args.mode == "forward"
    recompute = args.mode == "recompute"
    if recompute and nseq:
        raise SystemExit("--mode recompute takes the plain [BT, H] layout")
    if recompute:
        ws_bytes = flce.recompute_workspace_size(BT, H, V, Xd.dtype, args.vslice, eng.handle)
    elif fwd_only:
        del gh, gw
        ws_bytes = flce.forward_workspace_size(BT, H, V, Xd.dtype, eng.handle)
    elif nseq:
        ws_bytes = flce.workspace_size_rows(eng._seq_rows(Xd, Wd, yd, True, gh)[0], H, V, Xd.dtype, eng.handle)
    else:
        ws_bytes = eng.workspace_size(BT, H, V, Xd.dtype)
    torch.cuda.synchronize(dev)
    io_alloc = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step():
        if fwd_only and nseq:
            loss.copy_(eng.forward_seq(Xd, Wd, yd, True, -100, w.softcap, w.reduction, workspace=ws))
        elif fwd_only:
            loss.copy_(eng.forward(Xd, Wd, yd, -100, w.softcap, w.reduction, workspace=ws))
        elif recompute:
            eng.forward_backward_recompute(Xd, Wd, yd, -100, w.softcap, w.reduction, args.vslice,
                                           out=(loss, gh, gw), workspace=ws)
        elif nseq:
            eng.forward_backward_seq(Xd, Wd, yd, True, -100, w.softcap, w.reduction, 1.0, gh, gw, loss=loss,
                                     workspace=ws)
        else:
            eng.forward_backward(Xd, Wd, yd, -100, w.softcap, w.reduction, out=(loss, gh, gw), workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    print(f"# warmup done, loss {float(loss):.6f}", file=sys.stderr, flush=True)
    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)  # the reference dispatch: reads and writes exactly 1 GiB
        torch.cuda.synchronize(dev)
        del src, dst
    if args.profile_only:
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize(dev)
        print(f"# profiled {args.steps} steps", file=sys.stderr, flush=True)
        return

    stream = torch.cuda.current_stream(dev)

    def timed_pass():
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize(dev)
        t0 = time.perf_counter()
        for i in range(args.steps):
            ev[i][0].record(stream)
            step()
            ev[i][1].record(stream)
        torch.cuda.synchronize(dev)
        return sorted(a.elapsed_time(b) for a, b in ev), time.perf_counter() - t0

    # the headline: K steps with nothing but one event pair per step around them
    per, wall = timed_pass()
    ms_med = statistics.median(per)
    # the per-kernel breakdown: K more steps, each launch bracketed by a HIP event pair that the
    # library records on the launch stream (events created before the timed region)
    vs_eff = min(-(-(args.vslice or 8192) // 256) * 256, -(-V // 256) * 256)
    launches_per_step = 8 + n_chunks * (8 + (4 * -(-V // vs_eff) if recompute else 8))
    capacity = launches_per_step * args.steps
    eng.profile_begin(max_launches=capacity)
    per_prof, _ = timed_pass()
    kt = eng.profile_end(stream)
    # every launch was recorded: the events did not run out, and the last launch of every step (the
    # loss) is there
    if sum(c for _, c in kt.values()) >= capacity or kt["finalize"][1] < args.steps:
        raise SystemExit("kernel profile incomplete: more launches per step than events")
    peak_extra = torch.cuda.max_memory_allocated(dev) - io_alloc
    print(f"# kernel ms/launch: " + ", ".join(f"{k} {v[0] / max(v[1], 1):.3f}x{v[1] // args.steps}"
                                            for k, v in kt.items() if v[1]), file=sys.stderr, flush=True)
    gemm = {k: kt[k] for k in (("fwd",) if fwd_only else ("fwd", "dx", "dw"))}
    dom = max(gemm, key=lambda k: gemm[k][0])
    dom_ms = gemm[dom][0] / gemm[dom][1]
    # each product does 2*BT*H*V flop per step (the logits product twice in the recompute mode),
    # over one launch per chunk (per chunk and vocabulary slice in the recompute mode); the last
    # chunk may be shorter, so the flops are averaged over the launches actually made
    step_gemm_flops = {"fwd": 2.0 * BT * H * V * (2 if recompute else 1), "dx": 2.0 * BT * H * V,
                       "dw": 2.0 * BT * H * V}
    flops_per_launch = step_gemm_flops[dom] * args.steps / gemm[dom][1]
    achieved = flops_per_launch / (dom_ms * 1e-3)

    tokens_per_s = BT / (ms_med * 1e-3)
    step_flops = (2.0 if fwd_only else 6.0) * BT * H * V
    out = {
        "metric": METRIC_FWD if fwd_only else (METRIC_RECOMPUTE if recompute else METRIC),
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_med, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": w.name, "BT": BT, "H": H, "V": V, "softcap": w.softcap,
                   "labels": w.labels, "ignore_frac": w.ignore_frac, "reduction": w.reduction,
                   "chunk_rows": chunk_rows, "n_chunks": n_chunks, "parallelism": "single GPU",
                   "layout": (f"{nseq} sequences [B, T+1, H] = {list(Xd.shape)}, labels shifted by the library"
                              if nseq else "plain [BT, H]")},
        "mfma_frac_step": round(step_flops / (ms_med * 1e-3) / PEAK_BF16, 4),
        "ms_p10_p90": [round(per[len(per) // 10], 4), round(per[(9 * len(per)) // 10], 4)],
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 4),
        "ms_per_step_with_kernel_events": round(statistics.median(per_prof), 4),
        "peak_bytes": {"workspace": ws_bytes, "handle_device_bytes": 256, "max_allocated_beyond_io": int(peak_extra),
                       "inputs_outputs": int(io_alloc - base_alloc),
                       "full_bf16_logits_not_allocated": BT * V * 2},
        "mode": args.mode,
        "kernels_ms_per_launch": {k: round(v[0] / v[1], 4) for k, v in kt.items() if v[1]},
        "roofline": {"kernel": f"k_{dom}", "bound": "mfma", "achieved": round(achieved / 1e12, 2),
                     "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16, 4),
                     "traffic": (traffic_from_profiles("fwd_noq" if fwd_only else dom, w.name)
                                 if not (nseq or recompute) else None),
                     "flops_per_launch": flops_per_launch},
    }
    if not args.no_peak_calib:
        mp = measured_peaks(dev)
        out["measured_peaks"] = mp
        out["mfma_frac_step_of_measured"] = round(step_flops / (ms_med * 1e-3) / (mp["mfma_bf16_tflops"] * 1e12), 4)
        out["roofline"]["frac_of_measured_peak"] = round(achieved / (mp["mfma_bf16_tflops"] * 1e12), 4)
    if not args.no_cpu_baseline:
        rows = cpu_rows_for(BT, H, V, fwd_only, args.cpu_rows)
        Xc, yc = X, y
        if nseq:  # the call's rows: every position but the last of each sequence, scored against the next label
            Xc = X.reshape(nseq, BT // nseq + 1, H)[:, :-1].reshape(BT, H)
            yc = y.reshape(nseq, BT // nseq + 1)[:, 1:].reshape(BT)
        print(f"# timing the oracle on {rows} rows", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, Xc, W, yc, rows, fwd_only)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
