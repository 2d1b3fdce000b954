"""Benchmark of the HARP apply path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--blk f32|bf16|i8]
    python bench.py --mode latency [--workload NAME] [--blk ...]
    python bench.py --mode materialize [--workload NAME]

A step is one pass of the hot path over one batch: for the default workload
(cayley4096_bf16: 16384 rows x 4096, bf16 rows, schedule (8,8,8,8), Cayley
blocks over Sylvester H8) one harp_apply launch over the whole batch, inputs
resident in HBM.  Block materialisation (theta -> blocks, on the GPU) is setup
and is not timed.  Prints one JSON line.  The default workload brings the
d = 5120 one (mixed5120_bf16: 32768 rows x 5120, (8,8,8,5,2)) along as the
"d5120" sub-record, measured the same way (--single drops it).

value = rows/s of the whole job (K steps timed back to back, bracketed by
device synchronisation).  The defaults (W = 50 warm-up steps, K = 200) let
the GPU reach its steady clocks before the timed steps: after 5 warm-up
steps the first few dozen launches run up to 10% slower.
roofline.achieved = algorithmic bytes per launch (rows * d * 2 bytes read +
rows * d * 2 bytes written) / the kernel's mean duration, measured with HIP
events recorded on the stream the kernel runs on.
kernel_ms_mean_flushed = the same launches (up to 100), each after a 1 GiB
write that evicts L2 and the MALL (--no-flush skips it).
cpu_baseline = the fp64 numpy oracle, single-threaded, on a bounded sample
(the whole batch when it finishes within 30 s), and its comparison with the
GPU's output on that sample (oracle_max_row_rel_l2).

--mode latency: the per-token (decode) regime, 1 to 64 rows per call, for
harp_apply_decode and, beside it, harp_apply.  For each row count:
microseconds per call of K back-to-back calls issued from Python (host launch
cost included), and of the same calls captured once in a HIP graph and
replayed (device time per call, launch gaps included); the replay's output is
checked against the eager calls and the two entry points against each other
(parity with the oracle is the tests' job; only the cpu_baseline leg runs the
oracle here).

--mode vjp: the reverse mode used to fit the parameters (dx and the block
gradients for one batch, then the parameter gradient), milliseconds per call,
with the HBM bytes its stage-wise design moves.

--mode materialize: microseconds per call of the block materialisation on the
device from fp64 parameters and from int8 parameter codes, and of the int8
quantisation of the parameters (setup work, not part of a step).
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "cayley4096_bf16"      # 16384 x 4096 bf16 rows, (8,8,8,8)
SECOND_WORKLOAD = "mixed5120_bf16"        # 32768 x 5120 bf16 rows, (8,8,8,5,2)
FP32_PEAK_TFLOPS = 157.3      # MI355X fp32 (vector and matrix)


def kernel_hash(kernel: str) -> str:
    from structured_rotations_amd.build import source_hash
    return source_hash(kernel)


def traffic_from_profile(workload: str, blk: str):
    """Counter-measured HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled
    by a copy-kernel calibration), if a profile taken with the current kernel
    sources is committed; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}_{blk}.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash(rec.get("kernel", "")):
        return None
    return rec.get("bytes_per_launch")


def row_rel_l2(a, b) -> np.ndarray:
    """Per-row relative l2 distance ||a - b|| / ||b|| of two row batches."""
    a = np.atleast_2d(np.asarray(a, dtype=np.float64))
    b = np.atleast_2d(np.asarray(b, dtype=np.float64))
    den = np.linalg.norm(b, axis=1)
    return np.linalg.norm(a - b, axis=1) / np.where(den > 0, den, 1.0)


def cpu_baseline(w: dict, blk: str, y_gpu, budget_s: float = 30.0) -> dict:
    """Time the oracle (as it stands) single-threaded on a bounded sample of
    the workload, and compare its output on that sample with the GPU's output
    of the timed step (max per-row relative l2; the bound is 4e-3 for bf16
    rows): the only place this script runs the oracle."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import harp_oracle as O
    kind = w["workload"].kind

    def gpu_rows(lo, hi):
        return y_gpu[lo:hi].float().cpu().numpy().astype(np.float64)

    with threadpool_limits(1):
        if kind == "two_sided":
            t0 = time.perf_counter()
            bu = O.stored_blocks(O.materialize_blocks(w["su"], w["d_out"], w["theta_u"], w["gauss_u"]), blk)
            bv = O.stored_blocks(O.materialize_blocks(w["schedule"], w["d"], w["theta_v"], w["gauss_v"]), blk)
            t1 = time.perf_counter()
            ref = O.rotate_weight(w["x"].astype(np.float64), w["su"], bu, w["signs_u"].astype(float), w["schedule"],
                                  bv, w["signs_v"].astype(float))
            dt = time.perf_counter() - t1
            err = float(O.row_rel_l2(gpu_rows(0, ref.shape[0]), ref).max())
            return {"value": 1.0 / dt, "unit": "weights/s", "cores": 1, "kind": "oracle",
                    "sample": f"the full {w['d_out']}x{w['d']} weight, fp64 numpy, 1 thread "
                              f"(block setup {t1 - t0:.1f}s not counted)",
                    "oracle_max_row_rel_l2": err, "host": host_info()}
        x = w["x"]
        n = x.shape[0]
        if kind == "rht":
            chunk = 1024
            signs = w["signs"].astype(float)

            def one(lo, hi):
                return O.rht_compose(x[lo:hi].astype(np.float64), signs)
        else:
            chunk = 2048
            blocks = O.stored_blocks(O.materialize_blocks(w["schedule"], w["d"], w["theta"], w["gauss"]), blk)

            def one(lo, hi):
                return O.apply(x[lo:hi].astype(np.float64), w["schedule"], blocks, w["signs"].astype(float))

        def run(limit_s, check):
            t0 = time.perf_counter()
            done, worst, t_check = 0, 0.0, 0.0
            while done < n and time.perf_counter() - t0 - t_check < limit_s:
                hi = min(n, done + chunk)
                ref = one(done, hi)
                if check:
                    tc = time.perf_counter()
                    worst = max(worst, float(O.row_rel_l2(gpu_rows(done, hi), ref).max()))
                    t_check += time.perf_counter() - tc
                done = hi
            return done, time.perf_counter() - t0 - t_check, worst

        done, dt, worst = run(budget_s, True)
    out = {"value": done / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
           "sample": f"first {done} of {n} rows, fp64 numpy, 1 thread",
           "oracle_max_row_rel_l2": worst, "host": host_info()}
    # the same oracle with numpy's default thread pool (context only)
    n = done
    done, dt, _ = run(budget_s, False)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    out["all_cores"] = {"value": round(done / dt, 1), "unit": "rows/s", "cores": threads,
                        "sample": f"first {done} rows, fp64 numpy, default thread pool"}
    return out


def host_info() -> dict:
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu": model, "affinity_cores": len(os.sched_getaffinity(0))}


LAT_ROWS = (1, 2, 4, 8, 16, 32, 64, 128)


def latency_main(args) -> int:
    """Decode regime: microseconds per call at 1-64 rows, for harp_apply_decode
    (the small-batch entry point) and, beside it, harp_apply."""
    import torch

    from structured_rotations_amd import api
    from structured_rotations_amd import workloads as W

    torch.cuda.set_device(0)
    name = args.workload
    w = W.make(name, rows=max(LAT_ROWS))
    d, sch, io = w["d"], w["schedule"], w["io"]
    if w["workload"].kind != "apply":
        print("--mode latency runs an apply workload", file=sys.stderr)
        return 2
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    th = torch.from_numpy(w["theta"]).cuda()
    gs = torch.from_numpy(w["gauss"]).cuda() if w["gauss"].size else None
    blocks, scales = api.harp_materialize_blocks(sch, d, th, gs, args.blk)
    sg = torch.from_numpy(w["signs"]).cuda()
    xall = torch.from_numpy(w["x"]).to(tdt).cuda()
    ws_bytes = api.harp_apply_decode_workspace(sch, d, args.blk, max(LAT_ROWS))
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
    steps = max(args.steps, 20)
    warm = max(args.warmup, 5)
    stream = torch.cuda.Stream()

    def measure(call, y):
        """(eager us/call, host us/call, graph-replay us/call, output of the replay)."""
        with torch.cuda.stream(stream):
            for _ in range(warm):
                call()
            stream.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            # no garbage-collector pass inside the timed calls (as timeit does):
            # one pass over the setup's objects cost up to 40 ms of host time
            gc.collect()
            gc.disable()
            t0 = time.perf_counter()
            e0.record(stream)
            for _ in range(steps):
                call()
            e1.record(stream)
            host_s = time.perf_counter() - t0
            gc.enable()
            stream.synchronize()
            eager_us = e0.elapsed_time(e1) * 1e3 / steps
            y_eager = y.clone()
            y.zero_()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for _ in range(steps):
                    call()
            stream.synchronize()
            g.replay()
            stream.synchronize()
            reps = 5
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
            stream.synchronize()
            graph_us = e0.elapsed_time(e1) * 1e3 / (reps * steps)
            del g
        if not torch.equal(y, y_eager):
            raise RuntimeError("graph replay output differs from the eager output")
        return eager_us, host_s * 1e6 / steps, graph_us

    table = []
    worst = 0.0
    for r in LAT_ROWS:
        x = xall[:r].contiguous()
        yd = torch.empty_like(x)
        ya = torch.empty_like(x)
        dec = measure(lambda: api.harp_apply_decode(sch, d, blocks, scales, sg, x, yd, workspace=ws,
                                                    stream=stream), yd)
        app = measure(lambda: api.harp_apply(sch, d, blocks, scales, sg, x, ya, stream=stream), ya)
        # the two entry points compute the same transform (parity with the
        # oracle is the tests' job): their outputs agree to rounding
        worst = max(worst, float(row_rel_l2(yd.float().cpu().numpy(), ya.float().cpu().numpy()).max()))
        table.append({"rows": r,
                      "decode_us_graph": round(dec[2], 3), "decode_us_eager": round(dec[0], 3),
                      "decode_us_host": round(dec[1], 3),
                      "apply_us_graph": round(app[2], 3), "apply_us_eager": round(app[0], 3)})
    cbytes = sum(d * b for b in sch) * {"f32": 4, "bf16": 2, "i8": 1}[args.blk]
    line = {
        "metric": "HARP apply decode latency, microseconds per call (graph replay), rows=1",
        "value": table[0]["decode_us_graph"],
        "unit": "us/call",
        "n_gpus": 1, "steps": steps, "warmup": warm,
        "higher_is_better": False,
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded rows and parameters of the named workload, first 1-128 rows)",
        "config": {"workload": name, "d": d, "schedule": list(sch), "io": io, "blocks": args.blk,
                   "kind": "apply-latency", "parallelism": "single GPU"},
        "coefficient_bytes_per_call": cbytes,
        "rows_table": table,
        "decode_vs_apply_max_row_rel_l2": worst,
    }
    print(json.dumps(line), flush=True)
    return 0


def vjp_main(args) -> int:
    """Reverse mode over one batch: harp_apply_vjp (dx + dB) and harp_theta_vjp."""
    import torch

    from structured_rotations_amd import api
    from structured_rotations_amd import workloads as W

    torch.cuda.set_device(0)
    name = args.workload
    w = W.make(name)
    if w["workload"].kind != "apply":
        print("--mode vjp runs an apply workload", file=sys.stderr)
        return 2
    d, sch, io = w["d"], w["schedule"], w["io"]
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    eb = 2 if io == "bf16" else 4
    x = torch.from_numpy(w["x"]).to(tdt).cuda()
    rows = x.shape[0]
    dy = torch.from_numpy(np.random.default_rng(5).standard_normal((rows, d)).astype(np.float32)).to(tdt).cuda()
    dx = torch.empty_like(x)
    th = torch.from_numpy(w["theta"]).cuda()
    gs = torch.from_numpy(w["gauss"]).cuda() if w["gauss"].size else None
    blocks, scales = api.harp_materialize_blocks(sch, d, th, gs, args.blk)
    sg = torch.from_numpy(w["signs"]).cuda()
    nblk = api.harp_block_count(sch, d)
    db = torch.empty(nblk, dtype=torch.float32, device="cuda")
    dt = torch.empty_like(th)
    ws = torch.empty(api.harp_apply_vjp_workspace(sch, d, rows), dtype=torch.uint8, device="cuda")
    steps = max(args.steps, 3)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms_vjp = timed(lambda: api.harp_apply_vjp(sch, d, blocks, scales, sg, x, dy, dx, dblocks=db, workspace=ws))
    ms_theta = timed(lambda: api.harp_theta_vjp(sch, d, th, gs, db, dt))
    m = len(sch)
    rd = rows * d
    # fp32 block-gradient partial sums in the workspace: one slot per backward workgroup
    nslot = (ws.numel() - 4 * rd * ((m - 1) + (2 if m > 1 else 0))) // (4 * nblk)
    # the library fuses the last two stages into one backward launch for
    # these endings (and the forward then stops one stage earlier)
    pair = m >= 2 and (sch[-2], sch[-1]) in ((8, 8), (5, 2), (3, 3))
    nf = m - 2 if pair else m - 1                     # forward launches
    fwd = (rd * (eb + 4) + (nf - 1) * rd * 8) if nf > 0 else 0
    if m == 1:
        bwd = rd * 3 * eb
    elif pair and m == 2:
        bwd = rd * 3 * eb                             # x, dy -> dx
    else:
        # last launch(es): the pair reads x_{m-2} and dy, writes g_{m-2}; a
        # single last stage reads x_{m-1} and dy, writes g_{m-1}
        bwd = rd * (4 + eb + 4)
        mid = (m - 3) if pair else (m - 2)            # fp32 stage launches in between
        bwd += mid * rd * 12 + rd * (4 + eb + eb)     # ... and the first stage (x, dx in the I/O type)
    red = nslot * nblk * 4 * 2 + nblk * 4
    moved = fwd + bwd + red
    # dx = M^T dy is the inverse transform of dy for orthogonal blocks: the
    # reverse mode's dx agrees with harp_apply_inverse to rounding (parity
    # with the oracle is the tests' job)
    dx_inv = api.harp_apply_inverse(sch, d, blocks, scales, sg, dy)
    torch.cuda.synchronize()
    par = float(row_rel_l2(dx.float().cpu().numpy(), dx_inv.float().cpu().numpy()).max())
    line = {
        "metric": "HARP reverse mode (dx + block gradients) over one batch, ms per call",
        "value": round(ms_vjp, 4),
        "unit": "ms/call",
        "n_gpus": 1, "steps": steps, "warmup": 2,
        "higher_is_better": False,
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded rows and parameters of the named workload, seeded normal upstream gradient)",
        "config": {"workload": name, "rows": rows, "d": d, "schedule": list(sch), "io": io, "blocks": args.blk,
                   "kind": "vjp", "parallelism": "single GPU"},
        "hbm_bytes_moved_by_design": moved,
        "achieved_GBps_on_design_bytes": round(moved / (ms_vjp * 1e-3) / 1e9, 1),
        "io_bytes_x_dy_dx": 3 * rd * eb,
        "ms_theta_vjp": round(ms_theta, 4),
        "partial_slots": int(nslot),
        "dx_vs_inverse_max_row_rel_l2": par,
    }
    print(json.dumps(line), flush=True)
    return 0


def materialize_main(args) -> int:
    """Block materialisation and int8 parameter quantisation, microseconds per call."""
    import torch

    from structured_rotations_amd import api
    from structured_rotations_amd import workloads as W

    torch.cuda.set_device(0)
    name = args.workload
    w = W.make(name, rows=1)
    if w["workload"].kind == "two_sided":
        sides = [("u", w["su"], w["d_out"], w["theta_u"], w["gauss_u"]),
                 ("v", w["schedule"], w["d"], w["theta_v"], w["gauss_v"])]
    elif w["workload"].kind == "apply":
        sides = [("", w["schedule"], w["d"], w["theta"], w["gauss"])]
    else:
        print("--mode materialize needs a workload with learnable blocks", file=sys.stderr)
        return 2
    steps = max(args.steps, 10)
    out = []
    for side, sch, d, theta, gauss in sides:
        th = torch.from_numpy(theta).cuda()
        gs = torch.from_numpy(gauss).cuda() if np.size(gauss) else None
        codes, tsc = api.harp_quantize_theta(sch, d, th)
        blk_out = torch.empty(api.harp_block_count(sch, d), dtype=torch.float32, device="cuda")

        def timed(fn):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            return round(e0.elapsed_time(e1) * 1e3 / steps, 3)

        t_q = timed(lambda: api.harp_quantize_theta(sch, d, th, codes, tsc))
        t_f = timed(lambda: api.harp_materialize_blocks(sch, d, th, gs, "f32", blk_out))
        t_8 = timed(lambda: api.harp_materialize_blocks_q8(sch, d, codes, tsc, gs, "f32", blk_out))
        torch.cuda.synchronize()
        # how far int8 parameters move the blocks (context; parity is the tests' job)
        b_f, _ = api.harp_materialize_blocks(sch, d, th, gs, "f32")
        torch.cuda.synchronize()
        got, ref = blk_out.cpu().numpy().astype(np.float64), b_f.cpu().numpy().astype(np.float64)
        shift = float(np.max(np.abs(got - ref)))
        out.append({"side": side or "rows", "schedule": list(sch), "d": d,
                    "n_theta": int(th.numel()), "n_scales": int(tsc.numel()),
                    "us_quantize_theta": t_q, "us_materialize_f64_theta": t_f, "us_materialize_i8_theta": t_8,
                    "max_abs_block_change_from_int8_theta": shift})
    line = {
        "metric": "HARP block materialisation from int8 parameters, microseconds per call",
        "value": round(sum(o["us_materialize_i8_theta"] for o in out), 3),
        "unit": "us/call",
        "n_gpus": 1, "steps": steps, "warmup": 3,
        "higher_is_better": False,
        "vs_baseline": None,
        "dtype": "f64",
        "data": "synthetic (seeded parameters of the named workload)",
        "config": {"workload": name, "kind": "materialize", "parallelism": "single GPU"},
        "sides": out,
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--blk", default="f32", choices=["f32", "bf16", "i8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain device copy of the batch instead (counter calibration)")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the second timing pass with L2 and the MALL flushed (a 1 GiB write) before "
                         "every launch")
    ap.add_argument("--single", action="store_true",
                    help="the named workload only (the default workload otherwise brings the d = 5120 one along)")
    ap.add_argument("--fp32-intermediates", action="store_true",
                    help="two-sided workload: keep the passes' intermediates in an fp32 workspace")
    ap.add_argument("--mode", default="throughput", choices=["throughput", "latency", "materialize", "vjp"])
    ap.add_argument("--inverse", action="store_true",
                    help="row workloads: time harp_apply_inverse instead of harp_apply (no cpu_baseline and no "
                         "counter record: both belong to the forward transform)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the apply path has no cross-GPU step (rows are independent; "
              "sharding is by rows); run with --gpus 1.", file=sys.stderr)
        return 2
    if args.mode == "latency":
        return latency_main(args)
    if args.mode == "materialize":
        return materialize_main(args)
    if args.mode == "vjp":
        return vjp_main(args)

    import torch
    torch.cuda.set_device(0)
    line = throughput(args.workload, args, with_cpu=not args.no_cpu_baseline and not args.inverse)
    if args.workload == DEFAULT_WORKLOAD and not args.copy_calibration and not args.single and not args.inverse:
        # the headline metric names both row lengths: d = 5120 rides along as
        # a sub-record with the same timing, roofline and counter fields
        sub = throughput(SECOND_WORKLOAD, args, with_cpu=False)
        line["d5120"] = {k: sub[k] for k in ("value", "unit", "ms_per_step", "config", "roofline",
                                             "kernel_ms_mean", "kernel_ms_median", "kernel_ms_p10_p90",
                                             "kernel_ms_mean_flushed", "alg_bytes_per_launch", "compute",
                                             "roundtrip_max_row_rel_l2", "copy_ceiling")}
        if args.blk == "f32":
            # the stored-block options of the same d = 4096 workload (a9): the
            # blocks themselves are rounded, so these lines measure a
            # different operator and stay beside the fp32 headline
            for b in ("bf16", "i8"):
                sub = throughput(DEFAULT_WORKLOAD, argparse.Namespace(**{**vars(args), "blk": b}), with_cpu=False)
                line[f"blocks_{b}"] = {k: sub[k] for k in ("value", "unit", "ms_per_step", "roofline", "kernel_ms_mean",
                                                           "kernel_ms_median", "kernel_ms_mean_flushed",
                                                           "roundtrip_max_row_rel_l2")}
    print(json.dumps(line), flush=True)
    return 0


def throughput(name: str, args, with_cpu: bool) -> dict:
    """One workload: K timed steps back to back (per-launch HIP events on the
    launch stream), then the same launches each after an L2/MALL flush, then
    the untimed checks; returns the JSON record."""
    import torch

    from structured_rotations_amd import api
    from structured_rotations_amd import workloads as W

    w = W.make(name)
    wl = w["workload"]
    d, sch, io = w["d"], w["schedule"], w["io"]
    tdt = torch.bfloat16 if io == "bf16" else torch.float32
    eb = 2 if io == "bf16" else 4
    x = torch.from_numpy(w["x"]).to(tdt).cuda()
    rows = x.shape[0]
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    if args.copy_calibration:
        def step():
            y.copy_(x)
        alg_bytes = rows * d * eb * 2
        alg_flops = 0
        units = rows
    elif wl.kind == "rht":
        sg = torch.from_numpy(w["signs"]).cuda()

        def step():
            api.rht_compose(sch, d, sg, x, y)
        alg_bytes = rows * d * eb * 2
        # k fast Walsh-Hadamard transforms: d log2 d add/sub each, plus the scale
        alg_flops = rows * w["k"] * d * (int(np.log2(d)) + 1)
        units = rows
    elif wl.kind == "two_sided":
        bu, scu = api.harp_materialize_blocks(w["su"], w["d_out"], torch.from_numpy(w["theta_u"]).cuda(),
                                              torch.from_numpy(w["gauss_u"]).cuda(), args.blk)
        bv, scv = api.harp_materialize_blocks(sch, d, torch.from_numpy(w["theta_v"]).cuda(),
                                              torch.from_numpy(w["gauss_v"]).cuda(), args.blk)
        su_s = torch.from_numpy(w["signs_u"]).cuda()
        sv_s = torch.from_numpy(w["signs_v"]).cuda()

        # the rotation as planned for this workload: bf16 between the passes,
        # in place in the output (no workspace); --fp32-intermediates: the
        # binding's default, fp32 between the passes in a workspace allocated
        # once here
        ws = None
        if args.fp32_intermediates:
            ws = torch.empty(api.harp_rotate_weight_workspace(w["d_out"], d), dtype=torch.uint8, device="cuda")

        def step():
            api.harp_rotate_weight(w["su"], bu, scu, su_s, sch, bv, scv, sv_s, x, y, workspace=ws,
                                   fp32_intermediates=ws is not None)
        alg_bytes = rows * d * eb * 2
        # b_t FMAs per element per stage, both sides
        alg_flops = 2 * rows * d * (sum(sch) + sum(w["su"]))
        units = 1
    else:
        th = torch.from_numpy(w["theta"]).cuda()
        gs = torch.from_numpy(w["gauss"]).cuda() if w["gauss"].size else None
        blocks, scales = api.harp_materialize_blocks(sch, d, th, gs, args.blk)
        sg = torch.from_numpy(w["signs"]).cuda()

        if getattr(args, "inverse", False):
            def step():
                api.harp_apply_inverse(sch, d, blocks, scales, sg, x, y)
        else:
            def step():
                api.harp_apply(sch, d, blocks, scales, sg, x, y)
        alg_bytes = rows * d * eb * 2
        alg_flops = 2 * rows * d * sum(sch)      # b_t FMAs per element per stage
        units = rows
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    gc.collect()
    gc.disable()   # re-enabled after the timed steps
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gc.enable()
    total_ms = t_start.elapsed_time(t_end)
    per_launch = np.array([a.elapsed_time(b) for a, b in ev])
    flushed = None
    if not args.no_flush:
        # same launches, each after a 1 GiB write that evicts L2 and the MALL
        scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        evf = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(min(args.steps, 100))]
        for a, b in evf:
            scratch.fill_(1.0)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        flushed = np.array([a.elapsed_time(b) for a, b in evf])
        del scratch
    ms_per_step = total_ms / args.steps
    kern_ms = float(per_launch.mean())
    value = units / (ms_per_step * 1e-3)
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9

    # round trip of the whole batch through the inverse (one more launch,
    # untimed); the oracle's own check of the output is in cpu_baseline
    roundtrip = None
    inverse = wl.kind == "apply" and getattr(args, "inverse", False)
    if not args.copy_calibration and wl.kind == "apply":
        back = api.harp_apply if inverse else api.harp_apply_inverse
        xb = back(sch, d, blocks, scales, sg, y)
        torch.cuda.synchronize()
        roundtrip = float(row_rel_l2(xb.float().cpu().numpy(), x.float().cpu().numpy()).max())

    unit = {"apply": "rows/s", "rht": "rows/s", "two_sided": "weights/s"}[wl.kind]
    # counter records are taken on each workload's default configuration
    traffic = None if (args.copy_calibration or args.fp32_intermediates or inverse) else \
        traffic_from_profile(name, args.blk)
    line = {
        "metric": "HARP apply rows/s + achieved HBM GB/s (% of peak), d=4096/5120 bf16",
        "value": round(value, 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded Student-t nu=3 rows with outlier channels; random Cayley/Givens parameters)",
        "config": {"workload": name if not args.copy_calibration else "device copy of " + name,
                   "rows": rows, "d": d, "schedule": list(sch), "io": io, "blocks": args.blk,
                   "kind": wl.kind, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        "kernel_ms_mean": round(kern_ms, 5),
        "kernel_ms_median": round(float(np.median(per_launch)), 5),
        "kernel_ms_p10_p90": [round(float(np.percentile(per_launch, 10)), 5),
                              round(float(np.percentile(per_launch, 90)), 5)],
        "alg_bytes_per_launch": alg_bytes,
        "compute": {"alg_flops_per_launch": alg_flops,
                    "achieved_tflops": round(alg_flops / (kern_ms * 1e-3) / 1e12, 2),
                    "peak_tflops_fp32": FP32_PEAK_TFLOPS,
                    "frac": round(alg_flops / (kern_ms * 1e-3) / 1e12 / FP32_PEAK_TFLOPS, 4)},
        "kernel_ms_mean_flushed": None if flushed is None else round(float(flushed.mean()), 5),
        "wall_s_timed": round(wall, 4),
        "roundtrip_max_row_rel_l2": roundtrip,
    }
    if not args.copy_calibration:
        line["copy_ceiling"] = copy_ceiling(x, y, stream, achieved)
    if inverse:
        line["config"]["direction"] = "inverse"
    if wl.kind == "two_sided":
        line["config"]["intermediates"] = "fp32 workspace" if args.fp32_intermediates else "bf16, in place"
    if with_cpu and not args.copy_calibration:
        line["cpu_baseline"] = cpu_baseline(w, args.blk, y)
    return line


def copy_ceiling(x, y, stream, achieved_gbps: float, launches: int = 50) -> dict:
    """A plain device copy of the step's input into its output buffer (the
    same bytes read and written), timed like the kernel after the timed
    region: the practical HBM ceiling for this traffic pattern."""
    import torch

    nbytes = 2 * x.numel() * x.element_size()
    y = torch.empty_like(y)     # its own buffer: the step's output is still checked afterwards
    for _ in range(10):
        y.copy_(x)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for a, b in ev:
        a.record(stream)
        y.copy_(x)
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"what": "torch device copy, same bytes in and out", "achieved_GBps": round(gbps, 1),
            "kernel_frac_of_copy": round(achieved_gbps / gbps, 4)}


if __name__ == "__main__":
    sys.exit(main())
