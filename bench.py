#!/usr/bin/env python3
"""Radial attention forward pass on one MI355X: effective TFLOP/s on active blocks.

    python bench.py [--steps K] [--warmup W]
                    [--workload wan|hunyuan|long4x|small|tiny|wan-grid|hunyuan-grid]
                    [--element] [--backward] [--rule] [--varlen F1,F2,...]

A step is one call of the block-sparse forward kernel over the whole workload
(every batch, head and query block), with Q/K/V already resident in HBM. The static mask
is built once before timing, and its host build time is reported on its own. After W
untimed warm-up steps, exactly K steps are timed with HIP events on the stream the
kernel runs on, between device synchronisations. The same kernel with the all-active
mask gives the dense baseline. The CPU oracle is timed beside it on a bounded sample.
Rank 0 prints one JSON line. --element times element masking instead (the radial rule on
single entries inside the active blocks; the oracle runs the same option). --backward
times the backward pass (dq, dk, dv from the forward's o and lse, and a seeded dO),
counting 2.5 times the forward's work (the usual five products against two), and its
dense baseline and CPU oracle likewise. --varlen F1,F2,... times one packed launch over
videos of those frame counts (the workload's frame length, W0, heads and head_dim),
beside the same samples run as separate launches one after another (with --backward,
the backward pass likewise). --rule times the forward with the block mask derived in the
kernel from the rule instead of read from the CSR (the same key blocks, so the same work
is counted), also for --varlen. The default run (Wan, block semantics, forward) also
times the HunyuanVideo and the 4x-long workloads, sparse and dense, and adds them to the
line under "other_workloads", and element masking at the Wan shape (1-D and grid
distance; from the element table and with the rule in the kernel, against block
semantics) under "element_masking" (--no-extra skips both).

Work is counted on whole active 128x128 tiles: 4 * head_dim * 128^2 flops per tile per
(batch, head). QK^T and PV each contribute 2 * 128^2 * head_dim.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
# The forward kernel's sources: its traffic counters are valid while these are unchanged.
KERNEL_SRCS = [os.path.join(ROOT, "block_sparse_attention_radial_amd", "csrc", f)
               for f in ("radial_attn_fwd.hip", "radial_device.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_digest() -> str:
    """sha256 over the forward kernel's source files, in order."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes(workload_name: str):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counters.

    Null when no counters exist for this workload or the kernel source changed since.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha256") != kernel_digest():
        return None
    return rec.get("bytes_per_launch")


def time_launches(fn, steps: int, warmup: int):
    """Run `fn` warmup times, synchronise, then time exactly `steps` calls, each between its
    own pair of HIP events on torch's current stream (the stream the kernels run on),
    and synchronise again. Returns the mean, median and minimum per-call milliseconds
    and the host wall time of the timed region."""
    import statistics

    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
    t0 = time.perf_counter()
    for start, stop in events:
        start.record(stream)
        fn()
        stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [start.elapsed_time(stop) for start, stop in events]
    return {"mean": sum(ms) / len(ms), "median": statistics.median(ms), "min": min(ms),
            "wall": wall}


def cpu_baseline(wl, q, k, v, mask, seconds: float, element: bool = False, do=None):
    """Time the fp64 CPU oracle over heads 0, 1, ... (each head's query blocks in a seeded
    order) until about `seconds` of work has run. Report the same active-tile flop rate
    as the GPU."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import radial_oracle as ro

    t0 = time.perf_counter()
    rp, ci = ro.csr(ro.block_mask(wl.frames, wl.tokens_per_frame, wl.w0, grid_w=wl.grid_w))
    mask_s = time.perf_counter() - t0
    del mask  # the oracle walks its own CSR
    rule = (wl.tokens_per_frame, wl.w0) + ((wl.grid_w,) if wl.grid_w else ())
    order = np.random.default_rng(0).permutation(wl.nb)
    blocks, tiles, heads, elapsed = 0, 0, 0, 0.0
    for h in range(wl.batch * wl.heads):
        b, hh = divmod(h, wl.heads)
        qh, kh, vh = (x[b, hh].double().cpu().numpy() for x in (q, k, v))
        doh = None if do is None else do[b, hh].double().cpu().numpy()
        heads += 1
        t0 = time.perf_counter()
        for qb in order:
            if do is None:
                ro.attention(qh, kh, vh, rp, ci, wl.scale, query_blocks=[int(qb)],
                             element=rule if element else None)
            else:  # the backward of this query block (its dq and its share of dk, dv)
                ro.attention_backward(qh, kh, vh, doh, rp, ci, wl.scale,
                                      element=rule if element else None,
                                      query_blocks=[int(qb)])
            blocks += 1
            tiles += int(rp[qb + 1] - rp[qb])
            if elapsed + time.perf_counter() - t0 >= seconds:
                break
        elapsed += time.perf_counter() - t0
        if elapsed >= seconds:
            break
    flops = 4 * wl.head_dim * 128 * 128 * tiles * (2.5 if do is not None else 1)
    threads = [d.get("num_threads", 0) for d in threadpool_info()
               if d.get("user_api") == "blas"]
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": max(threads) if threads else 1,
        "kind": "oracle",
        "sample": f"{blocks} query blocks over {heads} of {wl.batch * wl.heads} heads "
                  f"({tiles} active tiles) in {elapsed:.1f} s, fp64 numpy; "
                  f"oracle block-mask build {mask_s:.2f} s",
    }


def bench_varlen(args, wl, dev):
    """One packed launch over videos of the given frame counts, against the same samples
    launched one by one (each as a strided [1, H, n, D] view of the packed tensors)."""
    import torch

    import block_sparse_attention_radial_amd as radial
    from block_sparse_attention_radial_amd.inputs import Workload, draw_packed_qkv

    frames = [int(f) for f in args.varlen.split(",")]
    t0 = time.perf_counter()
    masks = [radial.build_mask(f, wl.tokens_per_frame, wl.w0, grid_w=wl.grid_w) for f in frames]
    vmask = radial.concat_masks(masks)
    mask_ms = (time.perf_counter() - t0) * 1e3
    vdev = vmask.to(dev)
    if args.rule:  # the same samples, each mask derived in the kernel
        if args.backward:
            print("--rule times the forward only", file=sys.stderr)
            sys.exit(2)
        vdev = radial.VarlenRuleMask(frames, wl.tokens_per_frame, wl.w0, wl.grid_w or 0,
                                     vmask.pairs, vmask.npairs).to(dev)
    mdevs = [m.to(dev) for m in masks]
    if args.element and not args.element_rule and not args.rule:
        # element decisions from tables built once, for the packed batch and the samples
        vdev.with_element_table()
        for m in mdevs:
            m.with_element_table()
    total = sum(m.n for m in masks)
    q, k, v = draw_packed_qkv(total, wl.heads, wl.head_dim, wl.sigma, seed=0, device=dev)
    o = torch.empty_like(q)
    nnz = sum(m.nnz for m in masks)
    flops = 4 * wl.head_dim * 128 * 128 * nnz * wl.heads
    log(f"varlen {wl.name} frames {frames}: {total} tokens, {nnz} active blocks, "
        f"mask build {mask_ms:.2f} ms")

    work = 2.5 if args.backward else 1.0
    flops = int(flops * work)
    el = args.element
    if args.backward:
        gen = torch.Generator(device=dev).manual_seed(1)
        do = torch.randn(q.shape, generator=gen, device=dev).to(torch.bfloat16)
        lse = torch.empty(wl.heads, total, dtype=torch.float32, device=dev)
        radial.attn_fwd_varlen(q, k, v, vdev, out=o, lse=lse, element=el)
        run = lambda: radial.attn_bwd_varlen(q, k, v, o, do, lse, vdev, element=el)  # noqa: E731
    else:
        run = lambda: radial.attn_fwd_varlen(q, k, v, vdev, out=o, element=el)  # noqa: E731
    tm = time_launches(run, args.steps, args.warmup)
    ms, wall = tm["mean"], tm["wall"]
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"packed{' backward' if args.backward else ''}: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s "
        f"({tflops / PEAK_BF16_TFLOPS:.1%} of peak)")

    views, t0 = [], 0
    for i, m in enumerate(masks):
        sl = slice(t0, t0 + m.n)
        xs = (q, k, v, o) + ((do,) if args.backward else ())
        views.append(tuple(x[sl].permute(1, 0, 2).unsqueeze(0) for x in xs))
        if args.backward:  # this sample's own lse, as its own forward writes it
            views[-1] += (lse[:, sl].unsqueeze(0).contiguous(),)
        t0 += m.n

    def separate():
        for vw, md in zip(views, mdevs):
            if args.backward:
                qs, ks, vs, os_, dos, ls = vw
                radial.attn_bwd(qs, ks, vs, os_, dos, ls, md, element=el)
            else:
                qs, ks, vs, os_ = vw
                radial.attn_fwd(qs, ks, vs, md, out=os_, element=el)
    sms = time_launches(separate, args.steps, args.warmup)["mean"]
    log(f"separate launches: {sms:.3f} ms/step ({flops / (sms * 1e-3) / 1e12:.1f} TFLOP/s)")

    cpu = None
    if not args.no_cpu_baseline:
        # The oracle on the first sample alone (its own [1, H, n, D] views).
        swl = Workload(f"{wl.name}-sample0", 1, wl.heads, wl.head_dim, frames[0],
                       wl.tokens_per_frame, wl.w0, wl.sigma, grid_w=wl.grid_w)
        qs, ks, vs = views[0][:3]
        dos = views[0][4] if args.backward else None
        cpu = cpu_baseline(swl, qs, ks, vs, masks[0], args.cpu_seconds, args.element, dos)
        log(f"cpu oracle: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads; {cpu['sample']}")

    line = result_line(args, tflops, tm, {
        "workload": f"varlen-{wl.name}", "batch": len(frames), "heads": wl.heads,
        "head_dim": wl.head_dim, "frames": frames, "tokens_per_frame": wl.tokens_per_frame,
        "seq_len": total, "w0": wl.w0, "grid_w": wl.grid_w, "block": 128, "active_blocks": nnz,
        "total_blocks": sum(m.nb ** 2 for m in masks),
        "semantics": "element" if args.element else "block",
        "pass": "backward" if args.backward else "forward",
        "mask": "rule (in-kernel)" if args.rule else "csr"},
        traffic=None, cpu=cpu)
    line["separate_launches_ms"] = round(sms, 4)
    line["speedup_vs_separate"] = round(sms / ms, 3)
    line["mask_build_ms"] = round(mask_ms, 3)
    print(json.dumps(line), flush=True)


def result_line(args, tflops, tm, config, traffic, cpu):
    """The JSON result line, without the dense baseline fields. tm: time_launches' result;
    ms_per_step is the mean per-launch time, and value the work over it."""
    ms = tm["mean"]
    return {
        "metric": "active-block attention TFLOP/s (% bf16 MFMA peak) + speedup vs dense, 1 GPU",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) q/k/v in bf16 at the workload's shape",
        "config": config,
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "ms_median": round(tm["median"], 4),
        "ms_min": round(tm["min"], 4),
        "wall_s_timed": round(tm["wall"], 4),
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": cpu,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="with the default Wan workload, skip the HunyuanVideo and 4x-long "
                         "timings that the line otherwise carries")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--element", action="store_true",
                    help="element masking inside the active blocks (block semantics "
                         "otherwise); the forward reads the decisions from an element "
                         "table built once per mask, outside the timed region")
    ap.add_argument("--element-rule", action="store_true",
                    help="with --element, evaluate the rule in the kernels on every tile "
                         "instead of reading an element table")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dq, dk, dv) instead of the forward")
    ap.add_argument("--rule", action="store_true",
                    help="derive the block mask in the kernel from the rule (no CSR read)")
    ap.add_argument("--varlen", default="", metavar="F1,F2,...",
                    help="time a packed batch of videos with these frame counts")
    ap.add_argument("--heads", type=int, default=0,
                    help="run the workload with this many heads instead of its own (e.g. one "
                         "GPU's share when the heads are split across GPUs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (5 times), to scale "
                         "HBM traffic counters against a kernel of known size")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would shard across GPUs with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_radial_amd as radial
    from block_sparse_attention_radial_amd.inputs import WORKLOADS, draw_qkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        src = torch.ones(args.copy_calibration << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration} MiB 5 times")
        return
    radial.lib()
    wl = WORKLOADS[args.workload]
    if args.heads:
        if args.heads < 0:
            print("--heads must be positive", file=sys.stderr)
            sys.exit(2)
        wl = dataclasses.replace(wl, heads=args.heads)
    dev = torch.device("cuda:0")
    if args.varlen:
        bench_varlen(args, wl, dev)
        return

    t0 = time.perf_counter()
    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0, grid_w=wl.grid_w)
    mask_ms = (time.perf_counter() - t0) * 1e3
    mdev = mask.to(dev)
    table_ms = None
    if args.element and not args.element_rule and not args.rule:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        mdev.with_element_table()
        torch.cuda.synchronize()
        table_ms = (time.perf_counter() - t0) * 1e3
    if args.rule:
        if args.backward:
            print("--rule times the forward only", file=sys.stderr)
            sys.exit(2)
        mdev = radial.rule_mask(wl.frames, wl.tokens_per_frame, wl.w0, grid_w=wl.grid_w,
                                pairs=True).to(dev)
    q, k, v = draw_qkv(wl, seed=0, device=dev)
    o = torch.empty_like(q)
    bh = wl.batch * wl.heads
    flops = 4 * wl.head_dim * 128 * 128 * mask.nnz * bh
    log(f"workload {wl.name}: n={wl.n} nb={mask.nb} nnz={mask.nnz} "
        f"({mask.nnz / mask.nb ** 2:.3f} of blocks), mask build {mask_ms:.2f} ms")

    work = 2.5 if args.backward else 1.0
    flops = int(flops * work)
    do = None
    if args.backward:
        gen = torch.Generator(device=dev).manual_seed(1)
        do = torch.randn(q.shape, generator=gen, device=dev).to(torch.bfloat16)

        def step(m):
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
            out = radial.attn_fwd(q, k, v, m, lse=lse, element=args.element)
            torch.cuda.synchronize()
            return lambda: radial.attn_bwd(q, k, v, out, do, lse, m, element=args.element)
        run = step(mdev)
    else:
        run = lambda: radial.attn_fwd(q, k, v, mdev, out=o, element=args.element)  # noqa: E731
    tm = time_launches(run, args.steps, args.warmup)
    ms = tm["mean"]
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{'backward' if args.backward else 'sparse'}"
        f"{' (element masking' + (', table)' if table_ms is not None else ')') if args.element else ''}"
        f": {ms:.3f} ms/step "
        f"(median {tm['median']:.3f}, min {tm['min']:.3f}), {tflops:.1f} TFLOP/s "
        f"({tflops / PEAK_BF16_TFLOPS:.1%} of peak)")

    dense = None
    if not args.no_dense:
        dmask = radial.dense_mask(wl.n, device=dev)
        dsteps = max(3, args.steps // 2)
        drun = step(dmask) if args.backward else (
            lambda: radial.attn_fwd(q, k, v, dmask, out=o))
        dms = time_launches(drun, dsteps, min(args.warmup, 2))["mean"]
        dflops = 4 * wl.head_dim * 128 * 128 * dmask.nnz * bh * work
        dense = {"ms": dms, "tflops": dflops / (dms * 1e-3) / 1e12, "steps": dsteps,
                 "speedup": dms / ms, "ideal_speedup": dmask.nnz / mask.nnz}
        log(f"dense:  {dms:.3f} ms/step, {dense['tflops']:.1f} TFLOP/s; "
            f"speedup {dense['speedup']:.2f}x (block-count ceiling {dense['ideal_speedup']:.2f}x)")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, q, k, v, mask, args.cpu_seconds, args.element, do)
        log(f"cpu oracle: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads; {cpu['sample']}")

    traffic = None if args.backward or args.rule or args.heads else traffic_bytes(
        wl.name + ("-element" if args.element else "")
        + ("-table" if table_ms is not None else ""))
    line = result_line(args, tflops, tm, {
        "workload": wl.name, "batch": wl.batch, "heads": wl.heads,
        "head_dim": wl.head_dim, "frames": wl.frames,
        "tokens_per_frame": wl.tokens_per_frame, "seq_len": wl.n, "w0": wl.w0,
        "grid_w": wl.grid_w,
        "block": 128, "active_blocks": mask.nnz, "total_blocks": mask.nb ** 2,
        "semantics": "element" if args.element else "block",
        "pass": "backward" if args.backward else "forward",
        "mask": "rule (in-kernel)" if args.rule else "csr",
        "element_decisions": None if not args.element else (
            "table" if table_ms is not None else "rule (in-kernel)"),
    }, traffic=traffic, cpu=cpu)
    line["speedup_vs_dense"] = None if dense is None else round(dense["speedup"], 3)
    line["dense"] = None if dense is None else {k_: round(v_, 4) for k_, v_ in dense.items()}
    line["mask_build_ms"] = round(mask_ms, 3)
    if table_ms is not None:
        line["element_table_build_ms"] = round(table_ms, 3)
        line["element_table_bytes"] = mdev.element_table.numel() * 8

    plain = not (args.backward or args.element or args.rule or args.no_extra or args.heads)
    if plain and args.workload == "wan":
        # The pages' other two workloads, on the same kernel: the same line carries their
        # sparse and dense times (no CPU leg), with the ceiling that block skipping allows.
        del q, k, v, o, run, mdev
        torch.cuda.empty_cache()
        line["other_workloads"] = {key: other_workload(WORKLOADS[key], dev, args)
                                   for key in ("hunyuan", "long4x")}
        # Element masking (the rule on single entries inside the active blocks) at the
        # Wan shape, 1-D and grid distance: block semantics, the decisions read from the
        # element table, and the rule evaluated in the kernel, interleaved.
        line["element_masking"] = {key: element_workload(WORKLOADS[key], dev)
                                   for key in ("wan", "wan-grid")}
    print(json.dumps(line), flush=True)


def other_workload(wl, dev, args):
    """Sparse and dense forward times of a full-size workload (5 and 3 timed launches)."""
    import torch

    import block_sparse_attention_radial_amd as radial
    from block_sparse_attention_radial_amd.inputs import draw_qkv

    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0)
    mdev = mask.to(dev)
    q, k, v = draw_qkv(wl, seed=0, device=dev)
    o = torch.empty_like(q)
    flops = 4 * wl.head_dim * 128 * 128 * mask.nnz * wl.batch * wl.heads
    tm = time_launches(lambda: radial.attn_fwd(q, k, v, mdev, out=o), 5, 2)
    dmask = radial.dense_mask(wl.n, device=dev)
    dms = time_launches(lambda: radial.attn_fwd(q, k, v, dmask, out=o), 3, 1)["mean"]
    tflops = flops / (tm["mean"] * 1e-3) / 1e12
    rec = {
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads,
                   "head_dim": wl.head_dim, "frames": wl.frames,
                   "tokens_per_frame": wl.tokens_per_frame, "seq_len": wl.n, "w0": wl.w0,
                   "active_blocks": mask.nnz, "total_blocks": mask.nb ** 2},
        "steps": 5, "ms_per_step": round(tm["mean"], 4), "ms_median": round(tm["median"], 4),
        "ms_min": round(tm["min"], 4), "tflops": round(tflops, 3),
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "dense_ms": round(dms, 4), "dense_steps": 3,
        "speedup_vs_dense": round(dms / tm["mean"], 3),
        "block_count_ceiling": round(mask.nb ** 2 / mask.nnz, 3),
    }
    log(f"{wl.name}: sparse {tm['mean']:.3f} ms ({tflops:.1f} TFLOP/s, "
        f"{tflops / PEAK_BF16_TFLOPS:.1%}), dense {dms:.3f} ms, speedup "
        f"{rec['speedup_vs_dense']:.2f}x (block-count ceiling {rec['block_count_ceiling']:.2f}x)")
    del q, k, v, o
    torch.cuda.empty_cache()
    return rec


def element_workload(wl, dev):
    """Forward times of block semantics, element masking from the element table and from
    the rule in the kernel (10 timed launches each, twice, interleaved)."""
    import torch

    import block_sparse_attention_radial_amd as radial
    from block_sparse_attention_radial_amd.inputs import draw_qkv

    mask = radial.build_mask(wl.frames, wl.tokens_per_frame, wl.w0, grid_w=wl.grid_w)
    rule = mask.to(dev)
    table = mask.to(dev)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    table.with_element_table()
    torch.cuda.synchronize()
    build_ms = (time.perf_counter() - t0) * 1e3
    q, k, v = draw_qkv(wl, seed=0, device=dev)
    o = torch.empty_like(q)
    runs = {"block": lambda: radial.attn_fwd(q, k, v, rule, out=o),
            "element_table": lambda: radial.attn_fwd(q, k, v, table, out=o, element=True),
            "element_rule": lambda: radial.attn_fwd(q, k, v, rule, out=o, element=True)}
    ms = {key: [] for key in runs}
    for _ in range(2):
        for key, fn in runs.items():
            ms[key].append(time_launches(fn, 10, 2)["mean"])
    avg = {key: sum(v_) / len(v_) for key, v_ in ms.items()}
    rec = {"block_ms": round(avg["block"], 4),
           "element_table_ms": round(avg["element_table"], 4),
           "element_rule_ms": round(avg["element_rule"], 4),
           "table_overhead": round(avg["element_table"] / avg["block"] - 1, 4),
           "rule_overhead": round(avg["element_rule"] / avg["block"] - 1, 4),
           "table_build_ms": round(build_ms, 3),
           "table_bytes": table.element_table.numel() * 8,
           "grid_w": wl.grid_w, "w0": wl.w0}
    log(f"{wl.name} element masking: block {avg['block']:.3f} ms, from the table "
        f"{avg['element_table']:.3f} ms ({rec['table_overhead']:+.1%}), rule in the kernel "
        f"{avg['element_rule']:.3f} ms ({rec['rule_overhead']:+.1%})")
    del q, k, v, o
    torch.cuda.empty_cache()
    return rec


if __name__ == "__main__":
    main()
