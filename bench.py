#!/usr/bin/env python3
"""Benchmark of the STA forward (one GPU); ``--pass backward`` times the backward.

One step = one sta_forward call (the work order, then the fused attention
kernel reading q, k and v and writing out/lse in raster order; it enumerates
each query tile's window itself) on the workload's synthetic bf16 inputs,
which are resident in HBM before timing starts. Prints one JSON line with the
end-to-end effective TFLOP/s, the roofline of the fused attention kernel
(timed live with HIP events on the launch stream) and the fp64 CPU oracle's
throughput on a bounded sample of the same workload.

Effective FLOPs count 4*D per allowed (query, key) pair over the valid query
rows (video rows and the first text_length text rows), i.e. only the tiles
that are computed.

With ``--pass backward`` one step is one sta_backward call (row statistics,
tile lists, the dq pass, the dk/dv pass)
for the forward's out/lse and a synthetic dout; its effective FLOPs are
10*D per allowed pair (five products of 2*D: the recomputed scores, dP, dV,
dQ and dK), the usual count for an attention backward.
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

METRIC = "STA fwd ms/call + effective TFLOP/s (% bf16 MFMA peak), (30,48,80)+256 text"
# MI355X dense bf16 MFMA peak: 256 CUs x 4096 flop/clk x 2.4 GHz (published: 2.5 PFLOP/s)
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12


TILE = (6, 8, 8)


def _axis_pairs(size: int, tile: int, w: int) -> int:
    """Sum over the query tokens of one axis of the key tokens its window holds.

    The tile grid along the axis has ceil(size/tile) tiles, the last holding the
    remainder; tile c's window starts at clamp(c - w//2, 0, n - w). For sizes
    that are tile multiples this is size * w * tile.
    """
    n = -(-size // tile)
    sizes = [min(tile, size - i * tile) for i in range(n)]
    total = 0
    for c in range(n):
        start = min(max(c - w // 2, 0), n - w)
        total += sizes[c] * sum(sizes[start:start + w])
    return total


def effective_flops(wl, include_pad_rows=False) -> float:
    """4*D per allowed (query, key) pair: video queries see the existing tokens of
    their window's tiles (the count factors over the three axes) and the valid
    text keys; valid text queries see every video key and the valid text keys."""
    T, H, W = wl.video
    nv = T * H * W
    ell = wl.text_length if wl.has_text else 0
    text_rows = (256 if include_pad_rows else ell) if wl.has_text else 0
    pairs = 0
    for (wt, wh, ww) in wl.windows:
        video_pairs = 1
        for size, tile, w in zip(wl.video, TILE, (wt, wh, ww)):
            video_pairs *= _axis_pairs(size, tile, w)
        pairs += video_pairs + nv * ell + text_rows * (nv + ell)
    return 4.0 * wl.head_dim * pairs * wl.batch


def hilbert_flops(wl) -> float:
    """4*D per allowed pair of Hilbert slide/window attention: a video query sees
    the 64 tokens of each key tile of its window (W tiles for slide; the tiles of
    its aligned group for window) and the valid text keys; valid text queries
    see every video token and the valid text keys."""
    _, H, W = wl.video
    nv = H * W
    n = nv // 64
    ell = wl.text_length if wl.has_text else 0
    Wl = wl.hilbert_len
    if wl.hilbert_mode == 1:
        key_tiles = n * Wl
    else:
        key_tiles = sum(min(Wl, n - (i // Wl) * Wl) for i in range(n))
    pairs = 64 * (64 * key_tiles) + nv * ell + ell * (nv + ell)
    return 4.0 * wl.head_dim * pairs * wl.heads * wl.batch


def kernel_suffix(wl) -> str:
    """Template arguments of the backward kernels a workload runs: <D, PAD>, PAD
    when a video size is not a tile multiple."""
    pad = any(size % tile for size, tile in zip(wl.video, TILE))
    return f"<{wl.head_dim}, {'true' if pad else 'false'}>"


def square_units(wl) -> bool:
    """Whether the forward runs the workload with query units of 2x2 squares of
    tiles: a one-frame video whose every window spans at least two tiles
    along each axis that has two or more."""
    T, H, W = wl.video
    nh, nw = -(-H // TILE[1]), -(-W // TILE[2])
    return (not wl.hilbert_len and T == 1 and (nh > 1 or nw > 1)
            and all((w[1] >= 2 or nh == 1) and (w[2] >= 2 or nw == 1) for w in wl.windows))


def attention_kernel(wl) -> str:
    """Name of the forward attention kernel a workload runs: <D, PAD, GRP>, GRP
    0 for single-tile query units, 1 for Hilbert units, 2 for 2x2 squares, 3
    for 2x2 squares on an image whose last tile row or column is partial."""
    T, H, W = wl.video
    partial = H % TILE[1] != 0 or W % TILE[2] != 0
    grp = 1 if wl.hilbert_len else (3 if partial else 2) if square_units(wl) else 0
    return f"sta_attention_kernel{kernel_suffix(wl)[:-1]}, {grp}>"


# the files each kernel is compiled from; a counter summary applies only to the
# build whose sources hash to the value recorded with it
FORWARD_SOURCES = ("sta_attention.hip", "sta_device.h", "sta_internal.h")
BACKWARD_SOURCES = ("sta_backward.hip", "sta_device.h", "sta_internal.h")


def sources_hash(sources) -> str:
    """First 16 hex digits of the SHA-256 of the source files, concatenated in order."""
    h = hashlib.sha256()
    for name in sources:
        with open(os.path.join(ROOT, "block_sparse_sliding_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(summary: str, kernel: str, sources):
    """HBM bytes per launch of `kernel` from a committed rocprofv3 counter summary.

    `summary` is a file under profiles/; None when it is missing, holds no figure
    for the kernel, or when `sources` (the files the kernel is compiled from)
    changed since the counters were taken.
    """
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if not line.startswith("#") and ":" in line:
                key, _, val = line.partition(":")
                vals[key.strip()] = val.strip()
    if vals.get("kernel_sources") != " ".join(sources) or \
            vals.get("kernel_sources_sha256_16") != sources_hash(sources):
        return None
    try:
        return float(vals[f"hbm_bytes_per_launch[{kernel}]"])
    except (KeyError, ValueError):
        return None


def host_cpu() -> dict:
    """The host the CPU baseline ran on: CPU model, logical CPUs online and the
    CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.partition(":")[2].strip()
                    break
    except OSError:  # pragma: no cover - /proc is always present on Linux
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": usable, "logical_cpus": os.cpu_count() or 1}


def cpu_baseline(wl, q, k, v, budget_s: float, flops: float):
    """Time the fp64 oracle on a bounded row sample and scale to one full call."""
    import numpy as np

    import oracle
    import sta_inputs

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    # about 0.2 ms of oracle work per row at the headline shape on 16 host
    # threads: 512 rows per head fill a 10-30 s budget before every head is done
    rows = sta_inputs.sample_rows(wl, per_head=512).numpy()
    done_rows, elapsed, heads_done = 0, 0.0, 0
    for h in range(wl.heads):
        qh, kh, vh = (x[:, h:h + 1].cpu() for x in (q, k, v))
        t0 = time.perf_counter()
        oracle.sta_reference(qh, kh, vh, [wl.windows[h]], wl.text_length, wl.has_text, wl.video,
                             rows=rows)
        elapsed += time.perf_counter() - t0
        done_rows += len(rows) * wl.batch
        heads_done += 1
        if elapsed >= budget_s:
            break
    per_row = elapsed / done_rows
    full_call_s = per_row * wl.batch * wl.heads * wl.seq_len
    return {
        "value": flops / full_call_s / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "host": host_cpu(),
        "sample": (f"{done_rows} query rows ({len(rows)} stratified rows x {heads_done} heads), "
                   f"each dense over all {wl.seq_len} keys, {elapsed:.1f} s; extrapolated to "
                   f"B*heads*S = {wl.batch * wl.heads * wl.seq_len} rows"),
        "ms_per_call_extrapolated": full_call_s * 1e3,
    }


def data_label(args) -> str:
    return "zeros (power study, not a throughput figure)" if args.zero_inputs else "synthetic"


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="headline")
    ap.add_argument("--pass", dest="which", choices=("forward", "backward"), default="forward")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 to skip)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (3 times) so "
                         "that hardware byte counters can be scaled against known traffic")
    ap.add_argument("--zero-inputs", action="store_true",
                    help="power study: q, k, v (and dout) all zero. The kernels do the same "
                         "work on inputs that toggle no multiplier bits; the line's data field "
                         "says so and it is not a throughput figure")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the STA benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import block_sparse_sliding_amd as sta
    import sta_inputs

    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    wl = sta_inputs.WORKLOADS[args.workload]
    windows = list(wl.windows)
    q, k, v = sta_inputs.make_qkv(wl, "cuda")
    if args.zero_inputs:
        for t in (q, k, v):
            t.zero_()
        args.cpu_budget = 0.0
    dims = sta.make_dims(wl.batch, wl.heads, wl.head_dim, wl.video)
    out = torch.empty_like(q)
    lse = torch.empty(wl.batch, wl.heads, wl.seq_len, dtype=torch.float32, device="cuda")
    ws = torch.empty(sta.sta_workspace_bytes(dims, windows, wl.has_text), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    if wl.hilbert_len:
        if args.which == "backward":
            raise SystemExit("the Hilbert workload has no backward")
        return bench_hilbert(args, wl, q, k, v, dims, out, lse)
    if args.which == "backward":
        return bench_backward(args, wl, windows, q, k, v, dims, out, lse, ws)

    def step(events=None):
        if events is None:
            sta.sta_forward(dims, q, k, v, windows, wl.text_length, wl.has_text, out, lse, ws)
        else:
            sta.sta_forward_timed(dims, q, k, v, windows, wl.text_length, wl.has_text, out, lse,
                                  ws, events)

    for _ in range(args.warmup):
        step()
    ev_sets = []
    for _ in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(sta.TIMED_EVENTS)]
        for e in evs:
            e.record(stream)  # materialise the underlying hipEvent
        ev_sets.append(evs)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(ev_sets[i])
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps
    stage_ms = {name: 0.0 for name in sta.STAGES}
    for evs in ev_sets:
        for j, name in enumerate(sta.STAGES):
            stage_ms[name] += evs[j].elapsed_time(evs[j + 1]) / args.steps

    flops = effective_flops(wl)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    attn_ms = stage_ms["attention"]
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    attn_kernel = attention_kernel(wl)
    traffic = measured_traffic(f"attention_{args.workload}_pmc.txt", attn_kernel, FORWARD_SOURCES)
    result = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": data_label(args),
        "config": wl.describe(),
        "ms_per_call": ms_per_step,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "effective_flop_per_call": flops,
        "stages_ms": stage_ms,
        "roofline": {
            "kernel": attn_kernel,
            "bound": "mfma",
            "achieved": attn_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": attn_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "launch_ms": attn_ms,
        },
    }
    if args.copy_calibration_mib > 0:
        result["copy_calibration_bytes"] = copy_calibration(args.copy_calibration_mib)
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline(wl, q, k, v, args.cpu_budget, flops)
    print(json.dumps(result), flush=True)


def bench_hilbert(args, wl, q, k, v, dims, out, lse):
    """Hilbert-window attention (sta_hilbert_forward) on a 2D image workload:
    whole calls timed with events on the launch stream."""
    import numpy as np
    import torch

    import block_sparse_sliding_amd as sta
    import oracle

    lens = [w[2] for w in wl.windows]
    ws = torch.empty(sta.sta_hilbert_workspace_bytes(dims, wl.has_text), dtype=torch.uint8, device="cuda")

    def step():
        sta.sta_hilbert_forward(dims, q, k, v, lens, wl.hilbert_mode, wl.text_length, wl.has_text, out, lse, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / args.steps
    flops = hilbert_flops(wl)
    tflops = flops / (ms * 1e-3) / 1e12
    result = {
        "metric": "Hilbert-window attention fwd ms/call + effective TFLOP/s (% bf16 MFMA peak)",
        "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": data_label(args), "config": wl.describe(), "ms_per_call": ms,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS, "effective_flop_per_call": flops,
        "roofline": {"kernel": attention_kernel(wl) + " (whole call)",
                     "bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic("hilbert_pmc.txt", attention_kernel(wl), FORWARD_SOURCES),
                     "launch_ms": ms},
    }
    if args.copy_calibration_mib > 0:
        result["copy_calibration_bytes"] = copy_calibration(args.copy_calibration_mib)
    if args.cpu_budget > 0:
        mode = "slide" if wl.hilbert_mode == 1 else "window"
        rows = np.arange(0, wl.seq_len, max(1, wl.seq_len // 256))
        done, elapsed, heads = 0, 0.0, 0
        for h in range(wl.heads):
            t0 = time.perf_counter()
            oracle.hilbert_reference(q[:, h:h + 1].cpu(), k[:, h:h + 1].cpu(), v[:, h:h + 1].cpu(), [lens[h]],
                                     mode, wl.text_length, wl.has_text, wl.video[1:], rows=rows)
            elapsed += time.perf_counter() - t0
            done += len(rows)
            heads += 1
            if elapsed >= args.cpu_budget:
                break
        full_s = elapsed / done * wl.batch * wl.heads * wl.seq_len
        result["cpu_baseline"] = {"value": flops / full_s / 1e12, "unit": "TFLOP/s",
                                  "cores": int(os.cpu_count() or 1), "kind": "oracle", "host": host_cpu(),
                                  "sample": f"{done} evenly spaced rows x {heads} heads, {elapsed:.1f} s, "
                                            f"extrapolated to {wl.batch * wl.heads * wl.seq_len} rows"}
    print(json.dumps(result), flush=True)


def copy_calibration(mib: int) -> int:
    """A plain device copy of known size (3 times), for scaling byte counters."""
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    return n


def bench_backward(args, wl, windows, q, k, v, dims, out, lse, fwd_ws):
    import torch

    import block_sparse_sliding_amd as sta

    sta.sta_forward(dims, q, k, v, windows, wl.text_length, wl.has_text, out, lse, fwd_ws)
    del fwd_ws
    g = torch.Generator(device="cuda").manual_seed(10 * wl.seed_base + 3)
    dout = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    if args.zero_inputs:
        dout.zero_()
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(sta.sta_backward_workspace_bytes(dims, windows, wl.has_text),
                     dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(events=None):
        if events is None:
            sta.sta_backward(dims, q, k, v, out, lse, dout, windows, wl.text_length, wl.has_text,
                             dq, dk, dv, ws)
        else:
            sta.sta_backward_timed(dims, q, k, v, out, lse, dout, windows, wl.text_length,
                                   wl.has_text, dq, dk, dv, ws, events)

    for _ in range(args.warmup):
        step()
    ev_sets = []
    for _ in range(args.steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(sta.BWD_TIMED_EVENTS)]
        for e in evs:
            e.record(stream)
        ev_sets.append(evs)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(ev_sets[i])
    stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / args.steps
    stage_ms = {name: 0.0 for name in sta.BWD_STAGES}
    for evs in ev_sets:
        for j, name in enumerate(sta.BWD_STAGES):
            stage_ms[name] += evs[j].elapsed_time(evs[j + 1]) / args.steps
    flops = 2.5 * effective_flops(wl)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    # the dq pass executes three of the five products (S, dP, dQ), the dk/dv pass four
    dq_flops, dkv_flops = 0.6 * flops, 0.8 * flops
    sfx = kernel_suffix(wl)
    kernels = {}
    for name, kname, kfl in (("dq", "bwd_dq_kernel" + sfx, dq_flops),
                             ("dkv", "bwd_dkv_kernel" + sfx, dkv_flops)):
        t = kfl / (stage_ms[name] * 1e-3) / 1e12
        kernels[name] = {"kernel": kname, "bound": "mfma", "achieved": t,
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": t / PEAK_BF16_TFLOPS, "launch_ms": stage_ms[name],
                         "executed_flop": kfl,
                         "traffic": measured_traffic(f"backward_{args.workload}_pmc.txt", kname,
                                                     BACKWARD_SOURCES)}
    result = {
        "metric": "STA bwd ms/call + effective TFLOP/s (% bf16 MFMA peak)",
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": data_label(args),
        "config": wl.describe(),
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "effective_flop_per_call": flops,
        "stages_ms": stage_ms,
        "kernels": kernels,
    }
    if args.copy_calibration_mib > 0:
        result["copy_calibration_bytes"] = copy_calibration(args.copy_calibration_mib)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
