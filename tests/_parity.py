"""Shared helpers for the GPU tests: run the HIP path, run the oracle on the
same inputs, and compare at the stated tolerances.

Tolerances (bf16 inputs, fp32 accumulation, bf16 output):
  out: max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <= 2e-3
  lse: max |gpu - oracle| / |oracle| <= 1e-3
"""

from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import block_sparse_sliding_amd as sta
import oracle

OUT_MAX_ABS = 2e-2
OUT_MEAN_ABS = 2e-3
LSE_REL = 1e-3


def note(msg: str) -> None:
    """Name the case on stdout before a GPU step (survives a lost box)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def run_sta(q, k, v, windows, text_length, has_text, video, workspace=None):
    """One forward through the C ABI. out and lse start as NaN, so a row that no
    workgroup wrote fails every check made on it."""
    B, heads, S, D = q.shape
    dims = sta.make_dims(B, heads, D, video)
    assert sta.sta_seq_len(dims, has_text) == S
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, heads, S), float("nan"), dtype=torch.float32, device=q.device)
    need = sta.sta_workspace_bytes(dims, windows, has_text)
    assert need > 0
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    sta.sta_forward(dims, q, k, v, windows, text_length, has_text, out, lse, workspace)
    torch.cuda.synchronize()
    return out, lse


def oracle_rows(q, k, v, windows, text_length, has_text, video, rows=None):
    """Oracle output for all (b, head) slabs, optionally on a subset of rows.

    Runs head by head on host copies so the float64 working set stays small.
    """
    B, heads, S, D = q.shape
    R = S if rows is None else len(rows)
    out = np.empty((B, heads, R, D))
    lse = np.empty((B, heads, R))
    for h in range(heads):
        qh = q[:, h:h + 1].cpu()
        kh = k[:, h:h + 1].cpu()
        vh = v[:, h:h + 1].cpu()
        o, l = oracle.sta_reference(qh, kh, vh, [windows[h]], text_length, has_text, video,
                                    rows=rows)
        out[:, h] = o[:, 0]
        lse[:, h] = l[:, 0]
    return out, lse


def _oracle_threads(n_tasks: int) -> int:
    """Worker threads for per-head oracle calls: numpy releases the GIL in its
    loops and BLAS calls, so heads run in parallel on the host's cores (each
    thread's BLAS limited to one thread)."""
    try:
        cpus = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cpus = os.cpu_count() or 1
    return max(1, min(n_tasks, cpus, 16))


def map_heads(fn, heads):
    """[fn(h) for h in heads], evaluated on a thread pool (see _oracle_threads)."""
    from threadpoolctl import threadpool_limits

    heads = list(heads)
    with threadpool_limits(limits=1):
        with ThreadPoolExecutor(max_workers=_oracle_threads(len(heads))) as ex:
            return list(ex.map(fn, heads))


def oracle_rows_per_head(q, k, v, windows, text_length, has_text, video, rows_per_head):
    """Oracle out / lse of head h on its own query rows ``rows_per_head[h]``.

    Returns a list over heads of (out [B, R_h, D], lse [B, R_h]) float64 arrays.
    """
    heads = q.shape[1]
    host = [x.cpu() for x in (q, k, v)]

    def one(h):
        o, l = oracle.sta_reference(*(x[:, h:h + 1] for x in host), [windows[h]], text_length,
                                    has_text, video, rows=np.asarray(rows_per_head[h]))
        return o[:, 0], l[:, 0]

    return map_heads(one, range(heads))


def compare_per_head(out_gpu, lse_gpu, refs, rows_per_head, label=""):
    """Parity of every head on its own rows (refs from oracle_rows_per_head), at
    the same tolerances as compare(), pooled over the heads."""
    outs, lses, ros, rls = [], [], [], []
    for h, (ro, rl) in enumerate(refs):
        idx = torch.as_tensor(np.asarray(rows_per_head[h]), dtype=torch.int64)
        outs.append(out_gpu[:, h, idx.to(out_gpu.device)].float().cpu().numpy())
        lses.append(lse_gpu[:, h, idx.to(lse_gpu.device)].float().cpu().numpy())
        ros.append(ro)
        rls.append(rl)
    o = np.concatenate(outs, axis=1).astype(np.float64)
    l = np.concatenate(lses, axis=1).astype(np.float64)
    return _check(o, l, np.concatenate(ros, axis=1), np.concatenate(rls, axis=1), label)


def compare(out_gpu, lse_gpu, out_ref, lse_ref, rows=None, label=""):
    """Assert parity; returns the error summary."""
    o = out_gpu if rows is None else out_gpu[:, :, rows]
    l = lse_gpu if rows is None else lse_gpu[:, :, rows]
    o = o.float().cpu().numpy().astype(np.float64)
    l = l.float().cpu().numpy().astype(np.float64)
    return _check(o, l, out_ref, lse_ref, label)


def _check(o, l, out_ref, lse_ref, label):
    assert np.isfinite(o).all(), f"{label}: non-finite output"
    assert np.isfinite(l).all(), f"{label}: non-finite lse"
    err = np.abs(o - out_ref)
    lrel = np.abs(l - lse_ref) / np.abs(lse_ref)
    summary = dict(max_abs=float(err.max()), mean_abs=float(err.mean()),
                   lse_rel=float(lrel.max()),
                   rel_rms=float(np.sqrt((err ** 2).mean() / (out_ref ** 2).mean())))
    print(f"[parity] {label} {summary}", flush=True)
    assert summary["max_abs"] <= OUT_MAX_ABS, (label, summary)
    assert summary["mean_abs"] <= OUT_MEAN_ABS, (label, summary)
    assert summary["lse_rel"] <= LSE_REL, (label, summary)
    return summary


def scale_key_tiles(k, video, factors, text_factor, ell):
    """k with whole key tiles (t, h, w) multiplied by factors[(t, h, w)] and the
    valid text keys by text_factor: large, uneven score jumps between blocks."""
    B, heads, S, D = k.shape
    T, H, W = video
    nv = T * H * W
    kk = k.float().clone()
    kv = kk[:, :, :nv].view(B, heads, T, H, W, D)
    for (tt, th, tw), f in factors.items():
        kv[:, :, 6 * tt:6 * tt + 6, 8 * th:8 * th + 8, 8 * tw:8 * tw + 8] *= f
    kk[:, :, nv:nv + ell] *= text_factor
    return kk.to(torch.bfloat16)
