"""GPU parity of sta_forward against the fp64 oracle (through the C ABI).

Small shapes are compared on every row; full-size shapes (the five workloads
plus the headline shape) on stratified samples of rows, in the same launch
configuration the benchmark times.
"""

import numpy as np
import pytest
import torch

import sta_inputs
from _parity import (compare, compare_per_head, note, oracle_rows, oracle_rows_per_head, run_sta,
                     scale_key_tiles)

pytestmark = pytest.mark.gpu

FULL_SIZE_ROWS = 512  # sampled query rows per head at the full-size workloads


def rand(shape, seed, device="cuda"):
    g = torch.Generator(device=device).manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def qkv(B, heads, S, D, seed):
    return [rand((B, heads, S, D), seed + i) for i in range(3)]


def test_tiny_full():
    wl = sta_inputs.WORKLOADS["tiny"]
    note("tiny full: (18,24,24) D=64 window (1,3,3) no text")
    q, k, v = sta_inputs.make_qkv(wl, "cuda")
    out, lse = run_sta(q, k, v, list(wl.windows), 0, False, wl.video)
    ro, rl = oracle_rows(q, k, v, list(wl.windows), 0, False, wl.video)
    compare(out, lse, ro, rl, label="tiny")


SMALL = [
    # (B, heads, D, video, windows, text_length, has_text)
    (1, 2, 128, (18, 24, 32), [(3, 3, 3), (1, 2, 3)], 100, True),
    (2, 3, 128, (18, 24, 32), [(3, 3, 3), (1, 2, 3), (2, 1, 4)], 0, True),
    (1, 2, 128, (18, 24, 32), [(3, 1, 3), (2, 3, 1)], 1, True),
    (1, 2, 128, (18, 24, 32), [(3, 3, 3), (3, 3, 4)], 63, True),
    (1, 2, 128, (18, 24, 32), [(1, 1, 1), (3, 3, 3)], 64, True),
    (1, 2, 128, (18, 24, 32), [(2, 2, 2), (3, 3, 3)], 256, True),
    (1, 2, 128, (12, 16, 16), [(2, 2, 2), (1, 1, 1)], 226, True),
    (1, 2, 64, (18, 24, 32), [(3, 3, 3), (1, 3, 2)], 130, True),
    (2, 1, 64, (12, 24, 24), [(2, 3, 3)], 0, False),
    (1, 2, 128, (24, 16, 40), [(3, 1, 5), (4, 2, 2)], 0, False),
    (1, 1, 128, (6, 8, 8), [(1, 1, 1)], 17, True),
]


# Large score jumps: keys of some tiles (and the valid text keys) are scaled so
# that later key blocks hold scores far above the running reference (tens to
# hundreds of log2 units), which forces the online softmax to move its
# reference mid-stream, also in the last, ragged text block. Factors < 1
# give near-zero scores. Random N(0, 1) inputs never exercise this.
JUMPS = [
    # (D, video, windows, text_length, {key tile (tt, th, tw): factor}, text factor)
    (128, (18, 24, 32), [(3, 3, 3), (2, 2, 2)], 100,
     {(1, 1, 2): 2.5, (2, 2, 3): 4.0, (0, 0, 0): 0.05}, 3.5),
    (64, (18, 24, 32), [(3, 3, 3)], 37, {(2, 1, 1): 3.0, (0, 2, 3): 4.0}, 3.5),
]


@pytest.mark.parametrize("case", JUMPS, ids=[f"j{i}" for i in range(len(JUMPS))])
def test_large_score_jumps(case):
    D, video, windows, ell, factors, text_factor = case
    heads = len(windows)
    S = video[0] * video[1] * video[2] + 256
    note(f"score jumps {case}")
    q, k, v = qkv(1, heads, S, D, 900 + D + ell)
    k = scale_key_tiles(k, video, factors, text_factor, ell)
    out, lse = run_sta(q, k, v, windows, ell, True, video)
    ro, rl = oracle_rows(q, k, v, windows, ell, True, video)
    compare(out, lse, ro, rl, label=f"jumps D={D}")


@pytest.mark.parametrize("case", SMALL, ids=[f"s{i}" for i in range(len(SMALL))])
def test_small_all_rows(case):
    B, heads, D, video, windows, ell, text = case
    S = video[0] * video[1] * video[2] + (256 if text else 0)
    note(f"small {case}")
    q, k, v = qkv(B, heads, S, D, 100 + S + ell)
    out, lse = run_sta(q, k, v, windows, ell, text, video)
    nv = S - (256 if text else 0)
    if S * B * heads <= 60000:
        rows = None
    else:
        rng = np.random.default_rng(S)
        rows = np.unique(np.concatenate([rng.integers(0, nv, 1500), np.arange(nv, S),
                                         [0, nv - 1]]))
    ro, rl = oracle_rows(q, k, v, windows, ell, text, video, rows=rows)
    compare(out, lse, ro, rl, rows=None if rows is None else torch.from_numpy(rows),
            label=str(case))


@pytest.mark.parametrize("name", ["notext", "text", "mixed", "large", "headline", "ragged", "image"])
def test_full_size_sampled(name):
    wl = sta_inputs.WORKLOADS[name]
    note(f"full-size {name}: {wl.describe()}")
    q, k, v = sta_inputs.make_qkv(wl, "cuda")
    out, lse = run_sta(q, k, v, list(wl.windows), wl.text_length, wl.has_text, wl.video)
    # every row of every (batch, head) was written (the outputs start as NaN)
    assert bool(torch.isfinite(out).all()) and bool(torch.isfinite(lse).all()), name
    # 512 stratified rows per head, a different draw for every head: at these
    # shapes each workgroup of the persistent grid runs many query units in
    # turn, and the draws reach nearly every query tile of every head
    rows = [sta_inputs.sample_rows_stratified(wl, FULL_SIZE_ROWS, h).numpy()
            for h in range(wl.heads)]
    tiles_hit = min(len({sta_inputs.tile_of_row(wl, int(r)) for r in rh}) for rh in rows)
    note(f"full-size {name}: {FULL_SIZE_ROWS} rows per head, >= {tiles_hit} query units per head")
    refs = oracle_rows_per_head(q, k, v, list(wl.windows), wl.text_length, wl.has_text, wl.video,
                                rows)
    compare_per_head(out, lse, refs, rows, label=name)
    del q, k, v, out, lse
    torch.cuda.empty_cache()
