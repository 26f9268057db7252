"""GPU parity (through the C ABI) for video sizes that are not tile multiples.

Reading (the page's kernel takes only multiples of (6, 8, 8)): the tile grid
is (ceil(T/6), ceil(H/8), ceil(W/8)), the last tile along an axis holds the
remainder, windows are placed on that grid as for multiples, and a query sees
the tokens that exist in its window's tiles. The oracle implements exactly
this (dense masked attention over an explicit token mask); here the HIP
forward and backward are compared with it on every row of small shapes and on
sampled rows of a medium one. Outputs and gradients start as NaN, so a row
the kernels skip fails the checks.

The shapes cover partial tiles along each axis alone and together, a last
frame tile holding 1 frame (the second key unit of such a tile has no keys)
or 5 frames, a video of one frame, a single partial tile, every unit shape
of the partial-tile kernels (16 rows per wave on 4 or 8 waves, 4 waves x 48
rows for 129 to 192 tokens, 8 x 32, 8 x 48), both head sizes, with and without
text, and large score jumps between key tiles.
"""

import numpy as np
import pytest
import torch

import oracle
from _parity import compare, note, oracle_rows, run_sta, scale_key_tiles
from test_gpu_backward import compare_grad, inputs, run_backward

pytestmark = pytest.mark.gpu

CASES = [
    # (B, D, video, windows, text_length, has_text)
    (1, 128, (7, 9, 11), [(2, 2, 2), (1, 1, 2)], 77, True),
    (2, 64, (13, 8, 20), [(3, 1, 3), (1, 1, 1), (2, 1, 2)], 0, False),
    (1, 128, (1, 12, 20), [(1, 2, 3)], 256, True),
    (1, 64, (5, 7, 3), [(1, 1, 1)], 0, True),
    (1, 128, (11, 17, 9), [(2, 3, 2), (1, 1, 1)], 200, True),
    (1, 128, (12, 15, 16), [(2, 2, 2)], 63, True),
    (1, 64, (18, 24, 21), [(3, 3, 2), (1, 2, 3)], 0, False),
    # partial tiles of 150 and 180 tokens (4 waves x 48 rows), 240 and 320
    (1, 128, (17, 21, 30), [(2, 2, 2)], 100, True),
]
IDS = [f"g{i}" for i in range(len(CASES))]


def seq(video, has_text):
    return video[0] * video[1] * video[2] + (256 if has_text else 0)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_forward_partial_tiles_all_rows(case):
    B, D, video, windows, ell, has_text = case
    heads = len(windows)
    S = seq(video, has_text)
    note(f"forward partial tiles {case}")
    q, k, v, _ = inputs(B, heads, S, D, 3000 + S + D)
    out, lse = run_sta(q, k, v, windows, ell, has_text, video)
    ro, rl = oracle_rows(q, k, v, windows, ell, has_text, video)
    compare(out, lse, ro, rl, label=f"partial {case}")


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_backward_partial_tiles_all_rows(case):
    B, D, video, windows, ell, has_text = case
    heads = len(windows)
    S = seq(video, has_text)
    note(f"backward partial tiles {case}")
    q, k, v, dout = inputs(B, heads, S, D, 4000 + S + D)
    out, lse = run_sta(q, k, v, windows, ell, has_text, video)
    dq, dk, dv = run_backward(q, k, v, out, lse, dout, windows, ell, has_text, video)
    rq, rk, rv = oracle.sta_reference_backward(q.cpu(), k.cpu(), v.cpu(), dout.cpu(), windows,
                                               ell, has_text, video)
    compare_grad(dq, rq, f"dq {case}")
    compare_grad(dk, rk, f"dk {case}")
    compare_grad(dv, rv, f"dv {case}")


def test_partial_tiles_large_score_jumps():
    """Scaled key tiles on a partial grid: the running reference moves inside
    partial key tiles, whose missing keys must stay out of the maximum."""
    D, video, windows, ell = 128, (7, 9, 11), [(2, 2, 2), (1, 2, 1)], 100
    S = seq(video, True)
    note("partial tiles score jumps")
    q, k, v, dout = inputs(1, 2, S, D, 5151)
    k = scale_key_tiles(k, video, {(1, 1, 1): 4.0, (0, 1, 0): 2.5, (1, 0, 0): 0.05}, 3.0, ell)
    out, lse = run_sta(q, k, v, windows, ell, True, video)
    ro, rl = oracle_rows(q, k, v, windows, ell, True, video)
    compare(out, lse, ro, rl, label="partial jumps")
    dq, dk, dv = run_backward(q, k, v, out, lse, dout, windows, ell, True, video)
    rq, rk, rv = oracle.sta_reference_backward(q.cpu(), k.cpu(), v.cpu(), dout.cpu(), windows,
                                               ell, True, video)
    compare_grad(dq, rq, "dq partial jumps")
    compare_grad(dk, rk, "dk partial jumps")
    compare_grad(dv, rv, "dv partial jumps")


def test_partial_tiles_medium_sampled():
    """(20, 30, 45) + 256 text (tile grid (4, 4, 6), every border tile partial),
    two heads: sampled query rows and every key row of the far corner tile."""
    video, windows, ell, D = (20, 30, 45), [(3, 3, 3), (1, 2, 4)], 150, 128
    T, H, W = video
    nv = T * H * W
    S = nv + 256
    note(f"partial tiles medium {video}")
    q, k, v, dout = inputs(1, 2, S, D, 6060)
    out, lse = run_sta(q, k, v, windows, ell, True, video)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.integers(0, S, 300), [0, nv - 1, nv, S - 1]]))
    ro, rl = oracle_rows(q, k, v, windows, ell, True, video, rows=rows)
    compare(out, lse, ro, rl, rows=torch.from_numpy(rows), label="partial medium")
    assert bool(torch.isfinite(out).all() and torch.isfinite(lse).all())

    dq, dk, dv = run_backward(q, k, v, out, lse, dout, windows, ell, True, video)
    keys = [(t * H + h) * W + w for t in range(18, T) for h in range(24, H) for w in range(40, W)]
    keys = np.unique(np.asarray(keys + [0, nv + ell - 1]))
    for h in range(2):
        sl = slice(h, h + 1)
        rq, rk, rv = oracle.sta_reference_backward(
            q[:, sl].cpu(), k[:, sl].cpu(), v[:, sl].cpu(), dout[:, sl].cpu(), [windows[h]], ell,
            True, video, query_rows=rows, key_rows=keys)
        compare_grad(dq[:, sl][:, :, torch.from_numpy(rows)], rq, f"dq medium head {h}")
        compare_grad(dk[:, sl][:, :, torch.from_numpy(keys)], rk, f"dk medium head {h}")
        compare_grad(dv[:, sl][:, :, torch.from_numpy(keys)], rv, f"dv medium head {h}")
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), name


def test_backward_full_size_ragged():
    """(33, 45, 80) + 256 text, D = 128 (last tile row in t: 3 of 6 frames; in h:
    5 of 8 rows): every gradient written, sum rules per head, sampled dq rows
    and every key row of two partial key tiles, at the launch shape the
    benchmark times."""
    import sta_inputs

    wl = sta_inputs.WORKLOADS["ragged"]
    T, H, W = wl.video
    heads = 3
    windows = [(3, 3, 3), (1, 1, 1), (5, 6, 10)]
    ell = wl.text_length
    nv = T * H * W
    S = nv + 256
    note(f"backward full size ragged {wl.video}+256, {heads} heads")
    q, k, v, dout = inputs(1, heads, S, 128, 91)
    out, lse = run_sta(q, k, v, windows, ell, True, wl.video)
    assert bool(torch.isfinite(out).all() and torch.isfinite(lse).all())
    dq, dk, dv = run_backward(q, k, v, out, lse, dout, windows, ell, True, wl.video)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), name
    sdv, sdo, sdk = dv.double().sum(dim=2), dout.double().sum(dim=2), dk.double().sum(dim=2)
    assert bool(((sdv - sdo).abs() <= 1e-2 * dv.double().abs().sum(dim=2) + 1e-3).all())
    assert bool((sdk.abs() <= 1e-2 * dk.double().abs().sum(dim=2) + 1e-3).all())
    rng = np.random.default_rng(11)
    qrows = np.unique(np.concatenate([rng.integers(0, nv, 16), [nv - 1, nv, S - 1]]))
    # key tile (2, 5, 4): rows 40..44 exist (5 of 8); key tile (5, 2, 3): frames
    # 30..32 exist (3 of 6)
    keys = np.asarray([((12 + a) * H + 40 + b) * W + 32 + c
                       for a in range(6) for b in range(5) for c in range(8)]
                      + [((30 + a) * H + 16 + b) * W + 24 + c
                         for a in range(3) for b in range(8) for c in range(8)])
    for h in range(heads):
        sl = slice(h, h + 1)
        rq, rk, rv = oracle.sta_reference_backward(
            q[:, sl].cpu(), k[:, sl].cpu(), v[:, sl].cpu(), dout[:, sl].cpu(), [windows[h]], ell,
            True, wl.video, query_rows=qrows, key_rows=keys if h == 1 else [])
        compare_grad(dq[:, sl][:, :, torch.from_numpy(qrows)], rq, f"dq ragged head {h}")
        if h == 1:
            compare_grad(dk[:, sl][:, :, torch.from_numpy(keys)], rk, "dk ragged head 1")
            compare_grad(dv[:, sl][:, :, torch.from_numpy(keys)], rv, "dv ragged head 1")
    del q, k, v, dout, out, lse, dq, dk, dv
    torch.cuda.empty_cache()
