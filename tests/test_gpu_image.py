"""GPU parity (through the C ABI) of STA on one-frame videos (2D images) run
with query units of 2x2 squares of tiles.

Reading (the page's 2D STA names no tile size): a 2D image is a video of one
frame, so each (6, 8, 8) tile holds one frame of at most 8x8 tokens (fewer
in the last tile row or column when H or W is not a multiple of 8). When every
head's window spans at least two tiles along each axis that has two tile
rows (columns), the forward groups the query tiles in 2x2 squares; the
blocks on the edge of the four windows' union are seen by only some of the
square's tiles, and the text rows are split over several units by key tiles
on images of 256 tiles or more. The oracle (dense masked attention over an
explicit token mask) knows nothing of this; here the HIP forward is compared
with it on every row of small images and on sampled rows of larger ones.
Outputs start as NaN, so a row the kernel skips fails the checks, and padded
text K/V hold NaN on the GPU side, so a padded key that reaches a result
fails them too.

Source: Sliding Tile Attention README, "Usage" (windows in tiles, text slots)
and "How Does STA Work?" (2D STA on an image).
"""

import numpy as np
import pytest
import torch

import block_sparse_sliding_amd as sta
import oracle
from _parity import compare, note, oracle_rows, run_sta, scale_key_tiles
from test_gpu_backward import compare_grad, run_backward

pytestmark = pytest.mark.gpu

CASES = [
    # (B, D, image (H, W), windows (wh, ww) per head, text_length, has_text)
    (1, 128, (64, 64), [(5, 5), (2, 3)], 226, True),     # 8x8 tiles, windows clamped at the border
    (1, 64, (72, 88), [(3, 4)], 0, False),               # 9x11 tiles: squares of 2 and 1 tiles, even window
    (2, 128, (40, 48), [(2, 2), (5, 6)], 100, True),     # the smallest window, and the whole grid
    (1, 128, (8, 96), [(1, 5)], 17, True),               # one tile row
    (1, 64, (96, 8), [(6, 1), (3, 1)], 0, False),        # one tile column
    (1, 128, (24, 24), [(3, 3)], 256, True),             # 3x3 tiles, window = grid, every text slot valid
    (1, 128, (56, 40), [(4, 2), (7, 5)], 1, True),       # 7x5 tiles
    (1, 128, (100, 100), [(6, 6), (3, 2)], 64, True),    # 13x13 tiles, last row and column 4 wide
    (1, 64, (44, 30), [(3, 2)], 0, False),               # partial tiles along both axes
    (2, 128, (90, 40), [(5, 5)], 226, True),             # a last tile row 2 rows high
    (1, 128, (5, 100), [(1, 4)], 10, True),              # one partial tile row
]
IDS = [f"i{i}" for i in range(len(CASES))]


def inputs(seed, B, heads, S, D):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return [torch.randn(B, heads, S, D, generator=g, device="cuda").to(torch.bfloat16) for _ in range(3)]


def run_nan_padded(q, k, v, windows, ell, has_text, video):
    """The GPU call on copies of k and v whose padded text slots hold NaN."""
    nv = video[0] * video[1] * video[2]
    if has_text and ell < 256:
        k, v = k.clone(), v.clone()
        k[:, :, nv + ell:] = float("nan")
        v[:, :, nv + ell:] = float("nan")
    return run_sta(q, k, v, windows, ell, has_text, video)


def square_units(video, windows, has_text):
    """Video query units per head the forward plans: 2x2 squares, or None."""
    T, H, W = video
    nh, nw = -(-H // 8), -(-W // 8)
    ok = T == 1 and (nh > 1 or nw > 1) and \
        all((w[1] >= 2 or nh == 1) and (w[2] >= 2 or nw == 1) for w in windows)
    return ((nh + 1) // 2) * ((nw + 1) // 2) if ok else None


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_square_units_all_rows(case):
    B, D, (H, W), hw, ell, has_text = case
    video = (1, H, W)
    windows = [(1, a, b) for a, b in hw]
    assert square_units(video, windows, has_text) is not None
    S = H * W + (256 if has_text else 0)
    note(f"square units forward {case}")
    q, k, v = inputs(5000 + S + D, B, len(windows), S, D)
    out, lse = run_nan_padded(q, k, v, windows, ell, has_text, video)
    ro, rl = oracle_rows(q, k, v, windows, ell, has_text, video)
    compare(out, lse, ro, rl, label=f"squares {case}")


def test_square_units_score_jumps_redo():
    """Key tiles scaled by large, uneven factors (edge tiles of the squares'
    windows among them): scores jump by tens of log2 units between blocks,
    which triggers the redo pass; rows that do not see an edge block must keep
    it out of their maximum."""
    H = W = 64
    video, windows, ell = (1, H, W), [(1, 3, 3), (1, 2, 5)], 150
    S = H * W + 256
    note("square units forward, score jumps")
    q, k, v = inputs(77, 1, 2, S, 128)
    factors = {(0, th, tw): (8.0 if (th * 3 + tw) % 5 == 2 else 1.0) for th in range(8) for tw in range(8)}
    k = scale_key_tiles(k, video, factors, 5.0, ell)
    out, lse = run_nan_padded(q, k, v, windows, ell, True, video)
    ro, rl = oracle_rows(q, k, v, windows, ell, True, video)
    compare(out, lse, ro, rl, label="squares score jumps")


@pytest.mark.parametrize("side,D,windows,ell", [
    (128, 128, [(1, 5, 7), (1, 2, 2)], 226),   # 256 tiles: text rows in 2 parts
    (256, 64, [(1, 3, 3)], 1),                 # 1024 tiles: 8 parts, one valid text slot
], ids=["2-parts", "8-parts"])
def test_square_units_split_text_sampled(side, D, windows, ell):
    """Images of 256 tiles or more: the text rows are split over several
    units by key tiles and merged. Every text row, the image corners and a
    seeded uniform draw of video rows are compared with the oracle."""
    video = (1, side, side)
    S = side * side + 256
    note(f"square units forward, split text, {side}x{side}")
    q, k, v = inputs(91 + side, 1, len(windows), S, D)
    out, lse = run_nan_padded(q, k, v, windows, ell, True, video)
    rng = np.random.default_rng(side)
    fixed = [0, side - 1, side * (side - 1), side * side - 1]
    rows = np.unique(np.concatenate([fixed, rng.integers(0, side * side, 600), np.arange(side * side, S)]))
    ro, rl = oracle_rows(q, k, v, windows, ell, True, video, rows=rows)
    compare(out, lse, ro, rl, rows=torch.as_tensor(rows, device="cuda"), label=f"squares split text {side}")


def test_square_units_padding_isolation_bitwise():
    """Padded text K/V of any value (here large finite values, then NaN) leave
    out and lse bit for bit unchanged."""
    video, windows, ell = (1, 48, 64), [(1, 3, 3)], 100
    S = 48 * 64 + 256
    note("square units forward, padding isolation")
    q, k, v = inputs(123, 1, 1, S, 128)
    base_o, base_l = run_sta(q, k, v, windows, ell, True, video)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, 48 * 64 + ell:] = 100.0
    v2[:, :, 48 * 64 + ell:] = 1e4
    o2, l2 = run_sta(q, k2, v2, windows, ell, True, video)
    o3, l3 = run_nan_padded(q, k, v, windows, ell, True, video)
    for o, l in ((o2, l2), (o3, l3)):
        assert torch.equal(o.view(torch.int16), base_o.view(torch.int16))
        assert torch.equal(l.view(torch.int32), base_l.view(torch.int32))


def test_square_units_noalloc_matches():
    """sta_forward_noalloc takes the same square units (with the text rows
    kept whole when its scratch cannot hold the split's partial results) and
    matches sta_forward within the parity tolerances, and bit for bit where
    the text rows are not split."""
    video, windows, ell = (1, 256, 256), [(1, 3, 3)], 64
    S = 256 * 256 + 256
    note("square units forward, noalloc")
    q, k, v = inputs(7, 1, 2, S, 128)
    windows = windows * 2
    o1, l1 = run_sta(q, k, v, windows, ell, True, video)
    dims = sta.make_dims(1, 2, 128, video)
    o2 = torch.full_like(q, float("nan"))
    l2 = torch.full((1, 2, S), float("nan"), dtype=torch.float32, device="cuda")
    sta.sta_forward_noalloc(dims, q, k, v, windows, ell, True, o2, l2)
    torch.cuda.synchronize()
    nv = 256 * 256
    assert torch.equal(o1[:, :, :nv].view(torch.int16), o2[:, :, :nv].view(torch.int16))
    assert torch.equal(l1[:, :, :nv].view(torch.int32), l2[:, :, :nv].view(torch.int32))
    rows = np.arange(nv, S)
    ro, rl = oracle_rows(q, k, v, windows, ell, True, video, rows=rows)
    compare(o2, l2, ro, rl, rows=torch.as_tensor(rows, device="cuda"), label="squares noalloc text")


BWD_CASES = [
    # (B, D, image (H, W), windows (wh, ww) per head, text_length, has_text)
    (1, 128, (64, 64), [(5, 5), (2, 3)], 226, True),
    (1, 64, (72, 88), [(3, 4)], 0, False),
    (1, 128, (100, 100), [(6, 6)], 64, True),     # partial last tile row and column
    (2, 128, (44, 30), [(3, 2)], 17, True),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[f"b{i}" for i in range(len(BWD_CASES))])
def test_square_units_backward_all_rows(case):
    """The backward on one-frame videos: the dq pass runs 2x2-square query
    units and the dk/dv pass 2x2-square key units (waves skip the blocks their
    tile does not see); every gradient row against the oracle's."""
    B, D, (H, W), hw, ell, has_text = case
    video = (1, H, W)
    windows = [(1, a, b) for a, b in hw]
    assert square_units(video, windows, has_text) is not None
    S = H * W + (256 if has_text else 0)
    note(f"square units backward {case}")
    q, k, v, dout = inputs(7000 + S + D, B, len(windows), S, D) + inputs(7001 + S, B, len(windows), S, D)[:1]
    out, lse = run_sta(q, k, v, windows, ell, has_text, video)
    dq, dk, dv = run_backward(q, k, v, out, lse, dout, windows, ell, has_text, video)
    rq, rk, rv = oracle.sta_reference_backward(q.cpu(), k.cpu(), v.cpu(), dout.cpu(), windows, ell,
                                               has_text, video)
    compare_grad(dq, rq, f"dq {case}")
    compare_grad(dk, rk, f"dk {case}")
    compare_grad(dv, rv, f"dv {case}")
