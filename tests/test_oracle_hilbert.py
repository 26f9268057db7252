"""Pins of the Hilbert oracle (CPU): the curve, its tile-level order, the window
patterns and the block statistics, each checked against a property fixed by
the curve's definition or by the mathematics, not by re-running its code.

Source: the blog post "Boosting 2D Local Attention Efficiency with
Hilbert-Guided Sparsity" ("TLDR", "The Hilbert Curve Advantage"); the
orientation and the window readings are stated in the oracle's header.
"""

import numpy as np
import pytest
import torch

from oracle import hilbert_oracle as H


def curve(order):
    return [H.hilbert_d2xy(order, d) for d in range(1 << (2 * order))]


@pytest.mark.parametrize("order", range(0, 7))
def test_curve_is_a_bijection_and_inverse(order):
    pts = curve(order)
    n = 1 << order
    assert sorted(pts) == [(x, y) for x in range(n) for y in range(n)]
    assert all(H.hilbert_xy2d(order, x, y) == d for d, (x, y) in enumerate(pts))


@pytest.mark.parametrize("order", range(1, 7))
def test_consecutive_cells_are_neighbours(order):
    pts = np.array(curve(order))
    steps = np.abs(np.diff(pts, axis=0)).sum(axis=1)
    assert (steps == 1).all()


@pytest.mark.parametrize("order", range(1, 7))
def test_endpoints(order):
    n = 1 << order
    assert H.hilbert_d2xy(order, 0) == (0, 0)
    assert H.hilbert_d2xy(order, n * n - 1) == (n - 1, 0)


@pytest.mark.parametrize("order", range(1, 7))
def test_every_aligned_run_is_a_square(order):
    """Positions [q 4^j, (q + 1) 4^j) fill one aligned 2^j x 2^j square, at every scale."""
    pts = np.array(curve(order))
    for j in range(order + 1):
        run = 1 << (2 * j)
        side = 1 << j
        for q in range(len(pts) // run):
            blk = pts[q * run:(q + 1) * run]
            lo = blk.min(axis=0)
            assert (blk.max(axis=0) - lo == side - 1).all()
            assert (lo % side == 0).all()


def test_quadrant_order_of_the_definition():
    """Order k visits (x low, y low), (x low, y high), (x high, y high), (x high, y low)."""
    for order in range(1, 6):
        half = 1 << (order - 1)
        pts = np.array(curve(order))
        quads = [(int(x >= half), int(y >= half)) for x, y in pts[::half * half]]
        assert quads == [(0, 0), (0, 1), (1, 1), (1, 0)]


def planted(kind):
    """A copy of the oracle's d2xy with one plausible mistake in a quadrant transform."""
    def d2xy(order, d):
        if order == 0:
            return 0, 0
        half = 1 << (order - 1)
        quad, rest = divmod(d, half * half)
        x, y = d2xy(order - 1, rest)
        if quad == 0:
            return (x, y) if kind == "no_transpose" else (y, x)
        if quad == 1:
            return x, y + half
        if quad == 2:
            return x + half, y + half
        if kind == "plain_shift":
            return x + half, y
        if kind == "off_by_one":
            return 2 * half - y, half - 1 - x
        return 2 * half - 1 - y, half - 1 - x
    return d2xy


@pytest.mark.parametrize("kind", ["no_transpose", "plain_shift", "off_by_one"])
def test_pins_catch_planted_mistakes(kind):
    f = planted(kind)
    order = 3
    n = 1 << order
    pts = np.array([f(order, d) for d in range(n * n)])
    ok_bij = sorted(map(tuple, pts)) == [(x, y) for x in range(n) for y in range(n)]
    ok_adj = (np.abs(np.diff(pts, axis=0)).sum(axis=1) == 1).all()
    ok_end = tuple(pts[-1]) == (n - 1, 0)
    assert not (ok_bij and ok_adj and ok_end)


@pytest.mark.parametrize("m", [0, 1, 2, 3])
def test_token_blocks_are_tiles_in_tile_curve_order(m):
    """Tokens [64 i, 64 i + 64) of the image curve are the 8x8 tile at tile-curve position i."""
    side = 8 << m
    perm = H.hilbert_token_order((side, side))
    assert sorted(perm) == list(range(side * side))
    y, x = np.divmod(perm, side)
    for i in range(1 << (2 * m)):
        tx, ty = H.hilbert_d2xy(m, i)
        blk = slice(64 * i, 64 * i + 64)
        assert set(zip(x[blk] // 8, y[blk] // 8)) == {(tx, ty)}


@pytest.mark.parametrize("m,j", [(2, 0), (2, 1), (2, 2), (3, 1), (3, 2)])
def test_window_mode_of_4_to_the_j_tiles_is_the_aligned_square(m, j):
    """W = 4^j: the window of a query tile is the aligned 2^j x 2^j square of tiles holding it."""
    side = 8 << m
    W = 1 << (2 * j)
    rows = np.arange(0, side * side, 37)
    mask = H.hilbert_allowed_mask(rows, (side, side), W, "window", 0, False)
    ky, kx = np.divmod(np.arange(side * side), side)
    sq = 8 << j
    for r, t in enumerate(rows):
        y, x = divmod(int(t), side)
        expect = (kx // sq == x // sq) & (ky // sq == y // sq)
        assert np.array_equal(mask[r], expect)


@pytest.mark.parametrize("mode", ["slide", "window"])
def test_window_counts_and_extremes(mode):
    side, m = 32, 2
    n = 16
    rows = list(range(0, side * side, 13)) + [side * side, side * side + 255]
    for W in (1, 3, 4, 5, n):
        mask = H.hilbert_allowed_mask(rows, (side, side), W, mode, 100, True)
        for r, t in enumerate(rows):
            if t < side * side:
                y, x = divmod(t, side)
                i = H.hilbert_xy2d(m, x // 8, y // 8)
                cnt = W if mode == "slide" else min(W, n - W * (i // W))
                assert mask[r, :side * side].sum() == 64 * cnt
                assert mask[r, side * side:].sum() == 100
                # the query's own tile is always in its window
                own = (np.arange(side * side) // side // 8 == y // 8) & (np.arange(side * side) % side // 8 == x // 8)
                assert mask[r, :side * side][own].all()
            else:
                assert mask[r].sum() == side * side + 100
    full = H.hilbert_allowed_mask(range(side * side), (side, side), n, mode, 0, False)
    assert full.all()
    one = H.hilbert_allowed_mask(range(side * side), (side, side), 1, mode, 0, False)
    y, x = np.divmod(np.arange(side * side), side)
    tile = (y // 8) * 4 + x // 8
    assert np.array_equal(one, tile[:, None] == tile[None, :])


def test_slide_window_is_centred_and_clamped():
    n = 16
    assert H.window_span(0, 5, n, "slide") == (0, 5)
    assert H.window_span(7, 5, n, "slide") == (5, 5)
    assert H.window_span(15, 5, n, "slide") == (11, 5)
    assert H.window_span(7, 4, n, "slide") == (5, 4)
    assert H.window_span(13, 4, n, "window") == (12, 4)
    assert H.window_span(13, 5, n, "window") == (10, 5)
    assert H.window_span(15, 5, n, "window") == (15, 1)


def test_reference_q_zero_closed_form():
    """q = 0: every allowed key weighs the same, so out = mean of the allowed v and lse = ln(count)."""
    side, heads, D = 16, 2, 8
    g = torch.Generator().manual_seed(3)
    S = side * side + 256
    q = torch.zeros(1, heads, S, D, dtype=torch.float64)
    k = torch.randn(1, heads, S, D, generator=g, dtype=torch.float64)
    v = torch.randn(1, heads, S, D, generator=g, dtype=torch.float64)
    rows = [0, 17, 100, 255, 256, 300]
    out, lse = H.hilbert_reference(q, k, v, [1, 3], "slide", 40, True, (side, side), rows=rows)
    for h, W in enumerate([1, 3]):
        mask = H.hilbert_allowed_mask(rows, (side, side), W, "slide", 40, True)
        for r in range(len(rows)):
            sel = v[0, h, mask[r]].numpy()
            assert np.allclose(out[0, h, r], sel.mean(axis=0), atol=1e-12)
            assert np.isclose(lse[0, h, r], np.log(mask[r].sum()), atol=1e-12)


def test_reference_equals_torch_masked_attention():
    side, heads, D = 16, 1, 16
    g = torch.Generator().manual_seed(5)
    S = side * side + 256
    q, k, v = (torch.randn(1, heads, S, D, generator=g, dtype=torch.float64) for _ in range(3))
    mask = torch.from_numpy(H.hilbert_allowed_mask(range(S), (side, side), 2, "window", 77, True))
    expect = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask)
    out, _ = H.hilbert_reference(q, k, v, 2, "window", 77, True, (side, side))
    assert np.allclose(out, expect.numpy(), atol=1e-10)


def test_block_counts_square_windows_no_partial_in_hilbert_order():
    """Aligned 8x8 windows are 64 consecutive tokens on the curve: no partial block at all;
    in raster order they split every block."""
    side = 64
    mask = H.square_window_mask(side, 8)
    hil = H.block_counts(mask, H.hilbert_token_order((side, side)))
    ras = H.block_counts(mask, np.arange(side * side))
    assert hil == {"blocks": 4096, "empty": 4096 - 64, "full": 64, "partial": 0}
    assert ras["partial"] > 0 and ras["full"] == 0
    assert ras["blocks"] == hil["blocks"]


def test_block_counts_brute_force():
    mask = np.zeros((128, 128), dtype=bool)
    mask[:64, :64] = True          # one full block
    mask[70, 10] = True            # one partial block
    c = H.block_counts(mask, np.arange(128))
    assert c == {"blocks": 4, "empty": 2, "full": 1, "partial": 1}
