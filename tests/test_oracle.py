"""Pins for the fp64 CPU oracle, checked against what the page and mathematics fix.

No GPU. Each pin is independent of the oracle's own code path:

* the page's printed window example ((3,3,3) tiles on the (30,48,80) video
  gives an (18,24,24) token box; golden fixture ``tests/golden/window_example.json``);
* per-query attended-key counts (window tokens plus text length);
* full-grid windows reduce to a library routine (torch SDPA in float64);
* a pure-Python brute force from the definition on tiny grids;
* the tile-block structure of the mask (no mixed blocks, "Why is STA Fast?");
* a closed form at q = 0 (uniform attention), which pins window placement;
* flip symmetry for odd windows and permutation invariance inside a tile;
* planted mistakes in the oracle (wrong window placement, transposed
  coordinates, wrong scale) must each be caught by one of these pins.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import sta_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TILE = (6, 8, 8)


# ---------------------------------------------------------------- helpers
def nearest_box_start(c, w, n):
    """Window placement from its characterisation, not from a formula.

    Among all placements [s, s+w) that fit in [0, n), take the one whose
    centre is nearest to the query tile c; ties go to the smaller start.
    """
    best = None
    for s in range(0, n - w + 1):
        d = abs(s + (w - 1) / 2.0 - c)
        if best is None or d < best[0]:
            best = (d, s)
    return best[1]


def raster_coords(i, video):
    T, H, W = video
    return i // (H * W), (i // W) % H, i % W


def rand_qkv(B, heads, S, D, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(B, heads, S, D, generator=g, dtype=torch.float32).to(torch.bfloat16)
            for _ in range(3)]


def seq_len(video, has_text):
    return video[0] * video[1] * video[2] + (256 if has_text else 0)


def brute_force(q, k, v, video, window, ell, has_text, rows):
    """Element-by-element attention from the definition, pure Python."""
    T, H, W = video
    nv = T * H * W
    S = seq_len(video, has_text)
    ntiles = [-(-video[a] // TILE[a]) for a in range(3)]  # partial last tiles included
    D = q.shape[-1]
    qd, kd, vd = q.double().tolist(), k.double().tolist(), v.double().tolist()

    def sees(i, j):
        if j >= nv:
            return (j - nv) < ell
        if i >= nv:
            return True
        ci, cj = raster_coords(i, video), raster_coords(j, video)
        for a in range(3):
            s = nearest_box_start(ci[a] // TILE[a], window[a], ntiles[a])
            if not (s <= cj[a] // TILE[a] < s + window[a]):
                return False
        return True

    outs, lses = [], []
    for i in rows:
        sc = []
        for j in range(S):
            if sees(i, j):
                sc.append((j, sum(qd[i][d] * kd[j][d] for d in range(D)) / math.sqrt(D)))
        mx = max(s for _, s in sc)
        wts = [(j, math.exp(s - mx)) for j, s in sc]
        tot = sum(w for _, w in wts)
        outs.append([sum(w * vd[j][d] for j, w in wts) / tot for d in range(D)])
        lses.append(mx + math.log(tot))
    return np.array(outs), np.array(lses)


# ---------------------------------------------------------------- pins
def test_page_window_example():
    """(3,3,3) tiles -> (18,24,24) tokens for every video query of (30,48,80)."""
    with open(os.path.join(GOLDEN, "window_example.json")) as f:
        g = json.load(f)
    video, window = tuple(g["video"]), tuple(g["window"])
    T, H, W = video
    n = [video[a] // TILE[a] for a in range(3)]
    # one query per tile (its first token) plus random tokens: border tiles included
    rows = []
    for tt in range(n[0]):
        for th in range(n[1]):
            for tw in range(n[2]):
                t, h, w = tt * 6, th * 8, tw * 8
                rows.append((t * H + h) * W + w)
    rng = np.random.default_rng(0)
    rows += list(rng.integers(0, T * H * W, 64))
    mask = oracle.allowed_mask(rows, video, window, 0, False)
    t = np.arange(T).repeat(H * W)
    h = np.tile(np.arange(H).repeat(W), T)
    w = np.tile(np.arange(W), T * H)
    for r in range(len(rows)):
        on = mask[r]
        assert on.sum() == g["video_keys_per_query"]
        extent = [int(x[on].max() - x[on].min() + 1) for x in (t, h, w)]
        assert extent == g["box_tokens"]
        # a box: the count equals the product of the extents
        assert np.prod(extent) == on.sum()


@pytest.mark.parametrize("video,window,ell,has_text", [
    ((18, 24, 24), (1, 3, 3), 0, False),
    ((18, 24, 32), (3, 1, 3), 77, True),
    ((12, 16, 40), (2, 2, 4), 256, True),
    ((18, 16, 24), (3, 2, 1), 0, True),
])
def test_attended_key_counts(video, window, ell, has_text):
    nv = video[0] * video[1] * video[2]
    S = seq_len(video, has_text)
    rows = np.arange(S)
    mask = oracle.allowed_mask(rows, video, window, ell, has_text)
    counts = mask.sum(axis=1)
    per_video = window[0] * window[1] * window[2] * 384 + ell
    assert (counts[:nv] == per_video).all()
    if has_text:
        assert (counts[nv:] == nv + ell).all()


@pytest.mark.parametrize("video,window,ell,has_text", [
    ((7, 9, 11), (1, 2, 1), 0, False),
    ((13, 8, 20), (2, 1, 2), 40, True),
    ((6, 17, 8), (1, 3, 1), 0, True),
    ((1, 10, 10), (1, 1, 2), 0, False),
])
def test_attended_key_counts_partial_tiles(video, window, ell, has_text):
    """Sizes that are not tile multiples: a video query sees, per axis, the tokens that
    exist in the span of its window's tiles (placement from the characterisation)."""
    nv = video[0] * video[1] * video[2]
    S = seq_len(video, has_text)
    n = [-(-video[a] // TILE[a]) for a in range(3)]
    rows = np.arange(S)
    counts = oracle.allowed_mask(rows, video, window, ell, has_text).sum(axis=1)
    for i in range(0, nv, 7):
        c = raster_coords(i, video)
        span = 1
        for a in range(3):
            st = nearest_box_start(c[a] // TILE[a], window[a], n[a])
            span *= min(video[a], (st + window[a]) * TILE[a]) - st * TILE[a]
        assert counts[i] == span + ell, (i, counts[i], span + ell)
    if has_text:
        assert (counts[nv:] == nv + ell).all()


@pytest.mark.parametrize("ell,has_text", [(0, False), (0, True), (100, True), (256, True)])
def test_full_window_is_sdpa(ell, has_text):
    """A window covering the whole tile grid is plain attention (key padding for text)."""
    video = (12, 16, 16)
    window = (2, 2, 2)
    B, heads, D = 2, 2, 16
    S = seq_len(video, has_text)
    nv = S - (256 if has_text else 0)
    q, k, v = rand_qkv(B, heads, S, D, 3)
    out, lse = oracle.sta_reference(q, k, v, [window] * heads, ell, has_text, video)
    keep = torch.ones(S, dtype=torch.bool)
    keep[nv + ell:] = False
    q64, k64, v64 = q.double(), k.double(), v.double()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q64, k64, v64, attn_mask=keep.expand(S, S))
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-10, atol=1e-12)
    scores = (q64 @ k64.transpose(-1, -2)) / math.sqrt(D)
    ref_lse = torch.logsumexp(scores[..., keep], dim=-1)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("video,window,ell,has_text,D", [
    ((6, 16, 16), (1, 1, 1), 3, True, 4),
    ((18, 16, 32), (3, 1, 3), 0, False, 3),
    ((18, 16, 32), (1, 2, 3), 5, True, 2),
    ((7, 9, 11), (1, 2, 1), 5, True, 3),
    ((13, 8, 20), (2, 1, 2), 0, False, 2),
    ((1, 12, 20), (1, 1, 2), 9, True, 2),
])
def test_brute_force_tiny(video, window, ell, has_text, D):
    S = seq_len(video, has_text)
    nv = video[0] * video[1] * video[2]
    q, k, v = rand_qkv(1, 1, S, D, 11)
    rng = np.random.default_rng(1)
    rows = sorted(set([0, nv - 1, nv // 2] + list(rng.integers(0, S, 12))
                      + ([nv, S - 1, nv + ell] if has_text else [])))
    rows = [r for r in rows if r < S]
    out, lse = oracle.sta_reference(q, k, v, [window], ell, has_text, video, rows=rows)
    bo, bl = brute_force(q[0, 0], k[0, 0], v[0, 0], video, window, ell, has_text, rows)
    np.testing.assert_allclose(out[0, 0], bo, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], bl, rtol=1e-12, atol=1e-12)


def tile_major_perm(video):
    """Video positions listed tile by tile (tile raster order, then in-tile raster)."""
    T, H, W = video
    n = [video[a] // TILE[a] for a in range(3)]
    order = []
    for tt in range(n[0]):
        for th in range(n[1]):
            for tw in range(n[2]):
                for dt in range(6):
                    for dh in range(8):
                        for dw in range(8):
                            t, h, w = tt * 6 + dt, th * 8 + dh, tw * 8 + dw
                            order.append((t * H + h) * W + w)
    return np.array(order)


@pytest.mark.parametrize("video,window,ell", [
    ((6, 8, 8), (1, 1, 1), 0),
    ((12, 16, 16), (1, 2, 1), 1),
    ((18, 24, 24), (3, 3, 3), 127),
    ((18, 24, 24), (2, 1, 3), 128),
    ((18, 24, 24), (1, 3, 2), 255),
    ((12, 24, 16), (2, 2, 2), 256),
])
def test_no_mixed_blocks(video, window, ell):
    """In tile-major order every (query tile, key tile) block is all-on or all-off."""
    nv = video[0] * video[1] * video[2]
    S = nv + 256
    mask = oracle.allowed_mask(np.arange(S), video, window, ell, True)
    perm = tile_major_perm(video)
    nt = nv // 384
    vv = mask[perm][:, perm].reshape(nt, 384, nt, 384)
    on = vv.all(axis=(1, 3))
    off = ~vv.any(axis=(1, 3))
    assert (on | off).all()
    assert on.sum(axis=1).tolist() == [window[0] * window[1] * window[2]] * nt
    # video queries x text keys: the same valid-prefix pattern on every row
    text_cols = mask[:nv, nv:]
    assert (text_cols == (np.arange(256) < ell)[None, :]).all()


@pytest.mark.parametrize("video,window,ell,has_text", [
    ((18, 24, 32), (3, 1, 3), 0, False),
    ((18, 24, 32), (1, 3, 1), 40, True),
    ((30, 16, 24), (3, 2, 3), 200, True),
    ((12, 24, 40), (1, 3, 5), 256, True),
])
def test_uniform_attention_closed_form(video, window, ell, has_text):
    """q = 0: every score is 0, so lse = ln(count) and out = mean of the allowed v rows.

    v carries each key's tile coordinates (exact in bf16), so the output of a
    video query is the centre of its window, scaled by the video share of
    the attended keys; this pins the window placement.
    """
    T, H, W = video
    nv = T * H * W
    S = seq_len(video, has_text)
    n = [video[a] // TILE[a] for a in range(3)]
    q = torch.zeros(1, 1, S, 4)
    k = torch.randn(1, 1, S, 4, generator=torch.Generator().manual_seed(5))
    v = torch.zeros(1, 1, S, 4)
    for i in range(nv):
        t, h, w = raster_coords(i, video)
        v[0, 0, i, :3] = torch.tensor([t // 6, h // 8, w // 8], dtype=torch.float32)
    v[0, 0, nv:, 3] = 1.0
    rng = np.random.default_rng(2)
    rows = sorted(set(list(rng.integers(0, nv, 40)) + [0, nv - 1]
                      + ([nv, S - 1] if has_text else [])))
    out, lse = oracle.sta_reference(q, k, v, [window], ell, has_text, video, rows=rows)
    nwin = window[0] * window[1] * window[2] * 384
    for r, i in enumerate(rows):
        if i < nv:
            count = nwin + ell
            c = raster_coords(i, video)
            centre = [nearest_box_start(c[a] // TILE[a], window[a], n[a]) + (window[a] - 1) / 2
                      for a in range(3)]
            expect = [x * nwin / count for x in centre] + [ell / count]
        else:
            count = nv + ell
            expect = [(n[a] - 1) / 2 * nv / count for a in range(3)] + [ell / count]
        assert lse[0, 0, r] == pytest.approx(math.log(count), abs=1e-12)
        np.testing.assert_allclose(out[0, 0, r], expect, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_flip_symmetry(axis):
    video = (18, 16, 24)
    window = (3, 1, 3)
    ell = 50
    nv = video[0] * video[1] * video[2]
    S = nv + 256
    q, k, v = rand_qkv(1, 1, S, 8, 21)

    def flip(x):
        vid = x[:, :, :nv].reshape(1, 1, *video, -1).flip(2 + axis).reshape(1, 1, nv, -1)
        return torch.cat([vid, x[:, :, nv:]], dim=2)

    out, lse = oracle.sta_reference(q, k, v, [window], ell, True, video)
    fo, fl = oracle.sta_reference(flip(q), flip(k), flip(v), [window], ell, True, video)
    np.testing.assert_allclose(flip(torch.from_numpy(out)).numpy(), fo, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(flip(torch.from_numpy(lse[..., None])).numpy()[..., 0], fl,
                               rtol=1e-12, atol=1e-12)


def test_in_tile_permutation_and_heads():
    """Permuting tokens inside every tile (same for q, k, v) permutes the output;
    heads and batch entries are independent."""
    video = (12, 16, 16)
    nv = video[0] * video[1] * video[2]
    S = nv + 256
    windows = [(1, 1, 2), (2, 2, 1)]
    q, k, v = rand_qkv(2, 2, S, 8, 31)
    out, lse = oracle.sta_reference(q, k, v, windows, 17, True, video)
    perm = tile_major_perm(video)
    rng = np.random.default_rng(3)
    new = np.arange(S)
    for tile in range(nv // 384):
        seg = perm[tile * 384:(tile + 1) * 384]
        new[seg] = seg[rng.permutation(384)]
    pq, pk, pv = q[:, :, new], k[:, :, new], v[:, :, new]
    po, pl = oracle.sta_reference(pq, pk, pv, windows, 17, True, video)
    np.testing.assert_allclose(po, out[:, :, new], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(pl, lse[:, :, new], rtol=1e-12, atol=1e-12)
    o1, l1 = oracle.sta_reference(q[1:, 1:], k[1:, 1:], v[1:, 1:], windows[1:], 17, True, video)
    np.testing.assert_allclose(o1, out[1:, 1:], rtol=1e-12, atol=1e-14)


def test_key_tiles_from_mask_match_box():
    video = (30, 48, 80)
    n = (5, 6, 10)
    for window in [(3, 3, 3), (1, 6, 10), (5, 1, 1), (2, 4, 3)]:
        for qt in [0, 7, 59, 123, 299]:
            tiles = oracle.key_tiles_of_query_tile(video, window, qt)
            tt, rem = divmod(qt, n[1] * n[2])
            th, tw = divmod(rem, n[2])
            s = [nearest_box_start(c, w, m) for c, w, m in zip((tt, th, tw), window, n)]
            expect = sorted((a * n[1] + b) * n[2] + c
                            for a in range(s[0], s[0] + window[0])
                            for b in range(s[1], s[1] + window[1])
                            for c in range(s[2], s[2] + window[2]))
            assert tiles == expect


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.allowed_mask([0], (0, 8, 8), (1, 1, 1), 0, False)
    with pytest.raises(ValueError):
        oracle.allowed_mask([0], (6, 8, 8), (2, 1, 1), 0, False)
    with pytest.raises(ValueError):
        oracle.allowed_mask([0], (6, 8, 8), (1, 1, 1), 3, False)
    with pytest.raises(ValueError):
        oracle.allowed_mask([0], (6, 8, 8), (1, 1, 1), 257, True)


# ------------------------------------------------- planted mistakes are caught
def _counts_pin_holds():
    video, window = (18, 24, 32), (3, 3, 3)
    rows = np.arange(video[0] * video[1] * video[2])[::37]
    mask = oracle.allowed_mask(rows, video, window, 0, False)
    return bool((mask.sum(axis=1) == 27 * 384).all())


def _closed_form_pin_holds():
    try:
        test_uniform_attention_closed_form((18, 24, 32), (1, 3, 1), 40, True)
        return True
    except AssertionError:
        return False


def _sdpa_pin_holds():
    try:
        test_full_window_is_sdpa(100, True)
        return True
    except AssertionError:
        return False


@pytest.mark.parametrize("mutant", [
    "truncate", "off_by_one", "no_upper_clamp_shift", "swap_hw", "scale_1_over_d",
])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    if mutant == "truncate":
        # window cut at the border instead of shifted
        monkeypatch.setattr(so, "window_start", lambda c, w, n: c - w // 2)
    elif mutant == "off_by_one":
        monkeypatch.setattr(so, "window_start", lambda c, w, n: min(max(c - w // 2 - 1, 0), n - w))
    elif mutant == "no_upper_clamp_shift":
        monkeypatch.setattr(so, "window_start", lambda c, w, n: max(c - w // 2, 0))
    elif mutant == "swap_hw":
        # key coordinates read as if h, not w, were the fastest raster axis
        def swapped(video):
            T, H, W = video
            t = np.arange(T).repeat(H * W)
            i = np.arange(T * H * W) % (H * W)
            return t // 6, (i % H) // 8, (i // H) // 8
        monkeypatch.setattr(so, "_video_tile_coords", swapped)
    elif mutant == "scale_1_over_d":
        monkeypatch.setattr(so, "softmax_scale", lambda d: 1.0 / d)
    caught = not (_counts_pin_holds() and _closed_form_pin_holds() and _sdpa_pin_holds())
    assert caught, f"mutant {mutant} slipped through every pin"
