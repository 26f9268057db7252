"""Host code and index helpers under AddressSanitizer and UndefinedBehaviorSanitizer.

``tests/host/sta_host_checks.cpp`` is compiled here, with the host C++
compiler, together with the library's host source (argument validation,
geometry, workspace carving, the launch sequence); the kernel launchers are
recording stubs, so no GPU and no HIP runtime are involved. Its ``validate``
mode checks every argument error and that valid calls hand the kernels only
the caller's tensors and workspace regions. Its ``dump`` mode prints the index
helpers the kernels share with the host (window placement, tile extents,
blocks per window box, the tile-major to raster row map) for one geometry;
the tests below compare them with maps built from the oracle's token
coordinates (``oracle.window_start``, ``oracle.key_tiles_of_query_tile``,
token counts per tile from the oracle's coordinate map).
"""

from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from oracle import sta_oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_SRC = os.path.join(ROOT, "block_sparse_sliding_amd", "csrc", "sta_api" + ".hip")
CHECKS_SRC = os.path.join(ROOT, "tests", "host", "sta_host_checks.cpp")
SANITIZERS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
CXX_FLAGS = ["-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]
TILE = (6, 8, 8)


@pytest.fixture(scope="module")
def checks_bin(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path_factory.mktemp("host_checks") / "sta_host_checks"
    # the host source is compiled as plain C++ (its HIP calls are stubbed)
    sources = ["-x", "c++", HOST_SRC, "-x", "none", CHECKS_SRC]
    cmd = [cxx, *CXX_FLAGS, *SANITIZERS, *sources, "-o", str(exe)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    return str(exe)


def run(exe, *args):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe, *map(str, args)], stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                       text=True, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def test_validation_and_launch_sequence(checks_bin):
    out = run(checks_bin, "validate")
    assert out.startswith("ok "), out
    assert int(out.split()[1]) > 500


SHAPES = [
    # B, heads, D, video, has_text, ell, window
    (1, 1, 64, (18, 24, 24), 0, 0, (1, 3, 3)),
    (1, 24, 128, (30, 48, 80), 1, 226, (3, 3, 3)),
    (1, 24, 128, (30, 48, 80), 1, 256, (5, 6, 10)),
    (1, 24, 128, (33, 45, 80), 1, 226, (3, 3, 3)),
    (1, 24, 128, (48, 72, 128), 1, 128, (3, 3, 3)),
    (2, 3, 128, (7, 9, 11), 1, 50, (2, 2, 2)),
    (1, 2, 128, (17, 21, 30), 1, 77, (2, 3, 2)),
    (1, 2, 64, (13, 8, 20), 0, 0, (3, 1, 3)),
    (1, 1, 128, (20, 30, 45), 1, 100, (3, 2, 4)),
    (1, 2, 128, (1, 128, 128), 0, 0, (1, 5, 5)),
    (1, 2, 128, (1, 100, 100), 1, 33, (1, 6, 6)),
    (3, 5, 128, (1, 1, 1), 1, 256, (1, 1, 1)),
    (1, 1, 128, (6, 8, 8), 1, 17, (1, 1, 1)),
    (1, 1, 64, (5, 7, 9), 0, 0, (1, 1, 2)),
]


def oracle_maps(video):
    """Tile id of every raster video row and tokens per tile, from the oracle's
    token coordinates."""
    n = sta_oracle._check_video(video)
    kt, kh, kw = sta_oracle._video_tile_coords(video)
    tile = (kt * n[1] + kh) * n[2] + kw
    return n, tile, np.bincount(tile, minlength=n[0] * n[1] * n[2])


def forward_units(video, win, text):
    """Query units per head of the forward: single tiles (plus one text unit),
    or, on a one-frame video whose window spans at least
    two tiles along each axis with two or more tiles, 2x2 squares of tiles
    plus the text rows split into min(8, max(1, tiles // 128)) parts."""
    T, H, W = video
    nh, nw = -(-H // 8), -(-W // 8)
    n_tiles = -(-T // 6) * nh * nw
    if T == 1 and (nh > 1 or nw > 1) and (win[1] >= 2 or nh == 1) and (win[2] >= 2 or nw == 1):
        parts = min(8, max(1, n_tiles // 128)) if text else 0
        return ((nh + 1) // 2) * ((nw + 1) // 2) + parts
    return n_tiles + text


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[3]}w{s[6]}t{s[5] if s[4] else '-'}"
                                               for s in SHAPES])
def test_helpers_match_oracle_maps(checks_bin, shape):
    B, heads, D, video, text, ell, win = shape
    T, H, W = video
    out = run(checks_bin, "dump", B, heads, D, T, H, W, text, ell, *win).splitlines()
    n, tile_of_row, tokens = oracle_maps(video)
    nv = T * H * W
    n_tiles = int(np.prod(n))
    S = nv + (256 if text else 0)
    S_t = n_tiles * 384 + (256 if text else 0)

    sizes = [int(x) for x in out[0].split()[1:]]
    assert sizes == [S, S_t, heads * (n_tiles + text) + 1,
                     heads * (n_tiles * win[0] * win[1] * win[2] + (n_tiles if text else 0)),
                     B * heads * (n_tiles + text)]
    geom = [int(x) for x in out[1].split()[1:]]
    assert geom == [*n, n_tiles, nv, S, n_tiles * 384, S_t, int(n_tiles * 384 == nv),
                    forward_units(video, win, text), ell]

    ws = [ln for ln in out if ln.startswith("ws ")]
    assert len(ws) == sum(m * m for m in n)
    for ln in ws:
        ax, w, c, start = (int(x) for x in ln.split()[1:])
        assert start == oracle.window_start(c, w, n[ax]), ln

    tiles = [ln for ln in out if ln.startswith("tile ")]
    assert len(tiles) == n_tiles
    t_of = np.arange(T) // TILE[0]
    h_of = np.arange(H) // TILE[1]
    w_of = np.arange(W) // TILE[2]
    for ln in tiles:
        t, frames, rows, cols, tok, blocks = (int(x) for x in ln.split()[1:])
        tt, rest = divmod(t, n[1] * n[2])
        th, tw = divmod(rest, n[2])
        assert (frames, rows, cols) == (int((t_of == tt).sum()), int((h_of == th).sum()),
                                        int((w_of == tw).sum())), ln
        assert tok == tokens[t], ln
        # the window box of this query tile, placed by the oracle, in 64-token blocks
        box = [(a, b, c) for a in range(oracle.window_start(tt, win[0], n[0]),
                                         oracle.window_start(tt, win[0], n[0]) + win[0])
               for b in range(oracle.window_start(th, win[1], n[1]),
                              oracle.window_start(th, win[1], n[1]) + win[1])
               for c in range(oracle.window_start(tw, win[2], n[2]),
                              oracle.window_start(tw, win[2], n[2]) + win[2])]
        ids = [(a * n[1] + b) * n[2] + c for a, b, c in box]
        assert blocks == sum(-(-int(tokens[i]) // 64) for i in ids), ln
        if n_tiles <= 40:
            # the box is exactly the set of key tiles the oracle's mask reaches
            assert sorted(ids) == oracle.key_tiles_of_query_tile(video, win, t), ln
    grid = int(next(ln for ln in out if ln.startswith("grid ")).split()[1])
    assert grid == sum(-(-int(x) // 64) for x in tokens)

    # tile-major rows: tile t owns rows 384 t ..; its tokens come first, in raster
    # order (frame, row, column), then padding (-1); text rows follow the video
    t2r = np.array([int(x) for x in out[out.index(next(ln for ln in out if ln.startswith("grid "))) + 1:]])
    assert len(t2r) == S_t
    expect = np.full(S_t, -1, dtype=np.int64)
    order = np.argsort(tile_of_row, kind="stable")  # raster order inside each tile
    starts = np.concatenate([[0], np.cumsum(tokens)[:-1]])
    rank = np.arange(nv) - starts[tile_of_row[order]]
    expect[384 * tile_of_row[order] + rank] = order
    if text:
        expect[n_tiles * 384:] = nv + np.arange(256)
    assert np.array_equal(t2r, expect)


STREAM_SHAPES = [
    # video, has_text, ell, window
    ((18, 24, 24), 0, 0, (1, 3, 3)),
    ((12, 16, 24), 1, 226, (1, 2, 3)),
    ((13, 17, 20), 1, 226, (2, 2, 2)),   # partial tiles on every axis, ragged text
    ((33, 45, 80), 0, 0, (3, 3, 3)),
    ((7, 9, 11), 1, 50, (2, 2, 2)),
    ((5, 7, 9), 0, 0, (1, 1, 2)),         # one partial tile: remainder blocks only
    ((1, 1, 1), 1, 256, (1, 1, 1)),
    ((6, 8, 8), 1, 17, (1, 1, 1)),
    ((1, 100, 100), 1, 64, (1, 1, 6)),   # one frame, a window of 1 tile along h: single-tile units
    ((9, 11, 3), 1, 1, (2, 2, 1)),
]


@pytest.mark.parametrize("shape", STREAM_SHAPES, ids=[f"{s[0]}w{s[3]}t{s[2] if s[1] else '-'}"
                                                      for s in STREAM_SHAPES])
def test_forward_key_stream_matches_oracle_mask(checks_bin, shape):
    """Every query unit's key stream (as the forward kernel walks it) holds
    exactly the keys the oracle's mask allows a query of that unit, each once;
    masked blocks come only after the whole ones (checked in the program)."""
    video, text, ell, win = shape
    T, H, W = video
    out = run(checks_bin, "stream", T, H, W, text, ell, *win).splitlines()
    n, tile_of_row, tokens = oracle_maps(video)
    n_tiles = int(np.prod(n))
    nv = T * H * W
    assert len(out) == n_tiles + text
    first_row = np.full(n_tiles, -1)
    first_row[tile_of_row[::-1]] = np.arange(nv)[::-1]  # a raster row of each tile
    for ln in out:
        f = ln.split()
        u, n_blk, n_plain = int(f[1]), int(f[2]), int(f[3])
        keys = np.concatenate([np.arange(*map(int, r.split(":"))) for r in f[4:]]) if f[4:] else np.zeros(0, int)
        row = nv if u == n_tiles else int(first_row[u])
        allowed = np.nonzero(oracle.allowed_mask([row], video, win, ell, bool(text))[0])[0]
        assert np.array_equal(keys, allowed), f"unit {u}"
        # block counts: every key tile in ceil(tokens / 64) blocks, then the text
        if u == n_tiles:
            ids = range(n_tiles)
        else:
            ids = oracle.key_tiles_of_query_tile(video, win, u) if n_tiles <= 40 else None
        if ids is not None:
            assert n_blk == sum(-(-int(tokens[i]) // 64) for i in ids) + -(-ell // 64), f"unit {u}"
            assert n_plain == sum(int(tokens[i]) // 64 for i in ids) + ell // 64, f"unit {u}"


@pytest.mark.parametrize("k", range(0, 7))
def test_hilbert_curve_helpers_match_oracle(checks_bin, k):
    """The library's iterative Hilbert helpers give the oracle's recursive curve."""
    from oracle import hilbert_oracle
    out = run(checks_bin, "hcurve", k).split("\n")[:-1]
    assert [tuple(map(int, ln.split())) for ln in out] == \
        [hilbert_oracle.hilbert_d2xy(k, d) for d in range(1 << (2 * k))]


HSHAPES = [
    # side, has_text, ell, W, mode (1 slide, 2 window)
    (8, 1, 226, 1, 1),
    (16, 0, 0, 1, 1),
    (16, 1, 100, 3, 1),
    (32, 1, 64, 5, 1),
    (32, 0, 0, 16, 1),
    (32, 1, 1, 4, 2),
    (64, 1, 226, 5, 2),
    (64, 0, 0, 16, 2),
    (64, 1, 200, 9, 1),
    (64, 0, 0, 4, 1),
    (64, 1, 30, 6, 2),
    (128, 1, 226, 27, 1),
    (64, 1, 17, 6, 1),
    (16, 1, 256, 4, 1),
]


@pytest.mark.parametrize("shape", HSHAPES, ids=[f"{s[0]}W{s[3]}m{s[4]}t{s[2] if s[1] else '-'}" for s in HSHAPES])
def test_hilbert_key_stream_matches_oracle_mask(checks_bin, shape):
    """Every Hilbert unit's key stream (as the kernel walks it) is exactly the
    oracle's mask row for a query of that tile, each key once."""
    from oracle import hilbert_oracle
    side, text, ell, W, mode = shape
    out = run(checks_bin, "hstream", side, text, ell, W, mode).splitlines()
    n_tiles = (side // 8) ** 2
    nv = side * side
    m = (side // 8).bit_length() - 1
    # tiles per unit as the host picks them: six consecutive positions for
    # slide windows of at least 6 tiles, four for slide windows of at least 4
    # or fixed windows of a multiple of 4, one otherwise
    if mode == 1 and W >= 6:
        G = 6
    else:
        G = 4 if n_tiles % 4 == 0 and (W >= 4 if mode == 1 else W % 4 == 0) else 1
    assert len(out) == n_tiles + text  # one line per query tile (and one for the text unit)
    for ln in out:
        f = ln.split()
        u, t, tx, ty = int(f[1]), int(f[2]), int(f[3]), int(f[4])
        keys = np.concatenate([np.arange(*map(int, r.split(":"))) for r in f[5:]])
        if tx >= 0:
            assert (tx, ty) == hilbert_oracle.hilbert_d2xy(m, G * u + t)
            row = ty * 8 * side + tx * 8
        else:
            row = nv
        allowed = np.nonzero(hilbert_oracle.hilbert_allowed_mask(
            [row], (side, side), W, "slide" if mode == 1 else "window", ell, bool(text))[0])[0]
        assert np.array_equal(keys, allowed), f"unit {u} tile {t}"


SQSHAPES = [
    # H, W (one frame), has_text, ell, window (wh, ww) in tiles
    (64, 64, 1, 226, 5, 5),      # 8x8 tiles, clamped windows at the border
    (72, 88, 0, 0, 3, 4),        # 9x11 tiles: odd last row and column of squares, even window
    (40, 48, 1, 100, 2, 2),      # the smallest windows that group
    (32, 32, 1, 64, 4, 4),       # window = the whole grid
    (8, 96, 1, 17, 1, 5),        # one tile row: a window of 1 along h still groups
    (96, 8, 0, 0, 6, 1),         # one tile column
    (128, 128, 1, 226, 5, 7),    # 256 tiles: the text rows split in two parts
    (256, 256, 1, 1, 3, 3),      # 1024 tiles: eight text parts
    (24, 24, 1, 256, 3, 3),      # 3x3 tiles, window = the grid
    (64, 64, 1, 50, 1, 3),       # a window of 1 along h: single-tile units
    (100, 100, 1, 64, 6, 6),     # 13x13 tiles, the last row and column of 4 rows / 4 columns
    (90, 160, 1, 226, 5, 5),     # a 720p latent: 12x20 tiles, the last tile row 2 rows high
    (44, 30, 0, 0, 3, 2),        # partial tiles along both axes
    (5, 100, 1, 10, 1, 4),       # one partial tile row
    (100, 3, 0, 0, 3, 1),        # one partial tile column
]


@pytest.mark.parametrize("shape", SQSHAPES, ids=[f"{s[0]}x{s[1]}w{s[4]}{s[5]}t{s[3] if s[2] else '-'}"
                                                 for s in SQSHAPES])
def test_square_key_stream_matches_oracle_mask(checks_bin, shape):
    """STA on a one-frame video with query units of 2x2 squares of tiles:
    every tile of every unit sees, through the blocks whose mask holds it,
    exactly the oracle's mask row for a query of that tile, each key once;
    every tile is in one unit (checked in the program); the text rows (all
    their parts together) see every video key and the valid text keys."""
    H, W, text, ell, wh, ww = shape
    out = run(checks_bin, "sqstream", H, W, text, ell, wh, ww).splitlines()
    video = (1, H, W)
    win = (1, wh, ww)
    nh, nw = -(-H // 8), -(-W // 8)
    groups = (wh >= 2 or nh == 1) and (ww >= 2 or nw == 1)
    if not groups:
        assert out == ["single"]
        return
    assert len(out) == nh * nw + text  # one line per query tile (and one for the text rows)
    seen_tiles = set()
    for ln in out:
        f = ln.split()
        th, tw = int(f[3]), int(f[4])
        keys = np.concatenate([np.arange(*map(int, r.split(":"))) for r in f[5:]])
        if th >= 0:
            seen_tiles.add((th, tw))
            row = th * 8 * W + tw * 8
        else:
            row = H * W
        allowed = np.nonzero(oracle.allowed_mask([row], video, win, ell, bool(text))[0])[0]
        assert np.array_equal(keys, allowed), f"unit {f[1]} tile ({th}, {tw})"
    assert seen_tiles == {(a, b) for a in range(nh) for b in range(nw)}


def test_sta_log_prints_the_schedule(checks_bin):
    """STA_LOG=1: a forward call prints its derived schedule to stderr (the
    query units and their kind, the text parts, the workspace) before any
    launch; without STA_LOG nothing is printed."""
    def stderr_of(env_extra, *args):
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", **env_extra)
        env.pop("LD_PRELOAD", None)
        if not env_extra:
            env.pop("STA_LOG", None)
        r = subprocess.run([checks_bin, *map(str, args)], stdout=subprocess.PIPE,
                           stderr=subprocess.PIPE, text=True, env=env)
        assert r.returncode == 0, r.stderr[-4000:]
        return r.stderr
    # a 512x512 image, window 5x5 tiles: 32x32 squares plus 8 text parts
    err = stderr_of({"STA_LOG": "1"}, "sqstream", 512, 512, 1, 226, 5, 5)
    lines = [ln for ln in err.splitlines() if ln.startswith("[sta] sta_forward:")]
    assert lines, err[-2000:]
    ln = lines[-1]
    assert "video=(1,512,512)" in ln and "tiles=(1,64,64)=4096" in ln, ln
    assert "units/head=1032 (2x2-square, partial tiles, text parts 8)" in ln, ln
    assert "window[0]=(1,5,5)" in ln, ln
    # a video: single-tile units, one text unit
    err = stderr_of({"STA_LOG": "1"}, "stream", 30, 48, 80, 1, 226, 3, 3, 3)
    ln = [x for x in err.splitlines() if x.startswith("[sta] sta_forward:")][-1]
    assert "tiles=(5,6,10)=300" in ln and "units/head=301 (single-tile, text parts 1)" in ln, ln
    assert "[sta]" not in stderr_of({}, "stream", 30, 48, 80, 1, 226, 3, 3, 3)
