"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.

Every sta_forward call here fails validation, so nothing is enqueued.
"""

import ctypes
import os
import re

import pytest

import block_sparse_sliding_amd as sta

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sta.LIB_PATH):
        from block_sparse_sliding_amd import build

        build.build()
    return sta.load_library()


def header_functions():
    text = open(os.path.join(ROOT, "include", "sta.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sta_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(sta.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code, name in sta.STATUS.items():
        assert sta.status_str(code).startswith(name)
    assert "UNKNOWN" in sta.status_str(99)


DIMS = dict(batch=1, heads=2, head_dim=128, video=(30, 48, 80))


def fwd(lib, dims, q=16, k=32, v=48, windows=((3, 3, 3), (3, 3, 3)), ell=226, text=1, out=1 << 40,
        lse=0, ws=1 << 44, ws_bytes=1 << 40):
    wa = sta.window_array(list(windows), len(windows)) if windows is not None else None
    return lib.sta_forward(ctypes.byref(dims) if dims is not None else None, q, k, v, wa, ell, text,
                           out, lse or None, ws, ws_bytes, None)


def test_forward_rejects_bad_arguments(lib):
    d = sta.make_dims(1, 2, 128, (30, 48, 80))
    assert fwd(lib, None) == 1
    assert fwd(lib, sta.make_dims(0, 2, 128, (30, 48, 80))) == 1
    assert fwd(lib, sta.make_dims(1, 0, 128, (30, 48, 80))) == 1
    assert fwd(lib, d, q=0) == 1
    assert fwd(lib, d, out=0) == 1
    assert fwd(lib, d, windows=None) == 1
    assert fwd(lib, sta.make_dims(1, 2, 96, (30, 48, 80))) == 2
    assert fwd(lib, sta.make_dims(1, 2, 128, (0, 48, 80))) == 2
    assert fwd(lib, sta.make_dims(1, 2, 128, (30, -8, 80))) == 2
    assert fwd(lib, sta.make_dims(1, 2, 128, (30, 48, 0))) == 2
    # sizes that are not tile multiples are valid (tile grid (6, 6, 11) here):
    # the shape and windows pass, and the check after them (workspace) fails,
    # so nothing is launched on the fake pointers
    assert fwd(lib, sta.make_dims(1, 2, 128, (31, 44, 84)), windows=((3, 3, 11), (6, 6, 3)),
               ws_bytes=1) == 6
    assert fwd(lib, sta.make_dims(1, 2, 128, (31, 44, 84)), windows=((3, 7, 3), (3, 3, 3))) == 3
    assert fwd(lib, sta.make_dims(1, 257, 128, (30, 48, 80)), windows=[(1, 1, 1)] * 257) == 2
    # windows: each component in [1, tiles on the axis] = [1, (5, 6, 10)]
    assert fwd(lib, d, windows=((6, 3, 3), (3, 3, 3))) == 3
    assert fwd(lib, d, windows=((3, 3, 3), (3, 7, 3))) == 3
    assert fwd(lib, d, windows=((3, 3, 11), (3, 3, 3))) == 3
    assert fwd(lib, d, windows=((0, 3, 3), (3, 3, 3))) == 3
    # text length
    assert fwd(lib, d, ell=257) == 4
    assert fwd(lib, d, ell=-1) == 4
    assert fwd(lib, d, ell=5, text=0) == 4
    # alignment (pointer values are never dereferenced: validation comes first)
    assert fwd(lib, d, q=17) == 5
    assert fwd(lib, d, out=(1 << 40) + 8) == 5
    assert fwd(lib, d, lse=(1 << 41) + 4) == 5
    # workspace
    need = sta.sta_workspace_bytes(d, [(3, 3, 3)] * 2, True)
    assert fwd(lib, d, ws_bytes=need - 1) == 6
    assert fwd(lib, d, ws=0, ws_bytes=need) == 6
    assert fwd(lib, d, ws=(1 << 44) + 16, ws_bytes=need) == 5
    # aliasing: out over q, lse over out
    assert fwd(lib, d, q=1 << 40, ws_bytes=need) == 8
    assert fwd(lib, d, lse=(1 << 40) + 1024, ws_bytes=need) == 8


def test_layout_calls_reject_bad_arguments(lib):
    d = sta.make_dims(1, 1, 64, (18, 24, 24))
    assert lib.sta_tile_gather(ctypes.byref(d), 0, None, 16, None) == 1
    assert lib.sta_tile_gather(ctypes.byref(d), 0, 16, 24, None) == 5
    assert lib.sta_tile_gather(ctypes.byref(d), 0, 16, 32, None) == 8
    assert lib.sta_tile_gather(ctypes.byref(sta.make_dims(1, 1, 64, (0, 24, 24))), 0, 16,
                               1 << 30, None) == 2
    # sizes that are not tile multiples pass the shape checks: the tiled buffer
    # has sta_tiled_seq_len rows (S_t = 2*3*4*384 here, > S), so a raster buffer
    # starting inside it overlaps (the call stops there, before any launch)
    pd = sta.make_dims(1, 1, 64, (7, 24, 30))
    assert sta.sta_tiled_seq_len(pd, False) == 2 * 3 * 4 * 384
    assert lib.sta_tile_scatter(ctypes.byref(pd), 0, 1 << 30, (1 << 30) + 7 * 24 * 30 * 128, None) == 8
    assert lib.sta_tile_gather(ctypes.byref(pd), 0, (1 << 30) + 9216 * 128 - 16, 1 << 30, None) == 8


def seq(video, text):
    return video[0] * video[1] * video[2] + (256 if text else 0)


@pytest.mark.parametrize("B,heads,D,video,windows,text", [
    (1, 1, 64, (18, 24, 24), [(1, 3, 3)], False),
    (1, 24, 128, (30, 48, 80), [(3, 3, 3)] * 24, True),
    (2, 4, 128, (30, 48, 80), [(5, 6, 10), (3, 3, 3), (1, 6, 10), (5, 1, 1)], True),
    (1, 24, 128, (48, 72, 128), [(3, 3, 3)] * 24, True),
    (1, 2, 128, (7, 9, 11), [(2, 2, 2), (1, 1, 2)], True),
    (2, 3, 64, (13, 8, 20), [(3, 1, 3), (1, 1, 1), (2, 1, 2)], False),
])
def test_sizes(lib, B, heads, D, video, windows, text):
    d = sta.make_dims(B, heads, D, video)
    S = seq(video, text)
    assert sta.sta_seq_len(d, text) == S
    n_tiles = -(-video[0] // 6) * -(-video[1] // 8) * -(-video[2] // 8)  # ceil tile grid
    assert sta.sta_tiled_seq_len(d, text) == n_tiles * 384 + (256 if text else 0)
    n_q = n_tiles + (1 if text else 0)
    n_off, n_ids, n_work = sta.sta_schedule_sizes(d, windows, text)
    assert n_off == heads * n_q + 1
    assert n_ids == sum(n_tiles * w[0] * w[1] * w[2] + (n_tiles if text else 0) for w in windows)
    assert n_work == B * heads * n_q

    def up(x):
        return (x + 255) // 256 * 256
    queue_heads = 8 * 64 * 4  # one int per XCD queue, each on its own 256-byte line
    zero_row = 256            # the source of keys that must not contribute
    expect = up(n_work * 4) + queue_heads + zero_row
    assert sta.sta_workspace_bytes(d, windows, text) == expect


def test_workspace_bytes_invalid_is_zero(lib):
    assert sta.sta_workspace_bytes(sta.make_dims(1, 1, 64, (18, 24, 24)), [(4, 1, 1)], False) == 0
    assert sta.sta_workspace_bytes(sta.make_dims(1, 1, 32, (18, 24, 24)), [(1, 1, 1)], False) == 0
    assert sta.sta_seq_len(sta.make_dims(1, 1, 64, (18, 24, 23)), False) == 18 * 24 * 23
    assert sta.sta_seq_len(sta.make_dims(1, 1, 64, (18, 0, 23)), False) == 0


def bwd(lib, dims, q=16, k=1 << 36, v=1 << 37, out=1 << 38, lse=1 << 39, dout=(1 << 39) + (1 << 34),
        windows=((3, 3, 3), (3, 3, 3)), ell=226, text=1, dq=1 << 40, dk=1 << 41, dv=1 << 42,
        ws=1 << 44, ws_bytes=1 << 42):
    """sta_backward with fake, never dereferenced, well-separated device addresses."""
    wa = sta.window_array(list(windows), len(windows)) if windows is not None else None
    return lib.sta_backward(ctypes.byref(dims) if dims is not None else None, q, k, v, out, lse,
                            dout, wa, ell, text, dq, dk, dv, ws, ws_bytes, None)


def test_backward_rejects_bad_arguments(lib):
    d = sta.make_dims(1, 2, 128, (30, 48, 80))
    need = sta.sta_backward_workspace_bytes(d, [(3, 3, 3)] * 2, True)
    assert need > 0
    assert bwd(lib, None) == 1
    for name in ("q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv"):
        assert bwd(lib, d, **{name: 0}) == 1, name
    assert bwd(lib, d, windows=None) == 1
    assert bwd(lib, sta.make_dims(1, 2, 96, (30, 48, 80))) == 2
    assert bwd(lib, sta.make_dims(1, 2, 128, (30, 0, 80))) == 2
    assert bwd(lib, sta.make_dims(1, 2, 128, (31, 44, 84)), windows=((3, 3, 11), (6, 6, 3)),
               ws_bytes=1) == 6
    assert bwd(lib, d, windows=((6, 3, 3), (3, 3, 3))) == 3
    assert bwd(lib, d, ell=257) == 4
    assert bwd(lib, d, ell=3, text=0) == 4
    for name in ("q", "out", "lse", "dout", "dq", "dv"):
        assert bwd(lib, d, **{name: {"q": 16, "out": 1 << 38, "lse": 1 << 39,
                                     "dout": (1 << 39) + (1 << 34), "dq": 1 << 40,
                                     "dv": 1 << 42}[name] + 4}) == 5, name
    assert bwd(lib, d, ws_bytes=need - 1) == 6
    assert bwd(lib, d, ws=0, ws_bytes=need) == 6
    assert bwd(lib, d, ws=(1 << 44) + 16, ws_bytes=need) == 5
    # outputs may overlap nothing: an input, the workspace or each other
    assert bwd(lib, d, dq=16, ws_bytes=need) == 8
    assert bwd(lib, d, dk=(1 << 39) + (1 << 34) + 64, ws_bytes=need) == 8
    assert bwd(lib, d, dv=(1 << 44) + 1024, ws_bytes=need) == 8
    assert bwd(lib, d, dk=(1 << 40) + 256, ws_bytes=need) == 8


@pytest.mark.parametrize("B,heads,D,video,windows,text", [
    (1, 1, 64, (18, 24, 24), [(1, 3, 3)], False),
    (1, 24, 128, (30, 48, 80), [(3, 3, 3)] * 24, True),
    (2, 4, 128, (30, 48, 80), [(5, 6, 10), (3, 3, 3), (1, 6, 10), (5, 1, 1)], True),
    (1, 2, 128, (7, 9, 11), [(2, 2, 2), (1, 1, 2)], True),
])
def test_backward_workspace_bytes(lib, B, heads, D, video, windows, text):
    d = sta.make_dims(B, heads, D, video)
    n_off, n_ids, _ = sta.sta_schedule_sizes(d, windows, text)
    n_tiles = -(-video[0] // 6) * -(-video[1] // 8) * -(-video[2] // 8)
    S_t = n_tiles * 384 + (256 if text else 0)

    def up(x):
        return (x + 255) // 256 * 256
    rows = B * heads * S_t * 4
    queue_heads = 8 * 64 * 4
    zero_row = 256
    expect = 2 * up(rows) + up(n_off * 4) + up(n_ids * 4) + 2 * queue_heads + zero_row
    assert sta.sta_backward_workspace_bytes(d, windows, text) == expect
    assert sta.sta_backward_workspace_bytes(sta.make_dims(B, heads, 96, video), windows, text) == 0
