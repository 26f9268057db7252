"""GPU checks of the tile-major gather/scatter and the device-built schedule.

Gather/scatter are compared bit for bit with an index map built here from the
tile definition; the schedule's key-tile lists with the key tiles the
oracle's token mask touches (brute force per query tile), and their order by
coordinate residues; the work order is checked for being a permutation split
into 8 per-XCD queues, each heaviest first.
"""

import numpy as np
import pytest
import torch

import block_sparse_sliding_amd as sta
import oracle
from _parity import note

pytestmark = pytest.mark.gpu


def tile_major_index(video, has_text):
    """Raster row of every tile-major row, -1 for padding (text rows follow the video).

    Tile (tt, th, tw) owns 384 rows: the tokens of its (6, 8, 8) box that exist,
    in (frame, row, column) order, then padding (only for sizes that are not
    tile multiples, where the last tile along an axis holds the remainder).
    """
    T, H, W = video
    n = (-(-T // 6), -(-H // 8), -(-W // 8))
    idx = []
    for tt in range(n[0]):
        for th in range(n[1]):
            for tw in range(n[2]):
                t = np.arange(tt * 6, min(T, tt * 6 + 6))[:, None, None]
                h = np.arange(th * 8, min(H, th * 8 + 8))[None, :, None]
                w = np.arange(tw * 8, min(W, tw * 8 + 8))[None, None, :]
                rows = ((t * H + h) * W + w).reshape(-1)
                idx.append(np.concatenate([rows, -np.ones(384 - rows.size, dtype=rows.dtype)]))
    idx = np.concatenate(idx)
    if has_text:
        idx = np.concatenate([idx, T * H * W + np.arange(256)])
    return torch.from_numpy(idx)


@pytest.mark.parametrize("B,heads,D,video,has_text", [
    (1, 1, 64, (18, 24, 24), False),
    (2, 3, 128, (18, 24, 32), True),
    (1, 2, 128, (30, 48, 80), True),
    (1, 1, 64, (6, 8, 8), True),
    (2, 2, 128, (7, 9, 11), True),
    (1, 1, 64, (13, 8, 21), False),
    (1, 2, 128, (33, 45, 80), True),
])
def test_gather_scatter(B, heads, D, video, has_text):
    note(f"gather/scatter {B} {heads} {D} {video} {has_text}")
    dims = sta.make_dims(B, heads, D, video)
    S = sta.sta_seq_len(dims, has_text)
    S_t = sta.sta_tiled_seq_len(dims, has_text)
    g = torch.Generator(device="cuda").manual_seed(S)
    x = torch.randn(B, heads, S, D, generator=g, device="cuda").to(torch.bfloat16)
    tiled = torch.full((B, heads, S_t, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    back = torch.full_like(x, float("nan"))
    sta.sta_tile_gather(dims, has_text, x, tiled)
    sta.sta_tile_scatter(dims, has_text, tiled, back)
    torch.cuda.synchronize()
    idx = tile_major_index(video, has_text).cuda()
    assert idx.numel() == S_t
    real = idx >= 0
    assert torch.equal(tiled[:, :, real].view(torch.int16), x[:, :, idx[real]].view(torch.int16))
    assert bool((tiled[:, :, ~real] == 0).all())
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))


def build_schedule(B, heads, video, windows, ell, has_text):
    dims = sta.make_dims(B, heads, 128, video)
    n_off, n_ids, n_work = sta.sta_schedule_sizes(dims, windows, has_text)
    off = torch.full((n_off,), -1, dtype=torch.int32, device="cuda")
    ids = torch.full((n_ids,), -1, dtype=torch.int32, device="cuda")
    work = torch.full((n_work,), -1, dtype=torch.int32, device="cuda")
    sta.sta_build_schedule(dims, windows, ell, has_text, off, ids, work)
    torch.cuda.synchronize()
    return off.cpu().numpy(), ids.cpu().numpy(), work.cpu().numpy()


SCHED = [
    (1, 1, (18, 24, 24), [(1, 3, 3)], 0, False),
    (2, 3, (18, 24, 32), [(3, 3, 3), (1, 2, 3), (2, 1, 4)], 77, True),
    (1, 4, (30, 48, 80), [(5, 6, 10), (3, 3, 3), (1, 6, 10), (5, 1, 1)], 256, True),
    (1, 24, (30, 48, 80), [(3, 3, 3)] * 24, 226, True),
    (1, 24, (48, 72, 128), [(3, 3, 3)] * 24, 128, True),
    (3, 5, (12, 16, 24), [(1, 1, 1), (2, 2, 3), (2, 1, 2), (1, 2, 1), (2, 2, 1)], 5, True),
    # sizes that are not tile multiples: the same schedule on the ceil tile grid
    (1, 2, (7, 9, 11), [(2, 2, 2), (1, 1, 2)], 77, True),
    (1, 3, (33, 45, 80), [(3, 3, 3), (2, 4, 5), (6, 6, 10)], 226, True),
]


@pytest.mark.parametrize("case", SCHED, ids=[f"c{i}" for i in range(len(SCHED))])
def test_schedule_matches_mask(case):
    B, heads, video, windows, ell, has_text = case
    note(f"schedule {case[:3]}")
    off, ids, work = build_schedule(B, heads, video, windows, ell, has_text)
    nt, nh, nw = -(-video[0] // 6), -(-video[1] // 8), -(-video[2] // 8)  # ceil tile grid
    n_tiles = nt * nh * nw
    n_q = n_tiles + (1 if has_text else 0)
    assert off[0] == 0 and off[-1] == len(ids)
    assert (np.diff(off) >= 0).all()
    rng = np.random.default_rng(len(ids))
    first_head = {}
    for hd in range(heads):
        lists = [ids[off[hd * n_q + qt]:off[hd * n_q + qt + 1]].tolist() for qt in range(n_tiles)]
        if windows[hd] in first_head:
            # same window as an earlier head: the lists must be identical
            assert lists == first_head[windows[hd]], hd
        else:
            first_head[windows[hd]] = lists
            tiles = range(n_tiles) if n_tiles <= 40 else sorted(
                set(rng.integers(0, n_tiles, 6).tolist()) | {0, n_tiles - 1})
            w = windows[hd]
            digits = [(a, b, c) for a in range(w[0]) for b in range(w[1]) for c in range(w[2])]
            for qt in tiles:
                # the window's tiles, each once ...
                assert sorted(lists[qt]) == oracle.key_tiles_of_query_tile(video, windows[hd], qt), (hd, qt)
                # ... listed by the residues of their coordinates mod the window size
                res = [((x // (nh * nw)) % w[0], ((x // nw) % nh) % w[1], (x % nw) % w[2])
                       for x in lists[qt]]
                assert res == digits, (hd, qt)
            # every list has the window's tile count
            w = windows[hd]
            assert all(len(x) == w[0] * w[1] * w[2] for x in lists)
        if has_text:
            got = ids[off[hd * n_q + n_tiles]:off[hd * n_q + n_tiles + 1]].tolist()
            assert got == list(range(n_tiles))

    # the work order: a permutation of all query units
    assert sorted(work.tolist()) == list(range(B * heads * n_q))

    # queue x is work[x::8]; each queue must run heaviest first,
    # every class of equal-cost units must be split evenly over the XCDs, and
    # the XCD loads may differ by at most one unit's cost
    def cost(unit):
        u, bh = unit % n_q, unit // n_q
        hd = bh % heads
        if has_text and u == n_tiles:
            return 256 * (n_tiles * 384 + ell)
        w = windows[hd]
        return 384 * (w[0] * w[1] * w[2] * 384 + (ell if has_text else 0))

    def klass(unit):
        u, bh = unit % n_q, unit // n_q
        return (bh % heads, has_text and u == n_tiles)

    total = len(work)
    loads = []
    per_class = {}
    for x in range(8):
        queue = work[x::8]
        costs = np.array([cost(int(u)) for u in queue])
        assert (np.diff(costs) <= 0).all(), f"XCD {x} queue is not heaviest first"
        loads.append(costs.sum())
        for u in queue:
            per_class.setdefault(klass(int(u)), [0] * 8)[x] += 1
    assert max(loads) - min(loads) <= max(cost(int(u)) for u in work)
    for kc, counts in per_class.items():
        assert max(counts) - min(counts) <= 1, (kc, counts)
    assert total == B * heads * n_q
