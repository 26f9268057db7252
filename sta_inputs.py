"""Seeded synthetic inputs and workload shapes for Sliding Tile Attention.

This module is shared by the tests, the benchmark and the smoke check. It
holds no step of the method's arithmetic: it only names workload shapes and
draws seeded random tensors. Both the oracle and the HIP path receive the
exact same bf16 values from here.

Recipe: q, k, v are drawn as float32 N(0, 1) from a torch generator seeded
with ``10 * config_index + {0, 1, 2}`` and rounded to bfloat16 (round to
nearest even, torch's ``.to(torch.bfloat16)``). The pages measure on no
public dataset; their HunyuanVideo (text) and StepVideo (no text) latents are
not available, so these N(0, 1) tensors stand in for them at the same shapes.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import torch

TILE = (6, 8, 8)          # tile cube (t, h, w) in tokens
TEXT_SLOTS = 256          # padded text segment length when text is present


@dataclass(frozen=True)
class Workload:
    """One STA workload shape (no arithmetic of the method lives here)."""

    name: str
    batch: int
    heads: int
    head_dim: int
    video: Tuple[int, int, int]                 # (T, H, W) in tokens
    windows: Tuple[Tuple[int, int, int], ...]   # one (wt, wh, ww) per head
    has_text: bool
    text_length: int
    seed_base: int
    # Hilbert-window attention on a 2D image (video (1, 8*2^m, 8*2^m)): window
    # length in tiles and mode (1 slide, 2 window); 0 for STA workloads
    hilbert_len: int = 0
    hilbert_mode: int = 0

    @property
    def seq_len(self) -> int:
        T, H, W = self.video
        return T * H * W + (TEXT_SLOTS if self.has_text else 0)

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "batch": self.batch,
            "heads": self.heads,
            "head_dim": self.head_dim,
            "video": list(self.video),
            "seq_len": self.seq_len,
            "windows": sorted(set(self.windows)),
            "has_text": self.has_text,
            "text_length": self.text_length,
            **({"hilbert_window_tiles": self.hilbert_len,
                "hilbert_mode": "slide" if self.hilbert_mode == 1 else "window"}
               if self.hilbert_len else {}),
        }


def _per_head(heads: int, cycle: Sequence[Tuple[int, int, int]]):
    return tuple(tuple(cycle[h % len(cycle)]) for h in range(heads))


# Workloads: the tiny CPU-checkable case, the four full-size cases, the
# headline shape (video (30,48,80) + 256 text slots, 24 heads, D=128,
# window (3,3,3); its text length 226 is the one the text case uses) and the
# headline at a height that is not a tile multiple.
WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 64, (18, 24, 24), _per_head(1, [(1, 3, 3)]),
                     False, 0, 10),
    "notext": Workload("notext", 1, 24, 128, (30, 48, 80),
                       _per_head(24, [(3, 3, 3)]), False, 0, 20),
    "text": Workload("text", 1, 24, 128, (30, 48, 80),
                     _per_head(24, [(3, 3, 5)]), True, 226, 30),
    "mixed": Workload("mixed", 1, 24, 128, (30, 48, 80),
                      _per_head(24, [(5, 6, 10), (3, 3, 3), (1, 6, 10), (5, 1, 1)]),
                      True, 256, 40),
    "large": Workload("large", 1, 24, 128, (48, 72, 128),
                      _per_head(24, [(3, 3, 3)]), True, 128, 50),
    "headline": Workload("headline", 1, 24, 128, (30, 48, 80),
                         _per_head(24, [(3, 3, 3)]), True, 226, 60),
    # the headline at 33 frames and 45 rows (a 129-frame clip at 4x temporal
    # and a 720-pixel height at 16x spatial reduction): neither is a tile
    # multiple, so the last tile row in t holds 3 of 6 frames and the last in
    # h 5 of 8 rows; tile grid (6, 6, 10)
    "ragged": Workload("ragged", 1, 24, 128, (33, 45, 80),
                       _per_head(24, [(3, 3, 3)]), True, 226, 70),
    # 2D STA on a 512x512 image: a one-frame video, so each tile holds one
    # 8x8 frame (64 tokens) and the grid is 1x64x64 tiles; window 5x5 tiles
    # (25 key tiles, as many as the Hilbert workload's 27 nearly), the
    # headline's heads, head size and text
    "image": Workload("image", 1, 24, 128, (1, 512, 512),
                      _per_head(24, [(1, 5, 5)]), True, 226, 90),
    # Hilbert slide attention on a 512x512 image (a 64x64 grid of 8x8 tiles),
    # 27 key tiles per query tile along the curve, the headline's heads, head
    # size and text; the pages give no size for the Hilbert row
    "hilbert": Workload("hilbert", 1, 24, 128, (1, 512, 512),
                        _per_head(24, [(1, 1, 27)]), True, 226, 80, hilbert_len=27, hilbert_mode=1),
}


def custom(name: str, batch: int, heads: int, head_dim: int, video, windows,
           has_text: bool, text_length: int, seed_base: int = 1000) -> Workload:
    """A workload of arbitrary shape (tests use small ones)."""
    if len(windows) == 3 and isinstance(windows[0], int):
        windows = [tuple(windows)] * heads
    return Workload(name, batch, heads, head_dim, tuple(video),
                    _per_head(heads, [tuple(w) for w in windows]) if len(windows) != heads
                    else tuple(tuple(w) for w in windows),
                    has_text, text_length, seed_base)


def make_qkv(wl: Workload, device: str = "cpu", seed_offset: int = 0):
    """Draw q, k, v as bf16 [B, heads, S, D] from N(0, 1) with fixed seeds.

    On the CPU the draw uses torch's CPU generator; on a GPU it uses the
    device generator (a different stream of numbers, equally seeded). Tests
    that compare against the oracle hand the oracle the very tensors drawn
    here, copied to the host, so either source is consistent.
    """
    shape = (wl.batch, wl.heads, wl.seq_len, wl.head_dim)
    out = []
    for i in range(3):
        g = torch.Generator(device=device)
        g.manual_seed(wl.seed_base + i + seed_offset)
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        out.append(x.to(torch.bfloat16))
        del x
    return tuple(out)


def sample_rows(wl: Workload, per_head: int, seed: int = 7) -> torch.Tensor:
    """A stratified sample of query rows (sequence indices) for one head.

    Includes the eight corner tokens of the video, tokens on the centre of
    each face, a uniform random draw over the video, and when text is
    present the first, last-valid, first-padded and last text slots plus a
    few random text slots. Sorted, unique, int64.
    """
    T, H, W = wl.video
    nv = T * H * W

    def idx(t, h, w):
        return (t * H + h) * W + w

    picks = set()
    for t in (0, T - 1):
        for h in (0, H - 1):
            for w in (0, W - 1):
                picks.add(idx(t, h, w))
    for t, h, w in ((T // 2, H // 2, 0), (T // 2, H // 2, W - 1), (T // 2, 0, W // 2),
                    (T // 2, H - 1, W // 2), (0, H // 2, W // 2), (T - 1, H // 2, W // 2),
                    (T // 2, H // 2, W // 2)):
        picks.add(idx(t, h, w))
    g = torch.Generator().manual_seed(seed)
    n_rand = max(per_head - len(picks), 0)
    if wl.has_text:
        s = {nv, nv + TEXT_SLOTS - 1, nv + max(wl.text_length - 1, 0),
             nv + min(wl.text_length, TEXT_SLOTS - 1)}
        s |= {nv + int(x) for x in torch.randint(0, TEXT_SLOTS, (4,), generator=g)}
        picks |= s
        n_rand = max(per_head - len(picks), 0)
    picks |= {int(x) for x in torch.randint(0, nv, (n_rand,), generator=g)}
    return torch.tensor(sorted(picks), dtype=torch.int64)


def sample_rows_stratified(wl: Workload, per_head: int, head: int, seed: int = 11) -> torch.Tensor:
    """A stratified sample of query rows for head ``head`` (a different draw per head).

    Strata are the video tiles grouped by how many of their axes touch the
    border of the tile grid (0: interior, 1: face, 2: edge, 3: corner; a
    one-tile axis counts as border); each present stratum gets an equal share
    of random (tile, token) picks. Added to them: the rows of
    ``sample_rows`` (video corners and face centres, first / last-valid /
    first-padded / last text slots) and, with text, 8 further random text
    slots. Sorted, unique, int64; at least ``per_head`` rows when the video
    has that many.
    """
    T, H, W = wl.video
    nv = T * H * W
    n = tuple(-(-s // t) for s, t in zip(wl.video, TILE))
    g = torch.Generator().manual_seed(seed + 7919 * head + 104729 * wl.seed_base)
    picks = {int(x) for x in sample_rows(wl, per_head=0, seed=seed + head)}
    if wl.has_text:
        picks |= {nv + int(x) for x in torch.randint(0, TEXT_SLOTS, (8,), generator=g)}
    strata = {}
    for tt in range(n[0]):
        for th in range(n[1]):
            for tw in range(n[2]):
                b = sum(int(c == 0 or c == m - 1) for c, m in zip((tt, th, tw), n))
                strata.setdefault(b, []).append((tt, th, tw))
    want = max(per_head - len(picks), 0)
    share = -(-want // len(strata))
    for b in sorted(strata):
        tiles = strata[b]
        for _ in range(share):
            tt, th, tw = tiles[int(torch.randint(0, len(tiles), (1,), generator=g))]
            # a token that exists in the tile (the last tile along an axis may be partial)
            ft, fh, fw = (min(t, s - c * t) for t, s, c in zip(TILE, wl.video, (tt, th, tw)))
            dt, dh, dw = (int(torch.randint(0, f, (1,), generator=g)) for f in (ft, fh, fw))
            picks.add(((tt * TILE[0] + dt) * H + th * TILE[1] + dh) * W + tw * TILE[2] + dw)
    # top up (duplicates) with uniform draws over the video
    while len(picks) < min(per_head, nv):
        picks.add(int(torch.randint(0, nv, (1,), generator=g)))
    return torch.tensor(sorted(picks), dtype=torch.int64)


def tile_of_row(wl: Workload, row: int) -> int:
    """Query unit of a sequence row: its video tile (raster tile index) or, for a
    text slot, -1 (the text slots of a head form one unit)."""
    T, H, W = wl.video
    if row >= T * H * W:
        return -1
    n_h, n_w = -(-H // TILE[1]), -(-W // TILE[2])
    t, h, w = row // (H * W), (row // W) % H, row % W
    return ((t // TILE[0]) * n_h + h // TILE[1]) * n_w + w // TILE[2]
