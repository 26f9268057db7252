"""Plain CPU oracle for Hilbert-curve token order and Hilbert-window attention.

Test infrastructure only: imported by the tests, never by the HIP library,
with which it shares no code.

Source: the blog post "Boosting 2D Local Attention Efficiency with
Hilbert-Guided Sparsity", sections "TLDR" and "The Hilbert Curve Advantage".
What the post fixes, restated: the tokens of an image are reordered along a
Hilbert curve (a continuous space-filling curve that keeps points that are
close in the plane close in the 1D sequence); attention windows and
neighbourhoods built on that 1D order are much more contiguous, so a
block-sparse kernel sees more empty blocks and fewer partial blocks; the
method feeds existing block-sparse kernels unchanged.

Readings where the post is silent (it gives no curve orientation, no window
grouping and no sizes):

* the image is a one-frame video (T = 1) whose side is 8 * 2^m tokens, so its
  grid of 8x8 tiles is a 2^m x 2^m square; x is the column (w) and y the row
  (h) of a token, and raster order is y-major;
* the curve of order k on the 2^k x 2^k grid starts at (0, 0) and ends at
  (2^k - 1, 0). Order 0 is the single cell. Order k visits its four
  quadrants in the order (x low, y low), (x low, y high), (x high, y high),
  (x high, y low), running the order k - 1 curve transposed in the first,
  shifted in the second and third, and reflected through the anti-diagonal
  in the last, so that each quadrant's curve ends next to where the next one
  starts;
* with 64-token blocks, positions [64 i, 64 i + 64) of the order k = m + 3
  curve cover exactly one 8x8 tile: the block pattern lives on the tiles,
  taken in the order of the order-m curve on the tile grid;
* Hilbert slide attention: a video query of the tile at curve position i
  sees the key tiles at positions [s, s + W), s = clamp(i - W // 2, 0, n - W)
  (the STA window rule in one dimension, W tiles, n = 4^m), plus the valid
  text keys; Hilbert window attention: it sees positions
  [W * (i // W), min(W * (i // W) + W, n)). Text queries see every video key
  and the valid text keys, as in STA. W is counted in tiles (blocks).

Everything is computed in float64 from an explicit token-level mask.
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

from .sta_oracle import TEXT_SLOTS, _as_np64, softmax_scale

TILE_SIDE = 8      # tile side in tokens (the STA tile's (h, w) extent)
BLOCK = 64         # tokens per block (one 8x8 tile)


def hilbert_d2xy(order: int, d: int) -> Tuple[int, int]:
    """(x, y) of position d on the order-``order`` curve, by the recursive definition."""
    if order == 0:
        if d != 0:
            raise ValueError("order 0 has one cell")
        return 0, 0
    half = 1 << (order - 1)
    quad, rest = divmod(d, half * half)
    if not 0 <= quad < 4:
        raise ValueError("position outside the curve")
    x, y = hilbert_d2xy(order - 1, rest)
    if quad == 0:
        return y, x                                   # transposed
    if quad == 1:
        return x, y + half                            # shifted up
    if quad == 2:
        return x + half, y + half                     # shifted up and right
    return 2 * half - 1 - y, half - 1 - x             # anti-diagonal reflection, shifted right


def hilbert_xy2d(order: int, x: int, y: int) -> int:
    """Position of (x, y) on the order-``order`` curve (the inverse, by the same recursion)."""
    if order == 0:
        if (x, y) != (0, 0):
            raise ValueError("order 0 has one cell")
        return 0
    half = 1 << (order - 1)
    if not (0 <= x < 2 * half and 0 <= y < 2 * half):
        raise ValueError("cell outside the grid")
    if x < half and y < half:
        return hilbert_xy2d(order - 1, y, x)
    if x < half:
        return half * half + hilbert_xy2d(order - 1, x, y - half)
    if y >= half:
        return 2 * half * half + hilbert_xy2d(order - 1, x - half, y - half)
    return 3 * half * half + hilbert_xy2d(order - 1, half - 1 - y, 2 * half - 1 - x)


def _check_image(image: Tuple[int, int]) -> int:
    """The tile-grid order m of a (H, W) image, or ValueError."""
    H, W = image
    if H != W or H % TILE_SIDE:
        raise ValueError("a square image whose side is a multiple of 8 is required")
    n_side = H // TILE_SIDE
    m = n_side.bit_length() - 1
    if n_side != 1 << m:
        raise ValueError("the tile grid side must be a power of two")
    return m


def hilbert_token_order(image: Tuple[int, int]) -> np.ndarray:
    """perm[d] = raster index of the d-th token on the curve of the whole image."""
    m = _check_image(image)
    k = m + 3
    side = image[1]
    perm = np.empty(side * side, dtype=np.int64)
    for d in range(side * side):
        x, y = hilbert_d2xy(k, d)
        perm[d] = y * side + x
    return perm


def window_span(i: int, W: int, n: int, mode: str) -> Tuple[int, int]:
    """(first, count) of the curve positions of the key tiles of the query tile at position i."""
    if not 1 <= W <= n:
        raise ValueError("window length outside [1, n]")
    if mode == "slide":
        s = max(0, min(i - W // 2, n - W))
        return s, W
    if mode == "window":
        s = W * (i // W)
        return s, min(W, n - s)
    raise ValueError("mode is 'slide' or 'window'")


def hilbert_allowed_mask(rows: Sequence[int], image: Tuple[int, int], window_len: int,
                         mode: str, text_length: int, has_text: bool) -> np.ndarray:
    """mask[r, j]: query ``rows[r]`` may see key ``j`` (raster video tokens, then 256 text slots)."""
    m = _check_image(image)
    side = image[1]
    n_video = side * side
    n_tiles = 1 << (2 * m)
    seq = n_video + (TEXT_SLOTS if has_text else 0)
    if not has_text and text_length != 0:
        raise ValueError("text_length must be 0 without text")
    if not 0 <= text_length <= TEXT_SLOTS:
        raise ValueError("text_length must lie in [0, 256]")
    ky, kx = np.divmod(np.arange(n_video), side)
    key_tile_pos = np.array([hilbert_xy2d(m, int(a), int(b))
                             for a, b in zip(kx // TILE_SIDE, ky // TILE_SIDE)])
    rows = np.asarray(rows, dtype=np.int64)
    mask = np.zeros((len(rows), seq), dtype=bool)
    for r, i in enumerate(rows):
        if i < n_video:
            y, x = divmod(int(i), side)
            p = hilbert_xy2d(m, x // TILE_SIDE, y // TILE_SIDE)
            s, cnt = window_span(p, window_len, n_tiles, mode)
            mask[r, :n_video] = (key_tile_pos >= s) & (key_tile_pos < s + cnt)
        elif i < seq:
            mask[r, :n_video] = True
        else:
            raise IndexError(f"row {i} out of range for sequence length {seq}")
        if has_text:
            mask[r, n_video:n_video + text_length] = True
    return mask


def hilbert_reference(q, k, v, window_lens, mode: str, text_length: int, has_text: bool,
                      image: Tuple[int, int], rows: Optional[Iterable[int]] = None,
                      chunk: int = 128):
    """Hilbert slide/window attention in float64: dense softmax under the explicit mask.

    q, k, v: ``[B, heads, S, D]`` in raster token order (bf16 values are upcast
    exactly); ``window_lens``: one window length in tiles per head (or one
    integer for all). Returns ``(out, lse)`` like the STA oracle.
    """
    q64, k64, v64 = _as_np64(q), _as_np64(k), _as_np64(v)
    B, heads, S, D = q64.shape
    side = image[1]
    if S != side * side + (TEXT_SLOTS if has_text else 0):
        raise ValueError("sequence length does not match the image / text")
    if np.isscalar(window_lens):
        window_lens = [int(window_lens)] * heads
    if len(window_lens) != heads:
        raise ValueError("one window length per head is required")
    rows = np.arange(S) if rows is None else np.asarray(list(rows), dtype=np.int64)
    scale = softmax_scale(D)
    out = np.empty((B, heads, len(rows), D))
    lse = np.empty((B, heads, len(rows)))
    for h in range(heads):
        for r0 in range(0, len(rows), chunk):
            rr = rows[r0:r0 + chunk]
            mask = hilbert_allowed_mask(rr, image, int(window_lens[h]), mode, text_length, has_text)
            for b in range(B):
                scores = np.where(mask, (q64[b, h, rr] @ k64[b, h].T) * scale, -np.inf)
                mx = scores.max(axis=1, keepdims=True)
                p = np.exp(scores - mx)
                l = p.sum(axis=1, keepdims=True)
                out[b, h, r0:r0 + len(rr)] = (p @ v64[b, h]) / l
                lse[b, h, r0:r0 + len(rr)] = (mx + np.log(l))[:, 0]
    return out, lse


# ---- block statistics of token-level 2D patterns under an ordering (the post's claim)

def neighborhood_mask(side: int, radius: int) -> np.ndarray:
    """mask[a, b] for raster tokens a, b of a side x side image: |dx| <= r and |dy| <= r."""
    y, x = np.divmod(np.arange(side * side), side)
    return (np.abs(x[:, None] - x[None, :]) <= radius) & (np.abs(y[:, None] - y[None, :]) <= radius)


def square_window_mask(side: int, w: int) -> np.ndarray:
    """mask[a, b]: a and b lie in the same aligned w x w window (non-overlapping windows)."""
    y, x = np.divmod(np.arange(side * side), side)
    wid = (y // w) * (side // w + (side % w > 0)) + x // w
    return wid[:, None] == wid[None, :]


def block_counts(mask: np.ndarray, perm: np.ndarray, block: int = BLOCK) -> dict:
    """Counts of (query block, key block) pairs of a token mask taken in order ``perm``.

    ``perm[d]`` is the raster index of the d-th token of the order. A block is
    empty (no allowed pair), full (every pair allowed) or partial.
    """
    n = mask.shape[0]
    if n % block:
        raise ValueError("token count must be a multiple of the block")
    reordered = mask[np.ix_(perm, perm)]
    nb = n // block
    per_block = reordered.reshape(nb, block, nb, block).sum(axis=(1, 3))
    full = int((per_block == block * block).sum())
    empty = int((per_block == 0).sum())
    return {"blocks": nb * nb, "empty": empty, "full": full, "partial": nb * nb - empty - full}
