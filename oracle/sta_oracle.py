"""Plain fp64 CPU oracle for Sliding Tile Attention (STA): forward pass and its gradients.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the HIP library, with which it shares
no code.

Source: the README of the "Sliding Tile Atteniton Kernel" page (FastVideo,
``sta_kernel/thunderkitten``), sections "Usage" and "Why is STA Fast?".
What that page fixes, restated:

* q, k, v are ``[batch, heads, seq, head_dim]`` with ``seq = T*H*W + 256``
  when a text segment is present (Usage).
* the video is cut into tiles that are cubes of (6, 8, 8) tokens (Usage);
  the page's sizes are multiples of the tile;
* each head has a window given in tiles ``(w_t, w_h, w_w)``; a window of
  (3, 3, 3) lets a query see (18, 24, 24) video tokens of the (30, 48, 80)
  video (Usage, the window example);
* the text length is an integer in [0, 256]; with text (HunyuanVideo style)
  the call passes it, without text (StepVideo style) it passes 0 and False
  (Usage);
* attention is exact softmax attention whose map holds only fully-dense or
  fully-empty tile blocks, with no mixed blocks (Why is STA Fast?).

Readings where the page is silent:

* video tokens come in raster order (t slowest, w fastest), the text slots
  follow the video, and the valid text slots are the first ``text_length``;
* at the grid border the window is shifted, not truncated: its start along
  each axis is ``clamp(c - w // 2, 0, n - w)`` so every video query sees
  exactly ``w_t*w_h*w_w`` tiles, matching the page's fixed (18, 24, 24) count;
* video queries also see the valid text keys; text queries (all 256 slots,
  padded ones included) see every video key and the valid text keys;
* the softmax scale is ``1/sqrt(head_dim)``; ``lse`` is the natural log of
  the sum of ``exp(q.k * scale)`` over the allowed keys;
* a video size that is not a multiple of the tile is covered by the same
  grid of tiles, the last tile along that axis holding the remainder:
  windows are placed on that grid (``n = ceil(size / tile)`` tiles per
  axis) and a query sees the tokens that exist in its window tiles.

Precision: inputs are upcast exactly to float64 and everything is computed
in float64. The computation is the plain definition: an explicit
token-level boolean mask built from token coordinates (no tile list), a
dense masked softmax over all keys, and a dense product with V.

The gradients (``sta_reference_backward``) are those of that same function
with respect to q, k and v for an upstream gradient ``dout`` of the output:
the chain rule through the masked softmax, written out. The page shows only
the forward call; the backward is defined by it and by nothing else.
"""

from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

TILE = (6, 8, 8)       # tile cube in tokens (t, h, w), from the Usage section
TEXT_SLOTS = 256       # padded text segment, from the Usage section


def _as_np64(x) -> np.ndarray:
    """Upcast a torch tensor (any dtype, bf16 included) or array to float64."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover - torch is always present here
        pass
    return np.asarray(x, dtype=np.float64)


def softmax_scale(head_dim: int) -> float:
    """Scale applied to q.k before the softmax: 1/sqrt(head_dim) (a reading)."""
    return 1.0 / np.sqrt(head_dim)


def window_start(c: int, w: int, n: int) -> int:
    """First tile of a window of ``w`` tiles around tile ``c`` on an axis of ``n``.

    The window is centred on the query's tile when it fits and is shifted
    inward at the border so that it always holds exactly ``w`` tiles (the
    Usage section's (3,3,3) -> (18,24,24) example states one fixed count).
    """
    if not (1 <= w <= n):
        raise ValueError(f"window {w} must lie in [1, {n}]")
    return min(max(c - w // 2, 0), n - w)


def _video_tile_coords(video: Tuple[int, int, int]):
    """Tile coordinates (tile_t, tile_h, tile_w) of every video token, raster order."""
    T, H, W = video
    t = np.arange(T).repeat(H * W)
    h = np.tile(np.arange(H).repeat(W), T)
    w = np.tile(np.arange(W), T * H)
    return t // TILE[0], h // TILE[1], w // TILE[2]


def _check_video(video):
    """Tile-grid size: the (6, 8, 8) tiles that cover the video; when a size is not a
    multiple of the tile, the last tile along that axis holds the remainder (a reading)."""
    T, H, W = video
    if min(video) <= 0:
        raise ValueError(f"video {video} must have positive sizes")
    return -(-T // TILE[0]), -(-H // TILE[1]), -(-W // TILE[2])


def allowed_mask(rows: Sequence[int], video: Tuple[int, int, int],
                 window: Tuple[int, int, int], text_length: int,
                 has_text: bool) -> np.ndarray:
    """Explicit token-level mask: ``mask[r, j]`` is True iff query ``rows[r]`` may see key ``j``.

    Row and key indices are sequence positions: video tokens in raster order
    first, then (when ``has_text``) the 256 text slots.
    """
    n_t, n_h, n_w = _check_video(video)
    T, H, W = video
    n_video = T * H * W
    seq = n_video + (TEXT_SLOTS if has_text else 0)
    if not has_text and text_length != 0:
        raise ValueError("text_length must be 0 without text")
    if not 0 <= text_length <= TEXT_SLOTS:
        raise ValueError("text_length must lie in [0, 256]")
    rows = np.asarray(rows, dtype=np.int64)
    kt, kh, kw = _video_tile_coords(video)
    mask = np.zeros((len(rows), seq), dtype=bool)
    for r, i in enumerate(rows):
        if i < n_video:
            t, h, w = i // (H * W), (i // W) % H, i % W
            c = (t // TILE[0], h // TILE[1], w // TILE[2])
            s_t = window_start(c[0], window[0], n_t)
            s_h = window_start(c[1], window[1], n_h)
            s_w = window_start(c[2], window[2], n_w)
            mask[r, :n_video] = ((kt >= s_t) & (kt < s_t + window[0])
                                 & (kh >= s_h) & (kh < s_h + window[1])
                                 & (kw >= s_w) & (kw < s_w + window[2]))
        elif i < seq:
            mask[r, :n_video] = True
        else:
            raise IndexError(f"row {i} out of range for sequence length {seq}")
        if has_text:
            mask[r, n_video:n_video + text_length] = True
    return mask


def key_tiles_of_query_tile(video: Tuple[int, int, int], window: Tuple[int, int, int],
                            query_tile: int) -> list:
    """Key tiles a query tile sees, read off the token mask by brute force.

    ``query_tile`` is a raster tile index ``(tt*n_h + th)*n_w + tw``; every
    one of its 384 tokens' mask rows is built and the union of the key tiles
    they touch is returned in ascending raster tile order. (Text keys are not
    tiles and are left out.)
    """
    n_t, n_h, n_w = _check_video(video)
    T, H, W = video
    tt, rem = divmod(query_tile, n_h * n_w)
    th, tw = divmod(rem, n_w)
    rows = []
    for t in range(tt * TILE[0], min(T, tt * TILE[0] + TILE[0])):
        for h in range(th * TILE[1], min(H, th * TILE[1] + TILE[1])):
            for w in range(tw * TILE[2], min(W, tw * TILE[2] + TILE[2])):
                rows.append((t * H + h) * W + w)
    m = allowed_mask(rows, video, window, 0, False)
    kt, kh, kw = _video_tile_coords(video)
    tile_of_key = (kt * n_h + kh) * n_w + kw
    seen = np.unique(tile_of_key[m.any(axis=0)])
    return [int(x) for x in seen]


def sta_reference(q, k, v, window_sizes, text_length: int, has_text: bool,
                  video: Tuple[int, int, int], rows: Optional[Iterable[int]] = None,
                  chunk: int = 128):
    """STA forward in float64: dense softmax attention under the explicit token mask.

    Arguments follow the page's call ``sliding_tile_attention(q, k, v,
    window_size, text_length[, has_text])``, plus the video shape the page
    assumes implicitly.

    q, k, v: ``[B, heads, S, D]`` tensors or arrays (bf16 values are upcast
    exactly). ``window_sizes``: one ``(w_t, w_h, w_w)`` per head, or a single
    triple for all heads. ``rows``: optional query positions to evaluate
    (each is still computed densely over all S keys).

    Returns ``(out, lse)`` as float64 arrays ``[B, heads, R, D]`` and
    ``[B, heads, R]`` where R is ``S`` or ``len(rows)``; rows keep the input's
    sequence order.
    """
    q64, k64, v64 = _as_np64(q), _as_np64(k), _as_np64(v)
    B, heads, S, D = q64.shape
    n_video = video[0] * video[1] * video[2]
    if S != n_video + (TEXT_SLOTS if has_text else 0):
        raise ValueError(f"sequence length {S} does not match video {video} / text {has_text}")
    if k64.shape != q64.shape or v64.shape != q64.shape:
        raise ValueError("q, k, v must share one shape")
    if len(window_sizes) == 3 and np.isscalar(window_sizes[0]):
        window_sizes = [tuple(window_sizes)] * heads
    if len(window_sizes) != heads:
        raise ValueError("one window per head is required")
    rows = np.arange(S) if rows is None else np.asarray(list(rows), dtype=np.int64)
    scale = softmax_scale(D)
    out = np.empty((B, heads, len(rows), D))
    lse = np.empty((B, heads, len(rows)))
    for h in range(heads):
        win = tuple(int(x) for x in window_sizes[h])
        for r0 in range(0, len(rows), chunk):
            rr = rows[r0:r0 + chunk]
            mask = allowed_mask(rr, video, win, text_length, has_text)
            for b in range(B):
                scores = (q64[b, h, rr] @ k64[b, h].T) * scale
                scores = np.where(mask, scores, -np.inf)
                m = scores.max(axis=1, keepdims=True)
                p = np.exp(scores - m)
                l = p.sum(axis=1, keepdims=True)
                out[b, h, r0:r0 + len(rr)] = (p @ v64[b, h]) / l
                lse[b, h, r0:r0 + len(rr)] = (m + np.log(l))[:, 0]
    return out, lse


def query_rows_seeing(key_rows: Sequence[int], video: Tuple[int, int, int],
                      window: Tuple[int, int, int], text_length: int,
                      has_text: bool) -> np.ndarray:
    """Every query position whose mask row allows at least one of ``key_rows``.

    Video query tiles are tested one at a time with the same window rule
    ``allowed_mask`` applies to their tokens (all 384 tokens of a tile share
    one window); every text query sees every video key and every valid text
    key. Used to restrict a key-side gradient to the rows that reach it.
    """
    n_t, n_h, n_w = _check_video(video)
    T, H, W = video
    n_video = T * H * W
    key_rows = np.asarray(key_rows, dtype=np.int64)
    vid_keys = key_rows[key_rows < n_video]
    txt_keys = key_rows[key_rows >= n_video]
    if np.any(txt_keys >= n_video + (TEXT_SLOTS if has_text else 0)):
        raise IndexError("key row out of range")
    # key tiles touched by the requested video keys
    kt = (vid_keys // (H * W)) // TILE[0]
    kh = ((vid_keys // W) % H) // TILE[1]
    kw = (vid_keys % W) // TILE[2]
    touched = set(zip(kt.tolist(), kh.tolist(), kw.tolist()))
    sees_text = bool(np.any(txt_keys < n_video + text_length)) if has_text else False
    rows = []
    for tt in range(n_t):
        for th in range(n_h):
            for tw in range(n_w):
                s_t = window_start(tt, window[0], n_t)
                s_h = window_start(th, window[1], n_h)
                s_w = window_start(tw, window[2], n_w)
                hit = sees_text or any(s_t <= a < s_t + window[0] and s_h <= b < s_h + window[1]
                                       and s_w <= c < s_w + window[2] for a, b, c in touched)
                if not hit:
                    continue
                for t in range(tt * TILE[0], min(T, tt * TILE[0] + TILE[0])):
                    for h in range(th * TILE[1], min(H, th * TILE[1] + TILE[1])):
                        base = (t * H + h) * W + tw * TILE[2]
                        rows.extend(range(base, base + min(TILE[2], W - tw * TILE[2])))
    if has_text and (len(vid_keys) > 0 or sees_text):
        rows.extend(range(n_video, n_video + TEXT_SLOTS))
    return np.unique(np.asarray(rows, dtype=np.int64))


def _masked_probabilities(q64, k64, rr, mask, scale):
    """Softmax probabilities of query rows ``rr`` over all keys (0 where masked), fp64."""
    scores = (q64[rr] @ k64.T) * scale
    scores = np.where(mask, scores, -np.inf)
    m = scores.max(axis=1, keepdims=True)
    p = np.exp(scores - m)
    return p / p.sum(axis=1, keepdims=True)


def sta_reference_backward(q, k, v, dout, window_sizes, text_length: int, has_text: bool,
                           video: Tuple[int, int, int],
                           query_rows: Optional[Iterable[int]] = None,
                           key_rows: Optional[Iterable[int]] = None, chunk: int = 256):
    """Gradients of ``sta_reference``'s output, float64.

    For a query row i, allowed keys j and scale c = 1/sqrt(head_dim):
    ``p_ij = softmax_j(c q_i.k_j)`` (0 for masked j), ``out_i = sum_j p_ij v_j``.
    With ``dout`` the gradient of a scalar loss with respect to ``out``:

    * ``dv_j = sum_i p_ij dout_i``;
    * ``dp_ij = dout_i . v_j`` and ``delta_i = sum_j p_ij dp_ij`` (which
      equals ``dout_i . out_i``);
    * ``ds_ij = p_ij (dp_ij - delta_i)``, the gradient of the scaled score;
    * ``dq_i = c sum_j ds_ij k_j`` and ``dk_j = c sum_i ds_ij q_i``.

    ``query_rows`` selects the dq rows returned and ``key_rows`` the dk/dv
    rows (default: all). A key row's gradient sums over every query row that
    sees it, so those rows are all evaluated, each densely over all S keys.

    Returns ``(dq, dk, dv)`` as float64 arrays ``[B, heads, Rq, D]``,
    ``[B, heads, Rk, D]``, ``[B, heads, Rk, D]``.
    """
    q64, k64, v64, do64 = _as_np64(q), _as_np64(k), _as_np64(v), _as_np64(dout)
    B, heads, S, D = q64.shape
    n_video = video[0] * video[1] * video[2]
    if S != n_video + (TEXT_SLOTS if has_text else 0):
        raise ValueError(f"sequence length {S} does not match video {video} / text {has_text}")
    for x in (k64, v64, do64):
        if x.shape != q64.shape:
            raise ValueError("q, k, v, dout must share one shape")
    if len(window_sizes) == 3 and np.isscalar(window_sizes[0]):
        window_sizes = [tuple(window_sizes)] * heads
    if len(window_sizes) != heads:
        raise ValueError("one window per head is required")
    qrows = np.arange(S) if query_rows is None else np.asarray(list(query_rows), dtype=np.int64)
    krows = np.arange(S) if key_rows is None else np.asarray(list(key_rows), dtype=np.int64)
    scale = softmax_scale(D)
    dq = np.zeros((B, heads, len(qrows), D))
    dk = np.zeros((B, heads, len(krows), D))
    dv = np.zeros((B, heads, len(krows), D))
    for h in range(heads):
        win = tuple(int(x) for x in window_sizes[h])
        need = (np.arange(S) if key_rows is None
                else query_rows_seeing(krows, video, win, text_length, has_text))
        for b in range(B):
            qb, kb, vb, dob = q64[b, h], k64[b, h], v64[b, h], do64[b, h]
            # query side: dq
            for r0 in range(0, len(qrows), chunk):
                rr = qrows[r0:r0 + chunk]
                p = _masked_probabilities(qb, kb, rr, allowed_mask(rr, video, win, text_length,
                                                                   has_text), scale)
                dp = dob[rr] @ vb.T
                delta = (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - delta)
                dq[b, h, r0:r0 + len(rr)] = scale * (ds @ kb)
            # key side: dk, dv, summed over every query row that reaches the keys
            for r0 in range(0, len(need), chunk):
                rr = need[r0:r0 + chunk]
                p = _masked_probabilities(qb, kb, rr, allowed_mask(rr, video, win, text_length,
                                                                   has_text), scale)
                dp = dob[rr] @ vb.T
                delta = (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - delta)
                dk[b, h] += scale * (ds[:, krows].T @ qb[rr])
                dv[b, h] += p[:, krows].T @ dob[rr]
    return dq, dk, dv
