"""GPU parity of the STA backward (through the C ABI) with the fp64 oracle.

The forward's out and lse come from the HIP forward on the same inputs; the
oracle differentiates its own exact forward. Gradients start as NaN, so an
unwritten row fails every check.

Tolerance, per (batch, head) tensor, from the arithmetic: P and dS enter
their products rounded to bf16 (relative 2^-9 each), the products accumulate
in fp32, and the result is rounded to bf16 (2^-9). With independent rounding
errors the relative RMS error is a few times 2^-9 ~ 2e-3; the test allows
1e-2, and a largest element error of 2e-2 of the tensor's largest magnitude.
"""

import numpy as np
import pytest
import torch

import oracle
import sta_inputs
import block_sparse_sliding_amd as sta
from _parity import map_heads, note, run_sta, scale_key_tiles

pytestmark = pytest.mark.gpu

REL_RMS = 1e-2
MAX_REL = 2e-2
BWD_DQ_ROWS = 256  # sampled dq rows per head at full size


def run_backward(q, k, v, out, lse, dout, windows, ell, has_text, video):
    B, heads, S, D = q.shape
    dims = sta.make_dims(B, heads, D, video)
    need = sta.sta_backward_workspace_bytes(dims, windows, has_text)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    sta.sta_backward(dims, q, k, v, out, lse, dout, windows, ell, has_text, dq, dk, dv, ws)
    torch.cuda.synchronize()
    return dq, dk, dv


def compare_grad(got, ref, label):
    """got: torch [B, heads, R, D] (any float), ref: numpy float64 of the same shape."""
    g = got.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(g).all(), f"{label}: non-finite gradient"
    worst = {}
    for b in range(ref.shape[0]):
        for h in range(ref.shape[1]):
            r = ref[b, h]
            e = g[b, h] - r
            scale = np.abs(r).max()
            rms = np.sqrt((r ** 2).mean())
            if scale == 0:
                assert np.all(e == 0), (label, b, h)
                continue
            stats = dict(rel_rms=float(np.sqrt((e ** 2).mean()) / rms),
                         max_rel=float(np.abs(e).max() / scale))
            for kk, vv in stats.items():
                worst[kk] = max(worst.get(kk, 0.0), vv)
    print(f"[parity] {label} {worst}", flush=True)
    assert worst.get("rel_rms", 0.0) <= REL_RMS, (label, worst)
    assert worst.get("max_rel", 0.0) <= MAX_REL, (label, worst)
    return worst


def inputs(B, heads, S, D, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return [torch.randn(B, heads, S, D, generator=g, device="cuda").to(torch.bfloat16)
            for _ in range(4)]


SMALL = [
    # video, windows, ell, has_text, D, B
    ((12, 16, 16), [(1, 2, 1), (2, 1, 2)], 100, True, 128, 1),
    ((12, 16, 16), [(2, 2, 2)], 0, False, 128, 2),
    ((12, 16, 24), [(1, 1, 3), (2, 2, 1)], 37, True, 64, 1),
    ((18, 16, 16), [(3, 1, 1)], 256, True, 128, 1),
    ((12, 16, 16), [(1, 1, 1)], 0, True, 128, 1),
    ((6, 8, 8), [(1, 1, 1)], 64, True, 64, 1),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"s{i}" for i in range(len(SMALL))])
def test_backward_small_all_rows(case):
    video, windows, ell, has_text, D, B = case
    heads = len(windows)
    S = video[0] * video[1] * video[2] + (256 if has_text else 0)
    note(f"backward small {case}")
    q, k, v, dout = inputs(B, heads, S, D, 1000 + S + D + ell)
    out, lse = run_sta(q, k, v, windows, ell, has_text, video)
    dq, dk, dv = run_backward(q, k, v, out, lse, dout, windows, ell, has_text, video)
    rq, rk, rv = oracle.sta_reference_backward(q.cpu(), k.cpu(), v.cpu(), dout.cpu(), windows,
                                               ell, has_text, video)
    compare_grad(dq, rq, f"dq {case}")
    compare_grad(dk, rk, f"dk {case}")
    compare_grad(dv, rv, f"dv {case}")
    if has_text:
        nv = S - 256
        assert bool((dk[:, :, nv + ell:] == 0).all()) and bool((dv[:, :, nv + ell:] == 0).all())


def test_backward_padding_never_reaches_gradients():
    """Padded text K/V (even NaN/inf) change no gradient bit."""
    video, windows, ell = (12, 16, 16), [(1, 2, 1), (2, 1, 2)], 77
    nv = video[0] * video[1] * video[2]
    S = nv + 256
    note("backward padding isolation")
    q, k, v, dout = inputs(1, 2, S, 128, 55)
    out, lse = run_sta(q, k, v, windows, ell, True, video)
    g1 = run_backward(q, k, v, out, lse, dout, windows, ell, True, video)
    k2, v2 = k.clone(), v.clone()
    k2[:, :, nv + ell:] = float("nan")
    v2[:, :, nv + ell:] = float("inf")
    g2 = run_backward(q, k2, v2, out, lse, dout, windows, ell, True, video)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_backward_large_score_jumps():
    """Key tiles scaled by 0.05 .. 4 and text keys by 3.5: logits spread over tens of
    log2 units, so P is recomputed far from the row maximum on many blocks."""
    video, windows, ell, D = (12, 16, 24), [(1, 2, 2), (2, 1, 3)], 100, 128
    S = video[0] * video[1] * video[2] + 256
    note("backward score jumps")
    q, k, v, dout = inputs(1, 2, S, D, 4242)
    k = scale_key_tiles(k, video, {(0, 0, 1): 2.5, (1, 1, 2): 4.0, (0, 1, 0): 0.05}, 3.5, ell)
    out, lse = run_sta(q, k, v, windows, ell, True, video)
    dq, dk, dv = run_backward(q, k, v, out, lse, dout, windows, ell, True, video)
    rq, rk, rv = oracle.sta_reference_backward(q.cpu(), k.cpu(), v.cpu(), dout.cpu(), windows,
                                               ell, True, video)
    compare_grad(dq, rq, "dq jumps")
    compare_grad(dk, rk, "dk jumps")
    compare_grad(dv, rv, "dv jumps")


MEDIUM = [
    ((18, 24, 32), [(1, 2, 2), (2, 1, 3)], 226, True, 128),
    ((18, 24, 32), [(3, 3, 2)], 0, False, 64),
]


@pytest.mark.parametrize("case", MEDIUM, ids=[f"m{i}" for i in range(len(MEDIUM))])
def test_backward_medium_sampled(case):
    video, windows, ell, has_text, D = case
    heads = len(windows)
    nv = video[0] * video[1] * video[2]
    S = nv + (256 if has_text else 0)
    note(f"backward medium {case}")
    q, k, v, dout = inputs(1, heads, S, D, 2000 + S + D)
    out, lse = run_sta(q, k, v, windows, ell, has_text, video)
    dq, dk, dv = run_backward(q, k, v, out, lse, dout, windows, ell, has_text, video)
    rng = np.random.default_rng(S)
    qrows = np.unique(np.concatenate([rng.integers(0, S, 200), [0, nv - 1, S - 1]]))
    # two key tiles (all 384 rows each) and, with text, the first and last valid text keys
    T, H, W = video
    keys = []
    for tile in (0, (video[0] // 6) * (video[1] // 8) * (video[2] // 8) - 1):
        tt, rest = divmod(tile, (H // 8) * (W // 8))
        th, tw = divmod(rest, W // 8)
        for dt in range(6):
            for dh in range(8):
                base = ((tt * 6 + dt) * H + th * 8 + dh) * W + tw * 8
                keys.extend(range(base, base + 8))
    if has_text and ell > 0:
        keys += [nv, nv + ell - 1]
    keys = np.unique(np.asarray(keys))
    for h in range(heads):
        sl = slice(h, h + 1)
        rq, rk, rv = oracle.sta_reference_backward(
            q[:, sl].cpu(), k[:, sl].cpu(), v[:, sl].cpu(), dout[:, sl].cpu(), [windows[h]], ell,
            has_text, video, query_rows=qrows, key_rows=keys)
        compare_grad(dq[:, sl][:, :, torch.from_numpy(qrows)], rq, f"dq {case} head {h}")
        compare_grad(dk[:, sl][:, :, torch.from_numpy(keys)], rk, f"dk {case} head {h}")
        compare_grad(dv[:, sl][:, :, torch.from_numpy(keys)], rv, f"dv {case} head {h}")
    assert bool(torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all())


def tile_rows(video, tile):
    """Raster rows of the tokens of video tile (tt, th, tw) that exist."""
    T, H, W = video
    tt, th, tw = tile
    return [(t * H + h) * W + w
            for t in range(6 * tt, min(T, 6 * tt + 6))
            for h in range(8 * th, min(H, 8 * th + 8))
            for w in range(8 * tw, min(W, 8 * tw + 8))]


def corner_tiles(video, corner, interior):
    """Key tiles near one corner of the tile grid: the corner tile, the edge tile
    next to it along w, and (interior=True) the tile one step in along every axis
    (not on the border of any axis when the grid has at least 3 tiles per axis).
    corner: 3 bits, bit a set = the high end of axis a."""
    n = tuple(-(-s // t) for s, t in zip(video, (6, 8, 8)))

    def at(offsets):
        return tuple((m - 1 - o) if (corner >> a) & 1 else o for a, (m, o) in
                     enumerate(zip(n, offsets)))

    tiles = [at((0, 0, 0)), at((0, 0, 1))]
    if interior:
        tiles.append(at((1, 1, 1)))
    return tiles


def check_heads(q, k, v, dout, dq, dk, dv, windows, ell, has_text, video, heads, qrows_of,
                key_tiles_of, label):
    """Oracle backward of each listed head (on a thread pool): dq on the head's
    own query rows, dk and dv on every row of the head's key tiles."""
    host = [x.cpu() for x in (q, k, v, dout)]

    def one(h):
        keys = sorted({r for t in key_tiles_of(h) for r in tile_rows(video, t)})
        sl = slice(h, h + 1)
        ref = oracle.sta_reference_backward(*(x[:, sl] for x in host), [windows[h]], ell, has_text,
                                            video, query_rows=qrows_of(h), key_rows=keys)
        return keys, ref

    for h, (keys, (rq, rk, rv)) in zip(heads, map_heads(one, heads)):
        sl = slice(h, h + 1)
        qi = torch.as_tensor(np.asarray(qrows_of(h)), dtype=torch.int64)
        ki = torch.as_tensor(np.asarray(keys), dtype=torch.int64)
        compare_grad(dq[:, sl][:, :, qi], rq, f"dq {label} head {h}")
        if len(keys):
            compare_grad(dk[:, sl][:, :, ki], rk, f"dk {label} head {h} tiles {key_tiles_of(h)}")
            compare_grad(dv[:, sl][:, :, ki], rv, f"dv {label} head {h} tiles {key_tiles_of(h)}")


def sum_rules(dout, dq, dk, dv):
    """sum_j dv_j = sum_i dout_i and sum_j dk_j = 0, per (batch, head), in fp64."""
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert bool(torch.isfinite(t).all()), name
    sdv = dv.double().sum(dim=2)
    sdo = dout.double().sum(dim=2)
    sdk = dk.double().sum(dim=2)
    dv_scale = dv.double().abs().sum(dim=2)
    dk_scale = dk.double().abs().sum(dim=2)
    assert bool(((sdv - sdo).abs() <= 1e-2 * dv_scale + 1e-3).all())
    assert bool((sdk.abs() <= 1e-2 * dk_scale + 1e-3).all())


def test_backward_full_size():
    """(30,48,80) + 256 text at D = 128 with four different windows: every
    gradient written, sum rules on every head, 256 dq rows per head (its own
    stratified draw), and dk/dv on whole key tiles: a corner, an edge and an
    interior tile of the (1,1,1) head, a corner and an edge tile of the
    (3,3,3) and (3,3,5) heads (the (5,6,10) head sees every key from every
    query, so any key tile needs every query row: the sum rules cover it)."""
    wl = sta_inputs.WORKLOADS["headline"]
    video = wl.video
    heads = 4
    windows = [(1, 1, 1), (3, 3, 3), (5, 6, 10), (3, 3, 5)]
    ell = wl.text_length
    nv = video[0] * video[1] * video[2]
    S = nv + 256
    note(f"backward full size {video}+256, {heads} heads, windows {windows}")
    q, k, v, dout = inputs(1, heads, S, 128, 77)
    out, lse = run_sta(q, k, v, windows, ell, True, video)
    dq, dk, dv = run_backward(q, k, v, out, lse, dout, windows, ell, True, video)
    sum_rules(dout, dq, dk, dv)
    wl4 = sta_inputs.custom("bwd4", 1, heads, 128, video, windows, True, ell)
    qrows = {h: sta_inputs.sample_rows_stratified(wl4, BWD_DQ_ROWS, h).numpy() for h in range(heads)}
    tiles = {0: corner_tiles(video, 5, True), 1: corner_tiles(video, 2, False), 2: [],
             3: corner_tiles(video, 7, False)}
    check_heads(q, k, v, dout, dq, dk, dv, windows, ell, True, video, range(heads),
                qrows.__getitem__, tiles.__getitem__, "full")
    del q, k, v, dout, out, lse, dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("part", [0, 1])
def test_backward_headline_all_heads(part):
    """The benchmarked backward configuration ((30,48,80) + 256 text, 24 heads,
    window (3,3,3), text length 226, its seeded inputs): sum rules on every
    head; for half of the heads (``part``), 256 dq rows per head (its own
    stratified draw) and dk/dv on whole key tiles at one corner of the grid,
    a different corner per head: the corner tile and the edge tile next to it,
    and on every third head also the interior tile one step in on every axis."""
    wl = sta_inputs.WORKLOADS["headline"]
    windows = list(wl.windows)
    note(f"backward headline, all heads, part {part}")
    q, k, v = sta_inputs.make_qkv(wl, "cuda")
    g = torch.Generator(device="cuda").manual_seed(10 * wl.seed_base + 3)
    dout = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    out, lse = run_sta(q, k, v, windows, wl.text_length, wl.has_text, wl.video)
    dq, dk, dv = run_backward(q, k, v, out, lse, dout, windows, wl.text_length, wl.has_text,
                              wl.video)
    sum_rules(dout, dq, dk, dv)
    heads = list(range(part, wl.heads, 2))
    qrows = {h: sta_inputs.sample_rows_stratified(wl, BWD_DQ_ROWS, h, seed=23).numpy()
             for h in heads}
    tiles = {h: corner_tiles(wl.video, h % 8, h % 3 == 0) for h in heads}
    check_heads(q, k, v, dout, dq, dk, dv, windows, wl.text_length, wl.has_text, wl.video, heads,
                qrows.__getitem__, tiles.__getitem__, "headline")
    del q, k, v, dout, out, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_autograd_glue_matches_direct_calls():
    """loss.backward() through sliding_tile_attention_autograd gives exactly the
    gradients of a direct sta_backward call (the glue adds no arithmetic)."""
    video, windows, ell = (12, 16, 16), [(1, 2, 1), (2, 1, 2)], 90
    S = video[0] * video[1] * video[2] + 256
    note("autograd glue")
    q, k, v, dout = inputs(1, 2, S, 128, 31)
    qq, kk, vv = (x.clone().requires_grad_(True) for x in (q, k, v))
    out = sta.sliding_tile_attention_autograd(qq, kk, vv, windows, ell, True, video)
    out.backward(dout)
    torch.cuda.synchronize()
    o2, l2 = run_sta(q, k, v, windows, ell, True, video)
    assert torch.equal(out.detach().view(torch.int16), o2.view(torch.int16))
    g = run_backward(q, k, v, o2, l2, dout, windows, ell, True, video)
    for a, b in zip((qq.grad, kk.grad, vv.grad), g):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
