"""GPU checks of properties that hold at any size (through the C ABI).

* q = 0 closed form: every allowed score is 0, so lse = ln(count) and the
  output is the mean of the allowed v rows; with v carrying each key's tile
  coordinates this pins the window placement on every row, at full size,
  also for sizes that are not tile multiples (partial last tiles).
* padded text K/V rows never reach the result (bitwise).
* repeated calls are bitwise identical; batch entries are independent.
* lse is optional: without it, out is the same to the bit.
* the maximum head count (256), with per-head windows, forward and backward.
"""

import math

import numpy as np
import pytest
import torch

import block_sparse_sliding_amd as sta
import sta_inputs
from _parity import note, run_sta

pytestmark = pytest.mark.gpu

TILE = (6, 8, 8)


def nearest_box_start(c, w, n):
    """Placement of w tiles inside [0, n) whose centre is nearest to c (ties: lower)."""
    c = np.asarray(c)
    best_d = np.full(c.shape, np.inf)
    best_s = np.zeros(c.shape, dtype=np.int64)
    for s in range(0, n - w + 1):
        d = np.abs(s + (w - 1) / 2.0 - c)
        better = d < best_d
        best_d = np.where(better, d, best_d)
        best_s = np.where(better, s, best_s)
    return best_s


def coord_inputs(B, heads, D, video, has_text, seed=0):
    T, H, W = video
    nv = T * H * W
    S = nv + (256 if has_text else 0)
    q = torch.zeros(B, heads, S, D, dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(seed)
    k = torch.randn(B, heads, S, D, generator=g, device="cuda").to(torch.bfloat16)
    v = torch.zeros(B, heads, S, D, dtype=torch.bfloat16, device="cuda")
    t = torch.arange(T, device="cuda").repeat_interleave(H * W)
    h = torch.arange(H, device="cuda").repeat_interleave(W).repeat(T)
    w = torch.arange(W, device="cuda").repeat(T * H)
    v[:, :, :nv, 0] = (t // 6).to(torch.bfloat16)
    v[:, :, :nv, 1] = (h // 8).to(torch.bfloat16)
    v[:, :, :nv, 2] = (w // 8).to(torch.bfloat16)
    if has_text:
        v[:, :, nv:, 3] = 1
    return q, k, v


def expected_uniform(video, window, ell, has_text):
    """Closed-form output columns 0..3 and lse for q = 0, every row.

    Any video size: the tile grid along an axis has ceil(size/tile) tiles, the
    last holding the remainder. The allowed video keys of a row form a box, so
    their count is the product of the per-axis spans and the mean tile
    coordinate along an axis is that axis' token-weighted mean.
    """
    T, H, W = video
    nv = T * H * W
    n = [-(-video[a] // TILE[a]) for a in range(3)]
    sizes = [np.array([min(TILE[a], video[a] - i * TILE[a]) for i in range(n[a])])
             for a in range(3)]
    coords = (np.arange(T).repeat(H * W), np.tile(np.arange(H).repeat(W), T),
              np.tile(np.arange(W), T * H))
    span = np.ones(nv)
    mean = []
    for a, x in enumerate(coords):
        tiles = x // TILE[a]
        lo = {c: int(nearest_box_start(c, window[a], n[a])) for c in range(n[a])}
        start = np.vectorize(lo.get)(tiles)
        idx = start[:, None] + np.arange(window[a])[None, :]
        sz = sizes[a][idx]
        span = span * sz.sum(axis=1)
        mean.append((idx * sz).sum(axis=1) / sz.sum(axis=1))
    cnt = span + ell
    vid = np.stack([m * span / cnt for m in mean] + [ell / cnt], axis=1)
    lse = np.log(cnt)
    if has_text:
        ctext = nv + ell
        txt = np.array([(np.arange(n[a]) * sizes[a]).sum() / video[a] * nv / ctext
                        for a in range(3)] + [ell / ctext])
        vid = np.concatenate([vid, np.tile(txt, (256, 1))])
        lse = np.concatenate([lse, np.full(256, math.log(ctext))])
    return vid, lse


@pytest.mark.parametrize("video,windows,ell,has_text,D", [
    ((18, 24, 32), [(3, 3, 3), (1, 2, 3), (2, 1, 4)], 77, True, 128),
    ((30, 48, 80), [(3, 3, 3), (3, 3, 5)], 226, True, 128),
    ((30, 48, 80), [(5, 6, 10), (3, 3, 3), (1, 6, 10), (5, 1, 1)], 256, True, 128),
    ((30, 48, 80), [(3, 3, 3)], 0, False, 128),
    ((48, 72, 128), [(3, 3, 3)], 128, True, 128),
    ((18, 24, 24), [(1, 3, 3)], 0, False, 64),
    # sizes that are not tile multiples (partial last tiles)
    ((33, 45, 80), [(3, 3, 3), (1, 2, 4)], 226, True, 128),
    ((17, 21, 30), [(2, 2, 3), (3, 1, 1)], 100, True, 128),
    ((1, 12, 20), [(1, 2, 3)], 0, False, 64),
    ((13, 9, 33), [(3, 2, 5)], 256, True, 64),
])
def test_uniform_attention_closed_form(video, windows, ell, has_text, D):
    heads = len(windows)
    note(f"q=0 closed form {video} {windows} ell={ell} text={has_text} D={D}")
    q, k, v = coord_inputs(1, heads, D, video, has_text)
    out, lse = run_sta(q, k, v, windows, ell, has_text, video)
    for hd, win in enumerate(windows):
        exp_out, exp_lse = expected_uniform(video, win, ell, has_text)
        got = out[0, hd, :, :4].float().cpu().numpy()
        gl = lse[0, hd].cpu().numpy().astype(np.float64)
        # bf16 rounding of the output: half an ulp, 2^-9 relative
        assert np.all(np.abs(got - exp_out) <= np.abs(exp_out) * 2.0 ** -8 + 1e-6), (hd, win)
        assert np.all(out[0, hd, :, 4:].float().cpu().numpy() == 0.0)
        np.testing.assert_allclose(gl, exp_lse, rtol=2e-6)
    del q, k, v, out, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kfill", ["large", "nonfinite"])
@pytest.mark.parametrize("ell,video", [(0, (18, 24, 32)), (1, (18, 24, 32)), (100, (18, 24, 32)),
                                       (226, (18, 24, 32)), (255, (18, 24, 32)), (77, (17, 21, 30))])
def test_text_padding_never_reaches_output(ell, video, kfill):
    """Padded text K/V (slots at or after text_length) change no bit of out or lse:
    K padded with a large finite value, or with NaN, +inf and -inf (every slot
    of the last, partly valid text block included); V with NaN and +inf."""
    windows = [(3, 3, 3), (1, 2, 3)]
    nv = video[0] * video[1] * video[2]
    S = nv + 256
    note(f"text padding isolation ell={ell} k={kfill}")
    g = torch.Generator(device="cuda").manual_seed(ell)
    q, k, v = [torch.randn(1, 2, S, 128, generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3)]
    out1, lse1 = run_sta(q, k, v, windows, ell, True, video)
    k2, v2 = k.clone(), v.clone()
    if kfill == "large":
        k2[:, :, nv + ell:] = 100.0
    else:
        k2[:, :, nv + ell:] = float("nan")
        k2[:, :, nv + ell::3] = float("inf")
        k2[:, :, nv + ell + 1::3] = float("-inf")
        k2[:, :, nv + ell:, 5] = float("nan")  # inf - inf inside a dot product as well
    v2[:, :, nv + ell:] = float("nan")
    v2[:, :, nv + ell::2] = float("inf")
    out2, lse2 = run_sta(q, k2, v2, windows, ell, True, video)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))


def test_deterministic_and_batch_independent():
    wl = sta_inputs.WORKLOADS["headline"]
    video = wl.video
    heads = 4
    nv = video[0] * video[1] * video[2]
    S = nv + 256
    note("determinism / batch independence at (30,48,80)+256, 4 heads")
    g = torch.Generator(device="cuda").manual_seed(9)
    q, k, v = [torch.randn(1, heads, S, 128, generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3)]
    windows = [(3, 3, 3), (5, 6, 10), (1, 6, 10), (5, 1, 1)]
    out1, lse1 = run_sta(q, k, v, windows, 226, True, video)
    out2, lse2 = run_sta(q, k, v, windows, 226, True, video)
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1.view(torch.int32), lse2.view(torch.int32))
    g2 = torch.Generator(device="cuda").manual_seed(10)
    y = [torch.randn(1, heads, S, 128, generator=g2, device="cuda").to(torch.bfloat16)
         for _ in range(3)]
    outy, lsey = run_sta(*y, windows, 226, True, video)
    qb, kb, vb = (torch.cat([a, b], 0).contiguous() for a, b in zip((q, k, v), y))
    outb, lseb = run_sta(qb, kb, vb, windows, 226, True, video)
    assert torch.equal(outb[0].view(torch.int16), out1[0].view(torch.int16))
    assert torch.equal(lseb[0].view(torch.int32), lse1[0].view(torch.int32))
    assert torch.equal(outb[1].view(torch.int16), outy[0].view(torch.int16))
    assert torch.equal(lseb[1].view(torch.int32), lsey[0].view(torch.int32))


@pytest.mark.parametrize("video", [(18, 24, 32), (17, 21, 30)])
def test_lse_is_optional(video):
    """sta_forward with lse = NULL writes the same out bits as with lse."""
    nv = video[0] * video[1] * video[2]
    S = nv + 256
    windows = [(3, 3, 3), (1, 2, 3)]
    note(f"lse = NULL {video}")
    g = torch.Generator(device="cuda").manual_seed(31)
    q, k, v = [torch.randn(1, 2, S, 128, generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3)]
    out1, _ = run_sta(q, k, v, windows, 99, True, video)
    dims = sta.make_dims(1, 2, 128, video)
    ws = torch.empty(sta.sta_workspace_bytes(dims, windows, True), dtype=torch.uint8, device="cuda")
    out2 = torch.full_like(q, float("nan"))
    sta.sta_forward(dims, q, k, v, windows, 99, True, out2, None, ws)
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))


def test_max_heads():
    """256 heads (the maximum) with per-head windows on a small partial grid:
    every head's window is read from the kernel arguments; heads are checked
    against the oracle on a sample, forward and backward."""
    import oracle
    from _parity import compare
    from test_gpu_backward import compare_grad, run_backward

    video, D, ell = (7, 16, 17), 64, 10  # tile grid (2, 2, 3)
    heads = 256
    cycle = [(1, 1, 1), (2, 2, 3), (1, 2, 2), (2, 1, 1), (1, 1, 3)]
    windows = [cycle[h % len(cycle)] for h in range(heads)]
    S = video[0] * video[1] * video[2] + 256
    note(f"max heads {heads} {video}")
    g = torch.Generator(device="cuda").manual_seed(256)
    q, k, v, dout = [torch.randn(1, heads, S, D, generator=g, device="cuda").to(torch.bfloat16)
                     for _ in range(4)]
    out, lse = run_sta(q, k, v, windows, ell, True, video)
    dq, dk, dv = run_backward(q, k, v, out, lse, dout, windows, ell, True, video)
    for t in (out, lse, dq, dk, dv):
        assert bool(torch.isfinite(t).all())
    for h in (0, 1, 2, 3, 4, 127, 255):
        sl = slice(h, h + 1)
        ro, rl = oracle.sta_reference(q[:, sl].cpu(), k[:, sl].cpu(), v[:, sl].cpu(), [windows[h]],
                                      ell, True, video)
        compare(out[:, sl], lse[:, sl], ro, rl, label=f"max heads, head {h}")
        rq, rk, rv = oracle.sta_reference_backward(q[:, sl].cpu(), k[:, sl].cpu(), v[:, sl].cpu(),
                                                   dout[:, sl].cpu(), [windows[h]], ell, True, video)
        compare_grad(dq[:, sl], rq, f"dq head {h}")
        compare_grad(dk[:, sl], rk, f"dk head {h}")
        compare_grad(dv[:, sl], rv, f"dv head {h}")
