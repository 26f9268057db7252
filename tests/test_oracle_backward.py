"""Pins for the oracle's STA gradients (CPU only).

Each pin is independent of the oracle's code path:

* torch autograd (fp64) through a dense masked softmax whose mask is built
  here from the window's characterisation (nearest fitting placement), not
  from the oracle's mask;
* central finite differences of the scalar loss sum(out * dout), with the
  oracle's own forward as the function being differentiated;
* sum rules: every query row's probabilities sum to one, so
  sum_j dv_j = sum_i dout_i, and every row's score gradients sum to zero, so
  sum_j dk_j = 0;
* restricted row sets agree with the full computation;
* planted mistakes in the oracle are caught by the autograd pin.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import sta_oracle as so

TILE = (6, 8, 8)


def nearest_box_start(c, w, n):
    """Nearest fitting placement of w tiles around tile c (ties: lower start)."""
    best = None
    for s in range(0, n - w + 1):
        d = abs(s + (w - 1) / 2.0 - c)
        if best is None or d < best[0]:
            best = (d, s)
    return best[1]


def independent_mask(video, window, ell, has_text):
    """Token mask [S, S] from coordinates and the placement characterisation."""
    T, H, W = video
    nv = T * H * W
    S = nv + (256 if has_text else 0)
    n = [-(-video[a] // TILE[a]) for a in range(3)]  # partial last tiles included
    idx = np.arange(nv)
    tc = np.stack([(idx // (H * W)) // 6, ((idx // W) % H) // 8, (idx % W) // 8], 1)
    m = np.zeros((S, S), dtype=bool)
    lo = np.stack([np.array([nearest_box_start(c, window[a], n[a]) for c in range(n[a])])[tc[:, a]]
                   for a in range(3)], 1)
    inside = np.ones((nv, nv), dtype=bool)
    for a in range(3):
        inside &= (tc[None, :, a] >= lo[:, None, a]) & (tc[None, :, a] < lo[:, None, a] + window[a])
    m[:nv, :nv] = inside
    if has_text:
        m[nv:, :nv] = True
        m[:, nv:nv + ell] = True
    return m


def rand(shape, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64).to(dtype)


def autograd_grads(q, k, v, dout, video, windows, ell, has_text):
    """dq, dk, dv by torch autograd through a dense masked softmax (fp64)."""
    B, heads, S, D = q.shape
    qq, kk, vv = (x.detach().double().clone().requires_grad_(True) for x in (q, k, v))
    outs = []
    for h in range(heads):
        m = torch.from_numpy(independent_mask(video, windows[h], ell, has_text))
        sc = (qq[:, h] @ kk[:, h].transpose(-1, -2)) / D ** 0.5
        sc = sc.masked_fill(~m, float("-inf"))
        outs.append(torch.softmax(sc, dim=-1) @ vv[:, h])
    out = torch.stack(outs, 1)
    (out * dout.double()).sum().backward()
    return qq.grad.numpy(), kk.grad.numpy(), vv.grad.numpy()


CASES = [
    # video, windows per head, ell, has_text, D, B
    ((12, 16, 16), [(1, 2, 1), (2, 1, 2)], 0, False, 16, 1),
    ((12, 16, 24), [(1, 1, 3), (2, 2, 1)], 100, True, 8, 2),
    ((18, 8, 16), [(3, 1, 1)], 256, True, 8, 1),
    ((6, 16, 24), [(1, 1, 1)], 1, True, 4, 1),
    ((7, 9, 11), [(1, 2, 1), (2, 1, 2)], 30, True, 4, 1),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_backward_matches_autograd(case):
    video, windows, ell, has_text, D, B = case
    S = video[0] * video[1] * video[2] + (256 if has_text else 0)
    heads = len(windows)
    q, k, v, do = (rand((B, heads, S, D), 100 + i) for i in range(4))
    dq, dk, dv = oracle.sta_reference_backward(q, k, v, do, windows, ell, has_text, video)
    gq, gk, gv = autograd_grads(q, k, v, do, video, windows, ell, has_text)
    for name, a, b in (("dq", dq, gq), ("dk", dk, gk), ("dv", dv, gv)):
        np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11, err_msg=name)
    if has_text:
        nv = S - 256
        # padded text keys are seen by no query: no gradient reaches them
        assert np.all(dk[:, :, nv + ell:] == 0) and np.all(dv[:, :, nv + ell:] == 0)


def test_backward_finite_differences():
    """Central differences of L = sum(out * dout) through the oracle's forward."""
    video, windows, ell, has_text, D = (12, 8, 16), [(1, 1, 2)], 30, True, 4
    S = video[0] * video[1] * video[2] + 256
    q, k, v, do = (rand((1, 1, S, D), 7 + i) for i in range(4))
    dq, dk, dv = oracle.sta_reference_backward(q, k, v, do, windows, ell, has_text, video)
    grads = {"q": dq, "k": dk, "v": dv}
    base = {"q": q.numpy().copy(), "k": k.numpy().copy(), "v": v.numpy().copy()}
    do64 = do.numpy()
    rng = np.random.default_rng(3)
    eps = 1e-5
    rows = {"q": rng.integers(0, S, 6).tolist() + [S - 1, S - 256],
            "k": rng.integers(0, S - 256, 5).tolist() + [S - 256, S - 256 + ell - 1],
            "v": rng.integers(0, S - 256, 5).tolist() + [S - 256 + 3]}
    for name in ("q", "k", "v"):
        for r in rows[name]:
            d = int(rng.integers(0, D))
            vals = []
            for sgn in (1, -1):
                x = {n: a.copy() for n, a in base.items()}
                x[name][0, 0, r, d] += sgn * eps
                out, _ = oracle.sta_reference(x["q"], x["k"], x["v"], windows, ell, has_text, video)
                vals.append(float((out * do64).sum()))
            fd = (vals[0] - vals[1]) / (2 * eps)
            assert abs(fd - grads[name][0, 0, r, d]) <= 1e-6 * max(1.0, abs(fd)), (name, r, d, fd)


def test_backward_sum_rules():
    video, windows, ell, has_text, D = (12, 16, 16), [(2, 1, 1), (1, 2, 2)], 77, True, 8
    S = video[0] * video[1] * video[2] + 256
    q, k, v, do = (rand((2, 2, S, D), 40 + i) for i in range(4))
    dq, dk, dv = oracle.sta_reference_backward(q, k, v, do, windows, ell, has_text, video)
    np.testing.assert_allclose(dv.sum(axis=2), do.numpy().sum(axis=2), rtol=1e-10, atol=1e-9)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-9)


def test_restricted_rows_match_full():
    video, windows, ell, has_text, D = (12, 16, 24), [(1, 2, 1)], 50, True, 8
    S = video[0] * video[1] * video[2] + 256
    q, k, v, do = (rand((1, 1, S, D), 60 + i) for i in range(4))
    full = oracle.sta_reference_backward(q, k, v, do, windows, ell, has_text, video)
    qrows = [0, 17, 900, S - 256, S - 1]
    krows = [5, 1200, 3000, S - 256, S - 256 + ell, S - 1]
    part = oracle.sta_reference_backward(q, k, v, do, windows, ell, has_text, video,
                                         query_rows=qrows, key_rows=krows)
    np.testing.assert_allclose(part[0], full[0][:, :, qrows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(part[1], full[1][:, :, krows], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(part[2], full[2][:, :, krows], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("video,window,ell,has_text", [
    ((12, 16, 24), (1, 2, 1), 50, True),
    ((18, 16, 16), (3, 1, 2), 0, True),
    ((12, 24, 16), (2, 3, 1), 0, False),
])
def test_query_rows_seeing_matches_mask(video, window, ell, has_text):
    S = video[0] * video[1] * video[2] + (256 if has_text else 0)
    m = independent_mask(video, window, ell, has_text)
    rng = np.random.default_rng(S)
    for keys in ([0], [S - 1], rng.integers(0, S, 3).tolist(), [S - 256] if has_text else [1]):
        want = np.nonzero(m[:, keys].any(axis=1))[0]
        got = oracle.query_rows_seeing(keys, video, window, ell, has_text)
        assert np.array_equal(got, want), keys


def _autograd_pin_holds():
    try:
        test_backward_matches_autograd(CASES[1])
        return True
    except AssertionError:
        return False


@pytest.mark.parametrize("mutant", ["scale_1_over_d", "unnormalised", "off_by_one_window"])
def test_planted_backward_mistakes_are_caught(monkeypatch, mutant):
    if mutant == "scale_1_over_d":
        monkeypatch.setattr(so, "softmax_scale", lambda d: 1.0 / d)
    elif mutant == "unnormalised":
        def unnorm(q64, k64, rr, mask, scale):
            sc = np.where(mask, (q64[rr] @ k64.T) * scale, -np.inf)
            return np.exp(sc - sc.max(axis=1, keepdims=True))
        monkeypatch.setattr(so, "_masked_probabilities", unnorm)
    elif mutant == "off_by_one_window":
        monkeypatch.setattr(so, "window_start", lambda c, w, n: min(max(c - w // 2 - 1, 0), n - w))
    assert not _autograd_pin_holds(), f"mutant {mutant} slipped through"
