"""GPU tests of the Hilbert row (through the C ABI): the Hilbert gather/scatter
bit for bit against the oracle's curve, and Hilbert slide/window attention
against the Hilbert oracle at the stated tolerances.

Source: "Boosting 2D Local Attention Efficiency with Hilbert-Guided Sparsity"
(TLDR, "The Hilbert Curve Advantage"); readings in the Hilbert oracle's header.
"""

import numpy as np
import pytest
import torch

import block_sparse_sliding_amd as sta
from _parity import _check, note
from oracle import hilbert_oracle as HO

pytestmark = pytest.mark.gpu

MODES = {"slide": sta.HILBERT_SLIDE, "window": sta.HILBERT_WINDOW}


def inputs(seed, B, heads, side, D, has_text, ell, scale_k=1.0):
    S = side * side + (256 if has_text else 0)
    g = torch.Generator(device="cuda").manual_seed(seed)
    q, k, v = (torch.randn(B, heads, S, D, generator=g, device="cuda") for _ in range(3))
    k = k * scale_k
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    return q, k, v


def run_hilbert(q, k, v, lens, mode, ell, has_text, side):
    """The GPU call, on copies of k and v whose padded text slots hold NaN (they
    must never reach a result); the oracle gets the clean tensors."""
    B, heads, S, D = q.shape
    if has_text and ell < 256:
        k, v = k.clone(), v.clone()
        k[:, :, side * side + ell:] = float("nan")
        v[:, :, side * side + ell:] = float("nan")
    dims = sta.make_dims(B, heads, D, (1, side, side))
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, heads, S), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(sta.sta_hilbert_workspace_bytes(dims, has_text), dtype=torch.uint8, device="cuda")
    sta.sta_hilbert_forward(dims, q, k, v, lens, MODES[mode], ell, has_text, out, lse, ws)
    torch.cuda.synchronize()
    return out, lse


def oracle_rows(q, k, v, lens, mode, ell, has_text, side, rows):
    B, heads = q.shape[:2]
    outs, lses = [], []
    for h in range(heads):
        o, l = HO.hilbert_reference(q[:, h:h + 1].cpu(), k[:, h:h + 1].cpu(), v[:, h:h + 1].cpu(), [lens[h]],
                                    mode, ell, has_text, (side, side), rows=rows)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs, axis=1), np.concatenate(lses, axis=1)


@pytest.mark.parametrize("side,has_text,D", [(8, True, 64), (32, False, 128), (128, True, 128), (64, True, 64)])
def test_hilbert_gather_scatter_bit_exact(side, has_text, D):
    note(f"hilbert gather/scatter side={side} text={has_text} D={D}")
    B, heads = 2, 3
    S = side * side + (256 if has_text else 0)
    g = torch.Generator(device="cuda").manual_seed(side + D)
    x = torch.randn(B, heads, S, D, generator=g, device="cuda").to(torch.bfloat16)
    dims = sta.make_dims(B, heads, D, (1, side, side))
    xh = torch.full_like(x, float("nan"))
    sta.sta_hilbert_gather(dims, has_text, x, xh)
    back = torch.full_like(x, float("nan"))
    sta.sta_hilbert_scatter(dims, has_text, xh, back)
    torch.cuda.synchronize()
    perm = torch.as_tensor(HO.hilbert_token_order((side, side)), device="cuda")
    if has_text:
        perm = torch.cat([perm, torch.arange(side * side, S, device="cuda")])
    expect = x[:, :, perm]
    assert torch.equal(xh.view(torch.int16), expect.view(torch.int16))
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))


SMALL = [
    # side, heads, D, has_text, ell, mode, window length per head
    (8, 1, 64, True, 226, "slide", [1]),
    (16, 2, 128, False, 0, "slide", [1, 3]),
    (32, 2, 64, True, 100, "slide", [5, 16]),
    (32, 2, 128, True, 256, "window", [4, 3]),
    (64, 2, 128, True, 64, "window", [16, 1]),
    (64, 2, 64, False, 0, "slide", [9, 64]),
    (32, 1, 128, True, 226, "slide", [6]),
    (64, 2, 128, True, 17, "slide", [27, 7]),
    (128, 1, 128, True, 226, "slide", [27]),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"{c[0]}-{c[5]}{c[6]}-D{c[2]}-t{c[4] if c[3] else '-'}" for c in SMALL])
def test_hilbert_forward_all_rows(case):
    side, heads, D, has_text, ell, mode, lens = case
    note(f"hilbert forward side={side} heads={heads} D={D} text={ell if has_text else '-'} {mode} {lens}")
    q, k, v = inputs(7 + side, 1, heads, side, D, has_text, ell)
    out, lse = run_hilbert(q, k, v, lens, mode, ell, has_text, side)
    S = q.shape[2]
    rows = np.arange(S)
    ref_o, ref_l = oracle_rows(q, k, v, lens, mode, ell, has_text, side, rows)
    _check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l,
           f"hilbert {case}")


@pytest.mark.parametrize("lens", [[5, 7], [6, 11]], ids=["four-tile-units", "six-tile-units"])
def test_hilbert_forward_score_jumps_redo(lens):
    """Key tiles scaled by large, uneven factors: scores jump by tens of log2
    units between blocks, which triggers the redo pass of the fixed reference."""
    side, heads, D = 32, 2, 128
    note(f"hilbert forward, score jumps, {lens}")
    q, k, v = inputs(41, 1, heads, side, D, True, 150)
    y, x = np.divmod(np.arange(side * side), side)
    factor = torch.ones(side * side + 256, device="cuda")
    factor[torch.as_tensor(((y // 8) * 4 + (x // 8)) % 5 == 3, device="cuda").nonzero()[:, 0]] = 6.0
    factor[side * side:side * side + 150] = 4.0
    k = (k.float() * factor[None, None, :, None]).to(torch.bfloat16)
    out, lse = run_hilbert(q, k, v, lens, "slide", 150, True, side)
    rows = np.arange(q.shape[2])
    ref_o, ref_l = oracle_rows(q, k, v, lens, "slide", 150, True, side, rows)
    _check(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref_o, ref_l,
           "hilbert score jumps")


@pytest.mark.parametrize("slide_lens", [[1, 9, 27, 64], [6, 9, 27, 64]], ids=["single-tile-units", "six-tile-units"])
def test_hilbert_forward_full_size_sampled(slide_lens):
    """A 256x256 image (1024 tiles), 8 heads of different slide and window
    lengths, D = 128, ragged text; per head every text row (their keys are
    split over 8 units and merged), every corner and a seeded uniform draw of
    377 rows. The slide heads run with single-tile query units when one of them
    has a window of 1 tile, else with six-tile units."""
    side, heads, D, ell = 256, 8, 128, 226
    lens = slide_lens + [4, 16, 64, 256]
    modes = ["slide"] * 4 + ["window"] * 4
    note(f"hilbert full size 256x256, 8 heads, slide {slide_lens}")
    q, k, v = inputs(99, 1, heads, side, D, True, ell)
    S = q.shape[2]
    rng = np.random.default_rng(5)
    fixed = [0, side - 1, side * (side - 1), side * side - 1, side * side, side * side + ell - 1, S - 1]
    for mode in ("slide", "window"):
        hs = [h for h in range(heads) if modes[h] == mode]
        qm, km, vm = q[:, hs].contiguous(), k[:, hs].contiguous(), v[:, hs].contiguous()
        lm = [lens[h] for h in hs]
        out, lse = run_hilbert(qm, km, vm, lm, mode, ell, True, side)
        rows = np.unique(np.concatenate([fixed, rng.integers(0, S, 377), np.arange(side * side, S)]))
        ref_o, ref_l = oracle_rows(qm, km, vm, lm, mode, ell, True, side, rows)
        idx = torch.as_tensor(rows, device="cuda")
        _check(out[:, :, idx].float().cpu().numpy().astype(np.float64),
               lse[:, :, idx].cpu().numpy().astype(np.float64), ref_o, ref_l, f"hilbert 256^2 {mode}")
