"""sta_forward_noalloc (the forward that allocates nothing) against sta_forward.

Both run the same kernels; the no-workspace entry point puts the work order,
queue heads and zero row in the library's fixed per-GPU scratch array instead
of a caller workspace. Two calls in a row, the second on a smaller input (the
array then still holds the first call's contents), must each reproduce
sta_forward's out and lse bit for bit, with NaN in the padded text slots of k
and v as in the other parity tests. A shape whose workspace exceeds the array
is refused with STA_ERR_SCRATCH, before any launch.
"""

import pytest
import torch

import block_sparse_sliding_amd as sta
from _parity import note

pytestmark = pytest.mark.gpu

CASES = [
    # batch, heads, D, video, has_text, text_length, windows (one per head, cycled)
    (1, 4, 128, (18, 24, 32), True, 226, [(3, 3, 3), (1, 2, 3)]),
    (2, 2, 64, (13, 17, 20), True, 50, [(2, 2, 2)]),  # smaller; partial tiles, ragged text
]


def inputs(seed, batch, heads, D, video, has_text, ell):
    S = video[0] * video[1] * video[2] + (256 if has_text else 0)
    g = torch.Generator(device="cuda").manual_seed(seed)
    q, k, v = (torch.randn(batch, heads, S, D, generator=g, device="cuda").to(torch.bfloat16)
               for _ in range(3))
    if has_text and ell < 256:  # padded text slots: never read into a result
        first = video[0] * video[1] * video[2] + ell
        k[:, :, first:] = float("nan")
        v[:, :, first:] = float("nan")
    return q, k, v


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_noalloc_matches_forward_on_two_calls():
    results = []
    for i, (batch, heads, D, video, has_text, ell, wins) in enumerate(CASES):
        note(f"noalloc call {i}: B={batch} heads={heads} D={D} video={video} text={ell if has_text else '-'}")
        windows = [wins[h % len(wins)] for h in range(heads)]
        dims = sta.make_dims(batch, heads, D, video)
        q, k, v = inputs(100 + i, batch, heads, D, video, has_text, ell)
        S = q.shape[2]
        ws = torch.empty(sta.sta_workspace_bytes(dims, windows, has_text), dtype=torch.uint8, device="cuda")
        out_ref = torch.empty_like(q)
        lse_ref = torch.empty(batch, heads, S, dtype=torch.float32, device="cuda")
        sta.sta_forward(dims, q, k, v, windows, ell, has_text, out_ref, lse_ref, ws)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((batch, heads, S), float("nan"), dtype=torch.float32, device="cuda")
        sta.sta_forward_noalloc(dims, q, k, v, windows, ell, has_text, out, lse)
        torch.cuda.synchronize()
        assert torch.isfinite(out_ref.float()).all() and torch.isfinite(lse_ref).all()
        assert torch.equal(bits(out), bits(out_ref)), f"call {i}: out differs"
        assert torch.equal(bits(lse), bits(lse_ref)), f"call {i}: lse differs"
        results.append(out.shape)
    assert results[1].numel() < results[0].numel()  # the second call was the smaller one


def test_noalloc_refuses_a_shape_beyond_its_scratch():
    dims = sta.make_dims(16, 256, 64, (60, 64, 64))
    windows = [(1, 1, 1)] * 256
    assert sta.sta_workspace_bytes(dims, windows, False) > sta.NOALLOC_SCRATCH_BYTES
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")  # never read: refused before any launch
    with pytest.raises(RuntimeError, match="STA_ERR_SCRATCH"):
        sta.sta_forward_noalloc(dims, t, t, t, windows, 0, False, t, None)
