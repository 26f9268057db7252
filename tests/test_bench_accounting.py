"""The benchmark's effective-FLOP count, checked against the oracle's mask.

bench.py counts 4*D flop per allowed (query, key) pair with a closed form
that factors the video part over the three axes. Here the count is compared
with the number of True entries of the oracle's explicit token mask (summed
over the valid query rows), on shapes with and without partial tiles.
"""

import numpy as np
import pytest

import bench
import oracle
import sta_inputs


@pytest.mark.parametrize("video,windows,ell,has_text", [
    ((12, 16, 16), [(2, 2, 2)], 0, False),
    ((18, 24, 32), [(3, 3, 3), (1, 2, 4)], 100, True),
    ((7, 9, 11), [(2, 2, 2), (1, 1, 2)], 77, True),
    ((13, 8, 20), [(3, 1, 3)], 0, True),
    ((11, 17, 9), [(2, 3, 2), (1, 1, 1)], 256, True),
])
def test_effective_flops_counts_the_oracle_mask(video, windows, ell, has_text):
    D = 64
    wl = sta_inputs.custom("t", 1, len(windows), D, video, windows, has_text, ell)
    nv = video[0] * video[1] * video[2]
    valid_rows = np.arange(nv + (ell if has_text else 0))
    pairs = sum(int(oracle.allowed_mask(valid_rows, video, w, ell, has_text).sum())
                for w in windows)
    assert bench.effective_flops(wl) == 4.0 * D * pairs


def test_headline_count_is_the_tile_product():
    """For tile multiples the count is the familiar per-query window size."""
    wl = sta_inputs.WORKLOADS["headline"]
    nv = 30 * 48 * 80
    ell = wl.text_length
    pairs = 24 * (nv * (27 * 384 + ell) + ell * (nv + ell))
    assert bench.effective_flops(wl) == 4.0 * 128 * pairs
    assert bench.kernel_suffix(wl) == "<128, false>"
    assert bench.kernel_suffix(sta_inputs.WORKLOADS["ragged"]) == "<128, true>"
    assert bench.attention_kernel(wl) == "sta_attention_kernel<128, false, 0>"
    assert bench.attention_kernel(sta_inputs.WORKLOADS["ragged"]) == "sta_attention_kernel<128, true, 0>"
    assert bench.attention_kernel(sta_inputs.WORKLOADS["hilbert"]) == "sta_attention_kernel<128, true, 1>"
    assert bench.attention_kernel(sta_inputs.WORKLOADS["image"]) == "sta_attention_kernel<128, true, 2>"


@pytest.mark.parametrize("mode,W", [(1, 5), (1, 16), (2, 3), (2, 4)])
def test_hilbert_flop_count_matches_the_oracle_mask(mode, W):
    """bench.hilbert_flops counts 4*D per pair the Hilbert oracle's mask allows
    (video rows and the valid text rows)."""
    from oracle import hilbert_oracle as HO
    side, ell = 32, 77
    wl = sta_inputs.Workload("h", 1, 2, 64, (1, side, side), ((1, 1, W),) * 2, True, ell, 0,
                             hilbert_len=W, hilbert_mode=mode)
    nv = side * side
    rows = list(range(nv)) + list(range(nv, nv + ell))
    mask = HO.hilbert_allowed_mask(rows, (side, side), W, "slide" if mode == 1 else "window", ell, True)
    assert bench.hilbert_flops(wl) == 4.0 * 64 * int(mask.sum()) * 2
