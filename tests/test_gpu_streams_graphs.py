"""GPU checks of how the library behaves on streams and in graphs (through the C ABI).

* Captured in a HIP graph (torch.cuda.CUDAGraph), sta_forward followed by
  sta_backward replays to the same bits as the eager calls, replay after
  replay, with other eager work and synchronisations in between, on a video,
  on partial tiles and on 2D images whose text rows are split and merged.
  Every launch is a kernel (the queue heads are zeroed by a kernel, not a
  memset), so the calls are capturable.
* Two sta_forward calls running at once on two streams, each with its own
  workspace, give the same bits as the same calls run one after the other:
  the per-XCD queues and their heads live in each call's workspace.
"""

import pytest
import torch

import block_sparse_sliding_amd as sta
from _parity import note

pytestmark = pytest.mark.gpu

VIDEO = (18, 24, 32)
WINDOWS = [(3, 3, 3), (1, 2, 3)]
ELL = 141


def seq(video):
    return video[0] * video[1] * video[2] + 256


S = seq(VIDEO)


def tensors(seed, D=128, heads=2, video=VIDEO):
    g = torch.Generator(device="cuda").manual_seed(seed)
    return [torch.randn(1, heads, seq(video), D, generator=g, device="cuda").to(torch.bfloat16)
            for _ in range(4)]


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


# a video, partial tiles, and 2D images of 272 and 289 tiles: square query
# units whose text rows are split in two parts and merged by a third launch
# (whole 8x8 tiles, and a partial last tile row and column)
GRAPH_CASES = [(VIDEO, WINDOWS), ((17, 21, 30), WINDOWS),
               ((1, 128, 136), [(1, 3, 3), (1, 2, 5)]), ((1, 130, 133), [(1, 3, 3), (1, 2, 5)])]


@pytest.mark.parametrize("video,windows", GRAPH_CASES, ids=["video", "partial", "image", "image-partial"])
def test_graph_replays_match_eager(video, windows):
    note(f"graph capture of forward + backward {video} {windows}")
    q, k, v, dout = tensors(11, video=video)
    dims = sta.make_dims(1, 2, 128, video)
    fws = torch.empty(sta.sta_workspace_bytes(dims, windows, True), dtype=torch.uint8, device="cuda")
    bws = torch.empty(sta.sta_backward_workspace_bytes(dims, windows, True), dtype=torch.uint8,
                      device="cuda")
    out, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty(1, 2, seq(video), dtype=torch.float32, device="cuda")

    def step():
        sta.sta_forward(dims, q, k, v, windows, ELL, True, out, lse, fws)
        sta.sta_backward(dims, q, k, v, out, lse, dout, windows, ELL, True, dq, dk, dv, bws)

    # eager reference (and warm-up on a side stream, as graph capture expects)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = [x.clone() for x in (out, lse, dq, dk, dv)]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for x in (out, lse, dq, dk, dv):
            x.fill_(float("nan"))     # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(("out", "lse", "dq", "dk", "dv"), (out, lse, dq, dk, dv), ref):
            assert torch.equal(bits(x), bits(r)), (rep, name)


def test_two_streams_at_once_match_sequential():
    note("two concurrent forward calls")
    dims = sta.make_dims(1, 2, 128, VIDEO)
    a = tensors(21)[:3]
    b = tensors(22)[:3]
    outs = {}
    for mode in ("sequential", "concurrent"):
        res = []
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        for inputs, st in zip((a, b), streams):
            ws = torch.empty(sta.sta_workspace_bytes(dims, WINDOWS, True), dtype=torch.uint8,
                             device="cuda")
            out = torch.empty_like(inputs[0])
            lse = torch.empty(1, 2, S, dtype=torch.float32, device="cuda")
            res.append((inputs, st, ws, out, lse))
        torch.cuda.synchronize()
        for inputs, st, ws, out, lse in res:
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                sta.sta_forward(dims, *inputs, WINDOWS, ELL, True, out, lse, ws,
                                stream=st.cuda_stream)
            if mode == "sequential":
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        outs[mode] = [(out.clone(), lse.clone()) for _, _, _, out, lse in res]
    for (o1, l1), (o2, l2) in zip(outs["sequential"], outs["concurrent"]):
        assert torch.equal(bits(o1), bits(o2)) and torch.equal(bits(l1), bits(l2))
