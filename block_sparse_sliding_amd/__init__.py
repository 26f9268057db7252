"""Sliding Tile Attention (STA) forward and backward for AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libsta.so`` (declared in
``include/sta.h``). Every step of the computation runs in the library's HIP
kernels; this module only marshals arguments. PyTorch provides device memory
and the current stream.

The page's call ``sliding_tile_attention(q, k, v, window_size, text_length)``
(text mode) and ``sliding_tile_attention(q, k, v, window_size, 0, False)`` (no
text) is mirrored by :func:`sliding_tile_attention`, with the video size made
explicit; :func:`sliding_tile_attention_backward` gives its gradients.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsta.so")

STATUS = {
    0: "STA_OK", 1: "STA_ERR_NULL", 2: "STA_ERR_SHAPE", 3: "STA_ERR_WINDOW", 4: "STA_ERR_TEXT",
    5: "STA_ERR_ALIGN", 6: "STA_ERR_WORKSPACE", 7: "STA_ERR_HIP", 8: "STA_ERR_ALIAS",
    9: "STA_ERR_SCRATCH",
}
EXPORTS = (
    "sta_status_str", "sta_seq_len", "sta_tiled_seq_len", "sta_workspace_bytes", "sta_forward",
    "sta_forward_timed", "sta_forward_noalloc",
    "sta_hilbert_workspace_bytes", "sta_hilbert_forward", "sta_hilbert_gather", "sta_hilbert_scatter",
    "sta_tile_gather",
    "sta_tile_scatter", "sta_schedule_sizes", "sta_build_schedule",
    "sta_backward_workspace_bytes", "sta_backward", "sta_backward_timed",
)


class StaError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)} ({status_str(code)})")


class sta_dims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libsta.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m block_sparse_sliding_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I32 = ctypes.c_int32
    PD = ctypes.POINTER(sta_dims)
    PI32 = ctypes.POINTER(ctypes.c_int32)
    PI64 = ctypes.POINTER(ctypes.c_int64)
    lib.sta_status_str.argtypes = [ctypes.c_int]
    lib.sta_status_str.restype = ctypes.c_char_p
    lib.sta_seq_len.argtypes = [PD, I32]
    lib.sta_seq_len.restype = ctypes.c_int64
    lib.sta_tiled_seq_len.argtypes = [PD, I32]
    lib.sta_tiled_seq_len.restype = ctypes.c_int64
    lib.sta_workspace_bytes.argtypes = [PD, PI32, I32]
    lib.sta_workspace_bytes.restype = ctypes.c_size_t
    lib.sta_forward.argtypes = [PD, P, P, P, PI32, I32, I32, P, P, P, ctypes.c_size_t, P]
    lib.sta_forward.restype = ctypes.c_int
    lib.sta_forward_timed.argtypes = [PD, P, P, P, PI32, I32, I32, P, P, P, ctypes.c_size_t, P,
                                      ctypes.POINTER(ctypes.c_void_p)]
    lib.sta_forward_timed.restype = ctypes.c_int
    lib.sta_hilbert_workspace_bytes.argtypes = [PD, I32]
    lib.sta_hilbert_workspace_bytes.restype = ctypes.c_size_t
    lib.sta_hilbert_forward.argtypes = [PD, P, P, P, PI32, I32, I32, I32, P, P, P, ctypes.c_size_t, P]
    lib.sta_hilbert_forward.restype = ctypes.c_int
    lib.sta_hilbert_gather.argtypes = [PD, I32, P, P, P]
    lib.sta_hilbert_gather.restype = ctypes.c_int
    lib.sta_hilbert_scatter.argtypes = [PD, I32, P, P, P]
    lib.sta_hilbert_scatter.restype = ctypes.c_int
    lib.sta_forward_noalloc.argtypes = [PD, P, P, P, PI32, I32, I32, P, P, P]
    lib.sta_forward_noalloc.restype = ctypes.c_int
    lib.sta_tile_gather.argtypes = [PD, I32, P, P, P]
    lib.sta_tile_gather.restype = ctypes.c_int
    lib.sta_tile_scatter.argtypes = [PD, I32, P, P, P]
    lib.sta_tile_scatter.restype = ctypes.c_int
    lib.sta_schedule_sizes.argtypes = [PD, PI32, I32, PI64, PI64, PI64]
    lib.sta_schedule_sizes.restype = ctypes.c_int
    lib.sta_build_schedule.argtypes = [PD, PI32, I32, I32, PI32, PI32, PI32, P]
    lib.sta_build_schedule.restype = ctypes.c_int
    lib.sta_backward_workspace_bytes.argtypes = [PD, PI32, I32]
    lib.sta_backward_workspace_bytes.restype = ctypes.c_size_t
    bwd = [PD, P, P, P, P, P, P, PI32, I32, I32, P, P, P, P, ctypes.c_size_t, P]
    lib.sta_backward.argtypes = bwd
    lib.sta_backward.restype = ctypes.c_int
    lib.sta_backward_timed.argtypes = bwd + [ctypes.POINTER(ctypes.c_void_p)]
    lib.sta_backward_timed.restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(code: int) -> str:
    return load_library().sta_status_str(int(code)).decode()


def make_dims(batch: int, heads: int, head_dim: int, video: Sequence[int]) -> sta_dims:
    T, H, W = (int(x) for x in video)
    return sta_dims(int(batch), int(heads), int(head_dim), T, H, W)


def window_array(window_sizes, heads: int):
    """(heads*3) int32 ctypes array from one triple or one triple per head."""
    ws = list(window_sizes)
    if len(ws) == 3 and all(isinstance(x, int) for x in ws):
        ws = [tuple(ws)] * heads
    if len(ws) != heads:
        raise ValueError(f"need one window per head ({heads}), got {len(ws)}")
    flat = [int(c) for w in ws for c in w]
    if len(flat) != 3 * heads:
        raise ValueError("each window must be a (w_t, w_h, w_w) triple")
    return (ctypes.c_int32 * len(flat))(*flat)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _check(code: int, where: str):
    if code != 0:
        raise StaError(code, where)


# ----------------------------------------------------------------- C-ABI calls
def sta_seq_len(dims: sta_dims, has_text: bool) -> int:
    return int(load_library().sta_seq_len(ctypes.byref(dims), int(has_text)))


def sta_tiled_seq_len(dims: sta_dims, has_text: bool) -> int:
    return int(load_library().sta_tiled_seq_len(ctypes.byref(dims), int(has_text)))


def sta_workspace_bytes(dims: sta_dims, window_sizes, has_text: bool) -> int:
    wa = window_array(window_sizes, dims.heads)
    return int(load_library().sta_workspace_bytes(ctypes.byref(dims), wa, int(has_text)))


def sta_forward(dims: sta_dims, q, k, v, window_sizes, text_length: int, has_text: bool, out,
                lse, workspace, stream=None) -> None:
    """Enqueue STA forward (raster in, raster out) on the stream; see include/sta.h."""
    wa = window_array(window_sizes, dims.heads)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = load_library().sta_forward(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), wa, int(text_length), int(has_text),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream))
    _check(code, "sta_forward")


HILBERT_SLIDE = 1   # STA_HILBERT_SLIDE
HILBERT_WINDOW = 2  # STA_HILBERT_WINDOW


def sta_hilbert_workspace_bytes(dims: sta_dims, has_text: bool) -> int:
    return int(load_library().sta_hilbert_workspace_bytes(ctypes.byref(dims), int(has_text)))


def sta_hilbert_forward(dims: sta_dims, q, k, v, window_lens, mode: int, text_length: int,
                        has_text: bool, out, lse, workspace, stream=None) -> None:
    """Hilbert-window attention on a 2D image (raster in, raster out); see include/sta.h."""
    lens = list(window_lens) if hasattr(window_lens, "__len__") else [int(window_lens)] * dims.heads
    if len(lens) != dims.heads:
        raise ValueError("one window length per head")
    la = (ctypes.c_int32 * len(lens))(*[int(x) for x in lens])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = load_library().sta_hilbert_forward(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), la, int(mode), int(text_length), int(has_text),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream))
    _check(code, "sta_hilbert_forward")


def sta_hilbert_gather(dims: sta_dims, has_text: bool, x_raster, x_hilbert, stream=None) -> None:
    _check(load_library().sta_hilbert_gather(ctypes.byref(dims), int(has_text), _ptr(x_raster),
                                             _ptr(x_hilbert), _stream(stream)), "sta_hilbert_gather")


def sta_hilbert_scatter(dims: sta_dims, has_text: bool, x_hilbert, x_raster, stream=None) -> None:
    _check(load_library().sta_hilbert_scatter(ctypes.byref(dims), int(has_text), _ptr(x_hilbert),
                                              _ptr(x_raster), _stream(stream)), "sta_hilbert_scatter")


NOALLOC_SCRATCH_BYTES = 1 << 20  # STA_NOALLOC_SCRATCH_BYTES


def sta_forward_noalloc(dims: sta_dims, q, k, v, window_sizes, text_length: int, has_text: bool,
                        out, lse, stream=None) -> None:
    """sta_forward without a workspace argument: the library's fixed per-GPU
    scratch array takes its place (nothing is allocated); see include/sta.h."""
    wa = window_array(window_sizes, dims.heads)
    code = load_library().sta_forward_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), wa, int(text_length), int(has_text),
        _ptr(out), _ptr(lse), _stream(stream))
    _check(code, "sta_forward_noalloc")


TIMED_EVENTS = 3
STAGES = ("schedule_work", "attention")


def sta_forward_timed(dims: sta_dims, q, k, v, window_sizes, text_length: int, has_text: bool,
                      out, lse, workspace, events, stream=None) -> None:
    """sta_forward that records ``events`` (3 torch.cuda.Event, timing enabled)
    before the first launch and after each of the 2 launches on the stream."""
    if len(events) != TIMED_EVENTS:
        raise ValueError(f"need {TIMED_EVENTS} events")
    handles = (ctypes.c_void_p * TIMED_EVENTS)(*[e.cuda_event for e in events])
    wa = window_array(window_sizes, dims.heads)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = load_library().sta_forward_timed(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), wa, int(text_length), int(has_text),
        _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream), handles)
    _check(code, "sta_forward_timed")


def sta_tile_gather(dims: sta_dims, has_text: bool, x_raster, x_tiled, stream=None) -> None:
    _check(load_library().sta_tile_gather(ctypes.byref(dims), int(has_text), _ptr(x_raster),
                                          _ptr(x_tiled), _stream(stream)), "sta_tile_gather")


def sta_tile_scatter(dims: sta_dims, has_text: bool, x_tiled, x_raster, stream=None) -> None:
    _check(load_library().sta_tile_scatter(ctypes.byref(dims), int(has_text), _ptr(x_tiled),
                                           _ptr(x_raster), _stream(stream)), "sta_tile_scatter")


def sta_schedule_sizes(dims: sta_dims, window_sizes, has_text: bool) -> Tuple[int, int, int]:
    wa = window_array(window_sizes, dims.heads)
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().sta_schedule_sizes(ctypes.byref(dims), wa, int(has_text), ctypes.byref(a),
                                             ctypes.byref(b), ctypes.byref(c)), "sta_schedule_sizes")
    return a.value, b.value, c.value


def sta_build_schedule(dims: sta_dims, window_sizes, text_length: int, has_text: bool, offsets,
                       ids, work, stream=None) -> None:
    wa = window_array(window_sizes, dims.heads)
    i32p = ctypes.POINTER(ctypes.c_int32)
    _check(load_library().sta_build_schedule(
        ctypes.byref(dims), wa, int(text_length), int(has_text),
        ctypes.cast(_ptr(offsets), i32p), ctypes.cast(_ptr(ids), i32p),
        ctypes.cast(_ptr(work), i32p), _stream(stream)), "sta_build_schedule")


# ------------------------------------------------------------ convenience API
def sliding_tile_attention(q, k, v, window_size, text_length: int = 0, has_text: bool = True,
                           video: Sequence[int] = (30, 48, 80), return_lse: bool = False,
                           workspace=None):
    """The page's call, on device tensors: returns ``out`` (and ``lse`` if asked).

    q, k, v: bf16 CUDA/HIP tensors ``[B, heads, S, D]`` with S = T*H*W (+256
    with text). window_size: one (w_t, w_h, w_w) triple or one per head.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not (t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous bf16 tensor on the GPU")
    if q.shape != k.shape or q.shape != v.shape or q.dim() != 4:
        raise ValueError("q, k, v must share one [B, heads, S, D] shape")
    B, heads, S, D = q.shape
    dims = make_dims(B, heads, D, video)
    expect = sta_seq_len(dims, has_text)
    if S != expect:
        raise ValueError(f"sequence length {S} != {expect} for video {tuple(video)} "
                         f"(has_text={has_text})")
    out = torch.empty_like(q)
    lse = torch.empty((B, heads, S), dtype=torch.float32, device=q.device)
    need = sta_workspace_bytes(dims, window_size, has_text)
    if need == 0:
        raise ValueError("invalid arguments (window sizes or shapes)")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    sta_forward(dims, q, k, v, window_size, text_length, has_text, out, lse, workspace)
    return (out, lse) if return_lse else out


# ----------------------------------------------------------------- backward
BWD_TIMED_EVENTS = 5
BWD_STAGES = ("row_stats", "schedule_lists", "dq", "dkv")


def sta_backward_workspace_bytes(dims: sta_dims, window_sizes, has_text: bool) -> int:
    wa = window_array(window_sizes, dims.heads)
    return int(load_library().sta_backward_workspace_bytes(ctypes.byref(dims), wa, int(has_text)))


def _backward_args(dims, q, k, v, out, lse, dout, window_sizes, text_length, has_text, dq, dk,
                   dv, workspace, stream):
    wa = window_array(window_sizes, dims.heads)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), wa,
            int(text_length), int(has_text), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
            ws_bytes, _stream(stream))


def sta_backward(dims: sta_dims, q, k, v, out, lse, dout, window_sizes, text_length: int,
                 has_text: bool, dq, dk, dv, workspace, stream=None) -> None:
    """Enqueue the STA backward on the stream; see include/sta.h."""
    _check(load_library().sta_backward(*_backward_args(
        dims, q, k, v, out, lse, dout, window_sizes, text_length, has_text, dq, dk, dv, workspace,
        stream)), "sta_backward")


def sta_backward_timed(dims: sta_dims, q, k, v, out, lse, dout, window_sizes, text_length: int,
                       has_text: bool, dq, dk, dv, workspace, events, stream=None) -> None:
    """sta_backward recording ``events`` (6 torch.cuda.Event) around its launches."""
    if len(events) != BWD_TIMED_EVENTS:
        raise ValueError(f"need {BWD_TIMED_EVENTS} events")
    handles = (ctypes.c_void_p * BWD_TIMED_EVENTS)(*[e.cuda_event for e in events])
    _check(load_library().sta_backward_timed(*_backward_args(
        dims, q, k, v, out, lse, dout, window_sizes, text_length, has_text, dq, dk, dv, workspace,
        stream), handles), "sta_backward_timed")


def sliding_tile_attention_backward(q, k, v, out, lse, dout, window_size, text_length: int = 0,
                                    has_text: bool = True, video: Sequence[int] = (30, 48, 80),
                                    workspace=None):
    """Gradients (dq, dk, dv) of :func:`sliding_tile_attention` for ``dout``.

    ``out`` and ``lse`` are the forward's results for the same q, k, v
    (``sliding_tile_attention(..., return_lse=True)``).
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        if not (t.is_cuda and t.dtype == torch.bfloat16 and t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous bf16 tensor on the GPU")
        if t.shape != q.shape or t.dim() != 4:
            raise ValueError(f"{name} must have q's [B, heads, S, D] shape")
    B, heads, S, D = q.shape
    if not (lse.is_cuda and lse.dtype == torch.float32 and lse.is_contiguous()
            and tuple(lse.shape) == (B, heads, S)):
        raise ValueError("lse must be a contiguous fp32 [B, heads, S] tensor on the GPU")
    dims = make_dims(B, heads, D, video)
    need = sta_backward_workspace_bytes(dims, window_size, has_text)
    if need == 0:
        raise ValueError("invalid arguments (window sizes or shapes)")
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    sta_backward(dims, q, k, v, out, lse, dout, window_size, text_length, has_text, dq, dk, dv,
                 workspace)
    return dq, dk, dv


# ----------------------------------------------------------------- autograd
def _autograd_function():
    import torch

    class _STAFunction(torch.autograd.Function):
        """Autograd glue: forward = sta_forward, backward = sta_backward (no arithmetic here)."""

        @staticmethod
        def forward(ctx, q, k, v, window_size, text_length, has_text, video):
            out, lse = sliding_tile_attention(q, k, v, window_size, text_length, has_text, video,
                                              return_lse=True)
            ctx.save_for_backward(q, k, v, out, lse)
            ctx.args = (window_size, text_length, has_text, video)
            return out

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse = ctx.saved_tensors
            window_size, text_length, has_text, video = ctx.args
            dq, dk, dv = sliding_tile_attention_backward(q, k, v, out, lse, dout.contiguous(),
                                                         window_size, text_length, has_text, video)
            return dq, dk, dv, None, None, None, None

    return _STAFunction


_STA_FUNCTION = None


def sliding_tile_attention_autograd(q, k, v, window_size, text_length: int = 0,
                                    has_text: bool = True, video: Sequence[int] = (30, 48, 80)):
    """:func:`sliding_tile_attention` as a differentiable op: out.backward(...) runs
    sta_backward (dq, dk, dv in bf16, like the inputs)."""
    global _STA_FUNCTION
    if _STA_FUNCTION is None:
        _STA_FUNCTION = _autograd_function()
    return _STA_FUNCTION.apply(q, k, v, window_size, text_length, has_text, tuple(video))
