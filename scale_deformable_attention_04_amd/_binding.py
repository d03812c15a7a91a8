"""ctypes binding of libmsda.so (include/msda.h).

Argument marshalling only: shapes and dtypes are checked, outputs are
allocated with torch on the input's device, and the call goes to the HIP
library on torch's current stream.  There is no fallback: if the library is
missing or the GPU is absent, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmsda.so")

MSDA_OK = 0
MSDA_ERR_NULL = -1
MSDA_ERR_SHAPE = -2
MSDA_ERR_DTYPE = -3
MSDA_ERR_UNSUPPORTED = -4
MSDA_ERR_HIP = -5
MSDA_ERR_WORKSPACE = -6
MSDA_ERR_SCRATCH = -7
NOALLOC_SCRATCH_BYTES = 64 << 20
MSDA_F32 = 0
MSDA_BF16 = 1
MSDA_BWD_ACCUMULATE = 1
MSDA_ALIGN_CORNERS = 2
MSDA_SOFTMAX_PER_LEVEL = 4
MSDA_BWD_BINNED = 8

EXPORTED = ("msda_forward", "msda_backward_workspace_size", "msda_backward_workspace_min",
            "msda_backward", "msda_backward_noalloc", "msda_backward_events",
            "msda_forward_fused", "msda_backward_fused_workspace_size",
            "msda_backward_fused_workspace_min", "msda_backward_fused", "msda3d_forward",
            "msda3d_backward_workspace_size", "msda3d_backward_workspace_min",
            "msda3d_backward", "msda3d_validate_host",
            "msda_dat_attention_forward", "msda_dat_attention_workspace_size",
            "msda_dat_attention_backward",
            "msda_validate_host", "msda_status_string", "msda_last_hip_error")
BWD_STAGES = ("dots", "clear_bins", "count", "scan", "scatter", "tiles")
BWD_FUSED_STAGES = BWD_STAGES + ("prologue", "epilogue")

_lib = None


class MSDAError(RuntimeError):
    def __init__(self, code: int, where: str):
        detail = status_string(code)
        if code == MSDA_ERR_HIP:
            detail += f" (hipError_t {load().msda_last_hip_error()})"
        super().__init__(f"{where}: {detail} [{code}]")
        self.code = code


def load():
    """Load libmsda.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m scale_deformable_attention_04_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, ci, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
    lib.msda_forward.argtypes = [p, ci, p, p, p, p, p] + [i64] * 7 + [u32, p]
    lib.msda_forward.restype = ci
    lib.msda_backward.argtypes = ([p, ci, p, p, p, p, p, p, p, p] + [i64] * 7 +
                                  [p, ctypes.c_size_t, u32, p, p, p])
    lib.msda_backward.restype = ci
    lib.msda_backward_noalloc.argtypes = ([p, ci, p, p, p, p, p, p, p, p] + [i64] * 7 +
                                          [u32, p, p, p])
    lib.msda_backward_noalloc.restype = ci
    lib.msda_backward_events.argtypes = ([p, ci, p, p, p, p, p, p, p, p] + [i64] * 7 +
                                         [p, ctypes.c_size_t, u32, p, p, p, p])
    lib.msda_backward_events.restype = ci
    lib.msda_backward_workspace_size.argtypes = [i64] * 7
    lib.msda_backward_workspace_size.restype = ctypes.c_size_t
    lib.msda_backward_workspace_min.argtypes = [i64] * 7
    lib.msda_backward_workspace_min.restype = ctypes.c_size_t
    lib.msda_forward_fused.argtypes = [p, ci, p, p, p, p, p, p, p, p, p] + [i64] * 7 + [u32, p]
    lib.msda_forward_fused.restype = ci
    lib.msda_backward_fused_workspace_size.argtypes = [i64] * 7
    lib.msda_backward_fused_workspace_size.restype = ctypes.c_size_t
    lib.msda_backward_fused_workspace_min.argtypes = [i64] * 7
    lib.msda_backward_fused_workspace_min.restype = ctypes.c_size_t
    lib.msda_backward_fused.argtypes = ([p, ci, p, p, p, p, p, p, p, p, p, p, p, p, p, p] +
                                        [i64] * 7 +
                                        [p, ctypes.c_size_t, u32, p, p, p, p])
    lib.msda_backward_fused.restype = ci
    lib.msda3d_forward.argtypes = [p, ci, p, p, p, p, p] + [i64] * 7 + [u32, p]
    lib.msda3d_forward.restype = ci
    lib.msda3d_backward.argtypes = ([p, ci, p, p, p, p, p, p, p, p] + [i64] * 7 +
                                    [p, ctypes.c_size_t, u32, p, p, p])
    lib.msda3d_backward_workspace_size.argtypes = [i64] * 7
    lib.msda3d_backward_workspace_size.restype = ctypes.c_size_t
    lib.msda3d_backward_workspace_min.argtypes = [i64] * 7
    lib.msda3d_backward_workspace_min.restype = ctypes.c_size_t
    lib.msda3d_backward.restype = ci
    lib.msda3d_validate_host.argtypes = [p, p] + [i64] * 7
    lib.msda3d_validate_host.restype = ci
    f32 = ctypes.c_float
    lib.msda_dat_attention_forward.argtypes = [p] * 6 + [i64] * 5 + [f32, p]
    lib.msda_dat_attention_forward.restype = ci
    lib.msda_dat_attention_workspace_size.argtypes = [i64] * 5
    lib.msda_dat_attention_workspace_size.restype = ctypes.c_size_t
    lib.msda_dat_attention_backward.argtypes = ([p] * 12 + [ctypes.c_size_t] + [i64] * 5 +
                                                [f32, p])
    lib.msda_dat_attention_backward.restype = ci
    lib.msda_validate_host.argtypes = [p, p] + [i64] * 7
    lib.msda_validate_host.restype = ci
    lib.msda_status_string.argtypes = [ci]
    lib.msda_status_string.restype = ctypes.c_char_p
    lib.msda_last_hip_error.argtypes = []
    lib.msda_last_hip_error.restype = ci
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().msda_status_string(int(code)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MSDA_F32
    if t.dtype == torch.bfloat16:
        return MSDA_BF16
    raise TypeError(f"value must be float32 or bfloat16, got {t.dtype}")


def _need(t: torch.Tensor, name: str, dtype, device, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _dims(value, spatial_shapes, sampling_loc):
    if value.dim() != 4:
        raise ValueError(f"value must be [B, Nv, M, D], got {tuple(value.shape)}")
    B, Nv, M, D = value.shape
    if spatial_shapes.dim() != 2 or spatial_shapes.shape[1] != 2:
        raise ValueError("spatial_shapes must be [L, 2]")
    L = spatial_shapes.shape[0]
    if sampling_loc.dim() != 6:
        raise ValueError("sampling_loc must be [B, Nq, M, L, K, 2]")
    Nq, K = sampling_loc.shape[1], sampling_loc.shape[4]
    return int(B), int(Nv), int(Nq), int(M), int(D), int(L), int(K)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def validate_host(spatial_shapes, level_start_index, B, Nv, Nq, M, D, L, K) -> int:
    """msda_validate_host on host copies of the level table; returns the status code."""
    ss = torch.as_tensor(spatial_shapes, dtype=torch.int64).cpu().contiguous()
    st = torch.as_tensor(level_start_index, dtype=torch.int64).cpu().contiguous()
    return int(load().msda_validate_host(_ptr(ss), _ptr(st), B, Nv, Nq, M, D, L, K))


_workspaces = {}
_sides = {}


def workspace_size(B, Nv, Nq, M, D, L, K) -> int:
    """msda_backward_workspace_size: bytes of scratch the backward needs to
    compute grad_value in one pass."""
    return int(load().msda_backward_workspace_size(B, Nv, Nq, M, D, L, K))


def workspace_min(B, Nv, Nq, M, D, L, K) -> int:
    """msda_backward_workspace_min: the least scratch the backward accepts
    (grad_value then computed in passes)."""
    return int(load().msda_backward_workspace_min(B, Nv, Nq, M, D, L, K))


def _given_workspace(workspace, dev, size: int, least: int):
    """The caller's workspace (checked: >= least bytes), else the cached
    one of `size` bytes."""
    if workspace is None:
        return _workspace(dev, size)
    if workspace.device != dev or workspace.dtype != torch.uint8 or workspace.numel() < least:
        raise ValueError(f"workspace must be a uint8 tensor on {dev} of >= {least} bytes")
    return workspace


def _workspace(dev: torch.device, nbytes: int) -> Optional[torch.Tensor]:
    """A device buffer of at least nbytes (256-byte aligned, torch-owned),
    cached per (device, current stream): calls on one stream run in order and
    share it, calls on different streams get different buffers."""
    if nbytes == 0:
        return None
    key = (dev.type, dev.index, torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def _side_args(dev: torch.device, side_stream):
    """(side hipStream_t, hipEvent_t[2]) for a backward on torch's current stream.

    side_stream="auto": a second stream this module keeps for the current
    stream (created on first use, default priority), so that backwards issued
    on different streams each have their own; None: everything runs on the
    current stream; a torch.cuda.Stream: that stream.  The fork/join events
    are kept per (current stream, side stream) pair."""
    if side_stream is None:
        return ctypes.c_void_p(0), None
    cur = torch.cuda.current_stream(dev)
    auto = isinstance(side_stream, str)
    if auto and side_stream != "auto":
        raise ValueError("side_stream must be 'auto', None or a torch.cuda.Stream")
    key = (dev.index, cur.cuda_stream, None if auto else side_stream.cuda_stream)
    ent = _sides.get(key)
    if ent is None:
        side = torch.cuda.Stream(device=dev) if auto else side_stream
        evs = [torch.cuda.Event(), torch.cuda.Event()]
        for e in evs:
            e.record(side)  # torch creates the HIP event at its first record
        ent = (side, evs, (ctypes.c_void_p * 2)(*[e.cuda_event for e in evs]))
        _sides[key] = ent
    return ctypes.c_void_p(ent[0].cuda_stream), ent[2]


def _check_inputs(value, spatial_shapes, level_start_index, sampling_loc, attn_weight, validate):
    dev = value.device
    if dev.type != "cuda":
        raise ValueError(f"value must be a GPU tensor, got device {dev}")
    _dtype_code(value)
    B, Nv, Nq, M, D, L, K = _dims(value, spatial_shapes, sampling_loc)
    _need(value, "value", value.dtype, dev)
    _need(spatial_shapes, "spatial_shapes", torch.int64, dev, (L, 2))
    _need(level_start_index, "level_start_index", torch.int64, dev, (L,))
    _need(sampling_loc, "sampling_loc", torch.float32, dev, (B, Nq, M, L, K, 2))
    _need(attn_weight, "attn_weight", torch.float32, dev, (B, Nq, M, L, K))
    if validate:
        rc = validate_host(spatial_shapes, level_start_index, B, Nv, Nq, M, D, L, K)
        if rc != MSDA_OK:
            raise MSDAError(rc, "msda_validate_host")
    return dev, (B, Nv, Nq, M, D, L, K)


def forward(value: torch.Tensor, spatial_shapes: torch.Tensor, level_start_index: torch.Tensor,
            sampling_loc: torch.Tensor, attn_weight: torch.Tensor,
            out: Optional[torch.Tensor] = None, validate: bool = True,
            align_corners: bool = False) -> torch.Tensor:
    """msda_forward: out[B, Nq, M*D] (fp32) on torch's current stream.

    validate=True copies the level table to the host (one synchronization) and
    checks it with msda_validate_host; pass False when it is known good.
    align_corners=True selects the pixel convention x = u*(W-1), y = v*(H-1)."""
    lib = load()
    dev, (B, Nv, Nq, M, D, L, K) = _check_inputs(value, spatial_shapes, level_start_index,
                                                sampling_loc, attn_weight, validate)
    if out is None:
        out = torch.empty((B, Nq, M * D), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", torch.float32, dev, (B, Nq, M * D))
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.msda_forward(_ptr(value), _dtype_code(value), _ptr(spatial_shapes),
                              _ptr(level_start_index), _ptr(sampling_loc), _ptr(attn_weight),
                              _ptr(out), B, Nv, Nq, M, D, L, K,
                              MSDA_ALIGN_CORNERS if align_corners else 0,
                              ctypes.c_void_p(stream))
    if rc != MSDA_OK:
        raise MSDAError(rc, "msda_forward")
    return out


def stage_times(events: list) -> list:
    """Durations in us of the backward stages recorded by backward(events=...)
    or backward_fused(events=...), in the order of BWD_STAGES (BWD_FUSED_STAGES);
    call after the stream has been synchronized."""
    return [1000.0 * events[2 * i].elapsed_time(events[2 * i + 1])
            if events[2 * i] is not None else None for i in range(len(events) // 2)]


def make_events(stage: Optional[str] = None, fused: bool = False) -> list:
    """A fresh set of timing events for backward(events=...) (fused=False) or
    backward_fused(events=...): for every stage, or only for the named one
    (None in the other places)."""
    stages = BWD_FUSED_STAGES if fused else BWD_STAGES
    return [torch.cuda.Event(enable_timing=True)
            if stage is None or stages[i // 2] == stage else None
            for i in range(2 * len(stages))]


def _event_handles(events: list, n: int):
    if len(events) != 2 * n:
        raise ValueError(f"events: {2 * n} torch.cuda.Event expected")
    for e in events:
        if e is not None and not e.cuda_event:  # torch creates it at its first record
            e.record()
    return (ctypes.c_void_p * len(events))(
        *[e.cuda_event if e is not None else None for e in events])


def backward(value: torch.Tensor, spatial_shapes: torch.Tensor, level_start_index: torch.Tensor,
             sampling_loc: torch.Tensor, attn_weight: torch.Tensor, grad_out: torch.Tensor,
             grad_value: Optional[torch.Tensor] = None,
             grad_sampling_loc: Optional[torch.Tensor] = None,
             grad_attn_weight: Optional[torch.Tensor] = None,
             accumulate: bool = False, validate: bool = True,
             workspace: Optional[torch.Tensor] = None, events: Optional[list] = None,
             align_corners: bool = False, binned: bool = False, side_stream="auto"
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """msda_backward: (grad_value fp32 [B,Nv,M,D], grad_sampling_loc, grad_attn_weight).

    accumulate=True adds into the given grad_value instead of overwriting it.
    align_corners must be the value given to the forward.
    binned=True runs the binned grad_value pipeline even where the library
    would take its one-kernel path for small problems.
    workspace: a uint8 device tensor of at least workspace_min(...) bytes
    (workspace_size(...) for grad_value in one pass, the fastest); by default
    a buffer of workspace_size(...) bytes this module caches per (device,
    current stream).
    events: 2 * len(BWD_STAGES) torch.cuda.Event(enable_timing=True) objects
    or None; if given, msda_backward_events is called instead, which records
    events 2i and 2i + 1 around stage i (see stage_times), skipping None.
    side_stream: where the grad_attn_weight / grad_sampling_loc kernel runs
    (see _side_args): "auto" (default), None, or a torch.cuda.Stream."""
    lib = load()
    dev, (B, Nv, Nq, M, D, L, K) = _check_inputs(value, spatial_shapes, level_start_index,
                                                sampling_loc, attn_weight, validate)
    _need(grad_out, "grad_out", torch.float32, dev, (B, Nq, M * D))
    if grad_value is None:
        if accumulate:
            raise ValueError("accumulate=True needs a grad_value to add into")
        grad_value = torch.empty((B, Nv, M, D), dtype=torch.float32, device=dev)
    else:
        _need(grad_value, "grad_value", torch.float32, dev, (B, Nv, M, D))
    if grad_sampling_loc is None:
        grad_sampling_loc = torch.empty_like(sampling_loc)
    else:
        _need(grad_sampling_loc, "grad_sampling_loc", torch.float32, dev, sampling_loc.shape)
    if grad_attn_weight is None:
        grad_attn_weight = torch.empty_like(attn_weight)
    else:
        _need(grad_attn_weight, "grad_attn_weight", torch.float32, dev, attn_weight.shape)
    flags = ((MSDA_BWD_ACCUMULATE if accumulate else 0) |
             (MSDA_ALIGN_CORNERS if align_corners else 0) | (MSDA_BWD_BINNED if binned else 0))
    workspace = _given_workspace(workspace, dev, workspace_size(B, Nv, Nq, M, D, L, K),
                                 workspace_min(B, Nv, Nq, M, D, L, K))
    ws_bytes = workspace.numel() if workspace is not None else 0
    args = [_ptr(value), _dtype_code(value), _ptr(spatial_shapes), _ptr(level_start_index),
            _ptr(sampling_loc), _ptr(attn_weight), _ptr(grad_out), _ptr(grad_value),
            _ptr(grad_sampling_loc), _ptr(grad_attn_weight), B, Nv, Nq, M, D, L, K,
            _ptr(workspace), ws_bytes, flags]
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        side, side_ev = _side_args(dev, side_stream)
        if events is None:
            rc = lib.msda_backward(*args, stream, side, side_ev)
            where = "msda_backward"
        else:
            handles = _event_handles(events, len(BWD_STAGES))
            rc = lib.msda_backward_events(*args, stream, side, side_ev, handles)
            where = "msda_backward_events"
    if rc != MSDA_OK:
        raise MSDAError(rc, where)
    return grad_value, grad_sampling_loc, grad_attn_weight


def backward_noalloc(value: torch.Tensor, spatial_shapes: torch.Tensor,
                     level_start_index: torch.Tensor, sampling_loc: torch.Tensor,
                     attn_weight: torch.Tensor, grad_out: torch.Tensor,
                     grad_value: torch.Tensor, grad_sampling_loc: torch.Tensor,
                     grad_attn_weight: torch.Tensor, accumulate: bool = False,
                     align_corners: bool = False, binned: bool = False, side_stream=None
                     ) -> None:
    """msda_backward_noalloc into caller-allocated outputs: the backward with its
    workspace in the library's static per-GPU scratch: problems whose
    workspace_size exceeds NOALLOC_SCRATCH_BYTES run in passes, those whose
    workspace_min exceeds it raise MSDAError with MSDA_ERR_SCRATCH.  The
    call itself allocates nothing; calls overlapping in time on one GPU must
    not be made.  side_stream defaults to None here (everything on the
    current stream); a torch.cuda.Stream or "auto" work as for backward()."""
    lib = load()
    dev, (B, Nv, Nq, M, D, L, K) = _check_inputs(value, spatial_shapes, level_start_index,
                                                sampling_loc, attn_weight, False)
    _need(grad_out, "grad_out", torch.float32, dev, (B, Nq, M * D))
    _need(grad_value, "grad_value", torch.float32, dev, (B, Nv, M, D))
    _need(grad_sampling_loc, "grad_sampling_loc", torch.float32, dev, sampling_loc.shape)
    _need(grad_attn_weight, "grad_attn_weight", torch.float32, dev, attn_weight.shape)
    flags = ((MSDA_BWD_ACCUMULATE if accumulate else 0) |
             (MSDA_ALIGN_CORNERS if align_corners else 0) | (MSDA_BWD_BINNED if binned else 0))
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        side, side_ev = _side_args(dev, side_stream)
        rc = lib.msda_backward_noalloc(
            _ptr(value), _dtype_code(value), _ptr(spatial_shapes), _ptr(level_start_index),
            _ptr(sampling_loc), _ptr(attn_weight), _ptr(grad_out), _ptr(grad_value),
            _ptr(grad_sampling_loc), _ptr(grad_attn_weight), B, Nv, Nq, M, D, L, K, flags,
            stream, side, side_ev)
    if rc != MSDA_OK:
        raise MSDAError(rc, "msda_backward_noalloc")


# ---------------------------------------------------------------------------
# fused prologue: reference points + pixel offsets + attention logits
# ---------------------------------------------------------------------------
def _check_fused_inputs(value, spatial_shapes, level_start_index, reference_points,
                        sampling_offsets, attn_logits, validate, scale=None):
    dev = value.device
    if dev.type != "cuda":
        raise ValueError(f"value must be a GPU tensor, got device {dev}")
    _dtype_code(value)
    B, Nv, Nq, M, D, L, K = _dims(value, spatial_shapes, sampling_offsets)
    _need(value, "value", value.dtype, dev)
    _need(spatial_shapes, "spatial_shapes", torch.int64, dev, (L, 2))
    _need(level_start_index, "level_start_index", torch.int64, dev, (L,))
    _need(reference_points, "reference_points", torch.float32, dev, (B, Nq, L, 2))
    _need(sampling_offsets, "sampling_offsets", torch.float32, dev, (B, Nq, M, L, K, 2))
    _need(attn_logits, "attn_logits", torch.float32, dev, (B, Nq, M, L * K))
    if scale is not None:
        _need(scale, "scale", torch.float32, dev, (B, Nq, M, L, K))
    if validate:
        rc = validate_host(spatial_shapes, level_start_index, B, Nv, Nq, M, D, L, K)
        if rc != MSDA_OK:
            raise MSDAError(rc, "msda_validate_host")
    return dev, (B, Nv, Nq, M, D, L, K)


def _fused_flags(per_level: bool, align_corners: bool) -> int:
    return ((MSDA_SOFTMAX_PER_LEVEL if per_level else 0) |
            (MSDA_ALIGN_CORNERS if align_corners else 0))


def forward_fused(value: torch.Tensor, spatial_shapes: torch.Tensor,
                  level_start_index: torch.Tensor, reference_points: torch.Tensor,
                  sampling_offsets: torch.Tensor, attn_logits: torch.Tensor,
                  out: Optional[torch.Tensor] = None, validate: bool = True,
                  per_level: bool = False, align_corners: bool = False,
                  save: bool = False, scale: Optional[torch.Tensor] = None):
    """msda_forward_fused: out[B, Nq, M*D] (fp32) from reference points
    [B,Nq,L,2], pixel offsets [B,Nq,M,L,K,2] and logits [B,Nq,M,L*K].
    per_level=True normalizes the logits over each level's K points instead
    of all L*K; align_corners as in forward(); scale: an optional scale
    attention S [B,Nq,M,L,K] multiplying the softmax weights.  save=True
    returns (out, sampling_loc, attn_weight): the locations and weights it
    formed, to pass to backward_fused(saved=...)."""
    lib = load()
    dev, (B, Nv, Nq, M, D, L, K) = _check_fused_inputs(
        value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
        attn_logits, validate, scale)
    if out is None:
        out = torch.empty((B, Nq, M * D), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", torch.float32, dev, (B, Nq, M * D))
    loc = torch.empty((B, Nq, M, L, K, 2), dtype=torch.float32, device=dev) if save else None
    attn = torch.empty((B, Nq, M, L, K), dtype=torch.float32, device=dev) if save else None
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.msda_forward_fused(_ptr(value), _dtype_code(value), _ptr(spatial_shapes),
                                    _ptr(level_start_index), _ptr(reference_points),
                                    _ptr(sampling_offsets), _ptr(attn_logits), _ptr(scale),
                                    _ptr(out), _ptr(loc), _ptr(attn), B, Nv, Nq, M, D, L, K,
                                    _fused_flags(per_level, align_corners),
                                    ctypes.c_void_p(stream))
    if rc != MSDA_OK:
        raise MSDAError(rc, "msda_forward_fused")
    return (out, loc, attn) if save else out


def fused_workspace_size(B, Nv, Nq, M, D, L, K) -> int:
    """msda_backward_fused_workspace_size."""
    return int(load().msda_backward_fused_workspace_size(B, Nv, Nq, M, D, L, K))


def fused_workspace_min(B, Nv, Nq, M, D, L, K) -> int:
    """msda_backward_fused_workspace_min."""
    return int(load().msda_backward_fused_workspace_min(B, Nv, Nq, M, D, L, K))


def backward_fused(value: torch.Tensor, spatial_shapes: torch.Tensor,
                   level_start_index: torch.Tensor, reference_points: torch.Tensor,
                   sampling_offsets: torch.Tensor, attn_logits: torch.Tensor,
                   grad_out: torch.Tensor, grad_value: Optional[torch.Tensor] = None,
                   accumulate: bool = False, need_grad_ref: bool = True,
                   validate: bool = True, workspace: Optional[torch.Tensor] = None,
                   events: Optional[list] = None, per_level: bool = False,
                   align_corners: bool = False, saved: Optional[tuple] = None,
                   side_stream="auto", scale: Optional[torch.Tensor] = None):
    """msda_backward_fused: (grad_value, grad_sampling_offsets, grad_attn_logits,
    grad_reference_points or None when need_grad_ref is False), and
    grad_scale as a fifth element when scale (the forward's) is given.
    side_stream as for backward(); workspace too, with fused_workspace_min /
    fused_workspace_size.
    saved: the (sampling_loc, attn_weight) forward_fused(save=True) returned
    for these inputs, or None to recompute them.
    events: 2 * len(BWD_FUSED_STAGES) timing events or None (see stage_times)."""
    lib = load()
    dev, (B, Nv, Nq, M, D, L, K) = _check_fused_inputs(
        value, spatial_shapes, level_start_index, reference_points, sampling_offsets,
        attn_logits, validate, scale)
    _need(grad_out, "grad_out", torch.float32, dev, (B, Nq, M * D))
    if grad_value is None:
        if accumulate:
            raise ValueError("accumulate=True needs a grad_value to add into")
        grad_value = torch.empty((B, Nv, M, D), dtype=torch.float32, device=dev)
    else:
        _need(grad_value, "grad_value", torch.float32, dev, (B, Nv, M, D))
    s_loc = s_attn = None
    if saved is not None:
        s_loc, s_attn = saved
        _need(s_loc, "saved sampling_loc", torch.float32, dev, (B, Nq, M, L, K, 2))
        _need(s_attn, "saved attn_weight", torch.float32, dev, (B, Nq, M, L, K))
    g_off = torch.empty_like(sampling_offsets)
    g_logits = torch.empty_like(attn_logits)
    g_ref = torch.empty_like(reference_points) if need_grad_ref else None
    g_scale = torch.empty_like(scale) if scale is not None else None
    flags = _fused_flags(per_level, align_corners) | (MSDA_BWD_ACCUMULATE if accumulate else 0)
    workspace = _given_workspace(workspace, dev, fused_workspace_size(B, Nv, Nq, M, D, L, K),
                                 fused_workspace_min(B, Nv, Nq, M, D, L, K))
    ws_bytes = workspace.numel() if workspace is not None else 0
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        handles = None if events is None else _event_handles(events, len(BWD_FUSED_STAGES))
        side, side_ev = _side_args(dev, side_stream)
        rc = lib.msda_backward_fused(
            _ptr(value), _dtype_code(value), _ptr(spatial_shapes), _ptr(level_start_index),
            _ptr(reference_points), _ptr(sampling_offsets), _ptr(attn_logits), _ptr(scale),
            _ptr(s_loc), _ptr(s_attn), _ptr(grad_out), _ptr(grad_value), _ptr(g_off),
            _ptr(g_logits), _ptr(g_scale), _ptr(g_ref), B, Nv, Nq, M, D, L, K,
            _ptr(workspace), ws_bytes, flags, stream, side, side_ev, handles)
    if rc != MSDA_OK:
        raise MSDAError(rc, "msda_backward_fused")
    if scale is not None:
        return grad_value, g_off, g_logits, g_ref, g_scale
    return grad_value, g_off, g_logits, g_ref


# ---------------------------------------------------------------------------
# 3-D (trilinear) variant
# ---------------------------------------------------------------------------
def validate_host3d(volume_shapes, level_start_index, B, Nv, Nq, M, D, L, K) -> int:
    """msda3d_validate_host on host copies of the level table; returns the status code."""
    ss = torch.as_tensor(volume_shapes, dtype=torch.int64).cpu().contiguous()
    st = torch.as_tensor(level_start_index, dtype=torch.int64).cpu().contiguous()
    return int(load().msda3d_validate_host(_ptr(ss), _ptr(st), B, Nv, Nq, M, D, L, K))


def _check_inputs3d(value, volume_shapes, level_start_index, sampling_loc, attn_weight,
                    validate):
    dev = value.device
    if dev.type != "cuda":
        raise ValueError(f"value must be a GPU tensor, got device {dev}")
    _dtype_code(value)
    if value.dim() != 4:
        raise ValueError(f"value must be [B, Nv, M, D], got {tuple(value.shape)}")
    if volume_shapes.dim() != 2 or volume_shapes.shape[1] != 3:
        raise ValueError("volume_shapes must be [L, 3]")
    if sampling_loc.dim() != 6 or sampling_loc.shape[-1] != 3:
        raise ValueError("sampling_loc must be [B, Nq, M, L, K, 3]")
    B, Nv, M, D = (int(v) for v in value.shape)
    L = int(volume_shapes.shape[0])
    Nq, K = int(sampling_loc.shape[1]), int(sampling_loc.shape[4])
    _need(value, "value", value.dtype, dev)
    _need(volume_shapes, "volume_shapes", torch.int64, dev, (L, 3))
    _need(level_start_index, "level_start_index", torch.int64, dev, (L,))
    _need(sampling_loc, "sampling_loc", torch.float32, dev, (B, Nq, M, L, K, 3))
    _need(attn_weight, "attn_weight", torch.float32, dev, (B, Nq, M, L, K))
    if validate:
        rc = validate_host3d(volume_shapes, level_start_index, B, Nv, Nq, M, D, L, K)
        if rc != MSDA_OK:
            raise MSDAError(rc, "msda3d_validate_host")
    return dev, (B, Nv, Nq, M, D, L, K)


def forward3d(value: torch.Tensor, volume_shapes: torch.Tensor, level_start_index: torch.Tensor,
              sampling_loc: torch.Tensor, attn_weight: torch.Tensor,
              out: Optional[torch.Tensor] = None, validate: bool = True,
              align_corners: bool = False) -> torch.Tensor:
    """msda3d_forward: out[B, Nq, M*D] (fp32) on torch's current stream."""
    lib = load()
    dev, (B, Nv, Nq, M, D, L, K) = _check_inputs3d(value, volume_shapes, level_start_index,
                                                  sampling_loc, attn_weight, validate)
    if out is None:
        out = torch.empty((B, Nq, M * D), dtype=torch.float32, device=dev)
    else:
        _need(out, "out", torch.float32, dev, (B, Nq, M * D))
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = lib.msda3d_forward(_ptr(value), _dtype_code(value), _ptr(volume_shapes),
                                _ptr(level_start_index), _ptr(sampling_loc), _ptr(attn_weight),
                                _ptr(out), B, Nv, Nq, M, D, L, K,
                                MSDA_ALIGN_CORNERS if align_corners else 0,
                                ctypes.c_void_p(stream))
    if rc != MSDA_OK:
        raise MSDAError(rc, "msda3d_forward")
    return out


def workspace_size3d(B, Nv, Nq, M, D, L, K) -> int:
    """msda3d_backward_workspace_size."""
    return int(load().msda3d_backward_workspace_size(B, Nv, Nq, M, D, L, K))


def workspace_min3d(B, Nv, Nq, M, D, L, K) -> int:
    """msda3d_backward_workspace_min."""
    return int(load().msda3d_backward_workspace_min(B, Nv, Nq, M, D, L, K))


def backward3d(value: torch.Tensor, volume_shapes: torch.Tensor, level_start_index: torch.Tensor,
               sampling_loc: torch.Tensor, attn_weight: torch.Tensor, grad_out: torch.Tensor,
               grad_value: Optional[torch.Tensor] = None, accumulate: bool = False,
               validate: bool = True, align_corners: bool = False,
               workspace: Optional[torch.Tensor] = None, side_stream="auto"):
    """msda3d_backward: (grad_value fp32 [B,Nv,M,D], grad_sampling_loc, grad_attn_weight).
    side_stream as for backward(); workspace too, with workspace_min3d /
    workspace_size3d."""
    lib = load()
    dev, (B, Nv, Nq, M, D, L, K) = _check_inputs3d(value, volume_shapes, level_start_index,
                                                  sampling_loc, attn_weight, validate)
    _need(grad_out, "grad_out", torch.float32, dev, (B, Nq, M * D))
    if grad_value is None:
        if accumulate:
            raise ValueError("accumulate=True needs a grad_value to add into")
        grad_value = torch.empty((B, Nv, M, D), dtype=torch.float32, device=dev)
    else:
        _need(grad_value, "grad_value", torch.float32, dev, (B, Nv, M, D))
    g_loc = torch.empty_like(sampling_loc)
    g_attn = torch.empty_like(attn_weight)
    flags = (MSDA_BWD_ACCUMULATE if accumulate else 0) | (MSDA_ALIGN_CORNERS if align_corners else 0)
    workspace = _given_workspace(workspace, dev, workspace_size3d(B, Nv, Nq, M, D, L, K),
                                 workspace_min3d(B, Nv, Nq, M, D, L, K))
    ws_bytes = workspace.numel() if workspace is not None else 0
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        side, side_ev = _side_args(dev, side_stream)
        rc = lib.msda3d_backward(_ptr(value), _dtype_code(value), _ptr(volume_shapes),
                                 _ptr(level_start_index), _ptr(sampling_loc), _ptr(attn_weight),
                                 _ptr(grad_out), _ptr(grad_value), _ptr(g_loc), _ptr(g_attn),
                                 B, Nv, Nq, M, D, L, K, _ptr(workspace), ws_bytes, flags, stream,
                                 side, side_ev)
    if rc != MSDA_OK:
        raise MSDAError(rc, "msda3d_backward")
    return grad_value, g_loc, g_attn


# ---------------------------------------------------------------------------
# DAT: deformable sampling of keys/values and the attention against them
# ---------------------------------------------------------------------------
_dat_cache = {}


def _level_of(hw, dev):
    """The one-level table (H, W), start 0 on dev, built once per (H, W, device)
    (building it is a host-to-device copy)."""
    H, W = (int(v) for v in hw)
    key = ("level", H, W, dev.type, dev.index)
    if key not in _dat_cache:
        _dat_cache[key] = (torch.tensor([[H, W]], dtype=torch.int64, device=dev),
                           torch.zeros(1, dtype=torch.int64, device=dev))
    return _dat_cache[key]


def _ones_of(shape, dev):
    """A cached all-ones fp32 weight tensor of this shape on dev."""
    key = ("ones", tuple(shape), dev.type, dev.index)
    if key not in _dat_cache:
        _dat_cache[key] = torch.ones(shape, dtype=torch.float32, device=dev)
    return _dat_cache[key]


def dat_sample(x: torch.Tensor, hw, pos: torch.Tensor, validate: bool = True) -> torch.Tensor:
    """DAT's sampling step through msda_forward: x [B, H*W, G, Dg] (fp32 or
    bf16, channel-last), pos [B, Ns, G, 2] normalized (u, v); returns the
    sampled features [B, Ns, G*Dg] (bilinear, align_corners=True, zeros)."""
    B, Nv, G, Dg = x.shape
    Ns = pos.shape[1]
    ss, st = _level_of(hw, x.device)
    ones = _ones_of((B, Ns, G, 1, 1), x.device)
    return forward(x, ss, st, pos.reshape(B, Ns, G, 1, 1, 2), ones, validate=validate,
                   align_corners=True)


def dat_sample_backward(x: torch.Tensor, hw, pos: torch.Tensor, grad_sampled: torch.Tensor,
                        validate: bool = True):
    """(grad_x [B, H*W, G, Dg] fp32, grad_pos [B, Ns, G, 2]) through msda_backward."""
    B, Nv, G, Dg = x.shape
    Ns = pos.shape[1]
    ss, st = _level_of(hw, x.device)
    ones = _ones_of((B, Ns, G, 1, 1), x.device)
    gx, gl, _ = backward(x, ss, st, pos.reshape(B, Ns, G, 1, 1, 2), ones,
                         grad_sampled.contiguous(), validate=validate, align_corners=True)
    return gx, gl.reshape(B, Ns, G, 2)


def _attn_dims(q, k, v, bias):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, N, heads, d] and k, v [B, Ns, heads, d]")
    B, N, Hh, d = (int(t) for t in q.shape)
    Ns = int(k.shape[1])
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"q must be a GPU tensor, got device {dev}")
    _need(q, "q", torch.float32, dev)
    _need(k, "k", torch.float32, dev, (B, Ns, Hh, d))
    _need(v, "v", torch.float32, dev, (B, Ns, Hh, d))
    if bias is not None:
        _need(bias, "bias", torch.float32, dev, (B, Hh, N, Ns))
    return dev, (B, N, Ns, Hh, d)


def dat_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  bias: Optional[torch.Tensor] = None, scale: Optional[float] = None):
    """msda_dat_attention_forward: (out [B, N, heads, d], lse [B, heads, N])."""
    lib = load()
    dev, (B, N, Ns, Hh, d) = _attn_dims(q, k, v, bias)
    scale = d ** -0.5 if scale is None else float(scale)
    out = torch.empty((B, N, Hh, d), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hh, N), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        rc = lib.msda_dat_attention_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(out),
                                            _ptr(lse), B, N, Ns, Hh, d, scale, stream)
    if rc != MSDA_OK:
        raise MSDAError(rc, "msda_dat_attention_forward")
    return out, lse


def dat_attention_backward(q, k, v, out, lse, grad_out, bias=None, need_grad_bias=False,
                           scale=None, workspace: Optional[torch.Tensor] = None):
    """msda_dat_attention_backward: (grad_q, grad_k, grad_v, grad_bias or None)."""
    lib = load()
    dev, (B, N, Ns, Hh, d) = _attn_dims(q, k, v, bias)
    scale = d ** -0.5 if scale is None else float(scale)
    _need(out, "out", torch.float32, dev, (B, N, Hh, d))
    _need(lse, "lse", torch.float32, dev, (B, Hh, N))
    _need(grad_out, "grad_out", torch.float32, dev, (B, N, Hh, d))
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    gb = torch.empty_like(bias) if (need_grad_bias and bias is not None) else None
    need = int(lib.msda_dat_attention_workspace_size(B, N, Ns, Hh, d))
    if workspace is None:
        workspace = _workspace(dev, need)
    elif workspace.device != dev or workspace.dtype != torch.uint8 or workspace.numel() < need:
        raise ValueError(f"workspace must be a uint8 tensor on {dev} of >= {need} bytes")
    ws_bytes = workspace.numel() if workspace is not None else 0
    with torch.cuda.device(dev):
        stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        rc = lib.msda_dat_attention_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(bias), _ptr(out),
                                             _ptr(lse), _ptr(grad_out), _ptr(gq), _ptr(gk),
                                             _ptr(gv), _ptr(gb), _ptr(workspace), ws_bytes,
                                             B, N, Ns, Hh, d, scale, stream)
    if rc != MSDA_OK:
        raise MSDAError(rc, "msda_dat_attention_backward")
    return gq, gk, gv, gb
