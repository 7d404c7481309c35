"""Thin Python binding over libgla.so (include/gla.h).

Argument marshalling only: tensors supply device pointers, torch supplies the
current HIP stream, and every step of the computation runs in the library's
HIP kernels.  There is no CPU fallback: a missing library or a tensor that is
not on the GPU raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgla.so")

GLA_OK, GLA_ERR_INVALID_ARG, GLA_ERR_UNSUPPORTED, GLA_ERR_LAUNCH = 0, 1, 2, 3
GLA_BF16, GLA_F32 = 0, 1

_lib = None


class GLAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{status_string(status)}: {detail}")
        self.status = status


def load_library():
    """Open libgla.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sub_quadratic_sequence_amd.build` "
                "or __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        P, I = ctypes.c_void_p, ctypes.c_int
        lib.gla_chunk_fwd.restype = I
        lib.gla_chunk_fwd.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P]
        lib.gla_chunk_fwd_workspace_size.restype = ctypes.c_size_t
        lib.gla_chunk_fwd_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
        lib.gla_chunk_fwd_noalloc.restype = I
        lib.gla_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P]
        lib.gla_chunk_fwd_ws.restype = I
        lib.gla_chunk_fwd_ws.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P,
                                         ctypes.c_size_t, P]
        lib.gla_chunk_fwd_sliced.restype = I
        lib.gla_chunk_fwd_sliced.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, P]
        lib.gla_slice_plan.restype = I
        lib.gla_slice_plan.argtypes = [ctypes.c_longlong, I, I, I]
        lib.gla_split_plan.restype = I
        lib.gla_split_plan.argtypes = [ctypes.c_longlong, I, I, I, I, ctypes.POINTER(I)]
        lib.gla_chunk_fwd_segments_workspace_size.restype = ctypes.c_size_t
        lib.gla_chunk_fwd_segments_workspace_size.argtypes = [I, I, I, I, I, I]
        lib.gla_chunk_fwd_segments.restype = I
        lib.gla_chunk_fwd_segments.argtypes = [P] * 7 + [I] * 8 + [P, ctypes.c_size_t, P]
        lib.gla_chunk_bwd_workspace_size.restype = ctypes.c_size_t
        lib.gla_chunk_bwd_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
        lib.gla_chunk_bwd.restype = I
        lib.gla_chunk_bwd.argtypes = [P] * 13 + [I] * 8 + [P, ctypes.c_size_t, P]
        lib.gla_chunk_bwd_saved.restype = I
        lib.gla_chunk_bwd_saved.argtypes = [P] * 13 + [I] * 8 + [P, ctypes.c_size_t, P]
        lib.gla_chunk_fwd_states.restype = I
        lib.gla_chunk_fwd_states.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P,
                                             ctypes.c_size_t, P]
        lib.gdn_chunk_fwd.restype = I
        lib.gdn_chunk_fwd.argtypes = [P] * 9 + [I] * 8 + [P]
        lib.gla_recurrent_step.restype = I
        lib.gla_recurrent_step.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P]
        lib.gla_status_string.restype = ctypes.c_char_p
        lib.gla_status_string.argtypes = [I]
        lib.gla_last_error.restype = ctypes.c_char_p
        lib.gla_last_error.argtypes = []
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load_library().gla_status_string(int(status)).decode()


def last_error() -> str:
    return load_library().gla_last_error().decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GLA_BF16
    if t.dtype == torch.float32:
        return GLA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_gpu(name, t, dtype=None, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device}); there is no CPU path")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arguments on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def workspace_size(q, v, cu_seqlens=None, chunk_size: int = 64) -> int:
    """Bytes of workspace the sequence-split forward needs for these inputs (0: none)."""
    B, H, T, dk = q.shape
    num_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    return int(load_library().gla_chunk_fwd_workspace_size(num_seqs, B, H, T, dk, v.shape[-1],
                                                           int(chunk_size), _dtype_code(q)))


def gla_chunk_fwd(q, k, v, g, initial_state=None, output_final_state=False, cu_seqlens=None,
                  chunk_size: int = 64, out=None, final_state=None, split: bool = True,
                  workspace=None, noalloc: bool = False, dv_slice=None):
    """Chunkwise GLA forward.

    q, k, g: [B, H, T, dk]; v: [B, H, T, dv] (bfloat16 or float32, same dtype);
    initial_state: [Nseq, H, dk, dv] float32 or None; cu_seqlens: int32 [Nseq+1]
    on the GPU for packed sequences (B == 1).  Returns ``(o, final_state)``;
    ``final_state`` is None unless ``output_final_state`` (or ``final_state``
    is passed, which may alias ``initial_state``).

    With ``split`` (the default) the call goes through ``gla_chunk_fwd_ws``,
    which cuts long sequences into segments when the inputs have too few
    (sequence, head) units to fill the device; the workspace it needs is a
    torch allocation (or ``workspace``, a uint8 GPU tensor).  ``split=False``
    calls ``gla_chunk_fwd``, which never splits.  ``noalloc=True`` calls
    ``gla_chunk_fwd_noalloc`` (the same split, its scratch in the library's own
    device array; see ``gla_chunk_fwd_noalloc`` below).  ``dv_slice`` (64, 128
    or 0) calls ``gla_chunk_fwd_sliced``: never split, value columns per work
    item chosen by the caller (0: the library's choice, as ``split=False``).
    """
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _check_gpu("q", q)
    dt = q.dtype
    _check_gpu("k", k, dt, q.shape, device=q.device)
    _check_gpu("g", g, dt, q.shape, device=q.device)
    _check_gpu("v", v, dt, (B, H, T, dv), device=q.device)
    nseq = B
    num_seqs = 0
    if cu_seqlens is not None:
        _check_gpu("cu_seqlens", cu_seqlens, torch.int32, device=q.device)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be 1-D with num_seqs + 1 >= 2 offsets")
        num_seqs = cu_seqlens.numel() - 1
        nseq = num_seqs
    if initial_state is not None:
        _check_gpu("initial_state", initial_state, torch.float32, (nseq, H, dk, dv),
                   device=q.device)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dt, device=q.device)
    else:
        _check_gpu("out", out, dt, (B, H, T, dv), device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _check_gpu("final_state", final_state, torch.float32, (nseq, H, dk, dv), device=q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(initial_state), _ptr(out),
                _ptr(final_state), _ptr(cu_seqlens), num_seqs, B, H, T, dk, dv, int(chunk_size),
                _dtype_code(q))
        if dv_slice is not None:
            rc = lib.gla_chunk_fwd_sliced(*args, int(dv_slice), ctypes.c_void_p(stream))
        elif noalloc:
            rc = lib.gla_chunk_fwd_noalloc(*args, ctypes.c_void_p(stream))
        elif split:
            need = workspace_size(q, v, cu_seqlens, chunk_size)
            if need and workspace is None:
                workspace = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
            ws_ptr, ws_bytes = None, 0
            if workspace is not None:
                _check_gpu("workspace", workspace, torch.uint8, device=q.device)
                base = workspace.data_ptr()
                off = (-base) % 256
                ws_ptr, ws_bytes = ctypes.c_void_p(base + off), max(0, workspace.numel() - off)
            rc = lib.gla_chunk_fwd_ws(*args, ws_ptr, ws_bytes, ctypes.c_void_p(stream))
        else:
            rc = lib.gla_chunk_fwd(*args, ctypes.c_void_p(stream))
    if rc != GLA_OK:
        raise GLAError(rc, last_error())
    return out, final_state


def gla_chunk_fwd_noalloc(q, k, v, g, initial_state=None, output_final_state=False,
                          cu_seqlens=None, chunk_size: int = 64, out=None, final_state=None):
    """``gla_chunk_fwd`` through the C entry point ``gla_chunk_fwd_noalloc``: the
    sequence split of ``gla_chunk_fwd_ws`` with its scratch in a device array the
    library holds, so the C call allocates nothing.  Pass ``out`` (and
    ``final_state``) to keep this wrapper from allocating them with torch.  Calls
    that overlap on one device race on that array."""
    return gla_chunk_fwd(q, k, v, g, initial_state=initial_state,
                         output_final_state=output_final_state, cu_seqlens=cu_seqlens,
                         chunk_size=chunk_size, out=out, final_state=final_state, noalloc=True)


def gla_chunk_fwd_ws(q, k, v, g, initial_state=None, output_final_state=False, cu_seqlens=None,
                     chunk_size: int = 64, out=None, final_state=None, workspace=None):
    """``gla_chunk_fwd`` through the C entry point ``gla_chunk_fwd_ws`` (the sequence
    split when it pays; ``workspace`` a uint8 GPU tensor, else allocated with torch)."""
    return gla_chunk_fwd(q, k, v, g, initial_state=initial_state,
                         output_final_state=output_final_state, cu_seqlens=cu_seqlens,
                         chunk_size=chunk_size, out=out, final_state=final_state, split=True,
                         workspace=workspace)


def gla_chunk_fwd_sliced(q, k, v, g, dv_slice: int, initial_state=None, output_final_state=False,
                         cu_seqlens=None, chunk_size: int = 64, out=None, final_state=None):
    """``gla_chunk_fwd`` through the C entry point ``gla_chunk_fwd_sliced``: never split,
    ``dv_slice`` (64, 128, or 0 for the library's choice) value columns per work item."""
    return gla_chunk_fwd(q, k, v, g, initial_state=initial_state,
                         output_final_state=output_final_state, cu_seqlens=cu_seqlens,
                         chunk_size=chunk_size, out=out, final_state=final_state, dv_slice=dv_slice)


def split_plan(units: int, T: int, dv: int, dtype=torch.bfloat16, num_cus=None):
    """``(segments, segment_length)`` that the sequence-split forward uses for
    fixed-length inputs of ``units`` = B x H (sequence, head) pairs of ``T``
    tokens and ``dv`` value columns (``gla_split_plan``; host-only).
    ``num_cus`` defaults to the current GPU's compute-unit count."""
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    code = GLA_BF16 if dtype == torch.bfloat16 else GLA_F32
    seg_len = ctypes.c_int(0)
    n = load_library().gla_split_plan(int(units), int(T), int(dv), code, int(num_cus),
                                      ctypes.byref(seg_len))
    return int(n), int(seg_len.value)


def slice_plan(units: int, dv: int, dtype=torch.bfloat16, num_cus=None) -> int:
    """Value columns per work item (64 or 128) that the unsplit forward takes for
    ``units`` (sequence, head) pairs and ``dv`` value columns (``gla_slice_plan``;
    host-only).  ``num_cus`` defaults to the current GPU's compute-unit count."""
    if num_cus is None:
        num_cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    code = GLA_BF16 if dtype == torch.bfloat16 else GLA_F32
    return int(load_library().gla_slice_plan(int(units), int(dv), code, int(num_cus)))


gla_split_plan = split_plan   # the C entry point's name
gla_slice_plan = slice_plan


def gla_chunk_fwd_segments(q, k, v, g, num_segments: int, initial_state=None,
                           output_final_state=False, chunk_size: int = 64, out=None,
                           final_state=None, workspace=None):
    """The sequence-split forward with a caller-chosen segment count
    (``gla_chunk_fwd_segments``); fixed-length inputs.  Shapes and results as
    ``gla_chunk_fwd``; ``workspace`` (uint8 GPU tensor) is allocated with torch
    when not given."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _check_gpu("q", q)
    dt = q.dtype
    _check_gpu("k", k, dt, q.shape, device=q.device)
    _check_gpu("g", g, dt, q.shape, device=q.device)
    _check_gpu("v", v, dt, (B, H, T, dv), device=q.device)
    if initial_state is not None:
        _check_gpu("initial_state", initial_state, torch.float32, (B, H, dk, dv), device=q.device)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dt, device=q.device)
    else:
        _check_gpu("out", out, dt, (B, H, T, dv), device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _check_gpu("final_state", final_state, torch.float32, (B, H, dk, dv), device=q.device)
    lib = load_library()
    need = int(lib.gla_chunk_fwd_segments_workspace_size(B, H, T, dk, dv, int(num_segments)))
    if need and workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _aligned_workspace(workspace, q.device)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.gla_chunk_fwd_segments(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(initial_state),
                                        _ptr(out), _ptr(final_state), B, H, T, dk, dv,
                                        int(chunk_size), _dtype_code(q), int(num_segments), ws_ptr,
                                        ws_bytes, ctypes.c_void_p(stream))
    if rc != GLA_OK:
        raise GLAError(rc, last_error())
    return out, final_state


def bwd_workspace_size(q, v, cu_seqlens=None, chunk_size: int = 64) -> int:
    """Bytes of workspace ``gla_chunk_bwd`` needs for these inputs (its chunk states)."""
    B, H, T, dk = q.shape
    num_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    return int(load_library().gla_chunk_bwd_workspace_size(num_seqs, B, H, T, dk, v.shape[-1],
                                                           int(chunk_size), _dtype_code(q)))


def _aligned_workspace(workspace, device):
    """(pointer, bytes) of the 256-byte aligned part of a uint8 GPU tensor."""
    _check_gpu("workspace", workspace, torch.uint8, device=device)
    base = workspace.data_ptr()
    off = (-base) % 256
    return ctypes.c_void_p(base + off), max(0, workspace.numel() - off)


def gla_chunk_fwd_states(q, k, v, g, initial_state=None, output_final_state=False, cu_seqlens=None,
                         chunk_size: int = 64, out=None, final_state=None, chunk_states=None):
    """The forward (``gla_chunk_fwd_states``, bfloat16, d_k and d_v in {64, 128},
    unsplit, 64-column slices) that also writes the state entering every chunk into
    ``chunk_states``, the backward's workspace (a uint8 GPU tensor of at least
    ``bwd_workspace_size`` bytes; allocated when not given).  Returns
    ``(o, final_state, chunk_states)``; pass ``chunk_states`` to ``gla_chunk_bwd``
    with ``states_saved=True`` to skip the backward's state recomputation."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _check_gpu("q", q)
    dt = q.dtype
    _check_gpu("k", k, dt, q.shape, device=q.device)
    _check_gpu("g", g, dt, q.shape, device=q.device)
    _check_gpu("v", v, dt, (B, H, T, dv), device=q.device)
    nseq, num_seqs = B, 0
    if cu_seqlens is not None:
        _check_gpu("cu_seqlens", cu_seqlens, torch.int32, device=q.device)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be 1-D with num_seqs + 1 >= 2 offsets")
        num_seqs = cu_seqlens.numel() - 1
        nseq = num_seqs
    if initial_state is not None:
        _check_gpu("initial_state", initial_state, torch.float32, (nseq, H, dk, dv), device=q.device)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dt, device=q.device)
    else:
        _check_gpu("out", out, dt, (B, H, T, dv), device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _check_gpu("final_state", final_state, torch.float32, (nseq, H, dk, dv), device=q.device)
    if chunk_states is None:
        chunk_states = torch.empty(bwd_workspace_size(q, v, cu_seqlens, chunk_size) + 256,
                                   dtype=torch.uint8, device=q.device)
    ws_ptr, ws_bytes = _aligned_workspace(chunk_states, q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.gla_chunk_fwd_states(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(initial_state),
                                      _ptr(out), _ptr(final_state), _ptr(cu_seqlens), num_seqs, B, H,
                                      T, dk, dv, int(chunk_size), _dtype_code(q), ws_ptr, ws_bytes,
                                      ctypes.c_void_p(stream))
    if rc != GLA_OK:
        raise GLAError(rc, last_error())
    return out, final_state, chunk_states


def gla_chunk_bwd(q, k, v, g, do, initial_state=None, d_final_state=None, cu_seqlens=None,
                  chunk_size: int = 64, want_d_initial_state=None, workspace=None, out=None,
                  states_saved: bool = False):
    """Chunkwise GLA backward (C entry point ``gla_chunk_bwd``).

    Gradients of sum(o * do) + sum(final_state * d_final_state) for the forward
    ``gla_chunk_fwd(q, k, v, g, initial_state)``.  q, k, g: [B, H, T, dk]; v, do:
    [B, H, T, dv], bfloat16; initial_state, d_final_state: [Nseq, H, dk, dv]
    float32 or None.  Returns ``(dq, dk, dv, dg, d_initial_state)``;
    ``d_initial_state`` is computed when ``initial_state`` is given (or
    ``want_d_initial_state``), else None.  The workspace (the chunk states) is a
    torch allocation unless ``workspace`` (a uint8 GPU tensor) is passed;
    ``out`` optionally supplies (dq, dk, dv, dg) to write into.  With
    ``states_saved`` the workspace is the ``chunk_states`` of a
    ``gla_chunk_fwd_states`` call on the same inputs, and the backward
    (``gla_chunk_bwd_saved``) skips recomputing them.
    """
    if states_saved and workspace is None:
        raise ValueError("states_saved needs the workspace that gla_chunk_fwd_states filled")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _check_gpu("q", q)
    dt = q.dtype
    _check_gpu("k", k, dt, q.shape, device=q.device)
    _check_gpu("g", g, dt, q.shape, device=q.device)
    _check_gpu("v", v, dt, (B, H, T, dv), device=q.device)
    _check_gpu("do", do, dt, (B, H, T, dv), device=q.device)
    nseq, num_seqs = B, 0
    if cu_seqlens is not None:
        _check_gpu("cu_seqlens", cu_seqlens, torch.int32, device=q.device)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be 1-D with num_seqs + 1 >= 2 offsets")
        num_seqs = cu_seqlens.numel() - 1
        nseq = num_seqs
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None:
            _check_gpu(name, t, torch.float32, (nseq, H, dk, dv), device=q.device)
    if want_d_initial_state is None:
        want_d_initial_state = initial_state is not None
    if out is None:
        dq, dk_, dv_, dg = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                            torch.empty_like(g))
    else:
        dq, dk_, dv_, dg = out
        for name, t, ref in (("dq", dq, q), ("dk", dk_, k), ("dv", dv_, v), ("dg", dg, g)):
            _check_gpu(name, t, dt, tuple(ref.shape), device=q.device)
    ds0 = (torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=q.device)
           if want_d_initial_state else None)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        if workspace is None:
            need = bwd_workspace_size(q, v, cu_seqlens, chunk_size)
            workspace = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
        ws_ptr, ws_bytes = _aligned_workspace(workspace, q.device)
        entry = lib.gla_chunk_bwd_saved if states_saved else lib.gla_chunk_bwd
        rc = entry(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(initial_state), _ptr(do),
                   _ptr(d_final_state), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(ds0),
                   _ptr(cu_seqlens), num_seqs, B, H, T, dk, dv, int(chunk_size), _dtype_code(q),
                   ws_ptr, ws_bytes, ctypes.c_void_p(stream))
    if rc != GLA_OK:
        raise GLAError(rc, last_error())
    return dq, dk_, dv_, dg, ds0


def gla_chunk_bwd_saved(q, k, v, g, do, chunk_states, initial_state=None, d_final_state=None,
                        cu_seqlens=None, chunk_size: int = 64, want_d_initial_state=None, out=None):
    """``gla_chunk_bwd`` through the C entry point ``gla_chunk_bwd_saved``: the chunk
    states come from ``chunk_states``, the workspace a ``gla_chunk_fwd_states`` call on
    the same inputs filled."""
    return gla_chunk_bwd(q, k, v, g, do, initial_state=initial_state, d_final_state=d_final_state,
                         cu_seqlens=cu_seqlens, chunk_size=chunk_size,
                         want_d_initial_state=want_d_initial_state, workspace=chunk_states, out=out,
                         states_saved=True)


def _saves_states(q, v, cu_seqlens):
    """Whether the autograd forward keeps the chunk states: when the planned forward
    runs unsplit on 64-column slices anyway, so that writing them costs the forward
    nothing but the stores (long sequences of few units keep the faster split and
    let the backward recompute them)."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if q.dtype != torch.bfloat16 or dk not in (64, 128) or dv % 64 != 0:
        return False
    if workspace_size(q, v, cu_seqlens) > 0:
        return False
    nseq = B if cu_seqlens is None else cu_seqlens.numel() - 1
    cus = torch.cuda.get_device_properties(q.device).multi_processor_count
    return slice_plan(nseq * H, dv, q.dtype, cus) == 64


class GLAFunction(torch.autograd.Function):
    """Autograd wrapper: forward ``gla_chunk_fwd``, backward ``gla_chunk_bwd``
    (bfloat16, d_k and d_v in {64, 128}).  ``apply(q, k, v, g, initial_state,
    cu_seqlens, save_states)`` returns ``(o, final_state)``.  ``save_states``
    (default None: decided by ``_saves_states``) keeps the forward's chunk states
    for the backward (``gla_chunk_fwd_states`` / ``gla_chunk_bwd_saved``) instead
    of recomputing them there."""

    @staticmethod
    def forward(ctx, q, k, v, g, initial_state=None, cu_seqlens=None, save_states=None):
        if save_states is None:
            save_states = _saves_states(q, v, cu_seqlens)
        hs = None
        if save_states:
            o, sf, hs = gla_chunk_fwd_states(q, k, v, g, initial_state=initial_state,
                                             output_final_state=True, cu_seqlens=cu_seqlens)
        else:
            o, sf = gla_chunk_fwd(q, k, v, g, initial_state=initial_state, output_final_state=True,
                                  cu_seqlens=cu_seqlens)
        ctx.save_for_backward(q, k, v, g, initial_state, cu_seqlens, hs)
        return o, sf

    @staticmethod
    def backward(ctx, do, dsf):
        q, k, v, g, s0, cu, hs = ctx.saved_tensors
        dq, dk, dv, dg, ds0 = gla_chunk_bwd(q, k, v, g, do.contiguous(), initial_state=s0,
                                            d_final_state=None if dsf is None else dsf.contiguous(),
                                            cu_seqlens=cu, workspace=hs, states_saved=hs is not None)
        return dq, dk, dv, dg, ds0, None, None


def gla_recurrent_step(q, k, v, g, state, out=None):
    """One decode step (C entry point ``gla_recurrent_step``): q, k, g [N, H, dk],
    v [N, H, dv], state [N, H, dk, dv] float32 updated in place.  Returns o [N, H, dv]."""
    N, H, dk = q.shape
    dv = v.shape[-1]
    _check_gpu("q", q)
    dt = q.dtype
    _check_gpu("k", k, dt, q.shape, device=q.device)
    _check_gpu("g", g, dt, q.shape, device=q.device)
    _check_gpu("v", v, dt, (N, H, dv), device=q.device)
    _check_gpu("state", state, torch.float32, (N, H, dk, dv), device=q.device)
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=q.device)
    else:
        _check_gpu("out", out, dt, (N, H, dv), device=q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.gla_recurrent_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(state), _ptr(out),
                                    N, H, dk, dv, _dtype_code(q), ctypes.c_void_p(stream))
    if rc != GLA_OK:
        raise GLAError(rc, last_error())
    return out


def gdn_chunk_fwd(q, k, v, g, beta, initial_state=None, output_final_state=False,
                  cu_seqlens=None, chunk_size: int = 64, out=None, final_state=None):
    """Chunkwise Gated DeltaNet forward (C entry point ``gdn_chunk_fwd``).

    q, k: [B, H, T, dk] and v: [B, H, T, dv] bfloat16; g (log forget gate) and
    beta (update gate): [B, H, T] float32; initial_state: [Nseq, H, dk, dv]
    float32 or None; cu_seqlens: int32 [Nseq+1] on the GPU for packed sequences
    (B == 1).  Returns ``(o, final_state)``; ``final_state`` is None unless
    ``output_final_state`` (or ``final_state`` is passed; it may alias
    ``initial_state``).
    """
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    _check_gpu("q", q)
    dt = q.dtype
    _check_gpu("k", k, dt, q.shape, device=q.device)
    _check_gpu("v", v, dt, (B, H, T, dv), device=q.device)
    _check_gpu("g", g, torch.float32, (B, H, T), device=q.device)
    _check_gpu("beta", beta, torch.float32, (B, H, T), device=q.device)
    nseq = B
    num_seqs = 0
    if cu_seqlens is not None:
        _check_gpu("cu_seqlens", cu_seqlens, torch.int32, device=q.device)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be 1-D with num_seqs + 1 >= 2 offsets")
        num_seqs = cu_seqlens.numel() - 1
        nseq = num_seqs
    if initial_state is not None:
        _check_gpu("initial_state", initial_state, torch.float32, (nseq, H, dk, dv),
                   device=q.device)
    if out is None:
        out = torch.empty((B, H, T, dv), dtype=dt, device=q.device)
    else:
        _check_gpu("out", out, dt, (B, H, T, dv), device=q.device)
    if final_state is None and output_final_state:
        final_state = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=q.device)
    elif final_state is not None:
        _check_gpu("final_state", final_state, torch.float32, (nseq, H, dk, dv), device=q.device)
    lib = load_library()
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
        rc = lib.gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(initial_state),
                               _ptr(out), _ptr(final_state), _ptr(cu_seqlens), num_seqs, B, H, T,
                               dk, dv, int(chunk_size), _dtype_code(q), ctypes.c_void_p(stream))
    if rc != GLA_OK:
        raise GLAError(rc, last_error())
    return out, final_state
