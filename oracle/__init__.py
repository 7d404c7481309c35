"""Plain, slow, fp64 CPU oracle for Gated Linear Attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call, link or run anything in
this directory.  The product path (the HIP library and its Python binding)
never touches it, and this package imports nothing from the product package.

What is computed, and where the pages define it:

* ``recurrence`` - the token-by-token recurrence of the page "Gated Linear
  Attention (GLA): Mathematical Foundations ...", section "The Gated Recurrent
  Update": S_t = diag(alpha_t) S_{t-1} + k_t^T v_t, o_t = q_t S_t, with
  alpha_t = exp(g_t).  Written in plain C (``gla_oracle.c``), fp64, one token
  at a time, OpenMP only across independent (sequence, head) units.
* ``recurrence_numpy`` - the same definition as a NumPy loop over tokens (for
  small cases); it exists so the C code is cross-checked by a second,
  independently written evaluation of the definition.
* ``decode_step`` - one token of the same recurrence per sequence (the O(1)
  decode step of the FlashLinearAttention page, section "The O(1) Inference
  Memory Revolution").

* ``oracle.backward`` - gradients of the same recurrence with respect to q, k,
  v, g and the initial state, for given upstream gradients of the outputs and
  of the final state: PyTorch fp64 autograd of the token loop (module
  docstring there; pinned in ``tests/test_oracle_backward.py``).

Parity: the C and NumPy evaluations are pinned in ``tests/test_oracle_pins.py``
against the pages' unrolled dual form (brute force), the alpha = 1 (linear
attention) and alpha = gamma (RetNet) closed forms, exact rational arithmetic,
the chunkwise equations of the same page, superposition in the initial state,
split-call composition and varlen/separate-call equality.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gla_oracle.c")
_LIB = os.path.join(_HERE, "libgla_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (plain -O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        fn = lib.gla_oracle_recurrence
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 7 + [ctypes.POINTER(ctypes.c_int)]
        _lib = lib
    return _lib


def _f32(x) -> np.ndarray:
    """Exact float32 copy of a bf16/fp32 tensor or array (no rounding happens:
    every bf16 and fp32 value is a float32 value)."""
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _i32(x) -> np.ndarray:
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x).astype(np.int32))


def _f64(x) -> np.ndarray:
    if x is None:
        return None
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def recurrence(q, k, v, g, s0=None, cu_seqlens=None, nthreads: int | None = None,
               want_final: bool = True, return_threads: bool = False):
    """fp64 recurrence over [B,H,T,d] inputs (packed varlen when ``cu_seqlens``
    is given: B == 1 and sequence n owns tokens cu[n]:cu[n+1]).

    Returns ``(o, s_final)`` as float64 arrays (``s_final`` is None when
    ``want_final`` is false), plus the OpenMP thread count if requested.
    """
    lib = _load()
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape and v.shape == (B, H, T, dv)
    cu = None
    nseq = B
    if cu_seqlens is not None:
        cu = _i32(cu_seqlens)
        nseq = cu.shape[0] - 1
    s0a = _f64(s0)
    if s0a is not None:
        assert s0a.shape == (nseq, H, dk, dv), s0a.shape
    o = np.empty((B, H, T, dv), dtype=np.float64)
    sf = np.empty((nseq, H, dk, dv), dtype=np.float64) if want_final else None
    used = ctypes.c_int(0)
    ptr = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    rc = lib.gla_oracle_recurrence(
        ptr(q), ptr(k), ptr(v), ptr(g), ptr(s0a), ptr(o), ptr(sf), ptr(cu),
        nseq if cu is not None else 0, B, H, T, dk, dv,
        int(nthreads or 0), ctypes.byref(used))
    if rc != 0:
        raise ValueError(f"gla_oracle_recurrence rejected its arguments (code {rc})")
    if return_threads:
        return o, sf, used.value
    return o, sf


def decode_step(q, k, v, g, state, nthreads: int | None = None):
    """One decode step per (sequence, head): q,k,g [N,H,dk], v [N,H,dv],
    state [N,H,dk,dv].  Returns (o [N,H,dv], new_state), both fp64."""
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
    o, sf = recurrence(q[:, :, None], k[:, :, None], v[:, :, None], g[:, :, None],
                       s0=state, nthreads=nthreads)
    return o[:, :, 0], sf


def recurrence_numpy(q, k, v, g, s0=None):
    """The same recurrence as a NumPy loop over tokens, vectorised only across
    the leading (unit) axes.  q,k,g: [..., T, dk]; v: [..., T, dv];
    s0: [..., dk, dv] or None.  Returns (o, s_final) in fp64."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    lead = q.shape[:-2]
    S = np.zeros(lead + (dk, dv)) if s0 is None else _f64(s0).copy()
    o = np.empty(lead + (T, dv))
    for t in range(T):
        alpha = np.exp(g[..., t, :])                                   # [..., dk]
        S = alpha[..., :, None] * S + k[..., t, :, None] * v[..., t, None, :]
        o[..., t, :] = np.einsum("...c,...cj->...j", q[..., t, :], S)
    return o, S
