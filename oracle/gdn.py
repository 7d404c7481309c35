"""Plain, slow, fp64 CPU oracle for the Gated DeltaNet (GDN) recurrence.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it.

What is computed (page "Qwen Team Releases FlashQLA for High-Performance Linear
Attention": GDN's update gate beta and forget gate alpha, the transition
I - beta k k^T, one gate value per token, L2-normalised keys):

    S_t = alpha_t (I - beta_t k_t^T k_t) S_{t-1} + beta_t k_t^T v_t
    o_t = q_t S_t                      (the updated state), alpha_t = exp(g_t)

for every independent unit (sequence, head), one token at a time.

* ``recurrence`` - the C implementation (``gdn_oracle_recurrence`` in
  ``gla_oracle.c``), fp64, OpenMP across units, packed sequences by offsets.
* ``recurrence_numpy`` - the same definition as a NumPy loop (small cases), a
  second, independently written evaluation the C code is checked against.
* ``decode_step`` - one token of the same recurrence per sequence.

Parity unpinned against the pages for the update form: the page prints no
update equation and no values, so the form above is the plainest reading of
what it names, and no pin ties it to the page itself.  The pins check that
this code computes that reading.

Pins (``tests/test_oracle_gdn.py``): beta = 0 closed form, the exact-retrieval
identity (q_t = k_t, beta_t = 1/|k_t|^2 gives o_t = v_t), an orthonormal-key
overwrite closed form, the brute-force unrolled product of explicit transition
matrices, the chunkwise WY form at several chunk sizes, packed = separate
calls, and planted mistakes that the pins must reject.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _f32, _f64, _i32, _load


def _lib():
    lib = _load()
    fn = lib.gdn_oracle_recurrence
    if fn.restype is not ctypes.c_int:
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] * 7 + [ctypes.POINTER(ctypes.c_int)]
    return lib


def recurrence(q, k, v, g, beta, s0=None, cu_seqlens=None, nthreads: int | None = None,
               want_final: bool = True, return_threads: bool = False):
    """fp64 GDN recurrence.  q, k: [B,H,T,dk]; v: [B,H,T,dv]; g, beta: [B,H,T];
    s0: [Nseq,H,dk,dv] or None; packed sequences when ``cu_seqlens`` is given
    (B == 1).  Returns ``(o, s_final)`` in fp64."""
    lib = _lib()
    q, k, v, g, beta = _f32(q), _f32(k), _f32(v), _f32(g), _f32(beta)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape == (B, H, T, dv)
    assert g.shape == (B, H, T) and beta.shape == (B, H, T), (g.shape, beta.shape)
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
    rc = lib.gdn_oracle_recurrence(
        ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta), ptr(s0a), ptr(o), ptr(sf), ptr(cu),
        nseq if cu is not None else 0, B, H, T, dk, dv, int(nthreads or 0), ctypes.byref(used))
    if rc != 0:
        raise ValueError(f"gdn_oracle_recurrence rejected its arguments (code {rc})")
    if return_threads:
        return o, sf, used.value
    return o, sf


def decode_step(q, k, v, g, beta, state, nthreads: int | None = None):
    """One GDN token per (sequence, head): q, k [N,H,dk]; v [N,H,dv]; g, beta
    [N,H]; state [N,H,dk,dv].  Returns (o [N,H,dv], new_state) in fp64."""
    q, k, v, g, beta = _f32(q), _f32(k), _f32(v), _f32(g), _f32(beta)
    o, sf = recurrence(q[:, :, None], k[:, :, None], v[:, :, None], g[:, :, None],
                       beta[:, :, None], s0=state, nthreads=nthreads)
    return o[:, :, 0], sf


def recurrence_numpy(q, k, v, g, beta, s0=None):
    """The same recurrence as a NumPy loop over tokens, vectorised across the
    leading (unit) axes.  q, k: [..., T, dk]; v: [..., T, dv]; g, beta: [..., T];
    s0: [..., dk, dv] or None.  Returns (o, s_final) in fp64."""
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    T, dk = q.shape[-2:]
    dv = v.shape[-1]
    lead = q.shape[:-2]
    S = np.zeros(lead + (dk, dv)) if s0 is None else _f64(s0).copy()
    o = np.empty(lead + (T, dv))
    for t in range(T):
        a = np.exp(g[..., t])[..., None, None]
        b = beta[..., t][..., None, None]
        kt = k[..., t, :]
        erase = kt[..., :, None] * np.einsum("...c,...cj->...j", kt, S)[..., None, :]
        write = kt[..., :, None] * v[..., t, None, :]
        S = a * (S - b * erase) + b * write
        o[..., t, :] = np.einsum("...c,...cj->...j", q[..., t, :], S)
    return o, S
