"""fp64 CPU oracle for the GLA backward pass (gradients of the recurrence).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module; the
product path never does.  It shares no code with the HIP library.

What is computed.  The forward is the recurrence of the page "Gated Linear
Attention (GLA): Mathematical Foundations ...", section "The Gated Recurrent
Update": for every unit (sequence n, head h) and token t,

    S_t = diag(exp(g_t)) S_{t-1} + k_t^T v_t,      o_t = q_t S_t,

from the initial state S_0 (zeros when absent).  The same page's section
"I/O-Aware Kernel Design in FlashLinearAttention" describes the backward
kernel of the chunkwise training algorithm (it recomputes chunk states instead
of caching them).  Whatever its schedule, its exact result is the gradient of

    L = sum_t <dO_t, o_t> + <dS_T, S_T>

with respect to q, k, v, g and S_0, for a given upstream gradient dO of the
outputs and (optionally) dS_T of the final state.  This module writes the
recurrence out token by token with plain PyTorch fp64 CPU ops and lets
autograd differentiate it; nothing is chunked or reordered.  Inputs are the
exact values the device read (bf16 and fp32 values upcast exactly).

Pins (``tests/test_oracle_backward.py``): central finite differences on tiny
cases, a brute-force gradient of the page's unrolled (dual) form, the alpha = 1
linear-attention closed form, and the identity that the gate gradient is the
reverse cumulative sum of q*dq - k*dk plus the final-state term.
"""
from __future__ import annotations

from typing import Optional

import torch


def _f64(x):
    if x is None:
        return None
    return x.detach().to("cpu", torch.float64).clone()


def _recurrence_grads(q, k, v, g, do, s0, dsT):
    """q,k,g [U,T,dk], v,do [U,T,dv], s0/dsT [U,dk,dv] or None (fp64).
    Returns dq, dk, dv, dg, ds0 (ds0 is None when s0 is None)."""
    U, T, dk = q.shape
    dv = v.shape[-1]
    leaves = [q, k, v, g] + ([s0] if s0 is not None else [])
    for x in leaves:
        x.requires_grad_(True)
    S = s0 if s0 is not None else torch.zeros(U, dk, dv, dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(T):
        a = torch.exp(g[:, t])                                   # [U, dk]
        S = a[:, :, None] * S + k[:, t, :, None] * v[:, t, None, :]
        o_t = torch.einsum("uc,ucn->un", q[:, t], S)              # uses the updated S
        loss = loss + (o_t * do[:, t]).sum()
    if dsT is not None:
        loss = loss + (S * dsT).sum()
    grads = torch.autograd.grad(loss, leaves, allow_unused=True)
    out = [gr if gr is not None else torch.zeros_like(x) for gr, x in zip(grads, leaves)]
    if s0 is None:
        out.append(None)
    return tuple(out)


def backward(q, k, v, g, do, s0=None, dsT=None, cu_seqlens=None, units=None):
    """Gradients of the GLA recurrence, fp64.

    q, k, g: [B,H,T,dk]; v, do: [B,H,T,dv]; s0, dsT: [Nseq,H,dk,dv] or None.
    Packed variable length when ``cu_seqlens`` is given (B == 1, sequence n owns
    tokens cu[n]:cu[n+1]).  ``units`` optionally restricts the work to a list of
    (n, h) pairs; the other units' gradients are then left as NaN.

    Returns float64 tensors (dq, dk, dv, dg, ds0) in the input layouts; ds0 is
    None when s0 is None.
    """
    q, k, v, g, do = (_f64(x) for x in (q, k, v, g, do))
    s0, dsT = _f64(s0), _f64(dsT)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is None:
        spans = [(n, n, 0, T) for n in range(B)]          # (seq, batch row, start, end)
    else:
        cu = [int(c) for c in torch.as_tensor(cu_seqlens).tolist()]
        assert B == 1
        spans = [(n, 0, cu[n], cu[n + 1]) for n in range(len(cu) - 1)]
    nseq = len(spans)
    fill = float("nan") if units is not None else 0.0
    dq = torch.full_like(q, fill)
    dkk = torch.full_like(k, fill)
    dvv = torch.full_like(v, fill)
    dg = torch.full_like(g, fill)
    ds0 = torch.full((nseq, H, dk, dv), fill, dtype=torch.float64) if s0 is not None else None
    want = None if units is None else {(int(a), int(b)) for a, b in units}
    for n, b, lo, hi in spans:
        heads = [h for h in range(H) if want is None or (n, h) in want]
        if not heads:
            continue
        if s0 is not None and hi == lo:
            # An empty sequence passes its state through: S_T = S_0.
            ds0[n, heads] = dsT[n, heads] if dsT is not None else 0.0
        if hi == lo:
            continue
        sl = (b, heads, slice(lo, hi))
        r = _recurrence_grads(*(x[sl].clone() for x in (q, k, v, g, do)),
                              s0[n, heads].clone() if s0 is not None else None,
                              dsT[n, heads].clone() if dsT is not None else None)
        dq[sl], dkk[sl], dvv[sl], dg[sl] = r[0], r[1], r[2], r[3]
        if s0 is not None:
            ds0[n, heads] = r[4]
    return dq, dkk, dvv, dg, ds0
