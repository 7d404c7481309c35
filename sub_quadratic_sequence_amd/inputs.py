"""Seeded synthetic inputs for the GLA forward, backward and decode workloads,
and for the Gated DeltaNet (GDN) chunk forward.

This module only draws random numbers and casts them; it holds none of the
method's arithmetic, so both the HIP path's tests and the oracle can consume
its tensors.  Every draw happens on the CPU with ``torch.Generator`` in fp32,
in the fixed order (lengths), q, k, v, z, S0, and is then cast once to the
workload's dtype.  The device and the oracle read the same rounded values.

Gate recipes (g = log alpha, one value per key channel and token):
  * ``weak``   g = logsigmoid(z) / 16            (alpha close to 1)
  * ``strong`` g = logsigmoid(2 z - 1)            (tau = 1; alpha far from 1)
Edge-case tests may also ask for ``zero`` (g = 0, i.e. alpha = 1).

GDN (``gdn_inputs``): one forget gate g = log alpha and one update gate beta
per token and head ([B, H, T], fp32); q and k drawn N(0, 1) and scaled to unit
L2 norm per token before the cast, v ~ N(0, 1), beta = sigmoid(N(0, 1)).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch
import torch.nn.functional as F


@dataclasses.dataclass(frozen=True)
class ChunkWorkload:
    name: str
    B: int
    H: int
    T: int            # per-sequence length (fixed) or total tokens (varlen)
    dk: int
    dv: int
    dtype: str        # "bf16" or "f32": dtype of q, k, v, g and o
    seed: int
    gate: str = "weak"
    k_scaled: bool = False     # k *= dk ** -0.5
    s0: bool = False           # initial state ~ 0.1 * N(0, 1), fp32
    varlen: int = 0            # number of packed sequences (0 = fixed length)
    len_lo: int = 64
    len_hi: int = 4096
    chunk: int = 64

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    steps: int
    seed: int
    dtype: str = "bf16"
    gate: str = "weak"


# The workloads the forward pass and the decode step are specified on.
TINY_FP32 = ChunkWorkload("gla_fwd_tiny_b1h2t256d64_f32", B=1, H=2, T=256, dk=64, dv=64,
                          dtype="f32", seed=1, k_scaled=True)
TRAIN_BF16 = ChunkWorkload("gla_fwd_b8h16t2048d128_bf16", B=8, H=16, T=2048, dk=128, dv=128,
                           dtype="bf16", seed=2, k_scaled=True)
LONG_BF16 = ChunkWorkload("gla_fwd_long_b1h16t65536d128_bf16", B=1, H=16, T=65536, dk=128,
                          dv=128, dtype="bf16", seed=3, s0=True)
VARLEN_BF16 = ChunkWorkload("gla_fwd_varlen16_h16dk128dv256_strong_bf16", B=1, H=16, T=0,
                            dk=128, dv=256, dtype="bf16", seed=4, gate="strong", varlen=16)
DECODE_BF16 = DecodeWorkload("gla_decode_n256h16d128_x64", N=256, H=16, dk=128, dv=128,
                             steps=64, seed=5)

# The backward pass on the training shape (same q, k, v, g; upstream gradients
# from ``upstream_grads``).
TRAIN_BWD_BF16 = dataclasses.replace(TRAIN_BF16, name="gla_bwd_b8h16t2048d128_bf16")

# Gated DeltaNet chunk forward at the training shape (per-token scalar gates).
GDN_TRAIN_BF16 = ChunkWorkload("gdn_fwd_b8h16t2048d128_bf16", B=8, H=16, T=2048, dk=128, dv=128,
                               dtype="bf16", seed=6)

WORKLOADS = {w.name: w for w in (TINY_FP32, TRAIN_BF16, LONG_BF16, VARLEN_BF16, DECODE_BF16,
                                 TRAIN_BWD_BF16, GDN_TRAIN_BF16)}


def _gate(z: torch.Tensor, kind: str) -> torch.Tensor:
    if kind == "weak":
        return F.logsigmoid(z) / 16.0
    if kind == "strong":
        return F.logsigmoid(2.0 * z - 1.0)
    if kind == "zero":
        return torch.zeros_like(z)
    raise ValueError(f"unknown gate recipe {kind!r}")


def chunk_inputs(w: ChunkWorkload, *, T: Optional[int] = None, B: Optional[int] = None,
                 H: Optional[int] = None, seed: Optional[int] = None,
                 lengths: Optional[list] = None, gate: Optional[str] = None,
                 s0: Optional[bool] = None):
    """Draw one batch for a forward workload (overrides shrink it for tests).

    Returns a dict of CPU tensors: q, k, g [B,H,T,dk] and v [B,H,T,dv] in the
    workload dtype; ``s0`` [Nseq,H,dk,dv] fp32 or None; ``cu_seqlens`` int32
    [Nseq+1] or None (varlen: B == 1 and T is the packed total).
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    gate = w.gate if gate is None else gate
    want_s0 = w.s0 if s0 is None else s0
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    cu = None
    if w.varlen or lengths is not None:
        if lengths is None:
            lengths = torch.randint(w.len_lo, w.len_hi + 1, (w.varlen,), generator=gen).tolist()
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        B, T, nseq = 1, int(cu[-1]), len(lengths)
    else:
        T = w.T if T is None else T
        nseq = B
    q = torch.randn(B, H, T, w.dk, generator=gen)
    k = torch.randn(B, H, T, w.dk, generator=gen)
    v = torch.randn(B, H, T, w.dv, generator=gen)
    z = torch.randn(B, H, T, w.dk, generator=gen)
    s0_t = torch.randn(nseq, H, w.dk, w.dv, generator=gen) * 0.1 if want_s0 else None
    if w.k_scaled:
        k = k * (w.dk ** -0.5)
    g = _gate(z, gate)
    dt = w.torch_dtype
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), g=g.to(dt), s0=s0_t, cu_seqlens=cu,
                B=B, H=H, T=T, nseq=nseq)


def gdn_inputs(w: ChunkWorkload, *, T: Optional[int] = None, B: Optional[int] = None,
               H: Optional[int] = None, seed: Optional[int] = None,
               lengths: Optional[list] = None, gate: Optional[str] = None,
               s0: Optional[bool] = None, dk: Optional[int] = None, dv: Optional[int] = None):
    """Draw one batch for a GDN forward workload.

    Returns a dict of CPU tensors: q, k [B,H,T,dk] (unit L2 norm per token
    before the cast) and v [B,H,T,dv] in the workload dtype; g (log of the
    forget gate) and beta [B,H,T] fp32; ``s0`` [Nseq,H,dk,dv] fp32 or None;
    ``cu_seqlens`` int32 [Nseq+1] or None (varlen: B == 1, T = packed total).
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    dk = w.dk if dk is None else dk
    dv = w.dv if dv is None else dv
    gate = w.gate if gate is None else gate
    want_s0 = w.s0 if s0 is None else s0
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    cu = None
    if w.varlen or lengths is not None:
        if lengths is None:
            lengths = torch.randint(w.len_lo, w.len_hi + 1, (w.varlen,), generator=gen).tolist()
        cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
        cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
        B, T, nseq = 1, int(cu[-1]), len(lengths)
    else:
        T = w.T if T is None else T
        nseq = B
    q = torch.randn(B, H, T, dk, generator=gen)
    k = torch.randn(B, H, T, dk, generator=gen)
    v = torch.randn(B, H, T, dv, generator=gen)
    z = torch.randn(B, H, T, generator=gen)
    zb = torch.randn(B, H, T, generator=gen)
    s0_t = torch.randn(nseq, H, dk, dv, generator=gen) * 0.1 if want_s0 else None
    q = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    g = _gate(z, gate)
    beta = torch.sigmoid(zb)
    dt = w.torch_dtype
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), g=g.float(), beta=beta.float(), s0=s0_t,
                cu_seqlens=cu, B=B, H=H, T=T, nseq=nseq)


def decode_inputs(w: DecodeWorkload, *, N: Optional[int] = None, H: Optional[int] = None,
                  steps: Optional[int] = None, seed: Optional[int] = None,
                  dk: Optional[int] = None, dv: Optional[int] = None):
    """Draw a run of single-token decode steps: q, k, g [steps,N,H,dk] and
    v [steps,N,H,dv] in the workload dtype, initial state [N,H,dk,dv] fp32
    ~ 0.1 * N(0, 1)."""
    N = w.N if N is None else N
    H = w.H if H is None else H
    steps = w.steps if steps is None else steps
    dk = w.dk if dk is None else dk
    dv = w.dv if dv is None else dv
    gen = torch.Generator().manual_seed(w.seed if seed is None else seed)
    q = torch.randn(steps, N, H, dk, generator=gen)
    k = torch.randn(steps, N, H, dk, generator=gen)
    v = torch.randn(steps, N, H, dv, generator=gen)
    z = torch.randn(steps, N, H, dk, generator=gen)
    s0 = torch.randn(N, H, dk, dv, generator=gen) * 0.1
    g = _gate(z, w.gate)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), g=g.to(dt), s0=s0)


def upstream_grads(w: ChunkWorkload, d: dict, *, seed: Optional[int] = None,
                   final: bool = True):
    """Draw the upstream gradients of a backward call for the batch ``d`` of
    ``chunk_inputs``: dO [B,H,T,dv] ~ N(0, 1) in the workload dtype and, when
    ``final``, dS_T [Nseq,H,dk,dv] ~ 0.1 * N(0, 1) fp32.  A generator of its own
    (seed + 1000) leaves the forward draws untouched."""
    gen = torch.Generator().manual_seed((w.seed if seed is None else seed) + 1000)
    do = torch.randn(d["B"], d["H"], d["T"], w.dv, generator=gen)
    dsT = torch.randn(d["nseq"], d["H"], w.dk, w.dv, generator=gen) * 0.1 if final else None
    return dict(do=do.to(w.torch_dtype), dsT=dsT)


def expected_varlen_tokens(w: ChunkWorkload) -> float:
    return w.varlen * (w.len_lo + w.len_hi) / 2.0


__all__ = ["ChunkWorkload", "DecodeWorkload", "WORKLOADS", "TINY_FP32", "TRAIN_BF16",
           "LONG_BF16", "VARLEN_BF16", "DECODE_BF16", "TRAIN_BWD_BF16", "GDN_TRAIN_BF16",
           "chunk_inputs", "gdn_inputs",
           "decode_inputs", "upstream_grads", "expected_varlen_tokens"]
