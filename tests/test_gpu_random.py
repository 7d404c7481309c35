"""Seeded randomized GPU parity sweep over the configurations the entry points
accept: the GLA forward (both dtypes; fixed-length, packed and long sequences,
which take the sequence split), the backward, the decode step and the Gated
DeltaNet forward, each against its fp64 oracle on the same seeded inputs.

Every case is drawn from its own generator (numpy, seed [BASE, kind, index]),
so a failing case can be rerun alone by its test id; each prints its full
configuration before touching the GPU.  GLA_RANDOM_SCALE=k in the environment runs
k times as many cases.  Tolerances and the per-unit metric are
those of the hand-written parity tests (parity.py)."""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as OB
from oracle import gdn as ogdn
from parity import TOL_BF16, TOL_F32, to64, unit_err_fixed, unit_err_varlen
from sub_quadratic_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)
BASE = 20261202
# GLA_RANDOM_SCALE=k runs k times as many cases (a deeper sweep; the first cases are the same)
SCALE = max(1, int(os.environ.get("GLA_RANDOM_SCALE", "1")))
N_FWD, N_BWD, N_DEC, N_GDN = 48 * SCALE, 16 * SCALE, 16 * SCALE, 16 * SCALE


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_sequence_amd import gla

    gla.load_library()
    return torch.device("cuda:0")


def _rng(kind, i):
    return np.random.default_rng([BASE, kind, i])


def _lengths(r, nseq, hi):
    lengths = [int(x) for x in r.integers(0, hi + 1, nseq)]
    if sum(lengths) == 0:
        lengths[0] = 1
    return lengths


def _say(kind, i, c):
    print(f"\n[case] {kind} #{i}: " + " ".join(f"{k}={v}" for k, v in c.items()), flush=True)


def _to(dev, x):
    return None if x is None else x.to(dev)


# ------------------------------------------------------------------ GLA forward
def fwd_case(i):
    r = _rng(1, i)
    c = {"dtype": "f32" if r.random() < 0.3 else "bf16",
         "dk": int(r.choice([64, 128])), "dv": int(r.choice([64, 128, 192, 256])),
         "gate": str(r.choice(["weak", "weak", "strong", "zero"])),
         "s0": bool(r.random() < 0.5), "final": bool(r.random() < 0.7),
         "layout": str(r.choice(["fixed", "fixed", "varlen", "long"]))}
    if c["layout"] == "fixed":
        c.update(B=int(r.integers(1, 4)), H=int(r.integers(1, 5)), T=int(r.integers(1, 401)), lengths=None)
    elif c["layout"] == "varlen":
        c.update(B=1, H=int(r.integers(1, 4)), T=0, lengths=_lengths(r, int(r.integers(1, 7)), 300))
    else:   # few units, long sequences: the call goes through the sequence split when it pays
        c.update(B=1, H=int(r.integers(1, 3)), T=int(r.integers(1000, 2601)), lengths=None)
    # a caller-chosen d_v slice width (gla_chunk_fwd_sliced) on some bf16 calls
    c["dv_slice"] = None
    if c["dtype"] == "bf16" and c["dv"] % 128 == 0 and c["layout"] != "long":
        c["dv_slice"] = [0, 64, 128, 128][int(r.integers(0, 4))]
    return c


@pytest.mark.parametrize("i", range(N_FWD))
def test_random_forward(dev, i):
    from sub_quadratic_sequence_amd import gla

    c = fwd_case(i)
    _say("gla_chunk_fwd", i, c)
    w = I.ChunkWorkload("random_fwd", B=c["B"], H=c["H"], T=c["T"], dk=c["dk"], dv=c["dv"],
                        dtype=c["dtype"], seed=1000 + i, gate=c["gate"], s0=c["s0"])
    d = I.chunk_inputs(w, lengths=c["lengths"])
    cu = d["cu_seqlens"]
    o, sf = gla.gla_chunk_fwd(*(d[n].to(dev) for n in "qkvg"), initial_state=_to(dev, d["s0"]),
                              output_final_state=c["final"], cu_seqlens=_to(dev, cu),
                              dv_slice=c["dv_slice"])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], s0=d["s0"], cu_seqlens=cu,
                                     nthreads=NTHREADS)
    tol = TOL_BF16 if c["dtype"] == "bf16" else TOL_F32
    e_o = unit_err_fixed(o, o_ref) if cu is None else unit_err_varlen(o, o_ref, cu)
    e_s = unit_err_fixed(sf, s_ref) if c["final"] else 0.0
    print(f"forward #{i}: O err {e_o:.3e}  S err {e_s:.3e}  (tol {tol})", flush=True)
    assert np.all(np.isfinite(to64(o)))
    assert (sf is None) == (not c["final"])
    assert e_o <= tol and e_s <= tol, (e_o, e_s)


# ------------------------------------------------------------------ GLA backward
def bwd_case(i):
    r = _rng(2, i)
    c = {"dk": int(r.choice([64, 128])), "dv": int(r.choice([64, 128, 192, 256])),
         "gate": str(r.choice(["weak", "strong"])), "s0": bool(r.random() < 0.5),
         "final": bool(r.random() < 0.5), "layout": str(r.choice(["fixed", "varlen", "long"]))}
    if c["layout"] == "fixed":
        c.update(B=int(r.integers(1, 3)), H=int(r.integers(1, 4)), T=int(r.integers(1, 301)), lengths=None)
    elif c["layout"] == "varlen":
        c.update(B=1, H=int(r.integers(1, 3)), T=0, lengths=_lengths(r, int(r.integers(1, 5)), 200))
    else:   # one unit of 15-25 chunks: the backward splits it into segments
        c.update(B=1, H=1, T=int(r.integers(900, 1601)), lengths=None)
    return c


@pytest.mark.parametrize("i", range(N_BWD))
def test_random_backward(dev, i):
    from sub_quadratic_sequence_amd import gla

    c = bwd_case(i)
    _say("gla_chunk_bwd", i, c)
    w = I.ChunkWorkload("random_bwd", B=c["B"], H=c["H"], T=c["T"], dk=c["dk"], dv=c["dv"],
                        dtype="bf16", seed=2000 + i, gate=c["gate"], s0=c["s0"], k_scaled=True)
    d = I.chunk_inputs(w, lengths=c["lengths"])
    d.update(I.upstream_grads(w, d, final=c["final"]))
    cu = d["cu_seqlens"]
    got = gla.gla_chunk_bwd(*(d[n].to(dev) for n in ("q", "k", "v", "g", "do")),
                            initial_state=_to(dev, d["s0"]), d_final_state=_to(dev, d["dsT"]),
                            cu_seqlens=_to(dev, cu))
    torch.cuda.synchronize()
    ref = OB.backward(d["q"], d["k"], d["v"], d["g"], d["do"], d["s0"], d["dsT"], cu_seqlens=cu)
    errs = {}
    for name, x, r_ in zip(("dq", "dk", "dv", "dg"), got[:4], ref[:4]):
        assert np.all(np.isfinite(to64(x))), name
        errs[name] = unit_err_fixed(x, r_) if cu is None else unit_err_varlen(x, r_, cu)
    if d["s0"] is not None:
        errs["ds0"] = unit_err_fixed(got[4], ref[4])
    else:
        assert got[4] is None
    print(f"backward #{i}: " + "  ".join(f"{k} {v:.3e}" for k, v in errs.items()) + f"  (tol {TOL_BF16})",
          flush=True)
    for k, v in errs.items():
        assert v <= TOL_BF16, (k, v)


# ------------------------------------------------------------------ decode step
def dec_case(i):
    r = _rng(3, i)
    return {"dtype": "f32" if r.random() < 0.4 else "bf16", "dk": int(r.choice([64, 128, 256])),
            "dv": int(r.choice([64, 128, 256])), "N": int(r.integers(1, 6)), "H": int(r.integers(1, 4)),
            "steps": int(r.integers(1, 5)), "gate": str(r.choice(["weak", "strong"]))}


@pytest.mark.parametrize("i", range(N_DEC))
def test_random_decode(dev, i):
    from sub_quadratic_sequence_amd import gla

    c = dec_case(i)
    _say("gla_recurrent_step", i, c)
    w = I.DecodeWorkload("random_decode", N=c["N"], H=c["H"], dk=c["dk"], dv=c["dv"], steps=c["steps"],
                         seed=3000 + i, dtype=c["dtype"], gate=c["gate"])
    d = I.decode_inputs(w)
    st = d["s0"].to(dev).clone()
    outs = []
    for t in range(c["steps"]):
        outs.append(gla.gla_recurrent_step(*(d[n][t].to(dev) for n in "qkvg"), st).double().cpu())
    torch.cuda.synchronize()
    q, k, v, g = (d[n].permute(1, 2, 0, 3).contiguous() for n in "qkvg")   # [N, H, steps, d]
    o_ref, s_ref = oracle.recurrence(q, k, v, g, s0=d["s0"], nthreads=NTHREADS)
    tol = TOL_BF16 if c["dtype"] == "bf16" else TOL_F32
    e_o, e_s = unit_err_fixed(torch.stack(outs, 2), o_ref), unit_err_fixed(st, s_ref)
    print(f"decode #{i}: O err {e_o:.3e}  S err {e_s:.3e}  (tol {tol})", flush=True)
    assert e_o <= tol and e_s <= tol, (e_o, e_s)


# ------------------------------------------------------------------ Gated DeltaNet
def gdn_case(i):
    r = _rng(4, i)
    c = {"dk": int(r.choice([64, 128])), "dv": int(r.choice([64, 128, 192])),
         "gate": str(r.choice(["weak", "strong", "zero"])), "s0": bool(r.random() < 0.5),
         "final": bool(r.random() < 0.7), "layout": str(r.choice(["fixed", "fixed", "varlen"]))}
    if c["layout"] == "fixed":
        c.update(B=int(r.integers(1, 3)), H=int(r.integers(1, 4)), T=int(r.integers(1, 301)), lengths=None)
    else:
        c.update(B=1, H=int(r.integers(1, 3)), T=0, lengths=_lengths(r, int(r.integers(1, 5)), 250))
    return c


@pytest.mark.parametrize("i", range(N_GDN))
def test_random_gdn(dev, i):
    from sub_quadratic_sequence_amd import gla

    c = gdn_case(i)
    _say("gdn_chunk_fwd", i, c)
    d = I.gdn_inputs(I.GDN_TRAIN_BF16, B=c["B"], H=c["H"], T=c["T"], dk=c["dk"], dv=c["dv"],
                     gate=c["gate"], s0=c["s0"], lengths=c["lengths"], seed=4000 + i)
    cu = d["cu_seqlens"]
    o, sf = gla.gdn_chunk_fwd(*(d[n].to(dev) for n in ("q", "k", "v", "g", "beta")),
                              initial_state=_to(dev, d["s0"]), output_final_state=c["final"],
                              cu_seqlens=_to(dev, cu))
    torch.cuda.synchronize()
    o_ref, s_ref = ogdn.recurrence(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=d["s0"],
                                   cu_seqlens=cu, nthreads=NTHREADS)
    e_o = unit_err_fixed(o, o_ref) if cu is None else unit_err_varlen(o, o_ref, cu)
    e_s = unit_err_fixed(sf, s_ref) if c["final"] else 0.0
    print(f"gdn #{i}: O err {e_o:.3e}  S err {e_s:.3e}  (tol {TOL_BF16})", flush=True)
    assert np.all(np.isfinite(to64(o)))
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16, (e_o, e_s)
