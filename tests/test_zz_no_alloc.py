"""gla_chunk_fwd_noalloc, the forward entry point that allocates nothing (its
sequence-split scratch lives in the library's own device array), called through
the C ABI and compared with gla_chunk_fwd_ws on the same inputs: the same plan
and kernels, so outputs and final states must agree bit for bit.  Two calls in a
row, the second on a smaller input, so the second reuses the array the first
left behind; the first is also checked against the fp64 oracle."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
from parity import TOL_BF16, unit_err_fixed
from sub_quadratic_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_sequence_amd import gla

    return gla.load_library()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(lib, entry, d, s0, dev):
    """One forward through the named C entry point; outputs preallocated here."""
    q, k, v, g = (d[n].to(dev) for n in "qkvg")
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    o = torch.full((B, H, T, dv), float("nan"), dtype=torch.bfloat16, device=dev)
    sT = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device=dev)
    s0d = None if s0 is None else s0.to(dev)
    args = [_p(q), _p(k), _p(v), _p(g), _p(s0d), _p(o), _p(sT), None, 0, B, H, T, dk, dv, 64, 0]
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    if entry == "ws":
        need = lib.gla_chunk_fwd_workspace_size(0, B, H, T, dk, dv, 64, 0)
        assert need > 0, "the shape must take the sequence split"
        ws = torch.empty(need, dtype=torch.uint8, device=dev)   # torch aligns to 256 bytes
        assert ws.data_ptr() % 256 == 0
        rc = lib.gla_chunk_fwd_ws(*args, _p(ws), need, stream)
    else:
        assert need_fits(lib, B, H, T, dk, dv)
        rc = lib.gla_chunk_fwd_noalloc(*args, stream)
    assert rc == 0, lib.gla_last_error().decode()
    torch.cuda.synchronize()
    return o.cpu(), sT.cpu()


def need_fits(lib, B, H, T, dk, dv):
    return 0 < lib.gla_chunk_fwd_workspace_size(0, B, H, T, dk, dv, 64, 0) <= 32 << 20


def test_noalloc_matches_the_workspace_entry_point_twice(lib):
    dev = torch.device("cuda:0")
    cases = [
        # (H, T): split into segments (8 and 4 units of 128 columns on 256 compute
        # units); ragged last chunk; the second input is smaller
        (8, 8229, True),
        (4, 3000, False),
    ]
    for i, (H, T, check_oracle) in enumerate(cases):
        print(f"\n[case] noalloc call {i}: B1 H{H} T{T} d128 bf16 with initial state", flush=True)
        d = I.chunk_inputs(I.LONG_BF16, B=1, H=H, T=T, seed=100 + i)
        s0 = d["s0"]
        o_n, s_n = _call(lib, "noalloc", d, s0, dev)
        o_w, s_w = _call(lib, "ws", d, s0, dev)
        assert torch.isfinite(o_n.float()).all() and torch.isfinite(s_n).all()
        assert torch.equal(o_n, o_w), (o_n.float() - o_w.float()).abs().max()
        assert torch.equal(s_n, s_w), (s_n - s_w).abs().max()
        if check_oracle:
            o_ref, s_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], s0=s0, nthreads=NTHREADS)
            e_o, e_s = unit_err_fixed(o_n, o_ref), unit_err_fixed(s_n, s_ref)
            print(f"noalloc vs oracle: O err {e_o:.3e}  S err {e_s:.3e}", flush=True)
            assert e_o <= TOL_BF16 and e_s <= TOL_BF16
