"""GPU parity of the backward pass (``gla_chunk_bwd`` through the C ABI) against
the fp64 autograd oracle on the same seeded inputs.  Tolerance: per unit,
max |X_gpu - X_ref| / max |X_ref| <= 2e-2 for every gradient (bf16 path).
Every test prints the case it is about to run before touching the GPU."""
import os

import numpy as np
import pytest
import torch

from oracle import backward as OB
from parity import TOL_BF16, to64, unit_err_fixed, unit_err_varlen
from sub_quadratic_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_sequence_amd import gla

    gla.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def _case(B, H, T, dk, dv, gate="weak", s0=True, final=True, seed=11, lengths=None, k_scaled=True):
    w = I.ChunkWorkload("bwd_test", B=B, H=H, T=T, dk=dk, dv=dv, dtype="bf16", seed=seed, gate=gate,
                        k_scaled=k_scaled, s0=s0)
    d = I.chunk_inputs(w, lengths=lengths)
    d.update(I.upstream_grads(w, d, final=final))
    return d


def _gpu_bwd(dev, d):
    from sub_quadratic_sequence_amd import gla

    to = lambda x: None if x is None else x.to(dev)
    out = gla.gla_chunk_bwd(*(to(d[n]) for n in ("q", "k", "v", "g", "do")), initial_state=to(d["s0"]),
                            d_final_state=to(d["dsT"]), cu_seqlens=to(d["cu_seqlens"]))
    torch.cuda.synchronize()
    return out


def _check(d, got, label, units=None):
    ref = OB.backward(d["q"], d["k"], d["v"], d["g"], d["do"], d["s0"], d["dsT"],
                      cu_seqlens=d["cu_seqlens"], units=units)
    names = ("dq", "dk", "dv", "dg")
    errs = {}
    for name, x, r in zip(names, got[:4], ref[:4]):
        x64 = to64(x)
        assert np.all(np.isfinite(x64)), name
        if units is not None:
            errs[name] = max(_unit_err_one(x64, to64(r), n, h, d) for n, h in units)
        elif d["cu_seqlens"] is not None:
            errs[name] = unit_err_varlen(x64, r, d["cu_seqlens"])
        else:
            errs[name] = unit_err_fixed(x64, r)
    if d["s0"] is not None:
        x64, r64 = to64(got[4]), to64(ref[4])
        if units is not None:
            errs["ds0"] = max(float(np.abs(x64[n, h] - r64[n, h]).max() / np.abs(r64[n, h]).max())
                              for n, h in units)
        else:
            errs["ds0"] = unit_err_fixed(x64, r64)
    print(label + ": " + "  ".join(f"{k} {v:.3e}" for k, v in errs.items()) + f"  (tol {TOL_BF16})",
          flush=True)
    for k, v in errs.items():
        assert v <= TOL_BF16, (k, v)


def _unit_err_one(x, r, n, h, d):
    if d["cu_seqlens"] is None:
        a, b = x[n, h], r[n, h]
    else:
        cu = [int(c) for c in d["cu_seqlens"]]
        a, b = x[0, h, cu[n]:cu[n + 1]], r[0, h, cu[n]:cu[n + 1]]
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


@pytest.mark.parametrize("B,H,T,dk,dv,gate", [
    (1, 2, 100, 64, 64, "weak"),       # two chunks, ragged tail
    (2, 2, 300, 128, 128, "weak"),     # several chunks, ragged tail
    (1, 2, 256, 128, 128, "strong"),   # strong gates: every sub-chunk uses its own pivot range
    (1, 2, 130, 128, 64, "weak"),
    (1, 2, 130, 64, 128, "strong"),
    (1, 1, 1, 128, 128, "weak"),       # one token
    (1, 2, 128, 64, 64, "zero"),       # alpha = 1
    (1, 2, 200, 128, 256, "weak"),     # d_v 256: two 128-column slices, dq/dk/dg summed
    (2, 1, 150, 64, 192, "strong"),    # d_v 192: a 128- and a 64-column slice
])
def test_bwd_matches_oracle(dev, B, H, T, dk, dv, gate):
    say(f"gla_chunk_bwd B={B} H={H} T={T} dk={dk} dv={dv} gate={gate} s0 dsT")
    d = _case(B, H, T, dk, dv, gate=gate)
    _check(d, _gpu_bwd(dev, d), f"bwd B{B} H{H} T{T} dk{dk} dv{dv} {gate}")


@pytest.mark.parametrize("B,H,T,dk,dv,gate", [
    (1, 2, 1000, 128, 128, "weak"),    # 2 segments of 8 chunks, ragged tail
    (1, 1, 3000, 128, 128, "strong"),  # 5 segments
    (2, 2, 2050, 64, 64, "weak"),      # 4 segments, the last one a single token
    (1, 2, 1100, 128, 64, "strong"),
    (1, 1, 1500, 128, 256, "weak"),    # split and column slices together
])
def test_bwd_sequence_split(dev, B, H, T, dk, dv, gate):
    from sub_quadratic_sequence_amd import gla

    say(f"gla_chunk_bwd sequence split B={B} H={H} T={T} dk={dk} dv={dv} gate={gate} s0 dsT")
    d = _case(B, H, T, dk, dv, gate=gate)
    # the split is in use: its state-gradient workspace is part of the size
    nch = (T + 63) // 64
    unsplit = (H * (B + B * T // 64 + 1) * dk * dv * 2 + 255) // 256 * 256
    assert gla.bwd_workspace_size(d["q"].to(dev), d["v"].to(dev)) > unsplit, nch
    _check(d, _gpu_bwd(dev, d), f"bwd split B{B} H{H} T{T} dk{dk} dv{dv} {gate}")


def test_bwd_without_initial_or_final_state(dev):
    say("gla_chunk_bwd B=2 H=2 T=200 d128 no s0, no dsT")
    d = _case(2, 2, 200, 128, 128, s0=False, final=False)
    got = _gpu_bwd(dev, d)
    assert got[4] is None
    _check(d, got, "bwd no states")


@pytest.mark.parametrize("gate,dv,lengths", [
    ("weak", 128, [1, 0, 65, 200, 17, 64]),
    ("strong", 128, [1, 0, 65, 200, 17, 64]),
    ("strong", 256, [1, 0, 65, 200, 17, 64]),
    ("weak", 128, [0, 300, 65, 129]),        # 8 units: the state pass takes the longest first
])
def test_bwd_varlen_with_empty_and_short(dev, gate, dv, lengths):
    say(f"gla_chunk_bwd varlen lengths={lengths} H=2 dk128 dv{dv} gate={gate}")
    d = _case(1, 2, 0, 128, dv, gate=gate, lengths=lengths)
    got = _gpu_bwd(dev, d)
    _check(d, got, f"bwd varlen dv{dv} {gate}")
    # an empty sequence passes its state through: dS0 = dS_T
    for i, n in enumerate(lengths):
        if n == 0:
            assert torch.equal(got[4][i].cpu(), d["dsT"][i])


def test_bwd_training_shape_sampled_units(dev):
    w = I.TRAIN_BWD_BF16
    say(f"{w.name}: gla_chunk_bwd at full size, oracle on sampled units")
    d = I.chunk_inputs(w)
    d.update(I.upstream_grads(w, d, final=True))
    got = _gpu_bwd(dev, d)
    units = [(0, 0), (3, 7), (7, 15)]
    _check(d, got, w.name, units=units)
    for x in got[:4]:
        assert torch.isfinite(x).all()


def test_bwd_deterministic(dev):
    say("gla_chunk_bwd twice on B=2 H=4 T=500 d128: bitwise equal")
    d = _case(2, 4, 500, 128, 128, gate="strong")
    a = _gpu_bwd(dev, d)
    b = _gpu_bwd(dev, d)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_alpha_zero_gives_nan_only_in_that_sequence(dev):
    say("gla_chunk_bwd with one alpha = 0 gate in sequence 1: NaN there, sequence 0 exact")
    d = _case(2, 1, 150, 64, 64)
    d["g"][1, 0, 70, 5] = float("-inf")
    got = _gpu_bwd(dev, d)
    assert not torch.isfinite(got[0][1]).all() or not torch.isfinite(got[1][1]).all()
    d0 = {k: (v[:1] if isinstance(v, torch.Tensor) and k != "cu_seqlens" else v) for k, v in d.items()}
    _check(d0, tuple(x[:1] for x in got), "bwd sequence 0 next to an alpha = 0 sequence")


def test_autograd_function_matches_entry_point(dev):
    from sub_quadratic_sequence_amd import gla

    say("GLAFunction forward + backward vs gla_chunk_bwd, B=1 H=2 T=190 d128")
    d = _case(1, 2, 190, 128, 128)
    leaves = [d[n].to(dev).requires_grad_(True) for n in ("q", "k", "v", "g")]
    s0 = d["s0"].to(dev).requires_grad_(True)
    o, sf = gla.GLAFunction.apply(*leaves, s0, None)
    torch.autograd.backward([o, sf], [d["do"].to(dev), d["dsT"].to(dev)])
    torch.cuda.synchronize()
    ref = _gpu_bwd(dev, d)
    for leaf, r in zip(leaves + [s0], ref):
        assert torch.equal(leaf.grad, r)


def _aligned(ws, nbytes):
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes]


@pytest.mark.parametrize("label,B,H,T,dk,dv,gate,lengths", [
    ("fixed_d128_strong", 2, 2, 300, 128, 128, "strong", None),
    ("dk128_dv64", 1, 2, 130, 128, 64, "weak", None),
    ("dk64_dv128", 2, 1, 200, 64, 128, "weak", None),
    ("backward_split_T3000", 1, 1, 3000, 128, 128, "strong", None),
    ("varlen", 1, 2, 0, 128, 128, "weak", [1, 0, 65, 200, 17, 64]),
    ("dv256", 1, 2, 200, 128, 256, "weak", None),
    ("dv192_varlen", 1, 2, 0, 64, 192, "strong", [70, 0, 130]),
    ("varlen_longest_first", 1, 2, 0, 128, 128, "weak", [0, 300, 65, 129]),
])
def test_saved_chunk_states_equal_recomputed(dev, label, B, H, T, dk, dv, gate, lengths):
    """gla_chunk_fwd_states writes the chunk states the backward computes for itself
    (bitwise), its outputs are gla_chunk_fwd's (bitwise, 64-column slices), and
    gla_chunk_bwd_saved on them gives gla_chunk_bwd's gradients (bitwise)."""
    from sub_quadratic_sequence_amd import gla

    say(f"saved chunk states {label}: B={B} H={H} T={T} dk={dk} dv={dv} gate={gate} lengths={lengths}")
    d = _case(B, H, T, dk, dv, gate=gate, lengths=lengths)
    to = lambda x: None if x is None else x.to(dev)
    q, k, v, g, do = (to(d[n]) for n in ("q", "k", "v", "g", "do"))
    s0, dsT, cu = to(d["s0"]), to(d["dsT"]), to(d["cu_seqlens"])
    need = gla.bwd_workspace_size(q, v, cu)
    # both workspaces start zeroed: the slots no chunk starts in stay equal
    ws_a = torch.zeros(need + 256, dtype=torch.uint8, device=dev)
    ws_b = torch.zeros(need + 256, dtype=torch.uint8, device=dev)
    ga = gla.gla_chunk_bwd(q, k, v, g, do, initial_state=s0, d_final_state=dsT, cu_seqlens=cu,
                           workspace=ws_a)
    o_s, sf_s, _ = gla.gla_chunk_fwd_states(q, k, v, g, initial_state=s0, output_final_state=True,
                                            cu_seqlens=cu, chunk_states=ws_b)
    o_r, sf_r = gla.gla_chunk_fwd(q, k, v, g, initial_state=s0, output_final_state=True,
                                  cu_seqlens=cu, split=False)
    gb = gla.gla_chunk_bwd_saved(q, k, v, g, do, ws_b, initial_state=s0, d_final_state=dsT,
                                 cu_seqlens=cu)
    torch.cuda.synchronize()
    nseq = B if cu is None else len(lengths)
    tokens = B * T if cu is None else sum(lengths)
    state_bytes = H * (nseq + tokens // 64 + 1) * dk * dv * 2
    assert torch.equal(_aligned(ws_a, state_bytes), _aligned(ws_b, state_bytes))
    assert torch.equal(o_s, o_r) and torch.equal(sf_s, sf_r)
    for x, y in zip(ga, gb):
        assert (x is None and y is None) or torch.equal(x, y)
    _check(d, gb, f"bwd from saved states {label}")


@pytest.mark.parametrize("save", [True, False])
def test_autograd_saved_and_recomputed_states_agree(dev, save):
    from sub_quadratic_sequence_amd import gla

    say(f"GLAFunction save_states={save}, B=2 H=2 T=333 d128 strong gates")
    d = _case(2, 2, 333, 128, 128, gate="strong")
    leaves = [d[n].to(dev).requires_grad_(True) for n in ("q", "k", "v", "g")]
    s0 = d["s0"].to(dev).requires_grad_(True)
    o, sf = gla.GLAFunction.apply(*leaves, s0, None, save)
    torch.autograd.backward([o, sf], [d["do"].to(dev), d["dsT"].to(dev)])
    torch.cuda.synchronize()
    ref = _gpu_bwd(dev, d)
    for leaf, r in zip(leaves + [s0], ref):
        assert torch.equal(leaf.grad, r)
