"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same
seeded inputs.  Tolerances (per-unit max error over max |reference|, see
parity.py): 2e-2 on the bf16 path, 1e-4 on the fp32 path.  Every test prints
the case it is about to run before touching the GPU."""
import os

import numpy as np
import pytest
import torch

import oracle
from parity import TOL_BF16, TOL_F32, to64, unit_err_fixed, unit_err_varlen
from sub_quadratic_sequence_amd import inputs as I

pytestmark = pytest.mark.gpu

NTHREADS = min(16, os.cpu_count() or 1)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sub_quadratic_sequence_amd import gla

    gla.load_library()
    return torch.device("cuda:0")


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def _fwd(dev, d, s0=None, final=True, cu=None, dv_slice=None):
    from sub_quadratic_sequence_amd import gla

    args = [d[n].to(dev) for n in "qkvg"]
    o, sf = gla.gla_chunk_fwd(*args, initial_state=None if s0 is None else s0.to(dev),
                              output_final_state=final,
                              cu_seqlens=None if cu is None else cu.to(dev), dv_slice=dv_slice)
    torch.cuda.synchronize()
    return o, sf


def _check_fixed(d, o, sf, s0, tol, label):
    o_ref, s_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], s0=s0, nthreads=NTHREADS)
    e_o, e_s = unit_err_fixed(o, o_ref), unit_err_fixed(sf, s_ref)
    print(f"{label}: O err {e_o:.3e}  S err {e_s:.3e}  (tol {tol})", flush=True)
    assert np.all(np.isfinite(to64(o))) and np.all(np.isfinite(to64(sf)))
    assert e_o <= tol and e_s <= tol, (e_o, e_s)


# ------------------------------------------------------------------ the workloads
def test_tiny_fp32(dev):
    w = I.TINY_FP32
    say(f"{w.name} seed={w.seed} gla_chunk_fwd")
    d = I.chunk_inputs(w)
    o, sf = _fwd(dev, d)
    _check_fixed(d, o, sf, None, TOL_F32, w.name)


def test_train_bf16_full(dev):
    w = I.TRAIN_BF16
    say(f"{w.name} seed={w.seed} gla_chunk_fwd (full size)")
    d = I.chunk_inputs(w)
    o, sf = _fwd(dev, d)
    _check_fixed(d, o, sf, None, TOL_BF16, w.name)


def test_long_bf16_full(dev):
    w = I.LONG_BF16
    say(f"{w.name} seed={w.seed} gla_chunk_fwd (full size, initial state)")
    d = I.chunk_inputs(w)
    o, sf = _fwd(dev, d, s0=d["s0"])
    _check_fixed(d, o, sf, d["s0"], TOL_BF16, w.name)


def test_varlen_strong_bf16_full(dev):
    w = I.VARLEN_BF16
    say(f"{w.name} seed={w.seed} gla_chunk_fwd (full size, packed, strong gates)")
    d = I.chunk_inputs(w)
    o, sf = _fwd(dev, d, cu=d["cu_seqlens"])
    o_ref, s_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], cu_seqlens=d["cu_seqlens"],
                                     nthreads=NTHREADS)
    e_o = unit_err_varlen(o, o_ref, d["cu_seqlens"])
    e_s = unit_err_fixed(sf, s_ref)
    print(f"{w.name}: O err {e_o:.3e}  S err {e_s:.3e}", flush=True)
    assert np.all(np.isfinite(to64(o)))
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16


def test_decode_full(dev):
    from sub_quadratic_sequence_amd import gla

    w = I.DECODE_BF16
    say(f"{w.name} seed={w.seed} gla_recurrent_step x{w.steps} (full size)")
    d = I.decode_inputs(w)
    st = d["s0"].to(dev).clone()
    outs = []
    for t in range(w.steps):
        outs.append(gla.gla_recurrent_step(*(d[n][t].to(dev) for n in "qkvg"), st).float().cpu())
    torch.cuda.synchronize()
    # the oracle runs the same 64 tokens as one recurrence per (sequence, head)
    q, k, v, g = (d[n].permute(1, 2, 0, 3).contiguous() for n in "qkvg")   # [N, H, steps, d]
    o_ref, s_ref = oracle.recurrence(q, k, v, g, s0=d["s0"], nthreads=NTHREADS)
    o_gpu = torch.stack(outs, 2)                                            # [N, H, steps, dv]
    e_o, e_s = unit_err_fixed(o_gpu, o_ref), unit_err_fixed(st, s_ref)
    print(f"{w.name}: O err {e_o:.3e}  S err {e_s:.3e}", flush=True)
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16


# ------------------------------------------------------------------ fp32 path edge cases
FP32_CASES = [
    # (label, B, H, T, dv, gate, s0)
    ("ragged_T200_s0", 1, 2, 200, 64, "weak", True),
    ("T1", 2, 2, 1, 64, "weak", True),
    ("T63", 1, 3, 63, 64, "weak", False),
    ("T65_s0", 1, 2, 65, 64, "weak", True),
    ("alpha1_s0", 2, 2, 256, 64, "zero", True),
    ("strong_T300_s0", 1, 2, 300, 64, "strong", True),
    ("dv192_B3H3_T130", 3, 3, 130, 192, "weak", True),
    ("dv128_strong", 2, 1, 190, 128, "strong", False),
]


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("label,B,H,T,dv,gate,s0", FP32_CASES, ids=[c[0] for c in FP32_CASES])
def test_fp32_cases(dev, label, B, H, T, dv, gate, s0, dk):
    w = I.ChunkWorkload("fp32_edge", B=B, H=H, T=T, dk=dk, dv=dv, dtype="f32", seed=101,
                        k_scaled=True)
    say(f"fp32 {label}: B={B} H={H} T={T} dk={dk} dv={dv} gate={gate} s0={s0}")
    d = I.chunk_inputs(w, gate=gate, s0=s0)
    o, sf = _fwd(dev, d, s0=d["s0"])
    _check_fixed(d, o, sf, d["s0"], TOL_F32, label)


@pytest.mark.parametrize("dk", [64, 128])
def test_fp32_extreme_gates_exact_diagonal(dev, dk):
    """Some channels decay by far more than 2^100 inside one 16-token sub-chunk
    (and a few gates are -inf, alpha = 0): the diagonal score blocks are then
    evaluated element by element."""
    w = I.ChunkWorkload("fp32_extreme", B=1, H=2, T=192, dk=dk, dv=64, dtype="f32", seed=7,
                        k_scaled=True)
    say(f"fp32 extreme gates: B=1 H=2 T=192 dk={dk} dv=64, g down to -80 and -inf")
    d = I.chunk_inputs(w, s0=True)
    gen = torch.Generator().manual_seed(3)
    mask = torch.rand(d["g"].shape, generator=gen) < 0.3
    g = torch.where(mask, -80.0 * torch.rand(d["g"].shape, generator=gen), d["g"])
    g[0, 0, 70, 5] = float("-inf")
    d["g"] = g
    o, sf = _fwd(dev, d, s0=d["s0"])
    _check_fixed(d, o, sf, d["s0"], TOL_F32, f"extreme dk={dk}")


def test_fp32_tiny_recipe_at_dk128(dev):
    """The tiny fp32 workload's recipe at d_k = d_v = 128 (B1 H2 T256, k scaled
    by d_k^-1/2, weak gates): two 64-channel passes per chunk."""
    w = I.ChunkWorkload("fp32_tiny_d128", B=1, H=2, T=256, dk=128, dv=128, dtype="f32", seed=1,
                        k_scaled=True)
    say("fp32 tiny recipe at dk=dv=128: B=1 H=2 T=256")
    d = I.chunk_inputs(w)
    o, sf = _fwd(dev, d)
    _check_fixed(d, o, sf, None, TOL_F32, "fp32 tiny d128")


def test_fp32_dk128_passes_in_different_modes(dev):
    """d_k = 128 in fp32: strong gates on channels 64..127 only, so within a chunk
    the first 64-channel pass takes the single pivot and the second the
    sub-chunk pivots (and one channel of the second decays beyond 2^100)."""
    w = I.ChunkWorkload("fp32_mixed", B=2, H=2, T=200, dk=128, dv=64, dtype="f32", seed=29,
                        k_scaled=True)
    say("fp32 dk=128 mixed passes: weak gates on channels 0..63, strong on 64..127")
    d = I.chunk_inputs(w, s0=True)
    strong = I.chunk_inputs(w, gate="strong", s0=True)["g"]
    g = d["g"].clone()
    g[..., 64:] = strong[..., 64:]
    g[0, 1, 40:56, 100] = -20.0
    d["g"] = g
    o, sf = _fwd(dev, d, s0=d["s0"])
    _check_fixed(d, o, sf, d["s0"], TOL_F32, "fp32 mixed passes")


@pytest.mark.parametrize("dk", [128, 64])
def test_bf16_extreme_gates_exact_diagonal(dev, dk):
    """bf16 path with gates that decay by more than 2^100 inside a 16-token
    sub-chunk (and alpha = 0 tokens): exact diagonal partials."""
    w = I.ChunkWorkload("bf16_extreme", B=2, H=2, T=200, dk=dk, dv=128, dtype="bf16", seed=17,
                        k_scaled=True)
    say(f"bf16 extreme gates: B=2 H=2 T=200 dk={dk} dv=128, g down to -80 and -inf")
    d = I.chunk_inputs(w, s0=True)
    gen = torch.Generator().manual_seed(5)
    g = d["g"].float()
    mask = torch.rand(g.shape, generator=gen) < 0.3
    g = torch.where(mask, -80.0 * torch.rand(g.shape, generator=gen), g)
    g[0, 1, 100, 7] = float("-inf")
    g[1, 0, 10:20, :] = float("-inf")
    d["g"] = g.to(torch.bfloat16)
    o, sf = _fwd(dev, d, s0=d["s0"])
    _check_fixed(d, o, sf, d["s0"], TOL_BF16, f"bf16 extreme dk={dk}")


def test_bf16_mixed_fast_and_safe_slices(dev):
    """Strong gates on some key channels only: within one chunk some 32-channel
    slices take the single-pivot form and others the sub-chunk pivots."""
    w = I.ChunkWorkload("bf16_mixed", B=1, H=3, T=256, dk=128, dv=128, dtype="bf16", seed=23)
    say("bf16 mixed gates: strong on channels 32..63 and 100..101, weak elsewhere")
    d = I.chunk_inputs(w, s0=True)
    strong = I.chunk_inputs(w, gate="strong", s0=True)["g"]
    g = d["g"].clone()
    g[..., 32:64] = strong[..., 32:64]
    g[..., 100:102] = strong[..., 100:102]
    d["g"] = g
    o, sf = _fwd(dev, d, s0=d["s0"])
    _check_fixed(d, o, sf, d["s0"], TOL_BF16, "bf16 mixed")


@pytest.mark.parametrize("dk", [64, 128])
def test_fp32_varlen_with_empty_and_short(dev, dk):
    lengths = [5, 0, 64, 1, 130, 0, 77]
    w = I.ChunkWorkload("fp32_varlen", B=1, H=2, T=0, dk=dk, dv=64, dtype="f32", seed=11,
                        k_scaled=True)
    say(f"fp32 varlen dk={dk} lengths={lengths} with initial state")
    d = I.chunk_inputs(w, lengths=lengths, s0=True)
    o, sf = _fwd(dev, d, s0=d["s0"], cu=d["cu_seqlens"])
    o_ref, s_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], s0=d["s0"],
                                     cu_seqlens=d["cu_seqlens"])
    e_o, e_s = unit_err_varlen(o, o_ref, d["cu_seqlens"]), unit_err_fixed(sf, s_ref)
    print(f"varlen fp32: O err {e_o:.3e} S err {e_s:.3e}", flush=True)
    assert e_o <= TOL_F32 and e_s <= TOL_F32
    # empty sequences pass their initial state through unchanged
    assert torch.equal(sf[1].cpu(), d["s0"][1]) and torch.equal(sf[5].cpu(), d["s0"][5])


@pytest.mark.parametrize("H,lengths", [
    (2, [5, 0, 64, 1, 130, 0, 77, 300]),            # 16 units: longest-first work order
    (3, [5, 0, 64, 1, 130, 0, 77]),                  # 21 units: natural order
    (1, [700, 65, 64, 63, 1, 2, 3, 900]),           # 8 units, sorted, ties and tails
])
def test_bf16_varlen_with_empty_and_short(dev, H, lengths):
    """Packed bf16 sequences, some empty or a single token, with an initial
    state; with a multiple of 8 (sequence, head) units the work items are
    dispatched longest sequence first."""
    w = I.ChunkWorkload("bf16_varlen", B=1, H=H, T=0, dk=128, dv=128, dtype="bf16", seed=29,
                        k_scaled=True)
    say(f"bf16 varlen H={H} lengths={lengths} with initial state")
    d = I.chunk_inputs(w, lengths=lengths, s0=True)
    o, sf = _fwd(dev, d, s0=d["s0"], cu=d["cu_seqlens"])
    o_ref, s_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], s0=d["s0"],
                                     cu_seqlens=d["cu_seqlens"])
    e_o, e_s = unit_err_varlen(o, o_ref, d["cu_seqlens"]), unit_err_fixed(sf, s_ref)
    print(f"varlen bf16 H={H}: O err {e_o:.3e} S err {e_s:.3e}", flush=True)
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16
    for n, ln in enumerate(lengths):
        if ln == 0:   # an empty sequence passes its initial state through unchanged
            assert torch.equal(sf[n].cpu(), d["s0"][n])


# ------------------------------------------------------------------ bf16 shapes
BF16_CASES = [
    ("dk64_dv64_T300", 2, 4, 300, 64, 64, "weak"),
    ("dk128_dv192_T200", 1, 3, 200, 128, 192, "weak"),
    ("dk128_dv512_T128", 1, 2, 128, 128, 512, "weak"),
    ("dk128_strong_T257", 2, 2, 257, 128, 128, "strong"),
]


@pytest.mark.parametrize("label,B,H,T,dk,dv,gate", BF16_CASES, ids=[c[0] for c in BF16_CASES])
def test_bf16_shapes(dev, label, B, H, T, dk, dv, gate):
    w = I.ChunkWorkload("bf16_shape", B=B, H=H, T=T, dk=dk, dv=dv, dtype="bf16", seed=21)
    say(f"bf16 {label}: B={B} H={H} T={T} dk={dk} dv={dv} gate={gate}, initial state")
    d = I.chunk_inputs(w, gate=gate, s0=True)
    o, sf = _fwd(dev, d, s0=d["s0"])
    _check_fixed(d, o, sf, d["s0"], TOL_BF16, label)


# ------------------------------------------------------------------ 128-column d_v slice
# gla_chunk_fwd_sliced with dv_slice = 128 runs the bf16 forward with 128 value
# columns per workgroup at any unit count; gla_chunk_fwd takes that width where
# gla_slice_plan's model says it is faster.
WIDE_CASES = [
    ("dk128_dv256_weak_T130", 2, 3, 130, 128, 256, "weak"),
    ("dk128_dv128_strong_T97", 4, 2, 97, 128, 128, "strong"),
    ("dk64_dv256_weak_T200", 2, 2, 200, 64, 256, "weak"),
    ("dk64_dv384_strong_T65", 1, 3, 65, 64, 384, "strong"),
    ("dk128_dv128_weak_T1", 3, 2, 1, 128, 128, "weak"),
]


@pytest.mark.parametrize("label,B,H,T,dk,dv,gate", WIDE_CASES, ids=[c[0] for c in WIDE_CASES])
def test_bf16_wide_slice(dev, label, B, H, T, dk, dv, gate):
    w = I.ChunkWorkload("bf16_wide", B=B, H=H, T=T, dk=dk, dv=dv, dtype="bf16", seed=31)
    say(f"bf16 128-column slice {label}: B={B} H={H} T={T} dk={dk} dv={dv} gate={gate}, initial state")
    d = I.chunk_inputs(w, gate=gate, s0=True)
    o, sf = _fwd(dev, d, s0=d["s0"], dv_slice=128)
    _check_fixed(d, o, sf, d["s0"], TOL_BF16, label)


def test_bf16_wide_slice_extreme_gates(dev):
    """The 128-column slice with gates that decay by more than 2^100 inside a
    sub-chunk (exact diagonal partials) and alpha = 0 tokens."""
    w = I.ChunkWorkload("bf16_wide_extreme", B=2, H=4, T=80, dk=128, dv=128, dtype="bf16", seed=37,
                        k_scaled=True)
    say("bf16 128-column slice, extreme gates: B=2 H=4 T=80 dk=128 dv=128")
    d = I.chunk_inputs(w, s0=True)
    gen = torch.Generator().manual_seed(6)
    g = d["g"].float()
    mask = torch.rand(g.shape, generator=gen) < 0.3
    g = torch.where(mask, -80.0 * torch.rand(g.shape, generator=gen), g)
    g[0, 1, 40, 7] = float("-inf")
    g[1, 3, 10:20, :] = float("-inf")
    d["g"] = g.to(torch.bfloat16)
    o, sf = _fwd(dev, d, s0=d["s0"], dv_slice=128)
    _check_fixed(d, o, sf, d["s0"], TOL_BF16, "wide extreme")


@pytest.mark.parametrize("H,lengths", [(2, [300, 5, 0, 129, 1, 64, 200, 77]),
                                       (3, [300, 5, 0, 129, 1, 64, 200])])
def test_bf16_wide_slice_packed(dev, H, lengths):
    """Packed sequences (empty, one token, ragged tails) on the 128-column slice:
    16 units (a multiple of 8) are dispatched longest sequence first, 21 in order."""
    w = I.ChunkWorkload("bf16_wide_varlen", B=1, H=H, T=0, dk=128, dv=256, dtype="bf16", seed=41,
                        k_scaled=True)
    say(f"bf16 128-column slice, packed H={H} lengths={lengths} dv=256, strong gates")
    d = I.chunk_inputs(w, lengths=lengths, s0=True, gate="strong")
    o, sf = _fwd(dev, d, s0=d["s0"], cu=d["cu_seqlens"], dv_slice=128)
    o_ref, s_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], s0=d["s0"],
                                     cu_seqlens=d["cu_seqlens"], nthreads=NTHREADS)
    e_o, e_s = unit_err_varlen(o, o_ref, d["cu_seqlens"]), unit_err_fixed(sf, s_ref)
    print(f"wide packed: O err {e_o:.3e} S err {e_s:.3e}", flush=True)
    assert e_o <= TOL_BF16 and e_s <= TOL_BF16
    assert torch.equal(sf[2].cpu(), d["s0"][2])


def test_named_forward_wrappers(dev):
    """gla.gla_chunk_fwd_ws and gla.gla_chunk_fwd_sliced (the C entry points' names)
    give what gla_chunk_fwd gives with split=True and with dv_slice, bit for bit."""
    from sub_quadratic_sequence_amd import gla

    w = I.ChunkWorkload("wrappers", B=1, H=3, T=1500, dk=128, dv=256, dtype="bf16", seed=45)
    say("named wrappers: B=1 H=3 T=1500 dk=128 dv=256, initial state")
    d = I.chunk_inputs(w, s0=True)
    q, k, v, g, s0 = (d[n].to(dev) for n in ("q", "k", "v", "g", "s0"))
    a = gla.gla_chunk_fwd_ws(q, k, v, g, initial_state=s0, output_final_state=True)
    b = gla.gla_chunk_fwd(q, k, v, g, initial_state=s0, output_final_state=True, split=True)
    c = gla.gla_chunk_fwd_sliced(q, k, v, g, 128, initial_state=s0, output_final_state=True)
    e = gla.gla_chunk_fwd(q, k, v, g, initial_state=s0, output_final_state=True, dv_slice=128)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(c[0], e[0]) and torch.equal(c[1], e[1])
    _check_fixed(d, a[0], a[1], d["s0"], TOL_BF16, "gla_chunk_fwd_ws")


@pytest.mark.parametrize("dv_slice", [0, 64, 128])
def test_both_slice_widths_match_oracle(dev, dv_slice):
    """gla_chunk_fwd_sliced at either width, and at the plan's choice (0), on
    the same inputs: all within tolerance of the oracle."""
    w = I.ChunkWorkload("bf16_slices", B=2, H=3, T=190, dk=128, dv=256, dtype="bf16", seed=43)
    say(f"bf16 dv_slice={dv_slice}: B=2 H=3 T=190 dk=128 dv=256, initial state")
    d = I.chunk_inputs(w, s0=True, gate="strong")
    o, sf = _fwd(dev, d, s0=d["s0"], dv_slice=dv_slice)
    _check_fixed(d, o, sf, d["s0"], TOL_BF16, f"dv_slice {dv_slice}")


def test_planned_wide_slice_below_one_round(dev):
    """Work items of 128 columns that fill three quarters of the compute units:
    the plan takes the 128-column slice (one partial round against two of 64
    columns), and gla_chunk_fwd then gives the same bits as dv_slice = 128."""
    from sub_quadratic_sequence_amd import gla

    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    H = (3 * ncu + 3) // 4
    assert gla.slice_plan(H, 128) == 128
    assert gla.slice_plan((ncu + 1) // 2, 128) == 64
    w = I.ChunkWorkload("bf16_planned_wide", B=1, H=H, T=70, dk=128, dv=128, dtype="bf16", seed=47)
    say(f"bf16 planned 128-column slice: B=1 H={H} T=70 dk=128 dv=128 ({ncu} CUs)")
    d = I.chunk_inputs(w, s0=True)
    o, sf = _fwd(dev, d, s0=d["s0"])
    o_w, sf_w = _fwd(dev, d, s0=d["s0"], dv_slice=128)
    assert torch.equal(o, o_w) and torch.equal(sf, sf_w)
    _check_fixed(d, o, sf, d["s0"], TOL_BF16, "planned wide")


# ------------------------------------------------------------------ invariants
def test_decode_fp32_small(dev):
    from sub_quadratic_sequence_amd import gla

    w = I.DecodeWorkload("dec_f32", N=5, H=3, dk=64, dv=128, steps=6, seed=9, dtype="f32")
    say("gla_recurrent_step fp32 N=5 H=3 dk=64 dv=128 x6")
    d = I.decode_inputs(w)
    st = d["s0"].to(dev).clone()
    s_ref = d["s0"].double().numpy()
    for t in range(w.steps):
        o = gla.gla_recurrent_step(*(d[n][t].to(dev) for n in "qkvg"), st)
        o_ref, s_ref = oracle.decode_step(*(d[n][t] for n in "qkvg"), s_ref)
        torch.cuda.synchronize()
        assert unit_err_fixed(o, o_ref) <= TOL_F32
    assert unit_err_fixed(st, s_ref) <= TOL_F32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(a, b) for a in (64, 128, 256) for b in (64, 128, 256)])
def test_decode_every_accepted_shape(dev, dk, dv, dtype):
    """Every (d_k, d_v, dtype) that gla_recurrent_step accepts, against the oracle
    over a few steps (each shape is its own kernel instantiation: rows per lane,
    row groups and the cross-row reduction differ)."""
    from sub_quadratic_sequence_amd import gla

    w = I.DecodeWorkload(f"dec_{dtype}", N=3, H=2, dk=dk, dv=dv, steps=4, seed=11 + dk + dv,
                         dtype=dtype)
    tol = TOL_BF16 if dtype == "bf16" else TOL_F32
    say(f"gla_recurrent_step {dtype} N=3 H=2 dk={dk} dv={dv} x4")
    d = I.decode_inputs(w)
    st = d["s0"].to(dev).clone()
    s_ref = d["s0"].double().numpy()
    for t in range(w.steps):
        o = gla.gla_recurrent_step(*(d[n][t].to(dev) for n in "qkvg"), st)
        o_ref, s_ref = oracle.decode_step(*(d[n][t] for n in "qkvg"), s_ref)
        torch.cuda.synchronize()
        e_o = unit_err_fixed(o, o_ref)
        assert np.all(np.isfinite(to64(o)))
        assert e_o <= tol, (t, e_o)
    e_s = unit_err_fixed(st, s_ref)
    print(f"decode {dtype} dk={dk} dv={dv}: O err {e_o:.3e} S err {e_s:.3e}", flush=True)
    assert e_s <= tol


def test_decode_steps_equal_chunk_fwd(dev):
    """64 decode steps and one chunked call over the same 64 tokens give the same
    outputs and final state (fp32 path; both against each other)."""
    from sub_quadratic_sequence_amd import gla

    w = I.DecodeWorkload("dec_vs_chunk", N=3, H=2, dk=64, dv=64, steps=64, seed=13, dtype="f32")
    say("decode x64 vs gla_chunk_fwd T=64, fp32, N=3 H=2 d=64")
    d = I.decode_inputs(w)
    st = d["s0"].to(dev).clone()
    outs = [gla.gla_recurrent_step(*(d[n][t].to(dev) for n in "qkvg"), st) for t in range(64)]
    o_dec = torch.stack(outs, 2)
    q, k, v, g = (d[n].permute(1, 2, 0, 3).contiguous().to(dev) for n in "qkvg")
    o_ch, s_ch = gla.gla_chunk_fwd(q, k, v, g, initial_state=d["s0"].to(dev), output_final_state=True)
    torch.cuda.synchronize()
    assert unit_err_fixed(o_dec, o_ch) <= 2e-4
    assert unit_err_fixed(st, s_ch) <= 2e-4


def test_split_call_composition(dev):
    from sub_quadratic_sequence_amd import gla

    w = I.TRAIN_BF16
    say("split call: bf16 B=2 H=4 T=448 split at 192, state passed between calls")
    d = I.chunk_inputs(w, B=2, H=4, T=448, s0=True)
    args = [d[n].to(dev) for n in "qkvg"]
    o, sf = gla.gla_chunk_fwd(*args, initial_state=d["s0"].to(dev), output_final_state=True)
    a = [x[:, :, :192].contiguous() for x in args]
    b = [x[:, :, 192:].contiguous() for x in args]
    oa, sa = gla.gla_chunk_fwd(*a, initial_state=d["s0"].to(dev), output_final_state=True)
    ob, sb = gla.gla_chunk_fwd(*b, initial_state=sa, output_final_state=True)
    torch.cuda.synchronize()
    assert unit_err_fixed(torch.cat([oa, ob], 2).float(), o.float()) <= TOL_BF16
    assert unit_err_fixed(sb, sf) <= TOL_BF16


def test_bitwise_deterministic(dev):
    from sub_quadratic_sequence_amd import gla

    say("determinism: bf16 B=2 H=4 T=320 d=128, two identical calls")
    d = I.chunk_inputs(I.TRAIN_BF16, B=2, H=4, T=320, s0=True)
    args = [d[n].to(dev) for n in "qkvg"]
    s0 = d["s0"].to(dev)
    o1, s1 = gla.gla_chunk_fwd(*args, initial_state=s0, output_final_state=True)
    o2, s2 = gla.gla_chunk_fwd(*args, initial_state=s0, output_final_state=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_state_aliasing_in_place(dev):
    from sub_quadratic_sequence_amd import gla

    say("in place: final_state aliases initial_state, bf16 B=1 H=2 T=130")
    d = I.chunk_inputs(I.TRAIN_BF16, B=1, H=2, T=130, s0=True)
    args = [d[n].to(dev) for n in "qkvg"]
    s0 = d["s0"].to(dev)
    o1, s1 = gla.gla_chunk_fwd(*args, initial_state=s0.clone(), output_final_state=True)
    st = s0.clone()
    o2, s2 = gla.gla_chunk_fwd(*args, initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, st)


def test_zero_tokens_passes_state(dev):
    from sub_quadratic_sequence_amd import gla

    say("T=0: final state equals initial state")
    s0 = torch.randn(2, 3, 128, 128, device=dev)
    e = torch.empty(2, 3, 0, 128, dtype=torch.bfloat16, device=dev)
    o, sf = gla.gla_chunk_fwd(e, e, e, e, initial_state=s0, output_final_state=True)
    o0, sz = gla.gla_chunk_fwd(e, e, e, e, output_final_state=True)
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 128) and torch.equal(sf, s0) and not torch.any(sz)


def test_nan_propagates(dev):
    from sub_quadratic_sequence_amd import gla

    say("NaN in v at token 70 of unit (0,1): NaN in column 3 of that unit from its chunk on")
    d = I.chunk_inputs(I.TRAIN_BF16, B=1, H=2, T=192)
    d["v"][0, 1, 70, 3] = float("nan")
    o, sf = _fwd(dev, d)
    o = o.float().cpu()
    # the masked score (0) times NaN is NaN inside the 64-token chunk holding token 70,
    # so earlier tokens of that chunk (64..69) may show it too; nothing before 64 may
    assert torch.isfinite(o[0, 0]).all() and torch.isfinite(o[0, 1, :64]).all()
    assert torch.isfinite(o[0, 1, :, [0, 1, 2, 4]]).all()
    assert torch.isnan(o[0, 1, 70:, 3]).all()
    assert torch.isnan(sf[0, 1]).any() and torch.isfinite(sf[0, 0]).all()


# ------------------------------------------------------------------ sequence split
SPLIT_CASES = [
    # (label, B, H, T, dk, dv, gate, s0)
    ("weak_s0_T5000", 1, 2, 5000, 128, 128, "weak", True),
    ("strong_dv256_T3000", 1, 2, 3000, 128, 256, "strong", True),
    ("dk64_T2500", 2, 1, 2500, 64, 64, "weak", True),
    ("ragged_T1025", 1, 1, 1025, 128, 128, "weak", False),
    ("dk64_dv128_strong_T2100", 1, 2, 2100, 64, 128, "strong", True),
]


@pytest.mark.parametrize("label,B,H,T,dk,dv,gate,s0", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_sequence_split_matches_oracle(dev, label, B, H, T, dk, dv, gate, s0):
    """Few units and long sequences: gla_chunk_fwd_ws cuts the sequences into
    segments (state pass, segment scan, forward from the incoming states).  The
    result matches the oracle and the unsplit call."""
    from sub_quadratic_sequence_amd import gla

    w = I.ChunkWorkload("split", B=B, H=H, T=T, dk=dk, dv=dv, dtype="bf16", seed=31)
    say(f"sequence split {label}: B={B} H={H} T={T} dk={dk} dv={dv} gate={gate} s0={s0}")
    d = I.chunk_inputs(w, gate=gate, s0=s0)
    args = [d[n].to(dev) for n in "qkvg"]
    s0_dev = None if d["s0"] is None else d["s0"].to(dev)
    # the planned call (gla_chunk_fwd_ws) and a forced 4-segment split
    nseg, _ = gla.split_plan(B * H, T, dv)
    assert (gla.workspace_size(args[0], args[2]) > 0) == (nseg > 1)
    o, sf = gla.gla_chunk_fwd(*args, initial_state=s0_dev, output_final_state=True)
    o4, s4 = gla.gla_chunk_fwd_segments(*args, 4, initial_state=s0_dev, output_final_state=True)
    o1, s1 = gla.gla_chunk_fwd(*args, initial_state=s0_dev, output_final_state=True, split=False)
    torch.cuda.synchronize()
    say(f"  planned segments {nseg}")
    _check_fixed(d, o, sf, d["s0"], TOL_BF16, f"split {label}")
    _check_fixed(d, o4, s4, d["s0"], TOL_BF16, f"4 segments {label}")
    assert unit_err_fixed(o.float(), o1.float()) <= TOL_BF16
    assert unit_err_fixed(sf, s1) <= TOL_BF16


SEGMENT_GRID = [
    # (B, H, T, dv): segment counts 1, 2, 5, 16 and one segment per chunk
    (1, 1, 1025, 128),
    (1, 3, 2048, 128),
    (2, 4, 4100, 256),
    (1, 8, 3000, 64),
]


@pytest.mark.parametrize("B,H,T,dv", SEGMENT_GRID, ids=[f"B{c[0]}H{c[1]}T{c[2]}dv{c[3]}" for c in SEGMENT_GRID])
def test_forced_segment_counts_match_oracle(dev, B, H, T, dv):
    """gla_chunk_fwd_segments at segment counts from 1 to one per chunk (ragged last
    segments included): every count matches the oracle."""
    from sub_quadratic_sequence_amd import gla

    w = I.ChunkWorkload("segments", B=B, H=H, T=T, dk=128, dv=dv, dtype="bf16", seed=43)
    d = I.chunk_inputs(w, gate="weak", s0=True)
    args = [d[n].to(dev) for n in "qkvg"]
    o_ref, s_ref = oracle.recurrence(d["q"], d["k"], d["v"], d["g"], s0=d["s0"], nthreads=NTHREADS)
    nch = -(-T // 64)
    for n in (1, 2, 5, 16, nch):
        say(f"forced segments: B={B} H={H} T={T} dv={dv}, {n} requested")
        o, sf = gla.gla_chunk_fwd_segments(*args, n, initial_state=d["s0"].to(dev),
                                           output_final_state=True)
        torch.cuda.synchronize()
        e_o, e_s = unit_err_fixed(o, o_ref), unit_err_fixed(sf, s_ref)
        print(f"  O err {e_o:.3e}  S err {e_s:.3e}", flush=True)
        assert e_o <= TOL_BF16 and e_s <= TOL_BF16, (n, e_o, e_s)


PLAN_GRID = [(1, 1, 700), (1, 4, 2048), (2, 8, 4096), (1, 32, 1100), (4, 16, 1536), (8, 16, 640)]


@pytest.mark.parametrize("B,H,T", PLAN_GRID, ids=[f"B{c[0]}H{c[1]}T{c[2]}" for c in PLAN_GRID])
def test_planned_split_across_units_and_lengths(dev, B, H, T):
    """The cost model's plan across a grid of (B x H, T): the planned call matches
    the oracle, and its workspace follows the plan."""
    from sub_quadratic_sequence_amd import gla

    w = I.ChunkWorkload("plan", B=B, H=H, T=T, dk=128, dv=128, dtype="bf16", seed=47)
    d = I.chunk_inputs(w, gate="weak", s0=True)
    args = [d[n].to(dev) for n in "qkvg"]
    nseg, seg_len = gla.split_plan(B * H, T, 128)
    say(f"planned split: B={B} H={H} T={T} -> {nseg} segments of {seg_len} tokens")
    need = gla.workspace_size(args[0], args[2])
    if nseg > 1:
        assert need == -(-B * H * nseg * 128 * 128 * 4 // 256) * 256 + -(-B * H * nseg * 128 * 4 // 256) * 256
    else:
        assert need == 0
    o, sf = gla.gla_chunk_fwd(*args, initial_state=d["s0"].to(dev), output_final_state=True)
    torch.cuda.synchronize()
    _check_fixed(d, o, sf, d["s0"], TOL_BF16, f"plan B{B}H{H}T{T}")


def test_sequence_split_extreme_gates(dev):
    """alpha = 0 tokens and 16-token decays beyond 2^100 inside split segments:
    a segment's total decay underflows to zero and its state restarts."""
    w = I.ChunkWorkload("split_extreme", B=1, H=2, T=2100, dk=128, dv=128, dtype="bf16", seed=37,
                        k_scaled=True)
    say("sequence split, extreme gates: B=1 H=2 T=2100, g down to -80 and -inf")
    d = I.chunk_inputs(w, s0=True)
    gen = torch.Generator().manual_seed(41)
    g = d["g"].float()
    mask = torch.rand(g.shape, generator=gen) < 0.05
    g = torch.where(mask, -80.0 * torch.rand(g.shape, generator=gen), g)
    g[0, 1, 900, :] = float("-inf")
    g[0, 0, 1500:1510, 3] = float("-inf")
    d["g"] = g.to(torch.bfloat16)
    o, sf = _fwd(dev, d, s0=d["s0"])
    _check_fixed(d, o, sf, d["s0"], TOL_BF16, "split extreme")


def test_sequence_split_in_place_and_deterministic(dev):
    from sub_quadratic_sequence_amd import gla

    say("sequence split: final_state aliasing initial_state, and two identical calls")
    d = I.chunk_inputs(I.LONG_BF16, B=1, H=2, T=4100, s0=True)
    args = [d[n].to(dev) for n in "qkvg"]
    s0 = d["s0"].to(dev)
    o1, s1 = gla.gla_chunk_fwd(*args, initial_state=s0.clone(), output_final_state=True)
    st = s0.clone()
    o2, _ = gla.gla_chunk_fwd(*args, initial_state=st, final_state=st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, st)
