"""The C ABI library: it loads, exports every function include/gla.h declares,
and its host-side argument checks reject bad calls before any HIP call.  CPU
only: no call here reaches a kernel (every argument set is invalid)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gla.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*((?:gla|gdn)_\w+)\s*\(", text,
                                 flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    import torch  # noqa: F401  (torch first: the library binds to its HIP runtime)

    from sub_quadratic_sequence_amd import gla

    if not os.path.exists(gla.LIB_PATH):
        pytest.skip("libgla.so not built (run __graft_entry__.build())")
    return gla.load_library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    assert names == ["gdn_chunk_fwd", "gla_chunk_bwd", "gla_chunk_bwd_saved",
                     "gla_chunk_bwd_workspace_size", "gla_chunk_fwd", "gla_chunk_fwd_noalloc",
                     "gla_chunk_fwd_segments", "gla_chunk_fwd_segments_workspace_size",
                     "gla_chunk_fwd_sliced", "gla_chunk_fwd_states", "gla_chunk_fwd_workspace_size",
                     "gla_chunk_fwd_ws", "gla_last_error", "gla_recurrent_step", "gla_slice_plan",
                     "gla_split_plan", "gla_status_string"]


def test_binding_names_every_compute_entry_point():
    """The Python binding has a function of the same name for every entry point
    that computes or plans (status strings and size queries have their own names)."""
    from sub_quadratic_sequence_amd import gla

    for name in _declared_functions():
        if name.endswith("_workspace_size") or name in ("gla_status_string", "gla_last_error"):
            continue
        assert callable(getattr(gla, name, None)), name


def test_library_exports_every_declared_symbol(lib):
    from sub_quadratic_sequence_amd import gla

    out = subprocess.run(["nm", "-D", "--defined-only", gla.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    from sub_quadratic_sequence_amd import gla

    assert gla.status_string(0) == "GLA_OK"
    assert gla.status_string(1) == "GLA_ERR_INVALID_ARG"
    assert gla.status_string(2) == "GLA_ERR_UNSUPPORTED"
    assert gla.status_string(3) == "GLA_ERR_LAUNCH"
    assert gla.status_string(99) == "GLA_UNKNOWN_STATUS"


FAKE = 0x10000  # a 16-byte aligned address; never dereferenced (every call below is rejected)


def _chunk(lib, entry="gla_chunk_fwd", **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, s0=None, o=FAKE, sT=None, cu=None, num_seqs=0, B=1,
             H=2, T=64, dk=128, dv=128, C=64, dtype=0, dv_slice=0)
    a.update(kw)
    P = ctypes.c_void_p
    extra = (a["dv_slice"],) if entry == "gla_chunk_fwd_sliced" else ()
    return getattr(lib, entry)(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["s0"]), P(a["o"]),
                               P(a["sT"]), P(a["cu"]), a["num_seqs"], a["B"], a["H"], a["T"],
                               a["dk"], a["dv"], a["C"], a["dtype"], *extra, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), 1, "non-null"),
    (dict(o=None), 1, "non-null"),
    (dict(q=FAKE + 8), 1, "q is not 16-byte aligned"),
    (dict(sT=FAKE + 4), 1, "final_state is not 16-byte aligned"),
    (dict(B=0), 1, "must be positive"),
    (dict(T=-1), 1, "must be positive"),
    (dict(dtype=7), 1, "dtype"),
    (dict(C=128), 2, "chunk_size"),
    (dict(dk=96), 2, "dk=96"),
    (dict(dk=256, dtype=1), 2, "dk=256"),
    (dict(dv=96), 2, "dv=96"),
    (dict(dv=1024), 2, "dv=1024"),
    (dict(cu=FAKE, B=2, num_seqs=2), 1, "B == 1"),
    (dict(cu=FAKE, num_seqs=0), 1, "num_seqs"),
    (dict(B=4096, H=4096, T=4096), 1, "int32"),
])
@pytest.mark.parametrize("entry", ["gla_chunk_fwd", "gla_chunk_fwd_noalloc", "gla_chunk_fwd_sliced"])
def test_chunk_fwd_rejects(lib, entry, kw, status, needle):
    from sub_quadratic_sequence_amd import gla

    rc = _chunk(lib, entry, **kw)
    assert rc == status
    assert needle in gla.last_error()
    assert entry in gla.last_error()


@pytest.mark.parametrize("entry", ["gla_chunk_fwd", "gla_chunk_fwd_noalloc", "gla_chunk_fwd_sliced"])
def test_chunk_fwd_zero_tokens_without_outputs_is_a_noop(lib, entry):
    # T == 0 and no final state: nothing to do, returns OK without touching the GPU
    assert _chunk(lib, entry, q=None, k=None, v=None, g=None, o=None, T=0) == 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dv_slice=96), 1, "dv_slice = 96"),
    (dict(dv_slice=-1), 1, "dv_slice = -1"),
    (dict(dv_slice=256, dv=256), 1, "dv_slice = 256"),
    (dict(dv_slice=128, dtype=1), 2, "128-column slices"),
    (dict(dv_slice=128, dv=192), 2, "dv=192"),
    (dict(dv_slice=128, dv=64), 2, "dv=64"),
    (dict(dv_slice=128, dv=64, T=0, q=None, k=None, v=None, g=None, o=None), 2, "128-column"),
    (dict(dv_slice=96, T=0, q=None, k=None, v=None, g=None, o=None), 1, "dv_slice"),
])
def test_chunk_fwd_sliced_rejects(lib, kw, status, needle):
    from sub_quadratic_sequence_amd import gla

    assert _chunk(lib, "gla_chunk_fwd_sliced", **kw) == status
    assert needle in gla.last_error(), gla.last_error()
    assert "gla_chunk_fwd_sliced" in gla.last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(state=None), 1, "non-null"),
    (dict(dk=96), 2, "dk=96"),
    (dict(dv=512), 2, "dv=512"),
    (dict(N=0), 1, "must be positive"),
    (dict(o=FAKE + 2), 1, "o is not 16-byte aligned"),
    (dict(dtype=-1), 1, "dtype"),
])
def test_recurrent_step_rejects(lib, kw, status, needle):
    from sub_quadratic_sequence_amd import gla

    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, state=FAKE, o=FAKE, N=4, H=2, dk=128, dv=128, dtype=0)
    a.update(kw)
    P = ctypes.c_void_p
    rc = lib.gla_recurrent_step(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["state"]),
                                P(a["o"]), a["N"], a["H"], a["dk"], a["dv"], a["dtype"], None)
    assert rc == status
    assert needle in gla.last_error()


def test_last_error_is_per_thread(lib):
    """gla_last_error reports the calling thread's own last failure: two threads
    that fail differently, interleaved, each read back their own message."""
    import threading

    lib.gla_last_error.restype = ctypes.c_char_p
    barrier = threading.Barrier(2, timeout=30)   # a failing worker breaks it, not hangs it
    seen = {}

    def worker(name, kw, needle):
        try:
            for _ in range(50):
                assert _chunk(lib, "gla_chunk_fwd", **kw) != 0
                barrier.wait()   # the other thread fails in between
                msg = lib.gla_last_error().decode()
                if needle not in msg:
                    seen[name] = msg
                    barrier.abort()
                    return
                barrier.wait()
            seen[name] = "ok"
        except threading.BrokenBarrierError:
            seen.setdefault(name, "broken barrier")

    a = threading.Thread(target=worker, args=("a", dict(dk=96), "dk=96"))
    b = threading.Thread(target=worker, args=("b", dict(B=0), "must be positive"))
    a.start(); b.start(); a.join(); b.join()
    assert seen == {"a": "ok", "b": "ok"}, seen


def test_binding_refuses_cpu_tensors():
    import torch

    from sub_quadratic_sequence_amd import gla

    x = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError, match="GPU"):
        gla.gla_chunk_fwd(x, x, x, x)
    with pytest.raises(ValueError, match="GPU"):
        gla.gla_recurrent_step(x[0], x[0], x[0], x[0], torch.zeros(1, 64, 64, 64))


def test_workspace_size_only_for_few_long_fixed_length_sequences(lib):
    # long context, 16 units x 2 slices: split; training shape (256 work items),
    # packed sequences and fp32: no split
    assert lib.gla_chunk_fwd_workspace_size(0, 1, 16, 65536, 128, 128, 64, 0) > 0
    assert lib.gla_chunk_fwd_workspace_size(0, 8, 16, 2048, 128, 128, 64, 0) == 0
    assert lib.gla_chunk_fwd_workspace_size(16, 1, 16, 33000, 128, 256, 64, 0) == 0
    assert lib.gla_chunk_fwd_workspace_size(0, 1, 16, 65536, 64, 64, 64, 1) == 0
    assert lib.gla_chunk_fwd_workspace_size(0, 1, 16, 256, 128, 128, 64, 0) == 0   # too short
    # 16 units of d_v 128 take the 128-column slice when split: 16 segments fill 256 CUs
    # (the CPU build reads no device and plans for 256), fp32 states plus decays per segment
    assert lib.gla_chunk_fwd_workspace_size(0, 1, 16, 65536, 128, 128, 64, 0) == \
        16 * 16 * (128 * 128 + 128) * 4


@pytest.mark.parametrize("ws,nbytes,needle", [
    (None, 0, "workspace of 0 bytes"),
    (FAKE, 1024, "needed"),
    (FAKE + 16, 1 << 30, "256-byte aligned"),
])
def test_chunk_fwd_ws_rejects_workspace(lib, ws, nbytes, needle):
    from sub_quadratic_sequence_amd import gla

    P = ctypes.c_void_p
    rc = lib.gla_chunk_fwd_ws(P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE), None, None, 0,
                              1, 16, 65536, 128, 128, 64, 0, P(ws) if ws else None, nbytes, None)
    assert rc == 1
    assert needle in gla.last_error()


def test_bwd_workspace_size(lib):
    lib.gla_chunk_bwd_workspace_size.restype = ctypes.c_size_t
    # training shape: 16 heads x (8 sequences + 16384 / 64 tokens + 1) chunk states of 128 x 128
    # bf16, plus the sequence split (128 units < 256 compute units: 2 segments per sequence):
    # fp32 state gradients and decays per (unit, segment)
    states = 16 * 265 * 128 * 128 * 2
    split = 128 * 2 * 128 * 128 * 4 + 128 * 2 * 128 * 4
    assert lib.gla_chunk_bwd_workspace_size(0, 8, 16, 2048, 128, 128, 64, 0) == states + split
    # enough units to fill the device: no split
    assert lib.gla_chunk_bwd_workspace_size(0, 16, 16, 2048, 128, 128, 64, 0) == 16 * 529 * 128 * 128 * 2
    # packed: 16 heads x (16 sequences + 33000 // 64 + 1) states of 128 x 64, rounded up to 256 bytes
    assert lib.gla_chunk_bwd_workspace_size(16, 1, 16, 33000, 128, 64, 64, 0) == 16 * 532 * 128 * 64 * 2
    assert lib.gla_chunk_bwd_workspace_size(0, 8, 16, 2048, 128, 128, 64, 1) == 0   # fp32
    # dv 256: states of 128 x 256, the split's state gradients, and the fp32 partial
    # sums of dq, dk and dg over the two 128-column slices
    states256 = 16 * 265 * 128 * 256 * 2
    split256 = 128 * 2 * 128 * 256 * 4 + 128 * 2 * 128 * 4
    partial = 3 * 16 * 8 * 2048 * 128 * 4
    assert lib.gla_chunk_bwd_workspace_size(0, 8, 16, 2048, 128, 256, 64, 0) == states256 + split256 + partial
    assert lib.gla_chunk_bwd_workspace_size(0, 8, 16, 2048, 128, 96, 64, 0) == 0    # dv not a multiple of 64
    assert lib.gla_chunk_bwd_workspace_size(0, 8, 16, 2048, 128, 128, 128, 0) == 0  # chunk 128


def _bwd(lib, **kw):
    P = ctypes.c_void_p
    a = dict(q=P(FAKE), k=P(FAKE), v=P(FAKE), g=P(FAKE), s0=None, do=P(FAKE), dsT=None,
             dq=P(FAKE), dk_=P(FAKE), dv_=P(FAKE), dg=P(FAKE), ds0=None, cu=None, num_seqs=0,
             B=2, H=4, T=256, dk=128, dv=128, chunk=64, dtype=0, ws=None, ws_bytes=0)
    a.update(kw)
    return lib.gla_chunk_bwd(a["q"], a["k"], a["v"], a["g"], a["s0"], a["do"], a["dsT"], a["dq"],
                             a["dk_"], a["dv_"], a["dg"], a["ds0"], a["cu"], a["num_seqs"], a["B"],
                             a["H"], a["T"], a["dk"], a["dv"], a["chunk"], a["dtype"], a["ws"],
                             a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=1), 2, "only GLA_BF16"),
    (dict(dtype=7), 1, "dtype 7"),
    (dict(dv=96), 2, "dk=128 dv=96"),
    (dict(dv=256), 1, "workspace of 0 bytes"),   # d_v 256 is accepted: it needs its workspace
    (dict(dk=96), 2, "dk=96"),
    (dict(chunk=128), 2, "chunk_size 128"),
    (dict(do=None), 1, "must be non-null"),
    (dict(dg=None), 1, "must be non-null"),
    (dict(cu=ctypes.c_void_p(FAKE), num_seqs=3), 1, "need B == 1"),
    (dict(dq=ctypes.c_void_p(FAKE + 8)), 1, "d_q is not 16-byte aligned"),
    (dict(), 1, "workspace of 0 bytes"),
    (dict(ws=ctypes.c_void_p(FAKE), ws_bytes=4096), 1, "needed"),
    (dict(ws=ctypes.c_void_p(FAKE + 16), ws_bytes=1 << 30), 1, "256-byte aligned"),
    (dict(B=1, H=1, T=1 << 23, dk=128, dv=128), 1, "too long"),
])
def test_chunk_bwd_rejects(lib, kw, status, needle):
    from sub_quadratic_sequence_amd import gla

    assert _bwd(lib, **kw) == status
    assert needle in gla.last_error(), gla.last_error()


def test_chunk_bwd_zero_tokens_without_state_gradient_is_a_noop(lib):
    assert _bwd(lib, T=0) == 0


def _gdn(lib, **kw):
    P = ctypes.c_void_p
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, s0=None, o=FAKE, sT=None, cu=None,
             num_seqs=0, B=1, H=2, T=64, dk=128, dv=128, C=64, dtype=0)
    a.update(kw)
    return lib.gdn_chunk_fwd(P(a["q"]), P(a["k"]), P(a["v"]), P(a["g"]), P(a["beta"]), P(a["s0"]),
                             P(a["o"]), P(a["sT"]), P(a["cu"]), a["num_seqs"], a["B"], a["H"],
                             a["T"], a["dk"], a["dv"], a["C"], a["dtype"], None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(beta=None), 1, "non-null"),
    (dict(g=None), 1, "non-null"),
    (dict(q=FAKE + 8), 1, "q is not 16-byte aligned"),
    (dict(g=FAKE + 2), 1, "4-byte aligned"),
    (dict(B=0), 1, "must be positive"),
    (dict(dtype=1), 2, "only GLA_BF16"),
    (dict(dtype=9), 1, "dtype 9"),
    (dict(C=32), 2, "chunk_size"),
    (dict(dk=256), 2, "dk=256"),
    (dict(dv=100), 2, "dv=100"),
    (dict(cu=FAKE, B=2, num_seqs=2), 1, "B == 1"),
    (dict(B=4096, H=4096, T=4096), 1, "int32"),
])
def test_gdn_chunk_fwd_rejects(lib, kw, status, needle):
    from sub_quadratic_sequence_amd import gla

    assert _gdn(lib, **kw) == status
    assert needle in gla.last_error(), gla.last_error()


def test_gdn_zero_tokens_without_outputs_is_a_noop(lib):
    assert _gdn(lib, q=None, k=None, v=None, g=None, beta=None, o=None, T=0) == 0


# ------------------------------------------------------------ sequence-split plan
def _model_constants(ns="split_model"):
    """The constexpr doubles of namespace `ns` in csrc/split_model.h."""
    text = open(os.path.join(ROOT, "sub_quadratic_sequence_amd", "csrc", "split_model.h")).read()
    body = re.search(r"namespace %s \{(.*?)\}  // namespace %s" % (ns, ns), text, re.S).group(1)
    return {m.group(1): float(m.group(2))
            for m in re.finditer(r"constexpr double (k\w+) = ([0-9.eE+-]+);", body)}


def _plan(lib, units, T, dv, dtype=0, ncu=256):
    seg = ctypes.c_int(-1)
    lib.gla_split_plan.restype = ctypes.c_int
    lib.gla_split_plan.argtypes = [ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    n = lib.gla_split_plan(units, T, dv, dtype, ncu, ctypes.byref(seg))
    return n, seg.value


def _model_best(c, units, T, dv, ncu):
    """The documented choice, by brute force: the unsplit time mu_1 N + mu_0 against
    lambda_1 L + lambda_2 segments + lambda_0 for every segment count whose work items
    fit one wave (ties keep fewer segments)."""
    nch = -(-T // 64)
    best_t, best = c["kMu1"] * nch + c["kMu0"], (1, T)
    items = units * (dv // 128 if dv % 128 == 0 else dv // 64)
    for n in range(2, nch + 1):
        if items * n > ncu:
            break
        L = -(-nch // n)
        ns = -(-nch // L)
        t = c["kLambda1"] * L + c["kLambda2"] * ns + c["kLambda0"]
        if t < best_t:
            best_t, best = t, (ns, L * 64)
    return best


@pytest.mark.parametrize("ncu", [256, 80])
def test_split_plan_minimises_the_model(lib, ncu):
    c = _model_constants()
    assert set(c) == {"kLambda1", "kLambda2", "kLambda0", "kMu1", "kMu0"}
    seen = set()
    for units in (1, 2, 3, 5, 8, 16, 24, 33, 64, 100):
        for T in (1, 63, 64, 65, 600, 1025, 2048, 4097, 16384, 65536, 100000):
            for dv in (64, 128, 192, 256):
                n, seg = _plan(lib, units, T, dv, ncu=ncu)
                if units * (dv // 64) >= ncu:
                    assert (n, seg) == (1, T)   # the unsplit call already fills the device
                    continue
                assert (n, seg) == _model_best(c, units, T, dv, ncu), (units, T, dv)
                if n > 1:
                    items = units * (dv // 128 if dv % 128 == 0 else dv // 64)
                    assert seg % 64 == 0 and (n - 1) * seg < T <= n * seg
                    assert items * n <= ncu
                seen.add(n > 1)
    assert seen == {True, False}   # the grid reaches both decisions


def test_split_plan_declines_what_it_cannot_split(lib):
    assert _plan(lib, 4, 65536, 128, dtype=1) == (1, 65536)   # fp32
    assert _plan(lib, 4, 0, 128) == (1, 0)
    assert _plan(lib, 0, 4096, 128) == (1, 4096)
    assert _plan(lib, 4, 4096, 96) == (1, 4096)   # d_v not a multiple of 64
    assert _plan(lib, 4, 4096, 128, ncu=0) == (1, 4096)
    # the plan behind the workspace size of gla_chunk_fwd_ws (the CPU build plans for 256 CUs)
    n, _ = _plan(lib, 16, 65536, 128)
    assert lib.gla_chunk_fwd_workspace_size(0, 1, 16, 65536, 128, 128, 64, 0) == \
        n * 16 * (128 * 128 + 128) * 4


# ------------------------------------------------------------ d_v slice plan
def _slice(lib, units, dv, dtype=0, ncu=256):
    lib.gla_slice_plan.restype = ctypes.c_int
    lib.gla_slice_plan.argtypes = [ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    return lib.gla_slice_plan(units, dv, dtype, ncu)


def _rounds(items, ncu, partial):
    """Rounds of ncu work items, a last partial round weighted partial + (1 - partial) x fill."""
    full, rem = divmod(items, ncu)
    return full + (partial + (1 - partial) * rem / ncu if rem else 0)


@pytest.mark.parametrize("ncu", [256, 80, 304])
def test_slice_plan_follows_the_model(lib, ncu):
    c = _model_constants("slice_model")
    assert set(c) == {"kWide", "kPartial"}
    seen = set()
    for units in list(range(1, 1200, 7)) + [ncu // 2, ncu, 3 * ncu // 2, 2 * ncu]:
        for dv in (128, 256, 384, 512):
            wide = units * dv // 128
            cost_wide = c["kWide"] * _rounds(wide, ncu, c["kPartial"])
            want = 128 if cost_wide < _rounds(2 * wide, ncu, c["kPartial"]) else 64
            assert _slice(lib, units, dv, ncu=ncu) == want, (units, dv, ncu)
            seen.add(want)
    assert seen == {64, 128}   # the grid reaches both decisions


def test_slice_plan_decisions_measured_on_mi355x(lib):
    # (units = B x H, dv) -> the faster width in the bf16 timings (d_k = 128, T = 512 .. 8192)
    # on one MI355X (256 CUs) that the constants were chosen on
    for units, dv, width in [(128, 128, 64),    # B8 H16, the training shape
                             (96, 128, 64), (192, 128, 128), (224, 128, 128), (256, 128, 128),
                             (288, 128, 64), (384, 128, 64), (448, 128, 128), (512, 128, 128),
                             (64, 256, 64), (96, 256, 128),
                             (256, 256, 128)]:  # 16 packed sequences x H16 at dv 256
        assert _slice(lib, units, dv) == width, (units, dv)


def test_slice_plan_declines_what_has_no_wide_kernel(lib):
    assert _slice(lib, 512, 128, dtype=1) == 64     # fp32
    assert _slice(lib, 512, 192) == 64              # dv not a multiple of 128
    assert _slice(lib, 512, 64) == 64
    assert _slice(lib, 0, 128) == 64 and _slice(lib, -5, 128) == 64
    assert _slice(lib, 512, 0) == 64 and _slice(lib, 512, 128, ncu=0) == 64


def test_segments_workspace_size(lib):
    lib.gla_chunk_fwd_segments_workspace_size.restype = ctypes.c_size_t
    f = lib.gla_chunk_fwd_segments_workspace_size
    def rnd(x):
        return -(-x // 256) * 256
    assert f(1, 4, 4096, 128, 128, 1) == 0
    assert f(1, 4, 4096, 128, 128, 7) == rnd(4 * 7 * 128 * 128 * 4) + rnd(4 * 7 * 128 * 4)
    # 13 requested segments of 64 chunks give L = 5 chunks, 13 segments; 60 give L = 2, 32
    assert f(2, 3, 4096, 64, 256, 13) == rnd(6 * 13 * 64 * 256 * 4) + rnd(6 * 13 * 64 * 4)
    assert f(2, 3, 4096, 64, 256, 60) == rnd(6 * 32 * 64 * 256 * 4) + rnd(6 * 32 * 64 * 4)
    assert f(1, 4, 4096, 128, 128, 0) == 0 and f(1, 4, 4096, 128, 128, 65) == 0


@pytest.mark.parametrize("kw,status,needle", [
    (dict(num_segments=0), 1, "num_segments = 0"),
    (dict(num_segments=65), 1, "must be in [1, 64]"),
    (dict(num_segments=4, dtype=1), 2, "bf16 inputs only"),
    (dict(num_segments=4), 1, "workspace of 0 bytes"),
    (dict(num_segments=4, ws=FAKE + 16, nbytes=1 << 30), 1, "256-byte aligned"),
    (dict(num_segments=4, T=-1), 1, ""),
])
def test_chunk_fwd_segments_rejects(lib, kw, status, needle):
    from sub_quadratic_sequence_amd import gla

    P = ctypes.c_void_p
    a = dict(B=1, H=4, T=4096, dtype=0, ws=None, nbytes=0)
    a.update(kw)
    rc = lib.gla_chunk_fwd_segments(P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE), None, a["B"],
                                    a["H"], a["T"], 128, 128, 64, a["dtype"], a["num_segments"],
                                    P(a["ws"]) if a["ws"] else None, a["nbytes"], None)
    assert rc == status
    assert needle in gla.last_error()


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dtype=1), 2, "bf16 path only"),
    (dict(dk=256), 2, "dk=256"),
    (dict(ws=None), 1, "chunk_states of 0 bytes"),
    (dict(nbytes=1024), 1, "needed"),
    (dict(ws=FAKE + 16), 1, "256-byte aligned"),
])
def test_chunk_fwd_states_rejects(lib, kw, status, needle):
    from sub_quadratic_sequence_amd import gla

    P = ctypes.c_void_p
    a = dict(dtype=0, dk=128, ws=FAKE, nbytes=1 << 30)
    a.update(kw)
    rc = lib.gla_chunk_fwd_states(P(FAKE), P(FAKE), P(FAKE), P(FAKE), None, P(FAKE), None, None, 0, 2,
                                  4, 256, a["dk"], 128, 64, a["dtype"], P(a["ws"]) if a["ws"] else None,
                                  a["nbytes"], None)
    assert rc == status
    assert needle in gla.last_error()


def test_chunk_bwd_saved_checks_like_chunk_bwd(lib):
    from sub_quadratic_sequence_amd import gla

    P = ctypes.c_void_p
    rc = lib.gla_chunk_bwd_saved(*([P(FAKE)] * 4), None, P(FAKE), None, *([P(FAKE)] * 4), None, None,
                                 0, 2, 4, 256, 128, 128, 64, 0, None, 0, None)
    assert rc == 1 and "gla_chunk_bwd_saved: workspace of 0 bytes" in gla.last_error()
