"""Property tests of the fp64 oracle on random tiny shapes and gates (hypothesis,
derandomized so the CPU suite is repeatable): the C token recurrence against
the unrolled dual form computed by brute force, the chunk form at any chunk
length, split-call composition, linearity in v and in the initial state, and
packed sequences against separate calls.  Gates range from none (alpha = 1)
through the weak and strong recipes to decays of 2^-60 per token and alpha = 0
tokens.  CPU only."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from chunk_form_fp64 import chunk_form
from test_oracle_pins import _rel, _run_c, dual_form_bruteforce

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.function_scoped_fixture, HealthCheck.too_slow])


def _f32(a):
    return a.astype(np.float32).astype(np.float64)


def _case(seed, T, dk, dv, gate, s0=True, alpha_zero=False):
    """q, k, v, log-gates (rounded through fp32, as the oracle reads them) and S0."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk)) / np.sqrt(dk)
    v = rng.standard_normal((T, dv))
    z = rng.standard_normal((T, dk))
    if gate == "none":
        g = np.zeros((T, dk))
    elif gate == "weak":
        g = -np.log1p(np.exp(-z)) / 16.0
    elif gate == "strong":
        g = -np.log1p(np.exp(-(2 * z - 1)))
    else:   # "steep": per-token decays down to 2^-60
        g = -rng.uniform(0.0, 60.0 * np.log(2.0), (T, dk))
    if alpha_zero and T > 1:
        g[rng.integers(0, T), rng.integers(0, dk)] = -np.inf
    S0 = 0.1 * rng.standard_normal((dk, dv)) if s0 else None
    return _f32(q), _f32(k), _f32(v), _f32(g), S0


shapes = st.tuples(st.integers(0, 2**31 - 1), st.integers(1, 20), st.integers(1, 6), st.integers(1, 5),
                   st.sampled_from(["none", "weak", "strong", "steep"]))


@SETTINGS
@given(shapes, st.booleans())
def test_recurrence_equals_dual_form(oracle_mod, shape, alpha_zero):
    seed, T, dk, dv, gate = shape
    q, k, v, g, _ = _case(seed, T, dk, dv, gate, s0=False, alpha_zero=alpha_zero)
    o_c, s_c = _run_c(oracle_mod, q, k, v, g)
    o_d, s_d = dual_form_bruteforce(q, k, v, g)
    assert np.allclose(o_c, o_d, rtol=1e-11, atol=1e-12 * max(1.0, np.abs(o_d).max()))
    assert np.allclose(s_c, s_d, rtol=1e-11, atol=1e-12 * max(1.0, np.abs(s_d).max()))


@SETTINGS
@given(shapes, st.sampled_from([1, 2, 3, 5, 8, 16, 64]))
def test_chunk_form_equals_recurrence(oracle_mod, shape, C):
    seed, T, dk, dv, gate = shape
    q, k, v, g, s0 = _case(seed, T, dk, dv, gate)
    o_ch, s_ch = chunk_form(q, k, v, g, C, s0)
    o_c, s_c = _run_c(oracle_mod, q, k, v, g, s0)
    assert _rel(o_c, o_ch) < 1e-10
    assert _rel(s_c, s_ch) < 1e-10


@SETTINGS
@given(shapes, st.integers(0, 20))
def test_split_call_composition(oracle_mod, shape, cut):
    seed, T, dk, dv, gate = shape
    cut = min(cut, T)
    q, k, v, g, s0 = _case(seed, T, dk, dv, gate)
    o, s = _run_c(oracle_mod, q, k, v, g, s0)
    if cut == 0:
        oa, sa = np.zeros((0, dv)), s0
    else:
        oa, sa = _run_c(oracle_mod, q[:cut], k[:cut], v[:cut], g[:cut], s0)
    if cut == T:
        ob, sb = np.zeros((0, dv)), sa
    else:
        ob, sb = _run_c(oracle_mod, q[cut:], k[cut:], v[cut:], g[cut:], sa)
    assert np.array_equal(np.concatenate([oa, ob]), o)
    assert np.array_equal(sb, s)


@SETTINGS
@given(shapes)
def test_linear_in_values_and_initial_state(oracle_mod, shape):
    """O and S_T are linear in (V, S_0) jointly for fixed q, k, g.  V and S_0 are
    small dyadic rationals, so that a V1 + b V2 is exact in the fp32 the oracle
    reads its inputs in."""
    seed, T, dk, dv, gate = shape
    q, k, _, g, _ = _case(seed, T, dk, dv, gate)
    rng = np.random.default_rng(seed + 1)
    v1, v2 = (rng.integers(-8, 9, (T, dv)) / 8.0 for _ in range(2))
    s1, s2 = (rng.integers(-8, 9, (dk, dv)) / 64.0 for _ in range(2))
    a, b = 0.75, -1.25
    o1, t1 = _run_c(oracle_mod, q, k, v1, g, s1)
    o2, t2 = _run_c(oracle_mod, q, k, v2, g, s2)
    o3, t3 = _run_c(oracle_mod, q, k, a * v1 + b * v2, g, a * s1 + b * s2)
    scale_o = max(1.0, np.abs(o1).max(), np.abs(o2).max())
    scale_s = max(1.0, np.abs(t1).max(), np.abs(t2).max())
    assert np.allclose(o3, a * o1 + b * o2, rtol=0, atol=1e-12 * scale_o)
    assert np.allclose(t3, a * t1 + b * t2, rtol=0, atol=1e-12 * scale_s)


@SETTINGS
@given(st.integers(0, 2**31 - 1), st.lists(st.integers(0, 9), min_size=1, max_size=5),
       st.integers(1, 3), st.sampled_from(["weak", "strong", "steep"]))
def test_packed_sequences_equal_separate_calls(oracle_mod, seed, lengths, H, gate):
    dk, dv = 3, 2
    parts = [[_case(seed + 7 * n + h, L, dk, dv, gate) if L else None for h in range(H)]
             for n, L in enumerate(lengths)]
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    Ttot = int(cu[-1])
    Q = np.zeros((1, H, Ttot, dk)); K = np.zeros_like(Q); G = np.zeros_like(Q)
    V = np.zeros((1, H, Ttot, dv))
    S0 = 0.1 * rng.standard_normal((len(lengths), H, dk, dv))
    for n in range(len(lengths)):
        for h in range(H):
            if parts[n][h] is None:
                continue
            q, k, v, g, _ = parts[n][h]
            sl = slice(cu[n], cu[n + 1])
            Q[0, h, sl], K[0, h, sl], V[0, h, sl], G[0, h, sl] = q, k, v, g
    o, sf = oracle_mod.recurrence(Q, K, V, G, s0=S0, cu_seqlens=cu)
    for n, L in enumerate(lengths):
        for h in range(H):
            if L == 0:
                assert np.array_equal(sf[n, h], S0[n, h])
                continue
            q, k, v, g, _ = parts[n][h]
            o1, s1 = _run_c(oracle_mod, q, k, v, g, S0[n, h])
            assert np.array_equal(o[0, h, cu[n]:cu[n + 1]], o1)
            assert np.array_equal(sf[n, h], s1)
