"""Pins for the fp64 oracle: each test checks it against something other than
itself - a different formula from the pages, a closed form, exact rational
arithmetic, or an invariant - so a plausible mistake in the oracle (a dropped
term, a sign, an off-by-one between S_{t-1} and S_t, a transposed operand, the
gate applied to the wrong axis of S) fails at least one of them.  The last
test plants such mistakes in a copy of the recurrence and checks that the pins
reject every one.  CPU only.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from chunk_form_fp64 import chunk_form

RNG = np.random.default_rng(12345)


def _rand_case(T, dk, dv, gate="weak", rng=RNG, s0=False):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk)) / math.sqrt(dk)
    v = rng.standard_normal((T, dv))
    z = rng.standard_normal((T, dk))
    if gate == "weak":
        g = -np.log1p(np.exp(-z)) / 16.0
    elif gate == "strong":
        g = -np.log1p(np.exp(-(2 * z - 1)))
    else:
        raise ValueError(gate)
    S0 = 0.1 * rng.standard_normal((dk, dv)) if s0 else None
    # the oracle reads float32 values; round here so every side sees the same numbers
    f = lambda a: None if a is None else a.astype(np.float32).astype(np.float64)
    return f(q), f(k), f(v), f(g), (None if S0 is None else S0)


def _run_c(oracle_mod, q, k, v, g, s0=None):
    o, sf = oracle_mod.recurrence(q[None, None], k[None, None], v[None, None], g[None, None],
                                  s0=None if s0 is None else s0[None, None])
    return o[0, 0], sf[0, 0]


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --- (a) the unrolled dual form, by brute force --------------------------------------
def dual_form_bruteforce(q, k, v, g):
    """o_t = sum_{j<=t} ((q_t * k_j) . Lambda_{j,t}) v_j with
    Lambda_{j,t} = prod_{m=j+1}^{t} alpha_m (empty product = 1), and the unrolled
    state S_T = sum_j (prod_{m=j+1}^{T} diag alpha_m) k_j^T v_j (page "Gated
    Linear Attention (GLA) ...", section "The Gated Recurrent Update", the two
    equations after the recurrence).  Explicit products, no cumulative sums."""
    T, dk = q.shape
    dv = v.shape[1]
    alpha = np.exp(g)
    o = np.zeros((T, dv))
    for t in range(T):
        for j in range(t + 1):
            lam = np.ones(dk)
            for m in range(j + 1, t + 1):
                lam = lam * alpha[m]
            o[t] += np.sum(q[t] * k[j] * lam) * v[j]
    S = np.zeros((dk, dv))
    for j in range(T):
        lam = np.ones(dk)
        for m in range(j + 1, T):
            lam = lam * alpha[m]
        S += np.outer(lam * k[j], v[j])
    return o, S


@pytest.mark.parametrize("T,dk,dv,gate", [(1, 3, 2, "weak"), (7, 4, 3, "weak"),
                                          (24, 5, 4, "strong"), (19, 6, 5, "weak")])
def test_dual_form_bruteforce(oracle_mod, T, dk, dv, gate):
    q, k, v, g, _ = _rand_case(T, dk, dv, gate)
    o_ref, s_ref = dual_form_bruteforce(q, k, v, g)
    o_c, s_c = _run_c(oracle_mod, q, k, v, g)
    o_n, s_n = oracle_mod.recurrence_numpy(q, k, v, g)
    for o, s in ((o_c, s_c), (o_n, s_n)):
        assert _rel(o, o_ref) < 1e-12
        assert _rel(s, s_ref) < 1e-12


def test_dual_form_exact_rational(oracle_mod):
    """Exact rational arithmetic: alpha values are small fractions, inputs small
    integers; the dual form is evaluated with Fractions, so the expected value
    carries no rounding at all.  The oracle reads g = log(alpha) as float32, so
    each alpha carries a relative error of at most |g| 2^-24; the bound below is
    that error summed over the longest product, times the sum of |terms|."""
    T, dk, dv = 6, 3, 2
    alph = [[Fraction(1, 2), Fraction(3, 4), Fraction(1, 1)],
            [Fraction(1, 3), Fraction(1, 2), Fraction(7, 8)],
            [Fraction(5, 6), Fraction(1, 4), Fraction(1, 2)],
            [Fraction(1, 1), Fraction(2, 3), Fraction(3, 5)],
            [Fraction(1, 8), Fraction(9, 10), Fraction(1, 2)],
            [Fraction(2, 5), Fraction(1, 1), Fraction(1, 7)]]
    qi = [[1, -2, 3], [0, 1, -1], [2, 2, 1], [-1, 0, 4], [3, -1, 0], [1, 1, 1]]
    ki = [[2, 1, 0], [-1, 3, 1], [0, -2, 2], [1, 1, -3], [4, 0, 1], [-2, 1, 1]]
    vi = [[1, -1], [2, 0], [-3, 1], [0, 2], [1, 1], [-1, 3]]
    o_exact = [[Fraction(0)] * dv for _ in range(T)]
    o_abs = [[Fraction(0)] * dv for _ in range(T)]
    for t in range(T):
        for j in range(t + 1):
            w = Fraction(0)
            wa = Fraction(0)
            for c in range(dk):
                lam = Fraction(1)
                for m in range(j + 1, t + 1):
                    lam *= alph[m][c]
                w += qi[t][c] * ki[j][c] * lam
                wa += abs(qi[t][c] * ki[j][c]) * lam
            for e in range(dv):
                o_exact[t][e] += w * vi[j][e]
                o_abs[t][e] += wa * abs(vi[j][e])
    q = np.array(qi, float)
    k = np.array(ki, float)
    v = np.array(vi, float)
    g = np.log(np.array([[float(a) for a in row] for row in alph]))
    o_c, _ = _run_c(oracle_mod, q, k, v, g)
    ref = np.array([[float(x) for x in row] for row in o_exact])
    mag = np.array([[float(x) for x in row] for row in o_abs])
    g_err = T * float(np.max(np.abs(g))) * 2.0 ** -24 * 1.01
    assert np.all(np.abs(o_c - ref) <= g_err * mag + 1e-13 * np.max(np.abs(ref)))
    # first token: S_1 = k_1^T v_1 regardless of alpha_1 (S_0 = 0) -> o_1 = (q_1.k_1) v_1
    assert np.allclose(o_c[0], (q[0] @ k[0]) * v[0], rtol=0, atol=1e-15)


# --- (b) alpha == 1: vanilla linear attention ---------------------------------------
@pytest.mark.parametrize("T,dk,dv", [(33, 8, 8), (64, 16, 12)])
def test_alpha_one_is_linear_attention(oracle_mod, T, dk, dv):
    """g = 0 turns the recurrence into S_i = S_{i-1} + k_i^T v_i, O_i = q_i S_i
    (page 1, "Linearized Attention as Associative Memory"), whose closed form is
    O = (Q K^T masked to j <= i) V + Q S_0 and S_T = S_0 + K^T V."""
    q, k, v, _, s0 = _rand_case(T, dk, dv, s0=True)
    g = np.zeros_like(q)
    o_c, s_c = _run_c(oracle_mod, q, k, v, g, s0)
    mask = np.tril(np.ones((T, T)))
    o_ref = ((q @ k.T) * mask) @ v + q @ s0
    s_ref = s0 + k.T @ v
    assert _rel(o_c, o_ref) < 1e-12
    assert _rel(s_c, s_ref) < 1e-12


# --- (c) alpha == gamma: RetNet's fixed decay ---------------------------------------
@pytest.mark.parametrize("gamma", [0.9, 0.5])
def test_alpha_const_is_retnet(oracle_mod, gamma):
    """A fixed scalar decay gamma for every channel and token gives
    S_i = gamma S_{i-1} + k_i^T v_i (page 1, "The Retention and Recall
    Degradation Problem"), i.e. O = (Q K^T * D) V + diag(gamma^i) Q S_0 with
    D_ij = gamma^(i-j) for i >= j, and S_T = gamma^T S_0 + sum_j gamma^(T-j) k_j^T v_j
    (positions counted from 1)."""
    T, dk, dv = 40, 8, 6
    q, k, v, _, s0 = _rand_case(T, dk, dv, s0=True)
    g = np.full_like(q, np.float32(np.log(gamma)))
    gamma = float(np.exp(np.float64(g[0, 0])))   # the decay the float32 gate encodes
    o_c, s_c = _run_c(oracle_mod, q, k, v, g, s0)
    i = np.arange(1, T + 1)
    D = np.where(i[:, None] >= i[None, :], gamma ** (i[:, None] - i[None, :]).astype(float), 0.0)
    o_ref = ((q @ k.T) * D) @ v + (gamma ** i)[:, None] * (q @ s0)
    s_ref = gamma ** T * s0 + (k * (gamma ** (T - i))[:, None]).T @ v
    assert _rel(o_c, o_ref) < 1e-12
    assert _rel(s_c, s_ref) < 1e-12


# --- (d) chunked vs step-wise -------------------------------------------------------
@pytest.mark.parametrize("C", [1, 16, 64, 128])
@pytest.mark.parametrize("gate,T", [("weak", 200), ("strong", 150)])
def test_chunk_form_equals_recurrence(oracle_mod, C, gate, T):
    """The chunk equations of page 1 reproduce the recurrence exactly (up to
    fp64 rounding) for any chunk size, including a short last chunk and the
    strong gates whose in-chunk cumulative decay reaches about -150."""
    q, k, v, g, s0 = _rand_case(T, 16, 8, gate, s0=True)
    o_ch, s_ch = chunk_form(q, k, v, g, C, s0)
    o_c, s_c = _run_c(oracle_mod, q, k, v, g, s0)
    assert _rel(o_c, o_ch) < 1e-11
    assert _rel(s_c, s_ch) < 1e-11


# --- initial state -------------------------------------------------------------------
def test_initial_state_superposition(oracle_mod):
    """The recurrence is linear in S_0: O(S_0) - O(0) = (Q * exp(cumsum g)) S_0 and
    S_T(S_0) - S_T(0) = diag(exp(sum_t g_t)) S_0 (S_0 decays from the first token)."""
    T, dk, dv = 50, 8, 6
    q, k, v, g, s0 = _rand_case(T, dk, dv, s0=True)
    o1, s1 = _run_c(oracle_mod, q, k, v, g, s0)
    o0, s_0 = _run_c(oracle_mod, q, k, v, g, None)
    G = np.cumsum(g, axis=0)
    assert np.allclose(o1 - o0, (q * np.exp(G)) @ s0, rtol=1e-11, atol=1e-13)
    assert np.allclose(s1 - s_0, np.exp(G[-1])[:, None] * s0, rtol=1e-11, atol=1e-13)


def test_split_call_composition(oracle_mod):
    """Running [0, T1) and then [T1, T) from the first call's final state equals one
    call over [0, T): the state is the whole memory of the sequence."""
    T, T1 = 97, 41
    q, k, v, g, s0 = _rand_case(T, 8, 8, "strong", s0=True)
    o, s = _run_c(oracle_mod, q, k, v, g, s0)
    oa, sa = _run_c(oracle_mod, q[:T1], k[:T1], v[:T1], g[:T1], s0)
    ob, sb = _run_c(oracle_mod, q[T1:], k[T1:], v[T1:], g[T1:], sa)
    assert np.array_equal(np.concatenate([oa, ob]), o)
    assert np.array_equal(sb, s)


def test_varlen_equals_separate_calls(oracle_mod):
    lengths = [5, 1, 17, 0, 9]
    H, dk, dv = 2, 4, 3
    rng = np.random.default_rng(7)
    parts = [[_rand_case(L, dk, dv, "strong", rng, s0=True) for _ in range(H)] for L in lengths]
    Ttot = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    Q = np.zeros((1, H, Ttot, dk)); K = np.zeros_like(Q); G = np.zeros_like(Q)
    V = np.zeros((1, H, Ttot, dv)); S0 = np.zeros((len(lengths), H, dk, dv))
    for n, L in enumerate(lengths):
        for h in range(H):
            q, k, v, g, s0 = parts[n][h]
            Q[0, h, cu[n]:cu[n + 1]] = q; K[0, h, cu[n]:cu[n + 1]] = k
            G[0, h, cu[n]:cu[n + 1]] = g; V[0, h, cu[n]:cu[n + 1]] = v
            S0[n, h] = s0
    o, sf = oracle_mod.recurrence(Q, K, V, G, s0=S0, cu_seqlens=cu)
    for n, L in enumerate(lengths):
        for h in range(H):
            q, k, v, g, s0 = parts[n][h]
            if L == 0:
                assert np.array_equal(sf[n, h], S0[n, h])   # empty sequence: state passes through
                continue
            o1, s1 = _run_c(oracle_mod, q, k, v, g, S0[n, h])
            assert np.array_equal(o[0, h, cu[n]:cu[n + 1]], o1)
            assert np.array_equal(sf[n, h], s1)


def test_decode_step_is_one_token(oracle_mod):
    rng = np.random.default_rng(3)
    N, H, dk, dv = 3, 2, 8, 5
    q = rng.standard_normal((N, H, dk)).astype(np.float32)
    k = rng.standard_normal((N, H, dk)).astype(np.float32)
    v = rng.standard_normal((N, H, dv)).astype(np.float32)
    g = (-np.abs(rng.standard_normal((N, H, dk))) / 4).astype(np.float32)
    S = rng.standard_normal((N, H, dk, dv))
    o, S1 = oracle_mod.decode_step(q, k, v, g, S)
    a = np.exp(g.astype(np.float64))
    S_ref = a[..., None] * S + k.astype(np.float64)[..., None] * v.astype(np.float64)[..., None, :]
    o_ref = np.einsum("nhc,nhcj->nhj", q.astype(np.float64), S_ref)
    assert _rel(S1, S_ref) < 1e-14 and _rel(o, o_ref) < 1e-13


def test_c_and_numpy_agree_batched(oracle_mod):
    rng = np.random.default_rng(11)
    B, H, T, dk, dv = 2, 3, 70, 16, 24
    q = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    g = (-np.abs(rng.standard_normal((B, H, T, dk)))).astype(np.float32)
    s0 = rng.standard_normal((B, H, dk, dv))
    o_c, s_c = oracle_mod.recurrence(q, k, v, g, s0=s0, nthreads=3)
    o_n, s_n = oracle_mod.recurrence_numpy(q, k, v, g, s0)
    assert _rel(o_c, o_n) < 1e-12 and _rel(s_c, s_n) < 1e-12


def test_long_sequence_stays_bounded(oracle_mod):
    """With alpha in (0, 1) the transition has spectral radius below 1 (page 1,
    "Context Length Extrapolation"): every entry obeys
    |S_t| <= |S_0| + max|k v^T| / (1 - alpha_max), at any length."""
    rng = np.random.default_rng(5)
    T, dk, dv = 65536, 8, 8
    q = rng.standard_normal((1, 1, T, dk)).astype(np.float32)
    k = rng.standard_normal((1, 1, T, dk)).astype(np.float32)
    v = rng.standard_normal((1, 1, T, dv)).astype(np.float32)
    z = rng.standard_normal((1, 1, T, dk))
    g = (-np.log1p(np.exp(-z)) / 16).astype(np.float32)
    s0 = 0.1 * rng.standard_normal((1, 1, dk, dv))
    o, sf = oracle_mod.recurrence(q, k, v, g, s0=s0)
    a_max = float(np.exp(g.astype(np.float64)).max())
    kv_max = float(np.abs(k).max()) * float(np.abs(v).max())
    bound = np.abs(s0).max() + kv_max / (1 - a_max)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(sf))
    assert np.abs(sf).max() <= bound
    assert np.abs(o).max() <= np.abs(q).max() * dk * bound


# --- sensitivity: planted mistakes must fail the pins -------------------------------
def _mutant(kind, q, k, v, g, s0=None):
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else s0.copy()
    o = np.zeros((T, dv))
    for t in range(T):
        a = np.exp(g[t])
        if kind == "exclusive":           # o_t from S_{t-1}
            o[t] = q[t] @ S
        if kind == "sign":                # exp(-g)
            a = np.exp(-g[t])
        if kind == "gate_on_columns":     # diag(alpha) applied on the d_v side
            S = S * a[None, :dv] + np.outer(k[t], v[t])
        elif kind == "dropped_kv":
            S = a[:, None] * S + (np.outer(k[t], v[t]) if t > 0 else 0)
        elif kind == "transposed":        # k^T v replaced by v^T k (square case)
            S = a[:, None] * S + np.outer(v[t], k[t])
        elif kind == "decay_after_add":   # diag(alpha)(S + k^T v)
            S = a[:, None] * (S + np.outer(k[t], v[t]))
        else:
            S = a[:, None] * S + np.outer(k[t], v[t])
        if kind != "exclusive":
            o[t] = q[t] @ S
    return o, S


@pytest.mark.parametrize("kind", ["exclusive", "sign", "gate_on_columns", "dropped_kv",
                                  "transposed", "decay_after_add"])
def test_pins_reject_planted_mistakes(kind):
    q, k, v, g, _ = _rand_case(12, 6, 6, "strong", rng=np.random.default_rng(99))
    o_ref, s_ref = dual_form_bruteforce(q, k, v, g)
    o_m, s_m = _mutant(kind, q, k, v, g)
    assert _rel(o_m, o_ref) > 1e-3 or _rel(s_m, s_ref) > 1e-3
    o_ok, s_ok = _mutant("none", q, k, v, g)
    assert _rel(o_ok, o_ref) < 1e-12 and _rel(s_ok, s_ref) < 1e-12


# --- golden worked example --------------------------------------------------------
def test_golden_tiny_recurrence(oracle_mod):
    """tests/golden/tiny_recurrence.json (written by make_golden.py from the
    oracle) must still match the oracle, and its first two tokens must match the
    hand-expanded recurrence: o_1 = (q_1.k_1) v_1 + q_1 diag(alpha_1) S_0 and
    o_2 = q_2 (diag(alpha_2)(diag(alpha_1) S_0 + k_1^T v_1) + k_2^T v_2)."""
    import json
    import os

    with open(os.path.join(os.path.dirname(__file__), "golden", "tiny_recurrence.json")) as f:
        gold = json.load(f)
    g = np.array(gold["g_float32"], dtype=np.float32)
    q, k, v = (np.array(gold[n], dtype=np.float32) for n in ("q", "k", "v"))
    s0 = np.array(gold["s0"])
    a = np.exp(g.astype(np.float64))
    for name, s in (("zero_state", None), ("with_state", s0)):
        o, sf = _run_c(oracle_mod, q, k, v, g, s)
        case = gold["cases"][name]
        assert np.allclose(o, case["o"], rtol=1e-14, atol=0)
        assert np.allclose(sf, case["s_final"], rtol=1e-14, atol=0)
        S = np.zeros((2, 3)) if s is None else s
        S1 = a[0][:, None] * S + np.outer(k[0], v[0])
        S2 = a[1][:, None] * S1 + np.outer(k[1], v[1])
        assert np.allclose(case["o"][0], q[0] @ S1, rtol=1e-14, atol=1e-15)
        assert np.allclose(case["o"][1], q[1] @ S2, rtol=1e-14, atol=1e-15)
