"""Pins for the fp64 Gated DeltaNet oracle (CPU only).

Each test checks the oracle against something other than itself: a closed form
(beta = 0; keys of an orthonormal basis with alpha = beta = 1), an identity the
delta rule must satisfy (exact retrieval: with beta_t |k_t|^2 = 1 the state
returns v_t for the query k_t, whatever alpha_t and the earlier state), a
brute-force product of explicit d_k x d_k transition matrices, and the pages'
chunkwise WY steps.  The last test plants plausible mistakes in a copy of the
recurrence and checks that the pins reject every one.
"""
import math

import numpy as np
import pytest

from gdn_chunk_fp64 import gdn_chunk_form

RNG = np.random.default_rng(2024)


def _case(T, dk, dv, rng=RNG, s0=False, gate="weak", l2=True):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if l2:
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    z = rng.standard_normal(T)
    g = -np.log1p(np.exp(-z)) / (16.0 if gate == "weak" else 1.0)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    S0 = 0.1 * rng.standard_normal((dk, dv)) if s0 else None
    f = lambda a: None if a is None else a.astype(np.float32).astype(np.float64)
    return f(q), f(k), f(v), f(g), f(beta), S0


def _run(oracle_mod, q, k, v, g, beta, s0=None):
    from oracle import gdn

    o, sf = gdn.recurrence(q[None, None], k[None, None], v[None, None], g[None, None],
                           beta[None, None], s0=None if s0 is None else s0[None, None])
    return o[0, 0], sf[0, 0]


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def unrolled_bruteforce(q, k, v, g, beta, s0=None):
    """S_t = A_t S_{t-1} + beta_t k_t^T v_t with the explicit transition matrix
    A_t = alpha_t (I - beta_t k_t^T k_t); S_t is formed as
    (prod_{m<=t} A_m) S_0 + sum_{j<=t} (prod_{j<m<=t} A_m) beta_j k_j^T v_j with
    every product of d_k x d_k matrices written out, and o_t = q_t S_t."""
    T, dk = q.shape
    dv = v.shape[1]
    S0 = np.zeros((dk, dv)) if s0 is None else s0
    A = [math.exp(g[t]) * (np.eye(dk) - beta[t] * np.outer(k[t], k[t])) for t in range(T)]
    o = np.zeros((T, dv))
    S = None
    for t in range(T):
        P = np.eye(dk)
        for m in range(t, -1, -1):
            P = P @ A[m]
        S = P @ S0
        for j in range(t + 1):
            P = np.eye(dk)
            for m in range(t, j, -1):
                P = P @ A[m]
            S = S + P @ (beta[j] * np.outer(k[j], v[j]))
        o[t] = q[t] @ S
    return o, S


def test_c_matches_numpy(oracle_mod):
    from oracle import gdn

    rng = np.random.default_rng(7)
    B, H, T, dk, dv = 2, 3, 41, 16, 24
    q = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    k = rng.standard_normal((B, H, T, dk)).astype(np.float32)
    v = rng.standard_normal((B, H, T, dv)).astype(np.float32)
    g = (-rng.random((B, H, T))).astype(np.float32)
    beta = rng.random((B, H, T)).astype(np.float32)
    s0 = rng.standard_normal((B, H, dk, dv))
    o, sf = gdn.recurrence(q, k, v, g, beta, s0)
    o2, sf2 = gdn.recurrence_numpy(q, k, v, g, beta, s0)
    assert _rel(o, o2) < 1e-13 and _rel(sf, sf2) < 1e-13


@pytest.mark.parametrize("s0", [False, True])
def test_unrolled_products(oracle_mod, s0):
    q, k, v, g, beta, S0 = _case(12, 6, 5, s0=s0, gate="strong", l2=False)
    o, sf = _run(oracle_mod, q, k, v, g, beta, S0)
    o_b, s_b = unrolled_bruteforce(q, k, v, g, beta, S0)
    assert _rel(o, o_b) < 1e-12 and _rel(sf, s_b) < 1e-12


def test_beta_zero_closed_form(oracle_mod):
    """beta = 0: S_t = gamma_t S_0 (gamma_t = exp(cumsum g)), o_t = gamma_t q_t S_0."""
    q, k, v, g, _, S0 = _case(40, 8, 8, s0=True)
    beta = np.zeros(40)
    o, sf = _run(oracle_mod, q, k, v, g, beta, S0)
    gam = np.exp(np.cumsum(g))
    assert _rel(o, gam[:, None] * (q @ S0)) < 1e-13
    assert _rel(sf, gam[-1] * S0) < 1e-13


@pytest.mark.parametrize("gate", ["weak", "strong"])
def test_exact_retrieval(oracle_mod, gate):
    """With beta_t = 1/|k_t|^2 the update makes k_t S_t = v_t exactly, for any
    alpha_t and any earlier state: querying with q_t = k_t returns v_t."""
    q, k, v, g, _, S0 = _case(64, 16, 12, s0=True, gate=gate, l2=False)
    beta = 1.0 / np.sum(k * k, axis=1)
    o, _ = _run(oracle_mod, k, k, v, g, beta.astype(np.float32).astype(np.float64), S0)
    # beta is rounded to float32 as the oracle reads it: allow that rounding
    assert _rel(o, v) < 1e-6


def test_orthonormal_keys_overwrite(oracle_mod):
    """alpha = beta = 1 and keys from the standard basis: the update replaces
    row i_t of S by v_t, so S_T holds, in each row, the value last written to
    it (S_0's row where none was), and o_t = q_t S_t."""
    rng = np.random.default_rng(3)
    T, dk, dv = 30, 5, 4
    idx = rng.integers(0, dk, T)
    k = np.eye(dk)[idx]
    q = rng.standard_normal((T, dk)).astype(np.float32).astype(np.float64)
    v = rng.standard_normal((T, dv)).astype(np.float32).astype(np.float64)
    S0 = rng.standard_normal((dk, dv))
    o, sf = _run(oracle_mod, q, k, v, np.zeros(T), np.ones(T), S0)
    S = S0.copy()
    for t in range(T):
        S[idx[t]] = v[t]
        assert np.allclose(o[t], q[t] @ S, rtol=0, atol=1e-12)
    assert np.allclose(sf, S, rtol=0, atol=1e-12)


@pytest.mark.parametrize("C", [1, 16, 64])
@pytest.mark.parametrize("gate", ["weak", "strong"])
def test_chunk_form(oracle_mod, C, gate):
    q, k, v, g, beta, S0 = _case(200, 32, 24, s0=True, gate=gate)
    o, sf = _run(oracle_mod, q, k, v, g, beta, S0)
    oc, sc = gdn_chunk_form(q, k, v, g, beta, C, S0)
    assert _rel(o, oc) < 1e-10 and _rel(sf, sc) < 1e-10


def test_packed_equals_separate(oracle_mod):
    from oracle import gdn

    rng = np.random.default_rng(11)
    lens = [5, 0, 70, 1, 33]
    Tt, H, dk, dv = sum(lens), 2, 8, 6
    q = rng.standard_normal((1, H, Tt, dk)).astype(np.float32)
    k = rng.standard_normal((1, H, Tt, dk)).astype(np.float32)
    v = rng.standard_normal((1, H, Tt, dv)).astype(np.float32)
    g = (-rng.random((1, H, Tt))).astype(np.float32)
    beta = rng.random((1, H, Tt)).astype(np.float32)
    s0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    o, sf = gdn.recurrence(q, k, v, g, beta, s0, cu_seqlens=cu)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        o1, s1 = gdn.recurrence(q[:, :, a:b], k[:, :, a:b], v[:, :, a:b], g[:, :, a:b],
                                beta[:, :, a:b], s0[n:n + 1])
        assert np.array_equal(o[:, :, a:b], o1) and np.array_equal(sf[n:n + 1], s1)


def test_decode_step_is_one_token(oracle_mod):
    from oracle import gdn

    rng = np.random.default_rng(5)
    N, H, dk, dv = 3, 2, 8, 8
    q, k = rng.standard_normal((2, N, H, dk)).astype(np.float32)
    v = rng.standard_normal((N, H, dv)).astype(np.float32)
    g = (-rng.random((N, H))).astype(np.float32)
    beta = rng.random((N, H)).astype(np.float32)
    st = rng.standard_normal((N, H, dk, dv))
    o, s1 = gdn.decode_step(q, k, v, g, beta, st)
    o2, s2 = gdn.recurrence_numpy(q[:, :, None], k[:, :, None], v[:, :, None], g[:, :, None],
                                  beta[:, :, None], st)
    assert _rel(o, o2[:, :, 0]) < 1e-13 and _rel(s1, s2) < 1e-13


# ---- planted mistakes: each must fail at least one pin ---------------------------------
def _buggy(kind):
    def rec(q, k, v, g, beta, s0=None):
        T, dk = q.shape
        dv = v.shape[1]
        S = np.zeros((dk, dv)) if s0 is None else s0.copy()
        o = np.zeros((T, dv))
        for t in range(T):
            a, b, kt = math.exp(g[t]), beta[t], k[t]
            Sp = S
            if kind == "decay_after_write":
                S = a * ((S - b * np.outer(kt, kt @ S)) + b * np.outer(kt, v[t]))
            elif kind == "erase_without_beta":
                S = a * (S - np.outer(kt, kt @ S)) + b * np.outer(kt, v[t])
            elif kind == "erase_sign":
                S = a * (S + b * np.outer(kt, kt @ S)) + b * np.outer(kt, v[t])
            elif kind == "write_without_beta":
                S = a * (S - b * np.outer(kt, kt @ S)) + np.outer(kt, v[t])
            elif kind == "no_decay_on_erase":
                S = a * S - b * np.outer(kt, kt @ S) + b * np.outer(kt, v[t])
            else:
                S = a * (S - b * np.outer(kt, kt @ S)) + b * np.outer(kt, v[t])
            o[t] = q[t] @ (Sp if kind == "exclusive" else S)
        return o, S
    return rec


@pytest.mark.parametrize("kind", ["decay_after_write", "erase_without_beta", "erase_sign",
                                  "write_without_beta", "no_decay_on_erase", "exclusive"])
def test_pins_reject_planted_mistakes(kind):
    rec = _buggy(kind)
    caught = False
    # exact retrieval
    q, k, v, g, _, S0 = _case(32, 8, 6, s0=True, gate="strong", l2=False)
    beta = 1.0 / np.sum(k * k, axis=1)
    o, _ = rec(k, k, v, g, beta, S0)
    caught |= _rel(o, v) > 1e-6
    # brute-force unrolled products
    q, k, v, g, beta, S0 = _case(10, 5, 4, s0=True, gate="strong", l2=False)
    o, s = rec(q, k, v, g, beta, S0)
    o_b, s_b = unrolled_bruteforce(q, k, v, g, beta, S0)
    caught |= _rel(o, o_b) > 1e-9 or _rel(s, s_b) > 1e-9
    assert caught, kind
    # the correct recurrence passes the same checks
    ok = _buggy("none")
    o, s = ok(q, k, v, g, beta, S0)
    assert _rel(o, o_b) < 1e-12 and _rel(s, s_b) < 1e-12
