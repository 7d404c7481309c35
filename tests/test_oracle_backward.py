"""Pins for the fp64 backward oracle (``oracle.backward``), CPU only.

The oracle differentiates the token recurrence with autograd.  These tests tie
it to things other than itself:
  * central finite differences of the loss computed by the (separately pinned)
    NumPy recurrence;
  * a brute-force gradient of the unrolled dual form of the page "Gated Linear
    Attention (GLA): Mathematical Foundations ...", section "The Gated
    Recurrent Update" (o_t as a decay-weighted sum over earlier tokens),
    differentiated by hand pair by pair;
  * the alpha = 1 case, where the recurrence is causal linear attention and the
    gradients are plain masked matrix products;
  * the gate-gradient identity dg_t = sum_{s>=t} (q_s*dq_s - k_s*dk_s) plus the
    final-state term, which follows from q and k entering only through
    q*exp(Gamma) and k*exp(-Gamma);
  * packed sequences equal separate calls.
A planted-mistake test checks that these pins reject plausible errors.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import backward as OB

RNG = np.random.default_rng(1234)


def _case(T, dk, dv, gate="weak", s0=True, dsT=True, rng=RNG, U=2):
    q = rng.standard_normal((1, U, T, dk))
    k = rng.standard_normal((1, U, T, dk)) * 0.5
    v = rng.standard_normal((1, U, T, dv))
    z = rng.standard_normal((1, U, T, dk))
    if gate == "weak":
        g = -np.log1p(np.exp(-z)) / 16
    elif gate == "strong":
        g = -np.log1p(np.exp(-(2 * z - 1)))
    else:
        g = np.zeros_like(z)
    do = rng.standard_normal((1, U, T, dv))
    S0 = rng.standard_normal((1, U, dk, dv)) * 0.3 if s0 else None
    dS = rng.standard_normal((1, U, dk, dv)) * 0.3 if dsT else None
    t = lambda a: None if a is None else torch.from_numpy(a)
    return dict(q=t(q), k=t(k), v=t(v), g=t(g), do=t(do), s0=t(S0), dsT=t(dS))


def _loss_numpy(q, k, v, g, do, s0, dsT):
    o, S = oracle.recurrence_numpy(q, k, v, g, s0)
    L = float((o * do).sum())
    if dsT is not None:
        L += float((S * dsT).sum())
    return L


def _grads(c):
    return OB.backward(c["q"], c["k"], c["v"], c["g"], c["do"], c["s0"], c["dsT"])


def _rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


@pytest.mark.parametrize("gate", ["weak", "strong"])
def test_finite_differences(gate):
    rng = np.random.default_rng(7)
    c = _case(6, 3, 2, gate=gate, rng=rng, U=1)
    dq, dk, dv, dg, ds0 = _grads(c)
    arrs = {n: c[n].numpy().copy() for n in ("q", "k", "v", "g", "s0")}
    fixed = dict(do=c["do"].numpy(), dsT=c["dsT"].numpy())
    h = 1e-6
    for name, grad in (("q", dq), ("k", dk), ("v", dv), ("g", dg), ("s0", ds0)):
        x = arrs[name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss_numpy(arrs["q"], arrs["k"], arrs["v"], arrs["g"], fixed["do"], arrs["s0"], fixed["dsT"])
            x[idx] = old - h
            lm = _loss_numpy(arrs["q"], arrs["k"], arrs["v"], arrs["g"], fixed["do"], arrs["s0"], fixed["dsT"])
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        assert _rel(grad.numpy(), fd) < 1e-7, (name, _rel(grad.numpy(), fd))


def dual_form_gradients(q, k, v, g, do, s0, dsT):
    """Gradients of L = sum_i <dO_i, o_i> + <dS_T, S_T> from the unrolled form
        o_i = sum_{j<=i} sum_c q_ic k_jc exp(G_ic - G_jc) v_j + sum_c q_ic exp(G_ic) S0_c,
        S_T = sum_j diag(exp(G_T - G_j)) k_j^T v_j + diag(exp(G_T)) S0,
    with G_i = sum_{m<=i} g_m, differentiated by hand one pair (i, j) at a time.
    One unit: q,k,g [T,dk]; v,do [T,dv]; s0, dsT [dk,dv]."""
    T, dk = q.shape
    dv = v.shape[1]
    G = np.cumsum(g, axis=0)
    GT = G[-1]
    s0 = np.zeros((dk, dv)) if s0 is None else s0
    dsT = np.zeros((dk, dv)) if dsT is None else dsT
    dq = np.zeros((T, dk)); dkk = np.zeros((T, dk)); dvv = np.zeros((T, dv))
    dg = np.zeros((T, dk)); ds0 = np.zeros((dk, dv))
    ST = np.exp(GT)[:, None] * s0
    for j in range(T):
        ST += np.exp(GT - G[j])[:, None] * np.outer(k[j], v[j])
    for i in range(T):
        for j in range(i + 1):
            E = np.exp(G[i] - G[j])                     # per channel
            a = float(v[j] @ do[i])
            dq[i] += k[j] * E * a
            dkk[j] += q[i] * E * a
            dvv[j] += float((q[i] * k[j] * E).sum()) * do[i]
            for t in range(j + 1, i + 1):               # j < t <= i
                dg[t] += q[i] * k[j] * E * a
        eS = np.exp(G[i])
        dq[i] += eS * (s0 @ do[i])
        ds0 += np.outer(q[i] * eS, do[i])
        for t in range(i + 1):                          # t <= i
            dg[t] += q[i] * eS * (s0 @ do[i])
    for j in range(T):
        F = np.exp(GT - G[j])
        dkk[j] += F * (dsT @ v[j])
        dvv[j] += (k[j] * F) @ dsT
        for t in range(j + 1, T):                       # j < t <= T
            dg[t] += F * k[j] * (dsT @ v[j])
    ds0 += np.exp(GT)[:, None] * dsT
    dg += (np.exp(GT) * (dsT * s0).sum(1))[None, :]     # every g_t enters G_T
    return dq, dkk, dvv, dg, ds0, ST


@pytest.mark.parametrize("T,dk,dv,gate", [(1, 3, 2, "weak"), (9, 4, 3, "strong"),
                                          (16, 5, 4, "weak"), (13, 3, 5, "strong")])
def test_dual_form_gradient_bruteforce(T, dk, dv, gate):
    c = _case(T, dk, dv, gate=gate)
    got = _grads(c)
    for u in range(2):
        ref = dual_form_gradients(*(c[n][0, u].numpy() for n in ("q", "k", "v", "g", "do")),
                                  c["s0"][0, u].numpy(), c["dsT"][0, u].numpy())
        for name, a, b in zip(("dq", "dk", "dv", "dg"), got[:4], ref[:4]):
            assert _rel(a[0, u].numpy(), b) < 1e-12, (name, u, _rel(a[0, u].numpy(), b))
        assert _rel(got[4][0, u].numpy(), ref[4]) < 1e-12


@pytest.mark.parametrize("s0", [False, True])
def test_alpha_one_is_linear_attention(s0):
    c = _case(24, 6, 5, gate="zero", s0=s0)
    dq, dk, dv, dg, ds0 = _grads(c)
    Q, K, V, dO = (c[n][0].numpy() for n in ("q", "k", "v", "do"))
    dS = c["dsT"][0].numpy()
    M = np.tril(np.ones((24, 24)))
    for u in range(2):
        A = (dO[u] @ V[u].T) * M                       # dO_i . v_j for j <= i
        P = (Q[u] @ K[u].T) * M
        eq = A @ K[u]
        ek = A.T @ Q[u] + V[u] @ dS[u].T
        ev = P.T @ dO[u] + K[u] @ dS[u]
        if s0:
            S0 = c["s0"][0, u].numpy()
            eq = eq + dO[u] @ S0.T
            assert _rel(ds0[0, u].numpy(), Q[u].T @ dO[u] + dS[u]) < 1e-12
        assert _rel(dq[0, u].numpy(), eq) < 1e-12
        assert _rel(dk[0, u].numpy(), ek) < 1e-12
        assert _rel(dv[0, u].numpy(), ev) < 1e-12


@pytest.mark.parametrize("gate", ["weak", "strong"])
def test_gate_gradient_identity(gate):
    c = _case(40, 8, 6, gate=gate)
    dq, dk, dv, dg, ds0 = _grads(c)
    _, ST = oracle.recurrence_numpy(c["q"].numpy(), c["k"].numpy(), c["v"].numpy(),
                                    c["g"].numpy(), c["s0"].numpy())
    x = (c["q"] * dq - c["k"] * dk).numpy()
    rev = np.flip(np.cumsum(np.flip(x, axis=2), axis=2), axis=2)
    rev = rev + (c["dsT"].numpy() * ST).sum(-1)[:, :, None, :]
    assert _rel(dg.numpy(), rev) < 1e-12


def test_varlen_equals_separate_calls():
    rng = np.random.default_rng(3)
    lens = [5, 0, 17, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    Tt = int(cu[-1])
    c = _case(Tt, 4, 3, gate="strong", rng=rng)
    s0 = torch.from_numpy(rng.standard_normal((4, 2, 4, 3)) * 0.3)
    dsT = torch.from_numpy(rng.standard_normal((4, 2, 4, 3)) * 0.3)
    got = OB.backward(c["q"], c["k"], c["v"], c["g"], c["do"], s0, dsT, cu_seqlens=torch.from_numpy(cu))
    for n in range(4):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = lambda x: x[:, :, a:b]
        ref = OB.backward(sl(c["q"]), sl(c["k"]), sl(c["v"]), sl(c["g"]), sl(c["do"]),
                          s0[n:n + 1], dsT[n:n + 1])
        for x, y in zip(got[:4], ref[:4]):
            assert torch.equal(sl(x), y)
        assert torch.equal(got[4][n:n + 1], ref[4])
    assert torch.equal(got[4][1], dsT[1])           # empty sequence: dS0 = dS_T


def test_unit_subset_matches_full():
    c = _case(20, 4, 4, gate="weak")
    full = _grads(c)
    part = OB.backward(c["q"], c["k"], c["v"], c["g"], c["do"], c["s0"], c["dsT"], units=[(0, 1)])
    for x, y in zip(full, part):
        assert torch.equal(x[0, 1], y[0, 1])
        assert torch.isnan(y[0, 0]).all()


# --------------------------------------------------------------- planted mistakes
def _mutant_grads(kind, c):
    """The oracle's autograd recipe with one plausible mistake planted."""
    q, k, v, g, do = (c[n][0].clone().requires_grad_(True) for n in ("q", "k", "v", "g", "do"))
    s0 = c["s0"][0].clone().requires_grad_(True)
    dsT = c["dsT"][0]
    S = s0
    loss = 0.0
    for t in range(q.shape[1]):
        a = torch.exp(-g[:, t] if kind == "gate_sign" else g[:, t])
        S_new = a[:, :, None] * S + k[:, t, :, None] * v[:, t, None, :]
        o = torch.einsum("uc,ucn->un", q[:, t], S if kind == "exclusive" else S_new)
        S = S_new
        loss = loss + (o * do[:, t]).sum()
    if kind != "drop_final":
        loss = loss + (S * dsT).sum()
    return torch.autograd.grad(loss, [q, k, v, g, s0])


@pytest.mark.parametrize("kind", ["exclusive", "gate_sign", "drop_final"])
def test_pins_reject_planted_mistakes(kind):
    c = _case(10, 4, 3, gate="strong")
    bad = _mutant_grads(kind, c)
    worst = 0.0
    for u in range(2):
        ref = dual_form_gradients(*(c[n][0, u].numpy() for n in ("q", "k", "v", "g", "do")),
                                  c["s0"][0, u].numpy(), c["dsT"][0, u].numpy())
        for a, b in zip(bad, ref):
            worst = max(worst, _rel(a[u].detach().numpy(), b))
    assert worst > 1e-3, (kind, worst)
