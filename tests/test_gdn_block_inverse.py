"""The Gated DeltaNet forward inverts each 16 x 16 unit lower triangular
diagonal block I + L of M through the nilpotent factorisation
(I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8), evaluated in fp32 (L^16 = 0 for
a strictly lower 16 x 16 L).  These CPU tests pin that identity and its fp32
accuracy against an exact inverse, with L built as in the chunk form
(L = diag(beta) strict_lower(Gamma * K K^T)), in NumPy.  They test the method,
not the kernel (the GPU tests compare the kernel with the oracle)."""
import numpy as np
import pytest


def _factorised(L, dtype):
    L = L.astype(dtype)
    eye = np.eye(L.shape[0], dtype=dtype)
    L2 = L @ L
    L4 = L2 @ L2
    L8 = L4 @ L4
    return ((eye - L) @ (eye + L2)) @ ((eye + L4) @ (eye + L8))


def _block(K, beta, g):
    gam = np.cumsum(g)
    decay = np.exp(gam[:, None] - gam[None, :])
    return np.tril(beta[:, None] * decay * (K @ K.T), -1)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rel(a, b):
    return np.abs(a - b).max() / np.abs(b).max()


def test_identity_is_exact_in_fp64():
    rng = np.random.default_rng(1)
    for _ in range(20):
        L = np.tril(rng.standard_normal((16, 16)), -1)
        exact = np.linalg.inv(np.eye(16) + L)
        assert _rel(_factorised(L, np.float64), exact) < 1e-9


def test_every_factor_matters_for_correlated_keys():
    """With keys that share a direction, beta = 1 and no decay, L has entries
    near 1: leaving out any one factor changes the result by O(1)."""
    rng = np.random.default_rng(2)
    base = rng.standard_normal(128)
    K = _unit(rng.choice([-1.0, 1.0], (16, 1)) * base + 0.05 * rng.standard_normal((16, 128)))
    L = _block(K, np.ones(16), np.zeros(16))
    exact = np.linalg.inv(np.eye(16) + L)
    eye = np.eye(16)
    L2, L4, L8 = L @ L, L @ L @ L @ L, np.linalg.matrix_power(L, 8)
    factors = [eye - L, eye + L2, eye + L4, eye + L8]
    for drop in range(4):
        partial = eye
        for i, f in enumerate(factors):
            if i != drop:
                partial = partial @ f
        assert _rel(partial, exact) > 0.1, drop


def test_fp32_accuracy_for_random_unit_keys():
    """Independent random unit keys (the GDN workload): |L| is small and the fp32
    factorisation is as accurate as the inverse itself can be in fp32."""
    rng = np.random.default_rng(3)
    worst = 0.0
    for _ in range(200):
        K = _unit(rng.standard_normal((16, 128)))
        L = _block(K, rng.uniform(0, 1, 16), -rng.uniform(0, 0.2, 16))
        worst = max(worst, _rel(_factorised(L, np.float32), np.linalg.inv(np.eye(16) + L)))
    assert worst < 1e-6, worst


@pytest.mark.parametrize("seed", range(4))
def test_fp32_accuracy_bound_for_unit_keys_and_beta_at_most_one(seed):
    """Adversarial unit keys (one shared direction with random signs and little
    noise; a few directions), beta <= 1, no decay: |L| reaches 1 and the product
    form's intermediates grow (L^8 up to C(14, 7) = 3432 for an all-ones L), so
    fp32 cancellation costs accuracy.  Over these families the relative error of
    the inverse stays below 2e-3 -- far inside the bf16 path's 2e-2 -- while row
    by row substitution would give about 1e-7."""
    rng = np.random.default_rng(10 + seed)
    base = _unit(rng.standard_normal((3, 128)))
    worst = 0.0
    for trial in range(300):
        if trial % 2:
            K = _unit(rng.choice([-1.0, 1.0], (16, 1)) * base[0]
                      + rng.uniform(0, 0.2) * rng.standard_normal((16, 128)))
        else:
            K = _unit(base[rng.integers(0, 3, 16)] * rng.choice([-1.0, 1.0], (16, 1))
                      + 0.01 * rng.standard_normal((16, 128)))
        beta = np.ones(16) if trial % 3 else rng.uniform(0.5, 1.0, 16)
        L = _block(K, beta, np.zeros(16))
        worst = max(worst, _rel(_factorised(L, np.float32), np.linalg.inv(np.eye(16) + L)))
    assert worst < 2e-3, worst
