"""fp64 chunkwise (WY) form of the Gated DeltaNet recurrence, for pinning the
oracle (CPU, NumPy, small sizes).

The four steps the page "Qwen Team Releases FlashQLA for High-Performance
Linear Attention" lists for the GDN prefill, for one unit and chunk length C,
with gamma_i = prod_{m <= i} alpha_m the in-chunk cumulative gate and
Gamma_ij = gamma_i / gamma_j = exp(G_i - G_j) (G the in-chunk cumulative log
gate):
  1. the chunk's K K^T, gated and beta-scaled, as a unit lower-triangular
     matrix M = I + diag(beta) strict_lower(Gamma * K K^T), and its inverse T;
  2. the projections W = T diag(beta gamma) K and U_v = T diag(beta) V;
  3. the recurrence across chunks: U = U_v - W S, then
     S <- gamma_C S + (K * gamma_C / gamma)^T U;
  4. the outputs O = diag(gamma) Q S + (Q K^T * Gamma, j <= i) U,
with S the state entering the chunk.  Derivation: the update is
S_t = alpha_t S_{t-1} + k_t^T u_t with u_t = beta_t (v_t - alpha_t k_t S_{t-1});
expanding S_{t-1} inside the chunk gives (I + diag(beta) L) U = diag(beta)
(V - diag(gamma) K S_0) with L the strictly lower part of Gamma * K K^T.
"""
import numpy as np


def gdn_chunk_form(q, k, v, g, beta, C, s0=None):
    """q, k: [T, dk]; v: [T, dv]; g, beta: [T] (fp64).  Returns (o, S_T)."""
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        Q, K, V = q[c0:c0 + C], k[c0:c0 + C], v[c0:c0 + C]
        b = beta[c0:c0 + C]
        G = np.cumsum(g[c0:c0 + C])
        n = Q.shape[0]
        gam = np.exp(G)
        Gam = np.exp(G[:, None] - G[None, :])
        M = np.eye(n) + b[:, None] * np.tril(Gam * (K @ K.T), -1)
        Tinv = np.linalg.inv(M)
        W = Tinv @ ((b * gam)[:, None] * K)
        Uv = Tinv @ (b[:, None] * V)
        U = Uv - W @ S
        o[c0:c0 + C] = gam[:, None] * (Q @ S) + (np.tril(Gam) * (Q @ K.T)) @ U
        S = gam[-1] * S + ((gam[-1] / gam)[:, None] * K).T @ U
    return o, S
