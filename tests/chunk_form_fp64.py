"""fp64 NumPy evaluation of the chunkwise-parallel form, used only to pin the
oracle (chunked and step-wise evaluation must agree).

It follows the page "Gated Linear Attention (GLA): Mathematical Foundations
...", sections "Sequence Partitioning and State Factorization" and
"Mathematical Formulation of Chunk Computations": per chunk u of C tokens,
Gamma = inclusive cumulative sum of log alpha inside the chunk,
M = (Q K^T) masked with the channel-wise decay exp(Gamma_i - Gamma_j) for
i >= j, O_intra = M V, O_inter = (Q * exp(Gamma)) S_prev,
S_new = diag(exp(Gamma_last)) S_prev + (K * exp(Gamma_last - Gamma))^T V.
The page writes the decay as a C x C mask; with a per-channel gate it lives
inside the sum over key channels, which is how it is written here.  A last
chunk shorter than C uses Gamma at its own last row.
"""
import numpy as np


def chunk_form(q, k, v, g, C, s0=None):
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g))
    T, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if s0 is None else np.array(s0, dtype=np.float64)
    o = np.zeros((T, dv))
    for start in range(0, T, C):
        end = min(start + C, T)
        Q, K, V, A = q[start:end], k[start:end], v[start:end], g[start:end]
        Gam = np.cumsum(A, axis=0)                      # inclusive, restarts per chunk
        n = end - start
        M = np.zeros((n, n))
        for i in range(n):
            for j in range(i + 1):
                M[i, j] = np.sum(Q[i] * K[j] * np.exp(Gam[i] - Gam[j]))
        o_intra = M @ V
        o_inter = (Q * np.exp(Gam)) @ S
        o[start:end] = o_intra + o_inter
        last = Gam[-1]
        S = np.exp(last)[:, None] * S + (K * np.exp(last[None, :] - Gam)).T @ V
    return o, S
