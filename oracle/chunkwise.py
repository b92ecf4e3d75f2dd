"""Oracle C: the chunkwise-parallel form of KDA, NumPy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: GeekNews #31925 ("DeltaNet-family linear attention variants", a
summary of "You could have come up with Kimi Delta Attention"), section
"Chunkwise KDA: recasting the recurrence as matrix products" and its
subsections "Cumulative decay and provisional errors" and "Restoring causal
dependence"; and the F29 course outline ("Paper: Gated DeltaNet -> Kimi Delta
Attention"), Objectives: "pseudo-values from a triangular solve; log-space
decay ratios", exercise "recurrent, chunkwise (WY/UT form)".

The summary breaks off in the middle of the error-coupling formula, so the
text for the triangular solve, the state carry and the output is lost.  Steps
5-7 below are derived by unrolling the five-step recurrence over one chunk
with the same cumulative-decay bookkeeping the summary sets up; they are
pinned by the test that this form equals oracle R (the summary requires the
chunk form to give exactly the same states and outputs as the token loop).

Per (batch, head), with H the transposed state (Dk x Dv) entering a chunk of
L tokens i = 0 .. L-1:

 1. G_i = g_0 + ... + g_i                  (inclusive prefix of log gates;
                                            D_{0:i} = Diag(exp G_i))
 2. Gamma_ij = exp(G_i - G_j), j <= i       (= D_{j+1:i}; taken from the
                                            difference, so it never overflows)
 3. A_ij = beta_i * sum_c k_j[c] Gamma_ij[c] k_i[c]   for j < i
                                           (the summary's rho_ij)
 4. ebar_i = beta_i (v_i - H^T (exp(G_i) * k_i))      provisional errors
 5. e_i = ebar_i - sum_{j<i} A_ij e_j      forward substitution, i.e.
    (I + A) E = Ebar.  UT form: U = (I+A)^-1 Diag(beta) V,
    W = (I+A)^-1 Diag(beta) (K * exp(G)), E = U - W H ("pseudo-values").
 6. o_i = H^T (exp(G_i) * q~_i) + sum_{j<=i} e_j sum_c k_j[c] Gamma_ij[c] q~_i[c]
    (j <= i: the read happens after token i's own write)
 7. H <- Diag(exp G_{L-1}) H + sum_j (k_j * exp(G_{L-1} - G_j)) e_j^T
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _gate_block(g, mode, b, h, t0, t1, Dk):
    L = t1 - t0
    if mode == "channel":
        return np.asarray(g[b, t0:t1, h, :], np.float64)
    if mode == "scalar":
        return np.repeat(np.asarray(g[b, t0:t1, h], np.float64)[:, None], Dk, axis=1)
    return np.zeros((L, Dk), np.float64)


def chunkwise(q, k, v, g, beta, h0=None, *, chunk: int = 64,
              scale: Optional[float] = None, mode: str = "channel",
              solve: str = "substitution"):
    """Run oracle C.

    Same arguments and return values as :func:`oracle.recurrent`, plus the
    chunk length and ``solve`` in {"substitution", "ut"}: the per-row forward
    substitution of step 5, or the UT form with a dense solve of (I + A).
    A last chunk shorter than ``chunk`` is allowed.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, Hh, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    o = np.zeros((B, T, Hh, Dv), np.float64)
    hT = np.zeros((B, Hh, Dk, Dv), np.float64)
    for b in range(B):
        for h in range(Hh):
            S = np.zeros((Dk, Dv)) if h0 is None else np.array(h0[b, h], np.float64)
            for t0 in range(0, T, chunk):
                t1 = min(T, t0 + chunk)
                L = t1 - t0
                K = k[b, t0:t1, h, :]                   # L x Dk
                Q = q[b, t0:t1, h, :] * scale           # L x Dk  (q~)
                V = v[b, t0:t1, h, :]                   # L x Dv
                bt = beta[b, t0:t1, h]                  # L
                G = np.cumsum(_gate_block(g, mode, b, h, t0, t1, Dk), axis=0)   # step 1
                # step 2: Gamma[i, j, c] = exp(G_i - G_j) for j <= i, else 0
                diff = G[:, None, :] - G[None, :, :]
                lower = np.tril(np.ones((L, L), bool))
                Gamma = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
                # step 3: strictly lower coupling
                A = bt[:, None] * np.einsum("ic,ijc,jc->ij", K, Gamma, K)
                A = np.tril(A, -1)
                # step 4: provisional errors against the incoming state
                Ebar = bt[:, None] * (V - (K * np.exp(G)) @ S)
                # step 5
                if solve == "substitution":
                    E = np.zeros_like(Ebar)
                    for i in range(L):
                        E[i] = Ebar[i] - A[i, :i] @ E[:i]
                elif solve == "ut":
                    M = np.eye(L) + A
                    U = np.linalg.solve(M, bt[:, None] * V)
                    W = np.linalg.solve(M, bt[:, None] * (K * np.exp(G)))
                    E = U - W @ S
                else:
                    raise ValueError(solve)
                # step 6: inter-chunk read + intra-chunk (inclusive) read
                Aqk = np.einsum("ic,ijc,jc->ij", Q, Gamma, K)        # lower incl.
                o[b, t0:t1, h, :] = (Q * np.exp(G)) @ S + Aqk @ E
                # step 7: state carry
                S = np.exp(G[-1])[:, None] * S + (K * np.exp(G[-1][None, :] - G)).T @ E
            hT[b, h] = S
    return o, hT
