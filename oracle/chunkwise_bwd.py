"""Oracle C-bwd: the gradient of the chunkwise form, NumPy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages train KDA with the chunkwise algorithm (F29 course outline, "Paper:
Gated DeltaNet -> Kimi Delta Attention"; GeekNews #31925, section "Fused
recurrent kernel for decode": chunkwise for training and prefill) but print
no backward formulas.  This module differentiates the chunk map of
``chunkwise.py`` (same notation; H the transposed state entering a chunk of
L tokens, q~ = scale q, G the inclusive prefix of log gates,
Gamma_ij = exp(G_i - G_j) for j <= i):

  A    = strict lower part of  beta_i sum_c k_i k_j Gamma_ij     (coupling)
  T    = (I + A)^-1 ;  U = T Diag(beta) V ;  W = T Diag(beta) (K * e^G)
  E    = U - W H                                                 (pseudo-values)
  Aqk  = inclusive lower part of  sum_c q~_i k_j Gamma_ij
  O    = (Q~ * e^G) H + Aqk E
  H'   = Diag(e^{G_last}) H + (K * e^{G_last - G})^T E

Given dO and dH' (the gradient reaching the chunk's end state) reverse mode
gives, with every decay again taken from a difference of prefixes:

  dE   = Aqk^T dO + Kr dH'                 Kr = K * e^{G_last - G}
  dH   = Diag(e^{G_last}) dH' + (Q~ * e^G)^T dO - W^T dE   (to the previous chunk)
  dUt  = T^T dE ;  dV = Diag(beta) dUt
  dA   = -(strict lower part of dUt E^T)   (the solve's gradient collapses to
                                            this because E = U - W H)
  dAqk = inclusive lower part of dO E^T
  dq_i = scale (e^{G_i} (dO H^T)_i + sum_{j<=i} dAqk_ij k_j Gamma_ij)
  Pg_i = beta_i (-e^{G_i} (dUt H^T)_i + sum_{j<i} dA_ij k_j Gamma_ij)
  Pinv_j = sum_{i>j} dA_ij beta_i k_i Gamma_ij + sum_{i>=j} dAqk_ij q~_i Gamma_ij
  Pr_j = e^{G_last - G_j} (E dH'^T)_j
  dk   = Pg + Pinv + Pr
  dG_i = k_i (Pg_i - Pinv_i - Pr_i) + q_i dq_i ; dG_last += sum_j Pr_j k_j
         + e^{G_last} sum_v H dH'
  dbeta_i = dUt_i . v_i - (dUt H^T)_i . (k_i e^{G_i}) + sum_{j<i} dA_ij A_ij / beta_i
  dg   = suffix sums of dG within the chunk (G is a prefix sum of g)

(the last dbeta term is evaluated without the division, from the coupling
before the beta scaling).  The scalar-gate mode sums dg over channels; the
ungated mode has none.  The whole map is pinned by the test that it equals
the reverse-mode gradient of the token recurrence (oracle R-bwd), which is
itself pinned by finite differences of oracle R.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .chunkwise import _gate_block


def chunkwise_bwd(q, k, v, g, beta, h0, do, dhT=None, *, chunk: int = 64,
                  scale: Optional[float] = None, mode: str = "channel"):
    """Same arguments and return value as :func:`oracle.recurrent_bwd`, plus
    the chunk length (a last chunk shorter than ``chunk`` is allowed)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    do = np.asarray(do, np.float64)
    B, T, Hh, Dk = q.shape
    Dv = v.shape[-1]
    if scale is None:
        scale = Dk ** -0.5
    out = {
        "dq": np.zeros((B, T, Hh, Dk)), "dk": np.zeros((B, T, Hh, Dk)),
        "dv": np.zeros((B, T, Hh, Dv)), "dbeta": np.zeros((B, T, Hh)),
        "dg": None if mode == "none" else np.zeros(np.asarray(g).shape),
        "dh0": np.zeros((B, Hh, Dk, Dv)),
    }
    starts = list(range(0, T, chunk))
    for b in range(B):
        for h in range(Hh):
            S = np.zeros((Dk, Dv)) if h0 is None else np.array(h0[b, h], np.float64)
            saved = []
            # forward sweep over chunks: the state entering each chunk and
            # the chunk-local quantities
            for t0 in starts:
                t1 = min(T, t0 + chunk)
                L = t1 - t0
                K = k[b, t0:t1, h, :]
                Qs = q[b, t0:t1, h, :] * scale
                V = v[b, t0:t1, h, :]
                bt = beta[b, t0:t1, h]
                G = np.cumsum(_gate_block(g, mode, b, h, t0, t1, Dk), axis=0)
                lower = np.tril(np.ones((L, L), bool))
                diff = G[:, None, :] - G[None, :, :]
                Gam = np.where(lower[:, :, None],
                               np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
                Apre = np.tril(np.einsum("ic,ijc,jc->ij", K, Gam, K), -1)
                A = bt[:, None] * Apre
                Tm = np.linalg.inv(np.eye(L) + A)
                U = Tm @ (bt[:, None] * V)
                W = Tm @ (bt[:, None] * (K * np.exp(G)))
                E = U - W @ S
                Aqk = np.einsum("ic,ijc,jc->ij", Qs, Gam, K)
                Gl = G[-1]
                Kr = K * np.exp(Gl[None, :] - G)
                saved.append((t0, t1, K, Qs, V, bt, G, Gam, Apre, Tm, W, E, Aqk, Kr, S.copy()))
                S = np.exp(Gl)[:, None] * S + Kr.T @ E
            # reverse sweep
            dHn = np.zeros((Dk, Dv)) if dhT is None else np.array(dhT[b, h], np.float64)
            for (t0, t1, K, Qs, V, bt, G, Gam, Apre, Tm, W, E, Aqk, Kr, Hc) in reversed(saved):
                L = t1 - t0
                dO = do[b, t0:t1, h, :]
                eG = np.exp(G)
                Gl = G[-1]
                dE = Aqk.T @ dO + Kr @ dHn
                dUt = Tm.T @ dE
                X1 = dO @ Hc.T
                X2 = E @ dHn.T
                X3 = dUt @ Hc.T
                dAqk = np.tril(dO @ E.T)
                dA = -np.tril(dUt @ E.T, -1)
                dq = scale * (eG * X1 + np.einsum("ij,jc,ijc->ic", dAqk, K, Gam))
                Pg = bt[:, None] * (-eG * X3 + np.einsum("ij,jc,ijc->ic", dA, K, Gam))
                Pinv = np.einsum("ij,i,ic,ijc->jc", dA, bt, K, Gam) + \
                    np.einsum("ij,ic,ijc->jc", dAqk, Qs, Gam)
                Pr = np.exp(Gl[None, :] - G) * X2
                dk = Pg + Pinv + Pr
                dG = K * (Pg - Pinv - Pr) + (Qs / scale) * dq
                dG[-1] += np.sum(Pr * K, axis=0) + np.exp(Gl) * np.sum(Hc * dHn, axis=1)
                db = np.sum(dUt * V, axis=1) - np.sum(X3 * K * eG, axis=1) + \
                    np.sum(dA * Apre, axis=1)
                out["dq"][b, t0:t1, h] = dq
                out["dk"][b, t0:t1, h] = dk
                out["dv"][b, t0:t1, h] = bt[:, None] * dUt
                out["dbeta"][b, t0:t1, h] = db
                dg = np.cumsum(dG[::-1], axis=0)[::-1]
                if mode == "channel":
                    out["dg"][b, t0:t1, h] = dg
                elif mode == "scalar":
                    out["dg"][b, t0:t1, h] = dg.sum(axis=1)
                dHn = np.exp(Gl)[:, None] * dHn + (Qs * eG).T @ dO - W.T @ dE
            out["dh0"][b, h] = dHn
    return out
