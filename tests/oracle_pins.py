"""Pins for oracle R: properties fixed by the pages and by the mathematics.

Each ``pin_*`` takes a recurrence callable with the signature of
``oracle.recurrent`` and raises AssertionError when the property fails.  The
tests run them on the oracle proper (they must all pass) and on deliberately
wrong builds of it (each wrong build must fail at least one).

Citations name the page and the section on it:
  [KDA]  "You could have come up with Kimi Delta Attention" (gokawiil.com),
         the five state-update equations at the top of the article.
  [GN]   GeekNews #31925, summary of the same article, sections by title.
  [F29]  "Paper: Gated DeltaNet -> Kimi Delta Attention" course outline.
"""
from __future__ import annotations

import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _rand_case(seed, T=6, Dk=4, Dv=4, mode="channel", B=1, H=1, unit_k=True,
               h0=True, gate_scale=1.0):
    r = _rng(seed)
    q = r.standard_normal((B, T, H, Dk))
    k = r.standard_normal((B, T, H, Dk))
    if unit_k:
        k = _unit_rows(k)
    v = r.standard_normal((B, T, H, Dv))
    beta = r.uniform(0.05, 1.0, (B, T, H))
    if mode == "channel":
        g = -gate_scale * r.uniform(0.0, 1.0, (B, T, H, Dk))
    elif mode == "scalar":
        g = -gate_scale * r.uniform(0.0, 1.0, (B, T, H))
    else:
        g = None
    s0 = 0.3 * r.standard_normal((B, H, Dk, Dv)) if h0 else None
    return q, k, v, g, beta, s0


def _decay_rows(Hs, g_t, mode):
    """Diag(alpha_t) applied to the transposed state (rows = key channels)."""
    if mode == "channel":
        return np.exp(g_t)[:, None] * Hs
    if mode == "scalar":
        return np.exp(g_t) * Hs
    return Hs.copy()


def _prefix_state(rec, q, k, v, g, beta, s0, t, mode, scale):
    """State H_{t-1} after tokens 0..t-1 (t may be 0)."""
    if t == 0:
        Dk, Dv = q.shape[-1], v.shape[-1]
        return np.zeros((Dk, Dv)) if s0 is None else np.array(s0[0, 0])
    gp = None if g is None else g[:, :t]
    _, hT = rec(q[:, :t], k[:, :t], v[:, :t], gp, beta[:, :t], s0, scale=scale, mode=mode)
    return hT[0, 0]


# ---------------------------------------------------------------------------
def pin_p1_readback_beta1(rec):
    """P1: beta=1, alpha=1, unit key -> reading with the key returns v_t
    exactly ([GN] "DeltaNet: write the error, not the value": with beta_t = 1
    the immediate read-back is exactly v_t)."""
    for mode in ("channel", "scalar", "none"):
        q, k, v, g, beta, s0 = _rand_case(1, T=7, mode=mode)
        beta[:] = 1.0
        if g is not None:
            g[:] = 0.0
        o, _ = rec(k.copy(), k, v, g, beta, s0, scale=1.0, mode=mode)
        err = np.abs(o - v).max()
        assert err < TOL, (mode, err)


def pin_p2_readback_blend(rec):
    """P2: S_t k_t = (1 - beta_t) S~_t k_t + beta_t v_t for a unit key
    ([GN] "DeltaNet": the immediate read-back blends old prediction and
    target; "Gated DeltaNet"/"KDA": the prediction is taken after the decay)."""
    for mode in ("channel", "scalar", "none"):
        q, k, v, g, beta, s0 = _rand_case(2, T=6, mode=mode)
        o, _ = rec(k.copy(), k, v, g, beta, s0, scale=1.0, mode=mode)
        for t in range(k.shape[1]):
            Hp = _prefix_state(rec, k, k, v, g, beta, s0, t, mode, 1.0)
            gt = None if g is None else g[0, t, 0]
            Ht = _decay_rows(Hp, gt, mode)
            kt = k[0, t, 0]
            want = (1 - beta[0, t, 0]) * (Ht.T @ kt) + beta[0, t, 0] * v[0, t, 0]
            err = np.abs(o[0, t, 0] - want).max()
            assert err < 1e-11, (mode, t, err)


def pin_p3_gradient_step(rec):
    """P3: the write equals one gradient-descent step of size beta_t on
    1/2 ||S k_t - v_t||^2 taken at S~_t ([GN] "Derivation from a
    reconstruction loss"; [F29] "the delta rule as online least squares").
    The gradient is taken by central finite differences, not by formula."""
    for mode in ("channel", "none"):
        q, k, v, g, beta, s0 = _rand_case(3, T=4, Dk=3, Dv=4, mode=mode)
        t = 3
        Hp = _prefix_state(rec, q, k, v, g, beta, s0, t, mode, 1.0)
        Ht = _decay_rows(Hp, None if g is None else g[0, t, 0], mode)
        St = Ht.T                                   # article orientation, Dv x Dk
        kt, vt = k[0, t, 0], v[0, t, 0]

        def loss(S):
            r = S @ kt - vt
            return 0.5 * float(r @ r)

        grad = np.zeros_like(St)
        h = 1e-4
        for a in range(St.shape[0]):
            for c in range(St.shape[1]):
                Sp = St.copy(); Sp[a, c] += h
                Sm = St.copy(); Sm[a, c] -= h
                grad[a, c] = (loss(Sp) - loss(Sm)) / (2 * h)
        gp = None if g is None else g[:, :t + 1]
        _, hT = rec(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], gp, beta[:, :t + 1], s0,
                    scale=1.0, mode=mode)
        want = St - beta[0, t, 0] * grad
        err = np.abs(hT[0, 0].T - want).max()
        assert err < 1e-8, (mode, err)


def pin_p4_locality(rec):
    """P4: a query orthogonal to k_t sees no change from the write:
    S_t q = S~_t q ([GN] "DeltaNet": the update is local in key space)."""
    for mode in ("channel", "scalar", "none"):
        q, k, v, g, beta, s0 = _rand_case(4, T=5, Dk=5, Dv=3, mode=mode)
        t = 4
        kt = k[0, t, 0]
        qt = q[0, t, 0] - (q[0, t, 0] @ kt) * kt          # project out k_t
        q2 = q.copy(); q2[0, t, 0] = qt
        o, _ = rec(q2, k, v, g, beta, s0, scale=1.0, mode=mode)
        Hp = _prefix_state(rec, q2, k, v, g, beta, s0, t, mode, 1.0)
        Ht = _decay_rows(Hp, None if g is None else g[0, t, 0], mode)
        err = np.abs(o[0, t, 0] - Ht.T @ qt).max()
        assert err < TOL, (mode, err)
        if mode == "none":
            err2 = np.abs(o[0, t, 0] - Hp.T @ qt).max()
            assert err2 < TOL


def pin_p5_contraction(rec):
    """P5: with v = 0 and alpha = 1 the transition I - beta k k^T has
    eigenvalue 1 - beta along k and 1 elsewhere ([GN] "Structured state
    transition"), so S_t k_t = (1 - beta_t) S_{t-1} k_t and the Frobenius norm
    never grows for beta in [0, 1]."""
    q, k, v, g, beta, s0 = _rand_case(5, T=8, Dk=4, Dv=3, mode="none")
    v[:] = 0.0
    o, _ = rec(k.copy(), k, v, None, beta, s0, scale=1.0, mode="none")
    prev = np.linalg.norm(s0[0, 0])
    for t in range(k.shape[1]):
        Hp = _prefix_state(rec, k, k, v, None, beta, s0, t, "none", 1.0)
        want = (1 - beta[0, t, 0]) * (Hp.T @ k[0, t, 0])
        assert np.abs(o[0, t, 0] - want).max() < TOL
        Hn = _prefix_state(rec, k, k, v, None, beta, s0, t + 1, "none", 1.0)
        nrm = np.linalg.norm(Hn)
        assert nrm <= prev * (1 + 1e-12), (t, nrm, prev)
        prev = nrm


def pin_p6_dplr(rec):
    """P6: S_t = S_{t-1} (D_t - (D_t k_t)(beta_t k_t)^T) + beta_t v_t k_t^T
    ([GN] "Diagonal-plus-low-rank transition"), iterated here in the
    article's orientation (S is Dv x Dk) with dense matrix products, must give
    the same outputs o_t = S_t (scale q_t) and final state."""
    for mode in ("channel", "scalar", "none"):
        q, k, v, g, beta, s0 = _rand_case(6, T=9, Dk=5, Dv=4, mode=mode,
                                          unit_k=False)
        scale = 0.37
        o, hT = rec(q, k, v, g, beta, s0, scale=scale, mode=mode)
        S = s0[0, 0].T.copy()
        Dk = k.shape[-1]
        for t in range(k.shape[1]):
            if mode == "channel":
                D = np.diag(np.exp(g[0, t, 0]))
            elif mode == "scalar":
                D = np.exp(g[0, t, 0]) * np.eye(Dk)
            else:
                D = np.eye(Dk)
            kt, bt = k[0, t, 0], beta[0, t, 0]
            At = D - np.outer(D @ kt, bt * kt)
            S = S @ At + bt * np.outer(v[0, t, 0], kt)
            err = np.abs(o[0, t, 0] - S @ (scale * q[0, t, 0])).max()
            assert err < 1e-11, (mode, t, err)
        assert np.abs(hT[0, 0] - S.T).max() < 1e-11


def pin_p7_mode_reduction(rec):
    """P7: per-channel gates that are equal across channels reduce KDA to the
    scalar-gate case, and a zero scalar log-gate reduces Gated DeltaNet to
    DeltaNet ([GN] "Kimi Delta Attention": the only change from Gated
    DeltaNet is promoting alpha_t to Diag(alpha_t))."""
    q, k, v, gs, beta, s0 = _rand_case(7, T=6, Dk=4, Dv=5, mode="scalar")
    gc = np.repeat(gs[..., None], 4, axis=-1)
    o1, h1 = rec(q, k, v, gc, beta, s0, mode="channel")
    o2, h2 = rec(q, k, v, gs, beta, s0, mode="scalar")
    assert np.abs(o1 - o2).max() < 1e-14 and np.abs(h1 - h2).max() < 1e-14
    o3, h3 = rec(q, k, v, np.zeros_like(gs), beta, s0, mode="scalar")
    o4, h4 = rec(q, k, v, None, beta, s0, mode="none")
    assert np.abs(o3 - o4).max() < 1e-14 and np.abs(h3 - h4).max() < 1e-14


def pin_p9_closed_form(rec):
    """P9: with keys that never overlap, the prediction S~_t k_t is zero and
    the output has the gated-linear-attention closed form
    o_t = sum_{i<=t} beta_i v_i <k_i, D_{i+1:t} q~_t>  ([GN] "From quadratic
    attention to a linear state" plus the per-channel decay of "Kimi Delta
    Attention").  Channel gates: one-hot keys on distinct channels; scalar
    gates: any orthonormal key set."""
    r = _rng(9)
    Dk, Dv, T, scale = 8, 3, 6, 0.7
    perm = r.permutation(Dk)[:T]
    k = np.zeros((1, T, 1, Dk))
    for t in range(T):
        k[0, t, 0, perm[t]] = 1.0
    q = r.standard_normal((1, T, 1, Dk))
    v = r.standard_normal((1, T, 1, Dv))
    beta = r.uniform(0.1, 1.0, (1, T, 1))
    g = -r.uniform(0.0, 2.0, (1, T, 1, Dk))
    o, _ = rec(q, k, v, g, beta, None, scale=scale, mode="channel")
    for t in range(T):
        want = np.zeros(Dv)
        for i in range(t + 1):
            c = perm[i]
            decay = np.exp(np.sum(g[0, i + 1:t + 1, 0, c]))
            want += beta[0, i, 0] * v[0, i, 0] * decay * scale * q[0, t, 0, c]
        assert np.abs(o[0, t, 0] - want).max() < 1e-12, t
    # scalar gates, random orthonormal keys
    Qm, _ = np.linalg.qr(r.standard_normal((Dk, Dk)))
    k2 = Qm[:, :T].T.reshape(1, T, 1, Dk).copy()
    gs = -r.uniform(0.0, 2.0, (1, T, 1))
    o2, _ = rec(q, k2, v, gs, beta, None, scale=scale, mode="scalar")
    for t in range(T):
        want = np.zeros(Dv)
        for i in range(t + 1):
            decay = np.exp(np.sum(gs[0, i + 1:t + 1, 0]))
            want += beta[0, i, 0] * v[0, i, 0] * decay * scale * (k2[0, i, 0] @ q[0, t, 0])
        assert np.abs(o2[0, t, 0] - want).max() < 1e-12, t


def pin_p10_linearity(rec):
    """P10: from a zero state, e_t and S_t are linear in the values
    ([KDA] equations: v enters only through e_t), so V -> O is linear, and
    permuting value channels permutes o and the state's columns."""
    q, k, v, g, beta, _ = _rand_case(10, T=7, Dk=4, Dv=5, mode="channel", h0=False)
    v2 = _rng(11).standard_normal(v.shape)
    o1, h1 = rec(q, k, v, g, beta, None, mode="channel")
    o2, h2 = rec(q, k, v2, g, beta, None, mode="channel")
    o3, h3 = rec(q, k, 2.0 * v - 3.0 * v2, g, beta, None, mode="channel")
    assert np.abs(o3 - (2 * o1 - 3 * o2)).max() < 1e-12
    assert np.abs(h3 - (2 * h1 - 3 * h2)).max() < 1e-12
    perm = np.array([3, 0, 4, 1, 2])
    o4, h4 = rec(q, k, v[..., perm], g, beta, None, mode="channel")
    assert np.abs(o4 - o1[..., perm]).max() < 1e-14
    assert np.abs(h4 - h1[..., perm]).max() < 1e-14


def pin_p11_state_handoff(rec):
    """P11: the state is the resumable context ([GN] "Fused recurrent kernel
    for decode": stateful serving): running T1 + T2 tokens equals running
    T1 tokens and then T2 tokens from the returned state."""
    for mode in ("channel", "scalar", "none"):
        q, k, v, g, beta, s0 = _rand_case(12, T=9, Dk=4, Dv=3, mode=mode)
        o, hT = rec(q, k, v, g, beta, s0, mode=mode)
        t1 = 4
        ga = None if g is None else g[:, :t1]
        gb = None if g is None else g[:, t1:]
        oa, ha = rec(q[:, :t1], k[:, :t1], v[:, :t1], ga, beta[:, :t1], s0, mode=mode)
        ob, hb = rec(q[:, t1:], k[:, t1:], v[:, t1:], gb, beta[:, t1:], ha, mode=mode)
        assert np.abs(np.concatenate([oa, ob], axis=1) - o).max() < 1e-13
        assert np.abs(hb - hT).max() < 1e-13


def pin_p12_hand_derived(rec):
    """P12: a three-token, two-channel case worked by hand from the [KDA]
    equations (values in tests/golden/tiny_hand.json).

    t=1: H~ = 0, e = 0.5 * (2, 4) = (1, 2), H = [[1, 2], [0, 0]], o = (1, 2).
    t=2: H~ = Diag(.5, .25) H = [[.5, 1], [0, 0]], vhat = H~^T (.6, .8)
         = (.3, .6), e = (.7, -1.6), H = [[.92, .04], [.56, -1.28]],
         o = H^T (1, 0) = (.92, .04).
    t=3: H~ = Diag(1, .5) H = [[.92, .04], [.28, -.64]], vhat = (.28, -.64),
         e = .25 * (2.72, .64) = (.68, .16), H = [[.92, .04], [.96, -.48]],
         o = H^T (2, 2) = (3.76, -.88).
    """
    with open(os.path.join(HERE, "golden", "tiny_hand.json")) as f:
        d = json.load(f)
    T = len(d["k"])
    sh = (1, T, 1, 2)
    k = np.array(d["k"]).reshape(sh)
    v = np.array(d["v"]).reshape(sh)
    q = np.array(d["q"]).reshape(sh)
    beta = np.array(d["beta"]).reshape(1, T, 1)
    g = np.log(np.array(d["alpha"])).reshape(sh)
    o, hT = rec(q, k, v, g, beta, None, scale=d["scale"], mode="channel")
    assert np.abs(o[0, :, 0] - np.array(d["o"])).max() < 1e-12
    assert np.abs(hT[0, 0] - np.array(d["H_final"])).max() < 1e-12


ALL_PINS = [pin_p1_readback_beta1, pin_p2_readback_blend, pin_p3_gradient_step,
            pin_p4_locality, pin_p5_contraction, pin_p6_dplr, pin_p7_mode_reduction,
            pin_p9_closed_form, pin_p10_linearity, pin_p11_state_handoff,
            pin_p12_hand_derived]
