"""Oracle for packed variable-length batches.

TEST INFRASTRUCTURE ONLY (see the package docstring).

GeekNews #31925, section "Fused recurrent kernel for decode": the recurrent
form serves decode, short sequences and stateful serving, and different
sequences run independently.  A packed batch is therefore nothing but N
separate recurrences, one per sequence: sequence n takes tokens
cu[n] .. cu[n+1]-1 of the packed [T, H, D] tensors, starts from its own
state h0[n] and ends in hT[n].  This is that definition written out: a plain
loop calling oracle R once per sequence.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .grouped import recurrent_grouped


def recurrent_varlen(q, k, v, g, beta, cu, h0=None, *, scale: Optional[float] = None,
                     mode: str = "channel", threads: int = 0, mutant: int = 0):
    """q, k [T,Hqk,Dk]; v [T,H,Dv] (grouped value heads as in
    :func:`oracle.recurrent_grouped`); g [T,H,Dk] / [T,H] / None; beta [T,H];
    cu [N+1] nondecreasing offsets with cu[0] = 0 and cu[N] = T;
    h0 [N,H,Dk,Dv] or None.  Returns (o [T,H,Dv], hT [N,H,Dk,Dv]) in float64.

    ``mutant`` > 0 plants a deliberate mistake (tests only): 1 starts every
    sequence after the first one token late, 2 carries each final state into
    the next sequence."""
    cu = np.asarray(cu, np.int64)
    N = len(cu) - 1
    T, _, Dk = q.shape
    H, Dv = v.shape[-2], v.shape[-1]
    assert N >= 0 and cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    o = np.zeros((T, H, Dv), np.float64)
    hT = np.zeros((N, H, Dk, Dv), np.float64)
    carry = None
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        if mutant == 1 and n > 0 and s < e:
            s += 1
        hn = None if h0 is None else np.asarray(h0[n:n + 1], np.float64)
        if mutant == 2 and carry is not None:
            hn = carry
        if e == s:                      # an empty sequence keeps its state
            if hn is not None:
                hT[n] = hn[0]
            continue
        sl = lambda x: None if x is None else np.asarray(x[s:e])[None]
        on, hTn = recurrent_grouped(sl(q), sl(k), sl(v), sl(g), sl(beta), hn, scale=scale,
                                    mode=mode, threads=threads)
        o[s:e] = on[0]
        hT[n] = hTn[0]
        carry = hTn
    return o, hT


def recurrent_varlen_bwd(q, k, v, g, beta, cu, h0, do, dhT=None, *,
                         scale: Optional[float] = None, mode: str = "channel",
                         threads: int = 0):
    """Gradients of :func:`recurrent_varlen`: one call of the grouped
    gradient oracle per sequence (the sequences share nothing, so neither do
    their gradients).  ``do`` [T,H,Dv]; ``dhT`` [N,H,Dk,Dv] or None.  Returns
    the dict of :func:`oracle.recurrent_bwd` with packed token tensors (no
    batch axis) and dh0 [N,H,Dk,Dv]; an empty sequence passes dhT[n] through."""
    from .grouped import recurrent_grouped_bwd
    cu = np.asarray(cu, np.int64)
    N = len(cu) - 1
    T, Hq, Dk = q.shape
    H, Dv = v.shape[-2], v.shape[-1]
    assert N >= 0 and cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    out = {"dq": np.zeros((T, Hq, Dk)), "dk": np.zeros((T, Hq, Dk)), "dv": np.zeros((T, H, Dv)),
           "dbeta": np.zeros((T, H)), "dg": None if mode == "none" else np.zeros(np.shape(g)),
           "dh0": np.zeros((N, H, Dk, Dv))}
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        if e == s:
            if dhT is not None:
                out["dh0"][n] = dhT[n]
            continue
        sl = lambda x: None if x is None else np.asarray(x[s:e])[None]
        hn = None if h0 is None else np.asarray(h0[n:n + 1], np.float64)
        dn = None if dhT is None else np.asarray(dhT[n:n + 1], np.float64)
        r = recurrent_grouped_bwd(sl(q), sl(k), sl(v), sl(g), sl(beta), hn, sl(do), dn,
                                  scale=scale, mode=mode, threads=threads)
        for name in ("dq", "dk", "dv", "dbeta"):
            out[name][s:e] = r[name][0]
        if out["dg"] is not None:
            out["dg"][s:e] = r["dg"][0]
        out["dh0"][n] = r["dh0"][0]
    return out
