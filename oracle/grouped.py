"""Oracle for grouped value heads.

TEST INFRASTRUCTURE ONLY (see the package docstring).

GeekNews #31925, section "Fused recurrent kernel for decode": the recurrent
programs run per sequence and value head.  With grouped value heads there are
H value heads and Hqk query/key heads (H a multiple of Hqk); value head h has
its own state, gate, beta and values and reads query/key head h // (H / Hqk).
Written out: repeat every query/key head H / Hqk times along the head axis
and run oracle R on the result.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .recurrence import recurrent


def recurrent_grouped(q, k, v, g, beta, h0=None, *, scale: Optional[float] = None,
                      mode: str = "channel", threads: int = 0, mutant: int = 0):
    """q, k [B,T,Hqk,Dk]; v [B,T,H,Dv]; g, beta, h0 per value head as for
    :func:`oracle.recurrent`.  Returns (o [B,T,H,Dv], hT [B,H,Dk,Dv]).

    ``mutant`` = 1 plants a deliberate mistake (tests only): value head h
    reads query/key head h % Hqk instead of h // (H / Hqk)."""
    Hqk, H = q.shape[2], v.shape[2]
    assert k.shape == q.shape and H % Hqk == 0
    G = H // Hqk
    if mutant == 1:
        idx = np.arange(H) % Hqk
    else:
        idx = np.arange(H) // G
    qe = np.asarray(q)[:, :, idx]
    ke = np.asarray(k)[:, :, idx]
    return recurrent(qe, ke, v, g, beta, h0, scale=scale, mode=mode, threads=threads)


def recurrent_grouped_bwd(q, k, v, g, beta, h0, do, dhT=None, *,
                          scale: Optional[float] = None, mode: str = "channel",
                          threads: int = 0):
    """Gradients of :func:`recurrent_grouped`.  The repeat along the head axis
    is a copy, so its gradient is the sum over the copies: the query and key
    gradients of every value head of a group add up on their shared
    query/key head.  Returns the dict of :func:`oracle.recurrent_bwd` with
    dq, dk of shape [B,T,Hqk,Dk]."""
    from .recurrence import recurrent_bwd
    Hqk, H = q.shape[2], v.shape[2]
    assert k.shape == q.shape and H % Hqk == 0
    G = H // Hqk
    idx = np.arange(H) // G
    qe = np.asarray(q)[:, :, idx]
    ke = np.asarray(k)[:, :, idx]
    out = recurrent_bwd(qe, ke, v, g, beta, h0, do, dhT, scale=scale, mode=mode,
                        threads=threads)
    B, T = q.shape[:2]
    for name in ("dq", "dk"):
        x = out[name]
        out[name] = x.reshape(B, T, Hqk, G, x.shape[-1]).sum(axis=3)
    return out
