"""Oracle of the fused prologue.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The three optional input transforms, written out in float64 from their
definitions, to be applied before oracle R:
- NORMALIZE_QK: q and k of every token and head divided by their L2 norm
  over the key dimension, x / sqrt(sum x^2 + 1e-6) ("You could have come up
  with Kimi Delta Attention", notation note: the derivation assumes
  normalised keys; the 1e-6 guard is the library's reading);
- BETA_SIGMOID: the write strength beta = sigmoid(b) of a pre-activation b,
  which puts it inside [0, 1] (GeekNews #31925, section "DeltaNet: write the
  error, not the value");
- GATE_LOGSIGMOID: the retention alpha = sigmoid(a) of a pre-activation a,
  stored as g = log(alpha) (GeekNews #31925, section "Diagonal-plus-low-rank
  transition").
"""
from __future__ import annotations

import numpy as np

NORMALIZE_QK, BETA_SIGMOID, GATE_LOGSIGMOID = 1, 2, 4
NORM_EPS = 1e-6


def l2_normalize(x, mutant: int = 0):
    """x / sqrt(sum over the last axis of x^2 + 1e-6).  ``mutant`` = 1 plants
    a mistake (tests only): the sum runs over the head axis instead."""
    x = np.asarray(x, np.float64)
    axis = -2 if mutant == 1 else -1
    return x / np.sqrt(np.sum(x * x, axis=axis, keepdims=True) + NORM_EPS)


def sigmoid(x):
    x = np.asarray(x, np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def log_sigmoid(x):
    """log(1 / (1 + exp(-x))), evaluated without overflow."""
    x = np.asarray(x, np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def apply_prologue(q, k, g, beta, flags: int, mutant: int = 0):
    """The transformed (q, k, g, beta) for the given flag bits.  ``mutant`` =
    2 plants a mistake (tests only): beta = sigmoid(-b)."""
    q, k, beta = (np.asarray(x, np.float64) for x in (q, k, beta))
    g = None if g is None else np.asarray(g, np.float64)
    if flags & NORMALIZE_QK:
        q, k = l2_normalize(q, mutant), l2_normalize(k, mutant)
    if flags & BETA_SIGMOID:
        beta = sigmoid(-beta if mutant == 2 else beta)
    if (flags & GATE_LOGSIGMOID) and g is not None:
        g = log_sigmoid(g)
    return q, k, g, beta
