"""Pins of the prologue oracle (CPU only).

Closed forms and identities of the three transforms, checked against values
fixed by the mathematics rather than by re-evaluating the same formulas:
- a 3-4-5 vector normalises to (0.6, 0.8) up to the 1e-6 guard, and every
  row of a normalised tensor has norm sqrt(s / (s + 1e-6));
- sigmoid(0) = 1/2, log sigmoid(0) = -log 2, and the identity
  log sigmoid(x) - log sigmoid(-x) = x; the tails log sigmoid(-60) = -60
  and log sigmoid(60) = -exp(-60) to rounding;
- exp(log sigmoid(a)) equals the logistic function evaluated as e^a/(1+e^a);
- normalising already-unit keys changes the oracle's outputs by < 1e-5;
- planted mistakes (norm over the wrong axis, sigmoid of -b) fail a pin.
"""
import math

import numpy as np
import pytest

import oracle
from oracle.prologue import (BETA_SIGMOID, GATE_LOGSIGMOID, NORMALIZE_QK, NORM_EPS,
                             l2_normalize, log_sigmoid, sigmoid)
from kda_workloads import make_inputs
from tests.conftest import rel_err


def test_l2_normalize_closed_form():
    x = np.array([[3.0, 4.0]])
    y = l2_normalize(x)
    assert np.allclose(y, [[0.6, 0.8]], rtol=0, atol=1e-7)
    r = np.random.default_rng(0).standard_normal((5, 3, 16))
    n = np.sqrt((l2_normalize(r) ** 2).sum(-1))
    s = (r ** 2).sum(-1)
    assert np.allclose(n, np.sqrt(s / (s + NORM_EPS)), rtol=1e-12)


def test_sigmoid_and_log_sigmoid():
    assert sigmoid(0.0) == 0.5
    assert abs(log_sigmoid(0.0) + math.log(2.0)) < 1e-15
    x = np.linspace(-30, 30, 121)
    assert np.allclose(log_sigmoid(x) - log_sigmoid(-x), x, rtol=0, atol=1e-12)
    assert abs(log_sigmoid(-60.0) + 60.0) < 1e-12
    assert abs(log_sigmoid(60.0) + math.exp(-60.0)) < 1e-30
    a = np.linspace(-20, 20, 81)
    assert np.allclose(np.exp(log_sigmoid(a)), np.exp(a) / (1.0 + np.exp(a)), rtol=1e-12)
    assert np.all(log_sigmoid(a) <= 0.0)


def test_normalising_unit_keys_is_harmless():
    w = make_inputs(1, 12, 2, 16, 8, dtype="f32", seed=4, h0_std=0.2)   # unit keys
    q = l2_normalize(w.q)
    o1, h1 = oracle.recurrent(q, w.k, w.v, w.g, w.beta, w.h0, scale=w.scale)
    qq, kk, g, b = oracle.apply_prologue(w.q, w.k, w.g, w.beta, NORMALIZE_QK)
    o2, h2 = oracle.recurrent(qq, kk, w.v, g, b, w.h0, scale=w.scale)
    # keys are unit to float32 precision; the 1e-6 guard moves each by ~5e-7
    assert rel_err(o2, o1) < 1e-5 and rel_err(h2, h1) < 1e-5


def test_flags_are_independent():
    w = make_inputs(1, 5, 2, 8, 8, dtype="f32", seed=2, preact=True)
    q0, k0, g0, b0 = oracle.apply_prologue(w.q, w.k, w.g, w.beta, 0)
    assert np.array_equal(q0, w.q) and np.array_equal(g0, w.g) and np.array_equal(b0, w.beta)
    q, k, g, b = oracle.apply_prologue(w.q, w.k, w.g, w.beta, BETA_SIGMOID)
    assert np.array_equal(q, q0) and np.array_equal(g, g0) and np.all((b > 0) & (b < 1))
    q, k, g, b = oracle.apply_prologue(w.q, w.k, w.g, w.beta, GATE_LOGSIGMOID)
    assert np.array_equal(b, b0) and np.all(g <= 0)


@pytest.mark.parametrize("mutant", [1, 2])
def test_planted_mistakes_fail(mutant):
    w = make_inputs(1, 4, 3, 8, 8, dtype="f32", seed=1, preact=True)
    q, k, g, b = oracle.apply_prologue(w.q, w.k, w.g, w.beta, 7, mutant=mutant)
    if mutant == 1:
        n = np.sqrt((k ** 2).sum(-1))
        assert not np.allclose(n, 1.0, atol=1e-5)
    else:
        assert not np.allclose(b, sigmoid(w.beta))
