"""Oracle R against the pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as P
from tests.conftest import rel_err


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.recurrent)


def test_default_scale_is_inverse_sqrt_dk():
    """The read uses d_k^{-1/2} q_t by default (the fifth equation at the top
    of "You could have come up with Kimi Delta Attention")."""
    r = np.random.default_rng(0)
    q = r.standard_normal((1, 4, 1, 9)); k = r.standard_normal((1, 4, 1, 9))
    v = r.standard_normal((1, 4, 1, 2)); beta = r.uniform(0, 1, (1, 4, 1))
    g = -r.uniform(0, 1, (1, 4, 1, 9))
    o1, _ = oracle.recurrent(q, k, v, g, beta)
    o2, _ = oracle.recurrent(q / 3.0, k, v, g, beta, scale=1.0)
    assert np.abs(o1 - o2).max() < 1e-14


def test_batch_and_heads_are_independent():
    """Each (batch, head) pair is its own sequence: running the whole batch
    equals running each pair alone (the fused recurrent kernel of the
    GeekNews summary runs sequences and heads independently)."""
    r = np.random.default_rng(1)
    B, T, H, Dk, Dv = 2, 5, 3, 4, 3
    q = r.standard_normal((B, T, H, Dk)); k = r.standard_normal((B, T, H, Dk))
    v = r.standard_normal((B, T, H, Dv)); beta = r.uniform(0, 1, (B, T, H))
    g = -r.uniform(0, 1, (B, T, H, Dk)); h0 = r.standard_normal((B, H, Dk, Dv))
    o, hT = oracle.recurrent(q, k, v, g, beta, h0)
    for b in range(B):
        for h in range(H):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
            o1, h1 = oracle.recurrent(q[sl], k[sl], v[sl], g[sl], beta[sl],
                                      h0[b:b + 1, h:h + 1])
            assert np.abs(o1[:, :, 0] - o[b:b + 1, :, h]).max() == 0.0
            assert np.abs(h1[0, 0] - hT[b, h]).max() == 0.0


def test_threads_do_not_change_results():
    r = np.random.default_rng(2)
    B, T, H, Dk, Dv = 3, 17, 4, 8, 8
    q = r.standard_normal((B, T, H, Dk)); k = r.standard_normal((B, T, H, Dk))
    v = r.standard_normal((B, T, H, Dv)); beta = r.uniform(0, 1, (B, T, H))
    g = -r.uniform(0, 1, (B, T, H, Dk))
    o1, h1 = oracle.recurrent(q, k, v, g, beta, threads=1)
    o2, h2 = oracle.recurrent(q, k, v, g, beta, threads=4)
    assert rel_err(o2, o1) == 0.0 and rel_err(h2, h1) == 0.0


def test_empty_sequence_returns_initial_state():
    r = np.random.default_rng(3)
    h0 = r.standard_normal((2, 3, 4, 5))
    z = np.zeros((2, 0, 3, 4))
    o, hT = oracle.recurrent(z, z, np.zeros((2, 0, 3, 5)), np.zeros((2, 0, 3, 4)),
                             np.zeros((2, 0, 3)), h0)
    assert o.shape == (2, 0, 3, 5)
    assert np.array_equal(hT, h0)


def test_hard_forget_gate_clears_state():
    """Gate boundary (the F29 outline names a hand-set gate boundary probe):
    a log-gate of -30 forgets the state up to e^-30, g = 0 keeps it exactly."""
    r = np.random.default_rng(4)
    Dk = Dv = 4
    h0 = r.standard_normal((1, 1, Dk, Dv))
    k = np.zeros((1, 1, 1, Dk)); v = np.zeros((1, 1, 1, Dv))
    q = r.standard_normal((1, 1, 1, Dk)); beta = np.ones((1, 1, 1))
    _, hT = oracle.recurrent(q, k, v, np.full((1, 1, 1, Dk), -30.0), beta, h0)
    assert np.abs(hT).max() <= np.abs(h0).max() * np.exp(-30.0) * (1 + 1e-12)
    _, hT = oracle.recurrent(q, k, v, np.zeros((1, 1, 1, Dk)), beta, h0)
    assert np.array_equal(hT, h0)
