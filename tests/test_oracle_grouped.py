"""Pins of the grouped-value-head oracle (CPU only).

Value head h has its own state, gate, beta and values and reads query/key
head h // (H / Hqk) (GeekNews #31925, section "Fused recurrent kernel for
decode": programs run per value head).  Pinned against:
- per-head calls of oracle R built by slicing (a different code path from the
  head repetition inside the oracle);
- the ungrouped case, which must be oracle R itself;
- a planted mistake in the head mapping, which must fail the first pin.
"""
import numpy as np
import pytest

import oracle
from kda_workloads import make_inputs


def _grouped_inputs(Hqk, G, mode, Dk=8, Dv=6, seed=3):
    H = Hqk * G
    w = make_inputs(2, 11, H, Dk, Dv, mode=mode, dtype="f32", seed=seed, h0_std=0.3,
                    gate_law="softplus" if mode != "none" else "zero")
    q = np.ascontiguousarray(w.q[:, :, ::G])   # Hqk query/key heads
    k = np.ascontiguousarray(w.k[:, :, ::G])
    return w, q, k


@pytest.mark.parametrize("mode", ["channel", "scalar", "none"])
@pytest.mark.parametrize("Hqk,G", [(1, 4), (2, 3), (3, 1)])
def test_grouped_equals_per_head_calls(mode, Hqk, G):
    w, q, k = _grouped_inputs(Hqk, G, mode)
    o, hT = oracle.recurrent_grouped(q, k, w.v, w.g, w.beta, w.h0, scale=w.scale, mode=mode)
    for h in range(Hqk * G):
        hq = h // G
        sl = lambda x: None if x is None else np.ascontiguousarray(x[:, :, h:h + 1])
        o1, h1 = oracle.recurrent(q[:, :, hq:hq + 1], k[:, :, hq:hq + 1], sl(w.v), sl(w.g),
                                  sl(w.beta), w.h0[:, h:h + 1], scale=w.scale, mode=mode)
        assert np.array_equal(o[:, :, h], o1[:, :, 0])
        assert np.array_equal(hT[:, h], h1[:, 0])


def test_ungrouped_is_oracle_r():
    w = make_inputs(2, 9, 3, 8, 8, dtype="f32", seed=1, h0_std=0.2)
    a = oracle.recurrent_grouped(w.q, w.k, w.v, w.g, w.beta, w.h0, scale=w.scale)
    b = oracle.recurrent(w.q, w.k, w.v, w.g, w.beta, w.h0, scale=w.scale)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_planted_head_mapping_mistake_fails():
    w, q, k = _grouped_inputs(2, 3, "channel")
    o, hT = oracle.recurrent_grouped(q, k, w.v, w.g, w.beta, w.h0, scale=w.scale, mutant=1)
    ok = True
    for h in range(6):
        hq = h // 3
        sl = lambda x: np.ascontiguousarray(x[:, :, h:h + 1])
        o1, _ = oracle.recurrent(q[:, :, hq:hq + 1], k[:, :, hq:hq + 1], sl(w.v), sl(w.g),
                                 sl(w.beta), w.h0[:, h:h + 1], scale=w.scale)
        ok &= np.array_equal(o[:, :, h], o1[:, :, 0])
    assert not ok
