"""The seeded input generators reproduce their stated laws (CPU only)."""
import numpy as np

from kda_workloads import (bf16_bits, bf16_round, bf16_to_f32, make_config,
                           make_inputs, CONFIGS)


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 3.0e38, 1e-40], np.float32)
    r = bf16_round(x)
    assert r[0] == 1.0
    assert r[1] == 1.0                       # tie -> even
    assert r[2] == np.float32(1.0 + 2 ** -7)  # tie -> even (up)
    assert r[3] == -2.5
    assert np.array_equal(bf16_to_f32(bf16_bits(r)), r)


def test_seeded_and_deterministic():
    a = make_inputs(1, 8, 2, 16, 16, seed=3)
    b = make_inputs(1, 8, 2, 16, 16, seed=3)
    c = make_inputs(1, 8, 2, 16, 16, seed=4)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.g, b.g)
    assert not np.array_equal(a.q, c.q)


def test_key_normalisation_and_gate_range():
    w = make_inputs(1, 256, 4, 128, 128, dtype="f32", seed=0, gate_shift=2.0)
    n = np.linalg.norm(w.k.astype(np.float64), axis=-1)
    assert np.abs(n - 1).max() < 1e-5
    assert (w.g <= 0).all() and (w.beta > 0).all() and (w.beta < 1).all()
    # -softplus(z + 2): median alpha = exp(-softplus(2)) ~ 0.12
    assert abs(np.median(np.exp(w.g)) - np.exp(-np.log1p(np.exp(2.0)))) < 0.01


def test_config_laws_small():
    w = make_config("tiny_f32")
    assert w.q.dtype == np.float32 and w.h0 is None and w.g.shape == (1, 64, 1, 16)
    m = make_config("train_b8_h32_t8192", B=1, T=512, H=2)
    a = np.exp(m.g[0])
    # even channels ~0.3, odd ~0.999 at the median
    assert abs(np.median(a[..., 0::2]) - 0.3) < 0.03
    assert abs(np.median(a[..., 1::2]) - 0.999) < 0.0005
    s = make_config("long_t65536_scalar", T=1024)
    assert s.g.shape == (1, 1024, 8)
    assert 0.99 < np.median(np.exp(s.g)) < 1.0
    n = make_config("long_t65536_none", T=64)
    assert n.g is None and n.beta.min() >= 0.1 and n.beta.max() <= 1.0
    d = make_config("decode_b256_h32", B=2, H=2)
    assert d.h0.shape == (2, 2, 128, 128) and abs(d.h0.std() - 0.05) < 0.002


def test_bf16_workloads_hold_exact_bf16_values():
    w = make_config("prefill_h16_t4096", T=128, H=2)
    for x in (w.q, w.k, w.v):
        assert np.array_equal(bf16_round(x), x)
    assert set(CONFIGS) >= {"tiny_f32", "prefill_h16_t4096", "decode_b256_h32",
                            "train_b8_h32_t8192", "long_t65536_channel"}


def test_cotangents_shapes_rounding_and_independence():
    from kda_workloads import make_cotangents, bf16_round
    w = make_inputs(2, 5, 3, 16, 32, dtype="bf16", seed=1)
    c = make_cotangents(w, seed=4, dhT_std=0.5)
    assert c.do.shape == (2, 5, 3, 32) and c.dhT.shape == (2, 3, 16, 32)
    np.testing.assert_array_equal(c.do, bf16_round(c.do))
    assert abs(float(c.dhT.std()) - 0.5) < 0.1
    c2 = make_cotangents(w, seed=4, dhT_std=0.5)
    np.testing.assert_array_equal(c.do, c2.do)
    assert make_cotangents(w, seed=5).dhT is None
    assert not np.array_equal(make_cotangents(w, seed=5).do, c.do)
