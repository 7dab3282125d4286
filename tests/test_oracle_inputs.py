"""Pins of the oracle's input-side transforms (gate functions, q/k
normalisation, beta from logits) to closed forms and to the pages.

Sources cited:
  [DS] docsaid.org "Kimi Linear -- L'oubli canal par canal", section "Les
       autres pieces": q and k L2-normalised, beta = sigmoid of a projection,
       the decay from a gate function like GDN's and Mamba's.
  [RK] mkdocs.reaper.mx Kimi K3 "Attention lineaire et recurrence", section
       "Le piege numerique de la decroissance cumulee": Kimi Linear's
       g = -e^A softplus(z), unbounded; K3's scaled sigmoid bounded below by
       g_min = -5, so that each retention factor is at least e^-5 and a
       16-token tile's summed log-decay stays in (-80, 0).
Each test checks a value or an identity the mathematics fixes, not the
formula retyped.
"""
import math

import numpy as np

import oracle


def test_softplus_closed_forms():
    """softplus(0) = ln 2; softplus(ln(e - 1)) = 1; softplus(z) - softplus(-z)
    = z; softplus(z) -> z for large z and -> e^z for very negative z."""
    assert abs(oracle.softplus(0.0) - math.log(2.0)) < 1e-16
    assert abs(oracle.softplus(math.log(math.e - 1.0)) - 1.0) < 1e-15
    z = np.random.default_rng(0).standard_normal(1000) * 30
    np.testing.assert_allclose(oracle.softplus(z) - oracle.softplus(-z), z, rtol=0,
                               atol=1e-12)
    assert oracle.softplus(50.0) == 50.0
    assert abs(oracle.softplus(-50.0) / math.exp(-50.0) - 1.0) < 1e-14
    assert np.all(oracle.softplus(z) > 0)


def test_sigmoid_closed_forms():
    """sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(x) + sigmoid(-x) = 1."""
    assert oracle.sigmoid(0.0) == 0.5
    assert abs(oracle.sigmoid(math.log(3.0)) - 0.75) < 1e-16
    x = np.random.default_rng(1).standard_normal(500) * 10
    np.testing.assert_allclose(oracle.sigmoid(x) + oracle.sigmoid(-x), 1.0, rtol=0,
                               atol=1e-15)


def test_softplus_gate_retention_is_a_power():
    """[RK]: g = -e^A softplus(z), so the retention factor
    alpha = e^g = (1 + e^z)^(-e^A).  With A = ln 3 and z = 0 that is
    2^-3 = 1/8; with A = 0 it is 1 / (1 + e^z)."""
    z0 = np.zeros((1, 2, 4))
    g = oracle.gate_softplus(z0, np.array([math.log(3.0), 0.0]))
    np.testing.assert_allclose(np.exp(g[0, 0]), 0.125, rtol=1e-15)
    np.testing.assert_allclose(np.exp(g[0, 1]), 0.5, rtol=1e-15)
    z = np.random.default_rng(2).standard_normal((5, 3, 8))
    A = np.array([-1.0, 0.0, 0.7])
    alpha = np.exp(oracle.gate_softplus(z, A))
    np.testing.assert_allclose(alpha, (1.0 + np.exp(z)) ** (-np.exp(A)[:, None]),
                               rtol=1e-13)
    assert np.all(alpha < 1.0) and np.all(alpha > 0.0)   # unbounded below only


def test_sigmoid_gate_bounds_and_tile_range():
    """[RK]: g = g_min sigmoid(z) lies in (g_min, 0); with g_min = -5 every
    retention factor is above e^-5 (about 6.7e-3) and any 16 gates sum to
    more than -80."""
    z = np.random.default_rng(3).standard_normal((10000,)) * 4  # sigmoid unsaturated
    g = oracle.gate_sigmoid(z, -5.0)
    assert np.all(g > -5.0) and np.all(g < 0.0)
    gs = oracle.gate_sigmoid(np.array([-1e3, 1e3]), -5.0)     # saturated ends
    assert gs[0] == 0.0 and gs[1] == -5.0
    assert np.exp(g).min() > math.exp(-5.0)
    assert abs(math.exp(-5.0) - 6.7e-3) < 1e-4
    assert np.add.reduceat(g, np.arange(0, 10000, 16)).min() > -80.0
    assert oracle.gate_sigmoid(0.0, -5.0) == -2.5
    assert abs(oracle.gate_sigmoid(math.log(3.0), -4.0) - (-3.0)) < 1e-15


def test_l2_normalize_unit_norm_and_scale_invariance():
    """[DS]: q and k are L2-normalised per token and head.  (3, 4) -> (0.6,
    0.8) up to the 1e-6 guard; norms are 1 up to that guard; positive scaling
    of the input does not change the result."""
    x = oracle.l2_normalize(np.array([3.0, 4.0]))
    np.testing.assert_allclose(x, [0.6, 0.8], rtol=1e-7)
    r = np.random.default_rng(4).standard_normal((7, 3, 16)) * 5
    n = np.linalg.norm(oracle.l2_normalize(r), axis=-1)
    np.testing.assert_allclose(n, 1.0, rtol=0, atol=1e-6)
    np.testing.assert_allclose(oracle.l2_normalize(r * 9.0), oracle.l2_normalize(r),
                               rtol=0, atol=1e-8)
    assert np.all(oracle.l2_normalize(np.zeros(4)) == 0.0)


def test_prepare_inputs_defaults_are_identity_and_normalised_keys_erase():
    """With the default options prepare_inputs returns its inputs.  With raw
    (unnormalised) keys, beta = 1 from a large logit and l2norm_qk, the
    erase-then-write step reads back v ([RK] delta-rule section: beta = 1
    replaces; the erase operator is a projection only for unit keys)."""
    rng = np.random.default_rng(5)
    T, H, d = 6, 2, 8
    q, k = rng.standard_normal((T, H, d)), rng.standard_normal((T, H, d))
    g = -rng.random((T, H, d))
    b = rng.random((T, H))
    q2, k2, g2, b2 = oracle.prepare_inputs(q, k, g, b)
    for x, y in ((q, q2), (k, k2), (g, g2), (b, b2)):
        assert np.array_equal(x, y)
    v = rng.standard_normal((T, H, d))
    logits = np.full((T, H), 60.0)          # sigmoid(60) = 1 in fp64
    k3 = k * 7.0                            # raw keys, far from unit norm
    qn, kn, gn, bn = oracle.prepare_inputs(q, k3, g, logits, l2norm_qk=True,
                                           beta_logits=True)
    assert np.all(bn == 1.0)
    S0 = rng.standard_normal((1, H, d, d))
    _, S = oracle.recurrent(qn, kn, v, gn, bn, initial_state=S0)
    for h in range(H):
        np.testing.assert_allclose(S[0, h].T @ kn[-1, h], v[-1, h], rtol=0, atol=1e-6)


def test_rms_norm_unit_rms_and_scale_invariance():
    """[DS] "Les autres pieces": RMSNorm per head.  With unit weight the
    normalised row has root-mean-square 1 (up to eps); it does not depend on
    a positive scale of the row; the weight multiplies channel by channel;
    (3, 4) has RMS sqrt(12.5)."""
    rng = np.random.default_rng(6)
    o = rng.standard_normal((5, 3, 32)) * 4
    y = oracle.rms_norm(o, np.ones(32), 1e-12)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-10)
    np.testing.assert_allclose(oracle.rms_norm(o * 7.5, np.ones(32), 0.0),
                               oracle.rms_norm(o, np.ones(32), 0.0), rtol=1e-13)
    w = rng.random(32)
    np.testing.assert_allclose(oracle.rms_norm(o, w, 1e-6),
                               oracle.rms_norm(o, np.ones(32), 1e-6) * w, rtol=1e-14)
    np.testing.assert_allclose(oracle.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0),
                               np.array([3.0, 4.0]) / math.sqrt(12.5), rtol=1e-15)


def test_output_gate_halves_at_zero_and_passes_at_large_logits():
    """[DS]: the normalised output is multiplied by a sigmoid gate: a logit of
    0 halves it, a large logit passes it, no gate leaves it unchanged."""
    o = np.random.default_rng(7).standard_normal((4, 2, 16))
    w = np.ones(16)
    base = oracle.output_epilogue(o, w, 1e-6)
    np.testing.assert_array_equal(base, oracle.rms_norm(o, w, 1e-6))
    np.testing.assert_allclose(oracle.output_epilogue(o, w, 1e-6, np.zeros_like(o)),
                               0.5 * base, rtol=1e-15)
    np.testing.assert_allclose(oracle.output_epilogue(o, w, 1e-6, np.full_like(o, 60.0)),
                               base, rtol=1e-15)
