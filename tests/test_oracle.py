"""Pins of the fp64 oracle to what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a value the
pages print (tests/golden/), a closed form, a special case that reduces to a
differently derived rule, a library routine, or brute-force dense products on
tiny inputs.  Together they catch a dropped term, a wrong sign or index, a
transposed state or the wrong order of decay and erase.

Sources cited:
  [DS] docsaid.org "Kimi Linear -- L'oubli canal par canal", KDA section
       (GDN and KDA updates, two-channel decay table), cache section.
  [GN] fr.news.hada.io summary of Kimi Linear, sections on DeltaNet/GDN and
       on the chunk-parallel algorithm.
  [RK] mkdocs.reaper.mx Kimi K3 "Attention lineaire et recurrence", sections
       on the associative memory, decay, delta rule, chunkwise form,
       cumulative decay and the M_t operator.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def relerr(x, ref):
    """Normwise max relative error max|x - ref| / max|ref|."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / (den if den > 0 else 1.0))


def _rand_inputs(rng, T, H, dk, dv, g_scale=0.3):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -g_scale * rng.random((T, H, dk)) * 2.0
    beta = rng.random((T, H))
    return q, k, v, g, beta


# --------------------------------------------------------------------------
# Values printed on the pages
# --------------------------------------------------------------------------

def test_decay_table_worked_example():
    """[DS] KDA section table: the forget step alone (beta = 0 so nothing is
    erased or written) turns the state (8, 6) into (4, 3) under scalar 0.5
    and into (8, 0.6) under per-channel (1.0, 0.1)."""
    fx = _golden("decay_table.json")
    S0 = np.array(fx["state_before"]).reshape(1, 1, 2, 1)
    for case in fx["cases"]:
        g = np.log(np.array(case["alpha"])).reshape(1, 1, 2)
        k = np.array([0.6, 0.8]).reshape(1, 1, 2)
        q = np.array([1.0, 0.0]).reshape(1, 1, 2)
        v = np.array([5.0]).reshape(1, 1, 1)
        beta = np.zeros((1, 1))
        o, S = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
        np.testing.assert_allclose(S.reshape(2), case["state_after"], rtol=1e-15)
        # read-out on the decayed state, row 1 selected by q
        np.testing.assert_allclose(o.reshape(1), case["state_after"][0], rtol=1e-15)
        od, Sd = oracle.decode(q, k, v, g, beta, S0)
        np.testing.assert_allclose(Sd.reshape(2), case["state_after"], rtol=1e-15)


def test_cumulative_decay_example():
    """[RK] cumulative-decay section: alpha = 0.5 over 64 tokens gives a
    cumulative decay of about 5e-20 and an inverse of about 2e19."""
    fx = _golden("cumulative_decay.json")
    n = fx["tokens"]
    g = np.full((n, 1, 3), math.log(fx["alpha"]))
    G = oracle.chunk_cumsum(g, chunk_size=n)
    gamma = math.exp(G[-1, 0, 0])
    # matches the printed one-significant-figure values
    assert float(f"{gamma:.0e}") == fx["gamma_printed"]
    assert float(f"{1.0 / gamma:.0e}") == fx["inverse_gamma_printed"]
    # and the exact value 2^-64 (log-sum of 64 equal terms)
    assert abs(G[-1, 0, 0] - n * math.log(0.5)) <= 1e-12 * n


def test_state_sizes():
    """[DS] cache section printed output and [RK] state-size question: one
    head's state holds 128 x 128 = 16384 values; 20 layers x 32 heads hold
    10,485,760 values, 20 MiB in bf16.  Checks the oracle's state shape."""
    fx = _golden("state_sizes.json")
    d = fx["head_dim"]
    H = fx["heads_per_layer"]
    rng = np.random.default_rng(0)
    q, k, v, g, beta = _rand_inputs(rng, 1, H, d, d)
    _, S = oracle.recurrent(q, k, v, g, beta)
    assert S.shape == (1, H, d, d)
    assert S[0, 0].size == fx["values_per_head"]
    assert fx["kda_layers"] * S.size == fx["values_all_layers"]
    assert fx["kda_layers"] * S.size * 2 == fx["bf16_mib_all_layers"] * 2**20


# --------------------------------------------------------------------------
# Closed forms and special cases
# --------------------------------------------------------------------------

def test_beta_one_unit_key_reads_back_v():
    """[RK] delta-rule section: beta = 1 replaces completely.  After a write
    with beta = 1 and a unit key, S^T k equals v whatever the previous state
    and decay were."""
    rng = np.random.default_rng(1)
    for trial in range(5):
        dk, dv, T = 6, 4, 5
        q, k, v, g, beta = _rand_inputs(rng, T, 1, dk, dv)
        beta[-1] = 1.0
        S0 = rng.standard_normal((1, 1, dk, dv))
        _, S = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
        readback = S[0, 0].T @ k[-1, 0]
        np.testing.assert_allclose(readback, v[-1, 0], rtol=0, atol=1e-14)


def test_query_equal_key_reads_v():
    """Read-out after the update: with q_t = k_t (unit) and beta_t = 1 the
    output is exactly v_t."""
    rng = np.random.default_rng(2)
    dk, dv, T = 8, 5, 7
    q, k, v, g, beta = _rand_inputs(rng, T, 1, dk, dv)
    q = k.copy()
    beta[:] = 1.0
    o, _ = oracle.recurrent(q, k, v, g, beta,
                            initial_state=rng.standard_normal((1, 1, dk, dv)))
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-14)


@pytest.mark.parametrize("partial_beta", [False, True])
def test_orthonormal_keys_exact_retrieval(partial_beta):
    """[RK] associative-memory section: with orthonormal keys the read-out
    S^T k_i returns v_i exactly.  No decay (alpha = 1), empty initial state;
    with beta_i < 1 the memory holds beta_i v_i."""
    rng = np.random.default_rng(3)
    dk, dv = 8, 6
    n = dk
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm.T[:n].reshape(n, 1, dk)
    v = rng.standard_normal((n, 1, dv))
    q = rng.standard_normal((n, 1, dk))
    g = np.zeros((n, 1, dk))
    beta = rng.random((n, 1)) if partial_beta else np.ones((n, 1))
    _, S = oracle.recurrent(q, k, v, g, beta)
    for i in range(n):
        np.testing.assert_allclose(S[0, 0].T @ k[i, 0], beta[i, 0] * v[i, 0],
                                   rtol=0, atol=1e-13)


def test_alpha_one_is_deltanet_online_gradient_descent():
    """[GN] DeltaNet: online gradient descent on the reconstruction loss
    L(S) = 1/2 |S^T k - v|^2 with step beta.  With alpha = 1 KDA must equal
    S <- S - beta * dL/dS, where dL/dS = k (S^T k - v)^T."""
    rng = np.random.default_rng(4)
    T, dk, dv = 12, 5, 3
    q, k, v, _, beta = _rand_inputs(rng, T, 1, dk, dv)
    g = np.zeros((T, 1, dk))
    S0 = rng.standard_normal((dk, dv))
    o, Sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0.reshape(1, 1, dk, dv))
    S = S0.copy()
    for t in range(T):
        kt, vt = k[t, 0], v[t, 0]
        grad = np.outer(kt, S.T @ kt - vt)
        S = S - beta[t, 0] * grad
        assert relerr(o[t, 0], S.T @ q[t, 0]) < 1e-13
    assert relerr(Sf[0, 0], S) < 1e-13


def test_scalar_alpha_is_gated_deltanet():
    """[DS] first display equation (GDN): S_t = alpha_t (I - beta k k^T) S +
    beta k v^T with a scalar alpha_t.  KDA with the same value on every
    channel must reproduce it."""
    rng = np.random.default_rng(5)
    T, dk, dv = 10, 6, 4
    q, k, v, _, beta = _rand_inputs(rng, T, 1, dk, dv)
    a = np.exp(-rng.random(T))
    g = np.repeat(np.log(a)[:, None, None], dk, axis=2)
    S0 = rng.standard_normal((dk, dv))
    o, Sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0.reshape(1, 1, dk, dv))
    S = S0.copy()
    I = np.eye(dk)
    for t in range(T):
        kt = k[t, 0]
        S = a[t] * (I - beta[t, 0] * np.outer(kt, kt)) @ S + beta[t, 0] * np.outer(kt, v[t, 0])
        assert relerr(o[t, 0], S.T @ q[t, 0]) < 1e-13
    assert relerr(Sf[0, 0], S) < 1e-13


def test_pure_decay_closed_form():
    """[RK] decay section: after n steps an old entry is attenuated by
    alpha^n.  beta = 0 (no erase, no write), constant per-channel alpha."""
    rng = np.random.default_rng(6)
    n, dk, dv = 37, 5, 3
    alpha = rng.random(dk) * 0.5 + 0.5
    g = np.tile(np.log(alpha), (n, 1, 1))
    q, k, v, _, _ = _rand_inputs(rng, n, 1, dk, dv)
    beta = np.zeros((n, 1))
    S0 = rng.standard_normal((dk, dv))
    _, Sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0.reshape(1, 1, dk, dv))
    expected = (alpha ** n)[:, None] * S0
    assert relerr(Sf[0, 0], expected) < 1e-13


def test_dense_operator_form_and_order_of_decay_and_erase():
    """[DS] second display equation and [RK] M_t operator, brute force on a
    tiny state: S_t = M_t S_{t-1} + beta k v^T with the dense matrix
    M_t = (I - beta k k^T) Diag(alpha).  The other order, Diag(alpha)(I -
    beta k k^T), must give a different answer, so the test can tell them
    apart."""
    rng = np.random.default_rng(7)
    T, dk, dv = 9, 4, 3
    q, k, v, g, beta = _rand_inputs(rng, T, 1, dk, dv, g_scale=1.0)
    S0 = rng.standard_normal((dk, dv))
    o, Sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0.reshape(1, 1, dk, dv))
    S = S0.copy()
    Sw = S0.copy()
    I = np.eye(dk)
    for t in range(T):
        kt, bt = k[t, 0], beta[t, 0]
        D = np.diag(np.exp(g[t, 0]))
        M = (I - bt * np.outer(kt, kt)) @ D
        S = M @ S + bt * np.outer(kt, v[t, 0])
        Sw = D @ (I - bt * np.outer(kt, kt)) @ Sw + bt * np.outer(kt, v[t, 0])
        assert relerr(o[t, 0], S.T @ q[t, 0]) < 1e-13
    assert relerr(Sf[0, 0], S) < 1e-13
    assert relerr(Sf[0, 0], Sw) > 1e-3


def test_segment_pair_composition():
    """[RK] context-parallel question: a segment acts on its incoming state
    through the cumulative transition M (product of the M_t) plus a locally
    generated state S~ (the segment run from zero).  The oracle's final state
    from any S_in must equal M S_in + S~, with M built from dense products."""
    rng = np.random.default_rng(8)
    T, dk, dv = 11, 5, 4
    q, k, v, g, beta = _rand_inputs(rng, T, 1, dk, dv, g_scale=0.5)
    I = np.eye(dk)
    M = I.copy()
    for t in range(T):
        kt = k[t, 0]
        M = (I - beta[t, 0] * np.outer(kt, kt)) @ np.diag(np.exp(g[t, 0])) @ M
    _, S_loc = oracle.recurrent(q, k, v, g, beta)
    for _ in range(3):
        S_in = rng.standard_normal((1, 1, dk, dv))
        _, Sf = oracle.recurrent(q, k, v, g, beta, initial_state=S_in)
        assert relerr(Sf[0, 0], M @ S_in[0, 0] + S_loc[0, 0]) < 1e-13


def test_columns_of_state_are_independent():
    """Every factor multiplies the state from the left, so column j of S
    (and of o) depends only on column j of v and of S0.  Running the oracle on
    a subset of value columns must give those columns exactly."""
    rng = np.random.default_rng(9)
    T, H, dk, dv = 20, 2, 6, 5
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dk, dv))
    o, Sf = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
    cols = [1, 3]
    o2, Sf2 = oracle.recurrent(q, k, v[:, :, cols], g, beta,
                               initial_state=S0[..., cols])
    np.testing.assert_array_equal(o2, o[:, :, cols])
    np.testing.assert_array_equal(Sf2, Sf[..., cols])


# --------------------------------------------------------------------------
# UT transform / forward substitution
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 7, 16, 64])
def test_ut_inverse_forward_substitution(n):
    """[GN] chunk algorithm: (I + A)^{-1} for strictly lower A by forward
    substitution.  Checked against (I + A) T = I and LAPACK's triangular
    solve."""
    rng = np.random.default_rng(10 + n)
    A = np.tril(rng.standard_normal((n, n)) * 0.3, -1)
    junk = np.triu(rng.standard_normal((n, n)), 0)  # must be ignored
    Tm = oracle.ut_inverse(A + junk)
    I = np.eye(n)
    np.testing.assert_allclose((I + A) @ Tm, I, atol=1e-12)
    ref = scipy.linalg.solve_triangular(I + A, I, lower=True, unit_diagonal=True)
    np.testing.assert_allclose(Tm, ref, rtol=1e-12, atol=1e-13)
    assert np.all(np.triu(Tm, 1) == 0) and np.all(np.diag(Tm) == 1)


# --------------------------------------------------------------------------
# Chunked form, hand-off, varlen, decode
# --------------------------------------------------------------------------

def _varlen_case(rng, lengths, H, dk, dv, with_s0=True):
    T = int(sum(lengths))
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv, g_scale=0.4)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    S0 = rng.standard_normal((len(lengths), H, dk, dv)) * 0.1 if with_s0 else None
    return q, k, v, g, beta, cu, S0


@pytest.mark.parametrize("C", [1, 7, 16, 64, 100, 128])
def test_chunked_equals_recurrent(C):
    """[RK] chunkwise section: the block form is exact; [GN] chunk algorithm
    (state hand-off between chunks, WY/UT factors).  Ragged tails included."""
    rng = np.random.default_rng(20 + C)
    q, k, v, g, beta = _rand_inputs(rng, 100, 2, 8, 6)
    S0 = rng.standard_normal((1, 2, 8, 6))
    o_r, S_r = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
    o_c, S_c = oracle.chunked(q, k, v, g, beta, C, initial_state=S0)
    assert relerr(o_c, o_r) < 1e-12
    assert relerr(S_c, S_r) < 1e-12


def test_chunked_equals_recurrent_varlen_with_empty_sequence():
    """Chunks never straddle sequences; an empty sequence returns its
    initial state and writes no output rows."""
    rng = np.random.default_rng(30)
    lengths = [37, 0, 1, 64, 70]
    q, k, v, g, beta, cu, S0 = _varlen_case(rng, lengths, 3, 8, 8)
    o_r, S_r = oracle.recurrent(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0)
    for C in (16, 64):
        o_c, S_c = oracle.chunked(q, k, v, g, beta, C, cu_seqlens=cu, initial_state=S0)
        assert relerr(o_c, o_r) < 1e-12
        assert relerr(S_c, S_r) < 1e-12
    np.testing.assert_array_equal(S_r[1], S0[1])


def test_varlen_packed_equals_per_sequence():
    rng = np.random.default_rng(31)
    lengths = [5, 17, 33]
    q, k, v, g, beta, cu, S0 = _varlen_case(rng, lengths, 2, 6, 4)
    o, S = oracle.recurrent(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0)
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        o1, S1 = oracle.recurrent(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b],
                                  initial_state=S0[n:n + 1])
        np.testing.assert_array_equal(o1, o[a:b])
        np.testing.assert_array_equal(S1[0], S[n])


def test_equal_length_null_cu_seqlens_matches_explicit():
    rng = np.random.default_rng(32)
    q, k, v, g, beta = _rand_inputs(rng, 40, 2, 4, 4)
    cu = np.array([0, 20, 40])
    a = oracle.recurrent(q, k, v, g, beta, num_seqs=2)
    b = oracle.recurrent(q, k, v, g, beta, cu_seqlens=cu)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    c = oracle.chunked(q, k, v, g, beta, 16, num_seqs=2)
    assert relerr(c[0], a[0]) < 1e-12 and relerr(c[1], a[1]) < 1e-12


@pytest.mark.parametrize("split", [1, 16, 29])
def test_state_handoff_split_call(split):
    """[GN] chunk algorithm: the final state of one part is the initial state
    of the next.  Two calls with the state carried equal one call."""
    rng = np.random.default_rng(40 + split)
    q, k, v, g, beta = _rand_inputs(rng, 48, 2, 8, 8)
    S0 = rng.standard_normal((1, 2, 8, 8))
    o, S = oracle.recurrent(q, k, v, g, beta, initial_state=S0)
    oa, Sa = oracle.recurrent(q[:split], k[:split], v[:split], g[:split],
                              beta[:split], initial_state=S0)
    ob, Sb = oracle.recurrent(q[split:], k[split:], v[split:], g[split:],
                              beta[split:], initial_state=Sa)
    np.testing.assert_array_equal(np.concatenate([oa, ob]), o)
    np.testing.assert_array_equal(Sb, S)
    oc, Sc = oracle.chunked(q[:split], k[:split], v[:split], g[:split],
                            beta[:split], 16, initial_state=S0)
    od, Sd = oracle.chunked(q[split:], k[split:], v[split:], g[split:],
                            beta[split:], 16, initial_state=Sc)
    assert relerr(np.concatenate([oc, od]), o) < 1e-12
    assert relerr(Sd, S) < 1e-12


def test_decode_equals_one_token_prefill():
    rng = np.random.default_rng(50)
    B, H, d = 3, 2, 8
    q, k, v, g, beta = _rand_inputs(rng, B, H, d, d)
    state = rng.standard_normal((B, H, d, d))
    o, st = oracle.decode(q, k, v, g, beta, state)
    for b in range(B):
        o1, S1 = oracle.recurrent(q[b:b + 1], k[b:b + 1], v[b:b + 1], g[b:b + 1],
                                  beta[b:b + 1], initial_state=state[b:b + 1])
        np.testing.assert_array_equal(o1[0], o[b])
        np.testing.assert_array_equal(S1[0], st[b])


def test_chunk_cumsum_restarts_at_chunk_and_sequence_starts():
    g = -np.ones((40, 1, 2))
    cu = np.array([0, 25, 40])
    G = oracle.chunk_cumsum(g, 16, cu_seqlens=cu)
    expected = []
    for a, b in zip(cu[:-1], cu[1:]):
        for t in range(a, b):
            expected.append(-((t - a) % 16 + 1))
    np.testing.assert_array_equal(G[:, 0, 0], np.array(expected, dtype=float))


def test_rejects_bad_arguments():
    rng = np.random.default_rng(60)
    q, k, v, g, beta = _rand_inputs(rng, 10, 1, 4, 4)
    with pytest.raises(ValueError):
        oracle.recurrent(q, k, v, g, beta, num_seqs=3)  # 10 % 3 != 0
    with pytest.raises(ValueError):
        oracle.recurrent(q, k, v, g, beta, cu_seqlens=[0, 6, 5, 10])
    with pytest.raises(ValueError):
        oracle.recurrent(q, k, v, g, beta, cu_seqlens=[0, 4, 9])
