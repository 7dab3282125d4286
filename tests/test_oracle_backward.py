"""Pins of the oracle's backward (oracle.recurrent_backward, torch autograd
over the fp64 recurrence) to central finite differences of the C oracle's
forward and to closed forms.

Sources: fr.news.hada.io Kimi Linear summary, section "Algorithme parallele
par chunks" (training is what the chunk form is for); [RK] mkdocs.reaper.mx
"Attention lineaire et recurrence", section "Kimi Delta Attention = les trois
remedes combines" (the recurrence differentiated).
"""
import numpy as np
import pytest

import oracle


def _case(seed, T, H, dk, dv, n=1, s0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -rng.random((T, H, dk))
    b = rng.random((T, H))
    S0 = rng.standard_normal((n, H, dk, dv)) if s0 else None
    do = rng.standard_normal((T, H, dv))
    dsf = rng.standard_normal((n, H, dk, dv))
    return q, k, v, g, b, S0, do, dsf


def _loss(q, k, v, g, b, S0, do, dsf, cu=None, n=None):
    o, sf = oracle.recurrent(q, k, v, g, b, cu_seqlens=cu, num_seqs=n, initial_state=S0)
    return float(np.sum(o * do) + np.sum(sf * dsf))


@pytest.mark.parametrize("varlen", [False, True])
def test_backward_matches_central_differences(varlen):
    """Every gradient against (L(x + h e) - L(x - h e)) / 2h of the C
    oracle's forward, on all entries of a tiny problem (packed sequences with
    a tail when varlen)."""
    T, H, dk, dv = 7, 2, 3, 2
    cu = np.array([0, 3, 7]) if varlen else None
    n = 2 if varlen else 1
    q, k, v, g, b, S0, do, dsf = _case(11 + varlen, T, H, dk, dv, n=n)
    grads = oracle.recurrent_backward(q, k, v, g, b, do, dsf, cu_seqlens=cu, num_seqs=n,
                                      initial_state=S0)
    args = dict(q=q, k=k, v=v, g=g, b=b, S0=S0)
    names = dict(q="dq", k="dk", v="dv", g="dg", b="dbeta", S0="ds0")
    h = 1e-6
    for name, x in args.items():
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            a1 = dict(args, **{name: xp}); a2 = dict(args, **{name: xm})
            num[idx] = (_loss(a1["q"], a1["k"], a1["v"], a1["g"], a1["b"], a1["S0"], do, dsf,
                              cu, n) -
                        _loss(a2["q"], a2["k"], a2["v"], a2["g"], a2["b"], a2["S0"], do, dsf,
                              cu, n)) / (2 * h)
        np.testing.assert_allclose(grads[names[name]], num, rtol=1e-6, atol=1e-8,
                                   err_msg=f"d{name}")


def test_backward_one_token_closed_form():
    """One token from a zero state: o = beta (k . q) v, so for L = r . o:
    dq = beta (v . r) k, dk = beta (v . r) q, dv = beta (k . q) r,
    dbeta = (k . q)(v . r), dg = 0 (the decay acts on a zero state)."""
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((1, 1, 4)), rng.standard_normal((1, 1, 4))
    v, r = rng.standard_normal((1, 1, 3)), rng.standard_normal((1, 1, 3))
    g, b = -rng.random((1, 1, 4)), np.array([[0.7]])
    gr = oracle.recurrent_backward(q, k, v, g, b, r)
    kq, vr = float(k[0, 0] @ q[0, 0]), float(v[0, 0] @ r[0, 0])
    np.testing.assert_allclose(gr["dq"][0, 0], 0.7 * vr * k[0, 0], rtol=1e-14)
    np.testing.assert_allclose(gr["dk"][0, 0], 0.7 * vr * q[0, 0], rtol=1e-14)
    np.testing.assert_allclose(gr["dv"][0, 0], 0.7 * kq * r[0, 0], rtol=1e-14)
    np.testing.assert_allclose(gr["dbeta"][0, 0], kq * vr, rtol=1e-14)
    assert np.all(gr["dg"] == 0.0)


def test_backward_forward_agrees_with_c_oracle():
    """The torch forward used for the gradient is the C oracle's recurrence."""
    import torch
    T, H, dk, dv = 9, 2, 4, 3
    q, k, v, g, b, S0, do, dsf = _case(5, T, H, dk, dv)
    tt = lambda a: torch.tensor(a)
    o, sf = oracle._torch_recurrent(tt(q), tt(k), tt(v), tt(g), tt(b), [(0, T)], tt(S0))
    o_c, sf_c = oracle.recurrent(q, k, v, g, b, initial_state=S0)
    np.testing.assert_allclose(o.numpy(), o_c, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sf.numpy(), sf_c, rtol=0, atol=1e-13)
