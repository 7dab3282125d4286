"""The method's degenerate cases on the GPU path, against the oracle and,
where one exists, a closed form.

Sources: mkdocs.reaper.mx "Attention lineaire et recurrence": section
"Remede 1" (beta = 0 writes nothing, the state only decays), "Remede 2"
(beta = 1 replaces the value stored under a unit key), section "Le piege
numerique de la decroissance cumulee" (the in-chunk decay range);
fr.news.hada.io Kimi Linear summary, section "De l'attention lineaire a
Gated DeltaNet" (alpha = 1 is the plain delta rule).  The inputs are the
seeded workload draws with beta or g overwritten by constants.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from gated_delta_rule_chunked_amd import inputs as kin  # noqa: E402
from kda_testutil import TOL, from_device, relerr, upload_prefill  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [(kin.BF16, 128, 64), (kin.F32, 64, 32), (kin.F32, 32, 16)]


def _kda():
    import gated_delta_rule_chunked_amd as kda
    return kda


def _workload(seed, dtype, d, chunk, s0=True):
    return kin.make_prefill(seed, H=2, d=d, dtype=dtype, chunk_size=chunk,
                            lengths=[150, 1, 97], s0_std=0.05 if s0 else None)


def _run(w, flags=None):
    kda = _kda()
    dd = upload_prefill(w)
    o, s = kda.fwd_chunked(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"],
                           cu_seqlens=dd["cu_seqlens"], initial_state=dd["initial_state"],
                           chunk_size=w.chunk_size, flags=flags)
    torch.cuda.synchronize()
    return from_device(o), from_device(s)


def _check_oracle(w, o, s):
    q, k, v, g, b, s0 = w.f64()
    ro, rs = oracle.recurrent(q, k, v, g, b, cu_seqlens=w.cu_seqlens.astype(np.int64),
                              num_seqs=w.num_seqs, initial_state=s0)
    eo, es = relerr(o, ro), relerr(s, rs)
    print(f"  relerr o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]


@pytest.mark.parametrize("dtype,d,chunk", CASES)
def test_beta_zero_only_decays(dtype, d, chunk):
    """beta = 0: nothing is written; the final state is the initial state
    decayed channel by channel, S_N = Diag(exp(sum g)) S_0."""
    print(f"[degenerate] beta=0 {dtype} d={d} C={chunk}", flush=True)
    w = _workload(700 + d, dtype, d, chunk)
    w.beta[:] = 0.0
    o, s = _run(w)
    _check_oracle(w, o, s)
    cu = w.cu_seqlens
    for i in range(w.num_seqs):
        decay = np.exp(w.g[cu[i]:cu[i + 1]].astype(np.float64).sum(axis=0))  # [H, d]
        closed = decay[:, :, None] * w.initial_state[i].astype(np.float64)
        assert relerr(s[i], closed) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,chunk", CASES)
def test_alpha_one_is_the_delta_rule(dtype, d, chunk):
    """g = 0 (alpha = 1): no decay at all."""
    print(f"[degenerate] g=0 {dtype} d={d} C={chunk}", flush=True)
    w = _workload(710 + d, dtype, d, chunk)
    w.g[:] = 0.0
    _check_oracle(w, *_run(w))


@pytest.mark.parametrize("dtype,d,chunk", CASES)
def test_beta_one_with_q_equal_k_reads_back_v(dtype, d, chunk):
    """beta = 1 and q = k (unit keys): each token's output is the value it
    just wrote, o_t = v_t, whatever the state and the decay."""
    print(f"[degenerate] beta=1 q=k {dtype} d={d} C={chunk}", flush=True)
    w = _workload(720 + d, dtype, d, chunk)
    w.beta[:] = 1.0
    w.q[:] = w.k
    o, s = _run(w)
    _check_oracle(w, o, s)
    assert relerr(o, kin.as_f64(w.v, dtype)) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,chunk", CASES)
def test_decay_just_inside_the_chunk_bound(dtype, d, chunk):
    """Every channel decays so that a full chunk sums to -76.8, just inside
    the -80 bound of the chunk-start reference: results still match the
    oracle and the decay-range flag stays clear."""
    print(f"[degenerate] strong decay {dtype} d={d} C={chunk}", flush=True)
    w = _workload(730 + d, dtype, d, chunk)
    w.g[:] = -76.8 / chunk
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, s = _run(w, flags=flags)
    assert int(flags.item()) == 0
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    _check_oracle(w, o, s)
