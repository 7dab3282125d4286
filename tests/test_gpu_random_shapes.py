"""Seeded random shapes: prefill (forward and, for every third case, the
backward) against the fp64 oracle at the operator's tolerances.

Each case draws a dtype, head size, chunk size, head count and a packed
set of sequence lengths (empty and one-token sequences, tails of every
size, several chunks) from a fixed seed, so the cases are the same on
every run; the inputs themselves come from the shared seeded generators.
Sources: fr.news.hada.io Kimi Linear summary, section "Algorithme
parallele par chunks" (chunked form); docsaid.org "Kimi Linear", section
"KDA : une decroissance propre a chaque canal" (the recurrence).
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from gated_delta_rule_chunked_amd import inputs as kin  # noqa: E402
from kda_testutil import TOL, from_device, relerr, to_device, f32_device, upload_prefill  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = kin.BF16 if rng.random() < 0.6 else kin.F32
        d = int(rng.choice([32, 64, 128]))
        chunk = int(rng.choice([16, 32, 64]))
        H = int(rng.integers(1, 5))
        N = int(rng.integers(1, 7))
        lengths = [int(x) for x in rng.integers(0, 3 * chunk + 8, size=N)]
        lengths[int(rng.integers(0, N))] = int(rng.choice([0, 1, chunk, chunk + 1]))
        if sum(lengths) == 0:
            lengths[0] = chunk + 3
        s0 = bool(rng.random() < 0.7)
        out.append((i, dtype, d, chunk, H, lengths, s0))
    return out


CASES = _cases()


def _kda():
    import gated_delta_rule_chunked_amd as kda
    return kda


@pytest.mark.parametrize("case", CASES, ids=[f"case{c[0]}" for c in CASES])
def test_random_shape(case):
    i, dtype, d, chunk, H, lengths, s0 = case
    print(f"[random] case {i}: dtype={dtype} d={d} C={chunk} H={H} lengths={lengths} s0={s0}",
          flush=True)
    kda = _kda()
    w = kin.make_prefill(5000 + i, H=H, d=d, dtype=dtype, chunk_size=chunk, lengths=lengths,
                         s0_std=0.05 if s0 else None)
    tol = TOL[dtype]
    dd = upload_prefill(w)
    o, s = kda.fwd_chunked(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"],
                           cu_seqlens=dd["cu_seqlens"], initial_state=dd["initial_state"],
                           chunk_size=chunk)
    torch.cuda.synchronize()
    q, k, v, g, b, st0 = w.f64()
    cu = w.cu_seqlens.astype(np.int64)
    o_ref, s_ref = oracle.recurrent(q, k, v, g, b, cu_seqlens=cu, initial_state=st0)
    eo, es = relerr(from_device(o), o_ref), relerr(from_device(s), s_ref)
    print(f"  forward relerr o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= tol and es <= tol
    if i % 3:
        return
    do, dsf = kin.backward_inputs(6000 + i, w.total_tokens, H, d, w.num_seqs, dtype)
    gr = kda.bwd_chunked(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"],
                         to_device(do, dtype), cu_seqlens=dd["cu_seqlens"],
                         num_seqs=dd["num_seqs"], initial_state=dd["initial_state"],
                         d_final_state=f32_device(dsf), chunk_size=chunk)
    torch.cuda.synchronize()
    ref = oracle.recurrent_backward(q, k, v, g, b, kin.as_f64(do, dtype), dsf, cu_seqlens=cu,
                                    num_seqs=w.num_seqs, initial_state=st0)
    errs = {key: relerr(from_device(gr[key]), ref[key])
            for key in ("dq", "dk", "dv", "dg", "dbeta", "ds0")}
    print("  backward relerr " + " ".join(f"{kk}={e:.2e}" for kk, e in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= tol, f"{key} error {e:.3e} > {tol}"
