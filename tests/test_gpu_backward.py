"""Backward (kda_bwd_chunked) against the fp64 autograd oracle
(oracle.recurrent_backward), every gradient normwise at the operator's
tolerances.

fr.news.hada.io Kimi Linear summary, section "Algorithme parallele par
chunks" (the chunk form is what training runs).
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


def _kda():
    import gated_delta_rule_chunked_amd as kda
    return kda


def _run(w, do, dsf, chunk):
    kda = _kda()
    dd = upload_prefill(w)
    gr = kda.bwd_chunked(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"],
                         to_device(do, w.dtype), cu_seqlens=dd["cu_seqlens"],
                         num_seqs=dd["num_seqs"], initial_state=dd["initial_state"],
                         d_final_state=None if dsf is None else f32_device(dsf),
                         chunk_size=chunk)
    torch.cuda.synchronize()
    return {k: from_device(v) for k, v in gr.items()}


def _check(w, do, dsf, got):
    q, k, v, g, b, s0 = w.f64()
    cu = None if w.cu_seqlens is None else w.cu_seqlens.astype(np.int64)
    ref = oracle.recurrent_backward(q, k, v, g, b, kin.as_f64(do, w.dtype), dsf,
                                    cu_seqlens=cu, num_seqs=w.num_seqs, initial_state=s0)
    tol = TOL[w.dtype]
    errs = {key: relerr(got[key], ref[key]) for key in ("dq", "dk", "dv", "dg", "dbeta", "ds0")}
    print("  relerr " + " ".join(f"{k}={e:.2e}" for k, e in errs.items()), flush=True)
    for key, e in errs.items():
        assert e <= tol, f"{key} error {e:.3e} > {tol}"


@pytest.mark.parametrize("dtype,d,chunk", [(kin.BF16, 128, 64), (kin.BF16, 64, 32),
                                           (kin.BF16, 32, 16), (kin.F32, 32, 16),
                                           (kin.F32, 64, 64)])
def test_backward_ragged(dtype, d, chunk):
    """Packed sequences with tails, an empty and a one-token sequence,
    initial states and a final-state gradient."""
    print(f"[backward] dtype={dtype} d={d} C={chunk}", flush=True)
    w = kin.make_prefill(500 + d + chunk, H=2, d=d, dtype=dtype, chunk_size=chunk,
                         lengths=[70, 0, 1, 33], s0_std=0.05)
    do, dsf = kin.backward_inputs(501 + d, w.total_tokens, 2, d, w.num_seqs, dtype)
    _check(w, do, dsf, _run(w, do, dsf, chunk))


_EVERY_SHAPE = [(dt, d, c) for dt in (kin.BF16, kin.F32) for d in (32, 64, 128)
                for c in (16, 32, 64)]


@pytest.mark.parametrize("dtype,d,chunk", _EVERY_SHAPE)
def test_backward_every_shape(dtype, d, chunk):
    """Every supported (dtype, head size, chunk size): one full chunk plus a
    tail, a one-token sequence and two chunks plus a tail, one head, with
    initial states and a final-state gradient.  Each shape instantiates its
    own product tilings (whole tile columns per wave or not, 16-row tiles)."""
    print(f"[backward] every shape dtype={dtype} d={d} C={chunk}", flush=True)
    w = kin.make_prefill(700 + d + chunk, H=1, d=d, dtype=dtype, chunk_size=chunk,
                         lengths=[chunk + 5, 1, 2 * chunk + 3], s0_std=0.05)
    do, dsf = kin.backward_inputs(701 + d + chunk, w.total_tokens, 1, d, w.num_seqs, dtype)
    _check(w, do, dsf, _run(w, do, dsf, chunk))


@pytest.mark.parametrize("dtype,d,chunk,H", [(kin.BF16, 64, 32, 4), (kin.BF16, 128, 64, 2),
                                             (kin.F32, 64, 16, 4)])
def test_backward_many_pairs_two_launches(dtype, d, chunk, H):
    """Nine sequences: 36 (sequence, head) pairs at d=64 (chain grids of 160
    workgroups) or 18 at d=128 (192 workgroups), so the two chains no longer
    fit a 256-CU GPU together and run as two launches (the other cases run
    both chains in one launch)."""
    print(f"[backward] 9 seqs x {H} heads dtype={dtype} d={d} C={chunk}", flush=True)
    w = kin.make_prefill(909 + d, H=H, d=d, dtype=dtype, chunk_size=chunk,
                         lengths=[40, 0, 7, 65, 1, 33, 64, 16, 90], s0_std=0.05)
    do, dsf = kin.backward_inputs(910 + d, w.total_tokens, H, d, w.num_seqs, dtype)
    _check(w, do, dsf, _run(w, do, dsf, chunk))


def test_backward_equal_lengths_no_final_gradient():
    """B=2 sequences of 256 tokens, H=2, d=128, C=64, zero initial state and no
    final-state gradient (the default loss sum(o * d_o))."""
    print("[backward] B=2 T=256 d=128", flush=True)
    w = kin.make_prefill(77, B=2, T=256, H=2, d=128, dtype=kin.BF16, chunk_size=64)
    do, _ = kin.backward_inputs(78, w.total_tokens, 2, 128, 2, kin.BF16)
    _check(w, do, None, _run(w, do, None, 64))


def test_backward_headline_size_sampled_pairs():
    """The headline prefill (B=2, H=8, T=2048, d=128, C=64, bf16) with a
    final-state gradient, in the launch configuration the benchmark times;
    (sequence, head) pairs are independent, so two sampled pairs are checked
    against the fp64 oracle on their own tokens."""
    print("[backward] headline B=2 H=8 T=2048 d=128, sampled pairs", flush=True)
    w = kin.workload(1)
    H, d, T = w.num_heads, 128, w.total_tokens // w.num_seqs
    do, dsf = kin.backward_inputs(7, w.total_tokens, H, d, w.num_seqs, w.dtype)
    got = _run(w, do, dsf, w.chunk_size)
    q, k, v, g, b, s0 = w.f64()
    do64 = kin.as_f64(do, w.dtype)
    for seq, h in ((0, 3), (1, 6)):
        rows = slice(seq * T, (seq + 1) * T)
        pick = lambda a: a[rows, h:h + 1]
        ref = oracle.recurrent_backward(
            pick(q), pick(k), pick(v), pick(g), pick(b), pick(do64),
            dsf[seq:seq + 1, h:h + 1].astype(np.float64),
            initial_state=None if s0 is None else s0[seq:seq + 1, h:h + 1])
        mine = {key: pick(got[key]) for key in ("dq", "dk", "dv", "dg", "dbeta")}
        mine["ds0"] = got["ds0"][seq:seq + 1, h:h + 1]
        errs = {key: relerr(mine[key], ref[key]) for key in mine}
        print(f"  pair ({seq}, {h}) relerr " + " ".join(f"{kk}={e:.2e}" for kk, e in errs.items()),
              flush=True)
        for key, e in errs.items():
            assert e <= TOL[w.dtype], f"pair ({seq}, {h}) {key} error {e:.3e}"


@pytest.mark.parametrize("case", ["headline", "ragged"])
def test_backward_deterministic(case):
    """No atomics on any accumulation: two runs on the same inputs give the
    same bits for every gradient, at the headline size (B=2, H=8, T=2048,
    d=128, C=64, with a final-state gradient) and on ragged packed sequences
    with initial states (d=64, C=32)."""
    print(f"[backward] bitwise run-to-run, {case}", flush=True)
    if case == "headline":
        w = kin.workload(1)
        d, chunk = 128, 64
    else:
        w = kin.make_prefill(611, H=3, d=64, dtype=kin.BF16, chunk_size=32,
                             lengths=[95, 0, 1, 130, 33], s0_std=0.05)
        d, chunk = 64, 32
    do, dsf = kin.backward_inputs(612, w.total_tokens, w.num_heads, d, w.num_seqs, w.dtype)
    a = _run(w, do, dsf, chunk)
    b = _run(w, do, dsf, chunk)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "ds0"):
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
