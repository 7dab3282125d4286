"""Diagnostics of the prefill (kda_options.flags, check_inputs).

mkdocs.reaper.mx "Attention lineaire et recurrence", section "Le piege
numerique de la decroissance cumulee": the chunk form divides by the
cumulative decay, which must stay in range (summed log-decay >= -80 per
channel) over the span it is referenced to.  Chunks that decay further are
referenced per 16-token block; a block past the bound is reported in the
caller's flag word.  With check_inputs, cu_seqlens is validated on the
device first and a bad one stops every prefill kernel of the call.  The
malformed offsets used below stay inside the token range, so even a kernel
that ignored the check would not read past the tensors.
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


def _kda():
    import gated_delta_rule_chunked_amd as kda
    return kda


def _flags():
    return torch.zeros(1, dtype=torch.int32, device="cuda")


def test_decay_past_the_chunk_bound_is_exact_and_unflagged():
    """g = -1.5 on every channel of head 0: a 64-token chunk sums to -96, past
    the bound of the chunk-start reference, so those tiles reference each
    16-token block separately (blocks sum to -24).  Outputs stay finite and
    match the oracle, the flag stays clear, and asking for flags changes no
    output bit of the usual decays."""
    print("[diagnostics] decay past the chunk bound", flush=True)
    kda = _kda()
    w = kin.make_prefill(901, B=1, T=192, H=2, d=64, dtype=kin.BF16, chunk_size=64)
    dd = upload_prefill(w)
    o_ref, s_ref = kda.fwd_chunked(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"],
                                   chunk_size=64)
    f = _flags()
    o, s = kda.fwd_chunked(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"],
                           chunk_size=64, flags=f)
    torch.cuda.synchronize()
    assert int(f.item()) == 0
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
    g = dd["log_alpha"].clone()
    g[:, 0, :] = -1.5
    q, k, v, _, b, _ = w.f64()
    ro, rs = oracle.recurrent(q, k, v, from_device(g), b)
    for chunk in (64, 32, 16):
        f = _flags()
        o, s = kda.fwd_chunked(dd["q"], dd["k"], dd["v"], g, dd["beta"], chunk_size=chunk, flags=f)
        torch.cuda.synchronize()
        assert int(f.item()) == 0, (chunk, int(f.item()))
        eo, es = relerr(from_device(o), ro), relerr(from_device(s), rs)
        print(f"  C={chunk}: relerr o={eo:.3e} S={es:.3e}", flush=True)
        assert np.isfinite(from_device(o)).all() and np.isfinite(from_device(s)).all()
        assert eo <= TOL[w.dtype] and es <= TOL[w.dtype], (chunk, eo, es)


def test_decay_range_flag_set_past_the_block_bound():
    """g = -6 on head 0: a single 16-token block sums to -96, past the bound
    that remains (the tile bound the page states), and the flag is raised at
    every chunk size; with g = -5 (blocks at exactly -80) it stays clear."""
    print("[diagnostics] decay past the 16-token block bound", flush=True)
    kda = _kda()
    w = kin.make_prefill(905, B=1, T=128, H=2, d=32, dtype=kin.BF16, chunk_size=64)
    dd = upload_prefill(w)
    for gval, expect in ((-6.0, kda.FLAG_DECAY_RANGE), (-5.0, 0)):
        g = dd["log_alpha"].clone()
        g[:, 0, :] = gval
        for chunk in (16, 32, 64):
            f = _flags()
            kda.fwd_chunked(dd["q"], dd["k"], dd["v"], g, dd["beta"], chunk_size=chunk, flags=f)
            torch.cuda.synchronize()
            assert int(f.item()) == expect, (gval, chunk, int(f.item()))


@pytest.mark.parametrize("dtype,d", [(kin.BF16, 128), (kin.BF16, 64), (kin.BF16, 32),
                                     (kin.F32, 128), (kin.F32, 32)])
@pytest.mark.parametrize("chunk", [32, 64])
def test_strong_decay_parity(dtype, d, chunk):
    """Head 0 decays by -exp(N(0.5, 0.3)) per token and channel (about -1.7,
    chunk sums far below -80), head 1 by the usual -exp(N(-2, 0.5)): ragged
    packed sequences with initial states, every output and final state
    against the oracle.  Tiles of head 0 take the block-referenced form."""
    print(f"[parity] strong decay dtype={dtype} d={d} C={chunk}", flush=True)
    kda = _kda()
    w = kin.make_prefill(910 + d + chunk, H=2, d=d, dtype=dtype, chunk_size=chunk,
                         lengths=[150, 1, 70, 64], s0_std=0.05)
    rng = np.random.default_rng(911 + d)
    w.g[:, 0, :] = (-np.exp(rng.normal(0.5, 0.3, size=w.g[:, 0, :].shape))).astype(np.float32)
    dd = upload_prefill(w)
    f = _flags()
    o, s = kda.fwd_chunked(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"],
                           cu_seqlens=dd["cu_seqlens"], initial_state=dd["initial_state"],
                           chunk_size=chunk, flags=f)
    torch.cuda.synchronize()
    q, k, v, g, b, s0 = w.f64()
    ro, rs = oracle.recurrent(q, k, v, g, b, cu_seqlens=w.cu_seqlens.astype(np.int64),
                              initial_state=s0)
    eo, es = relerr(from_device(o), ro), relerr(from_device(s), rs)
    print(f"  relerr o={eo:.3e} S={es:.3e} flags={int(f.item())}", flush=True)
    assert int(f.item()) == 0
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_check_inputs_accepts_valid_offsets_bit_for_bit():
    """Packed sequences (tails, an empty one) with check_inputs: the flag stays
    clear and the outputs are those of the unchecked call, which match the
    oracle."""
    print("[diagnostics] check_inputs, valid cu_seqlens", flush=True)
    kda = _kda()
    w = kin.make_prefill(902, H=2, d=64, dtype=kin.BF16, chunk_size=32,
                         lengths=[70, 0, 33, 128], s0_std=0.02)
    dd = upload_prefill(w)
    args = (dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"])
    kw = dict(cu_seqlens=dd["cu_seqlens"], initial_state=dd["initial_state"], chunk_size=32)
    o_ref, s_ref = kda.fwd_chunked(*args, **kw)
    f = _flags()
    o, s = kda.fwd_chunked(*args, **kw, flags=f, check_inputs=True)
    torch.cuda.synchronize()
    assert int(f.item()) == 0
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
    q, k, v, g, b, s0 = w.f64()
    ro, rs = oracle.recurrent(q, k, v, g, b, cu_seqlens=w.cu_seqlens.astype(np.int64),
                              num_seqs=w.num_seqs, initial_state=s0)
    assert relerr(from_device(o), ro) <= TOL[w.dtype]
    assert relerr(from_device(s), rs) <= TOL[w.dtype]


@pytest.mark.parametrize("cu", [[0, 100, 50, 200], [0, 100, 150], [10, 100, 200]])
def test_check_inputs_rejects_bad_offsets_and_computes_nothing(cu):
    """A decreasing offset, a last offset short of total_tokens and a first
    offset other than 0 each set KDA_FLAG_BAD_CU_SEQLENS; o, the final states
    (and the output epilogue) are left as they were."""
    print(f"[diagnostics] check_inputs, cu_seqlens={cu}", flush=True)
    kda = _kda()
    T, H, d, n = 200, 2, 64, len(cu) - 1
    w = kin.make_prefill(903, B=1, T=T, H=H, d=d, dtype=kin.BF16, chunk_size=64)
    dd = upload_prefill(w)
    cu_t = torch.tensor(cu, dtype=torch.int32, device="cuda")
    o = torch.full((T, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    fs = torch.full((n, H, d, d), 3.0, dtype=torch.float32, device="cuda")
    wn = torch.ones(d, dtype=torch.float32, device="cuda")
    f = _flags()
    kda.fwd_chunked(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"], cu_seqlens=cu_t,
                    chunk_size=64, out=o, final_state=fs, out_norm_weight=wn, flags=f,
                    check_inputs=True)
    torch.cuda.synchronize()
    assert int(f.item()) & kda.FLAG_BAD_CU_SEQLENS
    assert bool(torch.all(o == 7.0)) and bool(torch.all(fs == 3.0))


def test_bounded_gate_at_its_limit_keeps_the_flag_clear():
    """K3's bounded gate g = g_min sigmoid(z) with g_min = -5 and z = 30:
    sigmoid rounds to 1 in fp32, so every token decays by exactly -5 and a
    16-token chunk sums to exactly -80, the bound itself (e^80 is finite in
    fp32 and bf16).  The flag stays clear and the outputs match the oracle."""
    print("[diagnostics] sigmoid gate at g_min = -5, z = 30, C = 16", flush=True)
    kda = _kda()
    T, H, d = 96, 2, 64
    w = kin.make_prefill(904, B=1, T=T, H=H, d=d, dtype=kin.BF16, chunk_size=16)
    dd = upload_prefill(w)
    z = torch.full((T, H, d), 30.0, dtype=torch.bfloat16, device="cuda")
    f = _flags()
    o, s = kda.fwd_chunked(dd["q"], dd["k"], dd["v"], z, dd["beta"], chunk_size=16,
                           gate="sigmoid", gate_min=-5.0, flags=f)
    torch.cuda.synchronize()
    assert int(f.item()) == 0, int(f.item())
    q, k, v, _, b, _ = w.f64()
    q, k, g, b = oracle.prepare_inputs(q, k, np.full((T, H, d), 30.0), b, gate="sigmoid",
                                       gate_min=-5.0)
    ro, rs = oracle.recurrent(q, k, v, g, b)
    eo, es = relerr(from_device(o), ro), relerr(from_device(s), rs)
    print(f"  relerr o={eo:.3e} S={es:.3e}", flush=True)
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype]
