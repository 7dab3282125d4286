"""Diagnostics of the prefill (kda_options.flags, check_inputs).

mkdocs.reaper.mx "Attention lineaire et recurrence", section "Le piege
numerique de la decroissance cumulee": the chunk form divides by the
cumulative decay, which must stay in range inside a chunk (summed log-decay
above -80 per channel here).  The intra-chunk kernel reports a breach in
the caller's flag word.  With check_inputs, cu_seqlens is validated on the
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


def test_decay_range_flag_set_only_past_the_bound():
    """g = -1.5 on every channel of head 0: a 64-token chunk sums to -96, past
    the bound, and the flag is set; with chunk 16 (-24) or the usual decays
    it stays clear, and asking for flags changes no output bit."""
    print("[diagnostics] decay-range flag", flush=True)
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
    for chunk, expect in ((64, kda.FLAG_DECAY_RANGE), (16, 0)):
        f = _flags()
        kda.fwd_chunked(dd["q"], dd["k"], dd["v"], g, dd["beta"], chunk_size=chunk, flags=f)
        torch.cuda.synchronize()
        assert int(f.item()) == expect, (chunk, int(f.item()))


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
