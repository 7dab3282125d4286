"""Parity past 32-bit element offsets: calls whose tensors hold more than
2^31 elements.

The operator treats every (sequence, head) independently, so a large call
can be built from a few distinct seeded sequences repeated many times: every
repeat must reproduce the oracle's result for its source sequence.  The
oracle runs once on the distinct sequences; the device output is compared
with it repeat by repeat, on the device, so every output row and final
state of the large call is checked.  Tolerance as in the other parity
tests: normwise max relative error <= 2e-2 (bf16 operands).
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from gated_delta_rule_chunked_amd import inputs as kin  # noqa: E402
from kda_testutil import TOL, f32_device, to_device  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

H, D = 32, 128
ELEMS_31 = 1 << 31


def _repeat_prefill(w, reps):
    """The base workload's device tensors, each sequence list repeated `reps` times."""
    q = to_device(w.q, w.dtype).repeat(reps, 1, 1)
    k = to_device(w.k, w.dtype).repeat(reps, 1, 1)
    v = to_device(w.v, w.dtype).repeat(reps, 1, 1)
    g = f32_device(w.g).repeat(reps, 1, 1)
    beta = f32_device(w.beta).repeat(reps, 1)
    s0 = f32_device(w.initial_state).repeat(reps, 1, 1, 1)
    cu = None
    if w.cu_seqlens is not None:
        base = w.cu_seqlens.astype(np.int64)
        total = int(base[-1])
        cu = np.concatenate([[0]] + [base[1:] + r * total for r in range(reps)])
        cu = torch.from_numpy(cu.astype(np.int32)).cuda()
    return q, k, v, g, beta, s0, cu


def _compare_repeats(o, s, o_ref, s_ref, reps, tol):
    """Normwise relative error of the whole repeated output and final state."""
    o_ref_d = torch.from_numpy(o_ref).cuda()
    s_ref_d = torch.from_numpy(s_ref).cuda()
    t_base, n_base = o_ref.shape[0], s_ref.shape[0]
    num_o = num_s = 0.0
    for r in range(reps):
        num_o = max(num_o, (o[r * t_base:(r + 1) * t_base].double() - o_ref_d).abs().max().item())
        num_s = max(num_s, (s[r * n_base:(r + 1) * n_base].double() - s_ref_d).abs().max().item())
    eo = num_o / float(np.max(np.abs(o_ref)))
    es = num_s / float(np.max(np.abs(s_ref)))
    print(f"  {reps} repeats: relerr o={eo:.3e} S={es:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol, f"output error {eo:.3e} > {tol}"
    assert es <= tol, f"final-state error {es:.3e} > {tol}"


@pytest.mark.parametrize("packed", [False, True], ids=["equal_lengths", "cu_seqlens"])
def test_prefill_past_32bit_element_offsets(packed):
    """8 distinct seeded sequences repeated until q, k, v and o hold more
    than 2^31 elements (g more than 8 GiB), H=32, d=128, C=64, bf16, with
    initial states.  Equal lengths of 2048 tokens (264 sequences), or ragged
    seeded lengths through cu_seqlens and the chunk table (296 sequences)."""
    import gated_delta_rule_chunked_amd as kda
    if packed:
        w = kin.make_prefill(801, H=H, d=D, dtype=kin.BF16, chunk_size=64, B=8,
                             len_range=(1500, 2600), s0_std=0.02)
    else:
        w = kin.make_prefill(802, H=H, d=D, dtype=kin.BF16, chunk_size=64, B=8, T=2048,
                             s0_std=0.02)
    t_base = w.total_tokens
    reps = -(-(ELEMS_31 + 1) // (t_base * H * D))  # smallest count past 2^31 elements
    assert reps * t_base * H * D > ELEMS_31
    q, k, v, g, beta, s0, cu = _repeat_prefill(w, reps)
    n = w.num_seqs * reps
    print(f"  {n} sequences, {reps * t_base} tokens, {reps * t_base * H * D} elements per "
          f"operand", flush=True)
    o, s = kda.fwd_chunked(q, k, v, g, beta, cu_seqlens=cu, num_seqs=n, initial_state=s0,
                           chunk_size=64)
    torch.cuda.synchronize()
    del q, k, v, g, beta, s0
    qo, ko, vo, go, bo, s0o = w.f64()
    cu_o = None if w.cu_seqlens is None else w.cu_seqlens.astype(np.int64)
    o_ref, s_ref = oracle.recurrent(qo, ko, vo, go, bo, cu_seqlens=cu_o, num_seqs=w.num_seqs,
                                    initial_state=s0o)
    _compare_repeats(o, s, o_ref, s_ref, reps, TOL[kin.BF16])
    del o, s
    torch.cuda.empty_cache()


def test_decode_past_32bit_element_offsets():
    """One decode step over 4,098 x 32 states (2 distinct sequences repeated
    2,049 times): the state pool holds more than 2^31 fp32 elements."""
    import gated_delta_rule_chunked_amd as kda
    base_b = 2
    st0 = kin.decode_states(base_b, H, D, seed=803)
    x = kin.decode_step(0, base_b, H, D, dtype=kin.BF16, seed_base=803)
    reps = -(-(ELEMS_31 + 1) // (base_b * H * D * D))
    assert reps * base_b * H * D * D > ELEMS_31
    state = f32_device(st0).repeat(reps, 1, 1, 1)
    q = to_device(x.q, kin.BF16).repeat(reps, 1, 1)
    k = to_device(x.k, kin.BF16).repeat(reps, 1, 1)
    v = to_device(x.v, kin.BF16).repeat(reps, 1, 1)
    g = f32_device(x.g).repeat(reps, 1, 1)
    beta = f32_device(x.beta).repeat(reps, 1)
    print(f"  {base_b * reps} x {H} states, {state.numel()} state elements", flush=True)
    o = kda.decode_step(q, k, v, g, beta, state)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.decode(*x.f64(), st0.astype(np.float64))
    _compare_repeats(o, state, o_ref, s_ref, reps, TOL[kin.BF16])
    del o, state, q, k, v, g, beta
    torch.cuda.empty_cache()
