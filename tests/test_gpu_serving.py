"""Serving paths: state slots (a cache pool of fixed-size states indexed per
request, continuous batching) for decode and prefill, and multi-token
verification with kda_fwd_chunked from a cached state.

docsaid.org "Kimi Linear", section "Calculer le cache a la main": the state
per request has a fixed size whatever the context length, so a server keeps
one pool of states and maps requests to slots.  fr.news.hada.io, section
"Algorithme parallele par chunks": the state at the end of a span is the
initial state of the next, so a span of draft tokens can be verified with one
prefill from the cached state.
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


@pytest.mark.parametrize("dtype,d", [(kin.BF16, 128), (kin.F32, 64)])
def test_decode_state_slots(dtype, d):
    """Decode over a pool of 7 states: requests map to slots 3, 0, 6 and two
    padding entries (-1 and 9, outside the pool).  Mapped slots advance as
    the oracle says, padding outputs are 0, other slots are untouched."""
    print(f"[serving] decode slots dtype={dtype} d={d}", flush=True)
    kda = _kda()
    B, H, NS = 5, 2, 7
    slots = np.array([3, -1, 0, 6, 9], dtype=np.int32)
    pool0 = kin.decode_states(NS, H, d, seed=90 + d)
    pool = f32_device(pool0)
    ref = pool0.astype(np.float64)
    sl = torch.from_numpy(slots).cuda()
    for step in range(3):
        x = kin.decode_step(step, B, H, d, dtype=dtype, seed_base=90 + d)
        o = kda.decode_step(to_device(x.q, dtype), to_device(x.k, dtype), to_device(x.v, dtype),
                            f32_device(x.g), f32_device(x.beta), pool, state_slots=sl)
        q, k, v, g, b = x.f64()
        live = [i for i, s in enumerate(slots) if 0 <= s < NS]
        o_ref, st = oracle.decode(q[live], k[live], v[live], g[live], b[live],
                                  ref[slots[live]])
        ref[slots[live]] = st
        oh = from_device(o)
        assert relerr(oh[live], o_ref) <= TOL[dtype]
        assert np.all(oh[[1, 4]] == 0.0)
    got = from_device(pool)
    untouched = [s for s in range(NS) if s not in slots]
    assert np.array_equal(got[untouched], pool0[untouched].astype(np.float64))
    assert relerr(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("d,chunk,lengths", [
    (64, 32, [70, 33, 50, 1]),
    # the split-role chain (bf16, d = 128, C = 64), without and with L2 warm-up loads
    (128, 64, [700, 330, 500, 10]),
    (128, 64, [9000, 8700, 8400, 8300]),
], ids=["d64_c32", "d128_c64", "d128_c64_long"])
def test_prefill_state_slots_in_place(d, chunk, lengths):
    """Four packed sequences whose states live in slots 5, 0, (padding -1)
    and 2 of a pool of 6, updated in place.  The padding sequence starts from
    zero and writes no state; slots 1, 3, 4 are untouched."""
    print(f"[serving] prefill slots d={d} chunk={chunk} lengths={lengths}", flush=True)
    kda = _kda()
    H, NS = 2, 6
    w = kin.make_prefill(31, H=H, d=d, dtype=kin.BF16, chunk_size=chunk, lengths=lengths)
    pool0 = kin.decode_states(NS, H, d, seed=31)
    slots = np.array([5, 0, -1, 2], dtype=np.int32)
    dd = upload_prefill(w)
    pool = f32_device(pool0)
    o, _ = kda.fwd_chunked(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"],
                           cu_seqlens=dd["cu_seqlens"], initial_state=pool, chunk_size=chunk,
                           state_slots=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    q, k, v, g, b, _ = w.f64()
    s0 = np.zeros((4, H, d, d))
    for i, s in enumerate(slots):
        if s >= 0:
            s0[i] = pool0[s]
    o_ref, s_ref = oracle.recurrent(q, k, v, g, b, cu_seqlens=w.cu_seqlens.astype(np.int64),
                                    initial_state=s0)
    got = from_device(pool)
    assert relerr(from_device(o), o_ref) <= 2e-2
    for i, s in enumerate(slots):
        if s >= 0:
            assert relerr(got[s], s_ref[i]) <= 2e-2
    for s in (1, 3, 4):
        assert np.array_equal(got[s], pool0[s].astype(np.float64))


def test_multi_token_verification():
    """Verify 6 draft tokens of 3 requests from their cached states in one
    prefill (final states into a scratch pool, cache untouched), then accept
    the first 4: a second prefill of those 4 tokens from the same cache gives
    the outputs of the first 4 positions and the state after them."""
    print("[serving] multi-token verification", flush=True)
    kda = _kda()
    H, d, NS, K, J = 4, 128, 8, 6, 4
    slots = np.array([7, 2, 4], dtype=np.int32)
    w = kin.make_prefill(41, H=H, d=d, dtype=kin.BF16, chunk_size=16, lengths=[K] * 3)
    pool0 = kin.decode_states(NS, H, d, seed=41)
    dd = upload_prefill(w)
    cache = f32_device(pool0)
    scratch = torch.zeros_like(cache)
    sl = torch.from_numpy(slots).cuda()
    o_all, _ = kda.fwd_chunked(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"],
                               cu_seqlens=dd["cu_seqlens"], initial_state=cache,
                               final_state=scratch, chunk_size=16, state_slots=sl)
    torch.cuda.synchronize()
    assert np.array_equal(from_device(cache), pool0.astype(np.float64))
    keep = np.concatenate([np.arange(i * K, i * K + J) for i in range(3)])
    kt = torch.from_numpy(keep).cuda()
    cu = torch.tensor([0, J, 2 * J, 3 * J], dtype=torch.int32, device="cuda")
    o_acc, _ = kda.fwd_chunked(dd["q"][kt].contiguous(), dd["k"][kt].contiguous(),
                               dd["v"][kt].contiguous(), dd["log_alpha"][kt].contiguous(),
                               dd["beta"][kt].contiguous(), cu_seqlens=cu, initial_state=cache,
                               chunk_size=16, state_slots=sl)
    torch.cuda.synchronize()
    q, k, v, g, b, _ = w.f64()
    o_ref, s_ref = oracle.recurrent(q[keep], k[keep], v[keep], g[keep], b[keep],
                                    cu_seqlens=np.array([0, J, 2 * J, 3 * J]),
                                    initial_state=pool0[slots].astype(np.float64))
    assert relerr(from_device(o_acc), o_ref) <= 2e-2
    assert relerr(from_device(o_all)[keep], o_ref) <= 2e-2
    got = from_device(cache)
    assert relerr(got[slots], s_ref) <= 2e-2
