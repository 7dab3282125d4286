"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerance: normwise max relative error max|x - ref| / max|ref| per output
tensor, <= 1e-4 for fp32 operands and <= 2e-2 for bf16 operands (fp32
accumulation and state).  Inputs come from the seeded generators; the oracle
sees exactly the bits the device sees.
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from gated_delta_rule_chunked_amd import inputs as kin  # noqa: E402
from kda_testutil import TOL, from_device, relerr, upload_prefill, to_device, f32_device  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _kda():
    import gated_delta_rule_chunked_amd as kda
    return kda


def _run_gpu(w, chunk=None, in_place=False):
    kda = _kda()
    d = upload_prefill(w)
    chunk = chunk or w.chunk_size
    s0 = d["initial_state"]
    kw = {}
    if in_place and s0 is not None:
        kw["final_state"] = s0
    o, s = kda.fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                           cu_seqlens=d["cu_seqlens"], num_seqs=d["num_seqs"],
                           initial_state=s0, chunk_size=chunk, **kw)
    torch.cuda.synchronize()
    return from_device(o), from_device(s)


def _oracle(w, heads=None):
    q, k, v, g, b, s0 = w.f64()
    if heads is not None:
        q, k, v, g, b = q[:, heads], k[:, heads], v[:, heads], g[:, heads], b[:, heads]
        s0 = None if s0 is None else s0[:, heads]
    cu = None if w.cu_seqlens is None else w.cu_seqlens.astype(np.int64)
    return oracle.recurrent(q, k, v, g, b, cu_seqlens=cu, num_seqs=w.num_seqs,
                            initial_state=s0)


def _check(w, o, s, heads=None, tol=None):
    tol = tol if tol is not None else TOL[w.dtype]
    o_ref, s_ref = _oracle(w, heads)
    if heads is not None:
        o, s = o[:, heads], s[:, heads]
    eo, es = relerr(o, o_ref), relerr(s, s_ref)
    print(f"  relerr o={eo:.3e} S={es:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol, f"output error {eo:.3e} > {tol}"
    assert es <= tol, f"final-state error {es:.3e} > {tol}"
    return eo, es


@pytest.mark.parametrize("wid", [0, 1])
def test_workload_full_parity(wid):
    """Tiny fp32 (d=32, C=16) and the B=2, H=8, T=2048 bf16 prefill, every
    output and final state against the oracle."""
    print(f"[parity] workload {wid}", flush=True)
    w = kin.workload(wid)
    o, s = _run_gpu(w)
    _check(w, o, s)


def test_long_context_full():
    """B=1, H=32, T=32768 (512 chunks per chain), in the launch configuration
    the benchmark times: every head's outputs and final state."""
    print("[parity] workload 2 (long), all 32 heads", flush=True)
    w = kin.workload(2)
    o, s = _run_gpu(w)
    _check(w, o, s)


def test_varlen_full():
    """16 packed sequences of U[512, 8192] tokens, H=16, initial states:
    every head's outputs and every sequence's final state."""
    print("[parity] workload 3 (varlen), all 16 heads", flush=True)
    w = kin.workload(3)
    o, s = _run_gpu(w)
    _check(w, o, s)


@pytest.mark.parametrize("dtype,d", [(kin.BF16, 128), (kin.BF16, 64), (kin.BF16, 32),
                                     (kin.F32, 32), (kin.F32, 64), (kin.F32, 128)])
@pytest.mark.parametrize("chunk", [16, 32, 64])
def test_ragged_varlen_shapes(dtype, d, chunk):
    """Several tiles, ragged tails, an empty sequence and a one-token sequence,
    initial states, every head size and chunk size."""
    print(f"[parity] ragged dtype={dtype} d={d} C={chunk}", flush=True)
    w = kin.make_prefill(100 + d + chunk, H=3, d=d, dtype=dtype, chunk_size=chunk,
                         lengths=[130, 0, 1, 64, 77], s0_std=0.05)
    o, s = _run_gpu(w)
    _check(w, o, s)
    np.testing.assert_array_equal(s[1], w.initial_state[1])


def test_chunk_size_invariance():
    """The chunk form is exact: C = 16, 32 and 64 all match the oracle and
    each other within the bf16 tolerance."""
    print("[parity] chunk-size invariance", flush=True)
    w = kin.make_prefill(7, B=2, T=500, H=4, d=128, dtype=kin.BF16, chunk_size=64)
    outs = {}
    for c in (16, 32, 64):
        o, s = _run_gpu(w, chunk=c)
        _check(w, o, s)
        outs[c] = (o, s)
    e = (relerr(outs[16][0], outs[64][0]), relerr(outs[16][1], outs[64][1]))
    print("  C=16 vs C=64 o, S:", ["%.2e" % x for x in e])
    assert max(e) < 2e-2


def test_in_place_state_and_split_call():
    """final_state may alias initial_state; a prefill split in two calls with
    the state carried equals one call."""
    print("[parity] in-place + split call", flush=True)
    kda = _kda()
    w = kin.make_prefill(11, B=1, T=300, H=2, d=128, dtype=kin.BF16, chunk_size=64,
                         s0_std=0.05)
    d = upload_prefill(w)
    o_full, s_full = kda.fwd_chunked(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"],
                                     initial_state=d["initial_state"])
    st = d["initial_state"].clone()
    cut = 137
    o1, _ = kda.fwd_chunked(d["q"][:cut].contiguous(), d["k"][:cut].contiguous(),
                            d["v"][:cut].contiguous(), d["log_alpha"][:cut].contiguous(),
                            d["beta"][:cut].contiguous(), initial_state=st, final_state=st)
    o2, _ = kda.fwd_chunked(d["q"][cut:].contiguous(), d["k"][cut:].contiguous(),
                            d["v"][cut:].contiguous(), d["log_alpha"][cut:].contiguous(),
                            d["beta"][cut:].contiguous(), initial_state=st, final_state=st)
    torch.cuda.synchronize()
    o_split = np.concatenate([from_device(o1), from_device(o2)])
    o_ref, s_ref = _oracle(w)
    e = (relerr(o_split, o_ref), relerr(from_device(st), s_ref),
         relerr(o_split, from_device(o_full)))
    print("  split o, split S, split-vs-single o:", ["%.2e" % x for x in e])
    assert max(e) < 2e-2


def test_deterministic():
    """No atomics: two runs give identical bits."""
    w = kin.workload(1)
    o1, s1 = _run_gpu(w)
    o2, s2 = _run_gpu(w)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_zero_tokens():
    """total_tokens = 0: no output rows, final state = initial state."""
    kda = _kda()
    H, d = 2, 128
    e = torch.empty((0, H, d), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((0, H, d), dtype=torch.float32, device="cuda")
    b = torch.empty((0, H), dtype=torch.float32, device="cuda")
    s0 = torch.randn((3, H, d, d), device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    o, s = kda.fwd_chunked(e, e, e, g, b, cu_seqlens=cu, initial_state=s0)
    torch.cuda.synchronize()
    assert o.shape == (0, H, d)
    assert torch.equal(s, s0)


# ---------------------------------------------------------------- decode

def _decode_case(seed, B, H, d, dtype, steps):
    st0 = kin.decode_states(B, H, d, seed=seed)
    ins = [kin.decode_step(s, B, H, d, dtype=dtype, seed_base=seed) for s in range(steps)]
    return st0, ins


@pytest.mark.parametrize("dtype,d", [(kin.BF16, 128), (kin.BF16, 64), (kin.BF16, 32),
                                     (kin.F32, 128), (kin.F32, 32)])
def test_decode_steps_parity(dtype, d):
    """A few dependent decode steps on a small batch, every output and the
    final states against the oracle."""
    print(f"[parity] decode dtype={dtype} d={d}", flush=True)
    kda = _kda()
    B, H, steps = 5, 3, 6
    st0, ins = _decode_case(40 + d, B, H, d, dtype, steps)
    state = f32_device(st0)
    ref = st0.astype(np.float64)
    tol = TOL[dtype]
    for x in ins:
        o = kda.decode_step(to_device(x.q, dtype), to_device(x.k, dtype),
                            to_device(x.v, dtype), f32_device(x.g), f32_device(x.beta), state)
        q, k, v, g, b = x.f64()
        o_ref, ref = oracle.decode(q, k, v, g, b, ref)
        eo = relerr(from_device(o), o_ref)
        assert eo <= tol, f"decode output error {eo:.3e}"
    es = relerr(from_device(state), ref)
    print(f"  decode relerr last o={eo:.3e} S={es:.3e}", flush=True)
    assert es <= tol, f"decode state error {es:.3e}"


def test_decode_matches_one_token_prefill():
    """A decode step equals a one-token prefill from the same state."""
    kda = _kda()
    B, H, d = 4, 2, 128
    st0, (x,) = _decode_case(9, B, H, d, kin.BF16, 1)
    state = f32_device(st0)
    o_dec = kda.decode_step(to_device(x.q, kin.BF16), to_device(x.k, kin.BF16),
                            to_device(x.v, kin.BF16), f32_device(x.g), f32_device(x.beta),
                            state)
    q = to_device(x.q, kin.BF16).reshape(B, H, d)
    o_pre, s_pre = kda.fwd_chunked(q, to_device(x.k, kin.BF16), to_device(x.v, kin.BF16),
                                   f32_device(x.g), f32_device(x.beta), num_seqs=B,
                                   initial_state=f32_device(st0), chunk_size=16)
    torch.cuda.synchronize()
    q64, k64, v64, g64, b64 = x.f64()
    o_ref, s_ref = oracle.decode(q64, k64, v64, g64, b64, st0)
    e = [relerr(from_device(o_dec), o_ref), relerr(from_device(state), s_ref),
         relerr(from_device(o_pre), o_ref), relerr(from_device(s_pre), s_ref),
         relerr(from_device(o_dec), from_device(o_pre))]
    print("  decode o/S, prefill o/S, decode-vs-prefill o:", ["%.2e" % x for x in e])
    # decode runs in fp32 and only rounds o to bf16 (unit roundoff 2^-8);
    # the state stays fp32.  The one-token prefill rounds its matrix-core
    # operands (S, Ke, U - W S) to bf16, hence the bf16 bar there.
    assert e[0] < 2.0 ** -8 + 1e-5, "decode o beyond bf16 output rounding"
    assert e[1] < 1e-5, "decode state beyond fp32 rounding"
    assert max(e[2:]) < 2e-2


def test_decode_full_batch_steps():
    """The decode workload at full size and in the benchmark's launch
    configuration (256 x 32 fp32 states, d = 128, bf16 inputs drawn per step
    as the benchmark draws them): 24 dependent steps, every output and the
    states after the last step against the oracle."""
    cfg = kin.WORKLOADS[4]
    B, H, d, steps = cfg["batch"], cfg["H"], cfg["d"], 24
    print(f"[parity] decode full batch {B} x {H}, {steps} steps", flush=True)
    kda = _kda()
    st0 = kin.decode_states(B, H, d, s0_std=cfg["s0_std"])
    state = f32_device(st0)
    ref = st0.astype(np.float64)
    worst = 0.0
    for s in range(steps):
        x = kin.decode_step(s, B, H, d, dtype=kin.BF16, g_mu=cfg["g_mu"], g_sigma=cfg["g_sigma"])
        o = kda.decode_step(to_device(x.q, kin.BF16), to_device(x.k, kin.BF16),
                            to_device(x.v, kin.BF16), f32_device(x.g), f32_device(x.beta), state)
        q, k, v, g, b = x.f64()
        o_ref, ref = oracle.decode(q, k, v, g, b, ref)
        worst = max(worst, relerr(from_device(o), o_ref))
    es = relerr(from_device(state), ref)
    print(f"  decode relerr worst o={worst:.3e} S={es:.3e}", flush=True)
    assert worst <= TOL[kin.BF16] and es <= TOL[kin.BF16]


def decode_sample_states(B, H, n=64):
    """n (batch, head) states spread over the batch and the heads: distinct
    batch rows 4 i + i % 4 and heads (7 i + 3) % H."""
    b = np.array([(4 * i + i % 4) % B for i in range(n)])
    h = np.array([(7 * i + 3) % H for i in range(n)])
    return b, h


def test_decode_workload_all_steps_sampled_states():
    """The whole decode workload: 256 x 32 fp32 states, d = 128, all 1000
    dependent steps with the benchmark's per-step inputs, run at full batch
    on the GPU.  For 64 states spread over batch and heads, every step's
    output and the states after the last step are compared with the oracle
    run on those states alone (the states never mix, so a sample is exact)."""
    import concurrent.futures
    cfg = kin.WORKLOADS[4]
    B, H, d, steps = cfg["batch"], cfg["H"], cfg["d"], cfg["steps"]
    print(f"[parity] decode workload {B} x {H}, all {steps} steps, 64 sampled states",
          flush=True)
    kda = _kda()
    sb, sh = decode_sample_states(B, H)
    st0 = kin.decode_states(B, H, d, s0_std=cfg["s0_std"])
    state = f32_device(st0)
    ref = st0[sb, sh][:, None].astype(np.float64)        # [64, 1, d, d]
    sb_d = torch.from_numpy(sb).cuda()
    sh_d = torch.from_numpy(sh).cuda()
    o_smp = torch.empty((steps, len(sb), d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    host = []

    def gen(s):
        return kin.decode_step(s, B, H, d, dtype=kin.BF16, g_mu=cfg["g_mu"],
                               g_sigma=cfg["g_sigma"])

    workers = min(16, len(os.sched_getaffinity(0)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for s0 in range(0, steps, 4 * workers):
            for s, x in zip(range(s0, steps), ex.map(gen, range(s0, min(steps, s0 + 4 * workers)))):
                kda.decode_step(to_device(x.q, kin.BF16), to_device(x.k, kin.BF16),
                                to_device(x.v, kin.BF16), f32_device(x.g), f32_device(x.beta),
                                state, out=o)
                o_smp[s] = o[sb_d, sh_d]
                host.append(tuple(a[sb, sh][:, None] for a in x.f64()))
            if s0 % 256 == 0:
                print(f"  steps done: {min(steps, s0 + 4 * workers)}", flush=True)
    torch.cuda.synchronize()
    o_gpu = from_device(o_smp)
    worst = 0.0
    for s, (q, k, v, g, b) in enumerate(host):
        o_ref, ref = oracle.decode(q, k, v, g, b, ref)
        worst = max(worst, relerr(o_gpu[s], o_ref[:, 0]))
    es = relerr(from_device(state)[sb, sh], ref[:, 0])
    print(f"  decode relerr worst o over {steps} steps={worst:.3e}, final S={es:.3e}",
          flush=True)
    assert worst <= TOL[kin.BF16], f"decode output error {worst:.3e}"
    assert es <= TOL[kin.BF16], f"decode state error {es:.3e}"


@pytest.mark.parametrize("dtype,d", [(kin.BF16, 128), (kin.BF16, 64), (kin.BF16, 32),
                                     (kin.F32, 128), (kin.F32, 64), (kin.F32, 32)])
@pytest.mark.parametrize("n_seqs", [10, 40, 65])
def test_many_pairs_every_slice_width(dtype, d, n_seqs):
    """Many short packed sequences (4 heads each, lengths 1..150, initial
    states): as the (sequence, head) count grows the inter-chunk launch moves
    from 16- to 32- and 64-column slices (on a 256-CU device: 40 and 260
    pairs at d = 128, 160 pairs at d = 64 and 32), every width against the
    oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"[parity] many pairs dtype={dtype} d={d} seqs={n_seqs} heads=4 cus={cus}", flush=True)
    w = kin.make_prefill(300 + d + n_seqs, B=n_seqs, H=4, d=d, dtype=dtype, chunk_size=32,
                         len_range=(1, 150), s0_std=0.05)
    o, s = _run_gpu(w)
    _check(w, o, s)


@pytest.mark.parametrize("dtype,d,chunk", [(kin.BF16, 128, 64), (kin.BF16, 64, 32),
                                           (kin.F32, 32, 16)])
def test_many_short_packed_sequences(dtype, d, chunk):
    """1,100 packed sequences of 1 to 100 tokens (some chunks straddle no
    boundary, many sequences are a single partial chunk), 2 heads, initial
    states: the chunk table built once per call locates every chunk; all
    outputs and final states against the oracle."""
    print(f"[parity] 1100 short sequences dtype={dtype} d={d} C={chunk}", flush=True)
    w = kin.make_prefill(1100 + d + chunk, B=1100, H=2, d=d, dtype=dtype, chunk_size=chunk,
                         len_range=(1, 100), s0_std=0.05)
    o, s = _run_gpu(w)
    _check(w, o, s)


@pytest.mark.parametrize("dtype,d,chunk,shape", [
    (kin.BF16, 128, 64, dict(B=1, T=8229, H=3)),
    (kin.F32, 64, 32, dict(lengths=[4150, 4303], H=2)),
    (kin.BF16, 32, 16, dict(B=2, T=2085, H=2)),
])
def test_long_chains_with_l2_warmup(dtype, d, chunk, shape):
    """Few (sequence, head) pairs with at least 128 chunks each: the
    inter-chunk launch takes 16-column slices with L2 warm-up loads, equal
    lengths with a partial last chunk and packed sequences, initial states;
    all outputs and final states against the oracle."""
    print(f"[parity] long chains dtype={dtype} d={d} C={chunk} {shape}", flush=True)
    w = kin.make_prefill(2000 + d + chunk, d=d, dtype=dtype, chunk_size=chunk, s0_std=0.05,
                         **shape)
    assert w.total_tokens >= 128 * chunk * w.num_seqs
    o, s = _run_gpu(w)
    _check(w, o, s)


def test_one_long_packed_sequence_among_short_ones():
    """A packed batch whose first sequence spans 1,094 chunks (more chunk-table
    entries than the table kernel has threads), then a 5-token and a
    3,000-token sequence, with initial states: every entry of the chunk table
    and every output against the oracle."""
    print("[parity] packed lengths 70000, 5, 3000, H=1, d=64, C=64", flush=True)
    w = kin.make_prefill(4321, lengths=[70000, 5, 3000], H=1, d=64, dtype=kin.BF16,
                         chunk_size=64, s0_std=0.05)
    o, s = _run_gpu(w)
    _check(w, o, s)


@pytest.mark.parametrize("dtype,d,chunk,shape", [
    (kin.BF16, 128, 64, dict(B=16, len_range=(1, 100), H=2)),
    (kin.BF16, 128, 64, dict(B=600, len_range=(1, 100), H=2)),
    (kin.F32, 64, 32, dict(B=300, len_range=(1, 60), H=2)),
    (kin.BF16, 32, 16, dict(B=64, T=30, H=3)),
    (kin.F32, 128, 64, dict(B=100, T=100, H=2)),
])
def test_short_sequences_one_buffer_chain(dtype, d, chunk, shape):
    """Sequences of at most two chunks on average: the inter-chunk launch takes
    its one-buffer form, with 16- or 32-column slices (packed and equal
    lengths, initial states); all outputs and final states against the
    oracle."""
    print(f"[parity] short sequences dtype={dtype} d={d} C={chunk} {shape}", flush=True)
    w = kin.make_prefill(3000 + d + chunk, d=d, dtype=dtype, chunk_size=chunk, s0_std=0.05,
                         **shape)
    assert w.total_tokens <= 2 * chunk * w.num_seqs
    o, s = _run_gpu(w)
    _check(w, o, s)
