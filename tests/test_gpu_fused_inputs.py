"""Input-side fusion (kda_options; kda_fwd_chunked_ex, kda_decode_step_ex):
parity of the fused calls with the fp64 oracle applied to the transformed
inputs (oracle.prepare_inputs: gate function, q/k L2 normalisation, beta
from logits), at the tolerances of the plain calls.

Sources: docsaid.org "Kimi Linear", section "Les autres pieces";
mkdocs.reaper.mx "Attention lineaire et recurrence", section "Le piege
numerique de la decroissance cumulee" (Kimi Linear's softplus gate and K3's
bounded sigmoid gate).
"""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from gated_delta_rule_chunked_amd import inputs as kin  # noqa: E402
from kda_testutil import TOL, from_device, relerr, to_device, f32_device  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _kda():
    import gated_delta_rule_chunked_amd as kda
    return kda


def _device_options(w):
    opt = w.options()
    if opt["gate_A"] is not None:
        opt["gate_A"] = f32_device(opt["gate_A"])
    return opt


def _run_raw(w, stage_split=False):
    kda = _kda()
    dt = w.dtype
    args = (to_device(w.q, dt), to_device(w.k, dt), to_device(w.v, dt), to_device(w.z, dt),
            f32_device(w.beta_logits))
    cu = None if w.cu_seqlens is None else torch.from_numpy(
        w.cu_seqlens.astype(np.int32)).cuda()
    s0 = None if w.initial_state is None else f32_device(w.initial_state)
    kw = dict(cu_seqlens=cu, num_seqs=w.num_seqs, initial_state=s0, chunk_size=w.chunk_size,
              **_device_options(w))
    if not stage_split:
        o, s = kda.fwd_chunked(*args, **kw)
    else:
        call, stages, o, s = kda.bind_fwd(*args, **kw)
        stages["intra"]()
        stages["inter"]()
    torch.cuda.synchronize()
    return from_device(o), from_device(s)


def _oracle_raw(w, heads=None):
    q, k, v, z, bl, s0 = w.f64()
    opt = w.options()
    q, k, g, b = oracle.prepare_inputs(q, k, z, bl, **opt)
    if heads is not None:
        q, k, v, g, b = q[:, heads], k[:, heads], v[:, heads], g[:, heads], b[:, heads]
        s0 = None if s0 is None else s0[:, heads]
    cu = None if w.cu_seqlens is None else w.cu_seqlens.astype(np.int64)
    return oracle.recurrent(q, k, v, g, b, cu_seqlens=cu, num_seqs=w.num_seqs,
                            initial_state=s0)


def _check(w, o, s, heads=None):
    tol = TOL[w.dtype]
    o_ref, s_ref = _oracle_raw(w, heads)
    if heads is not None:
        o, s = o[:, heads], s[:, heads]
    eo, es = relerr(o, o_ref), relerr(s, s_ref)
    print(f"  relerr o={eo:.3e} S={es:.3e} (tol {tol:g})", flush=True)
    assert eo <= tol, f"output error {eo:.3e} > {tol}"
    assert es <= tol, f"final-state error {es:.3e} > {tol}"


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
@pytest.mark.parametrize("dtype,d,chunk", [(kin.BF16, 128, 64), (kin.BF16, 64, 32),
                                           (kin.BF16, 32, 16), (kin.F32, 32, 16),
                                           (kin.F32, 64, 64)])
def test_fused_prefill_ragged(gate, dtype, d, chunk):
    """Raw q/k, gate input z and beta logits on ragged packed sequences (an
    empty and a one-token sequence, tails, initial states)."""
    print(f"[fused] prefill gate={gate} dtype={dtype} d={d} C={chunk}", flush=True)
    w = kin.make_prefill_raw(200 + d + chunk, H=3, d=d, dtype=dtype, chunk_size=chunk,
                             gate=gate, lengths=[130, 0, 1, 64, 77], s0_std=0.05)
    o, s = _run_raw(w)
    _check(w, o, s)


_EVERY_SHAPE = [(dt, d, c) for dt in (kin.BF16, kin.F32) for d in (32, 64, 128)
                for c in (16, 32, 64)]


@pytest.mark.parametrize("dtype,d,chunk", _EVERY_SHAPE)
def test_fused_prefill_every_shape(dtype, d, chunk):
    """Every supported (dtype, head size, chunk size) with the softplus gate:
    a full chunk plus a tail, a one-token sequence, two chunks plus a tail."""
    print(f"[fused] prefill every shape dtype={dtype} d={d} C={chunk}", flush=True)
    w = kin.make_prefill_raw(400 + d + chunk, H=2, d=d, dtype=dtype, chunk_size=chunk,
                             gate="softplus", lengths=[chunk + 5, 1, 2 * chunk + 3],
                             s0_std=0.05)
    o, s = _run_raw(w)
    _check(w, o, s)


def test_fused_headline_raw_workload():
    """The B=2, H=8, T=2048 prefill in raw form (softplus gate), every output
    and final state, run stage by stage through kda_fwd_chunked_ex."""
    print("[fused] prefill_raw B=2 H=8 T=2048", flush=True)
    w = kin.raw_prefill_workload(with_epilogue=False)
    o, s = _run_raw(w, stage_split=True)
    _check(w, o, s)


def test_ex_entry_without_options_is_the_plain_call():
    """kda_fwd_chunked_ex with all options off runs the plain call: the same
    bits as kda_fwd_chunked."""
    kda = _kda()
    lib = kda.library()
    import ctypes
    w = kin.make_prefill(11, H=2, d=64, dtype=kin.BF16, chunk_size=32, lengths=[90, 33])
    dt = w.dtype
    q, k, v = to_device(w.q, dt), to_device(w.k, dt), to_device(w.v, dt)
    g, b = f32_device(w.g), f32_device(w.beta)
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).cuda()
    o1, s1 = kda.fwd_chunked(q, k, v, g, b, cu_seqlens=cu, chunk_size=32)
    call, _, o2, s2 = kda.bind_fwd(q, k, v, g, b, cu_seqlens=cu, chunk_size=32)
    args = call._args
    opt = ctypes.pointer(kda.kda.KdaOptions(0, None, 0.0, 0, 0))
    st = lib.kda_fwd_chunked_ex(opt, 3, *args)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("gate", ["softplus", "sigmoid"])
@pytest.mark.parametrize("dtype,d", [(kin.BF16, 128), (kin.BF16, 64), (kin.BF16, 32),
                                     (kin.F32, 128), (kin.F32, 64), (kin.F32, 32)])
def test_fused_decode_steps(gate, dtype, d):
    """Dependent decode steps with raw inputs against oracle.decode on the
    transformed inputs."""
    print(f"[fused] decode gate={gate} dtype={dtype} d={d}", flush=True)
    kda = _kda()
    B, H, steps = 5, 3, 5
    st0 = kin.decode_states(B, H, d, seed=70 + d)
    state = f32_device(st0)
    ref = st0.astype(np.float64)
    tol = TOL[dtype]
    for step in range(steps):
        x = kin.decode_step_raw(step, B, H, d, dtype, gate, seed_base=70 + d)
        o = kda.decode_step(to_device(x.q, dtype), to_device(x.k, dtype),
                            to_device(x.v, dtype), to_device(x.z, dtype),
                            f32_device(x.beta_logits), state, **_device_options(x))
        q, k, v, z, bl, _ = x.f64()
        qn, kn, g, b = oracle.prepare_inputs(q, k, z, bl, **x.options())
        o_ref, ref = oracle.decode(qn, kn, v, g, b, ref)
        eo = relerr(from_device(o), o_ref)
        assert eo <= tol, f"decode output error {eo:.3e} at step {step}"
    es = relerr(from_device(state), ref)
    print(f"  relerr last o={eo:.3e} S={es:.3e}", flush=True)
    assert es <= tol, f"decode state error {es:.3e}"
