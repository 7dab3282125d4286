"""Output epilogue (kda_options.out_norm_weight / out_gate): per-head RMSNorm
and the sigmoid output gate, against the fp64 oracle (oracle.output_epilogue
applied to the recurrence's output).

docsaid.org "Kimi Linear", section "Les autres pieces"; fr.news.hada.io,
section "Configuration du modele Kimi Linear".

Tolerance.  RMSNorm divides each output row by its own root-mean-square, so
an error that the operator's bound allows (normwise, relative to max|o|)
grows by max|o| / rms(row) on a row with a small output (for instance the
first token of a sequence whose query is nearly orthogonal to its key).  The
epilogue is therefore checked two ways: its error scaled back by each row's
RMS must stay within the operator's tolerance in the operator's units, and
on the rows whose RMS is at least 5% of the median the plain normwise bar
applies.
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


def _epi_inputs(seed, T, H, d, dtype):
    return kin.epilogue_inputs(seed, (T, H), d, dtype)


def _check_epilogue(y, y_ref, o_ref, wn, tol):
    """The two bars of the module docstring; returns (scaled, well-conditioned)."""
    rms = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True))
    scaled = float(np.max(np.abs(y - y_ref) * rms) /
                   (np.max(np.abs(o_ref)) * np.max(np.abs(wn))))
    ok = (rms[..., 0] >= 0.05 * np.median(rms))
    well = relerr(y[ok], y_ref[ok])
    print(f"  epilogue: scaled {scaled:.3e}, well-conditioned rows {well:.3e} "
          f"({ok.mean():.5f} of rows)", flush=True)
    assert scaled <= tol, f"epilogue error in operator units {scaled:.3e} > {tol}"
    assert well <= tol, f"epilogue error on well-conditioned rows {well:.3e} > {tol}"
    return scaled, well


@pytest.mark.parametrize("with_gate", [True, False])
@pytest.mark.parametrize("dtype,d,chunk", [(kin.BF16, 128, 64), (kin.BF16, 64, 16),
                                           (kin.BF16, 32, 32), (kin.F32, 32, 16),
                                           (kin.F32, 64, 32), (kin.F32, 128, 64)])
def test_prefill_epilogue(dtype, d, chunk, with_gate):
    print(f"[epilogue] prefill dtype={dtype} d={d} C={chunk} gate={with_gate}", flush=True)
    kda = _kda()
    w = kin.make_prefill(300 + d, H=3, d=d, dtype=dtype, chunk_size=chunk,
                         lengths=[100, 1, 0, 45], s0_std=0.05)
    wn, z = _epi_inputs(301 + d, w.total_tokens, 3, d, dtype)
    dd = upload_prefill(w)
    o, s = kda.fwd_chunked(dd["q"], dd["k"], dd["v"], dd["log_alpha"], dd["beta"],
                           cu_seqlens=dd["cu_seqlens"], initial_state=dd["initial_state"],
                           chunk_size=chunk, out_norm_weight=f32_device(wn),
                           out_gate=to_device(z, dtype) if with_gate else None,
                           out_norm_eps=1e-6)
    torch.cuda.synchronize()
    q, k, v, g, b, s0 = w.f64()
    o_ref, s_ref = oracle.recurrent(q, k, v, g, b, cu_seqlens=w.cu_seqlens.astype(np.int64),
                                    initial_state=s0)
    y_ref = oracle.output_epilogue(o_ref, wn, 1e-6,
                                   kin.as_f64(z, dtype) if with_gate else None)
    es = relerr(from_device(s), s_ref)
    print(f"  relerr S={es:.3e}", flush=True)
    assert es <= TOL[dtype]
    _check_epilogue(from_device(o), y_ref, o_ref, wn, TOL[dtype])


@pytest.mark.parametrize("dtype,d", [(kin.BF16, 128), (kin.BF16, 64), (kin.BF16, 32),
                                     (kin.F32, 128), (kin.F32, 64), (kin.F32, 32)])
def test_decode_epilogue_fused(dtype, d):
    """The decode kernel applies the epilogue to its fp32 output row."""
    print(f"[epilogue] decode dtype={dtype} d={d}", flush=True)
    kda = _kda()
    B, H = 5, 3
    st0 = kin.decode_states(B, H, d, seed=310 + d)
    state = f32_device(st0)
    ref = st0.astype(np.float64)
    wn, _ = _epi_inputs(311 + d, 1, H, d, dtype)
    for step in range(3):
        x = kin.decode_step(step, B, H, d, dtype=dtype, seed_base=310 + d)
        _, z = _epi_inputs(320 + step, B, H, d, dtype)
        o = kda.decode_step(to_device(x.q, dtype), to_device(x.k, dtype), to_device(x.v, dtype),
                            f32_device(x.g), f32_device(x.beta), state,
                            out_norm_weight=f32_device(wn), out_gate=to_device(z, dtype))
        q, k, v, g, b = x.f64()
        o_ref, ref = oracle.decode(q, k, v, g, b, ref)
        y_ref = oracle.output_epilogue(o_ref, wn, 1e-6, kin.as_f64(z, dtype))
        eo = relerr(from_device(o), y_ref)
        assert eo <= TOL[dtype], f"decode epilogue error {eo:.3e} at step {step}"
    assert relerr(from_device(state), ref) <= TOL[dtype]


def test_model_form_headline():
    """The B=2, H=8, T=2048 prefill at the model boundary: raw inputs (softplus
    gate, q/k normalisation, beta logits) and the output epilogue, every
    output and final state against prepare_inputs -> recurrence ->
    output_epilogue in fp64."""
    print("[epilogue] model-form prefill B=2 H=8 T=2048", flush=True)
    kda = _kda()
    w = kin.raw_prefill_workload()
    dt = w.dtype
    opt = w.options()
    opt["gate_A"] = f32_device(opt["gate_A"])
    o, s = kda.fwd_chunked(to_device(w.q, dt), to_device(w.k, dt), to_device(w.v, dt),
                           to_device(w.z, dt), f32_device(w.beta_logits), num_seqs=w.num_seqs,
                           chunk_size=w.chunk_size, out_norm_weight=f32_device(w.out_norm_weight),
                           out_gate=to_device(w.out_gate, dt), **opt)
    torch.cuda.synchronize()
    q, k, v, z, bl, _ = w.f64()
    qn, kn, g, b = oracle.prepare_inputs(q, k, z, bl, **w.options())
    o_ref, s_ref = oracle.recurrent(qn, kn, v, g, b, num_seqs=w.num_seqs)
    y_ref = oracle.output_epilogue(o_ref, w.out_norm_weight, 1e-6, kin.as_f64(w.out_gate, dt))
    es = relerr(from_device(s), s_ref)
    print(f"  relerr S={es:.3e}", flush=True)
    assert es <= TOL[dt]
    _check_epilogue(from_device(o), y_ref, o_ref, w.out_norm_weight, TOL[dt])
