"""Seeded combinations of the prefill options against the fp64 oracle: the
gate (g itself, Kimi Linear's softplus gate or K3's bounded sigmoid, with
q/k normalisation and beta from logits), state slots with a padding entry
(the pool updated in place), and the output epilogue (RMSNorm alone or with
the output gate), on ragged packed sequences.

Sources: fr.news.hada.io Kimi Linear summary, section "Algorithme parallele
par chunks"; docsaid.org "Kimi Linear", sections "Les autres pieces" and
"Calculer le cache a la main".
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


def _cases(n=10, seed=88):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        chunk = int(rng.choice([16, 32, 64]))
        N = int(rng.integers(2, 6))
        lengths = [int(x) for x in rng.integers(0, 2 * chunk + 10, size=N)]
        lengths[int(rng.integers(0, N))] = 1
        out.append(dict(
            i=i, dtype=kin.BF16 if rng.random() < 0.6 else kin.F32,
            d=int(rng.choice([32, 64, 128])), chunk=chunk, H=int(rng.integers(1, 4)),
            lengths=lengths, gate=str(rng.choice(["log_alpha", "softplus", "sigmoid"])),
            slots=bool(rng.random() < 0.5),
            epilogue=str(rng.choice(["none", "norm", "norm+gate"]))))
    return out


CASES = _cases()


def _kda():
    import gated_delta_rule_chunked_amd as kda
    return kda


def _epilogue_bars(y, y_ref, o_ref, wn, tol):
    """The epilogue's two bars: its error scaled back by each row's RMS, and
    the plain normwise error on rows whose RMS is at least 5% of the median."""
    rms = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True))
    scaled = float(np.max(np.abs(y - y_ref) * rms) / (np.max(np.abs(o_ref)) * np.max(np.abs(wn))))
    ok = rms[..., 0] >= 0.05 * np.median(rms)
    well = relerr(y[ok], y_ref[ok])
    assert scaled <= tol, f"epilogue error in operator units {scaled:.3e}"
    assert well <= tol, f"epilogue error on well-conditioned rows {well:.3e}"
    return scaled, well


@pytest.mark.parametrize("c", CASES, ids=[f"case{c['i']}" for c in CASES])
def test_prefill_option_combination(c):
    print(f"[prefill options] {c}", flush=True)
    kda = _kda()
    i, dtype, d, chunk, H = c["i"], c["dtype"], c["d"], c["chunk"], c["H"]
    tol = TOL[dtype]
    kw = {}
    if c["gate"] == "log_alpha":
        w = kin.make_prefill(700 + i, H=H, d=d, dtype=dtype, chunk_size=chunk,
                             lengths=c["lengths"], s0_std=0.05)
        q, k, v, g, b, s0 = w.f64()
        args = (to_device(w.q, dtype), to_device(w.k, dtype), to_device(w.v, dtype),
                f32_device(w.g), f32_device(w.beta))
    else:
        w = kin.make_prefill_raw(700 + i, H=H, d=d, dtype=dtype, chunk_size=chunk,
                                 gate=c["gate"], lengths=c["lengths"], s0_std=0.05)
        q0, k0, v, z, bl, s0 = w.f64()
        opt = w.options()
        q, k, g, b = oracle.prepare_inputs(q0, k0, z, bl, **opt)
        kw.update(opt)
        if opt["gate_A"] is not None:
            kw["gate_A"] = f32_device(opt["gate_A"])
        args = (to_device(w.q, dtype), to_device(w.k, dtype), to_device(w.v, dtype),
                to_device(w.z, dtype), f32_device(w.beta_logits))
    N, T = w.num_seqs, w.total_tokens
    cu_h = w.cu_seqlens.astype(np.int64)
    cu = torch.from_numpy(w.cu_seqlens.astype(np.int32)).cuda()
    if c["slots"]:
        NS = N + 2
        slots = np.arange(N, dtype=np.int32) + 2
        slots[0] = -1  # a padding entry of the batch
        pool0 = kin.decode_states(NS, H, d, seed=800 + i)
        init = np.zeros((N, H, d, d))
        for s_i, s in enumerate(slots):
            if s >= 0:
                init[s_i] = pool0[s]
        pool = f32_device(pool0)
        kw.update(state_slots=torch.from_numpy(slots).cuda())
        state_arg = pool
    else:
        init = s0
        state_arg = f32_device(s0)
    wn = zo = None
    if c["epilogue"] != "none":
        wn, zo = kin.epilogue_inputs(900 + i, (T, H), d, dtype)
        kw.update(out_norm_weight=f32_device(wn), out_norm_eps=1e-6)
        if c["epilogue"] == "norm+gate":
            kw["out_gate"] = to_device(zo, dtype)
        else:
            zo = None
    o, s = kda.fwd_chunked(*args, cu_seqlens=cu, num_seqs=N, initial_state=state_arg,
                           chunk_size=chunk, **kw)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrent(q, k, v, g, b, cu_seqlens=cu_h, num_seqs=N,
                                    initial_state=init)
    oh = from_device(o)
    if c["epilogue"] != "none":
        y_ref = oracle.output_epilogue(o_ref, wn, 1e-6,
                                       None if zo is None else kin.as_f64(zo, dtype))
        _epilogue_bars(oh, y_ref, o_ref, wn, tol)
    else:
        assert relerr(oh, o_ref) <= tol
    if c["slots"]:
        got = from_device(pool)
        for s_i, sl in enumerate(slots):
            if sl >= 0:
                assert relerr(got[sl], s_ref[s_i]) <= tol
        for sl in (0, 1):  # slots no sequence maps to
            assert np.array_equal(got[sl], pool0[sl].astype(np.float64))
    else:
        assert relerr(from_device(s), s_ref) <= tol
