"""Seeded combinations of the decode options against the fp64 oracle:
the gate (g itself, Kimi Linear's softplus gate or K3's bounded sigmoid,
with q/k normalisation and beta from logits), state slots with padding
entries, and the output epilogue (RMSNorm alone or with the output gate),
over three dependent steps each.

Sources: mkdocs.reaper.mx "Attention lineaire et recurrence", section "Kimi
Delta Attention = les trois remedes combines" (the step); docsaid.org "Kimi
Linear", sections "Les autres pieces" (gate, normalisation, beta, epilogue)
and "Calculer le cache a la main" (a fixed state per request).
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


def _cases(n=12, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append(dict(
            i=i,
            dtype=kin.BF16 if rng.random() < 0.6 else kin.F32,
            d=int(rng.choice([32, 64, 128])),
            B=int(rng.integers(1, 7)),
            H=int(rng.integers(1, 4)),
            gate=str(rng.choice(["log_alpha", "softplus", "sigmoid"])),
            slots=bool(rng.random() < 0.5),
            epilogue=str(rng.choice(["none", "norm", "norm+gate"]))))
    return out


CASES = _cases()


def _kda():
    import gated_delta_rule_chunked_amd as kda
    return kda


@pytest.mark.parametrize("c", CASES, ids=[f"case{c['i']}" for c in CASES])
def test_decode_option_combination(c):
    print(f"[decode options] {c}", flush=True)
    kda = _kda()
    i, dtype, d, B, H = c["i"], c["dtype"], c["d"], c["B"], c["H"]
    tol = TOL[dtype]
    if c["slots"]:  # a pool with two more slots than live requests; one padding entry
        NS = B + 2
        slots = np.arange(B, dtype=np.int32)[::-1] + 1
        slots[0] = -1 if B > 1 else slots[0]
    else:
        NS, slots = B, None
    pool0 = kin.decode_states(NS, H, d, seed=300 + i)
    pool = f32_device(pool0)
    ref = pool0.astype(np.float64)
    sl = None if slots is None else torch.from_numpy(slots).cuda()
    live = list(range(B)) if slots is None else [b for b in range(B) if 0 <= slots[b] < NS]
    rows = np.arange(B) if slots is None else slots
    wn = None
    if c["epilogue"] != "none":
        wn, _ = kin.epilogue_inputs(400 + i, (1, H), d, dtype)
    for step in range(3):
        kw = {}
        if c["gate"] == "log_alpha":
            x = kin.decode_step(step, B, H, d, dtype=dtype, seed_base=500 + i)
            args = (to_device(x.q, dtype), to_device(x.k, dtype), to_device(x.v, dtype),
                    f32_device(x.g), f32_device(x.beta))
            q, k, v, g, b = x.f64()
        else:
            x = kin.decode_step_raw(step, B, H, d, dtype, c["gate"], seed_base=500 + i)
            opt = x.options()
            kw.update(opt)
            if opt["gate_A"] is not None:
                kw["gate_A"] = f32_device(opt["gate_A"])
            args = (to_device(x.q, dtype), to_device(x.k, dtype), to_device(x.v, dtype),
                    to_device(x.z, dtype), f32_device(x.beta_logits))
            q0, k0, v, z, bl, _ = x.f64()
            q, k, g, b = oracle.prepare_inputs(q0, k0, z, bl, **opt)
        zo = None
        if c["epilogue"] != "none":
            kw["out_norm_weight"] = f32_device(wn)
            kw["out_norm_eps"] = 1e-6
            if c["epilogue"] == "norm+gate":
                _, zo = kin.epilogue_inputs(600 + 10 * i + step, (B, H), d, dtype)
                kw["out_gate"] = to_device(zo, dtype)
        if sl is not None:
            kw["state_slots"] = sl
        o = kda.decode_step(*args, pool, **kw)
        o_ref, st = oracle.decode(q[live], k[live], v[live], g[live], b[live],
                                  ref[rows[live]])
        ref[rows[live]] = st
        if c["epilogue"] != "none":
            o_ref = oracle.output_epilogue(o_ref, wn, 1e-6,
                                           None if zo is None else kin.as_f64(zo, dtype)[live])
        oh = from_device(o)
        eo = relerr(oh[live], o_ref)
        assert eo <= tol, f"step {step}: output error {eo:.3e}"
        pad = [bb for bb in range(B) if bb not in live]
        assert np.all(oh[pad] == 0.0)
    es = relerr(from_device(pool), ref)
    print(f"  relerr last o={eo:.3e} state pool={es:.3e}", flush=True)
    assert es <= tol
