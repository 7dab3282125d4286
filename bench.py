#!/usr/bin/env python3
"""Throughput of the KDA operator (libkda.so) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--extra prefill,varlen,raw,bwd,decode]

Headline: long-context chunked prefill, B=1 sequence x T=32768 tokens,
H=32 heads, d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 log-decay/beta/state,
zero initial state (log-decay -exp(N(-4, 1))).  One step = one
kda_fwd_chunked call (intra-chunk kernel: cumulative log-decay + UT/WY
factors -> inter-chunk state pass) over that batch; `value` is prefill
tokens/s over K timed steps with every input resident in HBM.

Also reported on the same JSON line:
  roofline      the headline call's algorithmic HBM bytes (1,540 B per
                token-head for q, k, v, o in bf16, fp32 log-decay and beta,
                plus 64 KiB per final state) over the whole call's time
                (HIP events on the launch stream), against the larger of the
                HBM and bf16 matrix-core times; the same bytes over the
                dominant kernel's average launch time; the workspace-inclusive
                bytes that kernel moves; and the HBM traffic the FETCH_SIZE /
                WRITE_SIZE counters measured for the call
  cpu_baseline  the fp64 CPU oracle (test infrastructure) timed on the host
                cores on whole passes of the headline workload
  parity        every workload's max normwise relative error of o and of the
                final states against the fp64 oracle, from this run's own
                outputs (decode: 64 sampled states over every step)
  workloads     the B=2, H=8, T=2048 prefill, the varlen packed prefill (16
                seqs of U[512, 8192] tokens, H=16, initial states), that
                B=2 prefill in model-boundary form (input-side fusion:
                softplus gate from bf16 z, q/k L2-normalised, beta from
                logits; output epilogue: per-head RMSNorm and sigmoid output
                gate), the backward of the B=2 prefill (training) and
                recurrent decode (batch 256, H=32, 1000 steps) -- each with
                throughput, fraction of its roofline and its oracle errors.
Inputs come from gated_delta_rule_chunked_amd.inputs (seeded, synthetic).
Only one GPU is supported: --gpus above 1 exits with an error.

`traffic` comes from profiles/hbm_traffic_counters.md (FETCH_SIZE and
WRITE_SIZE, each from its own rocprofv3 --pmc run, scaled by what the same
counters read for a plain device copy of known size, `--only copy`).  A
kernel's reading counts only while its sources hash to the value recorded
with it; otherwise the field is null.
"""
import argparse
import concurrent.futures
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from gated_delta_rule_chunked_amd import inputs as kin  # noqa: E402

# MI355X published peaks (AMD specifications): HBM3E bandwidth and dense
# bf16 matrix throughput.
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
FP32_MFMA_PEAK_TFLOPS = 157.3  # dense fp32 on the matrix cores

METRIC = "KDA prefill tokens/s + decode steps/s on 1 GPU; % of MFMA / HBM roofline"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------- work model
# Algorithmic bytes and flops per unit (a token-head for prefill, a
# (sequence, head) state for decode).  E = bytes per q/k/v/o element, d the
# head size, C the chunk size.

def prefill_bytes_per_token_head(d, E, raw=False, epilogue=False):
    """q, k, v, o in the operand type, fp32 log-decay, fp32 beta; in raw form
    the gate input z in the operand type replaces the fp32 log-decay; the
    output epilogue adds the output-gate input."""
    return 4 * E * d + (E * d if raw else 4 * d) + 4 + (E * d if epilogue else 0)


def prefill_flops_per_token_head(d, C):
    """Chunked form, triangular blocks counted once: K K^T and Q K^T blocks
    (C d), UT substitution (C^2/3), W and U (2 C d), U - W S, Q S and the
    state update (6 d^2), P U (C d)."""
    return 5 * C * d + C * C / 3.0 + 6 * d * d


def state_bytes(d):
    return 4 * d * d


def backward_flops_per_token_head(d, C):
    """The method's matrix work in the backward, per token-head, triangular
    blocks counted once.  Per tile of C tokens, in multiply-adds: C d^2 for
    each of Qt^T dO, the two steps of each state chain, dO S^T, Unew dS^T,
    dUnew S^T and the recomputed U - W S (9); C^2 d / 2 for each triangular
    product (M, P, W, U, P^T dO, dP, dP Kh, the two terms of dT, T^T dW,
    T^T dUnew, dM Kh, dM^T Kt, dP^T Qt: 14); C^3 / 6 for T and for each of the
    two products of dA = -T^T dT T^T.  2 flops a multiply-add."""
    macs = 9 * C * d * d + 7 * C * C * d + C ** 3 / 2.0
    return 2 * macs / C


def backward_bytes_per_token_head(d, E):
    """Read q, k, v, d_o (operand type), log-decay (fp32), beta; write dq, dk,
    dv (operand type), dg (fp32), dbeta."""
    return 4 * E * d + 4 * d + 4 + 3 * E * d + 4 * d + 4


# ---------------------------------------------------------------- counters

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
CSRC = os.path.join(ROOT, "gated_delta_rule_chunked_amd", "csrc")
KERNEL_SOURCES = {"intra": ("kda_intra.hip",), "inter": ("kda_inter.hip", "kda_epilogue.hip"),
                  "decode_kernel": ("kda_decode.hip",), "bwd": ("kda_backward.hip",)}


def kernel_source_sha(kernel):
    """sha256 over the sources of a stage's kernels and the headers they
    include (the inter stage runs the output epilogue pass when asked)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ("kda_common.hpp", "kda_internal.hpp"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch from the committed counter readings, or None."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if m is None:
        return None
    data = json.loads(m.group(1))
    rec = data["kernels"].get(f"{workload}/{kernel}")
    if rec is None or rec["sources_sha256"] != kernel_source_sha(kernel):
        return None
    return (rec["fetch_kib"] * 1024 * data["fetch_scale"] +
            rec["write_kib"] * 1024 * data["write_scale"])


def kernel_bytes(stage, token_heads, pairs, d, E, C, with_s0, raw=False, epilogue=False):
    """Algorithmic HBM bytes of one launch of a prefill kernel: what it must
    read and write given the two-kernel split (workspace tensors count)."""
    CK = max(C, 32)
    # P is lower triangular: with C = 64 the token K-step 32..63 of token
    # blocks 0 and 1 is zero, neither stored nor read (a quarter of P)
    p_bytes = E * CK * (0.75 if C == 64 else 1.0)
    if stage == "intra":      # read q, k, v, g (or z), beta; write Qt, W, U, Ke, P, e^G_n
        gate = E * d if raw else 4 * d
        return token_heads * (3 * E * d + gate + 4 + 4 * E * d + p_bytes + 4 * d / C)
    if stage == "inter":      # read Qt, W, U, Ke, P, e^G_n; write o; states
        epi = 3 * E * d if epilogue else 0  # epilogue pass: read o, z_o; write o
        return (token_heads * (4 * E * d + p_bytes + E * d + 4 * d / C + epi) +
                pairs * state_bytes(d) * (2 if with_s0 else 1))
    raise ValueError(stage)


def decode_bytes_per_state(d, E):
    """State read + write (fp32), q, k, v, o, log-decay, beta."""
    return 2 * state_bytes(d) + 4 * E * d + 4 * d + 4


# ---------------------------------------------------------------- helpers

def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


# Milliseconds of untimed whole calls that precede a workload's warmup steps.
# After the host-side input set-up the GPU has been idle, and its clocks take
# tens of ms of sustained load to settle: the first ~25 calls of the long
# prefill after an idle pause run 5-20% slower than the later ones, so a
# short warmup would time part of that ramp instead of the sustained rate.
SETTLE_MS = 100.0


def settle(torch, fn, ms):
    """Runs fn() untimed until `ms` of wall time has passed, synchronizing
    every few calls so that the wall time is GPU time; returns the count."""
    n = 0
    t = time.perf_counter()
    while (time.perf_counter() - t) * 1e3 < ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def upload_prefill(torch, w):
    """Seeded host arrays -> device tensors (exact bits, no torch compute)."""
    def op(a):
        if w.dtype == kin.BF16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    cu = (None if w.cu_seqlens is None else
          torch.from_numpy(w.cu_seqlens.astype(np.int32)).cuda())
    s0 = None if w.initial_state is None else f32(w.initial_state)
    return dict(q=op(w.q), k=op(w.k), v=op(w.v), log_alpha=f32(w.g),
                beta=f32(w.beta), cu_seqlens=cu, num_seqs=w.num_seqs,
                initial_state=s0)


def upload_prefill_raw(torch, w):
    """Raw-form workload (inputs.RawPrefill) -> bind_fwd arguments."""
    def op(a):
        if w.dtype == kin.BF16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    opt = w.options()
    if opt["gate_A"] is not None:
        opt["gate_A"] = torch.from_numpy(np.ascontiguousarray(opt["gate_A"])).cuda()
    if w.out_norm_weight is not None:
        opt["out_norm_weight"] = torch.from_numpy(w.out_norm_weight).cuda()
        opt["out_gate"] = op(w.out_gate)
    return dict(q=op(w.q), k=op(w.k), v=op(w.v), log_alpha=op(w.z),
                beta=torch.from_numpy(np.ascontiguousarray(w.beta_logits)).cuda(),
                cu_seqlens=None, num_seqs=w.num_seqs, initial_state=None, options=opt)


def time_prefill(torch, kda, w, steps, warmup, per_kernel=True, settle_ms=SETTLE_MS):
    """Times `steps` whole prefill calls, then each kernel separately.  The
    outputs of the last call stay in res["o"], res["final_state"]."""
    raw = isinstance(w, kin.RawPrefill)
    d_in = upload_prefill_raw(torch, w) if raw else upload_prefill(torch, w)
    call, stages, o, fs = kda.bind_fwd(
        d_in["q"], d_in["k"], d_in["v"], d_in["log_alpha"], d_in["beta"],
        cu_seqlens=d_in["cu_seqlens"], num_seqs=d_in["num_seqs"],
        initial_state=d_in["initial_state"], chunk_size=w.chunk_size,
        **d_in.get("options", {}))
    settled = settle(torch, call, settle_ms)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    t_wall = time.perf_counter()
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / steps
    res = dict(ms_per_step=ms, wall_ms_per_step=1e3 * t_wall / steps, settle_calls=settled)
    if per_kernel:
        # the two kernels of the same call, each bracketed by events on
        # the launch stream, over the same number of passes
        names = ("intra", "inter")
        ev = [_events(torch, len(names) + 1) for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record()
            for j, nm in enumerate(names):
                stages[nm]()
                ev[i][j + 1].record()
        torch.cuda.synchronize()
        res["kernel_us"] = {
            nm: 1e3 * sum(ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(steps)) / steps
            for j, nm in enumerate(names)}
    # one more whole call, so that o and the final state are a clean call's
    call()
    torch.cuda.synchronize()
    res["o"] = o.detach().to(torch.float64).cpu().numpy()
    res["final_state"] = fs.detach().to(torch.float64).cpu().numpy()
    del d_in, call, stages, o, fs
    torch.cuda.empty_cache()
    return res


def prefill_algorithmic(w, d, E, C):
    """(bytes, flops) the method must move and compute for workload w."""
    th = w.total_tokens * w.num_heads
    s0 = w.initial_state is not None
    raw = isinstance(w, kin.RawPrefill)
    epi = raw and w.out_norm_weight is not None
    byts = th * prefill_bytes_per_token_head(d, E, raw, epi) + w.num_seqs * w.num_heads * \
        state_bytes(d) * (2 if s0 else 1)
    return byts, th * prefill_flops_per_token_head(d, C)


def roof_time(byts, flops):
    return max(byts / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))


def prefill_report(w, res, d, E, C):
    T = w.total_tokens
    byts, flops = prefill_algorithmic(w, d, E, C)
    t_roof = roof_time(byts, flops)
    sec = res["ms_per_step"] * 1e-3
    out = dict(tokens_per_s=T / sec, ms_per_step=res["ms_per_step"],
               roofline_tokens_per_s=T / t_roof, roofline_frac=t_roof / sec,
               algorithmic_bytes=byts, algorithmic_flops=flops,
               achieved_gbs=byts / sec / 1e9,
               mfma_frac_algorithmic=flops / sec / (BF16_PEAK_TFLOPS * 1e12))
    if "kernel_us" in res:
        out["kernel_us"] = res["kernel_us"]
    out["settle_calls"] = res.get("settle_calls", 0)
    return out


def call_roofline(wname, w, res, d, E, C):
    """The call's algorithmic bytes over the whole call's time (`frac`), and
    over the dominant kernel's average launch time; the workspace-inclusive
    bytes that kernel moves given the two-kernel split; the counter-measured
    HBM traffic of the call."""
    byts, flops = prefill_algorithmic(w, d, E, C)
    call_s = res["ms_per_step"] * 1e-3
    ach = byts / call_s / 1e9
    roof = dict(bound="hbm" if byts / (HBM_PEAK_GBS * 1e9) >= flops / (BF16_PEAK_TFLOPS * 1e12)
                else "mfma",
                achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=roof_time(byts, flops) / call_s,
                scope="whole kda_fwd_chunked call (intra-chunk + inter-chunk kernels)",
                algorithmic_bytes=byts, avg_call_us=call_s * 1e6)
    ku = res["kernel_us"]
    name = max(ku, key=ku.get)
    th = w.total_tokens * w.num_heads
    raw = isinstance(w, kin.RawPrefill)
    wsb = kernel_bytes(name, th, w.num_seqs * w.num_heads, d, E, C,
                       w.initial_state is not None, raw=raw,
                       epilogue=raw and w.out_norm_weight is not None)
    roof["dominant_kernel"] = dict(
        kernel=name, avg_launch_us=ku[name],
        achieved=byts / (ku[name] * 1e-6) / 1e9,
        frac=byts / (ku[name] * 1e-6) / 1e9 / HBM_PEAK_GBS,
        workspace_inclusive_bytes=wsb,
        workspace_inclusive_gbs=wsb / (ku[name] * 1e-6) / 1e9)
    tr = [measured_traffic(wname, k) for k in ("intra", "inter")]
    roof["traffic"] = None if None in tr else sum(tr)
    roof["traffic_over_algorithmic"] = None if None in tr else sum(tr) / byts
    return roof


# ---------------------------------------------------------------- parity

def normwise(x, ref):
    """max|x - ref| / max|ref| (0/0 = 0)."""
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    return num / den if den else num


def oracle_prefill(w):
    """The fp64 oracle's (o, final state) for workload w, and its wall time."""
    import oracle
    t0 = time.perf_counter()
    if isinstance(w, kin.RawPrefill):
        q, k, v, z, bl, s0 = w.f64()
        q, k, g, b = oracle.prepare_inputs(q, k, z, bl, **w.options())
    else:
        q, k, v, g, b, s0 = w.f64()
    cu = None if w.cu_seqlens is None else w.cu_seqlens.astype(np.int64)
    o, s = oracle.recurrent(q, k, v, g, b, cu_seqlens=cu, num_seqs=w.num_seqs,
                            initial_state=s0)
    return o, s, time.perf_counter() - t0


def prefill_parity(w, res, ref=None):
    """Errors of this run's outputs against the oracle.  With the output
    epilogue the error is measured in the operator's units: each row's
    error times that row's RMS over max|o| max|w| (RMSNorm divides a row by
    its own RMS, which magnifies a normwise-bounded error on small rows)."""
    import oracle
    o_ref, s_ref, _ = ref if ref is not None else oracle_prefill(w)
    tol = 1e-4 if w.dtype == kin.F32 else 2e-2
    out = dict(max_relerr_state=normwise(res["final_state"], s_ref), tol=tol,
               reference="fp64 oracle (token-by-token recurrence), whole workload")
    if isinstance(w, kin.RawPrefill) and w.out_norm_weight is not None:
        y_ref = oracle.output_epilogue(o_ref, w.out_norm_weight, 1e-6,
                                       kin.as_f64(w.out_gate, w.dtype))
        rms = np.sqrt(np.mean(o_ref * o_ref, axis=-1, keepdims=True))
        out["max_relerr_o"] = float(np.max(np.abs(res["o"] - y_ref) * rms) /
                                    (np.max(np.abs(o_ref)) * np.max(np.abs(w.out_norm_weight))))
        out["o_measure"] = "epilogue error scaled by each row's RMS (operator units)"
    else:
        out["max_relerr_o"] = normwise(res["o"], o_ref)
    out["pass"] = bool(out["max_relerr_o"] <= tol and out["max_relerr_state"] <= tol)
    return out


def time_backward(torch, kda, w, steps, warmup, d, E, settle_ms=SETTLE_MS):
    """Times `steps` kda_bwd_chunked calls on workload w with d_o ~ N(0, 1)."""
    d_in = upload_prefill(torch, w)
    do, _ = kin.backward_inputs(7, w.total_tokens, w.num_heads, d, w.num_seqs, w.dtype)
    d_o = torch.from_numpy(np.ascontiguousarray(do).view(np.int16)).view(torch.bfloat16).cuda()
    call, grads = kda.bind_bwd(d_in["q"], d_in["k"], d_in["v"], d_in["log_alpha"],
                               d_in["beta"], d_o, cu_seqlens=d_in["cu_seqlens"],
                               num_seqs=d_in["num_seqs"], initial_state=d_in["initial_state"],
                               chunk_size=w.chunk_size)
    settle(torch, call, settle_ms)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    call()
    torch.cuda.synchronize()
    got = {k: v.detach().to(torch.float64).cpu().numpy() for k, v in grads.items()
           if v is not None}
    th = w.total_tokens * w.num_heads
    byts = th * backward_bytes_per_token_head(d, E) + w.num_seqs * w.num_heads * state_bytes(d)
    flops = th * backward_flops_per_token_head(d, w.chunk_size)
    sec = ms * 1e-3
    t_hbm, t_mma = byts / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12)
    hbm_bound = t_hbm >= t_mma
    ach = (byts / sec / 1e9) if hbm_bound else (flops / sec / 1e12)
    peak = HBM_PEAK_GBS if hbm_bound else BF16_PEAK_TFLOPS
    traffic = measured_traffic("backward", "bwd")  # the call's three or four kernels
    return dict(tokens_per_s=w.total_tokens / sec, ms_per_step=ms,
                algorithmic_bytes=byts, algorithmic_flops=flops,
                roofline_frac=max(t_hbm, t_mma) / sec,
                mfma_frac_bf16=flops / sec / 1e12 / BF16_PEAK_TFLOPS,
                roofline=dict(bound="hbm" if hbm_bound else "mfma", achieved=ach, peak=peak,
                              unit="GB/s" if hbm_bound else "TFLOP/s",
                              frac=max(t_hbm, t_mma) / sec, traffic=traffic,
                              traffic_over_algorithmic=None if traffic is None else traffic / byts,
                              scope="whole kda_bwd_chunked call (3 or 4 kernels); bytes: q, k, v, "
                                    "d_o, dq, dk, dv in bf16, g and dg in fp32, beta and dbeta; "
                                    "flops: the method's, triangles once, priced at the bf16 peak",
                              avg_call_us=ms * 1e3)), got, do


BWD_PARITY_HEADS = [0, 5]


def backward_parity(w, got, do):
    """Gradients of two heads (heads never interact, so the check of a head
    is exact) against the fp64 autograd oracle, which needs ~5 s per head
    for this workload."""
    import oracle
    q, k, v, g, b, s0 = w.f64()
    hs = BWD_PARITY_HEADS
    cu = None if w.cu_seqlens is None else w.cu_seqlens.astype(np.int64)
    ref = oracle.recurrent_backward(q[:, hs], k[:, hs], v[:, hs], g[:, hs], b[:, hs],
                                    kin.as_f64(do, w.dtype)[:, hs], cu_seqlens=cu,
                                    num_seqs=w.num_seqs,
                                    initial_state=None if s0 is None else s0[:, hs])
    errs = {k: normwise(got[k][:, hs], ref[k]) for k in ("dq", "dk", "dv", "dg", "dbeta")
            if k in got}
    tol = 1e-4 if w.dtype == kin.F32 else 2e-2
    out = dict(max_relerr=errs, tol=tol,
               reference=f"fp64 oracle (autograd of the token-by-token recurrence), heads {hs}")
    out["pass"] = all(e <= tol for e in errs.values())
    return out


# ---------------------------------------------------------------- decode

def build_decode_inputs(torch, cfg, n_steps, sample):
    """Device tensors for n_steps decode steps, generated on host threads in
    batches (seeded per step) and uploaded as they are made; also each
    step's inputs of the sampled (batch, head) states, as fp64 host arrays."""
    B, H, d = cfg["batch"], cfg["H"], cfg["d"]
    q = torch.empty((n_steps, B, H, d), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    g = torch.empty((n_steps, B, H, d), dtype=torch.float32, device="cuda")
    be = torch.empty((n_steps, B, H), dtype=torch.float32, device="cuda")
    sb, sh = sample
    host = [None] * n_steps

    def gen(s):
        return s, kin.decode_step(s, B, H, d, dtype=kin.BF16, g_mu=cfg["g_mu"],
                                  g_sigma=cfg["g_sigma"])

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)

    workers = min(16, len(os.sched_getaffinity(0)))
    batch = 4 * workers
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for s0 in range(0, n_steps, batch):
            for s, x in ex.map(gen, range(s0, min(n_steps, s0 + batch))):
                q[s].copy_(bf(x.q))
                k[s].copy_(bf(x.k))
                v[s].copy_(bf(x.v))
                g[s].copy_(torch.from_numpy(x.g))
                be[s].copy_(torch.from_numpy(x.beta))
                host[s] = tuple(a[sb, sh][:, None] for a in x.f64())
    return (q, k, v, g, be), host


def decode_sample(B, H, n=64):
    """n (batch, head) states spread over batch and heads."""
    return (np.array([(4 * i + i % 4) % B for i in range(n)]),
            np.array([(7 * i + 3) % H for i in range(n)]))


def time_decode(torch, kda, cfg, n_steps, warmup, settle_ms=SETTLE_MS):
    B, H, d = cfg["batch"], cfg["H"], cfg["d"]
    t = time.perf_counter()
    sample = decode_sample(B, H)
    (q, k, v, g, be), host = build_decode_inputs(torch, cfg, n_steps, sample)
    st0_h = kin.decode_states(B, H, d, s0_std=cfg["s0_std"])
    st0 = torch.from_numpy(st0_h).cuda()
    log(f"decode inputs ready ({time.perf_counter() - t:.1f} s)")
    state = st0.clone()
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    calls = [kda.bind_decode(q[s], k[s], v[s], g[s], be[s], state, out=o)[0]
             for s in range(n_steps)]
    nxt = [0]

    def one_step():  # the steps in turn; the state is reset below
        calls[nxt[0] % n_steps]()
        nxt[0] += 1
    settle(torch, one_step, settle_ms)
    for s in range(min(warmup, n_steps)):
        calls[s]()
    state.copy_(st0)
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    e0.record()
    for c in calls:
        c()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    # untimed pass from the same states: the sampled rows of every step's o
    state.copy_(st0)
    sb_d = torch.from_numpy(sample[0]).cuda()
    sh_d = torch.from_numpy(sample[1]).cuda()
    o_smp = torch.empty((n_steps, len(sample[0]), d), dtype=torch.bfloat16, device="cuda")
    for s, c in enumerate(calls):
        c()
        o_smp[s] = o[sb_d, sh_d]
    torch.cuda.synchronize()
    got = (o_smp.to(torch.float64).cpu().numpy(),
           state[sb_d, sh_d].to(torch.float64).cpu().numpy())
    st_smp = st0_h[sample[0], sample[1]][:, None].astype(np.float64)
    del q, k, v, g, be, calls, state, st0, o, o_smp
    step_us = 1e3 * ms / n_steps
    byts = B * H * decode_bytes_per_state(d, 2)
    ach = byts / (step_us * 1e-6) / 1e9
    roof_us = byts / (HBM_PEAK_GBS * 1e9) * 1e6
    rep = dict(steps=n_steps, steps_per_s=n_steps / (ms * 1e-3),
               tokens_per_s=B * n_steps / (ms * 1e-3), us_per_step=step_us,
               roofline_steps_per_s=1e6 / roof_us, roofline_frac=roof_us / step_us,
               roofline=dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=ach / HBM_PEAK_GBS,
                             traffic=measured_traffic("decode", "decode_kernel"),
                             kernel="decode_kernel", bytes_per_launch=byts,
                             avg_launch_us=step_us))
    return rep, got, host, st_smp


def decode_parity(got, host, st_smp):
    """Every step's o and the states after the last step, for the sampled
    states, against the oracle run on those states alone."""
    import oracle
    o_gpu, s_gpu = got
    ref = st_smp
    worst = 0.0
    for s, (q, k, v, g, b) in enumerate(host):
        o_ref, ref = oracle.decode(q, k, v, g, b, ref)
        worst = max(worst, normwise(o_gpu[s], o_ref[:, 0]))
    es = normwise(s_gpu, ref[:, 0])
    out = dict(max_relerr_o=worst, max_relerr_state=es, tol=2e-2,
               reference=f"fp64 oracle on {len(st_smp)} sampled states (spread over batch "
                         f"and heads), every one of {len(host)} steps")
    out["pass"] = bool(worst <= 2e-2 and es <= 2e-2)
    return out


# ---------------------------------------------------------------- CPU oracle

def _cpu_model():
    """The host CPU's model name (/proc/cpuinfo), for the baseline record."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_prefill(w, seconds, wname):
    """The fp64 oracle on whole passes of workload w, repeated until
    `seconds` of wall time have passed.  Returns (record, first pass's
    (o, S, time))."""
    first = oracle_prefill(w)
    import oracle
    reps, el = 1, first[2]
    while el < seconds:
        el += oracle_prefill(w)[2]
        reps += 1
    return dict(value=reps * w.total_tokens / el, unit="tokens/s",
                cores=oracle.num_threads(), cpu=_cpu_model(), kind="oracle",
                sample=f"{reps} whole passes of the {wname} prefill workload "
                       f"({w.total_tokens} tokens x {w.num_heads} heads), fp64, {el:.1f} s"), first


def cpu_baseline_decode(cfg, seconds):
    import oracle
    B, H, d = cfg["batch"], cfg["H"], cfg["d"]
    st = kin.decode_states(B, H, d, s0_std=cfg["s0_std"]).astype(np.float64)
    n, spent = 0, 0.0
    while spent < seconds:
        x = kin.decode_step(n, B, H, d, dtype=kin.BF16, g_mu=cfg["g_mu"],
                            g_sigma=cfg["g_sigma"]).f64()
        t0 = time.perf_counter()
        _, st = oracle.decode(*x, st)
        spent += time.perf_counter() - t0
        n += 1
    return dict(value=n / spent, unit="steps/s", cores=oracle.num_threads(), cpu=_cpu_model(),
                kind="oracle",
                sample=f"{n} dependent decode steps of the full batch ({B} x {H} states), "
                       f"fp64, {spent:.1f} s (input generation excluded)")


# ---------------------------------------------------------------- copy

COPY_BYTES = 1 << 30


def copy_calibration(torch, steps, warmup):
    """A plain device copy of COPY_BYTES (read once, written once, negated): what the
    memory-traffic counters read for it scales their readings on the
    kernels."""
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    # an elementwise kernel (a same-type copy_ may go to a DMA engine)
    for _ in range(warmup):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    e0, e1 = _events(torch, 2)
    e0.record()
    for _ in range(steps):
        torch.neg(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    log(f"copy {COPY_BYTES} B: {ms * 1e3:.1f} us, {2 * COPY_BYTES / ms / 1e6:.0f} GB/s "
        f"(read + write)")
    print(json.dumps({"metric": "device copy (read + write) GB/s, counter calibration",
                      "value": 2 * COPY_BYTES / ms / 1e6, "unit": "GB/s", "n_gpus": 1,
                      "steps": steps, "warmup": warmup, "ms_per_step": ms,
                      "higher_is_better": True, "copy_bytes": COPY_BYTES}), flush=True)


# ---------------------------------------------------------------- main

PREFILL = {  # bench name -> (workload index or raw form, label)
    "long": (2, "long-context prefill B=1 H=32 T=32768"),
    "prefill": (1, "prefill B=2 H=8 T=2048"),
    "varlen": (3, "varlen prefill 16 x U[512,8192] tokens, H=16, initial states"),
    "raw": ("raw", "prefill B=2 H=8 T=2048 in model-boundary form (softplus gate, q/k L2 "
                   "norm, beta logits, RMSNorm + output gate, all in the kernels)"),
}
REPORT_NAME = {"raw": "prefill_fused", "bwd": "backward"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed whole calls for this many ms before each workload's "
                         "warmup steps, so that the GPU clocks have settled under load")
    ap.add_argument("--extra", default="prefill,varlen,raw,bwd,decode",
                    help="comma list of workloads besides the headline (prefill, varlen, raw, "
                         "bwd, decode) or 'none'")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU oracle baseline and the oracle parity checks")
    ap.add_argument("--only", choices=["prefill", "long", "varlen", "raw", "bwd", "decode",
                                       "copy"],
                    help="run one workload only (profiling runs); its throughput is `value`. "
                         "'copy' times a plain 1 GiB device copy, the reference for the "
                         "memory-traffic counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: the operator runs on one GPU only; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported", file=sys.stderr)
        sys.exit(2)
    if args.only is not None:
        todo = [args.only]
    else:
        todo = ["long"] + ([] if args.extra in ("", "none") else args.extra.split(","))

    import torch
    import gated_delta_rule_chunked_amd as kda
    if not torch.cuda.is_available():
        print("bench.py: no ROCm GPU visible", file=sys.stderr)
        sys.exit(1)
    kda.library()  # fail loudly if the HIP library is missing
    if args.only == "copy":
        copy_calibration(torch, args.steps, args.warmup)
        return

    d, C, E = 128, 64, 2
    workloads, parity = {}, {}
    cpu = None
    for name in todo:
        if name in PREFILL:
            idx, label = PREFILL[name]
            rname = REPORT_NAME.get(name, name)
            log(f"{label}: generating inputs")
            w = kin.raw_prefill_workload() if idx == "raw" else kin.workload(idx)
            steps = args.steps if name in ("long", "prefill", "raw") else min(args.steps, 20)
            log(f"  {args.warmup} warmup + {steps} timed calls")
            r = time_prefill(torch, kda, w, steps, args.warmup, settle_ms=args.settle_ms)
            rep = prefill_report(w, r, d, E, C)
            rep["roofline"] = call_roofline(rname, w, r, d, E, C)
            if name == "varlen":
                rep["total_tokens"] = w.total_tokens
            log(f"  {rep['tokens_per_s'] / 1e6:.2f} M tokens/s, {rep['ms_per_step'] * 1e3:.1f} "
                f"us/call, frac {rep['roofline_frac']:.3f}, kernels(us) "
                f"{json.dumps({k: round(v, 2) for k, v in r['kernel_us'].items()})}")
            if not args.no_cpu:
                ref = None
                if name == "long" and args.only is None:
                    log(f"  CPU oracle baseline on the whole workload (~{args.cpu_seconds:.0f} s)")
                    cpu, ref = cpu_baseline_prefill(w, args.cpu_seconds, "long-context")
                parity[rname] = prefill_parity(w, r, ref)
                log(f"  parity: o {parity[rname]['max_relerr_o']:.3e}, "
                    f"S {parity[rname]['max_relerr_state']:.3e}")
            workloads[rname] = rep
            del w, r
        elif name == "bwd":
            log("backward of the B=2 H=8 T=2048 prefill")
            w = kin.workload(1)
            rep, got, do = time_backward(torch, kda, w, min(args.steps, 20),
                                         min(args.warmup, 3), d, E, settle_ms=args.settle_ms)
            workloads["backward"] = rep
            if not args.no_cpu:
                parity["backward"] = backward_parity(w, got, do)
            log(f"  {rep['tokens_per_s'] / 1e6:.2f} M tokens/s, {rep['ms_per_step'] * 1e3:.1f} "
                f"us/call")
            del w, got
        elif name == "decode":
            cfg4 = kin.WORKLOADS[4]
            log(f"decode batch 256 H=32: {args.decode_steps} steps")
            rep, got, host, st_smp = time_decode(torch, kda, cfg4, args.decode_steps,
                                                 min(args.warmup, 50), settle_ms=args.settle_ms)
            workloads["decode"] = rep
            log(f"  {rep['steps_per_s']:.0f} steps/s, {rep['roofline']['achieved']:.0f} GB/s")
            if not args.no_cpu:
                parity["decode"] = decode_parity(got, host, st_smp)
                log(f"  parity: o {parity['decode']['max_relerr_o']:.3e}, "
                    f"S {parity['decode']['max_relerr_state']:.3e}")
                if args.only is None:
                    rep["cpu_baseline"] = cpu_baseline_decode(cfg4, max(2.0, args.cpu_seconds / 2))
            del got, host
        else:
            raise SystemExit(f"unknown workload {name!r}")
        torch.cuda.empty_cache()

    head_name = REPORT_NAME.get(todo[0], todo[0])
    head = workloads[head_name]
    if head_name == "decode":
        value, unit, ms = head["steps_per_s"], "steps/s", head["us_per_step"] * 1e-3
    else:
        value, unit, ms = head["tokens_per_s"], "tokens/s", head["ms_per_step"]
    configs = {
        "long": {"workload": "KDA long-context chunked prefill B=1 H=32 T=32768 d_k=d_v=128 "
                             "chunk=64, bf16 q/k/v, fp32 log-decay/beta/state, S_0=0",
                 "global_batch": 1, "seq_len": 32768, "heads": 32, "head_dim": 128,
                 "chunk": 64},
        "prefill": {"workload": "KDA chunked prefill B=2 H=8 T=2048 d_k=d_v=128 chunk=64, "
                                "bf16 q/k/v, fp32 state, S_0=0",
                    "global_batch": 2, "seq_len": 2048, "heads": 8, "head_dim": 128,
                    "chunk": 64},
    }
    cfg = dict(configs.get(head_name, {"workload": head_name}))
    cfg["parallelism"] = "single GPU"
    line = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64; q,k L2-normalised, v~N(0,1), "
                "beta=sigmoid(N(0,1)), log-alpha=-exp(N(mu,sigma)) per channel)",
        "config": cfg,
        "roofline": head.get("roofline"),
        "cpu_baseline": cpu,
        "parity": parity,
        "workloads": workloads,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
