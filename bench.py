#!/usr/bin/env python3
"""Throughput of the KDA operator (libkda.so) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--extra long,varlen,decode]

Headline: chunked prefill, B=2 sequences x T=2048 tokens, H=8 heads,
d_k=d_v=128, chunk 64, bf16 q/k/v, fp32 log-decay/beta/state, zero initial
state.  One step = one kda_fwd_chunked call (intra-chunk kernel:
cumulative log-decay + UT/WY factors -> inter-chunk state pass) over that
batch; `value` is
prefill tokens/s over K timed steps with every input resident in HBM.

Also reported on the same JSON line:
  roofline      the dominant prefill kernel's algorithmic HBM bytes per launch
                over its average launch time (HIP events on the launch stream)
  cpu_baseline  the fp64 CPU oracle (test infrastructure) timed on the host
                cores on repeated whole copies of the headline batch
  workloads     long-context prefill (B=1, H=32, T=32768), varlen packed
                prefill (16 seqs of U[512, 8192] tokens, H=16, initial
                states), the headline prefill in model-boundary form (input-side
                fusion: softplus gate from bf16 z, q/k L2-normalised, beta
                from logits; output epilogue: per-head RMSNorm and sigmoid
                output gate), the backward of the headline prefill (training:
                dq, dk, dv, dg, dbeta from d_o) and recurrent decode (batch 256,
                H=32, 1000 steps) -- each with throughput, fraction of its
                roofline and, for decode, the decode kernel's achieved HBM GB/s.
Inputs come from gated_delta_rule_chunked_amd.inputs (seeded, synthetic).
Only one GPU is supported: --gpus above 1 exits with an error.

`roofline.traffic` is the dominant kernel's HBM bytes per launch as read by
the FETCH_SIZE and WRITE_SIZE counters (profiles/hbm_traffic_counters.md,
scaled by what the same counters read for a plain device copy of known
size, `--only copy`).  It is null when that file holds no reading for the
kernel or when the kernel's sources have changed since the reading.
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
    """Matrix-core work of kda_bwd_chunked as computed (triangular blocks in
    full), per token-head: per tile of C tokens the recompute (M, P, W, U:
    4 C^2 d; T: C^3 / 6), the two state chains (2 C d^2 and C^2 d + 3 C d^2)
    and the per-tile gradients (4 C d^2 + 9 C^2 d + 2 C^3), 2 flops a
    multiply-add."""
    macs = 9 * C * d * d + 14 * C * C * d + (2 + 1 / 6) * C ** 3
    return 2 * macs / C


def backward_bytes_per_token_head(d, E):
    """Read q, k, v, d_o (operand type), log-decay (fp32), beta; write dq, dk,
    dv (operand type), dg (fp32), dbeta."""
    return 4 * E * d + 4 * d + 4 + 3 * E * d + 4 * d + 4


# ---------------------------------------------------------------- counters

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
CSRC = os.path.join(ROOT, "gated_delta_rule_chunked_amd", "csrc")
KERNEL_SOURCES = {"intra": ("kda_intra.hip",), "inter": ("kda_inter.hip", "kda_epilogue.hip"),
                  "decode_kernel": ("kda_decode.hip",)}


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
    if stage == "intra":      # read q, k, v, g (or z), beta; write Qt, W, U, Ke, P, e^G_n
        gate = E * d if raw else 4 * d
        return token_heads * (3 * E * d + gate + 4 + 4 * E * d + E * CK + 4 * d / C)
    if stage == "inter":      # read Qt, W, U, Ke, P, e^G_n; write o; states
        epi = 3 * E * d if epilogue else 0  # epilogue pass: read o, z_o; write o
        # P is lower triangular: with C = 64 the token K-step 32..63 of token
        # blocks 0 and 1 is zero and not read (a quarter of P)
        p_read = E * CK * (0.75 if C == 64 else 1.0)
        return (token_heads * (4 * E * d + p_read + E * d + 4 * d / C + epi) +
                pairs * state_bytes(d) * (2 if with_s0 else 1))
    raise ValueError(stage)


def decode_bytes_per_state(d, E):
    """State read + write (fp32), q, k, v, o, log-decay, beta."""
    return 2 * state_bytes(d) + 4 * E * d + 4 * d + 4


# ---------------------------------------------------------------- helpers

def _events(torch, n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


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


def time_prefill(torch, kda, w, steps, warmup, per_kernel=True):
    """Times `steps` whole prefill calls, then each kernel separately."""
    raw = isinstance(w, kin.RawPrefill)
    d_in = upload_prefill_raw(torch, w) if raw else upload_prefill(torch, w)
    call, stages, o, fs = kda.bind_fwd(
        d_in["q"], d_in["k"], d_in["v"], d_in["log_alpha"], d_in["beta"],
        cu_seqlens=d_in["cu_seqlens"], num_seqs=d_in["num_seqs"],
        initial_state=d_in["initial_state"], chunk_size=w.chunk_size,
        **d_in.get("options", {}))
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
    res = dict(ms_per_step=ms, wall_ms_per_step=1e3 * t_wall / steps)
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
    return res


def prefill_report(w, res, d, E, C):
    T = w.total_tokens
    H = w.num_heads
    th = T * H
    s0 = w.initial_state is not None
    raw = isinstance(w, kin.RawPrefill)
    epi = raw and w.out_norm_weight is not None
    byts = th * prefill_bytes_per_token_head(d, E, raw, epi) + w.num_seqs * H * state_bytes(
        d) * (2 if s0 else 1)
    flops = th * prefill_flops_per_token_head(d, C)
    t_roof = max(byts / (HBM_PEAK_GBS * 1e9), flops / (BF16_PEAK_TFLOPS * 1e12))
    sec = res["ms_per_step"] * 1e-3
    out = dict(tokens_per_s=T / sec, ms_per_step=res["ms_per_step"],
               roofline_tokens_per_s=T / t_roof, roofline_frac=t_roof / sec,
               algorithmic_bytes=byts, algorithmic_flops=flops,
               achieved_gbs=byts / sec / 1e9,
               mfma_frac_algorithmic=flops / sec / (BF16_PEAK_TFLOPS * 1e12))
    if "kernel_us" in res:
        out["kernel_us"] = res["kernel_us"]
    return out


def dominant_roofline(wname, w, res, d, E, C):
    ku = res["kernel_us"]
    name = max(ku, key=ku.get)
    th = w.total_tokens * w.num_heads
    raw = isinstance(w, kin.RawPrefill)
    b = kernel_bytes(name, th, w.num_seqs * w.num_heads, d, E, C,
                     w.initial_state is not None, raw=raw,
                     epilogue=raw and w.out_norm_weight is not None)
    ach = b / (ku[name] * 1e-6) / 1e9
    return dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s",
                frac=ach / HBM_PEAK_GBS, traffic=measured_traffic(wname, name), kernel=name,
                bytes_per_launch=b, avg_launch_us=ku[name])


def time_backward(torch, kda, w, steps, warmup, d, E):
    """Times `steps` kda_bwd_chunked calls on workload w with d_o ~ N(0, 1)."""
    d_in = upload_prefill(torch, w)
    do, _ = kin.backward_inputs(7, w.total_tokens, w.num_heads, d, w.num_seqs, w.dtype)
    d_o = torch.from_numpy(np.ascontiguousarray(do).view(np.int16)).view(torch.bfloat16).cuda()
    call, _ = kda.bind_bwd(d_in["q"], d_in["k"], d_in["v"], d_in["log_alpha"], d_in["beta"],
                           d_o, cu_seqlens=d_in["cu_seqlens"], num_seqs=d_in["num_seqs"],
                           initial_state=d_in["initial_state"], chunk_size=w.chunk_size)
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
    th = w.total_tokens * w.num_heads
    byts = th * backward_bytes_per_token_head(d, E) + w.num_seqs * w.num_heads * state_bytes(d)
    flops = th * backward_flops_per_token_head(d, w.chunk_size)
    tf = flops / (ms * 1e-3) / 1e12
    return dict(tokens_per_s=w.total_tokens / (ms * 1e-3), ms_per_step=ms,
                algorithmic_bytes=byts, algorithmic_flops=flops,
                hbm_frac=byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                roofline_frac=tf / FP32_MFMA_PEAK_TFLOPS,
                roofline=dict(bound="mfma", achieved=tf, peak=FP32_MFMA_PEAK_TFLOPS,
                              unit="TFLOP/s", frac=tf / FP32_MFMA_PEAK_TFLOPS, traffic=None,
                              kernel="kda_bwd_chunked (3 or 4 kernels, fp32 and bf16 matrix cores; "
                                     "priced at the fp32 peak)",
                              flops_per_launch=flops, avg_launch_us=ms * 1e3))


# ---------------------------------------------------------------- decode

def build_decode_inputs(torch, cfg, n_steps):
    """Device tensors for n_steps decode steps, generated on host threads in
    batches (seeded per step) and uploaded as they are made."""
    B, H, d = cfg["batch"], cfg["H"], cfg["d"]
    q = torch.empty((n_steps, B, H, d), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty_like(q)
    g = torch.empty((n_steps, B, H, d), dtype=torch.float32, device="cuda")
    be = torch.empty((n_steps, B, H), dtype=torch.float32, device="cuda")

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
    return q, k, v, g, be


def time_decode(torch, kda, cfg, n_steps, warmup):
    B, H, d = cfg["batch"], cfg["H"], cfg["d"]
    t = time.perf_counter()
    q, k, v, g, be = build_decode_inputs(torch, cfg, n_steps)
    st0 = torch.from_numpy(kin.decode_states(B, H, d, s0_std=cfg["s0_std"])).cuda()
    log(f"decode inputs ready ({time.perf_counter() - t:.1f} s)")
    state = st0.clone()
    o = torch.empty((B, H, d), dtype=torch.bfloat16, device="cuda")
    calls = [kda.bind_decode(q[s], k[s], v[s], g[s], be[s], state, out=o)[0]
             for s in range(n_steps)]
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
    step_us = 1e3 * ms / n_steps
    byts = B * H * decode_bytes_per_state(d, 2)
    ach = byts / (step_us * 1e-6) / 1e9
    roof_us = byts / (HBM_PEAK_GBS * 1e9) * 1e6
    return dict(steps=n_steps, steps_per_s=n_steps / (ms * 1e-3),
                tokens_per_s=B * n_steps / (ms * 1e-3), us_per_step=step_us,
                roofline_steps_per_s=1e6 / roof_us, roofline_frac=roof_us / step_us,
                roofline=dict(bound="hbm", achieved=ach, peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=ach / HBM_PEAK_GBS,
                              traffic=measured_traffic("decode", "decode_kernel"),
                              kernel="decode_kernel", bytes_per_launch=byts,
                              avg_launch_us=step_us))


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


def cpu_baseline_prefill(w, seconds):
    """The fp64 oracle on whole copies of the headline batch, repeated until
    `seconds` of wall time have passed."""
    import oracle
    q, k, v, g, b, s0 = w.f64()
    cu = None if w.cu_seqlens is None else w.cu_seqlens.astype(np.int64)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.recurrent(q, k, v, g, b, cu_seqlens=cu, num_seqs=w.num_seqs,
                         initial_state=s0)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return dict(value=reps * w.total_tokens / el, unit="tokens/s",
                cores=oracle.num_threads(), cpu=_cpu_model(), kind="oracle",
                sample=f"{reps} whole passes of the headline prefill batch "
                       f"({w.total_tokens} tokens x {w.num_heads} heads), fp64, {el:.1f} s")


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

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--extra", default="long,varlen,raw,bwd,decode",
                    help="comma list of extra workloads (long, varlen, raw, bwd, decode) or "
                         "'none'")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
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
    extra = [] if args.extra in ("", "none") else args.extra.split(",")
    if args.only is not None:
        extra = [] if args.only == "prefill" else [args.only]

    import torch
    import gated_delta_rule_chunked_amd as kda
    if not torch.cuda.is_available():
        print("bench.py: no ROCm GPU visible", file=sys.stderr)
        sys.exit(1)
    kda.library()  # fail loudly if the HIP library is missing
    if args.only == "copy":
        copy_calibration(torch, args.steps, args.warmup)
        return

    # headline: chunked prefill B=2, H=8, T=2048
    cfg1 = kin.WORKLOADS[1]
    w1 = kin.workload(1)
    d, C, E = cfg1["d"], cfg1["chunk_size"], 2
    workloads = {}
    roof = None
    if args.only in (None, "prefill"):
        log(f"prefill B=2 H=8 T=2048: {args.warmup} warmup + {args.steps} timed steps")
        r1 = time_prefill(torch, kda, w1, args.steps, args.warmup)
        workloads["prefill"] = prefill_report(w1, r1, d, E, C)
        roof = dominant_roofline("prefill", w1, r1, d, E, C)
        log(f"  {workloads['prefill']['tokens_per_s'] / 1e6:.2f} M tokens/s, "
            f"{workloads['prefill']['ms_per_step'] * 1e3:.1f} us/step, kernels(us) "
            f"{json.dumps({k: round(v, 2) for k, v in r1['kernel_us'].items()})}")
    if "long" in extra:
        log("long prefill B=1 H=32 T=32768: generating inputs")
        w2 = kin.workload(2)
        r2 = time_prefill(torch, kda, w2, min(args.steps, 20), min(args.warmup, 3))
        workloads["long"] = prefill_report(w2, r2, d, E, C)
        workloads["long"]["roofline"] = dominant_roofline("long", w2, r2, d, E, C)
        log(f"  {workloads['long']['tokens_per_s'] / 1e6:.2f} M tokens/s, "
            f"frac {workloads['long']['roofline_frac']:.3f}, kernels(us) "
            f"{json.dumps({k: round(v, 2) for k, v in r2['kernel_us'].items()})}")
        del w2
    if "varlen" in extra:
        log("varlen prefill 16 x U[512,8192], H=16: generating inputs")
        w3 = kin.workload(3)
        r3 = time_prefill(torch, kda, w3, min(args.steps, 20), min(args.warmup, 3))
        workloads["varlen"] = prefill_report(w3, r3, d, E, C)
        workloads["varlen"]["roofline"] = dominant_roofline("varlen", w3, r3, d, E, C)
        workloads["varlen"]["total_tokens"] = w3.total_tokens
        log(f"  {workloads['varlen']['tokens_per_s'] / 1e6:.2f} M tokens/s, "
            f"frac {workloads['varlen']['roofline_frac']:.3f}, kernels(us) "
            f"{json.dumps({k: round(v, 2) for k, v in r3['kernel_us'].items()})}")
        del w3
    if "raw" in extra:
        log("prefill in model-boundary form (softplus gate, q/k L2 norm, beta logits, "
            "RMSNorm + output gate, all in the kernels)")
        w5 = kin.raw_prefill_workload()
        r5 = time_prefill(torch, kda, w5, args.steps, args.warmup)
        workloads["prefill_fused"] = prefill_report(w5, r5, d, E, C)
        workloads["prefill_fused"]["roofline"] = dominant_roofline("prefill_fused", w5, r5, d,
                                                                   E, C)
        log(f"  {workloads['prefill_fused']['tokens_per_s'] / 1e6:.2f} M tokens/s, "
            f"{workloads['prefill_fused']['ms_per_step'] * 1e3:.1f} us/step, kernels(us) "
            f"{json.dumps({k: round(v, 2) for k, v in r5['kernel_us'].items()})}")
        del w5
    if "bwd" in extra:
        log("backward of the headline prefill (B=2 H=8 T=2048)")
        workloads["backward"] = time_backward(torch, kda, w1, min(args.steps, 20),
                                              min(args.warmup, 3), d, E)
        log(f"  {workloads['backward']['tokens_per_s'] / 1e6:.2f} M tokens/s, "
            f"{workloads['backward']['ms_per_step'] * 1e3:.1f} us/step")
    torch.cuda.empty_cache()
    if "decode" in extra:
        cfg4 = kin.WORKLOADS[4]
        log(f"decode batch 256 H=32: {args.decode_steps} steps")
        workloads["decode"] = time_decode(torch, kda, cfg4, args.decode_steps,
                                          min(args.warmup, 50))
        log(f"  {workloads['decode']['steps_per_s']:.0f} steps/s, "
            f"{workloads['decode']['roofline']['achieved']:.0f} GB/s")
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu and "prefill" in workloads:
        log(f"CPU oracle baseline (~{args.cpu_seconds:.0f} s)")
        cpu = cpu_baseline_prefill(w1, args.cpu_seconds)
        if "decode" in workloads:
            workloads["decode"]["cpu_baseline"] = cpu_baseline_decode(
                kin.WORKLOADS[4], max(2.0, args.cpu_seconds / 2))

    if "prefill" in workloads:
        head = workloads["prefill"]
        value, unit, ms = head["tokens_per_s"], "tokens/s", head["ms_per_step"]
    else:  # a single extra workload (profiling runs)
        name = {"raw": "prefill_fused", "bwd": "backward"}.get(args.only, args.only)
        head = workloads[name]
        roof = head["roofline"]
        if name == "decode":
            value, unit, ms = head["steps_per_s"], "steps/s", head["us_per_step"] * 1e-3
        elif name == "backward":
            value, unit, ms = head["tokens_per_s"], "tokens/s", head["ms_per_step"]
        else:
            value, unit, ms = head["tokens_per_s"], "tokens/s", head["ms_per_step"]
    line = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded numpy PCG64; q,k L2-normalised, v~N(0,1), "
                "beta=sigmoid(N(0,1)), log-alpha=-exp(N(-2,0.5)))",
        "config": {"workload": "KDA chunked prefill B=2 H=8 T=2048 d_k=d_v=128 chunk=64 "
                               "bf16 q/k/v, fp32 state, S_0=0",
                   "global_batch": 2, "seq_len": 2048, "heads": 8, "head_dim": 128,
                   "chunk": 64, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "workloads": workloads,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
