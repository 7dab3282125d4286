"""Seeded synthetic inputs for the KDA operator (shared by tests and bench).

This module only draws random numbers and prepares them the way the layer
above the operator would (L2-normalised q and k, beta from a sigmoid, a
negative log-decay); it holds none of the operator's arithmetic.  It imports
neither the HIP binding nor the oracle, so both sides can use it.

Recipe (one numpy PCG64 generator per workload, fp64 draws in this order):
  1. sequence lengths (varlen workloads only), integers uniform in [lo, hi];
  2. q, k ~ N(0, 1) [T, H, d], each token/head vector divided by its L2 norm;
  3. v ~ N(0, 1);
  4. beta = sigmoid(z), z ~ N(0, 1)                [T, H];
  5. g = log(alpha) = -exp(y), y ~ N(mu, sigma)     [T, H, d]  (per channel);
  6. initial states ~ N(0, s0_std) [N, H, d, d] when requested.
N(a, b) means mean a and standard deviation b.  q, k and v are rounded to the
operand dtype (bf16 by round-to-nearest-even on the fp32 bits, or fp32);
g, beta and states are fp32.  The arrays returned are exactly what the device
receives, and `as_f64` expands them exactly for the fp64 oracle.

Workloads (sizes from the operator's benchmark configurations):
  tiny     B=1,  H=1,  T=64,    d=32,  C=16, fp32, g: y ~ N(-2, 0.5)
  prefill  B=2,  H=8,  T=2048,  d=128, C=64, bf16, g: y ~ N(-2, 0.5)
  long     B=1,  H=32, T=32768, d=128, C=64, bf16, g: y ~ N(-4, 1)
  varlen   16 sequences of U[512, 8192] tokens, H=16, d=128, C=64, bf16,
           initial states ~ N(0, 0.02)
  decode   batch 256, H=32, d=128, fp32 states ~ N(0, 0.02), 1000 steps;
           step s draws q, k, v, beta, g from default_rng([4, s]).
The seed of workload i is i.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact expansion of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of an operand array as the device sees it."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _round_operand(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return f32_to_bf16_bits(x32) if dtype == BF16 else x32


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


@dataclasses.dataclass
class Prefill:
    """One prefill workload as device-ready host arrays."""
    q: np.ndarray                   # [T, H, d]  uint16 (bf16 bits) or float32
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray                   # [T, H, d]  float32, log(alpha) <= 0
    beta: np.ndarray                # [T, H]     float32
    cu_seqlens: Optional[np.ndarray]  # [N+1] int32, or None (equal lengths)
    num_seqs: int
    initial_state: Optional[np.ndarray]  # [N, H, d, d] float32 or None
    dtype: str
    chunk_size: int

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[2])

    def f64(self):
        """(q, k, v, g, beta, initial_state) expanded to float64 for the oracle."""
        s0 = None if self.initial_state is None else self.initial_state.astype(np.float64)
        return (as_f64(self.q, self.dtype), as_f64(self.k, self.dtype),
                as_f64(self.v, self.dtype), self.g.astype(np.float64),
                self.beta.astype(np.float64), s0)

    def seq_bounds(self):
        """List of (start, end) token ranges, one per sequence."""
        if self.cu_seqlens is not None:
            c = [int(x) for x in self.cu_seqlens]
            return list(zip(c[:-1], c[1:]))
        L = self.total_tokens // self.num_seqs
        return [(i * L, (i + 1) * L) for i in range(self.num_seqs)]


def make_prefill(seed, *, H: int, d: int, dtype: str, chunk_size: int,
                 B: int = 1, T: int = 0, lengths=None, len_range=None,
                 g_mu: float = -2.0, g_sigma: float = 0.5,
                 s0_std: Optional[float] = None, varlen: bool = False) -> Prefill:
    """Draw one prefill workload.

    Sequence layout: either B sequences of T tokens each (passed with
    cu_seqlens=None unless `varlen`), explicit `lengths`, or `len_range`
    (lo, hi) integer-uniform lengths for B sequences drawn first.
    """
    rng = np.random.default_rng(seed)
    if len_range is not None:
        lo, hi = len_range
        lengths = rng.integers(lo, hi, size=B, endpoint=True)
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        n = len(lengths)
    else:
        n = B
        cu = None
        if varlen:
            cu = (np.arange(B + 1) * T).astype(np.int32)
    total = int(cu[-1]) if cu is not None else B * T
    q = _unit_rows(rng.standard_normal((total, H, d)))
    k = _unit_rows(rng.standard_normal((total, H, d)))
    v = rng.standard_normal((total, H, d))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((total, H))))
    g = -np.exp(rng.normal(g_mu, g_sigma, size=(total, H, d)))
    s0 = None
    if s0_std is not None:
        s0 = rng.normal(0.0, s0_std, size=(n, H, d, d)).astype(np.float32)
    return Prefill(q=_round_operand(q, dtype), k=_round_operand(k, dtype),
                   v=_round_operand(v, dtype), g=g.astype(np.float32),
                   beta=beta.astype(np.float32), cu_seqlens=cu, num_seqs=n,
                   initial_state=s0, dtype=dtype, chunk_size=chunk_size)


# The five benchmark workloads, by index (seed = index).
WORKLOADS = {
    0: dict(name="tiny", kind="prefill", B=1, H=1, T=64, d=32, chunk_size=16,
            dtype=F32, g_mu=-2.0, g_sigma=0.5),
    1: dict(name="prefill", kind="prefill", B=2, H=8, T=2048, d=128,
            chunk_size=64, dtype=BF16, g_mu=-2.0, g_sigma=0.5),
    2: dict(name="long", kind="prefill", B=1, H=32, T=32768, d=128,
            chunk_size=64, dtype=BF16, g_mu=-4.0, g_sigma=1.0),
    3: dict(name="varlen", kind="prefill", B=16, len_range=(512, 8192), H=16,
            d=128, chunk_size=64, dtype=BF16, g_mu=-2.0, g_sigma=0.5,
            s0_std=0.02),
    4: dict(name="decode", kind="decode", batch=256, H=32, d=128, steps=1000,
            dtype=BF16, g_mu=-2.0, g_sigma=0.5, s0_std=0.02),
}


def workload(i: int) -> Prefill:
    """Prefill workload i (0..3) with seed i."""
    w = dict(WORKLOADS[i])
    if w.pop("kind") != "prefill":
        raise ValueError(f"workload {i} is not a prefill workload")
    w.pop("name")
    return make_prefill(i, **w)


def prefill_tokens(i: int) -> int:
    """Token count of prefill workload i (draws only the lengths)."""
    w = WORKLOADS[i]
    if "len_range" in w:
        rng = np.random.default_rng(i)
        lo, hi = w["len_range"]
        return int(rng.integers(lo, hi, size=w["B"], endpoint=True).sum())
    return w["B"] * w["T"]


@dataclasses.dataclass
class DecodeStep:
    q: np.ndarray      # [B, H, d] bf16 bits / float32
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray      # [B, H, d] float32
    beta: np.ndarray   # [B, H] float32
    dtype: str

    def f64(self):
        return (as_f64(self.q, self.dtype), as_f64(self.k, self.dtype),
                as_f64(self.v, self.dtype), self.g.astype(np.float64),
                self.beta.astype(np.float64))


def decode_states(batch: int = 256, H: int = 32, d: int = 128,
                  s0_std: float = 0.02, seed=4) -> np.ndarray:
    """Initial decode states ~ N(0, s0_std), float32 [batch, H, d, d]."""
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, s0_std, size=(batch, H, d, d)).astype(np.float32)


def decode_step(step: int, batch: int = 256, H: int = 32, d: int = 128,
                dtype: str = BF16, g_mu: float = -2.0, g_sigma: float = 0.5,
                seed_base: int = 4) -> DecodeStep:
    """Inputs of decode step `step`, drawn from default_rng([seed_base, step])."""
    rng = np.random.default_rng([seed_base, step])
    q = _unit_rows(rng.standard_normal((batch, H, d)))
    k = _unit_rows(rng.standard_normal((batch, H, d)))
    v = rng.standard_normal((batch, H, d))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((batch, H))))
    g = -np.exp(rng.normal(g_mu, g_sigma, size=(batch, H, d)))
    return DecodeStep(q=_round_operand(q, dtype), k=_round_operand(k, dtype),
                      v=_round_operand(v, dtype), g=g.astype(np.float32),
                      beta=beta.astype(np.float32), dtype=dtype)


# ---- raw inputs for the input-side fusion (kda_options) ----------------------
# Recipe (numpy PCG64, seed given, fp64 draws in this order):
#   1. q, k ~ N(0, 1) [T, H, d], not normalised (norms about sqrt(d));
#   2. v ~ N(0, 1);
#   3. beta logits ~ N(0, 1) [T, H];
#   4. gate input z ~ N(z_mu, 1) [T, H, d];
#   5. softplus gate: A[h] = log(u), u ~ U(0.05, 0.3) [H]; sigmoid gate:
#      g_min = -5 (Kimi K3's bound).
# q, k, v and z are rounded to the operand dtype; A and the beta logits are
# fp32.  With z_mu = 0 (softplus) the decays are -exp(A) softplus(z), about
# -0.03 .. -0.25 per token, and with z_mu = -3 (sigmoid) about -0.25: chunk
# sums of 64 tokens stay far above -80.

GATE_Z_MU = {"softplus": 0.0, "sigmoid": -3.0}


@dataclasses.dataclass
class RawPrefill:
    """A prefill workload in the form the layers before the operator
    produce it (raw q/k, gate input z, beta logits)."""
    q: np.ndarray          # [T, H, d] operand dtype, not normalised
    k: np.ndarray
    v: np.ndarray
    z: np.ndarray          # [T, H, d] operand dtype, gate input
    beta_logits: np.ndarray  # [T, H] float32
    gate: str              # "softplus" or "sigmoid"
    gate_A: Optional[np.ndarray]  # [H] float32 (softplus)
    gate_min: float
    cu_seqlens: Optional[np.ndarray]
    num_seqs: int
    initial_state: Optional[np.ndarray]
    dtype: str
    chunk_size: int
    out_norm_weight: Optional[np.ndarray] = None  # [d] float32: output epilogue
    out_gate: Optional[np.ndarray] = None         # [T, H, d] operand dtype

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])

    def options(self) -> dict:
        """The fusion options, as keyword arguments of the binding's calls
        and of the oracle's prepare_inputs (gate_A as a host array)."""
        return dict(gate=self.gate, gate_A=self.gate_A, gate_min=self.gate_min,
                    l2norm_qk=True, beta_logits=True)

    def f64(self):
        """(q, k, v, z, beta_logits, initial_state), exact float64."""
        s0 = None if self.initial_state is None else self.initial_state.astype(np.float64)
        return (as_f64(self.q, self.dtype), as_f64(self.k, self.dtype),
                as_f64(self.v, self.dtype), as_f64(self.z, self.dtype),
                self.beta_logits.astype(np.float64), s0)


def make_prefill_raw(seed, *, H: int, d: int, dtype: str, chunk_size: int, gate: str,
                     B: int = 1, T: int = 0, lengths=None,
                     s0_std: Optional[float] = None) -> RawPrefill:
    """Draw one raw-input prefill workload (recipe above)."""
    rng = np.random.default_rng(seed)
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        cu = np.zeros(len(lengths) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lengths)
        n, total = len(lengths), int(cu[-1])
    else:
        cu, n, total = None, B, B * T
    q = rng.standard_normal((total, H, d))
    k = rng.standard_normal((total, H, d))
    v = rng.standard_normal((total, H, d))
    bl = rng.standard_normal((total, H))
    z = rng.normal(GATE_Z_MU[gate], 1.0, size=(total, H, d))
    A = None
    if gate == "softplus":
        A = np.log(rng.uniform(0.05, 0.3, size=H)).astype(np.float32)
    s0 = None
    if s0_std is not None:
        s0 = rng.normal(0.0, s0_std, size=(n, H, d, d)).astype(np.float32)
    return RawPrefill(q=_round_operand(q, dtype), k=_round_operand(k, dtype),
                      v=_round_operand(v, dtype), z=_round_operand(z, dtype),
                      beta_logits=bl.astype(np.float32), gate=gate, gate_A=A,
                      gate_min=-5.0, cu_seqlens=cu, num_seqs=n, initial_state=s0,
                      dtype=dtype, chunk_size=chunk_size)


# Model-boundary form of the headline prefill, the fusion benchmark workload:
# raw inputs (Kimi Linear's softplus gate, seed 5) and the output epilogue
# (RMSNorm weight and output-gate logits from epilogue_inputs, seed 55).
RAW_PREFILL = dict(name="prefill_fused", B=2, H=8, T=2048, d=128, chunk_size=64,
                   dtype=BF16, gate="softplus")


def raw_prefill_workload(with_epilogue: bool = True) -> RawPrefill:
    w = dict(RAW_PREFILL)
    w.pop("name")
    r = make_prefill_raw(5, **w)
    if with_epilogue:
        r.out_norm_weight, r.out_gate = epilogue_inputs(55, (r.total_tokens, r.num_heads),
                                                        w["d"], w["dtype"])
    return r


def decode_step_raw(step: int, batch: int, H: int, d: int, dtype: str, gate: str,
                    seed_base: int = 6) -> RawPrefill:
    """Raw inputs of decode step `step` ([batch, H, d], one token per
    state): q, k, v, beta logits and z from default_rng([seed_base, step]) in
    the order of the recipe above; the per-head A (a parameter, the same at
    every step) from default_rng(seed_base)."""
    rng = np.random.default_rng([seed_base, step])
    q = rng.standard_normal((batch, H, d))
    k = rng.standard_normal((batch, H, d))
    v = rng.standard_normal((batch, H, d))
    bl = rng.standard_normal((batch, H))
    z = rng.normal(GATE_Z_MU[gate], 1.0, size=(batch, H, d))
    A = None
    if gate == "softplus":
        A = np.log(np.random.default_rng(seed_base).uniform(0.05, 0.3, size=H))
        A = A.astype(np.float32)
    return RawPrefill(q=_round_operand(q, dtype), k=_round_operand(k, dtype),
                      v=_round_operand(v, dtype), z=_round_operand(z, dtype),
                      beta_logits=bl.astype(np.float32), gate=gate, gate_A=A,
                      gate_min=-5.0, cu_seqlens=None, num_seqs=batch, initial_state=None,
                      dtype=dtype, chunk_size=0)


def epilogue_inputs(seed, rows_shape, d: int, dtype: str):
    """Output-epilogue inputs from default_rng(seed), in this order: RMSNorm
    weight 1 + 0.2 N(0, 1) [d] (fp32), then output-gate logits N(0, 1)
    [*rows_shape, d] rounded to the operand dtype."""
    rng = np.random.default_rng(seed)
    w = (1.0 + 0.2 * rng.standard_normal(d)).astype(np.float32)
    z = rng.standard_normal(tuple(rows_shape) + (d,))
    return w, _round_operand(z, dtype)


def backward_inputs(seed, T: int, H: int, d: int, n: int, dtype: str):
    """Gradients fed to the backward, from default_rng(seed) in this order:
    d_o ~ N(0, 1) [T, H, d] rounded to the operand dtype, then the final-state
    gradient ~ N(0, 0.1) [n, H, d, d] (fp32)."""
    rng = np.random.default_rng(seed)
    do = _round_operand(rng.standard_normal((T, H, d)), dtype)
    dsf = rng.normal(0.0, 0.1, size=(n, H, d, d)).astype(np.float32)
    return do, dsf
