"""fp64 CPU oracle for Kimi Delta Attention.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package
smoke check and the CPU-baseline leg of the benchmark may import this
module.  It shares no code with the HIP path and the HIP path never calls it.

The recurrence, its chunked form, the decode step, the chunk-local
cumulative sum and the UT inverse are ctypes wrappers of kda_oracle.c.  The
input-side transforms (gate functions, q/k normalisation, beta from logits)
and the output epilogue (RMSNorm, output gate) are plain numpy in fp64.  The
backward (recurrent_backward) is torch autograd in fp64 on the CPU over the
token-by-token recurrence.

Every function takes numpy arrays of any real dtype, converts them to
contiguous float64 (bf16 inputs must be expanded to float first; the
conversion is exact) and returns float64 arrays.  Layouts follow the
operator's: q, k, g [T, H, d_k]; v, o [T, H, d_v]; beta [T, H];
states [N, H, d_k, d_v]; cu_seqlens [N + 1].

Parity status: every function here is pinned to closed forms, special cases
and brute-force dense products taken from the pages: the C functions by
tests/test_oracle.py, the transforms and the epilogue by
tests/test_oracle_inputs.py, the backward by tests/test_oracle_backward.py
(central finite differences of the C forward, closed forms); none is
"parity unpinned".
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from oracle import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.kda_oracle_num_threads.restype = ctypes.c_int
    lib.kda_oracle_recurrent.argtypes = [_dp] * 5 + [_ip] + [_i64] * 5 + [_dp] * 3
    lib.kda_oracle_chunked.argtypes = [_dp] * 5 + [_ip] + [_i64] * 6 + [_dp] * 3
    lib.kda_oracle_decode.argtypes = [_dp] * 7 + [_i64] * 4
    lib.kda_oracle_chunk_cumsum.argtypes = [_dp, _ip] + [_i64] * 5 + [_dp]
    lib.kda_oracle_ut_inverse.argtypes = [_dp, _i64, _dp]
    for f in ("kda_oracle_recurrent", "kda_oracle_chunked", "kda_oracle_decode",
              "kda_oracle_chunk_cumsum", "kda_oracle_ut_inverse"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all cores)."""
    return int(_load().kda_oracle_num_threads())


def _f64(a):
    if a is None:
        return None, None
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    return a, a.ctypes.data_as(_dp)


def _cu(cu_seqlens):
    if cu_seqlens is None:
        return None, None
    c = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    return c, c.ctypes.data_as(_ip)


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (code {rc})")


def _dims(q, v, num_seqs, cu_seqlens):
    T, H, dk = q.shape
    dv = v.shape[2]
    if cu_seqlens is not None:
        n = len(cu_seqlens) - 1
    else:
        n = 1 if num_seqs is None else int(num_seqs)
    return T, H, dk, dv, n


def recurrent(q, k, v, g, beta, cu_seqlens=None, num_seqs=None,
              initial_state=None):
    """Token-by-token recurrence.  Returns (o [T,H,d_v], S_final [N,H,d_k,d_v])."""
    lib = _load()
    q, qp = _f64(q); k, kp = _f64(k); v, vp = _f64(v)
    g, gp = _f64(g); beta, bp = _f64(beta)
    cu, cp = _cu(cu_seqlens)
    T, H, dk, dv, n = _dims(q, v, num_seqs, cu)
    s0, sp = _f64(initial_state)
    o = np.zeros((T, H, dv))
    sf = np.zeros((n, H, dk, dv))
    _check(lib.kda_oracle_recurrent(qp, kp, vp, gp, bp, cp, n, T, H, dk, dv, sp,
                                    o.ctypes.data_as(_dp), sf.ctypes.data_as(_dp)),
           "kda_oracle_recurrent")
    return o, sf


def chunked(q, k, v, g, beta, chunk_size, cu_seqlens=None, num_seqs=None,
            initial_state=None):
    """Chunk-parallel form (for checking it against `recurrent`)."""
    lib = _load()
    q, qp = _f64(q); k, kp = _f64(k); v, vp = _f64(v)
    g, gp = _f64(g); beta, bp = _f64(beta)
    cu, cp = _cu(cu_seqlens)
    T, H, dk, dv, n = _dims(q, v, num_seqs, cu)
    s0, sp = _f64(initial_state)
    o = np.zeros((T, H, dv))
    sf = np.zeros((n, H, dk, dv))
    _check(lib.kda_oracle_chunked(qp, kp, vp, gp, bp, cp, n, T, H, dk, dv,
                                  int(chunk_size), sp, o.ctypes.data_as(_dp),
                                  sf.ctypes.data_as(_dp)),
           "kda_oracle_chunked")
    return o, sf


def decode(q, k, v, g, beta, state):
    """One recurrent step on a batch of states.  q,k,g [B,H,d_k]; v [B,H,d_v];
    beta [B,H]; state [B,H,d_k,d_v].  Returns (o, new_state); the input is not
    modified."""
    lib = _load()
    q, qp = _f64(q); k, kp = _f64(k); v, vp = _f64(v)
    g, gp = _f64(g); beta, bp = _f64(beta)
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    B, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((B, H, dv))
    _check(lib.kda_oracle_decode(qp, kp, vp, gp, bp, st.ctypes.data_as(_dp),
                                 o.ctypes.data_as(_dp), B, H, dk, dv),
           "kda_oracle_decode")
    return o, st


def chunk_cumsum(g, chunk_size, cu_seqlens=None, num_seqs=None):
    """Chunk-local inclusive cumulative sum of g = log(alpha), [T, H, d_k]."""
    lib = _load()
    g, gp = _f64(g)
    cu, cp = _cu(cu_seqlens)
    T, H, dk = g.shape
    n = len(cu) - 1 if cu is not None else (1 if num_seqs is None else int(num_seqs))
    out = np.zeros_like(g)
    _check(lib.kda_oracle_chunk_cumsum(gp, cp, n, T, H, dk, int(chunk_size),
                                       out.ctypes.data_as(_dp)),
           "kda_oracle_chunk_cumsum")
    return out


def ut_inverse(A):
    """(I + strictly_lower(A))^{-1} by forward substitution."""
    lib = _load()
    A, ap = _f64(A)
    n = A.shape[0]
    out = np.zeros((n, n))
    _check(lib.kda_oracle_ut_inverse(ap, n, out.ctypes.data_as(_dp)),
           "kda_oracle_ut_inverse")
    return out


# ---- input-side transforms (numpy, fp64) ------------------------------------
# The steps that produce the operator's inputs from the layers before it
# (docsaid.org "Kimi Linear", section "Les autres pieces"; fr.news.hada.io,
# section "Configuration du modele Kimi Linear"; mkdocs.reaper.mx "Attention
# lineaire et recurrence", section "Le piege numerique de la decroissance
# cumulee"), written from their definitions.  A fused call of the library is
# checked against `recurrent` / `decode` applied to what these return.

def softplus(z):
    """log(1 + e^z), computed as max(z, 0) + log1p(e^-|z|)."""
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def gate_softplus(z, A):
    """Kimi Linear's decay gate: g = -exp(A) softplus(z), one A per head.
    z: [..., H, d_k]; A: [H]."""
    A = np.asarray(A, dtype=np.float64)
    return -np.exp(A)[:, None] * softplus(z)


def gate_sigmoid(z, g_min):
    """The bounded gate g = g_min sigmoid(z), which lies in (g_min, 0)."""
    return float(g_min) * sigmoid(z)


def l2_normalize(x, eps=1e-6):
    """x / sqrt(|x|^2 + eps) over the last axis (per token and head)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def prepare_inputs(q, k, gate_in, beta_in, gate="log_alpha", gate_A=None, gate_min=-5.0,
                   l2norm_qk=False, beta_logits=False):
    """(q, k, g, beta) as the recurrence takes them, from the inputs of a
    fused call: gate "log_alpha" (gate_in is g), "softplus" or "sigmoid"
    (gate_in is z); q and k L2-normalised if asked; beta from logits if
    asked."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if gate == "log_alpha":
        g = np.asarray(gate_in, dtype=np.float64)
    elif gate == "softplus":
        g = gate_softplus(gate_in, gate_A)
    elif gate == "sigmoid":
        g = gate_sigmoid(gate_in, gate_min)
    else:
        raise ValueError(f"unknown gate {gate!r}")
    if l2norm_qk:
        q, k = l2_normalize(q), l2_normalize(k)
    b = sigmoid(beta_in) if beta_logits else np.asarray(beta_in, dtype=np.float64)
    return q, k, g, b


# ---- output epilogue (numpy, fp64) ------------------------------------------
# docsaid.org "Kimi Linear", section "Les autres pieces" and fr.news.hada.io,
# section "Configuration du modele Kimi Linear": the output goes through an
# RMSNorm per head, then is multiplied by a data-dependent sigmoid gate.

def rms_norm(o, weight, eps):
    """o / sqrt(mean(o^2) + eps) * weight over the last axis (per token and
    head); weight [d_v] is shared by the heads."""
    o = np.asarray(o, dtype=np.float64)
    return o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * np.asarray(
        weight, dtype=np.float64)


def output_epilogue(o, weight, eps, out_gate=None):
    """RMSNorm per head, then the sigmoid output gate (factor 1 without one)."""
    y = rms_norm(o, weight, eps)
    if out_gate is not None:
        y = y * sigmoid(out_gate)
    return y


# ---- backward (torch CPU, fp64) ---------------------------------------------
# The gradient of the recurrence for training (fr.news.hada.io, section
# "Algorithme parallele par chunks": the UT transform is there to use the
# matrix units in training).  The forward is the definition written out token
# by token in torch fp64 on the CPU (S' = Diag(alpha) S; u = beta (v - S'^T k);
# S = S' + k u^T; o = S^T q), and torch's reverse-mode autograd takes its
# gradient.  tests/test_oracle_backward.py pins it to central finite
# differences and to closed forms.

def _torch_recurrent(q, k, v, g, beta, bounds, s0):
    import torch
    T, H, dk = q.shape
    dv = v.shape[2]
    outs = []
    finals = []
    for n, (a, b) in enumerate(bounds):
        S = s0[n] if s0 is not None else torch.zeros((H, dk, dv), dtype=torch.float64)
        for t in range(a, b):
            Sp = torch.exp(g[t])[:, :, None] * S                          # [H, dk, dv]
            u = beta[t][:, None] * (v[t] - torch.einsum("hkv,hk->hv", Sp, k[t]))
            S = Sp + k[t][:, :, None] * u[:, None, :]
            outs.append(torch.einsum("hkv,hk->hv", S, q[t]))
        finals.append(S)
    o = torch.stack(outs) if outs else torch.zeros((0, H, dv), dtype=torch.float64)
    return o, torch.stack(finals)


def recurrent_backward(q, k, v, g, beta, d_o, d_final_state=None, cu_seqlens=None,
                       num_seqs=None, initial_state=None):
    """Gradients of L = sum(o * d_o) + sum(S_final * d_final_state) with
    respect to q, k, v, g, beta and the initial state.  Returns a dict with
    keys dq, dk, dv, dg, dbeta, ds0 (ds0 is zero-filled when there is no
    initial state, the gradient a zero initial state would get)."""
    import torch
    q = np.asarray(q, dtype=np.float64)
    T, H, dk = q.shape
    dv = np.asarray(v).shape[2]
    if cu_seqlens is not None:
        c = [int(x) for x in cu_seqlens]
        bounds = list(zip(c[:-1], c[1:]))
    else:
        n = 1 if num_seqs is None else int(num_seqs)
        L = T // n
        bounds = [(i * L, (i + 1) * L) for i in range(n)]
    n = len(bounds)
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), requires_grad=True)
    tq, tk, tv, tg, tb = t(q), t(k), t(v), t(g), t(beta)
    s0 = t(initial_state if initial_state is not None else np.zeros((n, H, dk, dv)))
    o, sf = _torch_recurrent(tq, tk, tv, tg, tb, bounds, s0)
    loss = (o * torch.tensor(np.asarray(d_o, dtype=np.float64))).sum()
    if d_final_state is not None:
        loss = loss + (sf * torch.tensor(np.asarray(d_final_state, dtype=np.float64))).sum()
    loss.backward()
    g_ = lambda x: x.grad.detach().numpy().copy() if x.grad is not None else np.zeros(x.shape)
    return dict(dq=g_(tq), dk=g_(tk), dv=g_(tv), dg=g_(tg), dbeta=g_(tb), ds0=g_(s0))
