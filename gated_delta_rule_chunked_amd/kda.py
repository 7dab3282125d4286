"""Python binding of libkda.so (include/kda.h): argument marshalling only.

Torch provides device memory and the current HIP stream; every step of the
operator runs in the library's HIP kernels.  There is no fallback: if the
library is missing or the tensors are not on a ROCm device, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libkda.so")

KDA_SUCCESS = 0
KDA_DTYPE_F32 = 0
KDA_DTYPE_BF16 = 1

_lib = None

GATES = {"log_alpha": 0, "softplus": 1, "sigmoid": 2}


class KdaOptions(ctypes.Structure):
    """kda_options (include/kda.h): input-side fusion, state slots, output
    epilogue, diagnostics."""
    _fields_ = [("gate", ctypes.c_int), ("gate_A", ctypes.c_void_p),
                ("gate_min", ctypes.c_float), ("l2norm_qk", ctypes.c_int32),
                ("beta_logits", ctypes.c_int32), ("state_slots", ctypes.c_void_p),
                ("num_slots", ctypes.c_int32), ("out_norm_weight", ctypes.c_void_p),
                ("out_gate", ctypes.c_void_p), ("out_norm_eps", ctypes.c_float),
                ("flags", ctypes.c_void_p), ("check_inputs", ctypes.c_int32)]


# bits of kda_options.flags (include/kda.h)
FLAG_DECAY_RANGE = 1
FLAG_BAD_CU_SEQLENS = 2


class KdaError(RuntimeError):
    """A KDA call returned a non-success status, or the library is missing."""


def library():
    """Load libkda.so (once).  Raises KdaError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise KdaError(
            f"{library_path} is not built; run "
            "`python -m gated_delta_rule_chunked_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(library_path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_version.restype = ctypes.c_int
    lib.kda_fwd_chunked_workspace_size.restype = sz
    lib.kda_fwd_chunked_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32, ctypes.c_int]
    lib.kda_fwd_chunked.restype = ctypes.c_int
    lib.kda_fwd_chunked.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                    ctypes.c_int, vp, vp, vp, vp, sz, vp]
    lib.kda_fwd_chunked_stage.restype = ctypes.c_int
    lib.kda_fwd_chunked_stage.argtypes = [ctypes.c_int] + lib.kda_fwd_chunked.argtypes
    lib.kda_decode_step.restype = ctypes.c_int
    lib.kda_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                    ctypes.c_int, vp]
    lib.kda_bwd_chunked_workspace_size.restype = sz
    lib.kda_bwd_chunked_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32, ctypes.c_int]
    lib.kda_bwd_chunked.restype = ctypes.c_int
    lib.kda_bwd_chunked.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                    ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                    sz, vp]
    lib.kda_fwd_chunked_noalloc.restype = ctypes.c_int
    lib.kda_fwd_chunked_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                            i32, ctypes.c_int, vp, vp, vp, vp]
    pin = ctypes.POINTER(KdaOptions)
    lib.kda_fwd_chunked_ex.restype = ctypes.c_int
    lib.kda_fwd_chunked_ex.argtypes = [pin, ctypes.c_uint32] + lib.kda_fwd_chunked.argtypes
    lib.kda_decode_step_ex.restype = ctypes.c_int
    lib.kda_decode_step_ex.argtypes = [pin] + lib.kda_decode_step.argtypes
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != KDA_SUCCESS:
        name = library().kda_status_string(status).decode()
        raise KdaError(f"{what} failed: {name}")


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KDA_DTYPE_BF16
    if t == torch.float32:
        return KDA_DTYPE_F32
    raise KdaError(f"unsupported operand dtype {t}; use bfloat16 or float32")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise KdaError(f"{name} must be a ROCm device tensor")
    if not t.is_contiguous():
        raise KdaError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise KdaError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise KdaError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_size(total_tokens: int, num_seqs: int, num_heads: int, head_dim: int,
                   chunk_size: int, dtype: torch.dtype) -> int:
    """Bytes of workspace fwd_chunked needs (0 = unsupported sizes)."""
    return int(library().kda_fwd_chunked_workspace_size(
        total_tokens, num_seqs, num_heads, head_dim, head_dim, chunk_size,
        _dtype_code(dtype)))


STAGES = {"intra": 0, "inter": 1}


def _inputs(gate, gate_A, gate_min, l2norm_qk, beta_logits, H, state_slots=None,
            num_slots=0, n=None, epilogue=None, flags=None, check_inputs=False):
    """kda_options for the options, or None for the plain call, and the
    tensors it points to.  `epilogue` = (out_norm_weight, out_gate,
    out_norm_eps, d, out_gate_shape, dtype) or None."""
    if gate not in GATES:
        raise KdaError(f"unknown gate {gate!r}; one of {sorted(GATES)}")
    no_epi = epilogue is None or (epilogue[0] is None and epilogue[1] is None)
    if (gate == "log_alpha" and not l2norm_qk and not beta_logits and state_slots is None
            and no_epi and flags is None and not check_inputs):
        return None, ()
    keep = ()
    f_ptr = None
    if flags is not None:
        _need(flags, "flags", torch.int32, (1,))
        f_ptr, keep = flags.data_ptr(), (flags,)
    elif check_inputs:
        raise KdaError("check_inputs needs a flags tensor (int32 [1]) to report into")
    a_ptr = None
    if gate == "softplus":
        if gate_A is None:
            raise KdaError("gate='softplus' needs gate_A, fp32 [H]")
        _need(gate_A, "gate_A", torch.float32, (H,))
        a_ptr, keep = gate_A.data_ptr(), keep + (gate_A,)
    s_ptr = None
    if state_slots is not None:
        _need(state_slots, "state_slots", torch.int32, (n,))
        s_ptr, keep = state_slots.data_ptr(), keep + (state_slots,)
    w_ptr = z_ptr = None
    eps = 0.0
    if not no_epi:
        w, z, eps, d, zshape, dtype = epilogue
        if w is None:
            raise KdaError("out_gate needs out_norm_weight (the epilogue is RMSNorm, then gate)")
        _need(w, "out_norm_weight", torch.float32, (d,))
        w_ptr, keep = w.data_ptr(), keep + (w,)
        if z is not None:
            _need(z, "out_gate", dtype, zshape)
            z_ptr, keep = z.data_ptr(), keep + (z,)
    return ctypes.pointer(KdaOptions(GATES[gate], a_ptr, float(gate_min), int(bool(l2norm_qk)),
                                     int(bool(beta_logits)), s_ptr, int(num_slots), w_ptr,
                                     z_ptr, float(eps), f_ptr, int(bool(check_inputs)))), keep


def _need_gate(g, gate, dtype, shape):
    _need(g, "gate" if gate != "log_alpha" else "log_alpha",
          torch.float32 if gate == "log_alpha" else dtype, shape)


def _prep_fwd(q, k, v, log_alpha, beta, cu_seqlens, num_seqs, initial_state, chunk_size,
              output_final_state, out, final_state, workspace, allow_alloc_ws=True,
              gate="log_alpha", state_slots=None):
    """Checks the tensors of a prefill call, allocates missing outputs and
    returns (ctypes argument tuple, o, final_state, workspace, num_slots).
    With a gate other than "log_alpha", `log_alpha` is the gate input z
    (q's dtype).  With state_slots the states are pools [num_slots, H, d, d]
    and the final states go to `final_state`, by default `initial_state`."""
    T, H, d = q.shape
    dt = _dtype_code(q.dtype)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype, (T, H, d))
    _need_gate(log_alpha, gate, q.dtype, (T, H, d))
    _need(beta, "beta", torch.float32, (T, H))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        n = cu_seqlens.numel() - 1
    else:
        n = 1 if num_seqs is None else int(num_seqs)
    dev = q.device
    num_slots = 0
    if state_slots is not None:
        pool = initial_state if initial_state is not None else final_state
        if pool is None:
            raise KdaError("state_slots needs an initial_state or final_state pool")
        num_slots = pool.shape[0]
        if output_final_state and final_state is None:
            final_state = initial_state
    ns = n if state_slots is None else num_slots
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (ns, H, d, d))
    o = out if out is not None else torch.empty((T, H, d), dtype=v.dtype, device=dev)
    _need(o, "out", v.dtype, (T, H, d))
    fs = None
    if output_final_state:
        fs = final_state if final_state is not None else torch.empty(
            (n, H, d, d), dtype=torch.float32, device=dev)
        _need(fs, "final_state", torch.float32, (ns, H, d, d))
    need = workspace_size(T, n, H, d, chunk_size, q.dtype)
    if need == 0:
        raise KdaError(f"unsupported sizes T={T} N={n} H={H} d={d} chunk={chunk_size} "
                       f"dtype={q.dtype}")
    if workspace is None or workspace.numel() < need:
        if not allow_alloc_ws:
            raise KdaError("a single stage needs the workspace of a full call")
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(cu_seqlens), n,
            T, H, d, d, chunk_size, dt, _ptr(initial_state), _ptr(fs), _ptr(o),
            _ptr(workspace), workspace.numel(), _stream(dev))
    return args, o, fs, workspace, num_slots


def fwd_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                log_alpha: torch.Tensor, beta: torch.Tensor,
                cu_seqlens: Optional[torch.Tensor] = None,
                num_seqs: Optional[int] = None,
                initial_state: Optional[torch.Tensor] = None,
                chunk_size: int = 64, output_final_state: bool = True,
                out: Optional[torch.Tensor] = None,
                final_state: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                stage: Optional[str] = None,
                gate: str = "log_alpha", gate_A: Optional[torch.Tensor] = None,
                gate_min: float = -5.0, l2norm_qk: bool = False,
                beta_logits: bool = False, state_slots: Optional[torch.Tensor] = None,
                out_norm_weight: Optional[torch.Tensor] = None,
                out_gate: Optional[torch.Tensor] = None, out_norm_eps: float = 1e-6,
                flags: Optional[torch.Tensor] = None, check_inputs: bool = False,
                ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked KDA prefill (kda_fwd_chunked, or kda_fwd_chunked_ex with
    input-side fusion).

    q, k: [T, H, d] and v: [T, H, d] (bf16 or fp32, same dtype);
    log_alpha: [T, H, d] fp32; beta: [T, H] fp32;
    cu_seqlens: int32 [N+1] device tensor, or None for `num_seqs` (default 1)
    equal-length sequences; initial_state: fp32 [N, H, d, d] or None.
    Returns (o [T, H, d] in v's dtype, final_state fp32 [N, H, d, d] or None).
    `final_state` may be passed as the same tensor as `initial_state` to
    update states in place.  `stage` ("intra" or "inter") runs only
    that kernel (kda_fwd_chunked_stage); it then needs the `workspace`, `out`
    and `final_state` of a preceding call with the same arguments.

    Input-side fusion (kda_options): gate="softplus" (g = -exp(gate_A[h])
    softplus(z)) or "sigmoid" (g = gate_min sigmoid(z)) makes `log_alpha`
    the gate input z, in q's dtype; l2norm_qk normalises q and k per token
    and head; beta_logits passes beta through a sigmoid.  state_slots (int32
    [N] device tensor) makes initial_state / final_state pools of states
    indexed by slot (final_state defaults to initial_state then).
    out_norm_weight (fp32 [d]) turns on the output epilogue: every output
    row becomes o / sqrt(mean(o^2) + out_norm_eps) * out_norm_weight *
    sigmoid(out_gate) (out_gate [T, H, d] in v's dtype, or None).

    Diagnostics: `flags` (int32 [1] device tensor, zeroed by the caller)
    collects FLAG_DECAY_RANGE (a 16-token block's summed log-decay fell
    below -80, the precondition of the chunk algorithm) and, with check_inputs,
    FLAG_BAD_CU_SEQLENS (cu_seqlens failed validation on the device; nothing
    was computed).  Read it after synchronising.
    """
    if stage is not None and stage not in STAGES:
        raise KdaError(f"unknown stage {stage!r}; one of {sorted(STAGES)}")
    args, o, fs, _, nsl = _prep_fwd(q, k, v, log_alpha, beta, cu_seqlens, num_seqs,
                                    initial_state, chunk_size, output_final_state, out,
                                    final_state, workspace, allow_alloc_ws=stage is None,
                                    gate=gate, state_slots=state_slots)
    opt, _keep = _inputs(gate, gate_A, gate_min, l2norm_qk, beta_logits, q.shape[1],
                         state_slots, nsl, args[6],
                         (out_norm_weight, out_gate, out_norm_eps, q.shape[2], tuple(o.shape),
                          v.dtype), flags, check_inputs)
    if opt is not None:
        mask = 3 if stage is None else 1 << STAGES[stage]
        _check(library().kda_fwd_chunked_ex(opt, mask, *args), "kda_fwd_chunked_ex")
    elif stage is None:
        _check(library().kda_fwd_chunked(*args), "kda_fwd_chunked")
    else:
        _check(library().kda_fwd_chunked_stage(STAGES[stage], *args),
               f"kda_fwd_chunked_stage({stage})")
    return o, fs


NOALLOC_SCRATCH_BYTES = 64 << 20  # KDA_NOALLOC_SCRATCH_BYTES (include/kda.h)


def fwd_chunked_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        log_alpha: torch.Tensor, beta: torch.Tensor,
                        cu_seqlens: Optional[torch.Tensor] = None,
                        num_seqs: Optional[int] = None,
                        initial_state: Optional[torch.Tensor] = None,
                        chunk_size: int = 64, out: Optional[torch.Tensor] = None,
                        final_state: Optional[torch.Tensor] = None,
                        ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """kda_fwd_chunked_noalloc: the prefill of fwd_chunked with the
    workspace taken from the library's per-GPU device array (no workspace
    argument, no allocation by the library).  Pass `out` and `final_state`
    to allocate nothing here either.  Calls that overlap on one GPU race."""
    T, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype, (T, H, d))
    _need(log_alpha, "log_alpha", torch.float32, (T, H, d))
    _need(beta, "beta", torch.float32, (T, H))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        n = cu_seqlens.numel() - 1
    else:
        n = 1 if num_seqs is None else int(num_seqs)
    dev = q.device
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (n, H, d, d))
    o = out if out is not None else torch.empty((T, H, d), dtype=v.dtype, device=dev)
    _need(o, "out", v.dtype, (T, H, d))
    fs = final_state if final_state is not None else torch.empty(
        (n, H, d, d), dtype=torch.float32, device=dev)
    _need(fs, "final_state", torch.float32, (n, H, d, d))
    _check(library().kda_fwd_chunked_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(cu_seqlens), n, T, H, d,
        d, chunk_size, _dtype_code(q.dtype), _ptr(initial_state), _ptr(fs), _ptr(o),
        _stream(dev)), "kda_fwd_chunked_noalloc")
    return o, fs


class BoundCall:
    """A C-ABI call with its arguments marshalled once.

    Calling the object re-issues the same call on the stream captured at
    bind time and raises KdaError on a non-success status.  The tensors the
    arguments point to are kept alive by `tensors`.
    """

    def __init__(self, fn, args, what, tensors):
        self._fn, self._args, self._what = fn, args, what
        self.tensors = tensors

    def __call__(self):
        st = self._fn(*self._args)
        if st != KDA_SUCCESS:
            _check(st, self._what)


def bind_fwd(q, k, v, log_alpha, beta, cu_seqlens=None, num_seqs=None,
             initial_state=None, chunk_size=64, output_final_state=True,
             out=None, final_state=None, workspace=None, gate="log_alpha", gate_A=None,
             gate_min=-5.0, l2norm_qk=False, beta_logits=False, state_slots=None,
             out_norm_weight=None, out_gate=None, out_norm_eps=1e-6, flags=None,
             check_inputs=False):
    """Validate and marshal a kda_fwd_chunked call once, for repeated calls.

    Nothing is launched here.  Returns (call, stage_calls, o, final_state):
    `call()` runs the whole prefill and `stage_calls[name]()` one of its
    kernels ("intra", "inter"; kda_fwd_chunked_stage) on the same workspace.
    The options (input-side fusion, slots, epilogue, diagnostics) are those
    of fwd_chunked.
    """
    args, o, fs, ws, nsl = _prep_fwd(q, k, v, log_alpha, beta, cu_seqlens, num_seqs,
                                     initial_state, chunk_size, output_final_state, out,
                                     final_state, workspace, gate=gate, state_slots=state_slots)
    opt, akeep = _inputs(gate, gate_A, gate_min, l2norm_qk, beta_logits, q.shape[1],
                         state_slots, nsl, args[6],
                         (out_norm_weight, out_gate, out_norm_eps, q.shape[2], tuple(o.shape),
                          v.dtype), flags, check_inputs)
    keep = (q, k, v, log_alpha, beta, cu_seqlens, initial_state, fs, o, ws, opt) + akeep
    lib = library()
    if opt is None:
        call = BoundCall(lib.kda_fwd_chunked, args, "kda_fwd_chunked", keep)
        stages = {name: BoundCall(lib.kda_fwd_chunked_stage, (sid,) + args,
                                  f"kda_fwd_chunked_stage({name})", keep)
                  for name, sid in STAGES.items()}
    else:
        call = BoundCall(lib.kda_fwd_chunked_ex, (opt, 3) + args, "kda_fwd_chunked_ex", keep)
        stages = {name: BoundCall(lib.kda_fwd_chunked_ex, (opt, 1 << sid) + args,
                                  f"kda_fwd_chunked_ex({name})", keep)
                  for name, sid in STAGES.items()}
    return call, stages, o, fs


def bind_decode(q, k, v, log_alpha, beta, state, out=None, gate="log_alpha", gate_A=None,
                gate_min=-5.0, l2norm_qk=False, beta_logits=False, state_slots=None,
                out_norm_weight=None, out_gate=None, out_norm_eps=1e-6):
    """Validate and marshal a kda_decode_step call once.  Returns (call, o);
    each `call()` advances `state` by one step in place.  The input-side
    fusion and state-slot options are those of decode_step."""
    B, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, q.dtype, (B, H, d))
    _need_gate(log_alpha, gate, q.dtype, (B, H, d))
    _need(beta, "beta", torch.float32, (B, H))
    nsl = state.shape[0] if state_slots is not None else 0
    _need(state, "state", torch.float32, (nsl if state_slots is not None else B, H, d, d))
    o = out if out is not None else torch.empty((B, H, d), dtype=v.dtype, device=q.device)
    _need(o, "out", v.dtype, (B, H, d))
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(state), _ptr(o),
            B, H, d, d, _dtype_code(q.dtype), _stream(q.device))
    opt, akeep = _inputs(gate, gate_A, gate_min, l2norm_qk, beta_logits, H, state_slots, nsl, B,
                         (out_norm_weight, out_gate, out_norm_eps, d, (B, H, d), v.dtype))
    keep = (q, k, v, log_alpha, beta, state, o, opt) + akeep
    if opt is None:
        return BoundCall(library().kda_decode_step, args, "kda_decode_step", keep), o
    return BoundCall(library().kda_decode_step_ex, (opt,) + args, "kda_decode_step_ex",
                     keep), o


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                log_alpha: torch.Tensor, beta: torch.Tensor, state: torch.Tensor,
                out: Optional[torch.Tensor] = None, gate: str = "log_alpha",
                gate_A: Optional[torch.Tensor] = None, gate_min: float = -5.0,
                l2norm_qk: bool = False, beta_logits: bool = False,
                state_slots: Optional[torch.Tensor] = None,
                out_norm_weight: Optional[torch.Tensor] = None,
                out_gate: Optional[torch.Tensor] = None,
                out_norm_eps: float = 1e-6) -> torch.Tensor:
    """One recurrent KDA step (kda_decode_step, or kda_decode_step_ex with
    input-side fusion); `state` is updated in place.

    q, k, v: [B, H, d] (bf16 or fp32); log_alpha: [B, H, d] fp32 (or the gate
    input z in q's dtype, see fwd_chunked); beta: [B, H] fp32;
    state: [B, H, d, d] fp32, or with state_slots (int32 [B] device tensor)
    a pool [num_slots, H, d, d] in which sequence b uses slot state_slots[b]
    (a slot outside the pool marks padding: o = 0, no state touched).
    The output epilogue options are those of fwd_chunked (out_gate
    [B, H, d]).  Returns o [B, H, d].
    """
    call, o = bind_decode(q, k, v, log_alpha, beta, state, out=out, gate=gate, gate_A=gate_A,
                          gate_min=gate_min, l2norm_qk=l2norm_qk, beta_logits=beta_logits,
                          state_slots=state_slots, out_norm_weight=out_norm_weight,
                          out_gate=out_gate, out_norm_eps=out_norm_eps)
    call()
    return o


def bwd_workspace_size(total_tokens: int, num_seqs: int, num_heads: int, head_dim: int,
                       chunk_size: int, dtype: torch.dtype) -> int:
    """Bytes of workspace bwd_chunked needs (0 = unsupported sizes)."""
    return int(library().kda_bwd_chunked_workspace_size(
        total_tokens, num_seqs, num_heads, head_dim, head_dim, chunk_size,
        _dtype_code(dtype)))


def bind_bwd(q, k, v, log_alpha, beta, d_o, cu_seqlens=None, num_seqs=None,
             initial_state=None, d_final_state=None, chunk_size=64, want_d_initial=True,
             workspace=None):
    """Validate and marshal a kda_bwd_chunked call once.  Returns (call,
    grads) with grads a dict of the output tensors dq, dk, dv (q's dtype),
    dg, dbeta and ds0 (fp32; ds0 None unless want_d_initial)."""
    T, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("d_o", d_o)):
        _need(t, name, q.dtype, (T, H, d))
    _need(log_alpha, "log_alpha", torch.float32, (T, H, d))
    _need(beta, "beta", torch.float32, (T, H))
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32)
        n = cu_seqlens.numel() - 1
    else:
        n = 1 if num_seqs is None else int(num_seqs)
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        if t is not None:
            _need(t, name, torch.float32, (n, H, d, d))
    dev = q.device
    grads = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
                 dg=torch.empty_like(log_alpha), dbeta=torch.empty_like(beta),
                 ds0=torch.empty((n, H, d, d), dtype=torch.float32, device=dev)
                 if want_d_initial else None)
    need = bwd_workspace_size(T, n, H, d, chunk_size, q.dtype)
    if need == 0:
        raise KdaError(f"unsupported sizes T={T} N={n} H={H} d={d} chunk={chunk_size}")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(cu_seqlens), n, T,
            H, d, d, chunk_size, _dtype_code(q.dtype), _ptr(initial_state), _ptr(d_o),
            _ptr(d_final_state), _ptr(grads["dq"]), _ptr(grads["dk"]), _ptr(grads["dv"]),
            _ptr(grads["dg"]), _ptr(grads["dbeta"]), _ptr(grads["ds0"]), _ptr(workspace),
            workspace.numel(), _stream(dev))
    keep = (q, k, v, log_alpha, beta, d_o, cu_seqlens, initial_state, d_final_state,
            workspace) + tuple(grads.values())
    return BoundCall(library().kda_bwd_chunked, args, "kda_bwd_chunked", keep), grads


def bwd_chunked(q, k, v, log_alpha, beta, d_o, cu_seqlens=None, num_seqs=None,
                initial_state=None, d_final_state=None, chunk_size=64, want_d_initial=True):
    """Gradients of the chunked prefill (kda_bwd_chunked) for the loss
    sum(o * d_o) + sum(final_state * d_final_state).  Arguments as for
    fwd_chunked; returns a dict dq, dk, dv, dg, dbeta, ds0."""
    call, grads = bind_bwd(q, k, v, log_alpha, beta, d_o, cu_seqlens=cu_seqlens,
                           num_seqs=num_seqs, initial_state=initial_state,
                           d_final_state=d_final_state, chunk_size=chunk_size,
                           want_d_initial=want_d_initial)
    call()
    return grads
