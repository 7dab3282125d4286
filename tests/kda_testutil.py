"""Helpers shared by the GPU tests: host -> device upload of seeded inputs and
the error measure.  (No operator arithmetic here.)"""
import numpy as np

from gated_delta_rule_chunked_amd import inputs as kin

TOL = {kin.F32: 1e-4, kin.BF16: 2e-2}


def relerr(x, ref):
    """Normwise max relative error max|x - ref| / max|ref| (0 if both are 0)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    if den == 0.0:
        return num
    return num / den


def to_device(a, dtype, device="cuda"):
    """numpy operand array (bf16 bits or float32) -> torch tensor on device."""
    import torch
    if dtype == kin.BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def f32_device(a, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def from_device(t):
    """torch tensor -> float64 numpy (exact for bf16 and fp32)."""
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def upload_prefill(w: "kin.Prefill", device="cuda"):
    import torch
    d = dict(q=to_device(w.q, w.dtype, device), k=to_device(w.k, w.dtype, device),
             v=to_device(w.v, w.dtype, device), log_alpha=f32_device(w.g, device),
             beta=f32_device(w.beta, device))
    d["cu_seqlens"] = (None if w.cu_seqlens is None else
                       torch.from_numpy(w.cu_seqlens.astype(np.int32)).to(device))
    d["initial_state"] = (None if w.initial_state is None else
                          f32_device(w.initial_state, device))
    d["num_seqs"] = w.num_seqs
    return d
