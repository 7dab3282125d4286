"""Kimi Delta Attention (KDA) on MI355X: chunked prefill and recurrent decode.

The operator is a C-ABI shared library of hand-written HIP kernels for gfx950
(``libkda.so``, declared in ``include/kda.h``); this package is its thin
Python binding.  ``fwd_chunked`` and ``decode_step`` only marshal torch
tensors (device memory and the current stream) into the C calls.

Submodules are loaded on first use so that ``gated_delta_rule_chunked_amd.inputs``
(the seeded input generators) can be imported without torch or the library.
"""
_BINDING_NAMES = ("fwd_chunked", "decode_step", "workspace_size", "library",
                  "KdaError", "library_path", "bind_fwd", "bind_decode", "bwd_chunked",
                  "bind_bwd", "bwd_workspace_size", "FLAG_DECAY_RANGE",
                  "FLAG_BAD_CU_SEQLENS")

__all__ = list(_BINDING_NAMES)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import kda as _kda
        return getattr(_kda, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
