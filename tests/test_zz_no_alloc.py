"""kda_fwd_chunked_noalloc (the prefill with the library's own per-GPU
workspace array, for callers that cannot allocate) against kda_fwd_chunked
with a caller workspace: the same kernels, so the outputs and final states
must agree bit for bit.  Two calls in a row, the second smaller than the
first, so that the second runs on an array the first has filled."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

from gated_delta_rule_chunked_amd import inputs as kin  # noqa: E402
from kda_testutil import from_device, upload_prefill  # noqa: E402

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _both(w):
    import gated_delta_rule_chunked_amd as kda
    from gated_delta_rule_chunked_amd import kda as kb
    d = upload_prefill(w)
    kw = dict(cu_seqlens=d["cu_seqlens"], num_seqs=d["num_seqs"],
              initial_state=d["initial_state"], chunk_size=w.chunk_size)
    need = kb.workspace_size(w.total_tokens, w.num_seqs, w.num_heads, w.head_dim,
                             w.chunk_size, d["q"].dtype)
    assert 0 < need <= kb.NOALLOC_SCRATCH_BYTES
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["beta"])
    o_ref, s_ref = kda.fwd_chunked(*args, **kw)
    o, s = kb.fwd_chunked_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return from_device(o), from_device(s), from_device(o_ref), from_device(s_ref)


def test_noalloc_matches_the_workspace_call_twice_second_smaller():
    print("[noalloc] call 1: B=2 H=8 T=2048 d=128 C=64 bf16", flush=True)
    w1 = kin.workload(1)
    o, s, o_ref, s_ref = _both(w1)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(s, s_ref)
    print("[noalloc] call 2: ragged packed sequences H=3 d=64 C=32 bf16, initial states",
          flush=True)
    w2 = kin.make_prefill(950, H=3, d=64, dtype=kin.BF16, chunk_size=32,
                          lengths=[100, 0, 1, 64, 77], s0_std=0.05)
    o, s, o_ref, s_ref = _both(w2)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(s, s_ref)
    np.testing.assert_array_equal(s[1], w2.initial_state[1])
