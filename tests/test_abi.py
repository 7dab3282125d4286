"""CPU-only checks of the C ABI library: it loads, exports every symbol that
include/kda.h declares, and rejects bad arguments on the host before any HIP
call (no compute is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")
LIB = os.path.join(ROOT, "gated_delta_rule_chunked_amd", "libkda.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from gated_delta_rule_chunked_amd import build
        build.build()
    from gated_delta_rule_chunked_amd import kda
    return kda.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kda_fwd_chunked", "kda_fwd_chunked_stage", "kda_decode_step",
              "kda_fwd_chunked_workspace_size", "kda_status_string", "kda_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in kda.h but not exported"


def test_status_strings(lib):
    assert lib.kda_status_string(0) == b"KDA_SUCCESS"
    assert lib.kda_status_string(1) == b"KDA_ERROR_INVALID_VALUE"
    assert lib.kda_status_string(2) == b"KDA_ERROR_NOT_SUPPORTED"
    assert lib.kda_status_string(3) == b"KDA_ERROR_LAUNCH_FAILED"
    assert lib.kda_status_string(4) == b"KDA_ERROR_SCRATCH_TOO_SMALL"
    assert lib.kda_status_string(77) == b"KDA_UNKNOWN_STATUS"
    assert lib.kda_version() >= 100


def test_workspace_size(lib):
    ws = lib.kda_fwd_chunked_workspace_size
    assert ws(4096, 2, 8, 128, 128, 64, 1) > 0
    assert ws(4096, 2, 8, 96, 96, 64, 1) == 0      # unsupported head size
    assert ws(4096, 2, 8, 128, 128, 48, 1) == 0    # unsupported chunk
    assert ws(4096, 2, 8, 128, 128, 64, 0) > 0     # fp32 at d = 128
    assert ws(4096, 2, 8, 96, 96, 64, 0) == 0      # unsupported head size
    assert ws(4096, 2, 8, 128, 64, 64, 1) == 0     # d_k != d_v
    assert ws(-1, 2, 8, 128, 128, 64, 1) == 0
    assert ws(0, 1, 1, 32, 32, 16, 0) > 0
    # varlen bound: more sequences never need less workspace
    assert ws(4096, 16, 8, 128, 128, 64, 1) >= ws(4096, 2, 8, 128, 128, 64, 1)


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first


def _fwd(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=None, n=2, T=256, H=2, dk=128,
             dv=128, C=64, dt=1, s0=None, sf=None, o=FAKE, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(over)
    return lib.kda_fwd_chunked(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["n"],
                               a["T"], a["H"], a["dk"], a["dv"], a["C"], a["dt"], a["s0"],
                               a["sf"], a["o"], a["ws"], a["wsb"], a["stream"])


def test_fwd_rejects_bad_arguments_on_host(lib):
    assert _fwd(lib, q=None) == 1
    assert _fwd(lib, o=None) == 1
    assert _fwd(lib, ws=None) == 1
    assert _fwd(lib, wsb=16) == 1                    # workspace too small
    assert _fwd(lib, q=ctypes.c_void_p((1 << 20) + 2)) == 1  # misaligned
    assert _fwd(lib, ws=ctypes.c_void_p((1 << 20) + 64)) == 1
    assert _fwd(lib, T=255) == 1                     # 255 % 2 sequences
    assert _fwd(lib, n=0) == 1
    assert _fwd(lib, H=0) == 1
    assert _fwd(lib, T=-5) == 1
    assert _fwd(lib, dt=7) == 1
    assert _fwd(lib, dk=96, dv=96) == 2
    assert _fwd(lib, dk=128, dv=64) == 2
    assert _fwd(lib, C=128) == 2
    assert _fwd(lib, n=1, T=1 << 24, H=1024) == 2    # 2^28 (chunk, head) tiles
    assert _fwd(lib, n=1, T=1 << 22, H=64, wsb=16) == 1  # 2^22 tiles pass, workspace fails


def test_stage_rejects_bad_stage_and_arguments(lib):
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, None, 2, 256, 2, 128, 128, 64, 1, None, None,
            FAKE, FAKE, 1 << 40, None)
    assert lib.kda_fwd_chunked_stage(2, *args) == 1  # stages are 0 (intra) and 1 (inter)
    assert lib.kda_fwd_chunked_stage(-1, *args) == 1
    bad = list(args)
    bad[0] = None
    assert lib.kda_fwd_chunked_stage(0, *bad) == 1
    bad = list(args)
    bad[9] = bad[10] = 96
    assert lib.kda_fwd_chunked_stage(1, *bad) == 2


def _dec(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, st=FAKE, o=FAKE, B=4, H=2, dk=128,
             dv=128, dt=1, stream=None)
    a.update(over)
    return lib.kda_decode_step(a["q"], a["k"], a["v"], a["g"], a["beta"], a["st"], a["o"],
                               a["B"], a["H"], a["dk"], a["dv"], a["dt"], a["stream"])


def test_decode_rejects_bad_arguments_on_host(lib):
    assert _dec(lib, st=None) == 1
    assert _dec(lib, o=None) == 1
    assert _dec(lib, B=0) == 1
    assert _dec(lib, dt=3) == 1
    assert _dec(lib, st=ctypes.c_void_p((1 << 20) + 4)) == 1
    assert _dec(lib, dk=48, dv=48) == 2
    assert _dec(lib, dk=128, dv=32) == 2


def test_binding_fails_loudly_without_device():
    """The Python binding never falls back to a CPU path."""
    torch = pytest.importorskip("torch")
    from gated_delta_rule_chunked_amd import kda
    x = torch.zeros((4, 1, 32), dtype=torch.float32)
    with pytest.raises(kda.KdaError):
        kda.fwd_chunked(x, x, x, x, torch.zeros((4, 1)))
    with pytest.raises(kda.KdaError):
        kda.decode_step(x, x, x, x, torch.zeros((4, 1)), torch.zeros((4, 1, 32, 32)))


def _opts(gate=0, A=None, gmin=0.0, norm=0, blog=0):
    from gated_delta_rule_chunked_amd import kda
    return ctypes.pointer(kda.KdaOptions(gate, A, gmin, norm, blog))


def _fwd_ex(lib, opt, stages=3, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=None, n=2, T=256, H=2, dk=128,
             dv=128, C=64, dt=1, s0=None, sf=None, o=FAKE, ws=FAKE, wsb=1 << 40,
             stream=None)
    a.update(over)
    return lib.kda_fwd_chunked_ex(opt, stages, a["q"], a["k"], a["v"], a["g"], a["beta"],
                                  a["cu"], a["n"], a["T"], a["H"], a["dk"], a["dv"], a["C"],
                                  a["dt"], a["s0"], a["sf"], a["o"], a["ws"], a["wsb"],
                                  a["stream"])


def test_fwd_ex_rejects_bad_options_on_host(lib):
    """Input-side fusion options are validated before anything is enqueued
    (every case below fails validation; none launches)."""
    assert _fwd_ex(lib, None, stages=0) == 1
    assert _fwd_ex(lib, None, stages=4) == 1
    assert _fwd_ex(lib, _opts(gate=7)) == 1
    assert _fwd_ex(lib, _opts(gate=1, A=None)) == 1              # softplus needs A
    assert _fwd_ex(lib, _opts(gate=2, gmin=0.0)) == 1            # g_min must be < 0
    assert _fwd_ex(lib, _opts(gate=2, gmin=float("nan"))) == 1
    assert _fwd_ex(lib, _opts(gate=2, gmin=float("-inf"))) == 1
    assert _fwd_ex(lib, _opts(gate=1, A=(1 << 20) + 2)) == 1     # misaligned A
    # valid options still meet the size and workspace checks
    assert _fwd_ex(lib, _opts(gate=2, gmin=-5.0, norm=1, blog=1), wsb=16) == 1
    assert _fwd_ex(lib, _opts(gate=1, A=1 << 20), dk=96, dv=96) == 2
    assert _fwd_ex(lib, _opts(gate=2, gmin=-5.0), g=ctypes.c_void_p((1 << 20) + 8)) == 1
    from gated_delta_rule_chunked_amd import kda
    bad_slots = ctypes.pointer(kda.KdaOptions(0, None, 0.0, 0, 0, (1 << 20) + 2, 4))
    assert _fwd_ex(lib, bad_slots) == 1                          # misaligned slots
    no_pool = ctypes.pointer(kda.KdaOptions(0, None, 0.0, 0, 0, 1 << 20, 0))
    assert _fwd_ex(lib, no_pool) == 1                            # num_slots < 1
    def epi(w, z, eps):
        return ctypes.pointer(kda.KdaOptions(0, None, 0.0, 0, 0, None, 0, w, z, eps))
    assert _fwd_ex(lib, epi(None, 1 << 20, 1e-6)) == 1           # gate without norm
    assert _fwd_ex(lib, epi(1 << 20, None, 0.0)) == 1            # eps must be > 0
    assert _fwd_ex(lib, epi(1 << 20, None, float("nan"))) == 1
    assert _fwd_ex(lib, epi((1 << 20) + 4, None, 1e-6)) == 1     # weight 16-byte aligned
    assert _fwd_ex(lib, epi(1 << 20, (1 << 20) + 8, 1e-6)) == 1  # out_gate 16-byte aligned
    assert _fwd_ex(lib, epi(1 << 20, 1 << 20, 1e-6), wsb=16) == 1
    def diag(flags, check):
        return ctypes.pointer(kda.KdaOptions(0, None, 0.0, 0, 0, None, 0, None, None, 0.0,
                                             flags, check))
    assert _fwd_ex(lib, diag(None, 1)) == 1                      # check_inputs needs flags
    assert _fwd_ex(lib, diag((1 << 20) + 2, 0)) == 1             # flags 4-byte aligned
    assert _fwd_ex(lib, diag(1 << 20, 1), wsb=16) == 1           # valid, still size-checked


def test_decode_ex_rejects_bad_options_on_host(lib):
    def dec_ex(opt, **over):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, st=FAKE, o=FAKE, B=4, H=2,
                 dk=128, dv=128, dt=1, stream=None)
        a.update(over)
        return lib.kda_decode_step_ex(opt, a["q"], a["k"], a["v"], a["g"], a["beta"],
                                      a["st"], a["o"], a["B"], a["H"], a["dk"], a["dv"],
                                      a["dt"], a["stream"])
    assert dec_ex(_opts(gate=3)) == 1
    assert dec_ex(_opts(gate=1)) == 1
    assert dec_ex(_opts(gate=2, gmin=1.0)) == 1
    assert dec_ex(_opts(gate=2, gmin=-5.0), st=None) == 1
    assert dec_ex(_opts(gate=1, A=1 << 20), dk=48, dv=48) == 2


def test_bwd_rejects_bad_arguments_on_host(lib):
    """kda_bwd_chunked validates before anything is enqueued (every case below
    fails validation)."""
    def bwd(**over):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, cu=None, n=2, T=256, H=2, dk=64,
                 dv=64, C=64, dt=1, s0=None, do=FAKE, dsf=None, dq=FAKE, dk_=FAKE, dv_=FAKE,
                 dg=FAKE, db=FAKE, ds0=None, ws=FAKE, wsb=16, stream=None)
        a.update(over)
        return lib.kda_bwd_chunked(a["q"], a["k"], a["v"], a["g"], a["beta"], a["cu"], a["n"],
                                   a["T"], a["H"], a["dk"], a["dv"], a["C"], a["dt"], a["s0"],
                                   a["do"], a["dsf"], a["dq"], a["dk_"], a["dv_"], a["dg"],
                                   a["db"], a["ds0"], a["ws"], a["wsb"], a["stream"])
    assert bwd() == 1                                   # workspace too small
    assert bwd(do=None) == 1
    assert bwd(dq=None) == 1
    assert bwd(db=ctypes.c_void_p((1 << 20) + 2)) == 1
    assert bwd(dsf=ctypes.c_void_p((1 << 20) + 4)) == 1
    assert bwd(dk=96, dv=96) == 2
    assert bwd(C=128) == 2
    assert bwd(T=255) == 1
    assert lib.kda_bwd_chunked_workspace_size(4096, 2, 8, 128, 128, 64, 1) > 0
    assert lib.kda_bwd_chunked_workspace_size(4096, 2, 8, 96, 96, 64, 1) == 0


def test_noalloc_rejects_calls_beyond_its_scratch_on_the_host(lib):
    """kda_fwd_chunked_noalloc refuses, before any HIP call, a prefill whose
    workspace exceeds KDA_NOALLOC_SCRATCH_BYTES (here B=1 x T=32768 x H=32,
    1.16 GiB), and returns the size errors of kda_fwd_chunked for invalid
    or unsupported sizes.  Device pointers are never dereferenced on the
    host, so aligned dummy addresses stand in for them."""
    p = [ctypes.c_void_p(0x100000 + 0x1000 * i) for i in range(8)]
    f = lib.kda_fwd_chunked_noalloc
    big = lib.kda_fwd_chunked_workspace_size(32768, 1, 32, 128, 128, 64, 1)
    assert big > 64 << 20
    assert f(p[0], p[1], p[2], p[3], p[4], None, 1, 32768, 32, 128, 128, 64, 1, None, p[5],
             p[6], None) == 4
    assert f(p[0], p[1], p[2], p[3], p[4], None, 1, 4096, 8, 96, 96, 64, 1, None, p[5], p[6],
             None) == 2  # unsupported head size
    assert f(p[0], p[1], p[2], p[3], p[4], None, 0, 4096, 8, 128, 128, 64, 1, None, p[5], p[6],
             None) == 1  # no sequences
