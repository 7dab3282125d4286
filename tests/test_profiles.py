"""The committed counter readings that bench.py reports as `roofline.traffic`
parse and cover every kernel the benchmark prices (CPU only).

The readings are only used while a kernel's sources hash to the recorded
value; this test checks the file's structure, not the hashes, so it keeps
passing between a kernel change and the next counter run (bench.py then
reports null traffic for that kernel).
"""
import importlib.util
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_readings_cover_every_priced_kernel():
    b = _bench()
    with open(b.TRAFFIC_FILE) as fh:
        text = fh.read()
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    assert m, "no JSON block of counter readings"
    data = json.loads(m.group(1))
    assert data["copy_bytes"] > 0
    # FETCH_SIZE counts a 128-byte read as 64 bytes; WRITE_SIZE counts bytes
    assert abs(data["fetch_scale"] - 2.0) < 0.01 and abs(data["write_scale"] - 1.0) < 0.01
    want = [f"{w}/{k}" for w in ("prefill", "prefill_fused", "long", "varlen")
            for k in ("intra", "inter")] + ["decode/decode_kernel", "backward/bwd"]
    for key in want:
        rec = data["kernels"][key]
        assert rec["fetch_kib"] > 0 and rec["write_kib"] > 0, key
        assert re.fullmatch(r"[0-9a-f]{64}", rec["sources_sha256"]), key
        stage = key.split("/")[1]
        assert stage in b.KERNEL_SOURCES, key


def test_kernel_trace_summaries_name_their_commands_and_kernels():
    prof = os.path.join(ROOT, "profiles")
    traces = [f for f in os.listdir(prof) if f.endswith("_kernels.md")]
    assert traces
    for f in traces:
        with open(os.path.join(prof, f)) as fh:
            text = fh.read()
        assert "rocprofv3 --kernel-trace --stats" in text, f
        assert "python3 bench.py" in text, f
        rows = [l for l in text.splitlines() if l.startswith("| `")]
        assert any("kda" in l for l in rows), f
