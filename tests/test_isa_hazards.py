"""CPU check of the compiled gfx950 code of the prefill and backward kernels.

A read of a matrix-core (MFMA) result placed right behind a branch or a
branch target has been seen to return the register's previous contents on
gfx950: the wait states the hardware needs between the instruction and the
read were missing on that path.  The kernels are written so that results are
read only in straight-line code after their MFMA; this test compiles the
sources that use the matrix cores to assembly (no GPU needed) and, for
every MFMA, follows every control-flow path for a few dozen instructions,
failing on a read of its destination registers after a branch or label
with fewer than MIN_WAIT wait states in between.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MIN_WAIT = 12  # wait states a read of a 16-pass MFMA result may need

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and
                                not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs ROCm's hipcc to compile gfx950 code")


def _regs(tok):
    m = re.match(r"([av])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([av])(\d+)$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _kernels(asm):
    out, name = {}, None
    for line in asm.split("\n"):
        m = re.match(r"^(_ZN3kda\S+):", line)
        if m:
            name = m.group(1)
            out[name] = []
        elif name is not None:
            out[name].append(line.strip())
    return out


def _suspect_reads(lines):
    labels = {l.split(":")[0]: i for i, l in enumerate(lines) if l.startswith(".LBB")}
    found = set()
    for i, line in enumerate(lines):
        if not line.startswith("v_mfma"):
            continue
        dst = _regs(line.split()[1].rstrip(","))
        stack, seen = [(i + 1, 0, False, 0)], set()
        while stack:
            j, ws, crossed, steps = stack.pop()
            while j < len(lines) and steps < 60:
                key = (j, ws >= MIN_WAIT, crossed)
                if key in seen:
                    break
                seen.add(key)
                t = lines[j]
                steps += 1
                if not t or t.startswith(";") or (t.startswith(".") and not t.startswith(".LBB")):
                    j += 1
                    continue
                if t.startswith(".LBB"):
                    crossed = True
                    j += 1
                    continue
                op = t.split()[0]
                if op == "s_endpgm":
                    break
                if op == "s_branch":
                    crossed = True
                    j = labels.get(t.split()[1], len(lines))
                    continue
                if op.startswith("s_cbranch"):
                    crossed = True
                    target = labels.get(t.split()[1])
                    if target is not None:
                        stack.append((target, ws, True, steps))
                    j += 1
                    continue
                if op == "s_nop":
                    ws += int(t.split()[1]) + 1
                    j += 1
                    continue
                ops = [x.rstrip(",") for x in t.split()[1:]]
                srcs = set()
                for o in ops[1:]:
                    srcs |= _regs(o)
                if op.startswith("v_mfma"):
                    if ops and _regs(ops[0]) & dst:
                        break
                    ws += 4
                    j += 1
                    continue
                if op.startswith(("global_store", "buffer_store", "ds_write", "flat_store")):
                    for o in ops:
                        srcs |= _regs(o)
                if srcs & dst:
                    if crossed and ws < MIN_WAIT:
                        found.add((line[:60], t[:60], ws))
                    break
                if ops and _regs(ops[0]) & dst:
                    break
                ws += 1
                j += 1
    return sorted(found)


@pytest.mark.parametrize("source", ["kda_intra.hip", "kda_inter.hip", "kda_backward.hip"])
def test_no_mfma_result_read_across_a_branch(source, tmp_path):
    from gated_delta_rule_chunked_amd import build
    out = tmp_path / "k.s"
    cmd = [build._hipcc()] + build.HIP_FLAGS + [
        "--cuda-device-only", "-S", os.path.join(build.CSRC, source), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = _kernels(out.read_text())
    assert kernels, "no kernels found in the assembly"
    bad = {name: s for name, s in ((n, _suspect_reads(l)) for n, l in kernels.items()) if s}
    assert not bad, "MFMA results read right behind a branch: " + repr(bad)[:2000]
