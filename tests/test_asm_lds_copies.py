"""Every workgroup barrier in the kernels that use gfx950's direct
global -> LDS copies is reached only after the wave has waited for all of
its copies (vmcnt(0)): a barrier alone does not wait for them, and LDS they
fill may be read by other waves right after it.  Checked on the AMD assembly
of this library's own sources (compiled here with hipcc; no GPU needed)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "routed_decode_attention_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


def pending_barriers(asm: str):
    """(function, barriers, barriers reached with a copy not yet waited for),
    scanning each function's code in layout order."""
    out, fn, pending, bars, bad = [], None, False, 0, 0
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            if fn:
                out.append((fn, bars, bad))
            fn, pending, bars, bad = m.group(1), False, 0, 0
            continue
        t = line.strip()
        if t.startswith("global_load_lds"):
            pending = True
        elif t.startswith("s_waitcnt") and re.search(r"vmcnt\(0\)", t):
            pending = False
        elif t.startswith("s_barrier"):
            bars += 1
            bad += pending
    if fn:
        out.append((fn, bars, bad))
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", ["score_bf16.hip", "prefill.hip", "writer.hip"])
def test_barriers_follow_the_copies_wait(src, tmp_path):
    asm = tmp_path / (src + ".s")
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
                           "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-S", os.path.join(CSRC, src),
                           "-o", str(asm)], stderr=subprocess.DEVNULL)
    text = asm.read_text()
    assert "global_load_lds" in text, "the kernel no longer uses direct copies: update this test"
    fns = pending_barriers(text)
    assert sum(b for _, b, _ in fns) > 0
    bad = [(f, n) for f, _, n in fns if n]
    assert not bad, bad
