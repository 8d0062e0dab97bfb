"""CPU: a property of the generated gfx950 code that the GPU tests only catch for the
shapes they run. The GEMM epilogues store under per-lane row conditions, which the
compiler lowers to regions with lanes switched off (an EXEC mask saved by
s_and_saveexec and restored by s_or_b64 exec). An MFMA reads the operands of every
lane of the wave, so an MFMA moved into such a region computes with the operands of
switched-off lanes missing, and a tile whose last 32-row block is partly filled
gets wrong columns. This compiles the GEMM sources as the library build does and
checks that no MFMA lies inside such a region."""
import os
import re
import shutil
import subprocess

import pytest

from mixture_experts_expert_softmax_amd import _build

SOURCES = ["gemm_bf16.hip", "gemm_mx.hip"]   # every MFMA kernel of the library


def _masked_mfmas(asm: str):
    """(function, count) of MFMAs between an EXEC save and its restore."""
    bad = []
    fn, inside, n = None, False, 0
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            if fn and n:
                bad.append((fn, n))
            fn, inside, n = m.group(1), False, 0
            continue
        if "s_and_saveexec" in line:
            inside = True
        elif re.search(r"s_or_b64\s+exec, exec", line):
            inside = False
        elif inside and "v_mfma" in line:
            n += 1
    if fn and n:
        bad.append((fn, n))
    return bad


@pytest.mark.skipif(shutil.which(_build.HIPCC) is None and not os.path.exists(_build.HIPCC),
                    reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_mfma_under_lane_masks(src, tmp_path):
    out = tmp_path / (src + ".s")
    cmd = [_build.HIPCC, *_build.FLAGS, "--offload-device-only", "-S",
           os.path.join(_build.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    asm = out.read_text()
    assert "v_mfma" in asm, "no MFMA found: wrong target?"
    assert _masked_mfmas(asm) == []
