"""CPU: a property of the generated gfx950 code that the GPU tests only catch for the
shapes they run. The GEMM epilogues store under per-lane row conditions, which the
compiler lowers to regions with lanes switched off (an EXEC mask saved by
s_and_saveexec and restored by s_or_b64 exec). An MFMA reads the operands of every
lane of the wave, so an MFMA moved into such a region computes with the operands of
switched-off lanes missing, and a tile whose last 32-row block is partly filled
gets wrong columns. This compiles the GEMM sources as the library build does and
checks that no MFMA can be reached inside such a region."""
import os
import re
import shutil
import subprocess

import pytest

from mixture_experts_expert_softmax_amd import _build

SOURCES = ["gemm_bf16.hip", "gemm_mx.hip", "bgmv.hip"]   # every MFMA kernel of the library


def _functions(asm: str):
    """(name, instruction lines) of every kernel in the assembly."""
    fns, name, body = [], None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            if name:
                fns.append((name, body))
            name, body = m.group(1), []
        elif name:
            if line.startswith(".Lfunc_end"):
                fns.append((name, body))
                name, body = None, []
            else:
                body.append(line)
    if name:
        fns.append((name, body))
    return fns


def _masked_mfmas(asm: str):
    """(function, count) of MFMAs reachable from an EXEC save before its restore.

    The control flow is followed instruction by instruction: fall-through, and the
    targets of s_branch / s_cbranch_*. From every s_and_saveexec the search runs until
    an s_or_b64 exec, exec (the restore) and reports every v_mfma it meets on the way.
    (A plain scan of the text in file order is not enough: the compiler places a
    loop's restore at a label above its saveexec and the blocks after it may belong to
    other code.)"""
    bad = []
    for fn, lines in _functions(asm):
        labels = {}
        ins = []
        for line in lines:
            m = re.match(r"^(\.LBB\w+):", line)
            if m:
                labels[m.group(1)] = len(ins)
                continue
            t = line.split(";")[0].strip()
            if t and not t.startswith("."):
                ins.append(t)

        def succ(i):
            t = ins[i]
            m = re.match(r"s_branch\s+(\.LBB\w+)", t)
            if m:
                return [labels[m.group(1)]]
            if t.startswith("s_endpgm") or t.startswith("s_setpc"):
                return []
            m = re.match(r"s_cbranch_\w+\s+(\.LBB\w+)", t)
            nxt = [i + 1] if i + 1 < len(ins) else []
            return nxt + [labels[m.group(1)]] if m else nxt

        hit = set()
        for i, t in enumerate(ins):
            if "s_and_saveexec" not in t:
                continue
            seen, todo = set(), list(succ(i))
            while todo:
                j = todo.pop()
                if j in seen:
                    continue
                seen.add(j)
                if re.match(r"s_or_b64\s+exec, exec", ins[j]):
                    continue
                if ins[j].startswith("v_mfma"):
                    hit.add(j)
                todo.extend(succ(j))
        if hit:
            bad.append((fn, len(hit)))
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


_SYNTH = """\
_Zpos:
\ts_and_saveexec_b64 s[4:5], vcc
\ts_cbranch_execz .LBB0_2
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
.LBB0_2:
\ts_or_b64 exec, exec, s[4:5]
\ts_endpgm
.Lfunc_end0:
_Zjump:
\ts_and_saveexec_b64 s[4:5], vcc
\ts_cbranch_execz .LBB1_3
\ts_branch .LBB1_9
.LBB1_3:
\ts_or_b64 exec, exec, s[4:5]
\ts_endpgm
.LBB1_9:
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
\ts_branch .LBB1_3
.Lfunc_end1:
_Zloop:
\ts_branch .LBB2_4
.LBB2_1:
\ts_or_b64 exec, exec, s[4:5]
\ts_cmp_lt_i32 s0, s1
\ts_cbranch_scc0 .LBB2_5
.LBB2_4:
\ts_and_saveexec_b64 s[4:5], vcc
\ts_cbranch_execz .LBB2_1
\tglobal_store_dwordx4 v[0:1], v[2:5], off
\ts_branch .LBB2_1
.LBB2_5:
\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]
\ts_endpgm
.Lfunc_end2:
"""


def test_masked_mfma_checker_on_synthetic_code():
    """The checker itself: an MFMA inside a masked if, and one reached by a jump out of a
    masked region before its restore, are found; an MFMA placed after a loop whose
    restore sits at a label above the loop's saveexec is not."""
    assert dict(_masked_mfmas(_SYNTH)) == {"_Zpos": 1, "_Zjump": 1}
