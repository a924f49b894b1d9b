"""The LM-head kernel's MFMAs are inline assembly (accumulators pinned to AGPRs),
so the compiler's hazard recognizer does not see them.  This CPU test compiles the
kernel for gfx950 and checks the generated code: no instruction reads or writes an
accumulator register within the wait-state window after an MFMA that wrote or read
it, and no MFMA reads an accumulator as its C operand right after an ordinary
instruction wrote it."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "draft_token_verification_online_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
KERNEL = "_ZN2sv14lm_head_kernelENS_6LmArgsE"
AFTER_MFMA = 20     # instructions after an MFMA in which its AGPRs are not touched
BEFORE_SRC_C = 4    # instructions after an AGPR write before an MFMA may read it


def _agprs(spec):
    m = re.fullmatch(r"a\[(\d+):(\d+)\]", spec)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.fullmatch(r"a(\d+)", spec)
    return {int(m.group(1))} if m else set()


@pytest.fixture(scope="module")
def lm_asm(tmp_path_factory):
    if not os.path.exists(HIPCC) and not shutil.which("hipcc"):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("lmasm")
    src = d / "lm.hip"
    src.write_text('#include <hip/hip_runtime.h>\n#include "sv_lmhead.hpp"\n')
    out = d / "lm.s"
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17",
                           "-mcode-object-version=5", "-Xclang", "-target-feature", "-Xclang",
                           "-packed-fp32-ops", "--cuda-device-only", "-S", f"-I{CSRC}",
                           "-o", str(out), str(src)], stderr=subprocess.DEVNULL)
    text = out.read_text()
    i = text.index(KERNEL + ":")
    j = text.index(".Lfunc_end", i)
    return [l.strip() for l in text[i:j].splitlines()
            if l.strip() and not l.strip().startswith((";", "."))]


def test_lm_head_uses_mfma_with_agpr_accumulators(lm_asm):
    mfma = [l for l in lm_asm if l.startswith("v_mfma_f32_16x16x32_bf16")]
    assert len(mfma) >= 128
    assert all(re.match(r"v_mfma_f32_16x16x32_bf16 a\[\d+:\d+\], v\[", l) for l in mfma)


def test_no_accumulator_hazards_around_inline_mfma(lm_asm):
    recent = []   # (index, kind, agprs written, agprs read)
    bad = []
    for n, line in enumerate(lm_asm):
        op = line.split()[0]
        ops = [x.strip() for x in line[len(op):].split(",")]
        if op.startswith("v_mfma"):
            dst, src_c = _agprs(ops[0]), _agprs(ops[3])
            for m, kind, w, r in recent:
                if kind == "write" and n - m <= BEFORE_SRC_C and src_c & w:
                    bad.append((lm_asm[m], line))
            recent.append((n, "mfma", dst, src_c))
        elif any(a.startswith("a") for a in ops) or op.startswith("v_accvgpr"):
            touched = set().union(*[_agprs(a) for a in ops]) if ops else set()
            for m, kind, w, r in recent:
                if kind == "mfma" and n - m <= AFTER_MFMA and touched & (w | r):
                    bad.append((lm_asm[m], line))
            recent.append((n, "write", _agprs(ops[0]) if ops else set(), set()))
        recent = [x for x in recent if n - x[0] <= AFTER_MFMA]
    assert not bad, bad[:5]
