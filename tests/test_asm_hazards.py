"""CPU check of the compiled GEMM kernels (no GPU): every matrix instruction
written as inline assembly (the in-place accumulating form, mfma16_tied in
lb_device.h) must take its A and B operands straight from memory loads.  The
compiler inserts no wait states for such an instruction, so an operand that a
vector ALU instruction wrote just before (a select that zeroes a step, a
register copy) could be read stale.  The test compiles k_gemm.hip to gfx950
assembly with the library's flags and scans every loop that holds an inline
MFMA: between the last load into each operand register and the MFMA there
must be no vector ALU write to it."""
import os
import re
import subprocess

import pytest

from decoder_only_transformer_amd import build as lib_build


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _violations(asm_text):
    lines = asm_text.split("\n")
    bad, loops, kern, i = [], 0, None, 0
    while i < len(lines):
        m = re.match(r"^(_Z\w+):", lines[i])
        if m:
            kern = m.group(1)
        m = re.match(r"^(\.LBB\w+):.*Loop Header", lines[i])
        if m:
            lab, j = m.group(1), i + 1
            while j < len(lines) and not re.search(r"(s_cbranch_\w+|s_branch) " + re.escape(lab) + r"\b", lines[j]):
                if re.match(r"^_Z\w+:", lines[j]):
                    break
                j += 1
            body = lines[i:j + 1]
            if any("v_mfma" in x for x in body):
                loops += 1
                inasm, written = False, {}
                for x in body:
                    if "ASMSTART" in x:
                        inasm = True
                        continue
                    if "ASMEND" in x:
                        inasm = False
                        continue
                    t = x.split()
                    if not t:
                        continue
                    op = t[0]
                    if op.startswith(("ds_read", "global_load", "buffer_load")) and "_lds" not in op:
                        for r in _regs(t[1].strip(",")):
                            written.pop(r, None)
                        continue
                    if not op.startswith("v_") or op.startswith("v_accvgpr"):
                        continue
                    ops = [o.strip(",") for o in t[1:]]
                    if op.startswith("v_mfma"):
                        if inasm:
                            for o in ops[1:3]:
                                for r in _regs(o):
                                    if r in written:
                                        bad.append((kern, written[r].strip(), x.strip()))
                        continue
                    for r in _regs(ops[0]):
                        written[r] = x
        i += 1
    return loops, bad


@pytest.mark.timeout(900)
@pytest.mark.parametrize("src", ["k_gemm.hip", "k_moe.hip"])
def test_inline_mfma_operands_come_from_loads(tmp_path, src):
    """The dense prefill GEMMs (k_gemm.hip) and the grouped expert GEMMs
    (k_moe.hip) share the tile body with the inline-assembly MFMAs."""
    out = tmp_path / (src + ".s")
    cmd = [lib_build.HIPCC] + lib_build.FLAGS + ["-x", "hip", os.path.join(lib_build.CSRC, src),
                                                 "-S", "--cuda-device-only", "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    assert "ASMSTART" in text and "v_mfma" in text
    loops, bad = _violations(text)
    assert loops > 0
    assert not bad, bad[:5]


def test_scan_flags_a_select_feeding_an_inline_mfma():
    """The scan itself: a v_cndmask into an operand of an inline MFMA is
    flagged, the same operand refilled by an LDS read first is not."""
    base = """_Zk:
.LBB0_1:                                ; =>This Inner Loop Header: Depth=1
	ds_read_b128 v[10:13], v2
	{between}
	;;#ASMSTART
	v_mfma_f32_16x16x32_f16 a[0:3], v[10:13], v[20:23], a[0:3]
	;;#ASMEND
	s_cbranch_scc0 .LBB0_1
"""
    _, bad = _violations(base.format(between="v_cndmask_b32_e64 v11, 0, v11, s[4:5]"))
    assert len(bad) == 1
    _, bad = _violations(base.format(between="v_add_u32_e32 v2, 16, v2"))
    assert not bad
