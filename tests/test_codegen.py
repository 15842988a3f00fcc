"""Static checks of the kernels' generated gfx950 code (no GPU needed).

The pipelined main loop reads its row-contiguous fragments (the dW / dH GEMM
operands) with ds_read_b64_tr_b16 through inline asm: the compiler does not see
that instruction's latency, so its destination registers are valid only after
the loop's explicit s_waitcnt lgkmcnt(0). The check below compiles the kernels
to gfx950 assembly with the library's own flags and walks every kernel in
program order: no MFMA may read a register written by such a read before the
next lgkmcnt(0) wait. (A build in which the scheduler had moved MFMAs above
that wait gave wrong dH on the GPU.)
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

from kl_knowledge_distillation_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc is not installed")

_RANGE = re.compile(r"v\[(\d+):(\d+)\]$")
_ONE = re.compile(r"v(\d+)$")


def _vregs(operand: str) -> set:
    m = _RANGE.match(operand)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = _ONE.match(operand)
    return {int(m.group(1))} if m else set()


def _kernels(asm: str):
    """(name, instruction lines) of every kernel function in the listing."""
    lines = asm.split("\n")
    for i, line in enumerate(lines):
        m = re.match(r"^(_ZN2kd\S+):", line)
        if not m:
            continue
        body = []
        for rest in lines[i + 1:]:
            if rest.startswith(".Lfunc_end"):
                break
            body.append(rest.strip())
        yield m.group(1), body


def unwaited_uses(asm: str):
    """(kernel, MFMA line) for every MFMA that reads a transposed-read
    destination before an lgkmcnt(0) wait, and the number of transposed reads."""
    bad, reads = [], 0
    for name, body in _kernels(asm):
        pending = set()
        for s in body:
            if s.startswith("ds_read_b64_tr_b16"):
                reads += 1
                pending |= _vregs(s.split(None, 1)[1].split(",")[0].strip())
            elif s.startswith("s_waitcnt") and "lgkmcnt(0)" in s:
                pending.clear()
            elif s.startswith("v_mfma"):
                ops = [o.strip() for o in s.split(None, 1)[1].split(",")]
                if (_vregs(ops[1]) | _vregs(ops[2])) & pending:
                    bad.append((name, s))
    return bad, reads


def test_checker_flags_a_use_before_the_wait():
    planted = "\n".join([
        "_ZN2kd6sampleEv:",
        "\tds_read_b64_tr_b16 v[10:11], v2",
        "\tv_mfma_f32_16x16x32_bf16 v[0:3], v[8:11], v[20:23], v[0:3]",
        "\ts_waitcnt lgkmcnt(0)",
        "\tv_mfma_f32_16x16x32_bf16 v[4:7], v[8:11], v[20:23], v[4:7]",
        ".Lfunc_end0:",
    ])
    bad, reads = unwaited_uses(planted)
    assert reads == 1
    assert len(bad) == 1 and "v[0:3]" in bad[0][1]


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "kd_kernels.s"
    cmd = [B.HIPCC, *B.COMMON, "--cuda-device-only", "-S", os.path.join(B.CSRC, "kd_kernels.hip"),
           "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def test_transposed_reads_are_waited_for_before_any_mfma_uses_them(device_asm):
    bad, reads = unwaited_uses(device_asm)
    assert reads > 0, "no transposed reads found: the check would be vacuous"
    assert not bad, f"{len(bad)} MFMAs read a transposed-read register before its wait, e.g. {bad[:3]}"
