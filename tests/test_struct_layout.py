"""The ctypes mirrors of the C descriptors have the header's exact layout.

A C program built here with gcc from include/kd_loss.h prints sizeof and the
offset of every field; each must equal what ctypes computes, so a field added
to one side and not the other (or in another order) fails here, not on a GPU.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

from kl_knowledge_distillation_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STRUCTS = {"kd_student": L.KdStudent, "kd_teacher": L.KdTeacher, "kd_params": L.KdParams,
           "kd_outputs": L.KdOutputs, "kd_trace": L.KdTrace}


def _c_layout(tmp_path):
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "kd_loss.h"', 'int main(void) {']
    for cname, cls in STRUCTS.items():
        lines.append(f'  printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f in cls._fields_:
            lines.append(f'  printf("{cname} {f[0]} %zu\\n", offsetof({cname}, {f[0]}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    return {tuple(l.split()[:2]): int(l.split()[2]) for l in out.splitlines()}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_ctypes_structs_match_the_header(tmp_path):
    c = _c_layout(tmp_path)
    for cname, cls in STRUCTS.items():
        assert c[(cname, "sizeof")] == ctypes.sizeof(cls), cname
        for f in cls._fields_:
            assert c[(cname, f[0])] == getattr(cls, f[0]).offset, f"{cname}.{f[0]}"
