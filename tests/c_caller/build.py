"""Build the plain C++ caller of the C ABI (kd_c_caller.cpp) next to its source.

It links the in-tree libkdloss.so (found at run time through an rpath relative
to the binary), so build the library first.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "kl_knowledge_distillation_amd")
BIN = os.path.join(HERE, "kd_c_caller")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build(verbose: bool = False) -> str:
    rpath = os.path.relpath(PKG, HERE)
    cmd = [HIPCC, "-O2", "-std=c++17", "-Wall", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(HERE, "kd_c_caller.cpp"), f"-L{PKG}", "-lkdloss",
           f"-Wl,-rpath,$ORIGIN/{rpath}", "-o", BIN + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"building the C caller failed:\n{r.stderr}")
    os.replace(BIN + ".tmp", BIN)
    if verbose:
        print(f"built {BIN}")
    return BIN


if __name__ == "__main__":
    build(verbose=True)
