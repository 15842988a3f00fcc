"""Fused LM-head + cross-entropy + KL distillation loss for AMD MI355X (gfx950).

The compute path is the HIP library ``libkdloss.so`` behind the C ABI declared
in ``include/kd_loss.h``; this package is its thin Python binding. Importing the
package is cheap: the shared library is loaded on first use, and every entry
point raises if it is missing (there is no CPU fallback).
"""
from __future__ import annotations

__all__ = [
    "distillation_loss", "flash_ce_kd_loss", "DistillationLossOutput", "Runner", "Tracer",
    "TiedTeacher", "SeparateTeacher", "PrecomputedTeacher", "TopKTeacher",
    "DistillationLoss", "KDLoss", "is_available", "lib",
]


def __getattr__(name):
    if name in __all__:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
