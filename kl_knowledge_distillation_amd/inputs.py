"""Seeded synthetic inputs for the distillation-loss workloads.

This module is shared by the tests, the benchmark and the oracle checks. It
holds shapes, distributions and random draws only: none of the loss arithmetic.

Every tensor is drawn in float32 from its own seeded generator and then stored
in the workload dtype (bf16 round-to-nearest-even, or fp32). Consumers read the
*stored* values; the float32 draws are never used directly. Large tensors are
drawn on the device in row slices, so a host copy of tens of GB is never made.

Workloads (shapes from the pages, distributions as stated):
  tiny_tied_fp32        N=64,    D=128,  V=1024,   fp32, tied teacher, T=2
  quickstart_tied_bf16  N=4096,  D=2048, V=32000,  bf16, tied teacher, T=2
                        (orda-kernel, Quickstart: bt, hidden, vocab)
  separate_bf16         N=8192,  D=2048, D_t=4096, V=128256, separate teacher
  topk_bf16             N=32768, D=4096, V=151936, K=100 cached top-K teacher
                        (Full-Chunked-KL-Loss, Quick start: sequence 32768,
                        --topk 100, batch 1)
  scorer_bf16           N=65536, D_t=4096, V=248320, student logits given,
                        forward only (flash_kd: vocab ~248k)
  kdloss_logits_bf16    N=4096, V=32000, student and teacher logits both given,
                        N(0, 4) each, T=2, KL only (nemo kd_loss, KDLoss.forward)
  quickstart_logits_bf16  the quickstart shape with a cached dense teacher
                        (orda-kernel, Teacher descriptors: PrecomputedTeacher
                        logits) of N(0,1) logits, the per-entry variance of
                        the projected quickstart teacher, T_s = 2, T_t = 1.5
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    n: int
    d: int
    v: int
    d_t: int = 0
    dtype: str = "bf16"            # "bf16" | "fp32"
    teacher: str = "tied"          # "tied" | "separate" | "topk" | "logits"
    student: str = "projection"    # "projection" | "logits"
    temperature: float = 1.0
    student_ce_weight: float = 1.0
    teacher_ce_weight: float = 0.0
    kl_weight: float = 1.0
    kl_divergence: str = "forward"  # "forward" | "reverse" | "jeffreys"
    teacher_temperature: Optional[float] = None  # None: the student temperature
    compact_valid: bool = False    # rows with an ignored label left out of the projections
    ignore_index: int = -100
    ignore_frac: float = 0.0
    k: int = 0
    student_hidden_std: float = 1.0
    teacher_hidden_std: float = 1.0
    logits_var: float = 0.0
    teacher_logits_var: float = 1.0   # dense teacher logits ~ N(0, var)
    teacher_neg_inf_frac: float = 0.0  # vocabulary columns whose teacher logit is -inf
    forward_only: bool = False
    has_labels: bool = True

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def teacher_dim(self) -> int:
        return self.d_t if self.teacher == "separate" else self.d

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny_tied_fp32": Workload(
        "tiny_tied_fp32", n=64, d=128, v=1024, dtype="fp32", teacher="tied",
        temperature=2.0, student_ce_weight=1.0, kl_weight=1.0, ignore_frac=0.10),
    "quickstart_tied_bf16": Workload(
        "quickstart_tied_bf16", n=4096, d=2048, v=32000, teacher="tied",
        temperature=2.0, student_ce_weight=1.0, kl_weight=1.0, ignore_frac=0.05),
    "separate_bf16": Workload(
        "separate_bf16", n=8192, d=2048, d_t=4096, v=128256, teacher="separate",
        temperature=1.0, student_ce_weight=1.0, teacher_ce_weight=1.0, kl_weight=1.0,
        teacher_hidden_std=1.5),
    "topk_bf16": Workload(
        "topk_bf16", n=32768, d=4096, v=151936, teacher="topk", k=100,
        temperature=1.0, student_ce_weight=0.0, kl_weight=1.0, has_labels=False),
    "scorer_bf16": Workload(
        "scorer_bf16", n=65536, d=0, d_t=4096, v=248320, teacher="separate",
        student="logits", temperature=1.0, student_ce_weight=1.0, kl_weight=1.0,
        ignore_index=-1, ignore_frac=0.03, logits_var=2.0, forward_only=True),
    "kdloss_logits_bf16": Workload(
        "kdloss_logits_bf16", n=4096, d=0, v=32000, teacher="logits", student="logits",
        temperature=2.0, student_ce_weight=0.0, kl_weight=1.0, ignore_frac=0.05,
        logits_var=4.0, teacher_logits_var=4.0, forward_only=True),
    "quickstart_logits_bf16": Workload(
        "quickstart_logits_bf16", n=4096, d=2048, v=32000, teacher="logits",
        temperature=2.0, teacher_temperature=1.5, student_ce_weight=1.0, kl_weight=1.0,
        ignore_frac=0.05),
}

# One generator stream per named tensor (seed 0 by default).
_STREAM = {"student_hidden": 1, "weight": 2, "teacher_hidden": 3, "teacher_weight": 4,
           "labels": 5, "ignore": 6, "topk": 7, "student_logits": 8, "teacher_logits": 9,
           "teacher_mask": 10}

_SLICE_ELEMS = 1 << 28  # rows are drawn in slices of at most this many elements


def _gen(device: torch.device, seed: int, name: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + _STREAM[name])
    return g


def _normal(shape, std: float, dtype: torch.dtype, device, seed: int, name: str) -> torch.Tensor:
    """Rows of N(0, std^2) drawn in fp32 slice by slice, stored in ``dtype``."""
    g = _gen(device, seed, name)
    rows, cols = shape
    out = torch.empty(shape, dtype=dtype, device=device)
    step = max(1, _SLICE_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = torch.randn((r1 - r0, cols), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[r0:r1] = x.to(dtype)
        del x
    return out


def make_labels(n: int, v: int, ignore_index: int, ignore_frac: float, seed: int = 0) -> torch.Tensor:
    """int64 labels uniform in [0, v); exactly round(frac*n) rows set to ignore_index.

    The ignored rows are the first round(frac*n) positions of a seeded permutation.
    """
    g = _gen(torch.device("cpu"), seed, "labels")
    y = torch.randint(0, v, (n,), generator=g, dtype=torch.int64)
    k = int(round(ignore_frac * n))
    if k:
        gi = _gen(torch.device("cpu"), seed, "ignore")
        rows = torch.randperm(n, generator=gi)[:k]
        y[rows] = ignore_index
    return y


def make_topk(n: int, v: int, k: int, seed: int = 0):
    """Cached sparse teacher: per row k distinct indices and their probabilities.

    Indices are uniform without replacement over [0, v) (int32). Probabilities
    are M * Dirichlet(0.1 * 1_k) with M ~ U(0.85, 0.99), stored in fp32 and not
    renormalised after rounding. With k^2 <= v rows with a repeated index are
    redrawn; beyond that (where a row without repeats is rare) each row is the
    first k of a random permutation of [0, v).
    """
    rng = np.random.Generator(np.random.PCG64(seed * 1000 + _STREAM["topk"]))
    if k * k > v:
        idx = np.argsort(rng.random((n, v)), axis=1)[:, :k].astype(np.int64)
    else:
        idx = rng.integers(0, v, size=(n, k), dtype=np.int64)
        while True:
            s = np.sort(idx, axis=1)
            dup = (s[:, 1:] == s[:, :-1]).any(axis=1) if k > 1 else np.zeros(n, bool)
            bad = np.nonzero(dup)[0]
            if bad.size == 0:
                break
            idx[bad] = rng.integers(0, v, size=(bad.size, k), dtype=np.int64)
    gam = rng.gamma(0.1, 1.0, size=(n, k))
    tot = gam.sum(axis=1, keepdims=True)
    tot[tot == 0] = 1.0
    mass = rng.uniform(0.85, 0.99, size=(n, 1))
    prob = (mass * gam / tot).astype(np.float32)
    return torch.from_numpy(idx.astype(np.int32)), torch.from_numpy(prob)


def make_inputs(w: Workload, device="cpu", seed: int = 0) -> Dict[str, Optional[torch.Tensor]]:
    """All tensors of one workload instance, on ``device``.

    Keys: student_hidden, weight, student_logits, teacher_hidden, teacher_weight,
    teacher_logits, labels, topk_idx, topk_prob (absent ones are None).

    Dense teacher logits: N(0, teacher_logits_var); with teacher_neg_inf_frac > 0
    the first round(frac * v) columns of a seeded permutation are -inf in every
    row, as a teacher projected from another vocabulary leaves its unmatched
    columns (orda-kernel, Cross-vocabulary distillation).
    """
    device = torch.device(device)
    dt = w.torch_dtype
    out: Dict[str, Optional[torch.Tensor]] = dict.fromkeys(
        ["student_hidden", "weight", "student_logits", "teacher_hidden", "teacher_weight",
         "teacher_logits", "labels", "topk_idx", "topk_prob"])
    if w.student == "projection":
        out["student_hidden"] = _normal((w.n, w.d), w.student_hidden_std, dt, device, seed,
                                        "student_hidden")
        out["weight"] = _normal((w.v, w.d), 1.0 / math.sqrt(w.d), dt, device, seed, "weight")
    else:
        out["student_logits"] = _normal((w.n, w.v), math.sqrt(w.logits_var), dt, device, seed,
                                        "student_logits")
    if w.teacher in ("tied", "separate"):
        out["teacher_hidden"] = _normal((w.n, w.teacher_dim), w.teacher_hidden_std, dt, device,
                                        seed, "teacher_hidden")
    if w.teacher == "separate":
        out["teacher_weight"] = _normal((w.v, w.d_t), 1.0 / math.sqrt(w.d_t), dt, device, seed,
                                        "teacher_weight")
    if w.teacher == "logits":
        tl = _normal((w.n, w.v), math.sqrt(w.teacher_logits_var), dt, device, seed,
                     "teacher_logits")
        k = int(round(w.teacher_neg_inf_frac * w.v))
        if k:
            cols = torch.randperm(w.v, generator=_gen(torch.device("cpu"), seed, "teacher_mask"))[:k]
            tl[:, cols.to(device)] = float("-inf")
        out["teacher_logits"] = tl
    if w.teacher == "topk":
        idx, prob = make_topk(w.n, w.v, w.k, seed)
        out["topk_idx"] = idx.to(device)
        out["topk_prob"] = prob.to(device)
    if w.has_labels:
        out["labels"] = make_labels(w.n, w.v, w.ignore_index, w.ignore_frac, seed).to(device)
    return out
