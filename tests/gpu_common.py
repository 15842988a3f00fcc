"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the float64 oracle on the same stored inputs, compare at the stated bar.

Tolerances (one rule per quantity):
  per-token values  |g - o| <= rtol * max(|o|, 1e-2)   rtol 1e-3 bf16, 1e-5 fp32
  scalar loss       |g - o| <= rtol * |o|
  dH, dW            ||g - o||_inf / ||o||_inf <= 2e-2 bf16, 1e-5 fp32
"""
from __future__ import annotations

import sys
from typing import Optional

import numpy as np
import torch

import oracle as O
from kl_knowledge_distillation_amd.api import Runner
from kl_knowledge_distillation_amd.inputs import Workload, make_inputs

TOK_RTOL = {"bf16": 1e-3, "fp32": 1e-5}
GRAD_RTOL = {"bf16": 2e-2, "fp32": 1e-5}
TOK_FLOOR = 1e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_np(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def params_of(w: Workload) -> O.Params:
    return O.Params(student_ce_weight=w.student_ce_weight, teacher_ce_weight=w.teacher_ce_weight,
                    kl_weight=w.kl_weight, temperature=w.temperature, ignore_index=w.ignore_index,
                    kl_divergence=w.kl_divergence, teacher_temperature=w.teacher_temperature,
                    compact_valid=w.compact_valid)


def oracle_problem(w: Workload, x: dict, rows=None):
    """Oracle descriptors from the stored tensors (float64, exact)."""
    def f64(t, r=None):
        if t is None:
            return None
        if r is not None:
            t = t[torch.as_tensor(r, device=t.device)]
        return to_np(t).astype(np.float64)
    if w.student == "logits":
        s = O.Student(logits=f64(x["student_logits"], rows))
    else:
        s = O.Student(hidden=f64(x["student_hidden"]), weight=f64(x["weight"]))
    if w.teacher == "tied":
        t = O.Teacher("tied", hidden=f64(x["teacher_hidden"]))
    elif w.teacher == "separate":
        t = O.Teacher("separate", hidden=f64(x["teacher_hidden"], rows) if w.student == "logits"
                      else f64(x["teacher_hidden"]), weight=f64(x["teacher_weight"]))
    elif w.teacher == "logits":
        t = O.Teacher("logits", logits=f64(x["teacher_logits"]))
    else:
        t = O.Teacher("topk", idx=to_np(x["topk_idx"]).astype(np.int64),
                      prob=to_np(x["topk_prob"]).astype(np.float64))
    labels = None if x["labels"] is None else to_np(x["labels"]).astype(np.int64)
    if labels is not None and rows is not None and w.student == "logits":
        labels = labels[np.asarray(rows)]
    return s, t, labels


def make_runner(w: Workload, x: dict, vocab_chunk: int = 0, reduction: str = "mean",
                want_grads: Optional[bool] = None,
                want_teacher_ce: Optional[bool] = None,
                keep_last_chunk: Optional[bool] = None, grad_dtype=torch.float32) -> Runner:
    kw = dict(labels=x["labels"], student_ce_weight=w.student_ce_weight,
              teacher_ce_weight=w.teacher_ce_weight, kl_weight=w.kl_weight,
              temperature=w.temperature, ignore_index=w.ignore_index, reduction=reduction,
              vocab_chunk=vocab_chunk,
              want_grads=(not w.forward_only) if want_grads is None else want_grads,
              want_teacher_ce=want_teacher_ce, kl_divergence=w.kl_divergence,
              teacher_temperature=w.teacher_temperature, compact_valid=w.compact_valid,
              keep_last_chunk=keep_last_chunk, grad_dtype=grad_dtype)
    if w.student == "logits":
        kw["student_logits"] = x["student_logits"]
    else:
        kw["student_hidden"] = x["student_hidden"]
        kw["weight"] = x["weight"]
    if w.teacher == "tied":
        kw.update(teacher_kind="tied", teacher_hidden=x["teacher_hidden"])
    elif w.teacher == "separate":
        kw.update(teacher_kind="separate", teacher_hidden=x["teacher_hidden"],
                  teacher_weight=x["teacher_weight"])
    elif w.teacher == "logits":
        kw.update(teacher_kind="logits", teacher_logits=x["teacher_logits"])
    else:
        kw.update(teacher_kind="topk", topk_idx=x["topk_idx"], topk_prob=x["topk_prob"])
    return Runner(**kw)


def run_gpu(w: Workload, x: dict, vocab_chunk: int = 0, grads: bool = True):
    r = make_runner(w, x, vocab_chunk)
    r.forward()
    dh = dw = None
    if grads and not w.forward_only:
        dh = torch.empty((r.n, r.d), dtype=torch.float32, device=r.device)
        dw = torch.empty((r.v, r.d), dtype=torch.float32, device=r.device)
        r.backward(dh, dw)
    torch.cuda.synchronize()
    return r, dh, dw


def assert_tokens(g, o, dtype: str, what: str, mask=None):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    if mask is not None:
        g, o = g[mask], o[mask]
    rtol = TOK_RTOL[dtype]
    err = np.abs(g - o)
    bound = rtol * np.maximum(np.abs(o), TOK_FLOOR)
    bad = err > bound
    if bad.any():
        j = int(np.argmax(err / bound))
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{g.size} outside tolerance; worst at {j}: gpu={g[j]!r} "
            f"oracle={o[j]!r} err={err[j]:.3e} bound={bound[j]:.3e}")


def assert_scalar(g: float, o: float, dtype: str, what: str):
    rtol = TOK_RTOL[dtype]
    assert abs(g - o) <= rtol * max(abs(o), 1e-30), f"{what}: gpu={g!r} oracle={o!r}"


def assert_grad(g, o, dtype: str, what: str):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    scale = np.max(np.abs(o))
    err = np.max(np.abs(g - o))
    rel = err / scale if scale > 0 else err
    assert rel <= GRAD_RTOL[dtype], f"{what}: max-norm relative error {rel:.3e} (scale {scale:.3e})"


def full_parity(w: Workload, vocab_chunk: int = 0, seed: int = 0, grads: bool = True):
    """Every output of the HIP path against the oracle on the whole problem."""
    say(f"[parity] {w.name} n={w.n} d={w.d} d_t={w.d_t} v={w.v} chunk={vocab_chunk} seed={seed}")
    x = make_inputs(w, "cuda", seed)
    r, dh, dw = run_gpu(w, x, vocab_chunk, grads)
    s, t, labels = oracle_problem(w, x)
    p = params_of(w)
    ref = O.forward(s, t, p, labels)
    assert r.read_status() == 0
    assert_tokens(to_np(r.kl), ref["kl"], w.dtype, f"{w.name} kl")
    if labels is not None:
        assert_tokens(to_np(r.student_ce), ref["student_ce"], w.dtype, f"{w.name} student_ce")
        if w.teacher_ce_weight > 0:
            assert_tokens(to_np(r.teacher_ce), ref["teacher_ce"], w.dtype, f"{w.name} teacher_ce")
    assert_scalar(float(r.loss), ref["loss"], w.dtype, f"{w.name} loss")
    if dh is not None:
        dH, dW = O.backward(s, t, p, labels)
        assert_grad(to_np(dh), dH, w.dtype, f"{w.name} dH")
        assert_grad(to_np(dw), dW, w.dtype, f"{w.name} dW")
    return r, x
