"""Float64 CPU oracle for the fused LM-head + cross-entropy + KL distillation loss.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
this module: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` use it. It shares no code with the HIP library and does not
import it.

The oracle reaches every result by its plain definition. It materialises the
full-vocabulary logits of each row block in float64, computes log-sum-exp over
all V columns at once, and forms the gradients of the logits in closed form
before contracting them with the inputs. It never streams over vocabulary
chunks: the flash_kd page (module description) states that the online-softmax
stream is numerically identical to the full computation, so the full
computation is the reference.

Inputs are the *stored* values (bf16 or fp32 tensors converted to float64,
which is exact). Arrays are NumPy; callers convert torch tensors first.

Sources (page title, then section):
  * orda-kernel (PyPI page): Quickstart, Teacher descriptors, Parameters.
  * flash_kd (Model-Optimizer API page): flash_ce_kd_loss, Parameters/Returns.
  * CompactifAI/Full-Chunked-KL-Loss (README): Methods, objective; Full Dense
    KL; Full Chunked KL.
  * nemo_automodel.components.loss.kd_loss (NeMo AutoModel API page): KDLoss
    parameters (temperature) and KDLoss.forward (num_batch_labels).

Readings of points the pages leave open (each is also listed in the design doc):
  R1  cross-entropy is always at temperature 1; T applies to the KL term only.
  R2  the per-token KL output includes the T**2 factor.
  R3  the per-token KL is reported for every row; loss and gradients exclude
      rows whose label is ignored; per-token CE is 0 on ignored rows.
  R4  an all-ignored batch divides by max(n_valid, 1): loss 0, gradients 0.
  R6  a frozen teacher's CE enters the loss value but gives no gradient. A
      teacher trained through its CE (orda-kernel, Teacher descriptors: the
      role follows the weights; teacher_ce_weight > 0 trains via CE) gets the
      gradient of w_t * CE(t) only: every KL variant here detaches the teacher
      (orda-kernel, KL variants), so the KL gives the teacher nothing. With a
      tied teacher the shared weight receives both halves.
  R7  top-K indices are int32, probabilities fp32; M is the sum of the stored p.
  R8  0 * log 0 = 0 in the teacher-entropy term.
  R10 top-K mode has no labels: every row is valid, there is no CE.
  R17 "reverse" KL(P_S || P_T) and "jeffreys" KL(P_T || P_S) + KL(P_S || P_T)
      take the same 1/T on both logits and the same T**2 factor as "forward".
  R18 the cached top-K teacher supports "forward" only (its distribution is
      zero off the support, so KL(P_S || P_T) is not finite).
  R19 with a teacher temperature T_t apart from the student's T_s, the teacher
      distribution is softmax(t / T_t), the student's softmax(z / T_s), and
      every KL direction is scaled by T_s**2.
  R20 a teacher logit of -inf (a cached or projected teacher with no mass on a
      column) is a zero teacher probability: its forward-KL term is 0, its
      reverse-KL term (with a nonzero student probability) is +inf.
  R21 a loss term whose weight is 0 is absent from the loss, not 0 times its
      value (which may be infinite, e.g. the teacher CE of R20's columns).
  R22 with compact_valid the rows whose label is ignored are excluded from the
      KL too (orda-kernel, Parameters: ignore_index is excluded from CE and
      KL; nemo kd_loss: only valid tokens are processed): their per-token KL
      is 0. Without it the KL is reported for every row (R3).
  --  a label outside [0, V) that is not ignore_index is treated as ignored.

Parity pins for every function live in tests/test_oracle.py (closed forms,
library cross-checks, invariants, finite differences). No function here is
parity unpinned.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

F64 = np.float64

# Rows per block when materialising (rows, V) float64 logits.
ROW_BLOCK = 256


@dataclass
class Params:
    """Loss configuration.

    Term weights and temperature follow orda-kernel, Parameters
    (student_ce_weight / teacher_ce_weight / kl_weight, kl_temperature);
    reduction and num_batch_labels follow nemo kd_loss, KDLoss.forward.
    ``normalizer > 0`` plays the role of num_batch_labels.
    """

    student_ce_weight: float = 1.0
    teacher_ce_weight: float = 0.0
    kl_weight: float = 0.0
    temperature: float = 1.0
    ignore_index: int = -100
    reduction: str = "mean"  # "mean" | "sum"
    normalizer: float = 0.0
    kl_divergence: str = "forward"  # "forward" | "reverse" | "jeffreys"
    # orda-kernel, Parameters (kl_teacher_temperature): None means T_s.
    teacher_temperature: Optional[float] = None
    # Rows whose label is ignored are left out of the per-token KL as well
    # (reading R22); the loss and the gradients do not change.
    compact_valid: bool = False


def teacher_temperature(p: Params) -> float:
    """T_t: the teacher's own temperature, or the student's when unset."""
    return p.temperature if p.teacher_temperature is None else p.teacher_temperature


# ---------------------------------------------------------------------------
# Elementary definitions
# ---------------------------------------------------------------------------

def as_f64(x) -> np.ndarray:
    """Exact conversion of stored values to float64."""
    return np.asarray(x, dtype=F64)


def project(hidden, weight) -> np.ndarray:
    """Logits of an LM head with no bias: hidden @ weight.T.

    orda-kernel, Quickstart: weight has shape (vocab, hidden); flash_kd,
    flash_ce_kd_loss: teacher logits are teacher_hidden @ weight[chunk].T.
    """
    return as_f64(hidden) @ as_f64(weight).T


def logsumexp(x: np.ndarray) -> np.ndarray:
    """log sum_v exp(x_v) over the last axis, shifted by the row maximum."""
    m = x.max(axis=-1)
    return m + np.log(np.exp(x - m[..., None]).sum(axis=-1))


def log_softmax(x: np.ndarray) -> np.ndarray:
    return x - logsumexp(x)[..., None]


def softmax(x: np.ndarray) -> np.ndarray:
    return np.exp(log_softmax(x))


def valid_mask(labels, vocab: int, ignore_index: int) -> np.ndarray:
    """Rows that carry a usable label.

    orda-kernel, Parameters (ignore_index): the ignored value is excluded from
    CE and KL and is never used as a memory index. A value outside [0, vocab)
    is treated like ignore_index (the library also raises a status flag).
    """
    y = np.asarray(labels, dtype=np.int64)
    return (y != ignore_index) & (y >= 0) & (y < vocab)


# ---------------------------------------------------------------------------
# Per-token terms
# ---------------------------------------------------------------------------

def cross_entropy(logits: np.ndarray, labels, valid: np.ndarray) -> np.ndarray:
    """Per-token CE at temperature 1: lse(x) - x[y]; 0 on ignored rows.

    flash_kd, flash_ce_kd_loss Parameters (labels): ignored entries get CE 0,
    as F.cross_entropy(reduction="none") does; Returns: standard CE.
    """
    y = np.where(valid, np.asarray(labels, dtype=np.int64), 0)
    picked = np.take_along_axis(logits, y[:, None], axis=1)[:, 0]
    return np.where(valid, logsumexp(logits) - picked, 0.0)


def forward_kl(student_logits: np.ndarray, teacher_logits: np.ndarray, T: float,
               Tt: Optional[float] = None) -> np.ndarray:
    """Per-token T**2 * KL(P_T || P_S), P_S = softmax(z / T), P_T = softmax(t / Tt).

    nemo kd_loss, KDLoss (temperature): both logits are divided by T and the
    loss is multiplied by T**2; orda-kernel, KL variants: "forward" is
    KL(teacher || student); orda-kernel, Parameters: the teacher temperature
    defaults to the student's and each row scales by T_s**2 (reading R19).
    Reported for every row (reading R3). A zero teacher probability adds 0
    (reading R20).
    """
    Tt = T if Tt is None else Tt
    lp_s = log_softmax(student_logits / T)
    lp_t = log_softmax(teacher_logits / Tt)
    q = np.exp(lp_t)
    return (T * T) * (q * np.where(q > 0, lp_t - lp_s, 0.0)).sum(axis=-1)


def reverse_kl(student_logits: np.ndarray, teacher_logits: np.ndarray, T: float,
               Tt: Optional[float] = None) -> np.ndarray:
    """Per-token T**2 * KL(P_S || P_T), P_S = softmax(z / T), P_T = softmax(t / Tt).

    orda-kernel, KL variants: p = student, q = teacher, "reverse" is KL(p || q);
    the temperature convention is the forward one (readings R17, R19).
    """
    Tt = T if Tt is None else Tt
    lp_s = log_softmax(student_logits / T)
    lp_t = log_softmax(teacher_logits / Tt)
    return (T * T) * (np.exp(lp_s) * (lp_s - lp_t)).sum(axis=-1)


def kl_term(student_logits: np.ndarray, teacher_logits: np.ndarray, T: float,
            variant: str = "forward", Tt: Optional[float] = None) -> np.ndarray:
    """The per-token KL of the selected variant (orda-kernel, KL variants):
    forward KL(q || p), reverse KL(p || q), jeffreys KL(q || p) + KL(p || q)."""
    if variant == "forward":
        return forward_kl(student_logits, teacher_logits, T, Tt)
    if variant == "reverse":
        return reverse_kl(student_logits, teacher_logits, T, Tt)
    if variant == "jeffreys":
        return (forward_kl(student_logits, teacher_logits, T, Tt)
                + reverse_kl(student_logits, teacher_logits, T, Tt))
    raise ValueError(f"unknown kl_divergence {variant!r}")


def topk_kl(student_logits: np.ndarray, idx, prob) -> np.ndarray:
    """Sparse forward KL against cached top-K teacher probabilities.

    CompactifAI/Full-Chunked-KL-Loss, Methods (objective): with support S,
    retained mass M = sum_S p (not renormalised) and student logits z,
        L = sum_S p log p - sum_S p z + M * logsumexp(z).
    0 * log 0 is taken as 0 (reading R8).
    """
    p = as_f64(prob)
    ix = np.asarray(idx, dtype=np.int64)
    safe = np.where(p > 0, p, 1.0)
    entropy_term = np.where(p > 0, p * np.log(safe), 0.0).sum(axis=1)
    cross_term = (p * np.take_along_axis(student_logits, ix, axis=1)).sum(axis=1)
    mass = p.sum(axis=1)
    return entropy_term - cross_term + mass * logsumexp(student_logits)


# ---------------------------------------------------------------------------
# Logit gradients (closed form)
# ---------------------------------------------------------------------------

def dce_dlogits(logits: np.ndarray, labels, valid: np.ndarray) -> np.ndarray:
    """d CE / d logits = softmax(x) - onehot(y) on valid rows, 0 elsewhere."""
    g = softmax(logits)
    rows = np.nonzero(valid)[0]
    g[rows, np.asarray(labels, dtype=np.int64)[rows]] -= 1.0
    g[~valid] = 0.0
    return g


def dkl_dstudent(student_logits: np.ndarray, teacher_logits: np.ndarray, T: float,
                 Tt: Optional[float] = None) -> np.ndarray:
    """d (T**2 KL(P_T || P_S)) / d z = T * (softmax(z/T) - softmax(t/Tt)).

    Only P_S depends on z, through z / T, so the teacher temperature enters
    through P_T alone.
    """
    Tt = T if Tt is None else Tt
    return T * (softmax(student_logits / T) - softmax(teacher_logits / Tt))


def dreverse_dstudent(student_logits: np.ndarray, teacher_logits: np.ndarray, T: float,
                      Tt: Optional[float] = None) -> np.ndarray:
    """d (T**2 KL(P_S || P_T)) / d z = T * P_S * (log P_S - log P_T - KL(P_S || P_T)).

    From d log P_S,v / d z_j = (delta_vj - P_S,j) / T: the T**2 and the 1/T of
    the softmax leave T, and the terms from differentiating log P_S sum to zero.
    """
    Tt = T if Tt is None else Tt
    lp_s = log_softmax(student_logits / T)
    lp_t = log_softmax(teacher_logits / Tt)
    p = np.exp(lp_s)
    kl = (p * (lp_s - lp_t)).sum(axis=-1, keepdims=True)
    return T * p * (lp_s - lp_t - kl)


def dkl_term(student_logits: np.ndarray, teacher_logits: np.ndarray, T: float,
             variant: str = "forward", Tt: Optional[float] = None) -> np.ndarray:
    """Gradient of kl_term with respect to the student logits."""
    if variant == "forward":
        return dkl_dstudent(student_logits, teacher_logits, T, Tt)
    if variant == "reverse":
        return dreverse_dstudent(student_logits, teacher_logits, T, Tt)
    if variant == "jeffreys":
        return (dkl_dstudent(student_logits, teacher_logits, T, Tt)
                + dreverse_dstudent(student_logits, teacher_logits, T, Tt))
    raise ValueError(f"unknown kl_divergence {variant!r}")


def dtopk_dstudent(student_logits: np.ndarray, idx, prob) -> np.ndarray:
    """Closed-form gradient of the sparse objective: M * softmax(z) - p scattered.

    CompactifAI/Full-Chunked-KL-Loss, Full Chunked KL: the backward applies
    M softmax(z) - p.
    """
    p = as_f64(prob)
    g = p.sum(axis=1)[:, None] * softmax(student_logits)
    rows = np.arange(g.shape[0])[:, None]
    np.subtract.at(g, (np.broadcast_to(rows, p.shape), np.asarray(idx, dtype=np.int64)), p)
    return g


# ---------------------------------------------------------------------------
# Whole-batch forward / backward
# ---------------------------------------------------------------------------

@dataclass
class Teacher:
    """Teacher descriptor (orda-kernel, Teacher descriptors).

    kind "tied": hidden only, projected with the student weight.
    kind "separate": hidden (N, D_t) and weight (V, D_t), detached.
    kind "topk": cached (idx, prob), each (N, K) (Full-Chunked-KL-Loss).
    kind "logits": cached dense logits (N, V), detached (orda-kernel, Teacher
    descriptors: PrecomputedTeacher(logits=...)).
    """

    kind: str
    hidden: Optional[np.ndarray] = None
    weight: Optional[np.ndarray] = None
    idx: Optional[np.ndarray] = None
    prob: Optional[np.ndarray] = None
    logits: Optional[np.ndarray] = None


@dataclass
class Student:
    """Student side: hidden (N, D) and weight (V, D), or given logits (N, V).

    The logits form is the flash_kd scorer (student_logits already
    materialised, forward only).
    """

    hidden: Optional[np.ndarray] = None
    weight: Optional[np.ndarray] = None
    logits: Optional[np.ndarray] = None

    @property
    def n(self) -> int:
        return (self.logits if self.logits is not None else self.hidden).shape[0]

    @property
    def v(self) -> int:
        return self.logits.shape[1] if self.logits is not None else self.weight.shape[0]


def _student_logits(s: Student, rows: np.ndarray) -> np.ndarray:
    if s.logits is not None:
        return as_f64(s.logits[rows])
    return project(s.hidden[rows], s.weight)


def _teacher_logits(t: Teacher, s: Student, rows: np.ndarray) -> Optional[np.ndarray]:
    if t.kind == "tied":
        return project(t.hidden[rows], s.weight)
    if t.kind == "separate":
        return project(t.hidden[rows], t.weight)
    if t.kind == "logits":
        return as_f64(t.logits[rows])
    return None


def per_token(student: Student, teacher: Teacher, p: Params, labels=None,
              rows: Optional[np.ndarray] = None) -> dict:
    """Per-token terms for the selected rows (all rows by default).

    Returns float64 arrays: student_ce, teacher_ce, kl (T**2 included), and for
    top-K mode the sparse objective in ``kl`` as well.
    """
    n = student.n
    v = student.v
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    if labels is None:
        lab = np.full(n, p.ignore_index, dtype=np.int64)
        valid_all = np.ones(n, dtype=bool)  # reading R10: top-K rows are all valid
    else:
        lab = np.asarray(labels, dtype=np.int64)
        valid_all = valid_mask(lab, v, p.ignore_index)
    out = {k: np.zeros(len(rows), F64) for k in ("student_ce", "teacher_ce", "kl")}
    out["valid"] = valid_all[rows]
    for b in range(0, len(rows), ROW_BLOCK):
        r = rows[b:b + ROW_BLOCK]
        z = _student_logits(student, r)
        vb = valid_all[r]
        if labels is not None:
            out["student_ce"][b:b + len(r)] = cross_entropy(z, lab[r], vb)
        if teacher.kind == "topk":
            if p.kl_divergence != "forward":
                raise ValueError("the cached top-K teacher supports forward KL only (reading R18)")
            out["kl"][b:b + len(r)] = topk_kl(z, teacher.idx[r], teacher.prob[r])
            continue
        t = _teacher_logits(teacher, student, r)
        if labels is not None:
            out["teacher_ce"][b:b + len(r)] = cross_entropy(t, lab[r], vb)
        kl = kl_term(z, t, p.temperature, p.kl_divergence, teacher_temperature(p))
        out["kl"][b:b + len(r)] = np.where(vb, kl, 0.0) if p.compact_valid else kl
    return out


def denominator(p: Params, n_valid: int) -> float:
    """Loss normaliser.

    nemo kd_loss, KDLoss.forward (num_batch_labels): divide by the given total
    when provided, else average over the valid tokens; orda-kernel, Parameters
    (reduction): "mean" or "sum". Reading R4: an all-ignored mean divides by 1.
    """
    if p.normalizer > 0:
        return float(p.normalizer)
    if p.reduction == "mean":
        return float(max(n_valid, 1))
    return 1.0


def forward(student: Student, teacher: Teacher, p: Params, labels=None) -> dict:
    """Per-token outputs plus the reduced loss.

    loss = sum over valid rows of (w_s ce_s + w_t ce_t + w_kl kl) / den
    (orda-kernel, Quickstart: DistillationLossOutput holds the loss and the
    unweighted components).
    """
    out = per_token(student, teacher, p, labels)
    valid = out["valid"]
    # A term whose weight is 0 is absent (reading R21), so an infinite teacher
    # CE at a zero-probability label does not enter an unweighted loss.
    contrib = np.zeros(len(valid), F64)
    for w_term, term in ((p.student_ce_weight, out["student_ce"]),
                         (p.teacher_ce_weight, out["teacher_ce"]), (p.kl_weight, out["kl"])):
        if w_term != 0.0:
            contrib = contrib + w_term * term
    n_valid = int(valid.sum())
    den = denominator(p, n_valid)
    out["n_valid"] = n_valid
    out["den"] = den
    out["loss"] = float(np.where(valid, contrib, 0.0).sum() / den)
    return out


def logit_grad(student: Student, teacher: Teacher, p: Params, labels, rows: np.ndarray,
               den: float, grad_loss: float = 1.0) -> np.ndarray:
    """d loss / d z for the given rows, shape (len(rows), V).

    (g / den) * valid * [w_s (softmax z - e_y) + w_kl T (softmax(z/T) - softmax(t/T_t))],
    or w_kl (M softmax z - p) in top-K mode. The teacher is detached (orda-kernel,
    KL variants: all variants except mutual/cojeffreys detach the teacher), so
    the teacher CE contributes no gradient (reading R6).
    """
    z = _student_logits(student, rows)
    v = student.v
    if labels is None:
        valid = np.ones(len(rows), dtype=bool)
        lab = None
    else:
        lab = np.asarray(labels, dtype=np.int64)[rows]
        valid = valid_mask(lab, v, p.ignore_index)
    g = np.zeros_like(z)
    if teacher.kind == "topk":
        if p.kl_divergence != "forward":
            raise ValueError("the cached top-K teacher supports forward KL only (reading R18)")
        g += p.kl_weight * dtopk_dstudent(z, teacher.idx[rows], teacher.prob[rows])
    else:
        if lab is not None and p.student_ce_weight != 0.0:
            g += p.student_ce_weight * dce_dlogits(z, lab, valid)
        if p.kl_weight != 0.0:
            t = _teacher_logits(teacher, student, rows)
            g += p.kl_weight * dkl_term(z, t, p.temperature, p.kl_divergence,
                                        teacher_temperature(p))
    g[~valid] = 0.0
    return g * (grad_loss / den)


def backward(student: Student, teacher: Teacher, p: Params, labels=None,
             grad_loss: float = 1.0, den: Optional[float] = None):
    """Gradients of the reduced loss with respect to student hidden and weight.

    dH = dZ @ W and dW = dZ.T @ H (CompactifAI/Full-Chunked-KL-Loss, Full
    Chunked KL: gradients of the hidden states and the projection from the
    closed-form logit gradient). Returns float64 (dH, dW).
    """
    n = student.n
    if den is None:
        if labels is None:
            n_valid = n
        else:
            n_valid = int(valid_mask(labels, student.v, p.ignore_index).sum())
        den = denominator(p, n_valid)
    W = as_f64(student.weight)
    dH = np.zeros((n, W.shape[1]), F64)
    dW = np.zeros_like(W)
    for b in range(0, n, ROW_BLOCK):
        r = np.arange(b, min(b + ROW_BLOCK, n))
        g = logit_grad(student, teacher, p, labels, r, den, grad_loss)
        dH[r] = g @ W
        dW += g.T @ as_f64(student.hidden[r])
    return dH, dW


def backward_rows(student: Student, teacher: Teacher, p: Params, labels, rows,
                  den: float, grad_loss: float = 1.0) -> np.ndarray:
    """dH restricted to the given rows (each row's gradient needs only that row)."""
    rows = np.asarray(rows, dtype=np.int64)
    W = as_f64(student.weight)
    out = np.zeros((len(rows), W.shape[1]), F64)
    for b in range(0, len(rows), ROW_BLOCK):
        r = rows[b:b + ROW_BLOCK]
        out[b:b + len(r)] = logit_grad(student, teacher, p, labels, r, den, grad_loss) @ W
    return out


def weight_grad_rows(student: Student, teacher: Teacher, p: Params, labels, vrows, den: float,
                     grad_loss: float = 1.0, progress=None) -> np.ndarray:
    """dW restricted to the vocabulary rows `vrows`: dW[v, :] = sum_i dz[i, v] H[i, :].

    Each dz[i, v] needs that token's normalisers over all V columns, so every
    row block's full-vocabulary logits are formed (logit_grad) and only the
    columns `vrows` of its gradient are kept (CompactifAI/Full-Chunked-KL-Loss,
    Full Chunked KL: the weight gradient from the closed-form logit gradient).
    `progress(done_rows, n)` is called after each row block. float64 (len(vrows), D).
    """
    vrows = np.asarray(vrows, dtype=np.int64)
    n = student.n
    out = np.zeros((len(vrows), student.hidden.shape[1]), F64)
    for b in range(0, n, ROW_BLOCK):
        r = np.arange(b, min(b + ROW_BLOCK, n))
        g = logit_grad(student, teacher, p, labels, r, den, grad_loss)
        out += g[:, vrows].T @ as_f64(student.hidden[r])
        if progress is not None:
            progress(int(r[-1]) + 1, n)
    return out


def teacher_logit_grad(student: Student, teacher: Teacher, p: Params, labels, rows: np.ndarray,
                       den: float, grad_loss: float = 1.0) -> np.ndarray:
    """d loss / d t for the given rows of a teacher trained through its CE.

    (g / den) * valid * w_t (softmax(t) - e_y): the teacher CE is taken at
    temperature 1 (reading R1) and the KL detaches the teacher (reading R6).
    """
    if teacher.kind not in ("tied", "separate"):
        raise ValueError("only a projected teacher (tied or separate) can be trained")
    lab = np.asarray(labels, dtype=np.int64)[rows]
    valid = valid_mask(lab, student.v, p.ignore_index)
    t = _teacher_logits(teacher, student, rows)
    g = p.teacher_ce_weight * dce_dlogits(t, lab, valid)  # 0 on invalid rows
    return g * (grad_loss / den)


def backward_teacher(student: Student, teacher: Teacher, p: Params, labels,
                     grad_loss: float = 1.0, den: Optional[float] = None):
    """Gradients of the reduced loss with respect to the teacher's hidden
    states and projection: dH_t = dT W_t and dW_t = dT^T H_t, dT from
    teacher_logit_grad (a tied teacher projects with the student weight, so
    its dW_t is the teacher half of that weight's gradient). float64."""
    n = student.n
    if den is None:
        den = denominator(p, int(valid_mask(labels, student.v, p.ignore_index).sum()))
    Wt = as_f64(student.weight if teacher.kind == "tied" else teacher.weight)
    dHt = np.zeros((n, Wt.shape[1]), F64)
    dWt = np.zeros_like(Wt)
    for b in range(0, n, ROW_BLOCK):
        r = np.arange(b, min(b + ROW_BLOCK, n))
        g = teacher_logit_grad(student, teacher, p, labels, r, den, grad_loss)
        dHt[r] = g @ Wt
        dWt += g.T @ as_f64(teacher.hidden[r])
    return dHt, dWt
