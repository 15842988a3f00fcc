"""PyTorch-facing API over the C ABI. Torch provides device memory and streams only.

Every computation runs in libkdloss.so; this module builds the descriptors,
allocates outputs / saved / workspace with the torch caching allocator and
passes pointers. If the library is missing, every entry point raises.

User API (orda-kernel, Quickstart / Teacher descriptors / Parameters):
    distillation_loss(student_hidden, weight, labels, teacher, *, student_ce_weight=1.0,
                      teacher_ce_weight=0.0, kl_weight=0.0, kl_temperature=1.0,
                      kl_teacher_temperature=None, kl_divergence="forward",
                      ignore_index=-100, reduction="mean", num_batch_labels=None,
                      vocab_chunk=0) -> DistillationLossOutput
    kl_divergence: "forward" | "reverse" | "jeffreys"
    teachers: TiedTeacher(hidden), SeparateTeacher(hidden, weight),
              PrecomputedTeacher(logits=...) or (teacher_hidden=..., teacher_weight=...),
              TopKTeacher(indices, probs)   (Full-Chunked-KL-Loss cached top-K)
Logits given on both sides (nemo kd_loss, KDLoss):
    KDLoss(ignore_index=-100, temperature=1.0).forward(student_logits, teacher_logits, labels,
                                                       num_batch_labels=None) -> scalar
Scorer (flash_kd, flash_ce_kd_loss):
    flash_ce_kd_loss(student_logits, teacher_hidden, teacher_lm_head_weight, labels, *,
                     temperature=1.0, ignore_index=-1, chunk_size=16384) -> (ce, kd)
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import NamedTuple, Optional

import torch

from . import _lib as L


# ---------------------------------------------------------------------------
# Teacher descriptors
# ---------------------------------------------------------------------------

@dataclass
class TiedTeacher:
    """Teacher that shares the student's projection weight; hidden: (BT, hidden)."""
    hidden: torch.Tensor
    mode: Optional[str] = None


@dataclass
class SeparateTeacher:
    """Teacher with its own hidden (BT, D_t) and projection (vocab, D_t); detached."""
    hidden: torch.Tensor
    weight: torch.Tensor


@dataclass
class PrecomputedTeacher:
    """Cached teacher, no gradient: dense ``logits`` (BT, vocab), or
    ``teacher_hidden`` (BT, D_t) with ``teacher_weight`` (vocab, D_t).
    A logit of -inf is a zero teacher probability."""
    logits: Optional[torch.Tensor] = None
    teacher_hidden: Optional[torch.Tensor] = None
    teacher_weight: Optional[torch.Tensor] = None

    def __post_init__(self):
        has_proj = self.teacher_hidden is not None or self.teacher_weight is not None
        if (self.logits is None) == (not has_proj) or \
                (has_proj and (self.teacher_hidden is None or self.teacher_weight is None)):
            raise ValueError("give either logits, or teacher_hidden and teacher_weight")


@dataclass
class TopKTeacher:
    """Cached sparse teacher: per row K distinct indices (int32) and probabilities (fp32),
    not renormalised."""
    indices: torch.Tensor
    probs: torch.Tensor


class DistillationLossOutput(NamedTuple):
    loss: torch.Tensor
    student_ce: torch.Tensor
    teacher_ce: torch.Tensor
    kl: torch.Tensor


def is_available(device: int = 0) -> bool:
    """True when the library is built and `device` is a gfx950 GPU."""
    try:
        lib = L.load()
    except Exception:
        return False
    if not torch.cuda.is_available():
        return False
    return bool(lib.kd_device_supported(device))


def lib():
    return L.load()


_DTYPES = {torch.float32: L.KD_F32, torch.bfloat16: L.KD_BF16}
_REDUCTIONS = {"mean": L.KD_REDUCE_MEAN, "sum": L.KD_REDUCE_SUM, "none": L.KD_REDUCE_NONE}
# orda-kernel, KL variants: KL(P_T || P_S), KL(P_S || P_T) and their sum.
_KL_DIVERGENCES = {"forward": L.KD_KL_FORWARD, "reverse": L.KD_KL_REVERSE,
                   "jeffreys": L.KD_KL_JEFFREYS}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


class Runner:
    """One configured loss call with its buffers; reusable across steps.

    Holds the C descriptors, the per-token outputs, the scalar loss, the saved
    statistics and the forward/backward workspaces. ``forward()`` and
    ``backward()`` enqueue on the current torch stream and return at once.
    """

    def __init__(self, *, student_hidden=None, weight=None, student_logits=None, labels=None,
                 teacher_kind="tied", teacher_hidden=None, teacher_weight=None, topk_idx=None,
                 topk_prob=None, teacher_logits=None, student_ce_weight=1.0,
                 teacher_ce_weight=0.0, kl_weight=0.0, temperature=1.0, ignore_index=-100,
                 reduction="mean", normalizer=0.0, vocab_chunk=0, want_grads=True,
                 want_teacher_ce=None, kl_divergence="forward", teacher_temperature=None,
                 compact_valid=False, keep_last_chunk=False, kl_output_unscaled=False,
                 grad_dtype=torch.float32):
        self.lib = L.load()
        ref = student_hidden if student_hidden is not None else student_logits
        if ref is None:
            raise ValueError("student_hidden or student_logits is required")
        if not ref.is_cuda:
            raise ValueError("inputs must be on a GPU device")
        self.device = ref.device
        dtype = _DTYPES.get(ref.dtype)
        if dtype is None:
            raise ValueError(f"unsupported dtype {ref.dtype}")
        # keep the tensors alive for the lifetime of the descriptors
        self._keep = [student_hidden, weight, student_logits, labels, teacher_hidden,
                      teacher_weight, topk_idx, topk_prob, teacher_logits]
        self.labels = labels
        s = L.KdStudent()
        s.dtype = dtype
        if student_logits is not None:
            s.kind = L.KD_STUDENT_LOGITS
            s.n, s.v = student_logits.shape
            s.d = 0
            s.logits = _ptr(student_logits)
        else:
            s.kind = L.KD_STUDENT_PROJECTION
            s.n, s.d = student_hidden.shape
            s.v = weight.shape[0]
            if weight.shape[1] != s.d:
                raise ValueError("weight must be (vocab, hidden)")
            s.hidden = _ptr(student_hidden)
            s.weight = _ptr(weight)
        t = L.KdTeacher()
        if teacher_kind == "tied":
            t.kind = L.KD_TEACHER_TIED
            t.d_t = teacher_hidden.shape[1]
            t.hidden = _ptr(teacher_hidden)
        elif teacher_kind == "separate":
            t.kind = L.KD_TEACHER_SEPARATE
            t.d_t = teacher_hidden.shape[1]
            t.hidden = _ptr(teacher_hidden)
            t.weight = _ptr(teacher_weight)
        elif teacher_kind == "logits":  # with student_logits: both given (nemo KDLoss)
            t.kind = L.KD_TEACHER_LOGITS
            if tuple(teacher_logits.shape) != (s.n, s.v) or teacher_logits.dtype != ref.dtype:
                raise ValueError("teacher logits must be (BT, vocab) in the student dtype")
            t.logits = _ptr(teacher_logits)
        elif teacher_kind == "topk":
            t.kind = L.KD_TEACHER_TOPK
            t.k = topk_idx.shape[1]
            t.topk_idx = _ptr(topk_idx)
            t.topk_prob = _ptr(topk_prob)
        else:
            raise ValueError(f"unknown teacher kind {teacher_kind}")
        p = L.KdParams()
        p.student_ce_weight = student_ce_weight
        p.teacher_ce_weight = teacher_ce_weight
        p.kl_weight = kl_weight
        p.temperature = temperature
        p.ignore_index = ignore_index
        p.reduction = _REDUCTIONS[reduction]
        p.normalizer = float(normalizer or 0.0)
        p.vocab_chunk = int(vocab_chunk)
        if kl_divergence not in _KL_DIVERGENCES:
            raise ValueError(f"kl_divergence={kl_divergence!r}; one of {tuple(_KL_DIVERGENCES)}")
        p.kl_divergence = _KL_DIVERGENCES[kl_divergence]
        p.teacher_temperature = 0.0 if teacher_temperature is None else float(teacher_temperature)
        p.compact_valid = 1 if compact_valid else 0
        # Opt-in: the forward keeps its last chunk's fp32 products for the
        # backward (identical results, one chunk fewer to recompute, at 4-8 B
        # per token and column of that chunk); off, peak memory stays at the
        # one-chunk slab.
        p.keep_last_chunk = 1 if keep_last_chunk else 0
        p.kl_output_unscaled = 1 if kl_output_unscaled else 0
        # dH / dW (and a trained teacher's) element type: fp32, or bf16 rounded once
        if grad_dtype not in _DTYPES:
            raise ValueError(f"unsupported gradient dtype {grad_dtype}")
        self.grad_dtype = grad_dtype
        p.dh_dtype = p.dw_dtype = _DTYPES[grad_dtype]
        self.s, self.t, self.p = s, t, p
        self.n, self.v, self.d = int(s.n), int(s.v), int(s.d)
        self.teacher_kind = teacher_kind
        self.dt = int(t.d_t) if teacher_kind == "separate" else self.d
        f32 = dict(dtype=torch.float32, device=self.device)
        self.loss = torch.zeros((), **f32)
        self.student_ce = torch.empty(self.n, **f32)
        self.teacher_ce = torch.empty(self.n, **f32)
        self.kl = torch.empty(self.n, **f32)
        if want_teacher_ce is None:
            want_teacher_ce = teacher_ce_weight > 0
        self.teacher_ce.zero_()
        # The teacher CE is computed only when it is weighted or asked for.
        self.out = L.KdOutputs(self.loss.data_ptr(), self.student_ce.data_ptr(),
                               self.teacher_ce.data_ptr() if want_teacher_ce else None,
                               self.kl.data_ptr())
        nb = ctypes.c_size_t(0)
        L.check(self.lib.kd_saved_bytes_for(ctypes.byref(s), ctypes.byref(t), ctypes.byref(p),
                                            ctypes.byref(nb)), "kd_saved_bytes_for")
        self.saved = torch.empty(int(nb.value), dtype=torch.uint8, device=self.device)
        p.saved_bytes = self.saved.numel()
        self.ws_fwd = self._workspace(0)
        self.ws_bwd = self._workspace(1) if (want_grads and s.kind == L.KD_STUDENT_PROJECTION) \
            else None
        self.dtype = ref.dtype
        self.labels_ptr = _ptr(labels)

    def _workspace(self, backward: int) -> torch.Tensor:
        nb = ctypes.c_size_t(0)
        L.check(self.lib.kd_workspace_bytes(ctypes.byref(self.s), ctypes.byref(self.t),
                                            ctypes.byref(self.p), backward, ctypes.byref(nb)),
                "kd_workspace_bytes")
        return torch.empty(max(int(nb.value), 256), dtype=torch.uint8, device=self.device)

    @staticmethod
    def _stream() -> int:
        return torch.cuda.current_stream().cuda_stream

    def forward(self, trace: Optional[L.KdTrace] = None) -> None:
        st = self.lib.kd_loss_fwd(ctypes.byref(self.s), ctypes.byref(self.t), ctypes.byref(self.p),
                                  self.labels_ptr, ctypes.byref(self.out), self.saved.data_ptr(),
                                  self.ws_fwd.data_ptr(), self.ws_fwd.numel(), self._stream(),
                                  ctypes.byref(trace) if trace is not None else None)
        L.check(st, "kd_loss_fwd")

    def backward(self, d_hidden: Optional[torch.Tensor], d_weight: Optional[torch.Tensor],
                 grad_loss: Optional[torch.Tensor] = None, accumulate: bool = False,
                 trace: Optional[L.KdTrace] = None) -> None:
        for g, shape in ((d_hidden, (self.n, self.d)), (d_weight, (self.v, self.d))):
            if g is not None and (g.dtype != self.grad_dtype or tuple(g.shape) != shape
                                  or not g.is_contiguous()):
                raise ValueError(f"gradient buffers must be contiguous {self.grad_dtype} {shape}")
        st = self.lib.kd_loss_bwd(ctypes.byref(self.s), ctypes.byref(self.t), ctypes.byref(self.p),
                                  self.labels_ptr, self.saved.data_ptr(), _ptr(grad_loss),
                                  _ptr(d_hidden), _ptr(d_weight), int(accumulate),
                                  self.ws_bwd.data_ptr(), self.ws_bwd.numel(), self._stream(),
                                  ctypes.byref(trace) if trace is not None else None)
        L.check(st, "kd_loss_bwd")

    def backward_logits(self, d_logits: Optional[torch.Tensor], grad_loss: Optional[torch.Tensor] = None,
                        accumulate: bool = False, trace: Optional[L.KdTrace] = None) -> None:
        """Gradient to given student logits (student and teacher logits both
        given): d_logits (BT, vocab) in the logits dtype."""
        if d_logits is not None and (d_logits.dtype != self.dtype or
                                     tuple(d_logits.shape) != (self.n, self.v) or
                                     not d_logits.is_contiguous()):
            raise ValueError(f"d_logits must be contiguous {self.dtype} {(self.n, self.v)}")
        st = self.lib.kd_loss_bwd_logits(
            ctypes.byref(self.s), ctypes.byref(self.t), ctypes.byref(self.p), self.labels_ptr,
            self.saved.data_ptr(), _ptr(grad_loss), _ptr(d_logits), int(accumulate), self._stream(),
            ctypes.byref(trace) if trace is not None else None)
        L.check(st, "kd_loss_bwd_logits")

    def backward_teacher(self, d_teacher_hidden: Optional[torch.Tensor],
                         d_teacher_weight: Optional[torch.Tensor],
                         grad_loss: Optional[torch.Tensor] = None, accumulate: bool = False,
                         trace: Optional[L.KdTrace] = None) -> None:
        """Gradient of w_t CE(t) to a tied or separate teacher (the KL detaches it).
        Tied: d_teacher_weight is the teacher half of the shared weight's gradient."""
        for g, shape in ((d_teacher_hidden, (self.n, self.dt)), (d_teacher_weight, (self.v, self.dt))):
            if g is not None and (g.dtype != self.grad_dtype or tuple(g.shape) != shape
                                  or not g.is_contiguous()):
                raise ValueError(f"gradient buffers must be contiguous {self.grad_dtype} {shape}")
        st = self.lib.kd_loss_bwd_teacher(
            ctypes.byref(self.s), ctypes.byref(self.t), ctypes.byref(self.p), self.labels_ptr,
            self.saved.data_ptr(), _ptr(grad_loss), _ptr(d_teacher_hidden), _ptr(d_teacher_weight),
            int(accumulate), self.ws_bwd.data_ptr(), self.ws_bwd.numel(), self._stream(),
            ctypes.byref(trace) if trace is not None else None)
        L.check(st, "kd_loss_bwd_teacher")

    def read_status(self, backward: bool = False) -> int:
        """Device flags of the last forward (or, with backward=True, the last
        backward): 1 = a label / top-K index out of range, 2 = `saved` without
        kept products of this layout."""
        ws = self.ws_bwd if backward else self.ws_fwd
        flags = ctypes.c_int32(0)
        self.lib.kd_read_status(ws.data_ptr(), self._stream(), ctypes.byref(flags))
        return int(flags.value)


class Tracer:
    """Brackets library launches with HIP events (kd_trace) and reports the
    mean duration per kernel class."""

    def __init__(self, capacity: int = 4096, kernels=("fwd",)):
        self.lib = L.load()
        self.capacity = capacity
        self.events = (ctypes.c_void_p * capacity)()
        self.kinds = (ctypes.c_int32 * (capacity // 2))()
        L.check(self.lib.kd_events_create(self.events, capacity), "kd_events_create")
        mask = 0
        for k in kernels:
            mask |= 1 << L.KERNEL_ID[k]
        self.trace = L.KdTrace(self.events, self.kinds, capacity, 0, mask)

    def reset(self) -> None:
        self.trace.count = 0

    def durations_ms(self) -> dict:
        out = {}
        ms = ctypes.c_float(0)
        for j in range(self.trace.count // 2):
            L.check(self.lib.kd_event_elapsed_ms(self.events[2 * j], self.events[2 * j + 1],
                                                 ctypes.byref(ms)), "kd_event_elapsed_ms")
            out.setdefault(L.KERNELS[self.kinds[j]], []).append(ms.value)
        return out

    def close(self) -> None:
        if self.events is not None:
            self.lib.kd_events_destroy(self.events, self.capacity)
            self.events = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------------------
# Autograd function (orda-kernel style API)
# ---------------------------------------------------------------------------

class _FusedLoss(torch.autograd.Function):
    @staticmethod
    def forward(ctx, student_hidden, weight, teacher_hidden, teacher_weight, runner: Runner):
        # teacher_hidden / teacher_weight are given only for a teacher trained
        # through its CE; otherwise None (the teacher is detached).
        runner.forward()
        # The backward recomputes from these tensors: saving them lets autograd's
        # version counters reject an in-place change between forward and backward.
        ctx.save_for_backward(student_hidden, weight, teacher_hidden, teacher_weight)
        ctx.runner = runner
        ctx.train_teacher = getattr(runner, "train_teacher", False)
        ctx.used = False
        return (runner.loss.clone(), runner.student_ce.clone(), runner.teacher_ce.clone(),
                runner.kl.clone())

    @staticmethod
    def backward(ctx, g_loss, g_sce, g_tce, g_kl):
        # Only the reduced loss is differentiated; the components are for logging
        # (orda-kernel, Quickstart: components are unweighted for logging).
        if ctx.used:
            raise RuntimeError("each fused forward supports one backward pass")
        ctx.used = True
        ctx.saved_tensors  # raises if a saved input was modified in place since the forward
        r: Runner = ctx.runner
        need_h, need_w = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        need_ht, need_wt = ctx.needs_input_grad[2], ctx.needs_input_grad[3]
        # gradients come out of the library in r.grad_dtype (the inputs' dtype,
        # rounded once from fp32 for bf16)
        f32 = dict(dtype=r.grad_dtype, device=r.device)
        dh = torch.empty((r.n, r.d), **f32) if need_h else None
        dw = torch.empty((r.v, r.d), **f32) if need_w else None
        g = (g_loss if g_loss is not None else torch.ones((), device=r.device))
        g = g.detach().to(torch.float32).contiguous()
        if dh is not None or dw is not None:
            r.backward(dh, dw, grad_loss=g)
        dht = dwt = None
        if need_ht or need_wt or (r.teacher_kind == "tied" and need_w and ctx.train_teacher):
            # accumulate: the tied weight's teacher half adds to dw; dht starts at 0
            dht = torch.zeros((r.n, r.dt), **f32) if need_ht else None
            if r.teacher_kind == "tied":
                dwt_buf = dw
            else:
                dwt_buf = torch.zeros((r.v, r.dt), **f32) if need_wt else None
            r.backward_teacher(dht, dwt_buf, grad_loss=g, accumulate=True)
            dwt = dwt_buf if r.teacher_kind != "tied" else None
        return dh, dw, dht, dwt, None


def distillation_loss(student_hidden, weight, labels, teacher, *, student_ce_weight=1.0,
                      teacher_ce_weight=0.0, kl_weight=0.0, kl_temperature=1.0,
                      kl_teacher_temperature=None, kl_divergence="forward", ignore_index=-100,
                      reduction="mean", num_batch_labels=None, vocab_chunk=0,
                      return_teacher_ce=True, compact_valid=False,
                      keep_last_chunk=False) -> DistillationLossOutput:
    """Fused LM-head + CE + KL loss; differentiable in student_hidden and weight.

    The teacher is always detached. Returns the loss and the unweighted per-token
    components (student_ce, teacher_ce, kl with T^2 included). With
    return_teacher_ce=False and teacher_ce_weight=0 the teacher CE is skipped
    (one exponential pass fewer per tile when the temperature is not 1) and
    reported as zeros. compact_valid=True leaves the rows whose label is
    ignored out of every projection (tied and projected teachers): their
    per-token terms are reported as 0, the loss and gradients are unchanged.
    keep_last_chunk=True (opt-in) keeps the forward's last vocabulary chunk of
    fp32 products for the backward, which then does not recompute it:
    identical results for 8 B per token and column of that chunk (4 B without
    a projected teacher). Off by default, so the extra memory stays at the
    one-chunk gradient slab.
    """
    if kl_divergence not in _KL_DIVERGENCES:
        raise ValueError(f"kl_divergence={kl_divergence!r}; one of {tuple(_KL_DIVERGENCES)}")
    if isinstance(teacher, TopKTeacher) and kl_divergence != "forward":
        raise NotImplementedError("the top-K teacher supports kl_divergence='forward' only")
    if kl_teacher_temperature is not None and not kl_teacher_temperature > 0:
        raise ValueError("kl_teacher_temperature must be positive")
    # A tied or separate teacher whose tensors require grad trains through its
    # CE when teacher_ce_weight > 0 (orda-kernel, Teacher descriptors); the KL
    # always detaches it. Cached (precomputed) teachers never receive gradients.
    if isinstance(teacher, PrecomputedTeacher) and any(
            x is not None and x.requires_grad
            for x in (teacher.logits, teacher.teacher_hidden, teacher.teacher_weight)):
        raise ValueError("PrecomputedTeacher tensors must not require grad")
    t_hidden = t_weight = None
    if teacher_ce_weight > 0 and isinstance(teacher, (TiedTeacher, SeparateTeacher)):
        if teacher.hidden.requires_grad:
            t_hidden = teacher.hidden
        if isinstance(teacher, SeparateTeacher) and teacher.weight.requires_grad:
            t_weight = teacher.weight
    train_teacher = t_hidden is not None or t_weight is not None or (
        teacher_ce_weight > 0 and isinstance(teacher, TiedTeacher))
    if isinstance(teacher, TiedTeacher) and teacher.mode is not None:
        # the mode asserts the role the weights give; it does not route
        role = "trained" if teacher_ce_weight > 0 else "frozen"
        if teacher.mode == "cotrained":
            raise NotImplementedError("co-trained teachers (mutual / cojeffreys) are not provided")
        if teacher.mode != role:
            raise ValueError(f"TiedTeacher(mode={teacher.mode!r}) but the weights make it {role}")
    # Gradients in the inputs' dtype straight from the library (bf16: the fp32
    # result rounded once, as a cast would). A trained tied teacher sums two
    # halves into the shared weight's gradient, which stays fp32 for that sum.
    grad_dtype = student_hidden.dtype
    if isinstance(teacher, TiedTeacher) and train_teacher:
        grad_dtype = torch.float32
    kw = dict(kl_divergence=kl_divergence, teacher_temperature=kl_teacher_temperature,
              grad_dtype=grad_dtype,
              student_hidden=student_hidden.detach().contiguous(),
              weight=weight.detach().contiguous(), student_ce_weight=student_ce_weight,
              teacher_ce_weight=teacher_ce_weight, kl_weight=kl_weight,
              temperature=kl_temperature, ignore_index=ignore_index, reduction=reduction,
              normalizer=float(num_batch_labels or 0), vocab_chunk=vocab_chunk,
              want_teacher_ce=bool(return_teacher_ce or teacher_ce_weight > 0))
    if isinstance(teacher, TiedTeacher):
        kw.update(teacher_kind="tied", teacher_hidden=teacher.hidden.detach().contiguous())
    elif isinstance(teacher, PrecomputedTeacher) and teacher.logits is not None:
        kw.update(teacher_kind="logits", teacher_logits=teacher.logits.detach().contiguous())
    elif isinstance(teacher, (SeparateTeacher, PrecomputedTeacher)):
        h = teacher.hidden if isinstance(teacher, SeparateTeacher) else teacher.teacher_hidden
        w = teacher.weight if isinstance(teacher, SeparateTeacher) else teacher.teacher_weight
        kw.update(teacher_kind="separate", teacher_hidden=h.detach().contiguous(),
                  teacher_weight=w.detach().contiguous())
    elif isinstance(teacher, TopKTeacher):
        kw.update(teacher_kind="topk", topk_idx=teacher.indices.to(torch.int32).contiguous(),
                  topk_prob=teacher.probs.to(torch.float32).contiguous())
        labels = None
    else:
        raise TypeError(f"unknown teacher descriptor {type(teacher).__name__}")
    if compact_valid and (labels is None or kw["teacher_kind"] not in ("tied", "separate")):
        raise NotImplementedError("compact_valid needs labels and a tied or projected teacher")
    kw["compact_valid"] = bool(compact_valid)
    # the kept products only pay off when a backward follows
    kw["keep_last_chunk"] = bool(keep_last_chunk) and torch.is_grad_enabled() and any(
        x is not None and x.requires_grad for x in (student_hidden, weight, t_hidden, t_weight))
    if labels is not None:
        kw["labels"] = labels.to(torch.int64).contiguous()
    runner = Runner(**kw)
    runner.train_teacher = train_teacher
    loss, sce, tce, kl = _FusedLoss.apply(student_hidden, weight, t_hidden, t_weight, runner)
    return DistillationLossOutput(loss, sce, tce, kl)


class DistillationLoss(torch.nn.Module):
    """Module form of distillation_loss with the weights fixed at construction."""

    def __init__(self, **kwargs):
        super().__init__()
        self.kwargs = kwargs

    def forward(self, student_hidden, weight, labels, teacher):
        return distillation_loss(student_hidden, weight, labels, teacher, **self.kwargs)


class _LogitsKD(torch.autograd.Function):
    """Loss from given student and teacher logits; differentiable in the student's."""

    @staticmethod
    def forward(ctx, student_logits, runner: Runner):
        runner.forward()
        ctx.runner = runner
        return runner.loss.clone()

    @staticmethod
    def backward(ctx, g_loss):
        r: Runner = ctx.runner
        if not ctx.needs_input_grad[0]:
            return None, None
        d = torch.empty((r.n, r.v), dtype=r.dtype, device=r.device)
        g = (g_loss if g_loss is not None else torch.ones((), device=r.device))
        r.backward_logits(d, grad_loss=g.detach().to(torch.float32).contiguous())
        return d, None


class KDLoss(torch.nn.Module):
    """Forward KL(P_T || P_S) x T^2 over the valid tokens, from student and
    teacher logits both given (nemo kd_loss, KDLoss and KDLoss.forward).

    Logits are [..., vocab] with labels [...]; rows whose label equals
    ignore_index are excluded. With num_batch_labels the summed KL is divided
    by it, else averaged over this batch's valid tokens. Differentiable in
    student_logits; the teacher is detached. Arithmetic is always fp32
    (``fp32_upcast`` is accepted for compatibility) and the whole vocabulary is
    streamed once per pass, so ``chunk_size`` changes nothing here.
    """

    def __init__(self, ignore_index: int = -100, temperature: float = 1.0, fp32_upcast: bool = True,
                 tp_group=None, chunk_size: int = 0):
        super().__init__()
        if tp_group is not None:
            raise NotImplementedError("tensor-parallel vocabulary shards are not provided (one GPU)")
        del fp32_upcast, chunk_size
        self.ignore_index = ignore_index
        self.temperature = temperature

    def forward(self, student_logits, teacher_logits, labels, num_batch_labels=None):
        v = student_logits.shape[-1]
        if teacher_logits.shape != student_logits.shape:
            raise ValueError("teacher_logits must have the student logits' shape")
        if teacher_logits.dtype != student_logits.dtype:
            # no silent cast: an fp32 teacher rounded to bf16 would lose precision
            raise TypeError(f"teacher_logits dtype {teacher_logits.dtype} differs from the student "
                            f"logits' {student_logits.dtype}; convert one of them explicitly")
        z = student_logits.reshape(-1, v)
        runner = Runner(student_logits=z.detach().contiguous(), teacher_kind="logits",
                        teacher_logits=teacher_logits.detach().reshape(-1, v).contiguous(),
                        labels=labels.reshape(-1).to(torch.int64).contiguous(),
                        student_ce_weight=0.0, teacher_ce_weight=0.0, kl_weight=1.0,
                        temperature=self.temperature, ignore_index=self.ignore_index,
                        normalizer=float(num_batch_labels or 0), want_grads=False)
        return _LogitsKD.apply(z, runner)


def flash_ce_kd_loss(student_logits, teacher_hidden, teacher_lm_head_weight, labels, *,
                     temperature=1.0, ignore_index=-1, chunk_size=16384, upcast=True):
    """Forward-only per-token CE and KL(P_T || P_S) from given student logits.

    flash_kd, flash_ce_kd_loss: teacher logits are recomputed chunk by chunk;
    ignore_index rows get CE 0; the returned KD is NOT multiplied by T^2.
    Accumulation is always fp32 (``upcast`` is accepted for compatibility).
    """
    del upcast
    with torch.no_grad():
        r = Runner(student_logits=student_logits.contiguous(), labels=labels.to(torch.int64)
                   .contiguous(), teacher_kind="separate",
                   teacher_hidden=teacher_hidden.contiguous(),
                   teacher_weight=teacher_lm_head_weight.contiguous(), student_ce_weight=1.0,
                   kl_weight=1.0, temperature=temperature, ignore_index=ignore_index,
                   reduction="none", vocab_chunk=chunk_size, want_grads=False,
                   kl_output_unscaled=True)
        r.forward()
        return r.student_ce.clone(), r.kl.clone()
