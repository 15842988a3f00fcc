"""Pins that tie the float64 oracle to facts outside itself.

Each ``check_*`` takes an oracle module ``O`` and raises AssertionError when
the oracle disagrees with something the pages or the mathematics fix:
closed forms, special cases that reduce to a library routine
(torch.nn.functional.cross_entropy / kl_div, autograd), invariants, and
central finite differences. None of them retypes the oracle's own formula.

tests/test_oracle.py runs them against the real oracle; tests/test_oracle_mutants.py
runs them against copies of the oracle with one planted mistake each and
requires that some pin fails.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

RNG_SEED = 1234


def _rng(k=0):
    return np.random.default_rng(RNG_SEED + k)


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    ok = np.allclose(a, b, rtol=rtol, atol=atol)
    assert ok, f"{what}: max abs diff {np.max(np.abs(a - b)):.3e}"


def _student_logits_case(O, n=6, v=9, k=0):
    r = _rng(k)
    z = r.normal(size=(n, v)) * 2.0
    return O.Student(logits=z), z


# ---------------------------------------------------------------------------
# Cross-entropy (flash_kd, flash_ce_kd_loss: standard CE, 0 on ignored rows)
# ---------------------------------------------------------------------------

def check_ce_uniform_logits(O):
    """W = 0 makes every logit 0: CE = log V exactly, softmax = 1/V, and the
    logit gradient of the mean CE is (1/V - e_y)/n_valid in closed form."""
    n, d, v = 5, 4, 11
    r = _rng(1)
    H = r.normal(size=(n, d))
    W = np.zeros((v, d))
    y = np.array([3, 0, -100, 10, 7])
    s = O.Student(hidden=H, weight=W)
    t = O.Teacher("tied", hidden=H)
    p = O.Params(student_ce_weight=1.0, kl_weight=0.0)
    out = O.forward(s, t, p, y)
    valid = y != -100
    _close(out["student_ce"], np.where(valid, math.log(v), 0.0), what="CE = log V")
    _close(out["loss"], math.log(v), what="mean CE = log V")
    g = O.logit_grad(s, t, p, y, np.arange(n), den=float(valid.sum()))
    expect = np.zeros((n, v))
    for i in range(n):
        if valid[i]:
            expect[i] = 1.0 / v
            expect[i, y[i]] -= 1.0
    _close(g, expect / valid.sum(), what="dCE/dz closed form")


def check_ce_library(O):
    """Per-token CE equals torch's cross_entropy(reduction='none') in float64,
    ignore_index rows included (flash_kd, labels parameter)."""
    s, z = _student_logits_case(O, n=7, v=13, k=2)
    y = np.array([0, 12, -100, 5, 5, -100, 9])
    p = O.Params(student_ce_weight=1.0, kl_weight=0.0)
    out = O.per_token(s, O.Teacher("topk", idx=np.zeros((7, 1), np.int64),
                                   prob=np.zeros((7, 1))), p, y)
    ref = F.cross_entropy(torch.from_numpy(z), torch.from_numpy(y), reduction="none",
                          ignore_index=-100).numpy()
    _close(out["student_ce"], ref, what="CE vs F.cross_entropy")
    mean = F.cross_entropy(torch.from_numpy(z), torch.from_numpy(y), ignore_index=-100).item()
    w = O.Teacher("topk", idx=np.zeros((7, 1), np.int64), prob=np.zeros((7, 1)))
    _close(O.forward(s, w, p, y)["loss"], mean, what="mean CE vs F.cross_entropy")


def check_ce_two_classes(O):
    """V = 2: CE = softplus(z_other - z_y)."""
    s, z = _student_logits_case(O, n=8, v=2, k=3)
    y = np.array([0, 1, 1, 0, 1, 0, 0, 1])
    p = O.Params(student_ce_weight=1.0, kl_weight=0.0)
    w = O.Teacher("topk", idx=np.zeros((8, 1), np.int64), prob=np.zeros((8, 1)))
    out = O.per_token(s, w, p, y)
    other = z[np.arange(8), 1 - y]
    own = z[np.arange(8), y]
    _close(out["student_ce"], np.log1p(np.exp(other - own)), what="CE softplus")


def check_ce_large_logits(O):
    """A shift of every logit by a constant leaves CE unchanged (lse is
    shift-equivariant); a shift of 1e4 overflows exp without the max shift."""
    s, z = _student_logits_case(O, n=4, v=6, k=4)
    y = np.array([1, 2, 3, 4])
    p = O.Params(student_ce_weight=1.0, kl_weight=0.0)
    w = O.Teacher("topk", idx=np.zeros((4, 1), np.int64), prob=np.zeros((4, 1)))
    a = O.per_token(s, w, p, y)["student_ce"]
    b = O.per_token(O.Student(logits=z + 1.0e4), w, p, y)["student_ce"]
    _close(a, b, rtol=1e-9, atol=1e-9, what="CE shift invariance")


# ---------------------------------------------------------------------------
# Forward KL (nemo kd_loss, KDLoss temperature; orda-kernel, KL variants)
# ---------------------------------------------------------------------------

def _tied_case(O, n=6, d=5, v=10, k=5, same=False):
    r = _rng(k)
    Hs = r.normal(size=(n, d))
    Ht = Hs.copy() if same else r.normal(size=(n, d)) * 1.3
    W = r.normal(size=(v, d)) * 0.7
    return O.Student(hidden=Hs, weight=W), O.Teacher("tied", hidden=Ht)


def check_kl_zero_for_identical(O):
    """KL = 0 when the teacher equals the student (tied with H_t = H_s;
    separate with W_t = W and H_t = H_s), at any temperature."""
    for T in (1.0, 2.0, 0.5):
        s, t = _tied_case(O, same=True)
        p = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=T)
        _close(O.per_token(s, t, p)["kl"], 0.0, atol=1e-13, what="KL tied identical")
        t2 = O.Teacher("separate", hidden=s.hidden.copy(), weight=s.weight.copy())
        _close(O.per_token(s, t2, p)["kl"], 0.0, atol=1e-13, what="KL separate identical")


def check_kl_nonnegative(O):
    """Gibbs' inequality: KL >= 0, and > 0 for distinct distributions."""
    s, t = _tied_case(O, k=6)
    for T in (1.0, 3.0):
        p = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=T)
        kl = O.per_token(s, t, p)["kl"]
        assert (kl > 0).all(), f"KL not positive: {kl}"


def check_kl_library(O):
    """T^2 * kl_div(log_softmax(z/T), log_softmax(t/T), log_target) summed over
    the vocabulary equals the oracle's per-token KL (nemo kd_loss: divide by T,
    multiply by T^2; flash_kd: T = 1 is the plain kl_div metric)."""
    s, t = _tied_case(O, n=7, d=4, v=12, k=7)
    z = torch.from_numpy(s.hidden @ s.weight.T)
    tt = torch.from_numpy(t.hidden @ s.weight.T)
    for T in (1.0, 2.0, 0.7):
        p = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=T)
        ref = F.kl_div(F.log_softmax(z / T, -1), F.log_softmax(tt / T, -1), log_target=True,
                       reduction="none").sum(-1) * T * T
        _close(O.per_token(s, t, p)["kl"], ref.numpy(), rtol=1e-11, atol=1e-12,
               what=f"KL vs F.kl_div T={T}")


def check_kl_two_classes(O):
    """V = 2: closed-form Bernoulli KL between sigmoid((t1-t0)/T) and
    sigmoid((z1-z0)/T), times T^2."""
    r = _rng(8)
    z = r.normal(size=(6, 2)) * 1.5
    tl = r.normal(size=(6, 2)) * 1.5
    T = 1.7
    qs = 1.0 / (1.0 + np.exp(-(z[:, 1] - z[:, 0]) / T))
    qt = 1.0 / (1.0 + np.exp(-(tl[:, 1] - tl[:, 0]) / T))
    ref = T * T * (qt * np.log(qt / qs) + (1 - qt) * np.log((1 - qt) / (1 - qs)))
    # separate teacher whose head is the identity: logits equal the hidden states
    s = O.Student(hidden=z, weight=np.eye(2))
    t = O.Teacher("separate", hidden=tl, weight=np.eye(2))
    p = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=T)
    _close(O.per_token(s, t, p)["kl"], ref, rtol=1e-11, atol=1e-13, what="Bernoulli KL")


def check_kl_temperature_identity(O):
    """KL at temperature T on (z, t) equals T^2 times KL at T = 1 on (z/T, t/T)."""
    s, t = _tied_case(O, k=9)
    T = 2.5
    z = s.hidden @ s.weight.T
    tl = t.hidden @ s.weight.T
    pT = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=T)
    p1 = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=1.0)
    eye = np.eye(z.shape[1])
    a = O.per_token(s, t, pT)["kl"]
    b = O.per_token(O.Student(hidden=z / T, weight=eye),
                    O.Teacher("separate", hidden=tl / T, weight=eye), p1)["kl"]
    _close(a, T * T * b, rtol=1e-11, atol=1e-13, what="KL temperature identity")


# ---------------------------------------------------------------------------
# Sparse top-K objective (Full-Chunked-KL-Loss, Methods / Full Dense KL)
# ---------------------------------------------------------------------------

def check_reverse_kl_library(O):
    """Reverse KL: T^2 * kl_div with the operands swapped (target = student),
    summed over the vocabulary (orda-kernel, KL variants: reverse = KL(p || q),
    p = student)."""
    s, t = _tied_case(O, n=7, d=4, v=12, k=3)
    z = torch.from_numpy(s.hidden @ s.weight.T)
    tt = torch.from_numpy(t.hidden @ s.weight.T)
    for T in (1.0, 2.0, 0.7):
        p = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=T, kl_divergence="reverse")
        ref = F.kl_div(F.log_softmax(tt / T, -1), F.log_softmax(z / T, -1), log_target=True,
                       reduction="none").sum(-1) * T * T
        _close(O.per_token(s, t, p)["kl"], ref.numpy(), rtol=1e-11, atol=1e-12,
               what=f"reverse KL vs F.kl_div T={T}")


def check_reverse_kl_two_classes(O):
    """V = 2: closed-form Bernoulli KL(P_S || P_T) times T^2."""
    r = _rng(9)
    z = r.normal(size=(6, 2)) * 1.5
    tl = r.normal(size=(6, 2)) * 1.5
    T = 1.3
    qs = 1.0 / (1.0 + np.exp(-(z[:, 1] - z[:, 0]) / T))
    qt = 1.0 / (1.0 + np.exp(-(tl[:, 1] - tl[:, 0]) / T))
    ref = T * T * (qs * np.log(qs / qt) + (1 - qs) * np.log((1 - qs) / (1 - qt)))
    s = O.Student(hidden=z, weight=np.eye(2))
    t = O.Teacher("separate", hidden=tl, weight=np.eye(2))
    p = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=T, kl_divergence="reverse")
    _close(O.per_token(s, t, p)["kl"], ref, rtol=1e-11, atol=1e-13, what="reverse Bernoulli")


def check_jeffreys_symmetric(O):
    """Jeffreys is symmetric: swapping the student and teacher logits leaves it
    unchanged, while forward and reverse trade places; forward + reverse = it."""
    r = _rng(11)
    z = r.normal(size=(5, 9)) * 2.0
    tl = r.normal(size=(5, 9)) * 2.0
    eye = np.eye(9)
    T = 1.6

    def kl(a, b, variant):
        p = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=T, kl_divergence=variant)
        return O.per_token(O.Student(hidden=a, weight=eye), O.Teacher("separate", hidden=b, weight=eye),
                           p)["kl"]

    _close(kl(z, tl, "jeffreys"), kl(tl, z, "jeffreys"), rtol=1e-12, what="jeffreys symmetric")
    _close(kl(z, tl, "forward"), kl(tl, z, "reverse"), rtol=1e-12, what="forward/reverse swap")
    _close(kl(z, tl, "jeffreys"), kl(z, tl, "forward") + kl(z, tl, "reverse"), rtol=1e-12,
           what="jeffreys = forward + reverse")


def check_reverse_zero_and_nonnegative(O):
    """Reverse and Jeffreys KL are 0 for identical logits and > 0 otherwise (Gibbs)."""
    for variant in ("reverse", "jeffreys"):
        p = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=1.9, kl_divergence=variant)
        s, t = _tied_case(O, n=5, d=4, v=11, k=4, same=True)
        _close(O.per_token(s, t, p)["kl"], 0.0, atol=1e-14, what=f"{variant} zero")
        s, t = _tied_case(O, n=5, d=4, v=11, k=4)
        assert (O.per_token(s, t, p)["kl"] > 0).all(), f"{variant} not positive"


# ---------------------------------------------------------------------------
# Independent teacher temperature and cached dense teacher logits
# (orda-kernel, Parameters: kl_teacher_temperature; Teacher descriptors:
# PrecomputedTeacher(logits=...))
# ---------------------------------------------------------------------------

def _eye_pair(O, z, tl):
    eye = np.eye(z.shape[1])
    return O.Student(hidden=z, weight=eye), O.Teacher("separate", hidden=tl, weight=eye)


def check_teacher_temperature_library(O):
    """T_s^2 * kl_div(log_softmax(z/T_s), log_softmax(t/T_t)) summed over the
    vocabulary, in both directions, for T_t apart from T_s."""
    r = _rng(30)
    z = r.normal(size=(6, 11)) * 2.0
    tl = r.normal(size=(6, 11)) * 2.0
    s, t = _eye_pair(O, z, tl)
    zt, tt = torch.from_numpy(z), torch.from_numpy(tl)
    for Ts, Tt in ((1.0, 2.0), (2.0, 0.7), (1.5, 1.5)):
        lp_s, lp_t = F.log_softmax(zt / Ts, -1), F.log_softmax(tt / Tt, -1)
        fwd = F.kl_div(lp_s, lp_t, log_target=True, reduction="none").sum(-1) * Ts * Ts
        rev = F.kl_div(lp_t, lp_s, log_target=True, reduction="none").sum(-1) * Ts * Ts
        for variant, ref in (("forward", fwd), ("reverse", rev), ("jeffreys", fwd + rev)):
            p = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=Ts,
                         teacher_temperature=Tt, kl_divergence=variant)
            _close(O.per_token(s, t, p)["kl"], ref.numpy(), rtol=1e-11, atol=1e-12,
                   what=f"{variant} KL T_s={Ts} T_t={Tt}")


def check_teacher_temperature_two_classes(O):
    """V = 2: Bernoulli KL(q || p) with q = sigmoid((t1-t0)/T_t), p = sigmoid((z1-z0)/T_s),
    times T_s^2."""
    r = _rng(31)
    z = r.normal(size=(6, 2)) * 1.5
    tl = r.normal(size=(6, 2)) * 1.5
    Ts, Tt = 1.2, 2.9
    ps = 1.0 / (1.0 + np.exp(-(z[:, 1] - z[:, 0]) / Ts))
    qt = 1.0 / (1.0 + np.exp(-(tl[:, 1] - tl[:, 0]) / Tt))
    ref = Ts * Ts * (qt * np.log(qt / ps) + (1 - qt) * np.log((1 - qt) / (1 - ps)))
    s, t = _eye_pair(O, z, tl)
    p = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=Ts, teacher_temperature=Tt)
    _close(O.per_token(s, t, p)["kl"], ref, rtol=1e-11, atol=1e-13, what="Bernoulli KL, T_t != T_s")


def check_teacher_temperature_unset_is_student(O):
    """teacher_temperature=None gives the same values and gradients as T_t = T_s."""
    s, t = _tied_case(O, k=12)
    y = np.array([1, 3, -100, 0, 9, 4])
    for variant in ("forward", "reverse"):
        a = O.Params(student_ce_weight=0.3, kl_weight=1.0, temperature=1.8, kl_divergence=variant)
        b = O.Params(student_ce_weight=0.3, kl_weight=1.0, temperature=1.8, teacher_temperature=1.8,
                     kl_divergence=variant)
        _close(O.forward(s, t, a, y)["loss"], O.forward(s, t, b, y)["loss"], rtol=1e-14)
        _close(O.backward(s, t, a, y)[0], O.backward(s, t, b, y)[0], rtol=1e-14, atol=1e-15)


def check_zero_teacher_probability(O):
    """Teacher logits of -inf are zero teacher probabilities: forward KL is
    T_s^2 * sum rel_entr(q, p) (scipy: rel_entr(0, y) = 0), reverse KL is +inf,
    and the forward-KL gradient stays finite with P_T = 0 on those columns."""
    from scipy.special import rel_entr, softmax as sp_softmax
    r = _rng(32)
    z = r.normal(size=(5, 10)) * 1.5
    tl = r.normal(size=(5, 10)) * 1.5
    tl[:, [2, 7]] = -np.inf
    tl[3, :6] = -np.inf
    Ts, Tt = 1.3, 0.9
    q = sp_softmax(tl / Tt, axis=1)
    pz = sp_softmax(z / Ts, axis=1)
    ref = Ts * Ts * rel_entr(q, pz).sum(axis=1)
    s = O.Student(hidden=z, weight=np.eye(10))
    t = O.Teacher("logits", logits=tl)
    p = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=Ts, teacher_temperature=Tt)
    _close(O.per_token(s, t, p)["kl"], ref, rtol=1e-11, atol=1e-13, what="KL with -inf teacher logits")
    g = O.logit_grad(s, t, p, None, np.arange(5), den=1.0)
    _close(g, Ts * (pz - q), rtol=1e-11, atol=1e-14, what="forward-KL gradient with P_T = 0")
    pr = O.Params(student_ce_weight=0.0, kl_weight=1.0, temperature=Ts, teacher_temperature=Tt,
                  kl_divergence="reverse")
    with np.errstate(invalid="ignore", divide="ignore"):
        assert np.isposinf(O.per_token(s, t, pr)["kl"]).all(), "reverse KL with P_T = 0 is +inf"


def check_zero_weight_term_is_absent(O):
    """With teacher_ce_weight = 0 the loss ignores the teacher CE, even where it
    is infinite (a label on a -inf teacher column): the loss equals the weighted
    mean of the student CE and the KL alone."""
    r = _rng(34)
    z = r.normal(size=(4, 6))
    tl = r.normal(size=(4, 6))
    tl[:, 5] = -np.inf
    y = np.array([5, 0, 5, 2])
    s = O.Student(hidden=z, weight=np.eye(6))
    t = O.Teacher("logits", logits=tl)
    p = O.Params(student_ce_weight=0.5, teacher_ce_weight=0.0, kl_weight=1.0, temperature=1.0)
    from scipy.special import rel_entr, softmax as sp_softmax
    ce = F.cross_entropy(torch.from_numpy(z), torch.from_numpy(y), reduction="none").numpy()
    kl = rel_entr(sp_softmax(tl, axis=1), sp_softmax(z, axis=1)).sum(1)
    _close(O.forward(s, t, p, y)["loss"], np.mean(0.5 * ce + kl), rtol=1e-12,
           what="zero-weighted infinite teacher CE")


def check_compact_valid_changes_only_ignored_kl(O):
    """compact_valid zeroes the per-token KL of ignored rows and leaves the
    loss, the valid rows' KL and the gradients exactly as they were (the
    ignored rows never entered them)."""
    s, t = _tied_case(O, n=6, d=5, v=10, k=13)
    y = np.array([3, -100, 9, -100, 0, 4])
    a = O.Params(student_ce_weight=0.7, kl_weight=1.0, temperature=2.0)
    b = O.Params(student_ce_weight=0.7, kl_weight=1.0, temperature=2.0, compact_valid=True)
    fa, fb = O.forward(s, t, a, y), O.forward(s, t, b, y)
    assert fa["loss"] == fb["loss"]
    valid = y != -100
    assert (fb["kl"][~valid] == 0).all() and (fa["kl"][~valid] > 0).all()
    assert np.array_equal(fa["kl"][valid], fb["kl"][valid])
    for ga, gb in zip(O.backward(s, t, a, y), O.backward(s, t, b, y)):
        assert np.array_equal(ga, gb)


def check_teacher_grad_autograd_library(O):
    """A teacher trained through its CE: autograd through w_s CE(z) + w_t CE(t)
    + w_kl KL(t.detach(), z) gives dH_t, dW_t (separate) and, tied, the
    shared weight's gradient as the student half plus the teacher half."""
    r = _rng(35)
    n, d, dt, v = 5, 4, 3, 11
    Hs, Ht = r.normal(size=(n, d)), r.normal(size=(n, d)) * 1.2
    Htt, Wt, W = r.normal(size=(n, dt)), r.normal(size=(v, dt)), r.normal(size=(v, d)) * 0.7
    y = np.array([3, -100, 10, 0, 7])
    yt = torch.from_numpy(y)
    valid = yt != -100
    for kind in ("tied", "separate"):
        for T, variant in ((1.0, "forward"), (1.7, "reverse")):
            p = O.Params(student_ce_weight=0.6, teacher_ce_weight=1.3, kl_weight=0.9,
                         temperature=T, kl_divergence=variant)
            W_ = torch.tensor(W, requires_grad=True)
            Hs_ = torch.tensor(Hs, requires_grad=True)
            if kind == "tied":
                Ht_ = torch.tensor(Ht, requires_grad=True)
                Wt_ = W_
            else:
                Ht_ = torch.tensor(Htt, requires_grad=True)
                Wt_ = torch.tensor(Wt, requires_grad=True)
            z, t = Hs_ @ W_.T, Ht_ @ Wt_.T
            ce_s = F.cross_entropy(z, yt, ignore_index=-100, reduction="none")
            ce_t = F.cross_entropy(t, yt, ignore_index=-100, reduction="none")
            lp_s, lp_t = F.log_softmax(z / T, -1), F.log_softmax(t.detach() / T, -1)
            if variant == "forward":
                kl = F.kl_div(lp_s, lp_t, log_target=True, reduction="none").sum(-1) * T * T
            else:
                kl = F.kl_div(lp_t, lp_s, log_target=True, reduction="none").sum(-1) * T * T
            loss = (0.6 * ce_s + 1.3 * ce_t + 0.9 * kl)[valid].sum() / float(valid.sum())
            loss.backward()
            s = O.Student(hidden=Hs, weight=W)
            te = O.Teacher("tied", hidden=Ht) if kind == "tied" else O.Teacher("separate", hidden=Htt, weight=Wt)
            dHs, dWs = O.backward(s, te, p, y)
            dHt, dWt = O.backward_teacher(s, te, p, y)
            _close(dHs, Hs_.grad.numpy(), rtol=1e-10, atol=1e-13, what=f"{kind} student dH")
            _close(dHt, Ht_.grad.numpy(), rtol=1e-10, atol=1e-13, what=f"{kind} teacher dH")
            if kind == "tied":
                _close(dWs + dWt, W_.grad.numpy(), rtol=1e-10, atol=1e-13, what="tied shared dW")
            else:
                _close(dWs, W_.grad.numpy(), rtol=1e-10, atol=1e-13, what="student dW")
                _close(dWt, Wt_.grad.numpy(), rtol=1e-10, atol=1e-13, what="teacher dW")


def check_teacher_grad_finite_differences(O):
    """Central differences of the teacher-CE part of the loss in H_t and W_t
    match backward_teacher (the KL part does not depend on a detached teacher)."""
    r = _rng(36)
    n, d, dt, v = 4, 3, 3, 7
    Hs, W = r.normal(size=(n, d)), r.normal(size=(v, d))
    Ht, Wt = r.normal(size=(n, dt)), r.normal(size=(v, dt))
    y = np.array([1, 6, -100, 2])
    p = O.Params(student_ce_weight=0.0, teacher_ce_weight=1.4, kl_weight=0.0, temperature=2.0)
    s = O.Student(hidden=Hs, weight=W)

    def loss(Ht_, Wt_):
        return O.forward(s, O.Teacher("separate", hidden=Ht_, weight=Wt_), p, y)["loss"] * 0.8

    dHt, dWt = O.backward_teacher(s, O.Teacher("separate", hidden=Ht, weight=Wt), p, y, grad_loss=0.8)
    h = 1e-6
    for X, G, which in ((Ht, dHt, "H_t"), (Wt, dWt, "W_t")):
        num = np.zeros_like(X)
        for ij in np.ndindex(*X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[ij] += h
            Xm[ij] -= h
            num[ij] = ((loss(Xp, Wt) - loss(Xm, Wt)) if which == "H_t" else
                       (loss(Ht, Xp) - loss(Ht, Xm))) / (2 * h)
        err = np.max(np.abs(num - G)) / np.max(np.abs(G))
        assert err < 1e-6, f"teacher finite differences d{which}: {err:.2e}"


def check_logit_grad_finite_differences(O):
    """Both sides given as logits (nemo KDLoss: student and teacher logits):
    central differences of the loss in the student logits match logit_grad for
    forward and reverse KL, with CE, a teacher temperature and an upstream
    gradient."""
    r = _rng(37)
    n, v = 5, 7
    z = r.normal(size=(n, v)) * 1.5
    tl = r.normal(size=(n, v)) * 1.5
    y = np.array([1, -100, 6, 0, 3])
    for variant, Tt in (("forward", None), ("reverse", 0.9), ("jeffreys", 1.6)):
        p = O.Params(student_ce_weight=0.4, kl_weight=1.1, temperature=2.0, teacher_temperature=Tt,
                     kl_divergence=variant, normalizer=3.0)
        t = O.Teacher("logits", logits=tl)

        def loss(z_):
            return O.forward(O.Student(logits=z_), t, p, y)["loss"] * 0.7

        g = O.logit_grad(O.Student(logits=z), t, p, y, np.arange(n), den=3.0, grad_loss=0.7)
        h = 1e-6
        num = np.zeros_like(z)
        for ij in np.ndindex(*z.shape):
            zp, zm = z.copy(), z.copy()
            zp[ij] += h
            zm[ij] -= h
            num[ij] = (loss(zp) - loss(zm)) / (2 * h)
        err = np.max(np.abs(num - g)) / np.max(np.abs(g))
        assert err < 1e-6, f"logit-gradient finite differences ({variant}): {err:.2e}"


def check_logits_teacher_matches_projection(O):
    """A dense cached teacher holding H_t W_t^T gives the separate teacher's
    per-token values and gradients."""
    r = _rng(33)
    n, d, dt, v = 6, 5, 4, 13
    Hs, W = r.normal(size=(n, d)), r.normal(size=(v, d)) * 0.6
    Ht, Wt = r.normal(size=(n, dt)), r.normal(size=(v, dt))
    y = np.array([0, 12, -100, 5, 7, 7])
    s = O.Student(hidden=Hs, weight=W)
    sep = O.Teacher("separate", hidden=Ht, weight=Wt)
    lg = O.Teacher("logits", logits=Ht @ Wt.T)
    p = O.Params(student_ce_weight=0.6, teacher_ce_weight=0.4, kl_weight=1.0, temperature=1.7,
                 teacher_temperature=1.1, kl_divergence="jeffreys")
    a, b = O.per_token(s, sep, p, y), O.per_token(s, lg, p, y)
    for k in ("student_ce", "teacher_ce", "kl"):
        _close(a[k], b[k], rtol=1e-12, atol=1e-13, what=f"logits teacher {k}")
    for ga, gb in zip(O.backward(s, sep, p, y), O.backward(s, lg, p, y)):
        _close(ga, gb, rtol=1e-12, atol=1e-14, what="logits teacher gradient")


def _topk_case(n=6, v=15, k=4, seed=10, zero_one=True):
    r = _rng(seed)
    z = r.normal(size=(n, v)) * 1.5
    idx = np.stack([r.choice(v, size=k, replace=False) for _ in range(n)])
    g = r.gamma(0.3, size=(n, k))
    p = g / g.sum(1, keepdims=True) * r.uniform(0.85, 0.99, size=(n, 1))
    if zero_one:
        p[0, 0] = 0.0  # a zero probability exercises 0 log 0 = 0
    return z, idx, p


def check_topk_dense_scatter(O):
    """The sparse objective equals the dense-scatter form, the pages' correctness
    baseline: q = p scattered to the vocabulary (0 elsewhere),
    L = sum_v q log q - sum_v q log_softmax(z), with 0 log 0 = 0."""
    z, idx, p = _topk_case()
    n, v = z.shape
    q = np.zeros((n, v))
    for i in range(n):
        q[i, idx[i]] = p[i]
    lsm = F.log_softmax(torch.from_numpy(z), -1).numpy()
    qlogq = np.where(q > 0, q * np.log(np.where(q > 0, q, 1.0)), 0.0)
    ref = qlogq.sum(1) - (q * lsm).sum(1)
    s = O.Student(logits=z)
    w = O.Teacher("topk", idx=idx, prob=p)
    got = O.per_token(s, w, O.Params(student_ce_weight=0.0, kl_weight=1.0))["kl"]
    _close(got, ref, rtol=1e-11, atol=1e-13, what="sparse = dense scatter")


def check_topk_full_support(O):
    """K = V with M = 1: the sparse objective is the dense forward KL with teacher
    probabilities p, i.e. kl_div(log_softmax(z), log p, log_target) summed."""
    r = _rng(11)
    n, v = 5, 8
    z = r.normal(size=(n, v))
    logits_t = r.normal(size=(n, v))
    p = torch.softmax(torch.from_numpy(logits_t), -1).numpy()
    idx = np.stack([r.permutation(v) for _ in range(n)])
    pp = np.take_along_axis(p, idx, 1)
    ref = F.kl_div(F.log_softmax(torch.from_numpy(z), -1), torch.from_numpy(np.log(p)),
                   log_target=True, reduction="none").sum(-1).numpy()
    got = O.per_token(O.Student(logits=z), O.Teacher("topk", idx=idx, prob=pp),
                      O.Params(student_ce_weight=0.0, kl_weight=1.0))["kl"]
    _close(got, ref, rtol=1e-11, atol=1e-13, what="full-support top-K = dense KL")


def check_topk_ce_bridge(O):
    """K = 1 with p = 1 on the label (M = 1) reduces the objective to CE(z, y)."""
    r = _rng(12)
    n, v = 6, 9
    z = r.normal(size=(n, v)) * 2
    y = r.integers(0, v, size=n)
    got = O.per_token(O.Student(logits=z), O.Teacher("topk", idx=y[:, None], prob=np.ones((n, 1))),
                      O.Params(student_ce_weight=0.0, kl_weight=1.0))["kl"]
    ref = F.cross_entropy(torch.from_numpy(z), torch.from_numpy(y), reduction="none").numpy()
    _close(got, ref, rtol=1e-12, atol=1e-13, what="top-K K=1 is CE")


def check_topk_mass_scaling(O):
    """Scaling every cached p by c changes the objective to
    c * L + c log c * M (from L = sum p log p - sum p z + M lse z)."""
    z, idx, p = _topk_case(seed=13, zero_one=False)
    c = 0.6
    s = O.Student(logits=z)
    prm = O.Params(student_ce_weight=0.0, kl_weight=1.0)
    a = O.per_token(s, O.Teacher("topk", idx=idx, prob=p), prm)["kl"]
    b = O.per_token(s, O.Teacher("topk", idx=idx, prob=c * p), prm)["kl"]
    _close(b, c * a + c * math.log(c) * p.sum(1), rtol=1e-11, atol=1e-13, what="mass scaling")


# ---------------------------------------------------------------------------
# Reduction (nemo kd_loss, KDLoss.forward num_batch_labels; orda reduction)
# ---------------------------------------------------------------------------

def check_reduction_modes(O):
    """mean divides by the valid count, sum by 1, a normaliser by itself; the
    mean of CE equals F.cross_entropy(reduction='mean', ignore_index)."""
    s, t = _tied_case(O, n=8, d=4, v=10, k=14)
    y = np.array([1, -100, 3, 9, -100, 0, 4, 4])
    z = torch.from_numpy(s.hidden @ s.weight.T)
    ce_mean = F.cross_entropy(z, torch.from_numpy(y), ignore_index=-100).item()
    ce_sum = F.cross_entropy(z, torch.from_numpy(y), ignore_index=-100, reduction="sum").item()
    base = dict(student_ce_weight=1.0, kl_weight=0.0)
    _close(O.forward(s, t, O.Params(**base, reduction="mean"), y)["loss"], ce_mean, what="mean")
    _close(O.forward(s, t, O.Params(**base, reduction="sum"), y)["loss"], ce_sum, what="sum")
    _close(O.forward(s, t, O.Params(**base, normalizer=40.0), y)["loss"], ce_sum / 40.0,
           what="normalizer")


def check_all_ignored(O):
    """Every row ignored: loss 0 and zero gradients (reading R4)."""
    s, t = _tied_case(O, n=4, d=3, v=6, k=15)
    y = np.full(4, -100)
    p = O.Params(student_ce_weight=1.0, kl_weight=1.0, temperature=2.0)
    out = O.forward(s, t, p, y)
    assert out["loss"] == 0.0 and out["den"] == 1.0
    dH, dW = O.backward(s, t, p, y)
    assert not dH.any() and not dW.any()


def check_out_of_range_label_is_ignored(O):
    """A label outside [0, V) behaves exactly like ignore_index."""
    s, t = _tied_case(O, n=5, d=3, v=7, k=16)
    p = O.Params(student_ce_weight=1.0, kl_weight=1.0, temperature=1.5)
    a = O.forward(s, t, p, np.array([1, 7, 2, -5, 0]))
    b = O.forward(s, t, p, np.array([1, -100, 2, -100, 0]))
    _close(a["loss"], b["loss"], what="out-of-range label")
    _close(a["student_ce"], b["student_ce"], what="out-of-range label CE")


# ---------------------------------------------------------------------------
# Gradients
# ---------------------------------------------------------------------------

def _fd_cases(O):
    r = _rng(20)
    n, d, v, dt = 4, 5, 9, 3
    Hs = r.normal(size=(n, d))
    W = r.normal(size=(v, d)) * 0.8
    Ht = r.normal(size=(n, d)) * 1.2
    Htt = r.normal(size=(n, dt))
    Wt = r.normal(size=(v, dt))
    y = np.array([2, -100, 8, 0])
    idx = np.stack([r.choice(v, size=3, replace=False) for _ in range(n)])
    g = r.gamma(0.5, size=(n, 3))
    pk = g / g.sum(1, keepdims=True) * 0.9
    tl_inf = r.normal(size=(n, v)) * 1.5
    tl_inf[:, [1, 4]] = -np.inf
    return [
        ("tied", O.Teacher("tied", hidden=Ht), y,
         O.Params(student_ce_weight=0.7, kl_weight=1.3, temperature=2.0)),
        ("separate", O.Teacher("separate", hidden=Htt, weight=Wt), y,
         O.Params(student_ce_weight=1.0, teacher_ce_weight=1.0, kl_weight=1.0, temperature=1.0)),
        ("topk", O.Teacher("topk", idx=idx, prob=pk), None,
         O.Params(student_ce_weight=0.0, kl_weight=1.0)),
        ("sum", O.Teacher("tied", hidden=Ht), y,
         O.Params(student_ce_weight=1.0, kl_weight=0.5, temperature=0.8, reduction="sum")),
        ("reverse", O.Teacher("tied", hidden=Ht), y,
         O.Params(student_ce_weight=0.4, kl_weight=1.1, temperature=2.0, kl_divergence="reverse")),
        ("jeffreys", O.Teacher("separate", hidden=Htt, weight=Wt), y,
         O.Params(student_ce_weight=1.0, kl_weight=0.9, temperature=1.3, kl_divergence="jeffreys")),
        ("teacher_T", O.Teacher("separate", hidden=Htt, weight=Wt), y,
         O.Params(student_ce_weight=0.8, kl_weight=1.2, temperature=1.4, teacher_temperature=2.3,
                  kl_divergence="jeffreys")),
        ("logits_inf", O.Teacher("logits", logits=tl_inf), y,
         O.Params(student_ce_weight=0.5, kl_weight=1.1, temperature=1.5, teacher_temperature=0.8)),
    ], Hs, W


def check_grad_finite_differences(O):
    """Central differences of the reduced loss (float64, h = 1e-6) match the
    analytic dH and dW to 1e-6 relative, including the upstream gradient."""
    cases, Hs, W = _fd_cases(O)
    h = 1e-6
    for name, t, y, p in cases:
        g_up = 1.7

        # The teacher is detached: a tied teacher keeps projecting with the
        # unperturbed W while the student's W moves.
        t_fixed = O.Teacher("separate", hidden=t.hidden, weight=W.copy()) if t.kind == "tied" else t

        def loss(H_, W_):
            return O.forward(O.Student(hidden=H_, weight=W_), t_fixed, p, y)["loss"] * g_up

        dH, dW = O.backward(O.Student(hidden=Hs, weight=W), t, p, y, grad_loss=g_up)
        for X, G, which in ((Hs, dH, "H"), (W, dW, "W")):
            num = np.zeros_like(X)
            for ij in np.ndindex(*X.shape):
                Xp = X.copy()
                Xm = X.copy()
                Xp[ij] += h
                Xm[ij] -= h
                if which == "H":
                    num[ij] = (loss(Xp, W) - loss(Xm, W)) / (2 * h)
                else:
                    num[ij] = (loss(Hs, Xp) - loss(Hs, Xm)) / (2 * h)
            err = np.max(np.abs(num - G)) / max(np.max(np.abs(G)), 1e-30)
            assert err < 1e-6, f"finite differences {name} d{which}: rel err {err:.2e}"


def check_grad_autograd_library(O):
    """dH and dW equal torch autograd through a loss built from library calls
    (F.cross_entropy with ignore_index, F.kl_div on F.log_softmax)."""
    cases, Hs, W = _fd_cases(O)
    for name, t, y, p in cases:
        if t.kind in ("topk", "logits"):  # kl_div has no 0 * log 0 = 0 for -inf targets
            continue
        H_ = torch.tensor(Hs, requires_grad=True)
        W_ = torch.tensor(W, requires_grad=True)
        z = H_ @ W_.T
        tl = torch.from_numpy(t.hidden @ (s_w := (W if t.kind == "tied" else t.weight)).T)
        del s_w
        yt = torch.from_numpy(y)
        valid = yt != -100
        T = p.temperature
        Tt = T if p.teacher_temperature is None else p.teacher_temperature
        ce = F.cross_entropy(z, yt, ignore_index=-100, reduction="none")
        lp_s, lp_t = F.log_softmax(z / T, -1), F.log_softmax(tl / Tt, -1)
        fwd = F.kl_div(lp_s, lp_t, log_target=True, reduction="none").sum(-1) * T * T
        rev = F.kl_div(lp_t, lp_s, log_target=True, reduction="none").sum(-1) * T * T
        kl = {"forward": fwd, "reverse": rev, "jeffreys": fwd + rev}[p.kl_divergence]
        total = (p.student_ce_weight * ce + p.kl_weight * kl)[valid].sum()
        den = float(valid.sum()) if p.reduction == "mean" else 1.0
        (total / den).backward()
        dH, dW = O.backward(O.Student(hidden=Hs, weight=W), t, p, y)
        _close(dH, H_.grad.numpy(), rtol=1e-10, atol=1e-13, what=f"autograd dH {name}")
        _close(dW, W_.grad.numpy(), rtol=1e-10, atol=1e-13, what=f"autograd dW {name}")


def check_grad_invariants(O):
    """Every logit-gradient row sums to zero, hence sum_v dW[v, :] = 0; and
    tr(dH^T H) = tr(dW^T W) (both equal sum dz * z)."""
    cases, Hs, W = _fd_cases(O)
    for name, t, y, p in cases:
        dH, dW = O.backward(O.Student(hidden=Hs, weight=W), t, p, y)
        scale = np.abs(dW).max()
        _close(dW.sum(0) / scale, 0.0, atol=1e-12, what=f"sum_v dW {name}")
        a = (dH * Hs).sum()
        b = (dW * W).sum()
        _close(a, b, rtol=1e-10, atol=1e-13, what=f"trace identity {name}")


def check_backward_rows_consistent(O):
    """dH for a subset of rows equals those rows of the full dH."""
    cases, Hs, W = _fd_cases(O)
    for name, t, y, p in cases:
        s = O.Student(hidden=Hs, weight=W)
        dH, _ = O.backward(s, t, p, y)
        out = O.forward(s, t, p, y)
        rows = np.array([3, 1])
        _close(O.backward_rows(s, t, p, y, rows, out["den"]), dH[rows], what=f"rows {name}")


def check_weight_grad_rows_finite_differences(O):
    """dW on a subset of vocabulary rows matches central differences of the
    reduced loss in those rows of W (float64, h = 1e-6, 1e-6 relative), for
    every teacher kind; rows given out of order and with the last row."""
    cases, Hs, W = _fd_cases(O)
    h = 1e-6
    vrows = np.array([7, 0, 8, 3])
    for name, t, y, p in cases:
        g_up = 0.6
        t_fixed = O.Teacher("separate", hidden=t.hidden, weight=W.copy()) if t.kind == "tied" else t

        def loss(W_):
            return O.forward(O.Student(hidden=Hs, weight=W_), t_fixed, p, y)["loss"] * g_up

        s = O.Student(hidden=Hs, weight=W)
        den = O.forward(s, t, p, y)["den"]
        got = O.weight_grad_rows(s, t, p, y, vrows, den, grad_loss=g_up)
        num = np.zeros_like(got)
        for a, v in enumerate(vrows):
            for j in range(W.shape[1]):
                Wp = W.copy()
                Wm = W.copy()
                Wp[v, j] += h
                Wm[v, j] -= h
                num[a, j] = (loss(Wp) - loss(Wm)) / (2 * h)
        err = np.max(np.abs(num - got)) / max(np.max(np.abs(got)), 1e-30)
        assert err < 1e-6, f"weight_grad_rows finite differences {name}: {err:.2e}"


ALL = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
