"""HIP path vs the float64 oracle, element by element, through the C ABI.

Sizes are chosen so the oracle finishes in seconds while the problem still
spans several 128-row tiles, several vocabulary slices / chunks, and ragged
tails in tokens and vocabulary.
"""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_common import (assert_grad, assert_scalar, assert_tokens, full_parity, make_runner,
                        oracle_problem, params_of, run_gpu, say, to_np)
from kl_knowledge_distillation_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

C1 = WORKLOADS["tiny_tied_fp32"]
C2 = WORKLOADS["quickstart_tied_bf16"]
C3 = WORKLOADS["separate_bf16"]
C4 = WORKLOADS["topk_bf16"]
C5 = WORKLOADS["scorer_bf16"]
C6 = WORKLOADS["quickstart_logits_bf16"]
C7 = WORKLOADS["kdloss_logits_bf16"]

SMALL = {
    "tiny_fp32": C1,
    "tiny_fp32_ragged": C1.scaled(n=70, v=1000, ignore_frac=0.2),
    "quickstart_small": C2.scaled(n=300, d=512, v=3000),
    "quickstart_ragged": C2.scaled(n=130, d=136, v=1029),
    "separate_small": C3.scaled(n=200, d=256, d_t=512, v=2000),
    "separate_small_T2": C3.scaled(n=200, d=256, d_t=512, v=2000, temperature=2.0,
                                   ignore_frac=0.1),
    "topk_small": C4.scaled(n=300, d=512, v=5000),
    "topk_ragged": C4.scaled(n=129, d=264, v=1031, k=7),
    # more entries per row than the prep sorts in LDS (the counting path)
    "topk_many": C4.scaled(n=40, d=256, v=3000, k=1100),
    "scorer_small": C5.scaled(n=300, d_t=512, v=5000),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_parity(name):
    full_parity(SMALL[name])


# Contractions of 1, 2 and 3 K steps of 64 on the pipelined bf16 path: the
# main loop's prologue alone, its last-two-steps loop alone, and one step of
# its copy loop (hidden sizes 64 / 128 / 192; token counts whose dW
# contraction, rounded up to 64, is 1, 2 or 3 steps too).
SHORT_K = {
    "tied_d64_n60": C2.scaled(n=60, d=64, v=1000),
    "tied_d128_n100": C2.scaled(n=100, d=128, v=1300),
    "tied_d192_n170": C2.scaled(n=170, d=192, v=900),
    "topk_d64_n100": C4.scaled(n=100, d=64, v=1500, k=8),
    "topk_d192_n170": C4.scaled(n=170, d=192, v=1500, k=8),
    "separate_d64_dt192": C3.scaled(n=130, d=64, d_t=192, v=1100),
    "separate_d192_dt64": C3.scaled(n=60, d=192, d_t=64, v=1100),
    "dense_teacher_d64": C6.scaled(n=90, d=64, v=1024),
    "scorer_dt64": C5.scaled(n=100, d_t=64, v=2000),
    "scorer_dt128": C5.scaled(n=170, d_t=128, v=1300),
}


@pytest.mark.parametrize("name", list(SHORT_K))
def test_short_contractions(name):
    full_parity(SHORT_K[name].scaled(name=f"short_{name}"), vocab_chunk=512)


@pytest.mark.parametrize("chunk", [128, 384, 1024])
def test_chunk_and_slice_sizes(chunk):
    full_parity(C2.scaled(n=260, d=256, v=2100, name=f"quickstart_chunk{chunk}"), vocab_chunk=chunk)


@pytest.mark.parametrize("chunk", [256, 2048, 8192, 16384])
def test_scorer_chunk_sweep(chunk):
    full_parity(C5.scaled(n=256, d_t=256, v=9000), vocab_chunk=chunk)


# Vocabulary spread over several forward launches (their records folded into a
# running record between launches), for every tile mode.
CHUNKED_FORWARD = {
    "topk": (C4.scaled(n=300, d=512, v=5000), 1024),
    "topk_staged": (C4.scaled(n=129, d=264, v=1031, k=7), 256),
    "separate_T2": (C3.scaled(n=200, d=256, d_t=512, v=2000, temperature=2.0), 512),
    "tied_compact": (C2.scaled(n=300, d=512, v=3000, ignore_frac=0.3, compact_valid=True), 768),
    "tied_jeffreys": (C2.scaled(n=260, d=256, v=2100, kl_divergence="jeffreys"), 512),
    "dense_teacher_logits": (C6.scaled(n=300, d=256, v=2000), 512),
}


@pytest.mark.parametrize("name", list(CHUNKED_FORWARD))
def test_chunked_forward(name):
    w, chunk = CHUNKED_FORWARD[name]
    full_parity(w.scaled(name=f"{w.name}_{name}"), vocab_chunk=chunk)


# dW and dH of a chunk share one launch, in which each XCD runs its tiles of one
# kind before the other's. With 8192 tokens, hidden 2048 and 1024-column chunks
# the dW tiles are few and long (K = 8192) next to many short dH tiles (K = the
# chunk), so the host puts the dW tiles first on both chunks (the full one and
# the 256-column last one); every element of dH and dW is compared.
def test_dual_launch_dw_tiles_first():
    full_parity(C4.scaled(n=8192, d=2048, v=1280, k=8, name="topk_dual_dw_first"), vocab_chunk=1024)


def test_reductions_and_normalizer():
    w = C2.scaled(n=200, d=256, v=1500)
    x = make_inputs(w, "cuda", seed=3)
    s, t, labels = oracle_problem(w, x)
    for red, norm in (("sum", 0.0), ("mean", 0.0), ("mean", 777.0)):
        say(f"[reduction] {red} normalizer={norm}")
        r = make_runner(w, x, reduction=red)
        r.p.normalizer = norm
        r.forward()
        dh = torch.empty((r.n, r.d), dtype=torch.float32, device="cuda")
        dw = torch.empty((r.v, r.d), dtype=torch.float32, device="cuda")
        g = torch.tensor(0.37, device="cuda")
        r.backward(dh, dw, grad_loss=g)
        torch.cuda.synchronize()
        p = params_of(w)
        p.reduction, p.normalizer = red, norm
        ref = O.forward(s, t, p, labels)
        assert_scalar(float(r.loss), ref["loss"], "bf16", f"loss {red}")
        dH, dW = O.backward(s, t, p, labels, grad_loss=0.37)
        assert_grad(to_np(dh), dH, "bf16", f"dH {red}")
        assert_grad(to_np(dw), dW, "bf16", f"dW {red}")


def test_accumulate_adds_into_gradients():
    w = C1.scaled(n=96, v=700)
    x = make_inputs(w, "cuda", seed=5)
    r, dh, dw = run_gpu(w, x)
    dh2 = torch.full_like(dh, 0.5)
    dw2 = torch.full_like(dw, -0.25)
    r.forward()
    r.backward(dh2, dw2, accumulate=True)
    torch.cuda.synchronize()
    assert torch.allclose(dh2, dh + 0.5, rtol=1e-6, atol=1e-6)
    assert torch.allclose(dw2, dw - 0.25, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("which", ["dh", "dw"])
def test_one_gradient_at_a_time(which):
    """Asking for dH or dW alone takes the single-GEMM launches (both together
    share one); each matches the oracle, and dW alone equals the joint launch's
    dW bit for bit (same tiles, same order)."""
    w = C2.scaled(n=600, d=512, v=3000)
    x = make_inputs(w, "cuda", seed=12)
    r, dh, dw = run_gpu(w, x)
    s, t, labels = oracle_problem(w, x)
    dH, dW = O.backward(s, t, params_of(w), labels)
    g = torch.empty_like(dh if which == "dh" else dw)
    r.forward()
    r.backward(g if which == "dh" else None, g if which == "dw" else None)
    torch.cuda.synchronize()
    if which == "dh":
        assert_grad(to_np(g), dH, "bf16", "dH alone")
    else:
        assert_grad(to_np(g), dW, "bf16", "dW alone")


@pytest.mark.parametrize("kl", ["forward", "reverse", "jeffreys"])
def test_kl_exactly_zero_for_identical_teacher(kl):
    """Tied teacher with H_t = H_s: the two logit tiles are computed by the same
    MFMA sequence, so every statistic matches and KL is 0 bit for bit in every
    direction."""
    w = C2.scaled(n=260, d=256, v=3000, kl_divergence=kl)
    x = make_inputs(w, "cuda", seed=1)
    x["teacher_hidden"] = x["student_hidden"].clone()
    r, dh, dw = run_gpu(w, x)
    assert torch.count_nonzero(r.kl).item() == 0


def test_deterministic_bitwise():
    w = C2.scaled(n=300, d=256, v=2500)
    x = make_inputs(w, "cuda", seed=2)
    outs = []
    for _ in range(2):
        r, dh, dw = run_gpu(w, x, vocab_chunk=1024)
        outs.append((r.loss.clone(), r.kl.clone(), r.student_ce.clone(), dh.clone(), dw.clone()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_out_of_range_label_flag():
    w = C2.scaled(n=150, d=128, v=900)
    x = make_inputs(w, "cuda", seed=4)
    lab = x["labels"].clone()
    lab[7] = w.v + 5
    lab[11] = -3
    x["labels"] = lab
    r, dh, dw = run_gpu(w, x)
    assert r.read_status() == 1
    s, t, labels = oracle_problem(w, x)
    ref = O.forward(s, t, params_of(w), labels)  # the oracle treats them as ignored
    assert_tokens(to_np(r.student_ce), ref["student_ce"], "bf16", "ce with bad labels")
    assert_scalar(float(r.loss), ref["loss"], "bf16", "loss with bad labels")
    dH, dW = O.backward(s, t, params_of(w), labels)
    assert_grad(to_np(dh), dH, "bf16", "dH with bad labels")


def test_topk_out_of_range_index_flag():
    """Top-K indices outside [0, V) are never used as addresses: the device
    status flags them, and every other row keeps its value."""
    w = C4.scaled(n=64, d=256, v=2000, k=10)
    x = make_inputs(w, "cuda", seed=8)
    idx = x["topk_idx"].clone()
    idx[5, 3] = w.v + 7
    idx[9, 0] = -2
    x["topk_idx"] = idx
    r, dh, dw = run_gpu(w, x)
    assert r.read_status() == 1
    good = np.array([i for i in range(w.n) if i not in (5, 9)])
    s = O.Student(hidden=to_np(x["student_hidden"]).astype(np.float64)[good],
                  weight=to_np(x["weight"]).astype(np.float64))
    t = O.Teacher("topk", idx=to_np(idx).astype(np.int64)[good],
                  prob=to_np(x["topk_prob"]).astype(np.float64)[good])
    ref = O.forward(s, t, params_of(w), None)
    assert_tokens(to_np(r.kl)[good], ref["kl"], "bf16", "top-K kl beside bad indices")


def test_all_labels_ignored():
    w = C2.scaled(n=140, d=128, v=700)
    x = make_inputs(w, "cuda", seed=6)
    x["labels"] = torch.full_like(x["labels"], w.ignore_index)
    r, dh, dw = run_gpu(w, x)
    assert float(r.loss) == 0.0
    assert torch.count_nonzero(dh).item() == 0 and torch.count_nonzero(dw).item() == 0


def test_full_quickstart_tied_bf16():
    """Whole quickstart-shaped problem (N=4096, D=2048, V=32000), every output."""
    full_parity(C2)


def test_full_tiny_fp32_default_and_chunked():
    full_parity(C1)
    full_parity(C1, vocab_chunk=256)


KL_VARIANTS = {
    "tied_T2_reverse": C2.scaled(n=300, d=512, v=3000, kl_divergence="reverse"),
    "tied_T2_jeffreys_ragged": C2.scaled(n=130, d=136, v=1029, kl_divergence="jeffreys",
                                         ignore_frac=0.2),
    "separate_T1.3_jeffreys_tce": C3.scaled(n=200, d=256, d_t=512, v=2000, temperature=1.3,
                                            kl_divergence="jeffreys", teacher_ce_weight=0.5),
    "separate_T1_reverse": C3.scaled(n=200, d=256, d_t=512, v=2000, kl_divergence="reverse"),
    "fp32_T2_reverse": C1.scaled(n=70, v=1000, kl_divergence="reverse"),
    "fp32_T2_jeffreys": C1.scaled(kl_divergence="jeffreys"),
    "scorer_reverse": C5.scaled(n=300, d_t=512, v=5000, kl_divergence="reverse"),
}


@pytest.mark.parametrize("name", list(KL_VARIANTS))
def test_kl_variants(name):
    """Reverse KL(P_S || P_T) and the Jeffreys sum, forward and backward, against
    the oracle, on the tied, separate, fp32 and logits-input paths."""
    w = KL_VARIANTS[name]
    full_parity(w)
    if w.dtype == "fp32":
        full_parity(w, vocab_chunk=256)


TEACHER_CASES = {
    # dense cached teacher logits: pipelined bf16 with vector loads (V % 4 == 0)
    "logits_small": C6.scaled(n=300, d=512, v=3000),
    # staged bf16 (D % 64 != 0) with element loads (V % 4 != 0), ragged tiles
    "logits_ragged": C6.scaled(n=130, d=136, v=1029, ignore_frac=0.2),
    "logits_fp32": C1.scaled(teacher="logits", teacher_temperature=0.7),
    # 30% of the columns -inf in every row: zero teacher probabilities
    "logits_neg_inf": C6.scaled(n=260, d=256, v=2100, teacher_neg_inf_frac=0.3),
    "logits_jeffreys_tce": C6.scaled(n=200, d=256, v=2048, kl_divergence="jeffreys",
                                     teacher_ce_weight=0.5),
    # teacher temperature apart from the student's on the projected teachers
    "tied_Ts2_Tt1": C2.scaled(n=300, d=512, v=3000, teacher_temperature=1.0, teacher_ce_weight=0.3),
    "separate_Ts1.5_Tt3_reverse_tce": C3.scaled(n=200, d=256, d_t=512, v=2000, temperature=1.5,
                                                teacher_temperature=3.0, kl_divergence="reverse"),
    "fp32_Ts2_Tt0.6_jeffreys": C1.scaled(teacher_temperature=0.6, kl_divergence="jeffreys"),
    "scorer_Tt2": C5.scaled(n=300, d_t=512, v=5000, teacher_temperature=2.0),
}


@pytest.mark.parametrize("name", list(TEACHER_CASES))
def test_teacher_logits_and_temperature(name):
    """Dense cached teacher logits (with -inf entries) and a teacher temperature
    of its own, forward and backward, against the oracle."""
    w = TEACHER_CASES[name]
    full_parity(w)
    if w.dtype == "fp32":
        full_parity(w, vocab_chunk=256)


def test_infinite_teacher_ce_with_zero_weight():
    """Labels on -inf teacher columns: the requested per-token teacher CE is +inf
    there, and with teacher_ce_weight = 0 the loss stays finite and equal to the
    oracle's (a zero-weighted term is left out)."""
    w = C6.scaled(n=200, d=256, v=2048, teacher_neg_inf_frac=0.5)
    x = make_inputs(w, "cuda", seed=9)
    r = make_runner(w, x, want_teacher_ce=True)
    r.forward()
    torch.cuda.synchronize()
    s, t, labels = oracle_problem(w, x)
    ref = O.forward(s, t, params_of(w), labels)
    tce = to_np(r.teacher_ce).astype(np.float64)
    inf_rows = np.isinf(ref["teacher_ce"]) & ref["valid"]
    assert inf_rows.sum() > 10
    assert np.isposinf(tce[inf_rows]).all()
    assert_tokens(tce[~inf_rows], ref["teacher_ce"][~inf_rows], "bf16", "finite teacher CE",
                  ref["valid"][~inf_rows])
    assert np.isfinite(float(r.loss))
    assert_scalar(float(r.loss), ref["loss"], "bf16", "loss")


COMPACT_CASES = {
    "tied_pipe": C2.scaled(n=300, d=512, v=3000, ignore_frac=0.3, compact_valid=True),
    "tied_reverse_pipe": C2.scaled(n=520, d=256, v=2100, ignore_frac=0.4, kl_divergence="reverse",
                                   compact_valid=True),
    "separate_T2_tce": C3.scaled(n=200, d=256, d_t=512, v=2000, temperature=2.0, ignore_frac=0.25,
                                 compact_valid=True),
    "ragged_staged": C2.scaled(n=130, d=136, v=1029, ignore_frac=0.5, compact_valid=True),
    "fp32": C1.scaled(compact_valid=True),
}


@pytest.mark.parametrize("name", list(COMPACT_CASES))
def test_compacted_valid_rows(name):
    """Rows with an ignored label left out of every projection: loss, gradients
    and the valid rows' terms as the oracle gives them, zeros on the others."""
    w = COMPACT_CASES[name]
    full_parity(w)
    if w.dtype == "fp32":
        full_parity(w, vocab_chunk=256)


def test_compacted_all_ignored_and_accumulate():
    """No usable label: nothing is projected, loss 0, dH and dW 0; with
    accumulate the gradients keep their values (the left-out rows of dH too)."""
    w = C2.scaled(n=200, d=256, v=1500, compact_valid=True)
    x = make_inputs(w, "cuda", seed=7)
    x["labels"] = torch.full_like(x["labels"], w.ignore_index)
    r, dh, dw = run_gpu(w, x)
    assert float(r.loss) == 0.0 and torch.count_nonzero(r.kl).item() == 0
    assert torch.count_nonzero(dh).item() == 0 and torch.count_nonzero(dw).item() == 0
    w = C2.scaled(n=300, d=256, v=1500, ignore_frac=0.3, compact_valid=True)
    x = make_inputs(w, "cuda", seed=8)
    r, dh, dw = run_gpu(w, x)
    dh2 = torch.full_like(dh, 0.5)
    dw2 = torch.full_like(dw, -0.25)
    r.forward()
    r.backward(dh2, dw2, accumulate=True)
    torch.cuda.synchronize()
    assert torch.allclose(dh2, dh + 0.5, rtol=1e-6, atol=1e-6)
    assert torch.allclose(dw2, dw - 0.25, rtol=1e-6, atol=1e-6)
    ignored = (x["labels"] == w.ignore_index)
    assert torch.count_nonzero(dh[ignored]).item() == 0


TEACHER_TRAIN_CASES = {
    "tied_pipe": C2.scaled(n=300, d=512, v=3000, teacher_ce_weight=0.7),
    "tied_compact": C2.scaled(n=300, d=256, v=2100, teacher_ce_weight=1.0, ignore_frac=0.3,
                              compact_valid=True),
    "separate_Ts1.5_Tt2.5": C3.scaled(n=200, d=256, d_t=512, v=2000, temperature=1.5,
                                      teacher_temperature=2.5, teacher_ce_weight=0.5),
    "ragged_staged": C2.scaled(n=130, d=136, v=1029, teacher_ce_weight=1.0, ignore_frac=0.2),
    "fp32": C1.scaled(teacher_ce_weight=1.0),
}


@pytest.mark.parametrize("name", list(TEACHER_TRAIN_CASES))
def test_teacher_trained_through_its_ce(name):
    """kd_loss_bwd_teacher: dH_t and dW_t of w_t CE(t) against the oracle; with
    accumulate the second call adds the same gradients again."""
    w = TEACHER_TRAIN_CASES[name]
    say(f"[teacher ce] {name}")
    x = make_inputs(w, "cuda", seed=3)
    r = make_runner(w, x)
    r.forward()
    dht = torch.empty((r.n, r.dt), dtype=torch.float32, device="cuda")
    dwt = torch.empty((r.v, r.dt), dtype=torch.float32, device="cuda")
    r.backward_teacher(dht, dwt)
    torch.cuda.synchronize()
    s, t, labels = oracle_problem(w, x)
    dHt, dWt = O.backward_teacher(s, t, params_of(w), labels)
    assert_grad(to_np(dht), dHt, w.dtype, f"{name} teacher dH")
    assert_grad(to_np(dwt), dWt, w.dtype, f"{name} teacher dW")
    dht2, dwt2 = dht.clone(), dwt.clone()
    r.backward_teacher(dht2, dwt2, accumulate=True)
    torch.cuda.synchronize()
    assert torch.allclose(dht2, 2 * dht, rtol=1e-6, atol=1e-7)
    assert torch.allclose(dwt2, 2 * dwt, rtol=1e-6, atol=1e-7)


def test_teacher_gradient_zero_without_teacher_ce():
    w = C2.scaled(n=200, d=256, v=1500)
    x = make_inputs(w, "cuda", seed=4)
    r = make_runner(w, x)
    r.forward()
    dht = torch.full((r.n, r.dt), 3.0, dtype=torch.float32, device="cuda")
    dwt = torch.full((r.v, r.dt), 3.0, dtype=torch.float32, device="cuda")
    r.backward_teacher(dht, dwt)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dht).item() == 0 and torch.count_nonzero(dwt).item() == 0


BOTH_LOGITS_CASES = {
    "bf16_vec": C7.scaled(n=300, v=3000),
    "bf16_ragged_rows": C7.scaled(n=130, v=1029, ignore_frac=0.2),
    "fp32": C7.scaled(n=64, v=1024, dtype="fp32"),
    "reverse_Tt": C7.scaled(n=200, v=2048, kl_divergence="reverse", teacher_temperature=1.3),
    "jeffreys_ce": C7.scaled(n=200, v=2048, kl_divergence="jeffreys", student_ce_weight=0.5,
                             teacher_ce_weight=0.25),
    "neg_inf_T1": C7.scaled(n=260, v=2100, temperature=1.0, teacher_neg_inf_frac=0.3),
    # T_s neither 1 nor 2: the T = 1 student terms from exponentials of their own
    "T1.5_jeffreys_ce": C7.scaled(n=150, v=2500, temperature=1.5, kl_divergence="jeffreys",
                                  student_ce_weight=0.7),
    # rows split into slices of two steps each, the last one ragged
    "multi_step_slices": C7.scaled(n=1000, v=20000, student_ce_weight=0.3),
    # a row shorter than one step: one slice per row
    "one_slice": C7.scaled(n=100, v=700),
}


@pytest.mark.parametrize("name", list(BOTH_LOGITS_CASES))
def test_both_logits_given(name):
    """Student and teacher logits both given (row kernels): per-token terms and
    loss, then the gradient to the student logits, against the oracle."""
    w = BOTH_LOGITS_CASES[name]
    full_parity(w, grads=False)
    x = make_inputs(w, "cuda", seed=0)
    r = make_runner(w, x, want_grads=False)
    r.forward()
    d = torch.empty((r.n, r.v), dtype=w.torch_dtype, device="cuda")
    r.backward_logits(d)
    torch.cuda.synchronize()
    s, t, labels = oracle_problem(w, x)
    p = params_of(w)
    ref = O.forward(s, t, p, labels)
    g = O.logit_grad(s, t, p, labels, np.arange(w.n), ref["den"])
    assert_grad(to_np(d), g, w.dtype, f"{name} d student logits")
    d2 = d.clone()
    r.backward_logits(d2, accumulate=True)
    torch.cuda.synchronize()
    assert_grad(to_np(d2), 2 * g, w.dtype, f"{name} accumulated")


def test_reverse_kl_infinite_for_zero_teacher_probability():
    """Reverse KL with -inf teacher columns (reading R20): +inf on every row,
    given logits and dense-teacher paths alike."""
    for w in (C7.scaled(n=130, v=1024, kl_divergence="reverse", teacher_neg_inf_frac=0.2),
              C6.scaled(n=130, d=256, v=1024, kl_divergence="reverse", teacher_neg_inf_frac=0.2)):
        x = make_inputs(w, "cuda", seed=5)
        r = make_runner(w, x, want_grads=False)
        r.forward()
        torch.cuda.synchronize()
        assert torch.isposinf(r.kl).all(), w.name


def test_full_quickstart_logits_teacher_bf16():
    """Quickstart shape with a dense cached teacher (N=4096, D=2048, V=32000,
    T_s = 2, T_t = 1.5), every output."""
    full_parity(C6)


@pytest.mark.parametrize("want", [True, False])
def test_teacher_ce_on_request_at_temperature_2(want):
    """Teacher CE weight 0 at T = 2: the per-token teacher CE (taken at T = 1) is
    computed when asked for and left at zero otherwise; the loss is the same."""
    w = C2.scaled(n=260, d=256, v=2100)
    x = make_inputs(w, "cuda", seed=8)
    r = make_runner(w, x, want_teacher_ce=want)
    r.forward()
    torch.cuda.synchronize()
    s, t, labels = oracle_problem(w, x)
    ref = O.forward(s, t, params_of(w), labels)
    assert_scalar(float(r.loss), ref["loss"], "bf16", "loss")
    assert_tokens(to_np(r.kl), ref["kl"], "bf16", "kl")
    if want:
        assert_tokens(to_np(r.teacher_ce), ref["teacher_ce"], "bf16", "teacher_ce")
    else:
        assert torch.count_nonzero(r.teacher_ce).item() == 0


@pytest.mark.parametrize("shape", [dict(n=8192, d=2048, v=1000), dict(n=256, d=8192, v=8192)],
                         ids=["wide_dh", "wide_dw"])
def test_wide_gemm_tiles(shape):
    """Shapes where the dH (first) or dW (second) GEMM has enough 256x256 tiles to
    use them, so both GEMM tile widths are checked against the oracle."""
    full_parity(C2.scaled(name="quickstart_" + "_".join(f"{k}{v}" for k, v in shape.items()), **shape))


def test_topk_zero_subnormal_and_cancelling_entries():
    """Planted top-K entries (readings R7, R8): p = 0 and fp32-subnormal p in
    some rows, and in every row one entry at a shared column v* whose p equals
    M softmax(z)[v*] (M = sum of the row's stored p), so that its logit gradient
    M softmax(z) - p cancels. Everything matches the oracle, and dW[v*], a sum
    of cancelled gradients, stays within what one rounding of each dz allows:
    subtracting p after rounding M softmax(z) to bf16 would leave ~2^-9 p per
    entry there."""
    w = C4.scaled(n=200, d=256, v=3000, k=20)
    x = make_inputs(w, "cuda", seed=21)
    idx = x["topk_idx"].cpu().numpy().copy()
    prob = x["topk_prob"].cpu().numpy().astype(np.float32).copy()
    vstar = 1500
    prob[:50, 1:5] = 0.0
    prob[50:100, 1:5] = np.array([1e-41, 3e-40, 1e-39, 1.4e-45], np.float32)
    assert (prob[50:100, 1:5] > 0).all() and (prob[50:100, 1:5] < np.finfo(np.float32).tiny).all()
    H = to_np(x["student_hidden"]).astype(np.float64)
    W = to_np(x["weight"]).astype(np.float64)
    z = H @ W.T
    sm = np.exp(z - z.max(1, keepdims=True))
    sm /= sm.sum(1, keepdims=True)
    for i in range(w.n):
        hit = np.flatnonzero(idx[i] == vstar)
        j = int(hit[0]) if hit.size else 0
        if not hit.size:
            idx[i, j] = vstar
        others = float(prob[i].astype(np.float64).sum() - prob[i, j])
        s_ = sm[i, vstar]
        prob[i, j] = np.float32(others * s_ / (1.0 - s_))  # p_j = (others + p_j) s
    assert all(len(set(r)) == w.k for r in idx.tolist())
    x["topk_idx"] = torch.from_numpy(idx).to("cuda")
    x["topk_prob"] = torch.from_numpy(prob).to("cuda")
    say(f"[planted top-K] n={w.n} d={w.d} v={w.v} k={w.k} v*={vstar}")
    r, dh, dw = run_gpu(w, x, vocab_chunk=1024)
    s, t, labels = oracle_problem(w, x)
    p = params_of(w)
    ref = O.forward(s, t, p, None)
    assert r.read_status() == 0
    assert_tokens(to_np(r.kl), ref["kl"], w.dtype, "planted top-K objective")
    assert_scalar(float(r.loss), ref["loss"], w.dtype, "planted top-K loss")
    dH, dW = O.backward(s, t, p, None)
    assert_grad(to_np(dh), dH, w.dtype, "planted top-K dH")
    assert_grad(to_np(dw), dW, w.dtype, "planted top-K dW")
    # the cancelled column
    pj = prob[np.arange(w.n), np.argmax(idx == vstar, axis=1)].astype(np.float64)
    scale = np.sqrt(((pj[:, None] * H) ** 2).sum(0)).max() / ref["den"]
    err = np.abs(to_np(dw)[vstar].astype(np.float64) - dW[vstar]).max()
    say(f"  dW[v*]: |gpu - oracle| = {err:.3e}, scale {scale:.3e}, ratio {err / scale:.2e}")
    assert err <= 2e-4 * scale, f"dW[v*] error {err / scale:.2e} of the p-term scale"


# bf16 gradient outputs: (workload, vocab chunk); several chunks unless noted
BF16_GRAD_CASES = {
    "tied": (C2.scaled(n=300, d=512, v=3000), 1024),
    "tied_one_chunk": (C2.scaled(n=300, d=512, v=3000), 0),
    "tied_compact": (C2.scaled(n=300, d=512, v=3000, ignore_frac=0.3, compact_valid=True), 768),
    "separate_train_teacher": (C3.scaled(n=200, d=256, d_t=512, v=2000, teacher_ce_weight=0.5), 512),
    "topk": (C4.scaled(n=300, d=512, v=5000), 1024),
    "fp32_inputs": (C1.scaled(n=70, v=1000, ignore_frac=0.2), 256),
}


@pytest.mark.parametrize("name", list(BF16_GRAD_CASES))
def test_bf16_gradient_outputs(name):
    """dH / dW (and a CE-trained teacher's) written as bf16 equal the fp32
    gradients rounded to nearest even, bit for bit: one rounding of the same
    fp32 sums (dH sums its chunks in an fp32 buffer first). With accumulate
    the old bf16 value is added in fp32 before that one rounding."""
    w, chunk = BF16_GRAD_CASES[name]
    say(f"[bf16 grads] {name} n={w.n} d={w.d} v={w.v} chunk={chunk}")
    x = make_inputs(w, "cuda", seed=9)
    trained = w.teacher_ce_weight > 0
    res = {}
    for gdt in (torch.float32, torch.bfloat16):
        r = make_runner(w, x, chunk, grad_dtype=gdt)
        r.forward()
        g = {"dh": torch.empty((r.n, r.d), dtype=gdt, device="cuda"),
             "dw": torch.empty((r.v, r.d), dtype=gdt, device="cuda")}
        r.backward(g["dh"], g["dw"])
        if trained:
            g["dht"] = torch.empty((r.n, r.dt), dtype=gdt, device="cuda")
            g["dwt"] = torch.empty((r.v, r.dt), dtype=gdt, device="cuda")
            r.backward_teacher(g["dht"], g["dwt"])
        torch.cuda.synchronize()
        res[gdt] = (r, g)
    r16, g16 = res[torch.bfloat16]
    g32 = res[torch.float32][1]
    for k in g16:
        assert torch.equal(g16[k], g32[k].to(torch.bfloat16)), f"{name}: bf16 {k} is not the rounded fp32 {k}"
    # accumulate: old + new in fp32, rounded once
    old = {k: v.clone() for k, v in g16.items()}
    r16.forward()
    r16.backward(g16["dh"], g16["dw"], accumulate=True)
    torch.cuda.synchronize()
    for k in ("dh", "dw"):
        want = old[k].float() + g32[k]
        err = (g16[k].float() - want).abs()
        assert (err <= 2.0 ** -8 * want.abs() + 1e-30).all(), f"{name}: accumulated bf16 {k}"
