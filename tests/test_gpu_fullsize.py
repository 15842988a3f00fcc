"""HIP path at the full workload sizes, in the launch configuration bench.py times.

The oracle cannot afford the whole problem at these sizes, so it checks what
it can compute one row at a time, and properties that hold at any size cover
the rest:

  * per-token student CE, teacher CE and KL (or the top-K objective) on sampled
    rows: the first and last rows, both sides of a 128-row token-tile edge, the
    ragged last token tile, ignored rows, and seeded random rows;
  * dH on the same rows (each row's gradient needs only that row's logits and
    the loss denominator, which the labels fix);
  * dW through two identities of dW = dz^T H and dH = dz W that need no oracle:
      - every column of dW sums to zero over the vocabulary (each row of dz sums
        to zero: softmax - one-hot for CE, P_S - P_T for KL, M softmax - p for
        top-K with M = sum p);
      - sum(dH * H) = sum(dW * W) = sum over (i, v) of dz[i, v] z[i, v];
  * the loss equals the masked, weighted sum of the per-token outputs over the
    labels' denominator.

  * dW itself, element by element, on 1024 seeded vocabulary rows (the first
    and last, both sides of a 256-row tile edge and of the chunk edges, and
    random rows): the oracle forms every token's full-vocabulary logits in
    float64 (its own lse over all V columns, never the GPU's saved values) and
    keeps those columns of the gradient.

The scorer is checked at each chunk of its sweep (2048, 8192, 16384) on the
same inputs.

Sizes: separate teacher N=8192, D=2048, D_t=4096, V=128256; top-K N=32768,
D=4096, V=151936, K=100; scorer N=65536, D_t=4096, V=248320 (32.5 GB of
student logits), all bf16.
"""
import gc
import time

import numpy as np
import pytest
import torch

import oracle as O
from gpu_common import (GRAD_RTOL, assert_grad, assert_scalar, assert_tokens, make_runner,
                        params_of, say, to_np)
from kl_knowledge_distillation_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

N_RANDOM = 12


def sample_rows(n: int, labels, ignore_index: int, seed: int = 0) -> np.ndarray:
    rows = {0, 1, 127, 128, n - 1, n - 2, (n // 128) * 128 - 1}
    if labels is not None:
        ign = np.flatnonzero(labels == ignore_index)
        rows.update(ign[:3].tolist())
    rng = np.random.default_rng(seed)
    rows.update(rng.choice(n, N_RANDOM, replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n), dtype=np.int64)


def f64_rows(t, rows):
    return to_np(t[torch.as_tensor(rows, device=t.device)]).astype(np.float64)


def f64_all(t):
    return to_np(t).astype(np.float64)


def oracle_subset(w, x, rows):
    """Oracle descriptors holding only the sampled rows (the weights in full)."""
    if w.student == "logits":
        s = O.Student(logits=f64_rows(x["student_logits"], rows))
    else:
        s = O.Student(hidden=f64_rows(x["student_hidden"], rows), weight=f64_all(x["weight"]))
    if w.teacher == "tied":
        t = O.Teacher("tied", hidden=f64_rows(x["teacher_hidden"], rows))
    elif w.teacher == "separate":
        t = O.Teacher("separate", hidden=f64_rows(x["teacher_hidden"], rows),
                      weight=f64_all(x["teacher_weight"]))
    else:
        t = O.Teacher("topk", idx=to_np(x["topk_idx"][torch.as_tensor(rows, device="cuda")]).astype(np.int64),
                      prob=f64_rows(x["topk_prob"], rows))
    return s, t


def check_dw_identities(r, x, dh, dw, dtype):
    hs = x["student_hidden"].double()
    W = x["weight"].double()
    col_sum = dw.double().sum(dim=0)
    scale = dw.abs().max().item() * float(np.sqrt(dw.shape[0]))
    rel = col_sum.abs().max().item() / scale
    say(f"  dW column sums: max |sum_v dW| / (max|dW| sqrt V) = {rel:.3e}")
    assert rel <= GRAD_RTOL[dtype], f"dW columns do not sum to zero: {rel:.3e}"
    a = (dh.double() * hs).sum().item()
    b = (dw.double() * W).sum().item()
    say(f"  sum(dH*H) = {a:.9e}, sum(dW*W) = {b:.9e}")
    assert abs(a - b) <= 1e-3 * max(abs(a), abs(b)), f"trace identity: {a} vs {b}"


def check_loss_consistency(r, w, labels_np, out_sce, out_tce, out_kl):
    p = params_of(w)
    if labels_np is None:
        valid = np.ones(w.n, bool)
    else:
        valid = O.valid_mask(labels_np, w.v, w.ignore_index)
    den = O.denominator(p, int(valid.sum()))
    contrib = (p.student_ce_weight * out_sce + p.teacher_ce_weight * out_tce + p.kl_weight * out_kl)
    ref = float(np.where(valid, contrib, 0.0).sum() / den)
    assert_scalar(float(r.loss), ref, w.dtype, f"{w.name} loss vs its per-token terms")
    return den


def vocab_sample(v: int, chunk: int = 16384, count: int = 1024, seed: int = 0) -> np.ndarray:
    """Seeded vocabulary rows for the element-by-element dW check: the edges of
    the vocabulary, of a 256-row tile and of every chunk, then random rows."""
    rows = {0, 1, 255, 256, v - 1, v - 2}
    for c in range(chunk, v, chunk):
        rows.update((c - 1, c))
    rows = {r for r in rows if 0 <= r < v}
    rng = np.random.default_rng(seed)
    rest = rng.choice(np.setdiff1d(np.arange(v), sorted(rows)), count - len(rows), replace=False)
    return np.array(sorted(rows | set(rest.tolist())), dtype=np.int64)


def check_dw_rows(w, x, dw, labels_np, den):
    """dW on seeded vocabulary rows against the oracle's, element by element."""
    vrows = vocab_sample(w.v)
    s = O.Student(hidden=f64_all(x["student_hidden"]), weight=f64_all(x["weight"]))
    if w.teacher == "separate":
        t = O.Teacher("separate", hidden=f64_all(x["teacher_hidden"]),
                      weight=f64_all(x["teacher_weight"]))
    else:
        t = O.Teacher("topk", idx=to_np(x["topk_idx"]).astype(np.int64), prob=f64_all(x["topk_prob"]))
    p = params_of(w)
    t0 = time.perf_counter()
    last = [t0]

    def progress(done, n):
        if time.perf_counter() - last[0] > 20 or done == n:
            last[0] = time.perf_counter()
            say(f"  oracle dW rows: {done}/{n} tokens, {last[0] - t0:.0f} s")

    ref = O.weight_grad_rows(s, t, p, labels_np, vrows, den, progress=progress)
    got = to_np(dw[torch.as_tensor(vrows, device=dw.device)]).astype(np.float64)
    assert_grad(got, ref, w.dtype, f"{w.name} dW on {len(vrows)} vocabulary rows")
    say(f"  dW on {len(vrows)} vocabulary rows matches")


def run_fullsize(name: str, grads: bool, dw_rows: bool = False, chunks=(0,)):
    w = WORKLOADS[name]
    say(f"[fullsize] {name}: n={w.n} d={w.d} d_t={w.d_t} v={w.v} k={w.k} grads={grads}")
    x = make_inputs(w, "cuda", seed=0)
    torch.cuda.synchronize()
    for chunk in chunks:
        run_fullsize_once(w, x, grads, dw_rows, chunk)
    del x
    gc.collect()
    torch.cuda.empty_cache()


def run_fullsize_once(w, x, grads: bool, dw_rows: bool, chunk: int):
    name = w.name
    say(f"  vocab chunk {chunk or 'default'}")
    r = make_runner(w, x, vocab_chunk=chunk, want_teacher_ce=w.teacher_ce_weight > 0)
    r.forward()
    dh = dw = None
    if grads:
        dh = torch.empty((r.n, r.d), dtype=torch.float32, device="cuda")
        dw = torch.empty((r.v, r.d), dtype=torch.float32, device="cuda")
        r.backward(dh, dw)
    torch.cuda.synchronize()
    assert r.read_status() == 0
    say("  GPU done")

    labels_np = None if x["labels"] is None else to_np(x["labels"]).astype(np.int64)
    sce, tce, kl = (to_np(r.student_ce).astype(np.float64), to_np(r.teacher_ce).astype(np.float64),
                    to_np(r.kl).astype(np.float64))
    den = check_loss_consistency(r, w, labels_np, sce, tce, kl)

    rows = sample_rows(w.n, labels_np, w.ignore_index)
    say(f"  sampled rows: {rows.tolist()}")
    s, t = oracle_subset(w, x, rows)
    p = params_of(w)
    lab_rows = None if labels_np is None else labels_np[rows]
    ref = O.per_token(s, t, p, lab_rows)
    assert_tokens(kl[rows], ref["kl"], w.dtype, f"{name} kl (sampled rows)")
    if labels_np is not None:
        valid = ref["valid"]
        assert_tokens(sce[rows], ref["student_ce"], w.dtype, f"{name} student_ce (sampled rows)", valid)
        if w.teacher_ce_weight > 0:
            assert_tokens(tce[rows], ref["teacher_ce"], w.dtype, f"{name} teacher_ce (sampled rows)", valid)
    say("  per-token terms match")

    if grads:
        ref_dh = O.backward_rows(s, t, p, lab_rows, np.arange(len(rows)), den)
        assert_grad(f64_rows(dh, rows), ref_dh, w.dtype, f"{name} dH (sampled rows)")
        say("  dH rows match")
        check_dw_identities(r, x, dh, dw, w.dtype)
        if dw_rows:
            check_dw_rows(w, x, dw, labels_np, den)
    del r, dh, dw
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.timeout(1200)
def test_fullsize_separate_teacher():
    run_fullsize("separate_bf16", grads=True, dw_rows=True)


@pytest.mark.timeout(1200)
def test_fullsize_topk():
    run_fullsize("topk_bf16", grads=True, dw_rows=True)


@pytest.mark.timeout(1200)
def test_fullsize_scorer_chunk_sweep():
    """The scorer at each chunk of its sweep on the same 32.5 GB of logits."""
    run_fullsize("scorer_bf16", grads=False, chunks=(2048, 8192, 16384))


def test_fullsize_quickstart_dw_identities():
    """The identities on the fully oracle-checked quickstart problem, so a
    failure of the identities themselves would show there first."""
    w = WORKLOADS["quickstart_tied_bf16"]
    x = make_inputs(w, "cuda", seed=0)
    r = make_runner(w, x)
    r.forward()
    dh = torch.empty((r.n, r.d), dtype=torch.float32, device="cuda")
    dw = torch.empty((r.v, r.d), dtype=torch.float32, device="cuda")
    r.backward(dh, dw)
    torch.cuda.synchronize()
    check_dw_identities(r, x, dh, dw, w.dtype)


def test_fullsize_given_logits_kdloss():
    """Student and teacher logits both given at the quickstart size (N=4096,
    V=32000): every per-token KL, the loss and the whole gradient to the student
    logits against the oracle (it fits: 4096 x 32000 float64 per side)."""
    w = WORKLOADS["kdloss_logits_bf16"]
    say(f"[fullsize] {w.name}")
    x = make_inputs(w, "cuda", seed=0)
    r = make_runner(w, x, want_grads=False)
    r.forward()
    d = torch.empty((r.n, r.v), dtype=w.torch_dtype, device="cuda")
    r.backward_logits(d)
    torch.cuda.synchronize()
    s = O.Student(logits=f64_all(x["student_logits"]))
    t = O.Teacher("logits", logits=f64_all(x["teacher_logits"]))
    labels = to_np(x["labels"]).astype(np.int64)
    p = params_of(w)
    ref = O.forward(s, t, p, labels)
    assert_tokens(to_np(r.kl), ref["kl"], w.dtype, "given-logits kl")
    assert_scalar(float(r.loss), ref["loss"], w.dtype, "given-logits loss")
    g = O.logit_grad(s, t, p, labels, np.arange(w.n), ref["den"])
    assert_grad(to_np(d), g, w.dtype, "given-logits d student logits")


def test_fullsize_compacted_quickstart():
    """The quickstart problem with 40% ignored labels and compaction: loss,
    valid rows' terms and dH against the oracle on sampled rows, dW through
    the identities."""
    w = WORKLOADS["quickstart_tied_bf16"].scaled(ignore_frac=0.4, compact_valid=True)
    run_fullsize_compact(w)


def run_fullsize_compact(w):
    say(f"[fullsize] {w.name} compacted, ignored {w.ignore_frac}")
    x = make_inputs(w, "cuda", seed=0)
    r = make_runner(w, x)
    r.forward()
    dh = torch.empty((r.n, r.d), dtype=torch.float32, device="cuda")
    dw = torch.empty((r.v, r.d), dtype=torch.float32, device="cuda")
    r.backward(dh, dw)
    torch.cuda.synchronize()
    labels_np = to_np(x["labels"]).astype(np.int64)
    kl = to_np(r.kl).astype(np.float64)
    sce = to_np(r.student_ce).astype(np.float64)
    check_loss_consistency(r, w, labels_np, sce, np.zeros_like(sce), kl)
    rows = sample_rows(w.n, labels_np, w.ignore_index)
    s, t = oracle_subset(w, x, rows)
    p = params_of(w)
    ref = O.per_token(s, t, p, labels_np[rows])
    assert_tokens(kl[rows], ref["kl"], w.dtype, "compacted kl (sampled rows)")
    den = O.denominator(p, int(O.valid_mask(labels_np, w.v, w.ignore_index).sum()))
    ref_dh = O.backward_rows(s, t, p, labels_np[rows], np.arange(len(rows)), den)
    assert_grad(f64_rows(dh, rows), ref_dh, w.dtype, "compacted dH (sampled rows)")
    check_dw_identities(r, x, dh, dw, w.dtype)
