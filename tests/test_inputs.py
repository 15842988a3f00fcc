"""Seeded input generators: determinism and the stated structure (CPU only)."""
import numpy as np
import torch

from kl_knowledge_distillation_amd.inputs import WORKLOADS, make_inputs, make_labels, make_topk


def test_labels_ignore_count_and_range():
    for name, frac, n, v, ign in (("tiny", 0.10, 64, 1024, -100), ("q", 0.05, 4096, 32000, -100),
                                  ("s", 0.03, 65536, 248320, -1)):
        y = make_labels(n, v, ign, frac, seed=0)
        assert y.dtype == torch.int64
        assert int((y == ign).sum()) == round(frac * n), name
        ok = y[y != ign]
        assert int(ok.min()) >= 0 and int(ok.max()) < v


def test_labels_deterministic():
    assert torch.equal(make_labels(100, 50, -100, 0.1, 3), make_labels(100, 50, -100, 0.1, 3))
    assert not torch.equal(make_labels(100, 50, -100, 0.1, 3), make_labels(100, 50, -100, 0.1, 4))


def test_topk_structure():
    idx, p = make_topk(2048, 151936, 100, seed=0)
    assert idx.dtype == torch.int32 and p.dtype == torch.float32
    assert idx.shape == (2048, 100) and p.shape == (2048, 100)
    s = np.sort(idx.numpy(), axis=1)
    assert (s[:, 1:] != s[:, :-1]).all(), "indices must be distinct per row"
    assert idx.min() >= 0 and idx.max() < 151936
    m = p.double().sum(1).numpy()
    assert (m > 0.85 - 1e-5).all() and (m < 0.99 + 1e-5).all()
    assert (p >= 0).all()
    i2, p2 = make_topk(2048, 151936, 100, seed=0)
    assert torch.equal(idx, i2) and torch.equal(p, p2)


def test_topk_structure_many_entries():
    # k^2 > v: rows are drawn as permutation prefixes (distinct, in range)
    idx, p = make_topk(40, 3000, 1100, seed=0)
    s = np.sort(idx.numpy(), axis=1)
    assert idx.shape == (40, 1100) and (s[:, 1:] != s[:, :-1]).all()
    assert s.min() >= 0 and s.max() < 3000
    m = p.double().sum(dim=1).numpy()
    assert (m > 0.85 - 1e-5).all() and (m < 0.99 + 1e-5).all()


def test_tiny_inputs_shapes_and_stats():
    w = WORKLOADS["tiny_tied_fp32"]
    x = make_inputs(w, "cpu", seed=0)
    assert x["student_hidden"].shape == (64, 128) and x["student_hidden"].dtype == torch.float32
    assert x["weight"].shape == (1024, 128)
    assert x["teacher_hidden"].shape == (64, 128)
    assert x["teacher_weight"] is None and x["topk_idx"] is None
    # W ~ N(0, 1/D): the sample variance is close to 1/128
    assert abs(float(x["weight"].double().var()) * 128 - 1.0) < 0.05
    y = make_inputs(w, "cpu", seed=0)
    assert torch.equal(x["weight"], y["weight"])


def test_bf16_storage():
    w = WORKLOADS["quickstart_tied_bf16"].scaled(n=16, v=64, d=32)
    x = make_inputs(w, "cpu")
    assert x["student_hidden"].dtype == torch.bfloat16 and x["weight"].dtype == torch.bfloat16
