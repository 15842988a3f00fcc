"""Host-side checks of the benchmark's flop accounting (no GPU)."""
import pytest

import bench
from kl_knowledge_distillation_amd.inputs import WORKLOADS


def test_method_flops_tied_quickstart():
    # fwd: student and teacher projections 2 x 2 N D V; bwd: their recompute,
    # then dW and dH, 2 N D V each
    w = WORKLOADS["quickstart_tied_bf16"]
    n, d, v = w.n, w.d, w.v
    f = bench.method_flops(w)
    assert f["fwd"] == 4 * n * d * v
    assert f["total"] == 12 * n * d * v
    assert f["useful"] == 8 * n * d * v


def test_method_flops_separate_and_topk():
    w = WORKLOADS["separate_bf16"]
    n, d, dt, v = w.n, w.d, w.d_t, w.v
    assert bench.method_flops(w)["total"] == n * v * (8 * d + 4 * dt)
    w = WORKLOADS["topk_bf16"]
    assert bench.method_flops(w)["total"] == 8 * w.n * w.d * w.v


def test_method_flops_scorer_is_forward_only():
    # given student logits, teacher projection only, no backward
    w = WORKLOADS["scorer_bf16"]
    f = bench.method_flops(w)
    assert f["total"] == f["useful"] == f["fwd"] == 2 * w.n * w.d_t * w.v


@pytest.mark.parametrize("kernel", ["fwd", "bwd_dz", "gemm_dwdh"])
def test_chunk_launch_flops_add_up(kernel):
    # the per-launch flops of a chunked kernel, summed over the chunks of a step
    w = WORKLOADS["quickstart_tied_bf16"]
    chunk = 16384
    n_chunks = -(-w.v // chunk)
    per = bench.kernel_flops_per_launch(w, kernel, chunk)
    want = 4 * w.n * w.d * w.v  # both projections (fwd, or their recompute), or dW + dH
    assert abs(per * n_chunks - want) <= 1e-9 * want


def test_kept_last_chunk_flops():
    # the forward keeps its last chunk (32000 - 16384 = 15616 columns): the
    # backward recomputes only the first chunk, a full one
    w = WORKLOADS["quickstart_tied_bf16"]
    n, d, v, chunk = w.n, w.d, w.v, 16384
    kept = bench.kept_columns(w, chunk, True)
    assert kept == v - chunk
    assert bench.kept_columns(w, chunk, False) == 0
    f = bench.method_flops(w, kept_cols=kept)
    assert abs(f["total"] - (4 * n * d * v + 4 * n * d * chunk + 4 * n * d * v)) <= 1e-6 * f["total"]
    assert f["useful"] == 8 * n * d * v
    per = bench.kernel_flops_per_launch(w, "bwd_dz", chunk, kept_cols=kept)
    assert abs(per - 4 * n * d * chunk) <= 1e-9 * per
    # one chunk covering the vocabulary: nothing is recomputed
    assert bench.kept_columns(w, 32768, True) == v
    assert bench.method_flops(w, kept_cols=v)["total"] == 8 * n * d * v
    # a teacher trained through its CE: its recompute shrinks the same way
    tt = bench.method_flops(w, train_teacher=True, kept_cols=kept)
    assert abs(tt["total"] - f["total"] - (2 * n * d * chunk + 4 * n * d * v)) <= 1e-6 * tt["total"]
    # nothing is kept without a backward through projections
    assert bench.kept_columns(WORKLOADS["scorer_bf16"], chunk, True) == 0
