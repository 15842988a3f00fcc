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


def test_matrix_records_a_failing_child_and_goes_on(tmp_path):
    """The matrix parent keeps going past a child that fails: the failed entry
    carries its exit status and stderr, the next entry's JSON line is kept."""
    import io
    import sys
    ok_py = tmp_path / "ok.py"
    ok_py.write_text('import json\nprint("progress")\nprint(json.dumps({"value": 1.5}))\n')
    bad_py = tmp_path / "bad.py"
    bad_py.write_text('import sys\nsys.stderr.write("kernel launch failed\\n")\nsys.exit(3)\n')
    silent_py = tmp_path / "silent.py"
    silent_py.write_text('print("no json here")\n')
    log = io.StringIO()
    res = bench.run_matrix([("bad", [sys.executable, str(bad_py)]),
                            ("ok", [sys.executable, str(ok_py)]),
                            ("silent", [sys.executable, str(silent_py)])], log=log)
    assert [r["status"] for r in res] == ["FAILED", "OK", "FAILED"]
    assert res[0]["exit"] == 3 and "kernel launch failed" in res[0]["error"]
    assert res[1]["result"] == {"value": 1.5}
    assert res[2]["exit"] == 0  # exited cleanly but printed no result line
    assert "bad: FAILED" in log.getvalue() and "ok: OK" in log.getvalue()


def test_matrix_times_out_a_hung_child(tmp_path):
    import io
    import sys
    hang = tmp_path / "hang.py"
    hang.write_text("import time\ntime.sleep(60)\n")
    res = bench.run_matrix([("hang", [sys.executable, str(hang)])], timeout_s=1.0, log=io.StringIO())
    assert res[0]["status"] == "FAILED" and res[0]["exit"] == "timeout"


def test_matrix_entries_cover_the_workloads_and_the_scorer_sweep():
    labels = [e[0] for e in bench.MATRIX]
    for w in ("tiny_tied_fp32", "quickstart_tied_bf16", "separate_bf16", "topk_bf16"):
        assert w in labels
    chunks = sorted(int(a[a.index("--vocab-chunk") + 1]) for _, a in bench.MATRIX
                    if "scorer_bf16" in a)
    assert chunks == [2048, 8192, 16384]


def test_bench_matrix_on_a_machine_without_the_gpu_path():
    """End to end on the CPU: `bench.py --matrix` runs the real child, which
    cannot reach a GPU here and fails; the parent records FAILED and exits 0."""
    import json
    import os
    import subprocess
    import sys
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible: the child would run")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--matrix",
                        "--matrix-only", "tiny_tied_fp32", "--steps", "1", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    lines = [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]
    assert lines[0]["label"] == "tiny_tied_fp32" and lines[0]["status"] == "FAILED"
    assert lines[0]["error"]
    assert lines[-1] == {"matrix": 1, "ok": 0, "failed": 1}


def test_cpu_baseline_reports_the_oracle_on_a_row_sample():
    """The oracle's own rate on a bounded row sample (the tiny workload caps it
    at its 64 rows), with the threads it used and what the sample was."""
    w = WORKLOADS["tiny_tied_fp32"]
    cb = bench.cpu_baseline(w, target_s=0.05)
    assert cb["kind"] == "oracle" and cb["unit"] == "tokens/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert cb["sample"].startswith(f"64 of {w.n} rows of {w.name}")
