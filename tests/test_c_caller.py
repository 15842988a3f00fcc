"""The C ABI from a plain C++ program (tests/c_caller/kd_c_caller.cpp): no
PyTorch, device memory from the HIP runtime, its own stream.

CPU: the program links and loads the in-tree library (kd_version agrees).
GPU: one forward + backward of a tied bf16 problem, written to files, equal
bit for bit to the same step through the Python binding, and within the
parity bar of the float64 oracle.
"""
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c_caller", "kd_c_caller")

needs_bin = pytest.mark.skipif(not os.path.exists(BIN),
                               reason="tests/c_caller/kd_c_caller not built (__graft_entry__.build())")


@needs_bin
def test_cpp_caller_links_the_library():
    from kl_knowledge_distillation_amd import _lib as L
    r = subprocess.run([BIN, "--version"], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == L.load().kd_version().decode()


@needs_bin
@pytest.mark.gpu
def test_cpp_caller_matches_the_binding_and_the_oracle(tmp_path):
    import torch

    import oracle as O
    from gpu_common import (assert_grad, assert_scalar, assert_tokens, make_runner, oracle_problem,
                            params_of, say, to_np)
    from kl_knowledge_distillation_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS["quickstart_tied_bf16"].scaled(n=300, d=512, v=3000)
    chunk = 1024
    say(f"[c caller] n={w.n} d={w.d} v={w.v} chunk={chunk}")
    x = make_inputs(w, "cuda", seed=6)
    for name, key in (("hidden", "student_hidden"), ("teacher_hidden", "teacher_hidden"), ("weight", "weight")):
        x[key].contiguous().view(torch.int16).cpu().numpy().tofile(str(tmp_path / f"{name}.bin"))
    x["labels"].cpu().numpy().astype(np.int64).tofile(str(tmp_path / "labels.bin"))
    (tmp_path / "meta.txt").write_text(f"{w.n} {w.d} {w.v} {w.temperature!r} {w.ignore_index} {chunk}\n")

    r = subprocess.run([BIN, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.stdout, r.stderr)
    assert r.stdout.split() == ["status", "0", "0", "flags", "0"], r.stdout

    def load(name, shape):
        return np.fromfile(str(tmp_path / f"{name}.bin"), dtype=np.float32).reshape(shape)

    c = {"loss": load("loss", ()), "kl": load("kl", (w.n,)), "student_ce": load("student_ce", (w.n,)),
         "dh": load("dh", (w.n, w.d)), "dw": load("dw", (w.v, w.d))}

    # the same step through the Python binding: identical bits
    rb = make_runner(w, x, vocab_chunk=chunk)
    rb.forward()
    dh = torch.empty((rb.n, rb.d), dtype=torch.float32, device="cuda")
    dw = torch.empty((rb.v, rb.d), dtype=torch.float32, device="cuda")
    rb.backward(dh, dw)
    torch.cuda.synchronize()
    for key, t in (("loss", rb.loss), ("kl", rb.kl), ("student_ce", rb.student_ce), ("dh", dh), ("dw", dw)):
        assert np.array_equal(c[key], to_np(t)), f"{key} differs from the binding's"

    # and the oracle, at the parity bar
    s, t, labels = oracle_problem(w, x)
    p = params_of(w)
    ref = O.forward(s, t, p, labels)
    dH, dW = O.backward(s, t, p, labels)
    assert_scalar(float(c["loss"]), ref["loss"], w.dtype, "loss")
    assert_tokens(c["kl"], ref["kl"], w.dtype, "kl")
    assert_tokens(c["student_ce"], ref["student_ce"], w.dtype, "student_ce")
    assert_grad(c["dh"], dH, w.dtype, "dH")
    assert_grad(c["dw"], dW, w.dtype, "dW")
