"""The forward and backward captured in a HIP graph (through torch's graph API)
and replayed: every launch goes to the stream it is given, nothing
synchronises or allocates inside the calls, and no step clears memory with
hipMemsetAsync, so a captured step must reproduce the eager step exactly. The
kernels use no atomics, so the results are compared bit for bit, after every
replay, with eager work and synchronisations between the replays and every
output overwritten with a sentinel before each step (an output a step should
write and does not keeps the sentinel)."""
import pytest
import torch

from gpu_common import make_runner, say
from kl_knowledge_distillation_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

C2 = WORKLOADS["quickstart_tied_bf16"]
C3 = WORKLOADS["separate_bf16"]
C4 = WORKLOADS["topk_bf16"]
C5 = WORKLOADS["scorer_bf16"]

# (workload, vocab chunk): several chunks with a ragged last one
CASES = {
    "tied": (C2.scaled(n=300, d=512, v=3000), 1024),
    "tied_compact": (C2.scaled(n=300, d=512, v=3000, ignore_frac=0.3, compact_valid=True), 768),
    "separate_T2": (C3.scaled(n=200, d=256, d_t=512, v=2000, temperature=2.0), 512),
    "topk": (C4.scaled(n=300, d=512, v=5000), 1024),
    "scorer": (C5.scaled(n=300, d_t=512, v=5000), 2048),
}


SENTINEL = -12345.0  # written into every output before each step


def _outputs(r, grads):
    return [r.loss, r.kl, r.student_ce, r.teacher_ce] + [g for g in grads if g is not None]


def _fill(r, grads):
    for t in _outputs(r, grads):
        t.fill_(SENTINEL)


@pytest.mark.parametrize("name", list(CASES))
def test_captured_step_replays_bit_identical(name):
    w, chunk = CASES[name]
    say(f"[graph] {name} n={w.n} d={w.d} v={w.v} chunk={chunk}")
    x = make_inputs(w, "cuda", seed=5)
    r = make_runner(w, x, vocab_chunk=chunk)
    grads = (None, None)
    if not w.forward_only:
        grads = (torch.empty((r.n, r.d), dtype=torch.float32, device="cuda"),
                 torch.empty((r.v, r.d), dtype=torch.float32, device="cuda"))

    def step():
        r.forward()
        if not w.forward_only:
            r.backward(*grads)

    # eager reference
    _fill(r, grads)
    step()
    torch.cuda.synchronize()
    assert r.read_status() == 0
    ref = [t.clone() for t in _outputs(r, grads)]

    # warm up on a side stream, as torch's graph capture asks, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    noise = torch.randn(1 << 20, device="cuda")
    for rep in range(3):
        _fill(r, grads)
        noise.mul_(1.5).add_(1.0)  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(_outputs(r, grads), ref):
            assert torch.equal(a, b), f"{name}: replay {rep} differs from the eager step"
    assert r.read_status() == 0


def test_captured_no_alloc_forward():
    """kd_loss_fwd_noalloc is meant for callers that cannot allocate, such as
    code under graph capture: its workspace is the library's per-device scratch
    (set up by an eager call before the capture). Every replay equals the
    workspace forward bit for bit."""
    import ctypes

    from kl_knowledge_distillation_amd import _lib as L

    w, chunk = CASES["tied"]
    say(f"[graph] no-alloc forward n={w.n} d={w.d} v={w.v} chunk={chunk}")
    x = make_inputs(w, "cuda", seed=7)
    r = make_runner(w, x, vocab_chunk=chunk)
    r.saved.zero_()
    r.forward()
    torch.cuda.synchronize()
    ref = [r.loss.clone(), r.student_ce.clone(), r.kl.clone(), r.saved.clone()]

    lib = L.load()
    f32 = dict(dtype=torch.float32, device="cuda")
    loss, sce, kl = torch.empty((), **f32), torch.empty(r.n, **f32), torch.empty(r.n, **f32)
    saved = torch.zeros_like(r.saved)
    flags = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    out = L.KdOutputs(loss.data_ptr(), sce.data_ptr(), None, kl.data_ptr())

    def call():
        st = lib.kd_loss_fwd_noalloc(ctypes.byref(r.s), ctypes.byref(r.t), ctypes.byref(r.p), r.labels_ptr,
                                     ctypes.byref(out), saved.data_ptr(), flags.data_ptr(),
                                     torch.cuda.current_stream().cuda_stream, None)
        assert st == L.KD_OK, lib.kd_status_string(st)

    call()  # eager: sets up the scratch of this device
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (loss, sce, kl):
            t.fill_(SENTINEL)
        flags.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip((loss, sce, kl, saved), ref):
            assert torch.equal(a, b), f"no-alloc replay {rep} differs from the workspace forward"
        assert int(flags.item()) == 0
