"""Benchmark: fused LM-head + CE + KL distillation loss, forward + backward, one GPU.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--vocab-chunk C]
    python bench.py --matrix [--matrix-only NAME ...]

One step is the whole hot path on one batch of synthetic input already
resident in HBM: prep, forward tiles, merge, finalize, then per vocabulary
chunk the backward recompute (dz) and the dW / dH GEMMs. The default workload
is the largest forward + backward one that fits a GPU: the precomputed sparse
top-K teacher (B=1, S=32768, hidden 4096, vocab 151936, K=100, bf16; the
Full-Chunked-KL-Loss benchmark's shape). Prints one JSON line.

--matrix runs every workload (and the scorer's chunk sweep) in a fresh child
process each, the parent importing neither torch nor the library, and
records each child's JSON line as OK or its error as FAILED (the
Full-Chunked-KL-Loss README, What it measures: every experiment isolated in
a subprocess, status OK / FAILED with the captured error).

Throughput `value` is tokens per second. Besides it the line carries the
method's MFMA TFLOP/s (including the backward recompute), peak HBM bytes,
the roofline of the dominant kernel (HIP events around its launches on the
library's stream, inside the timed region), and the float64 oracle timed on a
bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0


def method_flops(w, train_teacher: bool = False, n_rows: int = 0, kept_cols: int = 0) -> dict:
    """Algorithmic MFMA flops of one fwd+bwd step and of one launch of each kernel.

    Forward projection tiles: 2 N D V per student GEMM and per teacher GEMM;
    the backward recomputes them, then dW and dH cost 2 N D V each. A teacher
    trained through its CE adds its recompute, dW_t and dH_t: 6 N D_t V.
    n_rows: the rows projected (the usable-label rows when they are compacted).
    kept_cols: columns of the last chunk whose products the forward kept; the
    backward recomputes the other V - kept_cols (the teacher's too when trained).
    """
    n, d, v, dt = (n_rows or w.n), w.d, w.v, w.teacher_dim
    if w.teacher == "tied":
        fwd = 4 * n * d * v
    elif w.teacher == "separate":
        fwd = 2 * n * d * v + 2 * n * dt * v
    else:
        fwd = 2 * n * d * v
    if w.forward_only:  # a scorer: the forward tiles are the whole step
        return {"total": fwd, "useful": fwd, "fwd": fwd}
    recomputed = (v - kept_cols) / v
    total = fwd + fwd * recomputed + 4 * n * d * v
    useful = fwd + 4 * n * d * v
    if train_teacher:
        total += 2 * n * dt * v * recomputed + 4 * n * dt * v
        useful += 4 * n * dt * v
    return {"total": total, "useful": useful, "fwd": fwd}


def kept_columns(w, chunk: int, keep: bool) -> int:
    """Columns of the last vocabulary chunk when the forward keeps its products
    for the backward (projection students with a backward), else 0."""
    if not keep or w.forward_only or w.student == "logits":
        return 0
    return w.v - (-(-w.v // chunk) - 1) * chunk


def kernel_flops_per_launch(w, kernel: str, chunk: int, n_rows: int = 0,
                            train_teacher: bool = False, kept_cols: int = 0) -> float:
    """Flops of one launch of `kernel`; with a trained teacher the launches of a
    class alternate between the student's and the teacher's, so the mean.
    With a kept last chunk the recomputing bwd_dz launches are the full chunks
    before it."""
    n, d, v, dt = (n_rows or w.n), w.d, w.v, w.teacher_dim
    fl = method_flops(w, n_rows=n)
    n_chunks = -(-v // chunk)
    if kernel == "fwd":  # the forward tiles run one launch per vocabulary chunk
        return fl["fwd"] / n_chunks
    per_chunk_cols = v / n_chunks  # average columns per launch
    if kernel == "bwd_dz":
        cols = chunk if kept_cols else per_chunk_cols
        f = fl["fwd"] * cols / v
        return (f + 2 * n * dt * cols) / 2 if train_teacher else f
    if kernel in ("gemm_dw", "gemm_dh", "gemm_dwdh"):
        f = 2 * n * d * per_chunk_cols
        if train_teacher:
            f = (f + 2 * n * dt * per_chunk_cols) / 2
        return 2 * f if kernel == "gemm_dwdh" else f
    return 0.0


def source_digest() -> str:
    """Hash of the kernel sources with comments and blank lines removed, so a
    counter summary stays valid across edits that do not change the code."""
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kl_knowledge_distillation_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
        h.update(f.encode())
        h.update(text.encode())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_digest") != source_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


_KERNEL_CLASS = (("prep_kernel", "prep"), ("fwd_tiles_kernel", "fwd"), ("merge_kernel", "merge"),
                 ("fold_kernel", "merge"),
                 ("finalize_kernel", "finalize"), ("GeoPipe, true>", "bwd_kept"),
                 ("GeoStaged, true>", "bwd_kept"), ("bwd_dz_kernel", "bwd_dz"),
                 ("scatter_kernel", "scatter"), ("gemm_pipe_kernel<false, false", "gemm_dw"),
                 ("gemm_pipe_kernel<true, false", "gemm_dh"), ("gemm_kernel<float, false, false", "gemm_dw"),
                 ("gemm_kernel<unsigned short, false, false", "gemm_dw"),
                 ("gemm_kernel<float, true, false", "gemm_dh"),
                 ("gemm_kernel<unsigned short, true, false", "gemm_dh"),
                 ("gemm_dual_kernel", "gemm_dwdh"), ("compact_kernel", "prep"),
                 ("gather_rows_kernel", "prep"), ("zero_rows_kernel", "gemm_dh"),
                 ("fill_zero_kernel", "gemm_dh"))


def _counter_per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, counter summed over its instances)} from a
    rocprofv3 --pmc CSV (run_counter_collection.csv)."""
    import csv
    out = {}
    with open(path) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            name, val = out.get(d, (r["Kernel_Name"], 0.0))
            out[d] = (name, val + float(r["Counter_Value"]))
    return out


def traffic_from(fetch_csv: str, write_csv: str, calib_mib: int, workload: str, commands) -> dict:
    """HBM bytes per launch of each kernel class from FETCH_SIZE / WRITE_SIZE runs.

    Both counters read KiB per dispatch. Each is scaled by calib / reading of the
    largest buffer-copy dispatch, the calib_mib device-to-device copy the
    profiled bench run makes before its timed steps (a plain copy reads and
    writes exactly that many bytes)."""
    res = {}
    for key, path, ctr in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        per = _counter_per_dispatch(path, ctr)
        copies = [v for name, v in per.values() if "copyBuffer" in name]
        if not copies:
            raise SystemExit(f"no buffer-copy dispatch in {path}")
        factor = (calib_mib * 1024.0) / max(copies)
        cls = {}
        for name, v in per.values():
            for pat, c in _KERNEL_CLASS:
                if pat in name:
                    cls.setdefault(c, []).append(v * factor * 1024.0)
                    break
        res[key] = (factor, cls)
    digest = source_digest()
    written = {}
    for c in res["fetch"][1]:
        f = res["fetch"][1][c]
        wv = res["write"][1].get(c, [0.0])
        fb, wb = sum(f) / len(f), sum(wv) / len(wv)
        rec = {"kernel": c, "workload": workload, "source_digest": digest,
               "hbm_bytes_per_launch": round(fb + wb), "fetch_bytes_per_launch": round(fb),
               "write_bytes_per_launch": round(wb), "dispatches": len(f),
               "fetch_factor": round(res["fetch"][0], 4), "write_factor": round(res["write"][0], 4),
               "calib_copy_mib": calib_mib, "commands": list(commands)}
        path = os.path.join(ROOT, "profiles", f"traffic_{c}_{workload}.json")
        with open(path, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
        written[c] = rec
    return written


def cpu_baseline(w, target_s: float = 15.0) -> dict:
    """The float64 oracle (as it stands) on a bounded row sample of the workload."""
    import numpy as np
    import torch

    import oracle as O
    from kl_knowledge_distillation_amd.inputs import make_inputs

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1

    cap = w.n
    x = make_inputs(w.scaled(n=cap), "cpu", seed=0)
    f = lambda t: None if t is None else t.float().numpy().astype(np.float64)  # noqa: E731
    full = {k: f(v) if k not in ("labels", "topk_idx") else (None if v is None else v.numpy())
            for k, v in x.items()}
    p = O.Params(student_ce_weight=w.student_ce_weight, teacher_ce_weight=w.teacher_ce_weight,
                 kl_weight=w.kl_weight, temperature=w.temperature, ignore_index=w.ignore_index,
                 kl_divergence=w.kl_divergence, teacher_temperature=w.teacher_temperature,
                 compact_valid=w.compact_valid)

    def run(rows: int) -> float:
        g = lambda k: None if full[k] is None else full[k][:rows]  # noqa: E731
        if w.student == "logits":
            s = O.Student(logits=g("student_logits"))
        else:
            s = O.Student(hidden=g("student_hidden"), weight=full["weight"])
        if w.teacher == "tied":
            t = O.Teacher("tied", hidden=g("teacher_hidden"))
        elif w.teacher == "separate":
            t = O.Teacher("separate", hidden=g("teacher_hidden"), weight=full["teacher_weight"])
        elif w.teacher == "logits":
            t = O.Teacher("logits", logits=g("teacher_logits"))
        else:
            t = O.Teacher("topk", idx=g("topk_idx"), prob=g("topk_prob"))
        t0 = time.perf_counter()
        out = O.forward(s, t, p, g("labels"))
        if w.student == "logits" and w.teacher == "logits":  # the gradient to the given logits
            O.logit_grad(s, t, p, g("labels"), np.arange(rows), out["den"])
        elif not w.forward_only:
            O.backward(s, t, p, g("labels"))
        return time.perf_counter() - t0

    probe = 64
    run(probe)  # first call: allocation and thread start-up, not timed
    dt = run(probe)
    rows = int(min(cap, max(probe, probe * target_s / max(dt, 1e-3))))
    rows = max(probe, rows // 64 * 64)
    dt = run(rows)
    if dt < 0.6 * target_s and rows < cap:
        # the small probe overstates the cost per row (small float64 products
        # run slower per row): scale once more from the sized run
        rows = max(probe, int(min(cap, rows * target_s / max(dt, 1e-3))) // 64 * 64)
        dt = run(rows)
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{rows} of {w.n} rows of {w.name}, forward + backward "
                      f"({'d logits' if w.student == 'logits' else 'dH, dW'}) in float64, {dt:.1f} s"}


# The matrix: every workload of the five configurations, the scorer at each
# chunk of its sweep (flash_kd, flash_ce_kd_loss: chunk_size is the memory
# knob). Each entry: (label, bench arguments).
MATRIX = (
    ("tiny_tied_fp32", ["--workload", "tiny_tied_fp32"]),
    ("quickstart_tied_bf16", ["--workload", "quickstart_tied_bf16"]),
    ("separate_bf16", ["--workload", "separate_bf16"]),
    ("topk_bf16", ["--workload", "topk_bf16"]),
    ("scorer_bf16_chunk2048", ["--workload", "scorer_bf16", "--vocab-chunk", "2048"]),
    ("scorer_bf16_chunk8192", ["--workload", "scorer_bf16", "--vocab-chunk", "8192"]),
    ("scorer_bf16_chunk16384", ["--workload", "scorer_bf16", "--vocab-chunk", "16384"]),
)


def run_matrix(entries, timeout_s: float = 600.0, log=sys.stderr) -> list:
    """Run each (label, argv) as its own child process, one after another.

    A child that exits 0 and prints a JSON line is OK (the line is kept); any
    other end (a non-zero exit, a signal, no JSON line, the time limit) is
    FAILED with the exit status and the tail of its stderr, and the next
    entry still runs. The caller's process never touches the GPU."""
    import subprocess
    results = []
    for label, argv in entries:
        print(f"[matrix] {label}: {' '.join(argv)}", file=log, flush=True)
        t0 = time.perf_counter()
        rec = {"label": label, "argv": list(argv)}
        try:
            r = subprocess.run(argv, capture_output=True, text=True, timeout=timeout_s)
            rc, out, err = r.returncode, r.stdout, r.stderr
        except subprocess.TimeoutExpired as e:
            rc = "timeout"
            out = e.stdout.decode() if isinstance(e.stdout, bytes) else (e.stdout or "")
            err = e.stderr.decode() if isinstance(e.stderr, bytes) else (e.stderr or "")
        rec["wall_s"] = round(time.perf_counter() - t0, 2)
        line = None
        for ln in reversed(out.strip().splitlines()):
            if ln.startswith("{"):
                try:
                    line = json.loads(ln)
                    break
                except ValueError:
                    pass
        if rc == 0 and line is not None:
            rec["status"] = "OK"
            rec["result"] = line
        else:
            rec["status"] = "FAILED"
            rec["exit"] = rc
            rec["error"] = "\n".join((err or "no output").strip().splitlines()[-12:])
        print(f"[matrix] {label}: {rec['status']} ({rec['wall_s']} s)", file=log, flush=True)
        results.append(rec)
    return results


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="topk_bf16")
    ap.add_argument("--matrix", action="store_true",
                    help="every workload in a fresh child process; OK / FAILED per entry")
    ap.add_argument("--matrix-only", nargs="*", default=None,
                    help="with --matrix: only these entries (labels of MATRIX)")
    ap.add_argument("--vocab-chunk", type=int, default=0)
    ap.add_argument("--n", type=int, default=0, help="override the token count")
    ap.add_argument("--d", type=int, default=0, help="override the student hidden size")
    ap.add_argument("--v", type=int, default=0, help="override the vocabulary size")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--compact", action="store_true",
                    help="leave rows with an ignored label out of the projections (compact_valid)")
    ap.add_argument("--kl", choices=("forward", "reverse", "jeffreys"), default=None,
                    help="override the workload's KL direction")
    ap.add_argument("--keep-last-chunk", action="store_true",
                    help="keep_last_chunk on (opt-in): the forward keeps its last chunk's fp32 "
                         "products and the backward reads them instead of recomputing them")
    ap.add_argument("--train-teacher", action="store_true",
                    help="teacher trained through its CE (weight 1): the step adds its backward")
    ap.add_argument("--ignore-frac", type=float, default=None,
                    help="override the fraction of rows whose label is ignored")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="copy a buffer of this many MiB once before the timed steps, so a "
                         "counter run can scale FETCH_SIZE / WRITE_SIZE by a known transfer")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 counter CSVs of this bench (FETCH_SIZE, "
                         "WRITE_SIZE, both with --calib-copy-mib) into profiles/traffic_*.json")
    ap.add_argument("--traffic-commands", nargs="*", default=[],
                    help="the commands that produced the CSVs, recorded with the numbers")
    args = ap.parse_args()

    if args.traffic_from:
        name = args.workload
        over = [f"{k}{getattr(args, k)}" for k in ("n", "d", "v") if getattr(args, k)]
        if over:
            name = name + "_" + "_".join(over)
        out = traffic_from(args.traffic_from[0], args.traffic_from[1], args.calib_copy_mib or 1024,
                           name, args.traffic_commands)
        for c, rec in sorted(out.items()):
            print(f"{c:10s} {rec['hbm_bytes_per_launch'] / 1e6:10.1f} MB/launch "
                  f"(fetch {rec['fetch_bytes_per_launch'] / 1e6:.1f}, write "
                  f"{rec['write_bytes_per_launch'] / 1e6:.1f}, {rec['dispatches']} dispatches)")
        return 0

    if args.matrix:
        chosen = [e for e in MATRIX if args.matrix_only is None or e[0] in args.matrix_only]
        common = ["--steps", str(args.steps), "--warmup", str(args.warmup)]
        if args.no_cpu_baseline:
            common.append("--no-cpu-baseline")
        entries = [(label, [sys.executable, "-u", os.path.abspath(__file__), *a, *common])
                   for label, a in chosen]
        results = run_matrix(entries)
        for rec in results:
            print(json.dumps(rec), flush=True)
        ok = sum(r["status"] == "OK" for r in results)
        print(json.dumps({"matrix": len(results), "ok": ok, "failed": len(results) - ok}),
              flush=True)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        return 2

    import torch

    from kl_knowledge_distillation_amd import _lib as L
    from kl_knowledge_distillation_amd.api import Runner, Tracer
    from kl_knowledge_distillation_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    over = {k: getattr(args, k) for k in ("n", "d", "v") if getattr(args, k)}
    if args.kl:
        over["kl_divergence"] = args.kl
    if args.compact:
        over["compact_valid"] = True
    if args.ignore_frac is not None:
        over["ignore_frac"] = args.ignore_frac
    if args.train_teacher:
        over["teacher_ce_weight"] = 1.0
    if over:
        tag = {"kl_divergence": lambda v: v, "compact_valid": lambda v: "compact",
               "teacher_ce_weight": lambda v: "train_teacher",
               "ignore_frac": lambda v: f"ignore{v:g}"}
        w = w.scaled(name=w.name + "_" + "_".join(tag[k](v) if k in tag else f"{k}{v}"
                                                  for k, v in over.items()), **over)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = make_inputs(w, dev, seed=0)
    torch.cuda.synchronize()
    kw = dict(labels=x["labels"], student_ce_weight=w.student_ce_weight,
              teacher_ce_weight=w.teacher_ce_weight, kl_weight=w.kl_weight,
              temperature=w.temperature, ignore_index=w.ignore_index,
              vocab_chunk=args.vocab_chunk, want_grads=not w.forward_only,
              kl_divergence=w.kl_divergence, teacher_temperature=w.teacher_temperature,
              compact_valid=w.compact_valid,
              keep_last_chunk=bool(args.keep_last_chunk) and not w.forward_only
              and w.student != "logits")
    if w.student == "logits":
        kw["student_logits"] = x["student_logits"]
    else:
        kw.update(student_hidden=x["student_hidden"], weight=x["weight"])
    if w.teacher == "tied":
        kw.update(teacher_kind="tied", teacher_hidden=x["teacher_hidden"])
    elif w.teacher == "separate":
        kw.update(teacher_kind="separate", teacher_hidden=x["teacher_hidden"],
                  teacher_weight=x["teacher_weight"])
    elif w.teacher == "logits":
        kw.update(teacher_kind="logits", teacher_logits=x["teacher_logits"])
    else:
        kw.update(teacher_kind="topk", topk_idx=x["topk_idx"], topk_prob=x["topk_prob"])
    input_bytes = sum(t.numel() * t.element_size() for t in x.values() if t is not None)
    torch.cuda.reset_peak_memory_stats(dev)
    base_alloc = torch.cuda.memory_allocated(dev)
    r = Runner(**kw)
    dh = dw = None
    if not w.forward_only:
        dh = torch.empty((r.n, r.d), dtype=torch.float32, device=dev)
        dw = torch.empty((r.v, r.d), dtype=torch.float32, device=dev)
    both_logits = w.student == "logits" and w.teacher == "logits"
    dlog = torch.empty((r.n, r.v), dtype=w.torch_dtype, device=dev) if both_logits else None
    dht = dwt = None
    if args.train_teacher:
        dht = torch.empty((r.n, r.dt), dtype=torch.float32, device=dev)
        dwt = torch.empty((r.v, r.dt), dtype=torch.float32, device=dev)
    output_bytes = sum(t.numel() * t.element_size() for t in (dh, dw, dht, dwt, dlog) if t is not None)
    output_bytes += 3 * r.n * 4 + 4

    def step(trace=None):
        r.forward(trace)
        if dh is not None:
            r.backward(dh, dw, trace=trace)
        if dht is not None:
            r.backward_teacher(dht, dwt, trace=trace)
        if dlog is not None:
            r.backward_logits(dlog, trace=trace)

    # Warm-up, with every kernel class traced once to find the dominant one.
    all_tr = Tracer(capacity=4096, kernels=L.KERNELS)
    for i in range(max(args.warmup, 1)):
        all_tr.reset()
        step(all_tr.trace)
    torch.cuda.synchronize()
    last_step = all_tr.durations_ms()
    per_kernel = {k: sum(v) for k, v in last_step.items()}
    # the dominant class among the tile and GEMM kernels (the row-statistics
    # kernels of the given-logits path are its fwd / bwd_dz classes); the
    # first warm-up step also carries one-time start-up costs in prep
    work = {k: v for k, v in per_kernel.items() if k not in ("prep", "merge", "finalize")}
    dominant = max(work or per_kernel, key=(work or per_kernel).get)
    n_dom = len(last_step[dominant])
    all_tr.close()

    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    tr = Tracer(capacity=2 * n_dom * args.steps + 2, kernels=(dominant,))
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step(tr.trace)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    durs = tr.durations_ms().get(dominant, [])
    tr.close()
    status = r.read_status()
    peak = torch.cuda.max_memory_allocated(dev)

    ms_per_step = gpu_ms / args.steps
    tokens_per_s = r.n * args.steps / (gpu_ms / 1e3)
    # rows the kernels project: all, or the usable-label rows when compacted
    n_rows = w.n
    if w.compact_valid and x["labels"] is not None:
        y = x["labels"]
        n_rows = int(((y != w.ignore_index) & (y >= 0) & (y < w.v)).sum().item())
    # the backward chunk the library used (same rule as the C ABI's default)
    chunk = args.vocab_chunk if args.vocab_chunk > 0 else 16384
    chunk = min(-(-chunk // 128) * 128, -(-w.v // 128) * 128)
    kept = kept_columns(w, chunk, args.keep_last_chunk)
    # what the opt-in keep_last_chunk would add to `saved` (or adds, when on)
    keep_extra = 0
    if not w.forward_only and w.student != "logits":
        import ctypes
        p2 = L.KdParams.from_buffer_copy(r.p)
        p2.keep_last_chunk = 1
        nb = ctypes.c_size_t(0)
        L.check(r.lib.kd_saved_bytes_for(ctypes.byref(r.s), ctypes.byref(r.t), ctypes.byref(p2),
                                         ctypes.byref(nb)), "kd_saved_bytes_for")
        keep_extra = int(nb.value) - int(r.lib.kd_saved_bytes(r.n))
    fl = method_flops(w, args.train_teacher, n_rows, kept)
    peak_tflops = PEAK_FP32_TFLOPS if w.dtype == "fp32" else PEAK_BF16_TFLOPS
    tflops = fl["total"] / (ms_per_step / 1e3) / 1e12
    launch_ms = sum(durs) / len(durs) if durs else float("nan")
    kflops = kernel_flops_per_launch(w, dominant, chunk, n_rows, args.train_teacher, kept)
    achieved = kflops / (launch_ms / 1e3) / 1e12 if durs else None
    rec = {
        "metric": "fused LM-head+CE+KL fwd+bwd tokens/s" if not w.forward_only
        else "fused teacher-LM-head+CE+KL forward tokens/s",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "fp32" else "bf16",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": w.name, "n_tokens": w.n, "hidden": w.d, "teacher_hidden": w.teacher_dim,
                   "vocab": w.v, "teacher": w.teacher, "temperature": w.temperature,
                   "teacher_temperature": w.teacher_temperature, "kl_divergence": w.kl_divergence,
                   "compact_valid": w.compact_valid, "ignored_rows": w.ignore_frac,
                   "train_teacher": bool(args.train_teacher), "projected_rows": n_rows,
                   "top_k": w.k or None, "vocab_chunk": chunk, "keep_last_chunk": kept > 0,
                   "parallelism": "single GPU"},
        "mfma_tflops": round(tflops, 1),
        "mfma_frac_of_peak": round(tflops / peak_tflops, 4),
        "useful_tflops": round(fl["useful"] / (ms_per_step / 1e3) / 1e12, 1),
        "peak_hbm_bytes": int(peak),
        "peak_extra_hbm_bytes": int(peak - base_alloc - output_bytes),
        "keep_last_chunk_extra_bytes": keep_extra,
        "input_bytes": int(input_bytes),
        "wall_s": round(wall, 3),
        "device_status": status,
        # per-class kernel times of the last warm-up step, traced with events
        # around every launch (not the timed region, which traces only the
        # dominant class)
        "warmup_kernel_ms_per_step": {k: round(v, 4) for k, v in per_kernel.items()},
        "roofline": {
            "kernel": dominant,
            "bound": "mfma",
            "achieved": round(achieved, 1) if achieved else None,
            "peak": peak_tflops,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak_tflops, 4) if achieved else None,
            "traffic": traffic_for(dominant, w.name),
            "launch_ms": round(launch_ms, 4),
            "launches": len(durs),
            "flop_per_launch": kflops,
        },
    }
    if both_logits:
        # No projection: the row kernels stream the logits, HBM-bound. Bytes per
        # launch: the forward reads both matrices; the backward reads both and
        # writes the gradient.
        e = 2 if w.dtype == "bf16" else 4
        nbytes = {"fwd": 2 * w.n * w.v * e, "bwd_dz": 3 * w.n * w.v * e}.get(dominant, 0)
        gbs = nbytes / (launch_ms / 1e3) / 1e9 if durs and nbytes else None
        rec["metric"] = "KL from given logits fwd+bwd tokens/s"
        rec["mfma_tflops"] = rec["mfma_frac_of_peak"] = rec["useful_tflops"] = None
        rec["roofline"] = {
            "kernel": dominant, "bound": "hbm",
            "achieved": round(gbs, 1) if gbs else None, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4) if gbs else None,
            "traffic": traffic_for(dominant, w.name), "launch_ms": round(launch_ms, 4),
            "launches": len(durs), "bytes_per_launch": nbytes}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
