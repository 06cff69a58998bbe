#!/usr/bin/env python3
"""Benchmark of the fused linear cross-entropy forward+backward on one MI355X.

One step = cce_forward + cce_backward over one batch of synthetic input (all
of the hot path: logit tiles with online LSE partials, gather-dot, LSE
combine, reductions, filter, gradient tiles, dC and dE contractions).  The
default workload is the Llama-3.1-8B classifier head: N = 4x1024 tokens,
D = 4096, V = 128256, bf16 operands with fp32 accumulation, e ~ N(0,1),
c ~ N(0, 0.02^2), uniform targets, per-token loss (reduction 'none').

Prints one JSON line: tokens/s for forward+backward, MFMA utilisation over
the effective (unfiltered) 8*N*V*D flops, a roofline entry for the dominant
kernel (per-launch durations from HIP events recorded around that kernel's
launches on its stream during the timed region) and the CPU oracle timed on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
KERNELS = ["fwd_tile", "rows", "reduce", "bwd_prep", "filter", "grad_tile", "dC_gemm", "dE_gemm", "dE_reduce",
           "fill_zero", "transpose_e", "db_reduce", "colsum", "colsum_reduce", "vec_sum", "fill_rank1", "tile_list"]
MFMA_KERNELS = {"fwd_tile", "grad_tile", "dC_gemm", "dE_gemm"}
# Measured memory traffic per launch (bytes past L2: rocprofv3 FETCH_SIZE x 2.0
# + WRITE_SIZE x 1.0, the factors a 1 GiB device copy calibrates in the same
# runs), averaged over a step's launches.  Valid only for the kernel sources
# they were taken on: reported when the source hash matches, null otherwise.
TRAFFIC = {
    "source_sha256": "f8395baf768420397710a8e9cddbaaddfd8d1ff579461d44c8ca4819268ee8b6",
    "workload": "llama8b",
    "bytes_per_launch": {
        "fwd_tile": 9184.8e6, "grad_tile": 1778.7e6, "dC_gemm": 1658.6e6, "dE_gemm": 1058.8e6,
        "rows": 121.3e6, "filter": 37.2e6, "transpose_e": 67.3e6, "dE_reduce": 100.7e6,
    },
}


def source_sha256() -> str:
    import hashlib
    d = os.path.join(ROOT, "linear_cross_entropy_forward_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def traffic_for(kernel: str, workload: str):
    if TRAFFIC["workload"] != workload or TRAFFIC["source_sha256"] != source_sha256():
        return None
    return TRAFFIC["bytes_per_launch"].get(kernel)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--reduction", default=None)
    ap.add_argument("--no-filter", action="store_true")
    ap.add_argument("--accum", default="deterministic", choices=["deterministic", "atomic"])
    ap.add_argument("--vocab-chunk", type=int, default=0)
    ap.add_argument("--grad-dtype", default="operand", choices=["operand", "float32"],
                    help="element type of dE and dC: the operands' (as the autograd path returns them) or fp32")
    ap.add_argument("--cpu-rows", type=int, default=None, help="rows of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-materialized", action="store_true",
                    help="skip the materialised-logits PyTorch comparison")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the compact figures for the other workloads")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="run one plain device copy of BYTES first (HBM-counter calibration under rocprofv3)")
    return ap.parse_args()


def algorithmic(name, N, D, V, es, nVB, launches, tiles_kept=1.0):
    """(flops, bytes) per launch of `name`, averaged over its launches in a
    step: the work the tile filter leaves (the backward's three contractions
    on the kept 256x256 tiles; 2 flops per multiply-add).  Inside kept tiles
    dC and dE also skip the MFMAs of dropped 32x32 blocks: that is a saving
    of the kernels, not less work of the method, and is reported apart
    (blocks_kept_frac, mfma_flops_executed_per_launch)."""
    if name == "fwd_tile":
        return 2.0 * N * V * D, (N + V) * D * es + N * nVB * 8.0
    if name in ("grad_tile", "dC_gemm", "dE_gemm"):
        # one launch per vocabulary chunk: the chunks cover the vocabulary
        return 2.0 * N * V * D * tiles_kept / max(1.0, launches), 0.0
    if name == "rows":
        return 2.0 * N * D, N * (2.0 * D * es + 8 + nVB * 8.0 + 8)
    if name == "reduce":
        return 0.0, N * 12.0
    if name == "bwd_prep":
        return 0.0, N * 12.0
    if name == "filter":
        return 0.0, N * nVB * 8.0 + N * 12.0
    if name == "dE_reduce":
        return 0.0, 0.0
    if name == "transpose_e":
        return 0.0, 2.0 * N * D * es
    return 0.0, 0.0


def cpu_baseline(inp, rows_n):
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    e, c, t = inp["e"], inp["c"], inp["targets"]
    rows = np.arange(rows_n)
    t0 = time.perf_counter()
    f = O.forward(e[rows], c, t[rows], reduction="none")
    O.backward(e[rows], c, t[rows], reduction="none", grad_loss=np.ones(rows_n))
    dt = time.perf_counter() - t0
    assert np.isfinite(f.lse).all()
    return {"value": rows_n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 NumPy oracle forward+backward of the first {rows_n} of {e.shape[0]} tokens "
                      f"against the full classifier (V={c.shape[0]}, D={c.shape[1]}); {dt:.1f} s"}


def materialized(e, c, t, reduction, steps):
    """The conventional head that cut cross-entropy replaces (mlx-cross-entropy,
    "The problem"): the full logit matrix e @ c^T is materialised (here in fp32),
    then cross-entropy (mean) and its backward.  Returns ms per forward+backward
    step and the peak device memory it needs beyond its inputs."""
    import torch
    import torch.nn.functional as F
    ec = e.detach().clone().requires_grad_(True)
    cc = c.detach().clone().requires_grad_(True)

    def run():
        logits = (ec @ cc.t()).float()
        loss = F.cross_entropy(logits, t, ignore_index=-100, reduction="mean")
        loss.backward()
        ec.grad = None
        cc.grad = None

    run()
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    run()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(steps):
        run()
    s1.record()
    torch.cuda.synchronize()
    del ec, cc
    torch.cuda.empty_cache()
    return s0.elapsed_time(s1) / steps, peak


def autograd_memory(e, c, t, reduction):
    """Peak device memory of one training step through the autograd wrapper
    (forward, backward, gradients of e and c in their dtype) beyond its
    inputs, measured as for the materialised head, and the bytes autograd
    keeps from the forward to the backward beyond the inputs (the forward
    state, LSE and loss)."""
    import torch
    import linear_cross_entropy_forward_amd as M
    ec = e.detach().clone().requires_grad_(True)
    cc = c.detach().clone().requires_grad_(True)

    def run():
        loss = M.linear_cross_entropy(ec, cc, t, reduction="mean" if reduction != "none" else "none")
        (loss.sum() if reduction == "none" else loss).backward()
        ec.grad = None
        cc.grad = None

    run()
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    run()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    loss = M.linear_cross_entropy(ec, cc, t, reduction="mean")
    torch.cuda.synchronize()
    saved = torch.cuda.memory_allocated() - base
    del loss, ec, cc
    torch.cuda.empty_cache()
    return peak, saved


def hipblaslt_gemm_tflops(c, e, reps=5):
    """torch.mm (hipBLASLt) on the forward contraction's shape, c [V, D] x e^T:
    a practical MFMA ceiling for the same M, N, K."""
    import torch
    et = e.t().contiguous()
    out = torch.mm(c, et)
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(reps):
        torch.mm(c, et, out=out)
    s1.record()
    torch.cuda.synchronize()
    ms = s0.elapsed_time(s1) / reps
    del out, et
    return 2.0 * c.shape[0] * c.shape[1] * e.shape[0] / (ms * 1e-3) / 1e12


def make_bias(V, dtype, dev, seed=7):
    """Seeded classifier bias, N(0, 0.5^2), in the classifier's dtype."""
    import torch
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(V, generator=g) * 0.5).to(dtype).to(dev)


def config_summary(name, steps=5, warmup=2, materialized_too=True, with_bias=False, label_smoothing=0.0,
                   z_loss=0.0, softcap=0.0, filter=True, accum="deterministic", frozen_classifier=False,
                   grad_dtype="operand", graph=False):
    """Compact forward / forward+backward figures for one workload (defaults:
    filter on, deterministic, the workload's own reduction; with_bias adds a
    classifier bias and asks for its gradient; label_smoothing / z_loss add
    those loss terms; softcap soft-caps the logits; filter / accum select the
    backward's tile filter and accumulation mode)."""
    import torch
    import workloads as W
    import linear_cross_entropy_forward_amd as M
    w = W.WORKLOADS[name]
    inp = W.generate(w)
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    e = torch.from_numpy(inp["e"]).to(tdt).to(dev)
    c = torch.from_numpy(inp["c"]).to(tdt).to(dev)
    t = torch.from_numpy(inp["targets"]).to(dev)
    N, D = e.shape
    V = c.shape[0]
    n_valid = max(1, int((inp["targets"] != -100).sum()))
    del inp
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    state = torch.empty(M.state_size(N, D, V, tdt), dtype=torch.uint8, device=dev)
    ws = torch.empty(M.workspace_size(N, D, V, tdt), dtype=torch.uint8, device=dev)
    red = {"none": 0, "sum": 1, "mean": 2}[w.reduction]
    loss = torch.empty(N if red == 0 else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int32, device=dev)
    g = torch.full((N,) if red == 0 else (1,), 1.0 / n_valid if red == 0 else 1.0, dtype=torch.float32,
                   device=dev)
    gdt = tdt if grad_dtype == "operand" else torch.float32
    dE = torch.empty((N, D), dtype=gdt, device=dev)
    dC = None if frozen_classifier else torch.empty((V, D), dtype=gdt, device=dev)
    bias = make_bias(V, tdt, dev) if with_bias else None
    db = torch.empty(V, dtype=torch.float32, device=dev) if with_bias else None
    extra = torch.cuda.memory_allocated() - base
    L = M.lib()
    dcode = 0 if w.dtype == "bf16" else 1
    st = torch.cuda.current_stream()
    bp = bias.data_ptr() if with_bias else None
    dbp = db.data_ptr() if with_bias else None

    def fwd():
        # on the current stream (a graph capture runs on its own)
        r = L.cce_forward(e.data_ptr(), c.data_ptr(), bp, t.data_ptr(), N, D, V, dcode, -100, red, softcap,
                          label_smoothing, z_loss, loss.data_ptr(), lse.data_ptr(), nv.data_ptr(),
                          state.data_ptr(), state.numel(), torch.cuda.current_stream().cuda_stream)
        if r:
            raise RuntimeError(f"cce_forward failed: {r}")

    def step():
        fwd()
        r = L.cce_backward(e.data_ptr(), c.data_ptr(), bp, t.data_ptr(), N, D, V, dcode, -100, red, softcap,
                           label_smoothing, z_loss, lse.data_ptr(), g.data_ptr(), 1 if filter else 0,
                           0 if accum == "deterministic" else 1, 0, 1 if grad_dtype == "operand" else 0,
                           dE.data_ptr(),
                           None if dC is None else dC.data_ptr(), dbp, state.data_ptr(), state.numel(),
                           ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
        if r:
            raise RuntimeError(f"cce_backward failed: {r}")

    def timed(fn):
        for _ in range(warmup):
            fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(steps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    step_ms = timed(step)
    fwd_ms = timed(fwd)
    graph_ms = None
    if graph:
        # the same step captured once in a HIP graph and replayed (no launch
        # overhead per kernel; the library's calls are capture-safe)
        side = torch.cuda.Stream()
        side.wait_stream(st)
        with torch.cuda.stream(side):
            step()
        st.wait_stream(side)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            step()
        graph_ms = timed(gr.replay)
    stats = M.read_stats(state, N, V)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    # effective work: 2NVD per contraction (forward, recompute, dE, dC)
    eff = (6.0 if frozen_classifier else 8.0) * N * V * D / (step_ms * 1e-3) / 1e12
    # executed work: the forward in full, the recompute on the kept tiles,
    # the gradient contractions on the kept 32x32 blocks
    kept = stats["tiles_kept"] / max(1, stats["tiles_total"])
    kept_b = stats["blocks_kept"] / max(1, stats["blocks_total"])
    exec_frac = (2.0 + 2.0 * kept + (2.0 if frozen_classifier else 4.0) * kept_b) / (6.0 if frozen_classifier else 8.0)
    out = {"N": N, "D": D, "V": V, "dtype": w.dtype, "reduction": w.reduction, "fwd_ms": fwd_ms,
           "fwd_tokens_per_s": N / (fwd_ms * 1e-3), "step_ms": step_ms, "tokens_per_s": N / (step_ms * 1e-3),
           "tflops_effective": eff, "pct_of_peak_effective": 100.0 * eff / peak,
           "executed_flop_frac": exec_frac, "tflops_executed": eff * exec_frac,
           "pct_of_peak_executed": 100.0 * eff * exec_frac / peak,
           "tflops_useful": eff * (4.0 / 6.0 if frozen_classifier else 0.75), "filter": bool(filter),
           "accum": accum,
           # the accumulation mode concerns dE only: each dC element has one
           # owning work-group (whole token contraction), so dC is the same
           # kernel and the same bits in both modes
           "accum_applies_to": "dE",
           "frozen_classifier": bool(frozen_classifier),
           "grad_dtype": "bf16" if gdt == torch.bfloat16 else "f32", "step_ms_graph": graph_ms,
           "tiles_skipped_frac": 1.0 - stats["tiles_kept"] / max(1, stats["tiles_total"]),
           "blocks_skipped_frac": 1.0 - stats["blocks_kept"] / max(1, stats["blocks_total"]),
           "extra_hbm_bytes": int(extra), "state_bytes": int(state.numel()), "workspace_bytes": int(ws.numel()),
           "bias": bool(with_bias), "label_smoothing": label_smoothing,
           "z_loss": z_loss, "softcap": softcap}
    plain = (not with_bias and label_smoothing == 0.0 and z_loss == 0.0 and softcap == 0.0 and filter
             and accum == "deterministic" and not frozen_classifier and grad_dtype == "operand")
    if w.dtype == "bf16" and plain:
        out["hipblaslt_fwd_gemm_tflops"] = hipblaslt_gemm_tflops(c, e)
    del state, ws, loss, lse, nv, g, dE, dC, bias, db
    torch.cuda.empty_cache()
    if materialized_too and plain:
        mat_ms, mat_peak = materialized(e, c, t, w.reduction, max(1, min(steps, 3)))
        out["materialized_step_ms"] = mat_ms
        out["materialized_peak_extra_bytes"] = int(mat_peak)
    del e, c, t
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import workloads as W
    import linear_cross_entropy_forward_amd as M

    dev = torch.device("cuda:0")
    w = W.WORKLOADS[args.workload]
    reduction = args.reduction or w.reduction
    inp = W.generate(w)
    dt_name = w.dtype
    tdt = torch.bfloat16 if dt_name == "bf16" else torch.float32
    e = torch.from_numpy(inp["e"]).to(tdt).to(dev)
    c = torch.from_numpy(inp["c"]).to(tdt).to(dev)
    t = torch.from_numpy(inp["targets"]).to(dev)
    N, D = e.shape
    V = c.shape[0]
    es = 2 if dt_name == "bf16" else 4
    n_valid = int((inp["targets"] != -100).sum())
    L = M.lib()

    if args.copy_calibration:
        src = torch.empty(args.copy_calibration // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    base_alloc = torch.cuda.memory_allocated()
    state = torch.empty(M.state_size(N, D, V, tdt), dtype=torch.uint8, device=dev)
    ws = torch.empty(M.workspace_size(N, D, V, tdt, args.vocab_chunk), dtype=torch.uint8, device=dev)
    red = {"none": 0, "sum": 1, "mean": 2}[reduction]
    loss = torch.empty(N if red == 0 else 1, dtype=torch.float32, device=dev)
    lse = torch.empty(N, dtype=torch.float32, device=dev)
    nv = torch.empty(1, dtype=torch.int32, device=dev)
    # upstream gradient: for per-token loss, 1/n_valid per row (the mean's gradient)
    g = torch.full((N,) if red == 0 else (1,), 1.0 / n_valid if red == 0 else 1.0, dtype=torch.float32,
                   device=dev)
    gdt = tdt if args.grad_dtype == "operand" else torch.float32
    gcode = 1 if args.grad_dtype == "operand" else 0
    dE = torch.empty((N, D), dtype=gdt, device=dev)
    dC = torch.empty((V, D), dtype=gdt, device=dev)
    dcode = 0 if dt_name == "bf16" else 1
    flt = 0 if args.no_filter else 1
    acc = 0 if args.accum == "deterministic" else 1
    stream = torch.cuda.current_stream()

    def fwd(s):
        r = L.cce_forward(e.data_ptr(), c.data_ptr(), None, t.data_ptr(), N, D, V, dcode, -100, red, 0.0, 0.0, 0.0,
                          loss.data_ptr(), lse.data_ptr(), nv.data_ptr(), state.data_ptr(), state.numel(), s)
        if r:
            raise RuntimeError(f"cce_forward failed: {r}")

    def step():
        s = stream.cuda_stream
        fwd(s)
        r = L.cce_backward(e.data_ptr(), c.data_ptr(), None, t.data_ptr(), N, D, V, dcode, -100, red, 0.0, 0.0,
                           0.0, lse.data_ptr(), g.data_ptr(), flt, acc, args.vocab_chunk, gcode, dE.data_ptr(),
                           dC.data_ptr(), None, state.data_ptr(), state.numel(), ws.data_ptr(), ws.numel(), s)
        if r:
            raise RuntimeError(f"cce_backward failed: {r}")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stats = M.read_stats(state, N, V)

    def timed_steps():
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(args.steps):
            step()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    # timed region: K steps, nothing recorded between the kernels
    total_ms = timed_steps()

    # per-kernel split: the same K steps again with HIP events recorded by the
    # library around every kernel launch on the launch stream
    for k in range(len(KERNELS)):
        L.cce_profile_start(k, 64 * max(1, args.steps))
    profiled_ms = timed_steps()
    import ctypes
    per = {}
    for k, name in enumerate(KERNELS):
        ms, n = ctypes.c_double(), ctypes.c_int()
        L.cce_profile_stop(k, ctypes.byref(ms), ctypes.byref(n))
        if n.value:
            per[name] = {"launches_per_step": n.value / args.steps, "avg_ms": ms.value / n.value,
                         "ms_per_step": ms.value / args.steps}

    # forward alone (not part of the metric): separate short timing
    f0 = torch.cuda.Event(enable_timing=True)
    f1 = torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(args.steps):
        fwd(stream.cuda_stream)
    f1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = f0.elapsed_time(f1) / args.steps

    ms_step = total_ms / args.steps
    tok_s = N / (ms_step * 1e-3)
    eff_flops = 8.0 * N * V * D
    peak = PEAK_BF16_TFLOPS if dt_name == "bf16" else PEAK_F32_TFLOPS
    tflops = eff_flops / (ms_step * 1e-3) / 1e12
    kept_frac = stats["tiles_kept"] / max(1, stats["tiles_total"])
    kept_bfrac = stats["blocks_kept"] / max(1, stats["blocks_total"])
    # executed: forward, recompute of the kept tiles, contractions of the kept blocks
    exec_frac = (2.0 + 2.0 * kept_frac + 4.0 * kept_bfrac) / 8.0

    Vc = M.vocab_chunk(N, D, V, tdt, args.vocab_chunk)
    nVB = -(-V // 128)
    kernels = {}
    for name, d in per.items():
        fl, by = algorithmic(name, N, D, V, es, nVB, d["launches_per_step"], kept_frac)
        d = dict(d)
        d["tflops"] = fl / (d["avg_ms"] * 1e-3) / 1e12 if fl else None
        d["gbs"] = by / (d["avg_ms"] * 1e-3) / 1e9 if by else None
        d["traffic_bytes"] = traffic_for(name, args.workload)
        kernels[name] = d
    dom = max(per, key=lambda k: per[k]["ms_per_step"])
    fl, by = algorithmic(dom, N, D, V, es, nVB, per[dom]["launches_per_step"], kept_frac)
    if dom in MFMA_KERNELS:
        ach = fl / (per[dom]["avg_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak,
                "traffic": traffic_for(dom, args.workload), "kernel": dom,
                "avg_launch_ms": per[dom]["avg_ms"], "algorithmic_flops_per_launch": fl}
        if dom in ("dC_gemm", "dE_gemm"):
            # the MFMAs it issues: those of the kept 32x32 blocks
            roof["mfma_flops_executed_per_launch"] = fl * kept_bfrac / max(kept_frac, 1e-30)
    else:
        ach = by / (per[dom]["avg_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "traffic": traffic_for(dom, args.workload), "kernel": dom,
                "avg_launch_ms": per[dom]["avg_ms"], "algorithmic_bytes_per_launch": by}

    # device memory this path needs beyond its inputs: the forward state, the
    # backward workspace, loss/LSE and the two gradient outputs
    extra_bytes = torch.cuda.memory_allocated() - base_alloc
    ws_bytes = ws.numel()
    state_bytes = state.numel()
    hip_tf = hipblaslt_gemm_tflops(c, e) if dt_name == "bf16" else None
    mat = None
    ag_peak = ag_saved = None
    if not args.no_materialized:
        del dE, dC
        torch.cuda.empty_cache()
        ag_peak, ag_saved = autograd_memory(e, c, t, reduction)
        mat_ms, mat_peak = materialized(e, c, t, reduction, max(1, min(args.steps, 3)))
        mat = {"ms_per_step": mat_ms, "tokens_per_s": N / (mat_ms * 1e-3), "peak_extra_bytes": int(mat_peak),
               "what": "PyTorch: fp32 logits = e @ c^T, F.cross_entropy(mean), backward"}

    others = None
    if not args.no_configs:
        del e, c, t, state, ws, loss, lse, nv, g
        dE = dC = None
        torch.cuda.empty_cache()
        others = {}
        for name in ("tiny", "llama1b", "gemma2b", "gemma2b_cal", "long8b", "long8b_cal", "llama8b_pad25"):
            if name != args.workload:
                others[name] = config_summary(name, graph=name == "tiny")
        # the headline workload with a classifier bias and its gradient
        others[args.workload + "+bias"] = config_summary(args.workload, with_bias=True)
        # ... and with label smoothing 0.1 and z-loss 1e-4
        others[args.workload + "+smoothing+zloss"] = config_summary(args.workload, label_smoothing=0.1,
                                                                     z_loss=1e-4)
        # Gemma 2's final-logit soft-capping (30) on the calibrated Gemma-2-2B head
        others["gemma2b_cal+softcap30"] = config_summary("gemma2b_cal", softcap=30.0)
        # the filter off (Llama-3.2-1B) and fp32 atomic accumulation (long context)
        others["llama1b+nofilter"] = config_summary("llama1b", filter=False, materialized_too=False)
        others["long8b_cal+atomic"] = config_summary("long8b_cal", accum="atomic", materialized_too=False)
        # fp32 gradient outputs
        others[args.workload + "+fp32_grads"] = config_summary(args.workload, grad_dtype="float32",
                                                                materialized_too=False)
        # a frozen classifier: dE alone (dC's contraction does not run)
        others[args.workload + "+frozen_classifier"] = config_summary(args.workload, frozen_classifier=True,
                                                                       materialized_too=False)

    cpu = None
    if not args.no_cpu_baseline:
        rows_n = args.cpu_rows or (2048 if dt_name == "bf16" else N)
        cpu = cpu_baseline(inp, min(rows_n, N))

    out = {
        "metric": "fwd+bwd tokens/sec & MFMA util % at Llama-3.1-8B head (D=4096, V=128256)",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if dt_name == "bf16" else "f32",
        "data": "synthetic (seeded; e ~ N(0,1), c ~ N(0,0.02^2) bf16, uniform targets)",
        "config": {"workload": args.workload, "N": N, "D": D, "V": V, "reduction": reduction,
                   "filter": bool(flt), "accum": args.accum, "accum_applies_to": "dE", "vocab_chunk": Vc,
                   "grad_dtype": "bf16" if gdt == torch.bfloat16 else "f32"},
        # effective (unfiltered, 8NVD) flops of the step per second over the
        # dense bf16 peak; not a hardware counter (the matrix cores' busy
        # fraction per contraction, from SQ_VALU_MFMA_BUSY_CYCLES:
        # profiles/llama8b_mfma_lds_counters.md)
        "mfma_util_pct": 100.0 * tflops / peak,
        "mfma_util_what": "effective 8NVD flops / step time / dense bf16 peak (not a counter reading)",
        "tflops_effective": tflops,
        "tflops_useful": tflops * 0.75,  # 6NVD: the step without the recompute
        "executed_flop_frac": exec_frac,
        "tflops_executed": tflops * exec_frac,
        "profiled_pass_ms_per_step": profiled_ms / args.steps,
        "fwd_ms": fwd_ms,
        "fwd_tokens_per_s": N / (fwd_ms * 1e-3),
        "tiles_kept_frac": stats["tiles_kept"] / max(1, stats["tiles_total"]),
        "blocks_kept_frac": kept_bfrac,
        "state_bytes": state_bytes,
        "workspace_bytes": ws_bytes,
        "extra_hbm_bytes": int(extra_bytes),
        "autograd_peak_extra_bytes": ag_peak,
        "autograd_saved_bytes": ag_saved,
        "loss_path_overhead_bytes": int(N * nVB * 8 + N * 8),
        "materialized_logits_fp32_bytes": N * V * 4,
        "materialized_baseline": mat,
        "hipblaslt_fwd_gemm_tflops": hip_tf,
        "other_workloads": others,
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
