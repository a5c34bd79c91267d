#!/usr/bin/env python3
"""Benchmark of the DoRA forward hot path on one MI355X.

One step = the factored row norm (wnorm and g) followed by the magnitude
compose, over one batch of synthetic inputs already resident in HBM.
Default workload: d_out = d_in = 8192, r = 384, s = 0.5, bf16, compose over
T = 8192 rows (batch 2 x seq 4096).

The fused compose backward (d_base, d_lora, dg, dm) is timed after the
steps, on its own, and reported under "compose_backward"; "comparisons"
holds the eager PyTorch compose and a PEFT-style dense norm (time and peak
memory) measured the same way; "linear_forward" times the whole DoRA
linear layer (projections by hipBLASLt, norm and output by libdora) at the
workload's T beside a plain LoRA layer.

Prints one JSON line. `value` is the factored norm's algorithmic TFLOP/s;
the compose's GB/s and fraction of HBM peak, per-call times and the
roofline objects ride in the same line. Kernel times come from HIP events
recorded on the stream the kernels run on; the W-pass kernel inside the
norm call is timed by events dora_factored_norm_marked records around its
launch. Before the warm-up steps, steps run for PREWARM_S seconds whatever
--warmup says, so that the timed steps find the clocks up.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-backward]
                    [--no-comparisons] [--no-linear]
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
F32_MFMA_PEAK_TFLOPS = 157.3
NSETS = 3                       # input sets the steps rotate through
ROUNDS = 5                      # rounds of K back-to-back calls for the per-call times
PREWARM_S = 1.0                 # steps run before the warm-up, whatever --warmup says
METRIC = "factored-norm ms/TFLOP/s + compose GB/s (%HBM peak), 8192×8192 r=384 bf16"


def norm_flops(d_out, d_in, r):
    """U = W A^T, G = A A^T, B G, the base squares, and the two row dots."""
    return 2 * d_out * d_in * r + 2 * r * r * d_in + 2 * d_out * r * r + 2 * d_out * d_in + 4 * d_out * r


def w_pass_flops(d_out, d_in, r, plan):
    """Algorithmic work of the W-pass kernel alone: U = W A^T, the base
    squares and the row dot with B; with the Gram term inside it also B G,
    with G folded into it also G = A A^T."""
    f = 2 * d_out * d_in * r + 2 * d_out * d_in + 2 * d_out * r
    if plan["gram_term_fused"]:
        f += 2 * d_out * r * r
    if plan["gram_folded"]:
        f += 2 * r * r * d_in
    return f


def dense_flops(d_out, d_in, r):
    """The dense fused pass (plan mode 3): B A over r, then W + s (B A) and its square summed per row."""
    return 2 * d_out * d_in * r + 4 * d_out * d_in


def norm_bytes(d_out, d_in, r, esize):
    """W, A, B read once; m read, wnorm and g written (fp32)."""
    return (d_out * d_in + r * d_in + d_out * r) * esize + 12 * d_out


def compose_bytes(T, d_out, esize):
    """base and lora read, out written; g read once (fp32)."""
    return 3 * T * d_out * esize + 4 * d_out


def compose_bwd_bytes(T, d_out, esize, dm=True):
    """dy, base and lora read, d_base and d_lora written; g read and dg
    written (fp32); with the magnitude trained also wnorm read, dm written."""
    return 5 * T * d_out * esize + (16 if dm else 8) * d_out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, W, A, B, base, lora, g_host):
    """The fp64 CPU oracle, as it stands, on the same workload.

    Each leg is one untimed run, then the median of three timed runs: the
    whole norm (dense W + sBA in fp64 through BLAS) on every core BLAS uses
    and again on one BLAS thread, and the compose over all rows (elementwise
    numpy, one thread) rounded once to the storage type.
    """
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import dora_oracle as O

    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] or [1])
    affinity = len(os.sched_getaffinity(0))

    def median3(fn):
        fn()
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    t_norm = median3(lambda: O.dense_row_norm(W, A, B, w.s))
    with threadpool_limits(limits=1, user_api="blas"):
        t_norm1 = median3(lambda: O.dense_row_norm(W, A, B, w.s))
    t_comp = median3(lambda: O.round_to_dtype(O.compose(base, lora, g_host, w.s), w.dtype))
    esize = 2 if w.dtype == "bf16" else 4
    F = norm_flops(w.d_out, w.d_in, w.r)
    cpu = _cpu_model()
    return {
        "value": F / t_norm / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"whole workload, fp64, each leg one untimed run then the median of 3: the norm "
                   f"({w.d_out}x{w.d_in}, r={w.r}) {t_norm:.3f} s on {threads} BLAS threads and {t_norm1:.3f} s on "
                   f"one; the compose over all {w.T} rows (elementwise numpy, one thread) {t_comp:.3f} s; "
                   f"{affinity} cores in the affinity mask, {cpu}"),
        "cpu_model": cpu,
        "affinity_cores": affinity,
        "norm_ms": t_norm * 1e3,
        "value_1thread": F / t_norm1 / 1e12,
        "norm_ms_1thread": t_norm1 * 1e3,
        "compose_ms": t_comp * 1e3,
        "compose_gbs": compose_bytes(w.T, w.d_out, esize) / t_comp / 1e9,
    }


def time_compose_backward(args, w, lib, bnd, I, based, lorad, g, wnorm, stream, tdt, esize):
    """The fused compose backward, timed on its own after the forward steps
    (it is not part of a forward step): d_base, d_lora, dg and dm over the
    same T x d_out batch, with dy drawn like the other inputs."""
    import numpy as np
    import torch

    P = ctypes.c_void_p
    dy_h, _ = I.grad_inputs(w.T, w.d_out, w.dtype, w.seed)
    dy = torch.from_numpy(dy_h).cuda().to(tdt)
    del dy_h
    d_base, d_lora = torch.empty_like(dy), torch.empty_like(dy)
    dg = torch.empty(w.d_out, dtype=torch.float32, device="cuda")
    dm = torch.empty_like(dg)
    ws_bytes = bnd.dora_compose_backward_workspace_size(w.T, w.d_out)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    dt = bnd._dtype_code(w.dtype)
    a = (P(dy.data_ptr()), P(based.data_ptr()), P(lorad.data_ptr()), P(g.data_ptr()), w.s, dt, w.T, w.d_out,
         P(d_base.data_ptr()), P(d_lora.data_ptr()), P(dg.data_ptr()), P(wnorm.data_ptr()), w.eps,
         P(dm.data_ptr()), P(ws.data_ptr()), ws_bytes, P(stream.cuda_stream))

    def run():
        st = lib.dora_compose_backward(*a)
        if st:
            raise bnd.DoraError("dora_compose_backward", st)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    K = args.steps
    print(f"# timing {K} compose backward calls, {ROUNDS} rounds", file=sys.stderr, flush=True)
    rounds = [_event_ms(run, K, stream) for _ in range(ROUNDS)]
    ms = float(np.median(rounds))
    nb = compose_bwd_bytes(w.T, w.d_out, esize)
    gbs = nb / (ms * 1e-3) / 1e9
    eager_ms = eager_compose_backward_ms(args, w, based, lorad, g, dy, stream)
    return {"ms": ms, "rounds_ms": rounds, "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "algorithmic_bytes": nb, "workspace_bytes": ws_bytes,
            "eager_autograd_ms": eager_ms, "speedup_vs_eager": eager_ms / ms,
            "note": "d_base, d_lora, dg and dm in one C-ABI call (row-strip kernel + fixed-order column "
                    "reduction); timed separately, not part of the forward step"}


def eager_compose_backward_ms(args, w, based, lorad, g, dy, stream):
    """The eager baseline of the fused backward: PyTorch autograd through the
    eager compose (g - 1) * base + g * (s * lora) in the storage dtype, with
    base, lora and g (cast to the storage dtype) requiring gradients; only
    the backward (torch.autograd.grad on a retained graph) is timed, like the
    fused call it is set beside."""
    import numpy as np
    import torch

    base = based.detach().requires_grad_(True)
    lora = lorad.detach().requires_grad_(True)
    gg = g.detach().to(based.dtype).requires_grad_(True)
    out = (gg - 1) * base + gg * (w.s * lora)

    def bwd():
        return torch.autograd.grad(out, (base, lora, gg), dy, retain_graph=True)

    for _ in range(2):
        bwd()
    torch.cuda.synchronize()
    reps = max(3, min(args.steps, 20))
    ms = float(np.median([_event_ms(bwd, reps, stream) for _ in range(3)]))
    del out
    return ms


# The pages' norm-memory comparisons (cyqw.cn §1.3 Table 1 and the measured
# 768 -> 241 MB under it, at d = 8192, r = 512, fp32, 256 MB budget; §3.3,
# the 8192 x 28672 MoE-expert shape), as (name, d_out, d_in, r, dtype).
PAGE_NORM_CONFIGS = [
    ("square_8192x8192_r512_f32", 8192, 8192, 512, "f32"),
    ("mlp_28672x8192_r512_bf16", 28672, 8192, 512, "bf16"),
]


def page_norm_comparisons(bnd, stream, seed=7):
    """Peak allocator memory and time of three ways to get ||W + sBA||_row at
    the pages' shapes, on synthetic seeded inputs (W, A ~ N(0, 1/d_in),
    B ~ N(0, 0.02^2); s = 0.5; 256 MiB budget):

    - dense: torch.linalg.norm(W + s * (B @ A), dim=1), the plain form;
    - identity form: the adapter weight built by running the adapter on an
      identity matrix, (I A^T) B^T, transposed and added to W, then the row
      norm, as the pages describe PEFT doing it (cyqw.cn §1.1: an identity
      matrix of d_in x d_in plus several dense temporaries);
    - factored: dora_factored_norm (workspace and outputs included).

    Peaks are torch.cuda.max_memory_allocated above what was resident before
    the call."""
    import numpy as np
    import torch

    out = []
    for name, d_out, d_in, r, dt in PAGE_NORM_CONFIGS:
        tdt = torch.float32 if dt == "f32" else torch.bfloat16
        gen = torch.Generator(device="cuda")
        gen.manual_seed(seed)
        W = (torch.randn(d_out, d_in, device="cuda", generator=gen) / d_in ** 0.5).to(tdt)
        A = (torch.randn(r, d_in, device="cuda", generator=gen) / d_in ** 0.5).to(tdt)
        B = (torch.randn(d_out, r, device="cuda", generator=gen) * 0.02).to(tdt)
        s, budget = 0.5, 256 << 20

        def dense():
            return torch.linalg.norm(W + s * (B @ A), dim=1)

        def identity_form():
            eye = torch.eye(d_in, dtype=tdt, device="cuda")
            lora_w = (eye @ A.t()) @ B.t()            # [d_in, d_out]: the adapter applied to I
            return torch.linalg.norm(W + s * lora_w.t(), dim=1)

        def factored():
            return bnd.dora_factored_norm(W, A, B, s, budget_bytes=budget)[0]

        res = {"config": name, "d_out": d_out, "d_in": d_in, "r": r, "dtype": dt, "budget_MiB": budget >> 20}
        vals = {}
        for key, fn in (("dense", dense), ("identity_form", identity_form), ("factored", factored)):
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
            base_mem = torch.cuda.memory_allocated()
            torch.cuda.reset_peak_memory_stats()
            v = fn()
            torch.cuda.synchronize()
            res[f"{key}_peak_bytes"] = torch.cuda.max_memory_allocated() - base_mem
            vals[key] = v.float()
            del v
            fn()
            torch.cuda.synchronize()
            res[f"{key}_ms"] = float(np.median([_event_ms(fn, 5, stream) for _ in range(3)]))
        res["dense_over_factored_memory"] = res["dense_peak_bytes"] / max(res["factored_peak_bytes"], 1)
        res["identity_form_over_factored_memory"] = res["identity_form_peak_bytes"] / max(res["factored_peak_bytes"], 1)
        res["max_rel_diff_factored_vs_dense"] = float(((vals["factored"] - vals["dense"]).abs()
                                                        / vals["dense"].abs()).max())
        out.append(res)
        del W, A, B, vals
        torch.cuda.empty_cache()
    return out


def _event_ms(fn, reps, stream):
    """Mean milliseconds of fn() over reps back-to-back calls: HIP events on
    `stream` before the first call and after the last (none in between)."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def comparisons(args, w, bnd, Wd, Ad, Bd, based, lorad, g, md, comp_ms, norm_ms, stream, tdt):
    """The pages' own comparisons, measured on this GPU (not part of a step):

    - eager compose: the PyTorch expression (g-1)*base + g*(s*lora) in the
      storage dtype, four elementwise launches over T x d_out, against the
      fused compose;
    - dense norm: the PEFT-style ||W + s*(B @ A)||_row, which materialises
      the d_out x d_in product, against the factored norm, in time and in
      peak allocator memory (torch.cuda.max_memory_allocated).
    """
    import torch

    reps = max(3, min(args.steps, 20))
    gb = g.to(tdt)
    gm1 = gb - 1

    def eager():
        return gm1 * based + gb * (w.s * lorad)

    for _ in range(2):
        eager()
    torch.cuda.synchronize()
    eager_ms = _event_ms(eager, reps, stream)

    def dense():
        return torch.linalg.norm(Wd + w.s * (Bd @ Ad), dim=1)

    ws_bytes = bnd.dora_norm_workspace_size(w.d_out, w.d_in, w.r, w.dtype, w.s, w.budget)

    def factored():
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        return bnd.dora_factored_norm(Wd, Ad, Bd, w.s, budget_bytes=w.budget, m=md, eps=w.eps, workspace=ws)

    def peak(fn):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base_mem = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        out = fn()
        torch.cuda.synchronize()
        extra = torch.cuda.max_memory_allocated() - base_mem
        del out
        return extra

    dense()
    torch.cuda.synchronize()
    dense_ms = _event_ms(dense, reps, stream)
    dense_peak = peak(dense)
    fact_peak = peak(factored)
    return {
        "eager_compose_ms": eager_ms,
        "fused_compose_ms": comp_ms,
        "compose_speedup_vs_eager": eager_ms / comp_ms,
        "dense_norm_ms": dense_ms,
        "factored_norm_ms": norm_ms,
        "norm_speedup_vs_dense": dense_ms / norm_ms,
        "dense_norm_peak_bytes": dense_peak,
        "factored_norm_peak_bytes": fact_peak,
        "norm_memory_ratio": dense_peak / max(fact_peak, 1),
        "note": "eager compose: 4 elementwise torch launches in the storage dtype; dense norm: "
                "torch.linalg.norm(W + s*(B @ A), dim=1) as PEFT forms it; peaks are "
                "torch.cuda.max_memory_allocated above the resident inputs, the factored one "
                "including its workspace and wnorm/g outputs",
    }


def eager_factored_norm(W, A, B, s, chunk):
    """||W + s B A||_row by the three-term identity in eager PyTorch, fp32
    ("DoRA优化技术解析：从内存瓶颈到高效实现", cyqw.cn, §1.2, §1.2.1): the
    row sums of W^2 and U = W A^T built over d_in chunks of `chunk` columns
    (the pages' budget rule bounds the fp32 copy of a chunk), then
    cross = rowsum(B * U) and ba = rowsum((B G) * B) with G = A A^T. The
    comparison baseline for the whole layer; not the library's path."""
    import torch

    d_out, d_in = W.shape
    sq = torch.zeros(d_out, dtype=torch.float32, device=W.device)
    U = torch.zeros(d_out, A.shape[0], dtype=torch.float32, device=W.device)
    for c0 in range(0, d_in, chunk):
        Wc = W[:, c0:c0 + chunk].float()
        sq += Wc.square().sum(dim=1)
        U += torch.mm(Wc, A[:, c0:c0 + chunk].float().t().contiguous())
    Bf = B.float()
    Af = A.float()
    G = torch.mm(Af, Af.t().contiguous())
    cross = (Bf * U).sum(dim=1)
    ba = (torch.mm(Bf, G) * Bf).sum(dim=1)
    return torch.sqrt(torch.clamp_min(sq + 2 * s * cross + s * s * ba, 0))


def linear_forward(args, w, I, Wd, Ad, Bd, md, stream, tdt):
    """The whole DoRA linear layer at this workload's T (not part of a step):
    x W^T and (x A^T) B^T by hipBLASLt, the factored norm and the single-pass
    layer output by libdora. Beside it:
    - the plain LoRA layer (the same two products, then base + s * lora), to
      show what DoRA's magnitude costs;
    - the same layer in eager PyTorch in the pages' standard form (the
      factored norm in fp32 over d_in chunks, g = m / max(wnorm, eps), the
      stable compose (g-1) base + g (s lora) in fp32 added to base), the
      baseline of the pages' end-to-end speed-ups (cyqw.cn, §3.1, §6.1
      Table 9);
    - and in PEFT's form (the dense norm of W + s (B @ A), then the compose
      in the storage dtype, cyqw.cn, §1.1)."""
    import torch

    from dora_weight_norm_amd import binding as bnd
    from dora_weight_norm_amd.layer import dora_linear

    x = torch.from_numpy(I.activations(w.T, w.d_in, w.dtype, w.seed)).cuda().to(tdt)
    reps = max(3, min(args.steps, 20))
    chunk = bnd.dora_norm_chunk_size(w.d_out, w.d_in, w.budget)

    def dora():
        return dora_linear(x, Wd, Ad, Bd, md, w.s, eps=w.eps, budget_bytes=w.budget)

    def lora():
        return torch.mm(x, Wd.t()) + w.s * torch.mm(torch.mm(x, Ad.t()), Bd.t())

    def standard():
        base = torch.mm(x, Wd.t())
        lora_out = torch.mm(torch.mm(x, Ad.t()), Bd.t())
        g = md / torch.clamp_min(eager_factored_norm(Wd, Ad, Bd, w.s, chunk), w.eps)
        bf = base.float()
        delta = (g - 1) * bf + g * (w.s * lora_out.float())
        return (bf + delta).to(tdt)

    def peft():
        base = torch.mm(x, Wd.t())
        lora_out = torch.mm(torch.mm(x, Ad.t()), Bd.t())
        wnorm = torch.linalg.norm(Wd + w.s * (Bd @ Ad), dim=1).float()
        g = (md / torch.clamp_min(wnorm, w.eps)).to(tdt)
        return base + ((g - 1) * base + g * (w.s * lora_out))

    y_fused = dora()
    y_std = standard()
    for fn in (lora, peft):
        fn()
    torch.cuda.synchronize()
    # the fused layer against the standard form: both round y once from fp32
    agree = ((y_fused.float() - y_std.float()).abs().max() / y_std.float().abs().max().clamp_min(1e-30)).item()
    del y_fused, y_std
    dora_ms = _event_ms(dora, reps, stream)
    lora_ms = _event_ms(lora, reps, stream)
    std_ms = _event_ms(standard, reps, stream)
    peft_ms = _event_ms(peft, reps, stream)
    flops = 2 * w.T * w.d_out * w.d_in + 2 * w.T * w.r * (w.d_in + w.d_out)
    return {
        "T": w.T,
        "dora_linear_ms": dora_ms,
        "tokens_per_s": w.T / (dora_ms * 1e-3),
        "gemm_tflops": flops / (dora_ms * 1e-3) / 1e12,
        "lora_linear_ms": lora_ms,
        "dora_overhead_vs_lora": dora_ms / lora_ms,
        "eager_standard_dora_ms": std_ms,
        "speedup_vs_eager_standard": std_ms / dora_ms,
        "eager_peft_dora_ms": peft_ms,
        "speedup_vs_eager_peft": peft_ms / dora_ms,
        "max_rel_diff_vs_standard": agree,
        "note": "y = x (m V/||V||)^T with V = W + sBA; projections by torch.mm (hipBLASLt), norm and "
                "output by libdora; lora_linear is torch.mm(x, W^T) + s * (x A^T) B^T; eager_standard: "
                "factored norm in fp32 torch over the budget's d_in chunks and the fp32 stable compose; "
                "eager_peft: dense norm of W + s (B @ A) and the compose in the storage dtype",
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="headline_8192x8192_r384")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the separately timed compose backward")
    ap.add_argument("--no-comparisons", action="store_true",
                    help="skip the eager-compose and dense-norm comparisons")
    ap.add_argument("--no-linear", action="store_true",
                    help="skip the whole DoRA linear layer forward")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling profiler byte counters)")
    ap.add_argument("--traffic", default=None,
                    help="JSON of measured HBM bytes per call (default: profiles/traffic_<workload>.json)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from dora_weight_norm_amd import binding as bnd
    from dora_weight_norm_amd import inputs as I

    w = I.WORKLOADS[args.workload]
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    esize = 2 if w.dtype == "bf16" else 4
    print(f"# workload {w.name}: generating inputs", file=sys.stderr, flush=True)
    W, A, B = I.norm_inputs(w.d_out, w.d_in, w.r, w.dtype, w.seed)
    base, lora, _ = I.compose_inputs(w.T, w.d_out, w.dtype, w.seed)

    def dev(x):
        return torch.from_numpy(x).cuda().to(tdt)

    Wd, Ad, Bd, based, lorad = dev(W), dev(A), dev(B), dev(base), dev(lora)
    ws_bytes = bnd.dora_norm_workspace_size(w.d_out, w.d_in, w.r, w.dtype, w.s, w.budget)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    wnorm = torch.empty(w.d_out, dtype=torch.float32, device="cuda")
    g = torch.empty(w.d_out, dtype=torch.float32, device="cuda")
    out = torch.empty_like(based)
    # The magnitude vector: m = wnorm * (1 + 0.0015 N(0,1)), so g sits near 1.
    wn0, _ = bnd.dora_factored_norm(Wd, Ad, Bd, w.s, budget_bytes=w.budget)
    noise = torch.from_numpy(I.m_noise(w.d_out, w.seed).astype(np.float32)).cuda()
    md = (wn0 * (1.0 + I.G_SPREAD * noise)).contiguous()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    lib = bnd.load()
    P = ctypes.c_void_p
    sptr = P(stream.cuda_stream)
    dt = bnd._dtype_code(w.dtype)
    # Steps rotate through NSETS copies of the inputs (same values, distinct
    # buffers): one step's W, A, B, base and lora take about 400 MB, so the
    # three sets (1.2 GB) exceed the 256 MB Infinity Cache and the L2, and
    # every step reads its inputs from HBM rather than from what the
    # previous step left in the caches.
    sets = [(Wd, Ad, Bd, based, lorad)] + [tuple(t.clone() for t in (Wd, Ad, Bd, based, lorad))
                                           for _ in range(NSETS - 1)]
    torch.cuda.synchronize()
    norm_args = [(P(S[0].data_ptr()), P(S[1].data_ptr()), P(S[2].data_ptr()), dt, w.d_out, w.d_in, w.r, w.s,
                  w.budget, P(ws.data_ptr()), ws_bytes, P(wnorm.data_ptr()), P(md.data_ptr()), w.eps,
                  P(g.data_ptr()), sptr) for S in sets]
    comp_args = [(P(S[3].data_ptr()), P(S[4].data_ptr()), P(g.data_ptr()), w.s, dt, w.T, w.d_out,
                  P(out.data_ptr()), sptr) for S in sets]

    def run_norm(k=0):
        st = lib.dora_factored_norm(*norm_args[k % NSETS])
        if st:
            raise bnd.DoraError("dora_factored_norm", st)

    def run_compose(k=0):
        st = lib.dora_compose(*comp_args[k % NSETS])
        if st:
            raise bnd.DoraError("dora_compose", st)

    # Pre-warm: steps for PREWARM_S seconds whatever --warmup says, so that
    # the timed steps find the GPU's clocks up (a few warm-up steps last only
    # a millisecond or two, and the first rounds after them run slower).
    print(f"# pre-warm {PREWARM_S:.2f} s, then warmup {args.warmup} steps", file=sys.stderr, flush=True)
    t_pw = time.perf_counter()
    prewarm_steps = 0
    while time.perf_counter() - t_pw < PREWARM_S:
        for _ in range(50):
            run_norm(prewarm_steps)
            run_compose(prewarm_steps)
            prewarm_steps += 1
        torch.cuda.synchronize()
    prewarm_ms = (time.perf_counter() - t_pw) * 1e3
    for k in range(args.warmup):
        run_norm(k)
        run_compose(k)
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    K = args.steps

    def span(fn):
        """Milliseconds per call of fn(k), k = 0 .. K-1, between one event on
        the stream before the first call and one after the last. (An event
        recorded between two launches adds about 3 us to the gap between
        them, so no event is recorded between calls.)"""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(K):
            fn(k)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    def step(k):
        run_norm(k)
        run_compose(k)

    # The timed region: K steps, one norm call and one compose call each.
    print(f"# timing {K} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ms_per_step = span(step)
    wall = time.perf_counter() - t0
    # Per-call times: K calls of each back to back, rotating through the
    # input sets as the steps do, in ROUNDS rounds; the median round counts.
    print(f"# timing the norm and compose calls: {ROUNDS} rounds of {K} calls each", file=sys.stderr, flush=True)
    norm_rounds, comp_rounds = [], []
    for _ in range(ROUNDS):
        norm_rounds.append(span(run_norm))
        comp_rounds.append(span(run_compose))
    norm_ms = float(np.median(norm_rounds))
    comp_ms = float(np.median(comp_rounds))

    # The W-pass kernel inside the norm call: K more steps whose norm call is
    # dora_factored_norm_marked, which records one event on the stream just
    # before that launch and one just after it (launch w_launch lies between
    # marks w_launch and w_launch + 1).
    plan = bnd.dora_norm_plan_info(w.d_out, w.d_in, w.r, w.dtype, w.s, w.budget)
    wl = plan["w_launch"]
    marks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    for pair in marks:
        for e in pair:
            e.record(stream)          # creates the HIP event behind each
    torch.cuda.synchronize()
    mark_arrays = [(P * (wl + 2))(*([None] * wl + [a.cuda_event, b.cuda_event])) for a, b in marks]
    print(f"# timing the W-pass launch over {K} more steps", file=sys.stderr, flush=True)
    for k in range(K):
        st = lib.dora_factored_norm_marked(*norm_args[k % NSETS], mark_arrays[k], wl + 2)
        if st:
            raise bnd.DoraError("dora_factored_norm_marked", st)
        run_compose(k)
    torch.cuda.synchronize()
    w_times = [a.elapsed_time(b) for a, b in marks]
    w_ms = float(np.median(w_times))

    # (the algorithm the plan runs: the factored norm, or the dense fused pass)
    F = dense_flops(w.d_out, w.d_in, w.r) if plan["mode"] == 3 else norm_flops(w.d_out, w.d_in, w.r)
    nb = norm_bytes(w.d_out, w.d_in, w.r, esize)
    cb = compose_bytes(w.T, w.d_out, esize)
    norm_tflops = F / (norm_ms * 1e-3) / 1e12
    norm_gbs = nb / (norm_ms * 1e-3) / 1e9
    comp_gbs = cb / (comp_ms * 1e-3) / 1e9
    mfma_peak = BF16_MFMA_PEAK_TFLOPS if w.dtype == "bf16" else F32_MFMA_PEAK_TFLOPS

    # Measured HBM bytes per call, from rocprofv3 FETCH_SIZE/WRITE_SIZE runs of
    # this same command (see profiles/); null when the kernels changed since.
    from dora_weight_norm_amd import profiling as prof

    tpath = args.traffic or os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    traffic, traffic_note = {}, "no counter run for this workload"
    tj_fields = {}
    if os.path.exists(tpath):
        with open(tpath) as f:
            tj = json.load(f)
        if tj.get("source_hash") == prof.source_hash() and tj.get("w_pass_us_per_launch"):
            tj_fields["w_pass_us_per_launch"] = tj["w_pass_us_per_launch"]
        if tj.get("source_hash") == prof.source_hash():
            traffic = {"norm": tj["norm_bytes_per_call"], "compose": tj["compose_bytes_per_call"],
                       "compose_bwd": tj.get("compose_bwd_bytes_per_call") or None,
                       "w_pass": tj.get("w_pass_bytes_per_launch")}
            traffic_note = os.path.relpath(tpath, ROOT)
        else:
            traffic_note = "kernels changed since the counters in " + os.path.relpath(tpath, ROOT)

    roof_compose = {"bound": "hbm", "achieved": comp_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": comp_gbs / HBM_PEAK_GBS, "traffic": traffic.get("compose"),
                    "kernel": "compose_kernel", "algorithmic_bytes": cb, "traffic_source": traffic_note}
    dense = plan["mode"] == 3
    if dense:
        launches = "dense pass over tiles of W + s B A, assembly"
    elif plan["gram_folded"]:
        launches = "W pass with the G blocks, gram_reduce, Gram term + assembly"
    elif plan["gram_term_fused"]:
        launches = "Gram pass, gram_reduce, W pass with the Gram term, assembly"
    else:
        launches = "Gram pass, gram_reduce, W pass, Gram term + assembly"
    roof_norm = {"bound": "mfma", "achieved": norm_tflops, "peak": mfma_peak, "unit": "TFLOP/s",
                 "frac": norm_tflops / mfma_peak, "traffic": traffic.get("norm"),
                 "kernel": f"dora_factored_norm: {launches} (one C-ABI call, timed as a unit)",
                 "algorithmic_flops": F, "algorithmic_bytes": nb, "hbm_gbs": norm_gbs,
                 "hbm_frac": norm_gbs / HBM_PEAK_GBS, "traffic_source": traffic_note}
    Fw = dense_flops(w.d_out, w.d_in, w.r) if dense else w_pass_flops(w.d_out, w.d_in, w.r, plan)
    w_tflops = Fw / (w_ms * 1e-3) / 1e12
    w_name = ("dense pass" if dense else "W pass with the Gram term" if plan["gram_term_fused"]
              else "W pass with the G blocks" if plan["gram_folded"] else "W pass")
    roof_w = {"bound": "mfma", "achieved": w_tflops, "peak": mfma_peak, "unit": "TFLOP/s",
              "frac": w_tflops / mfma_peak, "traffic": traffic.get("w_pass"),
              "kernel": f"{'norm_dense_kernel' if dense else 'norm_fast_kernel'} ({w_name}; launch {wl} of the norm call)",
              "algorithmic_flops": Fw, "launch_ms": w_ms, "launch_ms_mean": float(np.mean(w_times)),
              "timing": "median over the steps of the interval between the events the library records just "
                        "before and just after the launch (includes its dispatch gap)",
              "traffic_source": traffic_note}
    # The dominant part of a step is the longer of its two calls, as this run
    # timed them: the norm call (its launches back to back, timed as a unit
    # with no event between them; at the headline its W pass is most of it)
    # or the compose call (one launch). Events recorded between the norm
    # call's launches lengthen the gaps around the W pass, so the W-pass
    # interval above reads above the kernel's own duration; the rocprofv3
    # average of the same kernel is given beside it.
    dominant = roof_compose if comp_ms > norm_ms else roof_norm
    dominant = dict(dominant, chosen_by=(f"longer call of a step in this run: norm {norm_ms * 1e3:.1f} us, "
                                         f"compose {comp_ms * 1e3:.1f} us"))
    if "w_pass_us_per_launch" in tj_fields:
        kus = tj_fields["w_pass_us_per_launch"]
        roof_w["kernel_avg_us_rocprofv3"] = kus
        roof_w["achieved_by_rocprofv3_avg"] = Fw / (kus * 1e-6) / 1e12
        roof_w["frac_by_rocprofv3_avg"] = roof_w["achieved_by_rocprofv3_avg"] / mfma_peak

    res = {
        "metric": METRIC,
        "value": norm_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "prewarm_ms": prewarm_ms,
        "prewarm_steps": prewarm_steps,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "d_out": w.d_out, "d_in": w.d_in, "r": w.r, "s": w.s, "T": w.T,
                   "budget_MiB": w.budget >> 20, "parallelism": "single-gpu"},
        "norm_ms": norm_ms,
        "norm_rounds_ms": norm_rounds,
        "norm_tflops": norm_tflops,
        "norm_gbs": norm_gbs,
        "compose_ms": comp_ms,
        "compose_rounds_ms": comp_rounds,
        "compose_gbs": comp_gbs,
        "compose_hbm_frac": comp_gbs / HBM_PEAK_GBS,
        "wall_ms_per_step": wall / K * 1e3,
        "roofline": dominant,
        "roofline_w_pass": roof_w,
        "roofline_norm": roof_norm,
        "roofline_compose": roof_compose,
        "plan": plan,
    }
    if not args.no_backward:
        res["compose_backward"] = time_compose_backward(args, w, lib, bnd, I, based, lorad, g, wnorm, stream,
                                                        tdt, esize)
        res["compose_backward"]["traffic"] = traffic.get("compose_bwd")
    if not args.no_comparisons:
        print("# comparisons: eager compose, dense norm", file=sys.stderr, flush=True)
        res["comparisons"] = comparisons(args, w, bnd, Wd, Ad, Bd, based, lorad, g, md, comp_ms, norm_ms, stream, tdt)
        if "compose_backward" in res:
            cb = res["compose_backward"]
            res["comparisons"].update({"eager_compose_backward_ms": cb["eager_autograd_ms"],
                                       "fused_compose_backward_ms": cb["ms"],
                                       "compose_backward_speedup_vs_eager": cb["speedup_vs_eager"]})
        print("# comparisons: norm memory at the pages' shapes", file=sys.stderr, flush=True)
        res["comparisons"]["page_norm_memory"] = page_norm_comparisons(bnd, stream)
    if not args.no_linear:
        print("# whole DoRA linear layer", file=sys.stderr, flush=True)
        res["linear_forward"] = linear_forward(args, w, I, Wd, Ad, Bd, md, stream, tdt)
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w, W, A, B, base, lora, g.cpu().numpy())
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
