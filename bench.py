"""Benchmark of the AWQ scale search + INT4 group quantization hot path on one MI355X.

One step = one whole layer: activation statistic, candidate scales, quantize->delta for every
candidate, the error GEMM with its fused squared-error epilogue, losses + argmin, and the final
quantize + pack, each through the C ABI on the current stream. Where awq_search_scales would take
the Gram form of the loss (more tokens than input channels: G = X^T X once, then one quadratic form
delta G delta^T per candidate), the step does the same: G, float16 delta, the quadratic-form GEMM. Inputs are generated on the host
(seeded, synthetic) and copied to HBM before timing; outputs and workspaces are preallocated.

Prints one JSON line. `value` = candidate evaluations per second for the whole layer search
(n_grid / seconds per step). `roofline` is for the error GEMM (the dominant kernel), timed with
HIP events on the stream it runs on. `cpu_baseline` times the CPU oracle on a bounded row sample
of the same layer and scales it to the whole layer.

The default workload is the largest single-GPU layer, the 70B down_proj stress layer (X 65536 x
28672 bf16, W 8192 x 28672, n_grid 40); `--config N` selects another. The only error-GEMM launches
of a default run are the timed steps' (and the warm-up's), so a kernel trace of the same command
averages exactly those launches; `--variant-searches` adds whole searches with the other pages'
formula / grid / quantizer pairings.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "layer scale-search time, grid candidates/s, error-GEMM TFLOP/s (% bf16 MFMA peak)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix peak
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E


def _log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _copy_probe(nbytes: int, reps: int) -> None:
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch

    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    a.fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}))


def _source_digest(*paths) -> str:
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


GEMM_SOURCES = ("post_quantization_mean_amd/csrc/err_gemm.hip", "post_quantization_mean_amd/csrc/gemm.h",
                "post_quantization_mean_amd/csrc/lds_dma.h")


def measured_traffic(workload_name: str, gram: bool = False):
    """HBM bytes per launch of the dominant kernel (the error GEMM, or in the Gram form the
    quadratic-form GEMM) from the committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE,
    scaled by a plain copy's readings), or None when the kernel source has changed since the
    counters were taken or no summary exists for this workload."""
    stem = "gram_error_sse" if gram else "error_sse"
    path = os.path.join(ROOT, "profiles", f"{stem}_{workload_name.replace('-', '_')}_traffic.md")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path, encoding="utf-8") as f:
        for line in f:
            if line.startswith("<!-- traffic:"):
                rec = json.loads(line[len("<!-- traffic:"):].rsplit("-->", 1)[0])
    if not rec or rec.get("kernel_digest") != _source_digest(*GEMM_SOURCES):
        return None
    return rec["hbm_bytes_per_launch"]


def cpu_baseline(wl, x_np, w_np, target_s: float) -> dict:
    """The CPU oracle as it stands on a row sample of the layer, scaled to the whole layer."""
    from oracle import awq_oracle as O
    from workloads import to_f32

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    X = to_f32(x_np).astype(np.float64)

    def run(rows: int) -> float:
        W = to_f32(w_np[:rows]).astype(np.float64)
        t0 = time.perf_counter()
        O.search_scales(X, W, wl.group_size, wl.n_grid)
        return time.perf_counter() - t0

    rows = 64
    t = run(rows)
    rows_full = min(wl.d_out, max(rows, int(rows * target_s / max(t, 1e-3))))
    rows_full = max(64, rows_full // 64 * 64)
    if rows_full != rows:
        t = run(rows_full)
        rows = rows_full
    layer_s = t * wl.d_out / rows
    out = {"value": wl.n_grid / layer_s, "unit": "candidates/s", "cores": int(threads), "kind": "oracle",
           "sample": f"full search (act_mean over all {wl.n_tokens} tokens, {wl.n_grid} candidates, float64) on "
                     f"the first {rows} of {wl.d_out} weight rows; {t:.1f} s, scaled by d_out/rows to the layer",
           "layer_seconds_est": layer_s,
           # the oracle's dominant work is the error product X (What - W)^T per candidate, in float64
           "gflops_fp64": 2.0 * wl.n_tokens * wl.d_in * rows * wl.n_grid / t / 1e9,
           "cpu_model": _cpu_model(), "blas": _blas_name()}
    if wl.d_out * wl.d_in <= 1 << 20:  # the tiny workload: also the oracle on one thread
        try:
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                out["single_thread_layer_seconds"] = run(wl.d_out)
        except Exception:  # pragma: no cover
            pass
    return out


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_name() -> str:
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"]
        return ", ".join(libs) or "unknown"
    except Exception:  # pragma: no cover
        return "unknown"



def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", type=int, default=5,
                    help="workload id (5 = 70B down_proj stress, the largest single-GPU layer)")
    ap.add_argument("--cand-per-pass", type=int, default=0, help="candidates per GEMM launch (0 = all)")
    ap.add_argument("--loss-form", choices=("auto", "direct", "gram"), default="auto",
                    help="the error GEMM or the Gram form of the loss (auto: what awq_search_scales chooses)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="also time the step captured once as a HIP graph")
    ap.add_argument("--variant-searches", action="store_true",
                    help="also time whole searches with the other pages' formula/grid/quantizer pairings")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-probe", type=int, default=0, help="only run a device copy of this many bytes")
    ap.add_argument("--print-digest", action="store_true", help="print the error-GEMM source digest and exit")
    args = ap.parse_args()

    if args.print_digest:
        print(_source_digest(*GEMM_SOURCES))
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the search shards by weight "
              "rows with one tiny loss exchange, which this single-GPU build does not implement.",
              file=sys.stderr)
        return 2

    import torch

    if args.copy_probe:
        _copy_probe(args.copy_probe, 10)
        return 0

    from post_quantization_mean_amd import binding as B
    from workloads import make_w, make_x, to_torch, workload

    wl = workload(args.config)
    cpp = args.cand_per_pass or wl.n_grid
    torch.cuda.set_device(0)
    B.load_library()
    _log(f"generating {wl.name}: X {wl.n_tokens}x{wl.d_in} W {wl.d_out}x{wl.d_in} {wl.dtype}")
    x_np, w_np = make_x(wl), make_w(wl)
    x = to_torch(x_np, "cuda")
    w = to_torch(w_np, "cuda")
    parts = list(wl.parts) or [wl.d_out]
    w_parts, r = [], 0
    for p in parts:
        w_parts.append(w[r:r + p])
        r += p
    dev = x.device
    dt = B.AWQ_DTYPE_BF16 if wl.dtype == "bf16" else B.AWQ_DTYPE_F32
    n_tiles = B.awq_error_tiles(wl.n_tokens, wl.d_out)
    G = wl.d_in // wl.group_size
    act = torch.empty(wl.d_in, dtype=torch.float64, device=dev)
    ws_act = torch.empty(B.awq_act_stats_workspace_bytes(dt, wl.n_tokens, wl.d_in), dtype=torch.uint8, device=dev)
    cand = torch.empty((wl.n_grid, wl.d_in), dtype=torch.float64, device=dev)
    if args.loss_form == "auto":
        gram = B.awq_search_loss_form(dt, wl.n_tokens, wl.d_in, wl.d_out, wl.n_grid) == B.AWQ_LOSS_GRAM
    else:
        gram = args.loss_form == "gram"
    if gram:
        # the Gram form: float16 G, its exponent and X^T / float32 G workspace; delta in float16
        g16 = torch.empty((wl.d_in, wl.d_in), dtype=torch.float16, device=dev)
        gexp = torch.empty(1, dtype=torch.int32, device=dev)
        ws_gram = torch.empty(B.awq_gram_workspace_bytes(wl.n_tokens, wl.d_in), dtype=torch.uint8, device=dev)
        dexp = torch.empty(cpp + 1, dtype=torch.int32, device=dev)
        delta16 = torch.empty((cpp, wl.d_out, wl.d_in), dtype=torch.float16, device=dev)
        delta = delta16.view(torch.bfloat16)  # the same bytes, for the bfloat16 delta timed alone below
    else:
        delta = torch.empty((cpp, wl.d_out, wl.d_in), dtype=x.dtype, device=dev)
    sse = torch.empty((wl.n_grid, n_tiles), dtype=torch.float64, device=dev)
    losses = torch.empty(wl.n_grid, dtype=torch.float64, device=dev)
    best = torch.empty(wl.d_in, dtype=torch.float64, device=dev)
    info = torch.empty(2, dtype=torch.int32, device=dev)
    pack_out = {"codes": torch.empty((wl.d_out, wl.d_in // 2), dtype=torch.uint8, device=dev),
                "qscales": torch.empty((wl.d_out, G), dtype=torch.float32, device=dev),
                "zeros": torch.empty((wl.d_out, G), dtype=torch.int32, device=dev)}
    stream = torch.cuda.current_stream()
    ev = {}

    def mark(name):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ev.setdefault(name, []).append(e)

    def step(timed: bool):
        if timed:
            mark("act0")
        B.awq_act_stats(x, act, ws_act)
        B.awq_candidate_scales(act, wl.n_grid, cand)
        if gram:
            if timed:
                mark("gram0")
            B.awq_gram(x, g16, gexp, ws_gram)
            if timed:
                mark("gram1")
        for k0 in range(0, wl.n_grid, cpp):
            nk = min(cpp, wl.n_grid - k0)
            if timed:
                mark("q0")
            if gram:
                B.awq_quant_delta_f16(w_parts, cand[k0:k0 + nk], wl.group_size, delta16[:nk], dexp)
            else:
                B.awq_quant_delta(w_parts, cand[k0:k0 + nk], wl.group_size, delta[:nk])
            if timed:
                mark("g0")
            if gram:
                B.awq_gram_error_sse(g16, gexp, delta16[:nk], dexp, wl.n_tokens, sse[k0:k0 + nk])
            else:
                B.awq_error_sse(x, delta[:nk], sse[k0:k0 + nk])
            if timed:
                mark("g1")
        B.awq_loss_argmin(sse, wl.n_tokens, wl.d_out, cand, losses, best, info)
        if timed:
            mark("p0")
        B.awq_quantize_pack(w_parts, best, wl.group_size, pack_out)
        if timed:
            mark("p1")

    _log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    _log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    def span(a, b):
        return float(sum(s.elapsed_time(e) for s, e in zip(ev[a], ev[b])))

    n_gemm = len(ev["g0"])
    gemm_ms = span("g0", "g1") / n_gemm
    quant_ms = span("q0", "g0") / n_gemm
    pack_ms = span("p0", "p1") / args.steps
    first = "gram0" if gram else "q0"
    act_ms = float(sum(ev["act0"][i].elapsed_time(ev[first][i * (1 if gram else n_gemm // args.steps)])
                       for i in range(args.steps))) / args.steps
    gram_ms = span("gram0", "gram1") / args.steps if gram else None
    n_pad = (wl.n_tokens + 63) // 64 * 64
    tg = (wl.d_in + 255) // 256  # 256-tiles along G's side
    # algorithmic flops of one launch of the dominant kernel: the error GEMM's products, or in the
    # Gram form the quadratic form's delta G products over G's 256-blocks on and right of the
    # diagonal, which G's symmetry leaves to compute (G itself is timed apart)
    if gram:
        rows_k = sum(min(256, wl.d_in - 256 * i) * (wl.d_in - 256 * i) for i in range(tg))
        flops_launch = 2.0 * wl.d_out * rows_k * min(cpp, wl.n_grid)
    else:
        flops_launch = 2.0 * wl.n_tokens * wl.d_in * wl.d_out * min(cpp, wl.n_grid)
    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved = flops_launch / (gemm_ms * 1e-3) / 1e12
    esz = 2 if wl.dtype == "bf16" else 4
    q_bytes = wl.d_out * wl.d_in * esz * (1 + min(cpp, wl.n_grid))
    p_bytes = wl.d_out * wl.d_in * (esz + 0.5) + wl.d_out * G * 8 + wl.d_in * 8
    info_h = info.cpu().tolist()
    _log(f"k*={info_h[0]} flags={info_h[1]} ms/step={ms_step:.3f} gemm={gemm_ms:.3f} ms ({achieved:.1f} TFLOP/s)")

    graph_rep = None
    if args.graph:
        # the same step captured once as a HIP graph (the library allocates, copies and synchronizes
        # nothing, so the whole layer is capturable) and replayed: no per-launch host overhead
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(False)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        g_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        graph_rep = {"ms_per_step": g_ms, "candidates_per_s": wl.n_grid / (g_ms * 1e-3)}
        _log(f"graph replay: {g_ms:.3f} ms/step")
        del g

    # HBM kernels on their own, after the timed steps: before every repetition a 1 GiB buffer is
    # overwritten so that the 256 MB memory-side cache holds none of the kernel's inputs; the median
    # of 5 repetitions, HIP events on the launch stream
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)

    def isolated(fn, reps=5):
        ts = []
        for _ in range(reps):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    a_bytes = wl.n_tokens * wl.d_in * esz + wl.d_in * 8
    iso_ms = {
        "act_stats+finalize": isolated(lambda: B.awq_act_stats(x, act, ws_act)),
        "quant_delta": isolated(lambda: B.awq_quant_delta(w_parts, cand[:cpp], wl.group_size, delta[:cpp])),
        "quantize_pack": isolated(lambda: B.awq_quantize_pack(w_parts, best, wl.group_size, pack_out)),
    }
    if gram:  # the step's own delta: float16 with the per-candidate scales (max |W| pass included)
        iso_ms["quant_delta_f16"] = isolated(
            lambda: B.awq_quant_delta_f16(w_parts, cand[:cpp], wl.group_size, delta16[:cpp], dexp))
    # Around the search: the fold of best_scales into the source operator of this layer (the
    # norm weight for a fused norm-linear set, the up_proj rows for a down_proj search), and the
    # float16 / packed-zero export of the pack's output
    src_rows = wl.d_in
    src_cols = 1 if wl.parts else (4096 if wl.d_in == 11008 else 8192 if wl.d_in == 28672 else wl.d_in)
    src_kind = "norm weight" if src_cols == 1 else f"up_proj [{src_rows}, {src_cols}]"
    gen = torch.Generator(device=dev).manual_seed(wl.config_id)
    fold_src = (torch.randn((src_rows, src_cols), generator=gen, device=dev, dtype=torch.float32) * 0.02).to(x.dtype)
    fold_dst = torch.empty_like(fold_src)
    iso_ms["fold_scales"] = isolated(lambda: B.awq_fold_scales(fold_src, best, dst=fold_dst))
    exp_out = {"counts": torch.zeros(2, dtype=torch.int32, device=dev)}
    exp_out.update(B.awq_export_fp16(pack_out["qscales"], pack_out["zeros"], out=exp_out))
    iso_ms["export_fp16"] = isolated(lambda: B.awq_export_fp16(pack_out["qscales"], pack_out["zeros"], out=exp_out))
    # Grid and quantizer variants at this workload: the per-row quantizers' delta step (same
    # algorithmic bytes as the group quantizer's), the |W| column mean of the duo formula, and the
    # whole search with each page's pairing of formula, grid and quantizer
    wm = B.awq_weight_mean(w_parts)
    var_ms = {
        "weight_mean": isolated(lambda: B.awq_weight_mean(w_parts, wm)),
        "quant_delta_int4_row": isolated(lambda: B.awq_quant_delta_ex(w_parts, cand[:cpp], B.AWQ_QUANT_INT4_ROW,
                                                                      delta[:cpp])),
        "quant_delta_int8_row_sym": isolated(lambda: B.awq_quant_delta_ex(w_parts, cand[:cpp],
                                                                          B.AWQ_QUANT_INT8_ROW_SYM, delta[:cpp])),
    }
    # The export's consumer: the W4A16 product on this layer's deployment form, at decode token
    # counts (weight-streaming, HBM-bound) and at the calibration token count (matrix-core-bound)
    w4_ex = B.awq_export_fp16(pack_out["qscales"], pack_out["zeros"])
    w4_ms, w4_rate = {}, {}
    w4_bytes_w = wl.d_out * wl.d_in // 2 + wl.d_out * G * 2 + wl.d_out * ((G + 1) // 2)
    if wl.dtype == "bf16":
        for m in (1, 16, 32, wl.n_tokens):
            ym = torch.empty((m, wl.d_out), dtype=x.dtype, device=dev)
            t_ms = isolated(lambda: B.awq_w4a16_gemm(x[:m], pack_out["codes"], w4_ex["steps_f16"],
                                                     w4_ex["zeros_u4"], out_dtype=x.dtype, y=ym))
            w4_ms[f"tokens_{m}"] = t_ms
            if m <= 32:
                w4_rate[f"tokens_{m}"] = {"gbps": (w4_bytes_w + m * wl.d_in * 2 + m * wl.d_out * 2) / (t_ms * 1e-3) / 1e9}
            else:
                w4_rate[f"tokens_{m}"] = {"tflops": 2.0 * m * wl.d_in * wl.d_out / (t_ms * 1e-3) / 1e12}
        # context: the library's dense bf16 GEMM on the same shape (weights already 16-bit)
        wd = w.view(wl.d_out, wl.d_in)
        yd = torch.empty((wl.n_tokens, wl.d_out), dtype=x.dtype, device=dev)
        w4_ms["dense_bf16_torch_matmul"] = isolated(lambda: torch.matmul(x, wd.t(), out=yd))
        del yd
    # The block-level objective: the gate/up search scored at the gated MLP's output, at the LLaMA-7B
    # MLP widths (4096 -> 11008 -> 4096) on this layer's 4096-wide activations, random-init weights
    blk = {}
    if wl.dtype == "bf16" and wl.d_in == 4096:
        d_ff, d_model = 11008, 4096
        gen_b = torch.Generator(device=dev).manual_seed(7)
        wg_b = (torch.randn((d_ff, 4096), generator=gen_b, device=dev) * 0.02).to(torch.bfloat16)
        wu_b = (torch.randn((d_ff, 4096), generator=gen_b, device=dev) * 0.02).to(torch.bfloat16)
        wd_b = (torch.randn((d_model, d_ff), generator=gen_b, device=dev) * 0.015).to(torch.bfloat16)
        cpp_b = min(cpp, wl.n_grid)
        ws_b = torch.empty(B.awq_search_workspace_bytes_mlp(wl.n_tokens, 4096, d_ff, d_model, wl.n_grid, cpp_b),
                           dtype=torch.uint8, device=dev)
        out_b = {}
        run_b = lambda: B.awq_search_scales_mlp(x, wg_b, wu_b, wd_b, act, B.AWQ_ACT_SILU, wl.n_grid, cpp_b,
                                                workspace=ws_b, out=out_b)
        out_b.update(run_b())
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run_b()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        g_ref, u_ref = B.awq_mlp_hidden_ref(x, wg_b, wu_b)
        # a candidate pass reads two distinct delta matrices (gate and up), as in the search
        dwg = (torch.randn((d_ff, 4096), generator=gen_b, device=dev) * 0.001).to(torch.bfloat16)
        dwu = (torch.randn((d_ff, 4096), generator=gen_b, device=dev) * 0.001).to(torch.bfloat16)
        dh_b = torch.empty((wl.n_tokens, d_ff), dtype=torch.bfloat16, device=dev)
        t_ref = isolated(lambda: B.awq_mlp_hidden_ref(x, wg_b, wu_b, g_ref, u_ref))
        t_dh = isolated(lambda: B.awq_mlp_hidden_delta(x, dwg, dwu, g_ref, u_ref, B.AWQ_ACT_SILU, dh_b))
        sse_b = torch.empty((1, B.awq_error_tiles(wl.n_tokens, d_model)), dtype=torch.float64, device=dev)
        t_dn = isolated(lambda: B.awq_error_sse(dh_b, wd_b.view(1, d_model, d_ff), sse_b))
        f_gu = 2.0 * 2 * wl.n_tokens * 4096 * d_ff
        f_dn = 2.0 * wl.n_tokens * d_ff * d_model
        blk = {"shape": {"d_in": 4096, "d_ff": d_ff, "d_model": d_model, "n_tokens": wl.n_tokens,
                         "n_grid": wl.n_grid},
               "search_ms": float(np.median(ts)), "candidates_per_s": wl.n_grid / (float(np.median(ts)) * 1e-3),
               "k_star": int(out_b["best_info"][0].item()),
               "ms": {"mlp_hidden_ref": t_ref, "mlp_hidden_delta": t_dh, "error_sse_down": t_dn},
               "tflops": {"mlp_hidden_ref": f_gu / (t_ref * 1e-3) / 1e12, "mlp_hidden_delta": f_gu / (t_dh * 1e-3) / 1e12,
                          "error_sse_down": f_dn / (t_dn * 1e-3) / 1e12}}
        del ws_b, g_ref, u_ref, dh_b, wg_b, wu_b, wd_b, dwg, dwu
    del flush
    var_gbps = {"weight_mean": (wl.d_out * wl.d_in * esz + wl.d_in * 8) / (var_ms["weight_mean"] * 1e-3) / 1e9,
                "quant_delta_int4_row": q_bytes / (var_ms["quant_delta_int4_row"] * 1e-3) / 1e9,
                "quant_delta_int8_row_sym": q_bytes / (var_ms["quant_delta_int8_row_sym"] * 1e-3) / 1e9}
    ws_s = torch.empty(B.awq_search_workspace_bytes(dt, wl.n_tokens, wl.d_in, wl.d_out, 128, 20,
                                                    min(cpp, 20)) if args.variant_searches else 0,
                       dtype=torch.uint8, device=dev)
    pairings = {"duo/linspace20/int4_row": (B.AWQ_FORMULA_DUO, [k / 19 for k in range(20)], B.AWQ_QUANT_INT4_ROW),
                "rms/tenths/int4_group": (B.AWQ_FORMULA_RMS, [k / 10 for k in range(11)], B.AWQ_QUANT_INT4_GROUP),
                "msmodelslim/ms20/int8_row_sym": (B.AWQ_FORMULA_MSMODELSLIM, [k / 20 for k in range(20)],
                                                  B.AWQ_QUANT_INT8_ROW_SYM)}
    search_ms = {}
    for name, (formula, ratios, quantizer) in (pairings.items() if args.variant_searches else ()):
        c = min(cpp, len(ratios))
        fn = lambda: B.awq_search_scales_ex(x, w_parts, act, ratios, formula, quantizer, w_mean=wm,
                                            cand_per_pass=c, workspace=ws_s)
        fn()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        search_ms[name] = {"ms": float(np.median(ts)), "candidates": len(ratios),
                           "candidates_per_s": len(ratios) / (float(np.median(ts)) * 1e-3)}
    del ws_s
    f_bytes = 2 * src_rows * src_cols * esz + src_rows * 8
    e_bytes = wl.d_out * G * (4 + 4 + 2) + wl.d_out * ((G + 1) // 2)
    iso_gbps = {"act_stats+finalize": a_bytes / (iso_ms["act_stats+finalize"] * 1e-3) / 1e9,
                "quant_delta": q_bytes / (iso_ms["quant_delta"] * 1e-3) / 1e9,
                "quantize_pack": p_bytes / (iso_ms["quantize_pack"] * 1e-3) / 1e9,
                "fold_scales": f_bytes / (iso_ms["fold_scales"] * 1e-3) / 1e9,
                "export_fp16": e_bytes / (iso_ms["export_fp16"] * 1e-3) / 1e9}
    if gram:
        iso_gbps["quant_delta_f16"] = q_bytes / (iso_ms["quant_delta_f16"] * 1e-3) / 1e9

    out = {
        "metric": METRIC,
        "value": wl.n_grid / (ms_step * 1e-3),
        "unit": "candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {"workload": wl.name, "n_tokens": wl.n_tokens, "d_in": wl.d_in, "d_out": wl.d_out,
                   "parts": parts, "group_size": wl.group_size, "n_grid": wl.n_grid, "cand_per_pass": cpp},
        "loss_form": "gram" if gram else "direct",
        "roofline": {"bound": "mfma",
                     "kernel": "error_sse_kernel<unsigned short, 2> (quadratic form, float16)" if gram
                     else "error_sse_kernel<unsigned short, 0>",
                     "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": measured_traffic(wl.name, gram),
                     "launch_ms": gemm_ms, "flops_per_launch": flops_launch},
        "search_ms": ms_step,
        "error_gemm_tflops": achieved,
        "kernels_ms": {"act_stats+candidate_scales": act_ms, "quant_delta": quant_ms, "error_sse": gemm_ms,
                       "quantize_pack": pack_ms},
        "gram": None if not gram else {
            "ms": gram_ms, "note": "X^T, G = X^T X (the 256 x 256 tiles on and above the diagonal, float32), its "
                                   "scale and float16 form; TFLOP/s of those tiles' products over the whole step",
            "gram_gemm_tflops": 2.0 * n_pad * 256 * 256 * (tg * (tg + 1) // 2) / (gram_ms * 1e-3) / 1e12},
        "hbm_kernels": {"note": "each kernel alone, memory-side cache flushed before every repetition, median of 5; "
                                "algorithmic bytes / time against 8000 GB/s",
                        "fold_source": src_kind, "ms": iso_ms, "gbps": iso_gbps,
                        "frac_of_peak": {k: v / PEAK_HBM_GBPS for k, v in iso_gbps.items()}},
        "variants": {"note": "per-row quantizers and |W| mean alone (cache flushed, median of 5, algorithmic bytes "
                             "/ time); searches with each page's formula/grid/quantizer (median of 3)",
                     "ms": var_ms, "gbps": var_gbps,
                     "frac_of_peak": {k: v / PEAK_HBM_GBPS for k, v in var_gbps.items()},
                     "search": search_ms},
        "w4a16": {"note": "awq_w4a16_gemm on this layer's float16 export, cache flushed, median of 5; decode token "
                           "counts in GB/s of codes + steps + zeros + X + Y against 8000, the calibration token count in "
                           "TFLOP/s against 2500; dense_bf16_torch_matmul is the library bf16 GEMM of the same shape",
                  "ms": w4_ms, "rate": w4_rate},
        "block_mlp": dict(blk, note="gate/up search scored at the gated MLP's output (LLaMA-7B MLP widths, "
                                    "random-init weights): whole search median of 3; per-launch kernels cache "
                                    "flushed, median of 5, TFLOP/s against 2500"),
        "best_k": info_h[0],
        "graph": graph_rep,
    }
    if not args.no_cpu_baseline:
        _log("cpu baseline (oracle on a row sample)")
        out["cpu_baseline"] = cpu_baseline(wl, x_np, w_np, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
