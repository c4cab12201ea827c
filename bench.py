#!/usr/bin/env python3
"""Benchmark of the GPTQ layer solver on one MI355X.

One step = one whole layer through the three C-ABI calls with the inputs
already resident in HBM: H := 0; H += 2 X^T X over all calibration rows;
damping + U; the lazy-batch loop with the output error.  The timed steps
replay that step captured once in a HIP graph (about 110 dependent launches
per step); every replay's outputs are first checked bitwise against an eager
step's, and the per-stage times come from an eager pass with HIP events
between the stages (--eager times the eager steps instead).  Workload: a
4096 x 4096 fp16 attention projection, X = 262144 x 4096 fp16 (rank-64
covariance, 1% outlier channels at 20x), 4-bit asymmetric grid, group 128,
block 128, 1% damping.  With --act-order the same layer is quantized with the
columns in descending-diagonal order (order from the GPU's H, then the
reordered factor and loop), as a separate measurement.

Prints one JSON line.  The metric is seconds per layer (lower is better), with
per-stage TFLOP/s and three roofline entries: the dominant kernel (the Hessian
syrk, against the fp16 matrix peak) and, from a separate pass of the same run
whose launches are bracketed one by one with HIP events, the in-block panel
(algorithmic bytes against the HBM peak) and the out-of-block products (flop
against the fp32 matrix peak).  The CPU baseline is the fp64 oracle run on the
whole layer (every calibration row, every weight row) on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_F16_MFMA_TFLOPS = 2516.6     # MI355X dense fp16 matrix peak
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_F64_TFLOPS = 78.6
PEAK_HBM_GBS = 8000.0
METRIC = "GPTQ s/layer + Hessian/trailing-GEMM TFLOPS (4096×4096, 4-bit g128) at 1 GPU"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time the layer steps as launched one by one instead of replaying the "
                         "step captured once in a HIP graph")
    ap.add_argument("--act-order", action="store_true",
                    help="quantize the columns in act-order (descending Hessian diagonal)")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "syrk_f16_attn4096_traffic.json"),
                    help="rocprofv3 --pmc derived HBM bytes of the dominant kernel (JSON), if any")
    ap.add_argument("--packed-gemv", action="store_true",
                    help="time the dequantizing product Y = X What^T from packed codes on a "
                         "49152 x 12288 3-bit group-128 layer (one token) instead of the solver")
    ap.add_argument("--gemv-m", type=int, default=1, help="rows of X for --packed-gemv (1..8)")
    ap.add_argument("--gemv-iters", type=int, default=200, help="products per step for --packed-gemv")
    ap.add_argument("--pipeline", action="store_true",
                    help="time the whole-model procedure on a 6-block d=384 GPT-style stack (24 layers, "
                         "163840 calibration tokens) instead of the single layer")
    ap.add_argument("--independent", action="store_true",
                    help="with --pipeline: every block sees the unquantized model's activations")
    ap.add_argument("--gptq2d", action="store_true",
                    help="time two-sided adaptive rounding of a 4096 x 4096 fp16 matrix instead of the layer")
    ap.add_argument("--loop-ffn", action="store_true",
                    help="time the lazy-batch loop alone at the 175B-class FFN shape (49152 x 12288)")
    ap.add_argument("--configs", action="store_true",
                    help="seconds per layer for every layer shape of the five configurations")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="run two plain device-to-device copies of BYTES bytes and exit (the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _traffic(path):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if any."""
    try:
        with open(path) as f:
            return json.load(f).get("hbm_bytes_per_launch")
    except Exception:
        return None


def loop_rooflines(G, run_once, reps, a8_flop, tag):
    """A separate pass over the quantization loop with every panel launch and every
    out-of-block product launch bracketed by HIP events on the library's stream:
    the panel's algorithmic bytes per second against the HBM peak, the products'
    flop per second against the fp32 matrix peak."""
    G.gptq_launch_timing(True)
    try:
        for _ in range(reps):
            run_once()
    finally:
        G.gptq_launch_timing(False)
    p_ms, p_n, p_bytes = G.gptq_launch_timing_read(G.TIMING_PANEL)
    g_ms, g_n, g_flop = G.gptq_launch_timing_read(G.TIMING_PRODUCT)
    panel_gbs = p_bytes / (p_ms / 1e3) / 1e9
    gemm_tfs = g_flop / (g_ms / 1e3) / 1e12
    log(f"bench: panel {p_n // reps} launches/layer, {p_ms / p_n * 1e3:.2f} us each, {panel_gbs:.1f} GB/s; "
        f"out-of-block product {g_n // reps} launches/layer, {g_ms / g_n * 1e3:.2f} us each, "
        f"{gemm_tfs:.2f} TFLOP/s")
    roof_panel = {"bound": "hbm", "kernel": "in-block panel launches (a7)",
                  "achieved": round(panel_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                  "frac": round(panel_gbs / PEAK_HBM_GBS, 4),
                  "bytes_per_launch": round(p_bytes / p_n), "us_per_launch": round(p_ms / p_n * 1e3, 3),
                  "launches_per_layer": p_n // reps,
                  "traffic": _traffic(os.path.join(ROOT, "profiles", f"panel_{tag}_traffic.json"))}
    roof_gemm = {"bound": "mfma", "kernel": "out-of-block product launches (trail_dma_kernel, a8)",
                 "achieved": round(gemm_tfs, 2), "peak": PEAK_F32_MFMA_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(gemm_tfs / PEAK_F32_MFMA_TFLOPS, 4),
                 "flop_per_layer": g_flop / reps, "a8_flop_per_layer": float(a8_flop),
                 "us_per_launch": round(g_ms / g_n * 1e3, 3), "launches_per_layer": g_n // reps,
                 "traffic": _traffic(os.path.join(ROOT, "profiles", f"trail_{tag}_traffic.json"))}
    return roof_panel, roof_gemm


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(spec, W, X_chunks, act_order=False):
    """The fp64 oracle on the whole layer: H over every calibration row, the
    sketch route's factor, the loop over every weight row, the error."""
    import numpy as np
    import oracle as O
    t0 = time.perf_counter()
    H = O.hessian(X_chunks)
    t_h = time.perf_counter() - t0
    t0 = time.perf_counter()
    if act_order:
        perm = O.act_order_perm(H)
        Hl, lam = O.damp(H[np.ix_(perm, perm)], spec.percdamp)
    else:
        Hl, lam = O.damp(H, spec.percdamp)
    U = O.inv_hessian_factor(Hl)
    t_f = time.perf_counter() - t0
    t0 = time.perf_counter()
    if act_order:
        res = O.gptq_quantize_act_order(W.astype(np.float64), U, perm, spec.bits, spec.group_size,
                                        spec.block_size)
    else:
        res = O.gptq_quantize(W.astype(np.float64), U, spec.bits, spec.group_size, spec.block_size)
    err = O.output_error(W, res.w_hat, H)
    t_q = time.perf_counter() - t0
    total = t_h + t_f + t_q
    return {"value": total, "unit": "s/layer", "cores": int(_blas_threads()), "kind": "oracle",
            "sample": (f"the whole layer, unsampled: H over all {spec.n_rows} calibration rows, the "
                       f"{spec.d_col}x{spec.d_col} fp64 factor, the loop over all {spec.d_row} weight "
                       f"rows and the output error"),
            "stages_s": {"hessian": t_h, "factor": t_f, "loop_and_error": t_q}, "err": err}


GEMV_TRAFFIC = os.path.join(ROOT, "profiles", "dequant_gemv_fc49152_traffic.json")


def packed_gemv_cpu_baseline(packed, bits, scales, zeros, group, X, d_col, d_row):
    """The fp64 oracle's product on the sample rows given (the first rows of the
    layer), scaled to all d_row rows."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    rows = packed.shape[0]
    t0 = time.perf_counter()
    O.dequant_matmul(packed, bits, scales, zeros, group, X, d_col)
    t = (time.perf_counter() - t0) * (d_row / rows)
    return {"value": round(t * 1e6, 1), "unit": "us/product", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} of {d_row} weight rows (x{d_row // rows}), scaled to the whole layer"}


def packed_gemv(args):
    """Y = X What^T from packed 3-bit codes (the consumer of the solver's codes) on
    the 175B-class MLP shape.  Four distinct layers are cycled so that the packed
    words (4 x 226 MB) come from HBM rather than the 256 MB last-level cache."""
    import numpy as np
    import torch
    import post_weight_quantization_02_amd as G

    d_row, d_col, bits, group, m = 49152, 12288, 3, 128, args.gemv_m
    nlay = 4
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(20221031)
    words = G.gptq_packed_words_per_row(d_col, bits)
    ng = d_col // group
    layers = []
    for _ in range(nlay):
        codes = torch.randint(0, 1 << bits, (d_row, d_col), dtype=torch.uint8, device=dev, generator=gen)
        packed = G.gptq_pack_codes(codes, bits)
        del codes
        scales = torch.rand(d_row, ng, device=dev, generator=gen) * 0.01 + 1e-3
        zeros = torch.randint(0, 1 << bits, (d_row, ng), dtype=torch.int32, device=dev, generator=gen)
        layers.append((packed, scales, zeros))
    X = torch.randn(m, d_col, device=dev, generator=gen).to(torch.float16)
    Y = torch.empty(m, d_row, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        for i in range(args.gemv_iters):
            p, s, z = layers[i % nlay]
            G.gptq_dequant_matmul(p, bits, s, z, group, X, d_col, Y=Y, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_launch = args.steps * args.gemv_iters
    t_launch = e0.elapsed_time(e1) / 1e3 / n_launch
    # algorithmic bytes of one product: packed words, per-group scale and zero, X once, Y once
    alg = d_row * words * 4 + d_row * ng * 8 + m * d_col * 2 + m * d_row * 4
    ach = alg / t_launch / 1e9
    traffic = None
    if os.path.exists(GEMV_TRAFFIC):
        try:
            with open(GEMV_TRAFFIC) as f:
                tr = json.load(f)
            if tr.get("m") == m:
                traffic = tr.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    # context: the same product with the fp16 weights through torch (hipBLASLt / rocBLAS)
    W16 = torch.randn(d_row, d_col, device=dev, generator=gen).to(torch.float16)
    for _ in range(5):
        torch.matmul(X, W16.t())
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record(stream)
    for _ in range(50):
        torch.matmul(X, W16.t())
    f1.record(stream)
    torch.cuda.synchronize()
    t_f16 = f0.elapsed_time(f1) / 1e3 / 50
    del W16
    # context: a plain device copy of the same packed bytes (read + write)
    src = torch.cat([p.view(-1) for p, _, _ in layers])
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    f0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    f1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 10 / (f0.elapsed_time(f1) / 1e3) / 1e9
    del src, dst

    out = {
        "metric": "dequantizing product Y = X What^T from packed 3-bit codes, us per product",
        "value": round(t_launch * 1e6, 3),
        "unit": "us/product",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32-packed 3-bit codes, f16 X, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": f"fc_49152x12288: W 49152x12288 3-bit asymmetric, group 128, X {m}x12288 fp16, "
                               f"{nlay} layers cycled",
                   "d_row": d_row, "d_col": d_col, "bits": bits, "group_size": group, "m": m,
                   "products_per_step": args.gemv_iters, "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm",
                     "kernel": "gemv1_f16_kernel" if m == 1 else "gemm_mfma_f16_kernel",
                     "achieved": round(ach, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": alg},
        "fp16_weights_torch_matmul_us": round(t_f16 * 1e6, 3),
        "speedup_vs_fp16_weights": round(t_f16 / t_launch, 3),
        "plain_copy_gbs": round(copy_gbs, 1),
    }
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle's product on a bounded sample (CPU)")
        p, s, z = layers[0]
        out["cpu_baseline"] = packed_gemv_cpu_baseline(
            p[:8192].cpu().numpy().view(np.uint32), bits, s[:8192].cpu().numpy(),
            z[:8192].cpu().numpy(), group, X.float().cpu().numpy(), d_col, d_row)
        out["gpu_speedup_vs_cpu_oracle"] = round(out["cpu_baseline"]["value"] / (t_launch * 1e6), 1)
    print(json.dumps(out), flush=True)


def pipeline_cpu_baseline(spec, act_order):
    """The fp64 oracle's procedure on one block: one calibration batch through the
    forward pass (scaled to 2 passes x all batches x all blocks) and the block's
    four layer solves on that batch's H (scaled to all blocks)."""
    import numpy as np
    import oracle as O
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    MP = O.model_pipeline
    p = {k: v.astype(np.float64) for k, v in wl.gpt_block_params(spec, 0).items()}
    x = wl.gpt_embeddings(spec, 0).astype(np.float64)
    cap = {}
    t0 = time.perf_counter()
    MP.block_forward(p, x, spec.n_head, capture=cap)
    t_fwd = time.perf_counter() - t0
    t0 = time.perf_counter()
    for name in MP.LINEARS:
        H = O.hessian(cap[name]) * spec.n_batch
        if act_order:
            perm = O.act_order_perm(H)
            Hl, _ = O.damp(H[np.ix_(perm, perm)], spec.percdamp)
            O.gptq_quantize_act_order(p[name + "_w"], O.inv_hessian_factor(Hl), perm, spec.bits, spec.group_size,
                                      spec.block_size)
        else:
            Hl, _ = O.damp(H, spec.percdamp)
            O.gptq_quantize(p[name + "_w"], O.inv_hessian_factor(Hl), spec.bits, spec.group_size, spec.block_size)
    t_solve = time.perf_counter() - t0
    total = t_fwd * 2 * spec.n_batch * spec.n_block + t_solve * spec.n_block
    return {"value": round(total, 2), "unit": "s/model", "cores": int(threads), "kind": "oracle",
            "sample": (f"block 0: one batch of {spec.n_seq}x{spec.seq} tokens through the fp64 forward "
                       f"(x{2 * spec.n_batch * spec.n_block}: two passes, {spec.n_batch} batches, "
                       f"{spec.n_block} blocks) and its 4 layer solves (x{spec.n_block}); scaled to the model"),
            "stages_s": {"forward_per_batch_block": t_fwd, "solves_per_block": t_solve}}


def pipeline_bench(args):
    """The whole-model procedure: 6 GPT-style blocks (d 384, 6 heads), 10 calibration
    batches of 64 x 256 tokens, 4-bit per-row grid, block 128, 1% damping."""
    import torch
    import post_weight_quantization_02_amd as G  # noqa: F401
    from post_weight_quantization_02_amd import pipeline as P
    import workloads as wl
    from workloads import torch_gpt

    spec = wl.GPTSpec()
    dev = torch.device("cuda:0")
    blocks = torch_gpt.build_model(spec, device=dev)
    orig = [{n: m.weight.detach().clone() for n, m in P.linear_layers(b)} for b in blocks]
    xs = [torch.from_numpy(wl.gpt_embeddings(spec, i)).to(dev) for i in range(spec.n_batch)]
    torch.cuda.synchronize()
    sequential = not args.independent

    def restore():
        with torch.no_grad():
            for b, o in zip(blocks, orig):
                for n, m in P.linear_layers(b):
                    m.weight.copy_(o[n])

    def step():
        return P.quantize_model(blocks, xs, spec.bits, spec.group_size, spec.block_size, spec.percdamp,
                                act_order=args.act_order, sequential=sequential)

    for _ in range(args.warmup):
        restore()
        step()
    torch.cuda.synchronize()
    times, errs = [], None
    for _ in range(args.steps):
        restore()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res, _ = step()
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
        errs = {f"h{i}.{n}": float(L.err.item()) for i, r in enumerate(res) for n, L in r.layers.items()}
    per_step = sum(times) / len(times)
    # one forward pass of the unquantized model over all batches, for the stage split
    restore()
    with torch.no_grad():
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for b in blocks:
            ys = [b(x) for x in xs]
        torch.cuda.synchronize()
        t_fwd = time.perf_counter() - t0
    passes = 2 if sequential else 1
    # the quantizer's dominant kernel in this procedure: the fp32 syrk of
    # gptq_hessian_accumulate at the model's shapes (one calibration batch of rows,
    # widths d and 4d), timed with events on the stream it runs on
    rows = spec.n_seq * spec.seq
    t_h = {}
    for width in (spec.d, 4 * spec.d):
        Xh = torch.randn(rows, width, device=dev)
        Hh = torch.zeros(width, width, device=dev)
        for _ in range(3):
            G.gptq_hessian_accumulate(Hh, Xh)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            G.gptq_hessian_accumulate(Hh, Xh)
        e1.record()
        torch.cuda.synchronize()
        t_h[width] = e0.elapsed_time(e1) / 1e3 / 20
    f = lambda w: rows * w * (w + 1)  # noqa: E731  (upper triangle, 2 flop per multiply-add)
    per_batch_block_flops = 3 * f(spec.d) + f(4 * spec.d)
    per_batch_block_time = 3 * t_h[spec.d] + t_h[4 * spec.d]
    ach = per_batch_block_flops / per_batch_block_time / 1e12
    roof = {"bound": "mfma", "kernel": "gptq_hessian_accumulate: syrk_f32_kernel + split reduce (fp32 X)",
            "achieved": round(ach, 2), "peak": PEAK_F32_MFMA_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_F32_MFMA_TFLOPS, 4), "traffic": None,
            "per_call_us": {str(k): round(v * 1e6, 2) for k, v in t_h.items()}}
    out = {
        "metric": "whole-model GPTQ, s per model (6-block d=384 GPT-style stack, 24 layers, 163840 tokens)",
        "value": round(per_step, 5),
        "unit": "s/model",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(per_step * 1e3, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 model forward / f32-mfma syrk / f64 Cholesky / f32 loop",
        "data": "synthetic",
        "config": {"workload": (f"gpt6x384: {spec.n_block} blocks, d {spec.d}, {spec.n_head} heads, "
                                f"{spec.n_batch} batches x {spec.n_seq} seqs x {spec.seq} tokens, "
                                f"{spec.bits}-bit per-row, block {spec.block_size}, 1% damping, "
                                + ("sequential" if sequential else "independent")
                                + (", act-order" if args.act_order else "")),
                   "sequential": sequential, "act_order": bool(args.act_order), "parallelism": "single-gpu"},
        "stages": {"model_forward_all_blocks_ms": round(t_fwd * 1e3, 3), "forward_passes_per_block": passes,
                   "quantizer_and_hooks_ms_estimate": round((per_step - passes * t_fwd) * 1e3, 3)},
        "roofline": roof,
        "layer_errors": errs,
    }
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle's procedure on a bounded sample (CPU)")
        cb = pipeline_cpu_baseline(spec, args.act_order)
        out["cpu_baseline"] = cb
        out["gpu_speedup_vs_cpu_oracle"] = round(cb["value"] / per_step, 1)
    print(json.dumps(out), flush=True)


PEAK_F32_VALU_TFLOPS = 157.3    # 256 CUs x 4 SIMDs x 2.4 GHz x 64 flop per cycle (fp32 vector)


def gptq2d_cpu_baseline(bits):
    """The fp64 oracle's sweep on a 256 x 256 problem of the same recipe, scaled by
    m n (m + n) to 4096 x 4096."""
    import numpy as np
    import oracle as O
    rng = np.random.default_rng(5)
    k = 256
    X = (0.015 * rng.standard_normal((k, k))).astype(np.float16).astype(np.float64)
    Z = rng.standard_normal((4 * k, k))
    Q = 2 * Z.T @ Z
    Z = rng.standard_normal((4 * k, k))
    P = 2 * Z.T @ Z
    UQ = O.inv_hessian_factor(O.damp(Q, 0.01)[0])
    UP = O.inv_hessian_factor(O.damp(P, 0.01)[0])
    t0 = time.perf_counter()
    O.gptq2d.gptq2d(X, UQ, UP, bits)
    t = (time.perf_counter() - t0) * (4096 * 4096 * 8192) / (k * k * 2 * k)
    return {"value": round(t, 1), "unit": "s/matrix", "cores": 1, "kind": "oracle",
            "sample": "the sweep on a 256 x 256 problem of the same recipe, scaled by m n (m + n) to 4096 x 4096"}


def gptq2d_bench(args):
    """Two-sided rounding of a 4096 x 4096 fp16 matrix (the attn_4096 weight recipe)
    with A^T A and B B^T = 2 Z^T Z of two seeded 16384-row low-rank streams, 1%
    damping, 4 bits; the timed call is gptq2d_quantize (the factors are inputs)."""
    import torch
    import post_weight_quantization_02_amd as G
    import workloads as wl

    m = n = 4096
    bits = 4
    dev = torch.device("cuda:0")
    spec = wl.workload_layers(3)[0]
    X = torch.from_numpy(wl.make_weight(spec)).to(dev)
    grams = []
    for layer in (201, 202):
        zs = wl.LayerSpec(3, layer, "side", 8, m, 16384, "f32", "f16", 0.0, 4, 0, x_kind="lowrank")
        Hs = torch.zeros(m, m, device=dev)
        G.gptq_hessian_accumulate(Hs, torch.from_numpy(wl.make_x_chunk(zs, 0)).to(dev))
        grams.append(Hs)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    UQ, _, iq = G.gptq_prepare_hinv(grams[0], 0.01)
    UP, _, ip = G.gptq_prepare_hinv(grams[1], 0.01)
    e1.record()
    torch.cuda.synchronize()
    if int(iq.item()) or int(ip.item()):
        raise SystemExit("side factor failed")
    t_factors = e0.elapsed_time(e1) / 1e3
    codes = torch.empty(m, n, dtype=torch.uint8, device=dev)
    scale = torch.empty(1, device=dev)
    zero = torch.empty(1, dtype=torch.int32, device=dev)
    err = torch.empty(1, dtype=torch.float64, device=dev)
    ws = torch.empty(G.gptq2d_quantize_workspace_size(m, n), dtype=torch.uint8, device=dev)
    for _ in range(args.warmup):
        G.gptq2d_quantize(X, UQ, UP, bits, codes, scale, zero, err, ws)
    torch.cuda.synchronize()
    e0.record()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        G.gptq2d_quantize(X, UQ, UP, bits, codes, scale, zero, err, ws)
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    t = e0.elapsed_time(e1) / 1e3 / args.steps
    flops = m * n * (m + n + 2)          # every entry's dot product and row update, 2 flop per multiply-add
    ach = flops / t / 1e12
    out = {
        "metric": "two-sided adaptive rounding (GPTQ-2D), s per 4096 x 4096 matrix",
        "value": round(t, 6),
        "unit": "s/matrix",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 X, f32 sweep, f64 error sums",
        "data": "synthetic",
        "config": {"workload": "2d_4096: X 4096x4096 fp16 (N(0, 0.015^2)), A^T A and B B^T from two 16384-row "
                               "rank-64 fp16 streams, 1% damping, 4-bit, one grid per matrix",
                   "m": m, "n": n, "bits": bits, "parallelism": "single-gpu"},
        "stages": {"side_factors_ms": round(t_factors * 1e3, 3), "sweep_launches": m // 32 + n // 32 - 1,
                   "err": float(err.item())},
        "roofline": {"bound": "alu", "kernel": "the sweep: fc2d_kernel (corrections and feedback) + tile2d_kernel "
                                               "per 32-tile anti-diagonal",
                     "achieved": round(ach, 3), "peak": PEAK_F32_VALU_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_F32_VALU_TFLOPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle's sweep on a bounded sample (CPU)")
        cb = gptq2d_cpu_baseline(bits)
        out["cpu_baseline"] = cb
        out["gpu_speedup_vs_cpu_oracle"] = round(cb["value"] / t, 1)
    print(json.dumps(out), flush=True)


def loop_ffn_bench(args):
    """The lazy-batch loop alone at the 175B-class FFN shape: W_fc 49152 x 12288 fp16,
    3-bit, group 128, B = 128.  U comes from H = 2 X^T X of the first 16384-row
    chunk of the layer's calibration stream with 1% damping (the factor at this d is
    timed separately as a stage); the timed call is gptq_quantize_layer."""
    import torch
    import post_weight_quantization_02_amd as G
    import workloads as wl

    spec = wl.workload_layers(5)[0]
    dr, d = spec.d_row, spec.d_col
    dev = torch.device("cuda:0")
    W = torch.from_numpy(wl.make_weight(spec)).to(dev)
    H = torch.zeros(d, d, device=dev)
    G.gptq_hessian_accumulate(H, torch.from_numpy(wl.make_x_chunk(spec, 0)).to(dev))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    U, lam, info = G.gptq_prepare_hinv(H, spec.percdamp)
    e1.record()
    torch.cuda.synchronize()
    if int(info.item()) != 0:
        raise SystemExit(f"factor failed: info={int(info.item())}")
    t_factor = e0.elapsed_time(e1) / 1e3
    ng = d // spec.group_size
    codes = torch.empty(dr, d, dtype=torch.uint8, device=dev)
    scales = torch.empty(dr, ng, device=dev)
    zeros = torch.empty(dr, ng, dtype=torch.int32, device=dev)
    err = torch.empty(1, dtype=torch.float64, device=dev)
    ws = torch.empty(G.gptq_quantize_layer_workspace_size(dr, d, spec.block_size), dtype=torch.uint8,
                     device=dev)

    def step():
        G.gptq_quantize_layer(W, U, lam, spec.bits, spec.group_size, spec.block_size, codes, scales, zeros,
                              err, ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0.record()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    t = e0.elapsed_time(e1) / 1e3 / args.steps
    flops_gemm = dr * d * (d - spec.block_size)     # sum over blocks of 2 * d_row * B * (d - i2)
    ach = flops_gemm / t / 1e12
    log(f"bench: lazy-batch loop {t * 1e3:.2f} ms at {dr}x{d}; factor {t_factor * 1e3:.2f} ms")
    roof_panel, roof_gemm = loop_rooflines(G, step, 1, flops_gemm, "ffn49152")
    out = {
        "metric": "lazy-batch loop s/layer (175B-class FFN W_fc 49152x12288, 3-bit g128)",
        "value": round(t, 6),
        "unit": "s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 loop (fp32 MFMA out-of-block correction)",
        "data": "synthetic",
        "config": {"workload": "w_fc: W 49152x12288 fp16 N(0, 0.01^2); H from one 16384-row chunk of the "
                               "k^-1 power-law stream, 1% damping; 3-bit asymmetric, group 128, block 128",
                   "d_row": dr, "d_col": d, "bits": spec.bits, "group_size": spec.group_size,
                   "block_size": spec.block_size, "parallelism": "single-gpu"},
        "stages": {"factor_ms": round(t_factor * 1e3, 3), "err": float(err.item()),
                   "trailing_gemm_tflop": round(flops_gemm / 1e12, 3)},
        "roofline": roof_gemm,
        "roofline_panel": roof_panel,
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def configs_bench(args):
    """Seconds per layer for every layer of the five configurations, at their full
    weight shapes and calibration row counts, through the three library calls on
    resident inputs.  Timing-only inputs: X and W are seeded Gaussian tensors of the
    configurations' shapes and dtypes drawn on the GPU (the host cannot synthesise
    the 25.8 GB power-law stream of the widest layer in a benchmark's time); the
    recipe inputs are checked for parity at these shapes by the GPU tests."""
    import torch
    import post_weight_quantization_02_amd as G
    import workloads as wl

    dev = torch.device("cuda:0")
    out = {}
    for cfg in (1, 2, 3, 4, 5):
        layers = wl.workload_layers(cfg)
        if cfg == 2:
            layers = layers[:4]          # the six blocks repeat the same four shapes
        for spec in layers:
            gen = torch.Generator(device=dev)
            gen.manual_seed(1000 * cfg + spec.layer)
            xdt = torch.float16 if spec.x_dtype == "f16" else torch.float32
            wdt = torch.float16 if spec.w_dtype == "f16" else torch.float32
            X = torch.randn(spec.n_rows, spec.d_col, device=dev, generator=gen).to(xdt)
            W = (spec.w_std * torch.randn(spec.d_row, spec.d_col, device=dev, generator=gen)).to(wdt)
            d, dr = spec.d_col, spec.d_row
            H = torch.zeros(d, d, device=dev)
            ws_h = torch.empty(G.gptq_hessian_accumulate_workspace_size(d, spec.n_rows, G.GPTQ_F16 if spec.x_dtype == "f16" else G.GPTQ_F32),
                               dtype=torch.uint8, device=dev)
            ws_f = torch.empty(G.gptq_prepare_hinv_workspace_size(d), dtype=torch.uint8, device=dev)
            ws_q = torch.empty(G.gptq_quantize_layer_workspace_size(dr, d, spec.block_size), dtype=torch.uint8,
                               device=dev)
            U = torch.empty(d, d, device=dev)
            lam = torch.empty(1, device=dev)
            info = torch.empty(1, dtype=torch.int32, device=dev)
            ng = -(-d // spec.group_size) if spec.group_size else 1
            codes = torch.empty(dr, d, dtype=torch.uint8, device=dev)
            scales = torch.empty(dr, ng, device=dev)
            zeros = torch.empty(dr, ng, dtype=torch.int32, device=dev)
            err = torch.empty(1, dtype=torch.float64, device=dev)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]

            def step(rec):
                H.zero_()
                if rec:
                    ev[0].record()
                G.gptq_hessian_accumulate(H, X, ws=ws_h)
                if rec:
                    ev[1].record()
                G.gptq_prepare_hinv(H, spec.percdamp, U, lam, info, ws=ws_f)
                if rec:
                    ev[2].record()
                G.gptq_quantize_layer(W, U, lam, spec.bits, spec.group_size, spec.block_size, codes, scales,
                                      zeros, err, ws=ws_q)
                if rec:
                    ev[3].record()

            step(False)
            torch.cuda.synchronize()
            reps = max(1, min(args.steps, 3))
            st = [0.0, 0.0, 0.0]
            for _ in range(reps):
                step(True)
                torch.cuda.synchronize()
                for k in range(3):
                    st[k] += ev[k].elapsed_time(ev[k + 1]) / 1e3 / reps
            if int(info.item()) != 0:
                raise SystemExit(f"{spec.name}: factor failed (info={int(info.item())})")
            key = f"config{cfg}:{spec.name}"
            out[key] = {"d_row": dr, "d_col": d, "n_rows": spec.n_rows, "bits": spec.bits,
                        "group_size": spec.group_size, "s_per_layer": round(sum(st), 6),
                        "hessian_ms": round(st[0] * 1e3, 3), "factor_ms": round(st[1] * 1e3, 3),
                        "quantize_ms": round(st[2] * 1e3, 3)}
            log(f"bench: {key} {sum(st) * 1e3:.2f} ms (H {st[0] * 1e3:.2f}, factor {st[1] * 1e3:.2f}, "
                f"loop {st[2] * 1e3:.2f})")
            del X, W, H, ws_h, ws_f, ws_q, U, codes, scales, zeros
            torch.cuda.empty_cache()
    print(json.dumps({"metric": "GPTQ s/layer per configuration (timing-only Gaussian inputs of the "
                                "configurations' shapes, drawn on the GPU)",
                      "unit": "s/layer", "n_gpus": 1, "higher_is_better": False, "data": "synthetic",
                      "layers": out}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print("bench.py: this solver runs on one GPU; multi-GPU runs are not supported "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copied {args.copy_calibration} bytes twice")
        return

    if args.packed_gemv:
        packed_gemv(args)
        return
    if args.pipeline:
        pipeline_bench(args)
        return
    if args.gptq2d:
        gptq2d_bench(args)
        return
    if args.loop_ffn:
        loop_ffn_bench(args)
        return
    if args.configs:
        configs_bench(args)
        return

    import post_weight_quantization_02_amd as G
    import workloads as wl

    spec = wl.workload_layers(3)[0]
    dev = torch.device("cuda:0")
    log(f"bench: generating {spec.name} W {spec.d_row}x{spec.d_col}, X {spec.n_rows}x{spec.d_col} fp16")
    t0 = time.perf_counter()
    W = wl.make_weight(spec)
    Xd = torch.empty(spec.n_rows, spec.d_col, dtype=torch.float16, device=dev)
    x_host = []                    # the same bytes, kept for the CPU oracle's run
    for c in range(wl.n_chunks(spec)):
        xc = wl.make_x_chunk(spec, c)
        if not args.no_cpu_baseline:
            x_host.append(xc)
        Xd[c * wl.CHUNK_ROWS:(c + 1) * wl.CHUNK_ROWS].copy_(torch.from_numpy(xc))
    Wd = torch.from_numpy(W).to(dev)
    torch.cuda.synchronize()
    log(f"bench: inputs resident in {time.perf_counter() - t0:.1f}s")

    d, n, dr = spec.d_col, spec.n_rows, spec.d_row
    ng = d // spec.group_size
    H = torch.zeros(d, d, dtype=torch.float32, device=dev)
    U = torch.empty(d, d, dtype=torch.float32, device=dev)
    lam = torch.empty(1, dtype=torch.float32, device=dev)
    info = torch.empty(1, dtype=torch.int32, device=dev)
    codes = torch.empty(dr, d, dtype=torch.uint8, device=dev)
    scales = torch.empty(dr, ng, dtype=torch.float32, device=dev)
    zeros = torch.empty(dr, ng, dtype=torch.int32, device=dev)
    err = torch.empty(1, dtype=torch.float64, device=dev)
    perm = torch.empty(d, dtype=torch.int32, device=dev)
    g_idx = torch.empty(d, dtype=torch.int32, device=dev)
    ws_h = torch.empty(G.gptq_hessian_accumulate_workspace_size(d, n, G.GPTQ_F16), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(G.gptq_prepare_hinv_workspace_size(d), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(G.gptq_quantize_layer_workspace_size(dr, d, spec.block_size), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        # the caller's current stream: the default one, or the capture stream
        stream = torch.cuda.current_stream()
        H.zero_()
        if ev:
            ev[0].record(stream)
        G.gptq_hessian_accumulate(H, Xd, ws=ws_h, stream=stream)
        if ev:
            ev[1].record(stream)
        if args.act_order:
            G.gptq_act_order_perm(H, perm, stream=stream)
            G.gptq_prepare_hinv_perm(H, perm, spec.percdamp, U, lam, info, ws=ws_f, stream=stream)
        else:
            G.gptq_prepare_hinv(H, spec.percdamp, U, lam, info, ws=ws_f, stream=stream)
        if ev:
            ev[2].record(stream)
        if args.act_order:
            G.gptq_quantize_layer_perm(Wd, U, lam, perm, spec.bits, spec.group_size, spec.block_size,
                                       codes, scales, zeros, g_idx, err, ws=ws_q, stream=stream)
        else:
            G.gptq_quantize_layer(Wd, U, lam, spec.bits, spec.group_size, spec.block_size, codes,
                                  scales, zeros, err, ws=ws_q, stream=stream)
        if ev:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(info.item()) != 0:
        raise SystemExit(f"factor failed: info={int(info.item())}")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3])]
                   for e in evs]) / 1e3   # seconds: hessian, factor, quantize
    per_step = wall / args.steps
    timing = "eager launches"
    if not args.eager:
        # the same step captured once and replayed; each replay's outputs must
        # equal the eager step's bitwise before the replays are timed
        ref = [t.clone() for t in (H, U, lam, codes, scales, zeros, err)]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        for r in range(2):
            graph.replay()
            torch.cuda.synchronize()
            got = (H, U, lam, codes, scales, zeros, err)
            if not all(torch.equal(a, b) for a, b in zip(ref, got)):
                raise SystemExit(f"graph replay {r} differs from the eager step")
        t0 = time.perf_counter()
        for k in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_step = (time.perf_counter() - t0) / args.steps
        log(f"bench: eager {per_step * 1e3:.3f} ms per step, graph replay {graph_step * 1e3:.3f} ms")
        per_step = graph_step
        timing = "HIP graph replay of the whole step (captured once, replays checked bitwise against an eager step)"
        del graph
    t_h, t_f, t_q = (float(np.mean(st[:, i])) for i in range(3))
    flops_h = n * d * (d + 1)                       # upper triangle of X^T X, 2 flop per MAC
    flops_f = 2.0 * d ** 3 / 3.0                    # Cholesky d^3/3 + triangular inverse d^3/3
    flops_gemm = dr * d * (d - spec.block_size)     # sum over blocks of 2 * d_row * B * (d - i2)
    log(f"bench: stages ms hessian {t_h * 1e3:.3f} factor {t_f * 1e3:.3f} quantize {t_q * 1e3:.3f}; "
        f"wall/step {per_step * 1e3:.3f} ms; err {float(err.item()):.6g}")

    def quantize_once():
        if args.act_order:
            G.gptq_quantize_layer_perm(Wd, U, lam, perm, spec.bits, spec.group_size, spec.block_size,
                                       codes, scales, zeros, g_idx, err, ws=ws_q, stream=stream)
        else:
            G.gptq_quantize_layer(Wd, U, lam, spec.bits, spec.group_size, spec.block_size, codes,
                                  scales, zeros, err, ws=ws_q, stream=stream)

    roof_panel, roof_gemm = loop_rooflines(G, quantize_once, 3, flops_gemm, "attn4096")

    traffic = None
    if args.traffic and os.path.exists(args.traffic):
        try:
            with open(args.traffic) as f:
                tr = json.load(f)
            traffic = tr.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None
    ach = flops_h / t_h / 1e12
    roof = {"bound": "mfma", "kernel": "gptq_hessian_accumulate: syrk_f16_kernel + fixed-order split reduce",
            "achieved": round(ach, 2), "peak": PEAK_F16_MFMA_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_F16_MFMA_TFLOPS, 4), "traffic": traffic}

    out = {
        "metric": METRIC,
        "value": round(per_step, 6),
        "unit": "s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(per_step * 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-mfma(f32 acc) syrk / f64 Cholesky / f32 loop",
        "data": "synthetic",
        "config": {"workload": "attn_4096: W 4096x4096 fp16, X 262144x4096 fp16 rank-64 + 1% 20x outliers, "
                               "4-bit asymmetric, group 128, block 128, 1% damping"
                               + (", act-order" if args.act_order else ""),
                   "act_order": bool(args.act_order),
                   "d_row": dr, "d_col": d, "n_rows": n, "bits": spec.bits,
                   "group_size": spec.group_size, "block_size": spec.block_size,
                   "parallelism": "single-gpu"},
        "stages": {
            "hessian_ms": round(t_h * 1e3, 4), "hessian_tflops": round(flops_h / t_h / 1e12, 2),
            "factor_ms": round(t_f * 1e3, 4), "factor_tflops": round(flops_f / t_f / 1e12, 3),
            "quantize_ms": round(t_q * 1e3, 4),
            "err": float(err.item()),
        },
        "roofline": roof,
        "roofline_panel": roof_panel,
        "roofline_gemm": roof_gemm,
        "timing": timing + "; stage times from eager steps with HIP events between the stages",
    }
    if not args.no_cpu_baseline:
        log("bench: timing the fp64 oracle on the whole layer (CPU)")
        del Xd
        torch.cuda.empty_cache()
        cb = cpu_baseline(spec, W, x_host, args.act_order)
        cb["err_rel_to_gpu"] = round(abs(cb["err"] - float(err.item())) / cb["err"], 6)
        out["cpu_baseline"] = cb
        out["gpu_speedup_vs_cpu_oracle"] = round(cb["value"] / per_step, 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
