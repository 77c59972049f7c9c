"""Benchmark: milliseconds per layer of GPTQ on one MI355X.

One step = the whole hot path for one linear layer over its calibration
batch: zero H, accumulate H over the token chunks, damping + act-order +
inverse-Hessian factor, the quantization sweep with its trailing updates,
and packing of codes and zero points.  Inputs (X in bf16, a pristine W per
step) are resident in HBM before the timed region starts.

Prints one JSON line.  The timed steps run without instrumentation; the
per-kernel split and the roofline come from the same number of steps run
again with the library's own HIP events recorded around every launch on the
launch stream (gptq_profile_*).

``--w4a16`` instead measures the W4A16 product of stored 4-bit layers
(y = x W^T, int4 codes, fp16 activations) at several batch sizes, one JSON
line per layer shape and batch.  Each call uses the next of several copies of
the prepared layer, more than 1 GiB in all, so the weights come from HBM and
not from the 256 MB last-level cache, as in a model whose layers run in turn.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from post_weight_quantization_layer_amd import inputs as I  # noqa: E402

METRIC = "ms per layer GPTQ (int4 g128, 4096×11008) + MFMA util of SYRK/GEMM"
# TFLOP/s, GB/s.  "f32_bf16x6": fp32 products formed from six bf16 MFMA
# products (three-term operand splits), so a sixth of the bf16 peak.
PEAK = {"bf16_mfma": 2500.0, "f32_mfma": 157.3, "f32_bf16x6": 2500.0 / 6, "hbm": 8000.0}

# HBM bytes per launch of the dominant kernel, from two rocprofv3 --pmc passes
# over this script with --pmc-calibration (FETCH_SIZE, then WRITE_SIZE), each
# counter scaled by what it reads for a plain streaming kernel of known size in
# the same run.  Reported only while the kernel's source is the one measured.
MEASURED_TRAFFIC = {
    "hessian_syrk_bf16": {
        "workload": "down_proj_4096x11008_int4_g128_actorder",
        "chunk_tokens": 32768,
        "source": "post_weight_quantization_layer_amd/csrc/hessian.hip",
        "sha256": "ef336cccea3118549352c296cfd6c8a383fe3b494543b992cd2200868438c271",
        # 10.090 GB fetched + 0.385 GB written at 32768 tokens per launch
        # (profiles/counters_down_proj_4096x11008_int4_g128.md)
        "bytes_per_launch": 10474580272,
    },
}
CALIB_BYTES = 1 << 30     # the streaming kernel reads and writes this many bytes


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def lazy_widths(cfg):
    """Columns per lazy super-block (SB) and per far group (FG) of the sweep:
    SB the largest multiple m B <= 512 of the block B, FG the largest
    multiple of SB <= 2048, each dividing the group size or a multiple of it
    (SB = B when B is not a multiple of 4)."""
    B = cfg.block
    G = 256 if cfg.grid == "q4k" else cfg.group
    ok = lambda w: G % w == 0 or w % G == 0
    sb = B
    if B % 4 == 0:
        sb = next((m * B for m in range(512 // B, 1, -1) if ok(m * B)), B)
    fg = next((c * sb for c in range(2048 // sb, 1, -1) if ok(c * sb)), sb)
    return sb, fg


def kernel_work(cfg, chunk):
    """Algorithmic work of the main kernels.

    hessian_syrk_bf16: d(d+1) n_c flops per launch (upper triangle incl.
    diagonal, 2 per multiply-add).  The sweep's lazy updates past a
    super-block of SB columns: trailing_group applies each super-block's
    errors to the rest of its far group of FG columns (2 r SB (g2 - s2)
    flops), trailing_gemm each far group's errors to every later column
    (2 r FG (d - g2)); "trailing" is the two together.  The updates inside
    a super-block run inside the sweep kernel and are not counted here.
    The trailing products run on bf16 MFMAs with three-term splits of the
    fp32 operands (launches of fewer than 256 128x128 tiles on fp32 MFMAs),
    so their fraction is taken against a sixth of the bf16 peak."""
    d, r = cfg.cols, cfg.rows
    sb, fg = lazy_widths(cfg)
    work = {"hessian_syrk_bf16": ("bf16_mfma", d * (d + 1) * chunk)}
    tg = tf = 0
    for g1 in range(0, d, fg):
        g2 = min(g1 + fg, d)
        tf += 2 * r * (g2 - g1) * (d - g2)
        for s1 in range(g1, g2, sb):
            s2 = min(s1 + sb, g2)
            tg += 2 * r * (s2 - s1) * (g2 - s2)
    work["trailing_group"] = ("f32_bf16x6", tg)
    work["trailing_gemm"] = ("f32_bf16x6", tf)
    work["trailing"] = ("f32_bf16x6", tg + tf)
    return work


def measured_traffic(kernel, workload, chunk_tokens):
    """The counter-measured bytes per launch, for the workload and launch size
    they were measured on, while the kernel's source is unchanged."""
    m = MEASURED_TRAFFIC.get(kernel)
    if not m or m["sha256"] is None:
        return None
    if m["workload"] != workload or m["chunk_tokens"] != chunk_tokens:
        return None
    with open(os.path.join(ROOT, m["source"]), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != m["sha256"]:
            return None
    return m["bytes_per_launch"]


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def _blas() -> tuple[str, int]:
    """BLAS library numpy calls and the threads it uses."""
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        if info:
            p = info[0]
            return f"{p.get('internal_api')} {p.get('version')}", int(p.get("num_threads", 1))
    except Exception:  # pragma: no cover
        pass
    return "unknown", os.cpu_count() or 1


def cpu_baseline(cfg, chunk_tokens):
    """The float64 oracle, as it stands, on a bounded sample of the same
    workload, scaled to milliseconds per layer with the cost model of the
    pages (H linear in tokens, the inverse factor cubic in d, the sweep and
    packing linear in rows).  Each part is timed on a sample large enough
    that its per-call overheads are amortized: one 8192-token chunk of X,
    the leading d/2 block of H, 256 rows of W over all columns."""
    import oracle as O
    blas, threads = _blas()
    d, r = cfg.cols, cfg.rows
    ntok = min(8192, cfg.tokens)
    x = I.x_chunk(cfg, 0, ntok)
    t0 = time.perf_counter()
    H = O.hessian([x])
    diag = O.hessian_diag([x])
    t_h = time.perf_counter() - t0
    del x
    ds = max(d // 2, 1)
    t0 = time.perf_counter()
    perm = O.act_order_perm(diag[:ds]) if cfg.act_order else np.arange(ds)
    Hp = O.damped_processing_hessian(H[:ds, :ds], diag[:ds], perm, cfg.percdamp)
    O.inverse_cholesky_upper(Hp)
    t_u = time.perf_counter() - t0
    del H, Hp
    nrow = min(256, r)
    W = I.weight_rows(cfg, np.arange(nrow)).astype(np.float64)
    U = np.eye(d)   # the sweep's cost does not depend on U's values
    t0 = time.perf_counter()
    sw = O.gptq_sweep(W, U, O.GridSpec(cfg.grid, cfg.bits, cfg.group))
    t_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    O.pack(sw.q.astype(np.int64), cfg.bits)
    t_p = time.perf_counter() - t0
    scale = {"hessian": cfg.tokens / ntok, "inverse_factor": (d / ds) ** 3,
             "sweep": r / nrow, "pack": r / nrow}
    meas = {"hessian": t_h, "inverse_factor": t_u, "sweep": t_s, "pack": t_p}
    split = {k: round(meas[k] * scale[k] * 1e3, 1) for k in meas}
    total_ms = sum(split.values())
    return {"value": round(total_ms, 1), "unit": "ms", "cores": int(threads), "kind": "oracle",
            "extrapolated": True,
            "sample": (f"H on {ntok} of {cfg.tokens} tokens; damping, act-order and inverse "
                       f"factor on the leading {ds}x{ds} block; sweep and pack over all {d} "
                       f"columns of {nrow} of {r} rows; each part scaled by its cost model "
                       f"(tokens, d^3, rows); float64 numpy"),
            "measured_s": {k: round(v, 2) for k, v in meas.items()},
            "scale": {k: round(v, 3) for k, v in scale.items()},
            "split_ms": split, "cpu_model": _cpu_model(), "blas": blas}


# W4A16 product workloads: the shapes of the quantization workloads, stored as
# int4 with groups of 128 (rows, cols, group, activation order).
W4A16_SHAPES = {
    "q_proj_4096x4096_int4_g128": (4096, 4096, 128, False),
    "down_proj_4096x11008_int4_g128_actorder": (4096, 11008, 128, True),
    "up_proj_28672x8192_int4_g128_actorder": (28672, 8192, 128, True),
    "mlp_14336x4096_int4_g128": (14336, 4096, 128, False),
}
W4A16_ROTATE_BYTES = 1 << 30


def w4a16_bytes(rows, cols, group, batch):
    """Algorithmic HBM bytes of one product: 4-bit codes, float32 scales,
    4-bit zero points, fp16 x and y."""
    ng = cols // group
    return rows * cols // 2 + rows * ng * 4 + (rows * ng + 1) // 2 + 2 * batch * (cols + rows)


def bench_w4a16(args):
    import ctypes

    import torch
    from post_weight_quantization_layer_amd import binding as B
    from post_weight_quantization_layer_amd.w4a16 import W4A16Linear

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    batches = [int(b) for b in args.w4a16_batches.split(",")]
    shapes = args.w4a16_shapes.split(",") if args.w4a16_shapes else list(W4A16_SHAPES)
    for name in shapes:
        rows, cols, group, act = W4A16_SHAPES[name]
        St = I.stored_int4_layer(rows, cols, group, act, seed=rows + cols)
        base = W4A16Linear.from_codes(torch.from_numpy(St.codes).to(dev),
                                      torch.from_numpy(St.g_idx).to(dev),
                                      torch.from_numpy(St.scale).to(dev),
                                      torch.from_numpy(St.zero).to(dev), group)
        del St
        copies = max(2, -(-W4A16_ROTATE_BYTES // base.mem.numel()))
        mems = [base.mem] + [base.mem.clone() for _ in range(copies - 1)]
        layers = []
        for m in mems:
            lay = B.gptq_w4a16_layer()
            ctypes.pointer(lay)[0] = base.layer
            lay.mem = m.data_ptr()
            layers.append(lay)
        torch.cuda.synchronize()
        log(f"[w4a16] {name}: {copies} copies of {base.mem.numel() / 2**20:.1f} MiB")
        for b in batches:
            x = torch.from_numpy(I.activations_f16(b, cols, seed=b).view(np.int16)).to(dev)
            x = x.view(torch.float16)
            y = torch.empty((b, rows), dtype=torch.float16, device=dev)
            nws = B.gptq_w4a16_workspace_bytes(layers[0], b)
            ws = torch.empty(max(nws, 256), dtype=torch.uint8, device=dev)
            iters = max(args.w4a16_iters, copies)
            for i in range(copies):
                B.gptq_w4a16_gemm(layers[i], x, y, ws)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(iters):
                B.gptq_w4a16_gemm(layers[i % copies], x, y, ws)
            e1.record()
            e1.synchronize()
            us_call = e0.elapsed_time(e1) * 1e3 / iters
            B.gptq_profile_reset()
            B.gptq_profile_enable(True)
            for i in range(iters):
                B.gptq_w4a16_gemm(layers[i % copies], x, y, ws)
            torch.cuda.synchronize()
            B.gptq_profile_enable(False)
            n_g, ms_g = B.gptq_profile_query("w4a16_gemm")
            n_x, ms_x = B.gptq_profile_query("w4a16_gather_x")
            k_us = ms_g / n_g * 1e3
            nbytes = w4a16_bytes(rows, cols, group, b)
            gbs = nbytes / (k_us * 1e-6) / 1e9
            line = {
                "metric": "W4A16 product, HBM GB/s of the product kernel",
                "value": round(gbs, 1), "unit": "GB/s", "higher_is_better": True,
                "dtype": "int4 x f16 -> f32 sums -> f16", "data": "synthetic",
                "config": {"workload": name, "rows": rows, "cols": cols, "group": group,
                           "act_order": act, "batch": b},
                "us_per_call": round(us_call, 2),
                "kernel_us": {"w4a16_gemm": round(k_us, 2),
                              "w4a16_gather_x": round(ms_x / n_x * 1e3, 2) if n_x else None},
                "roofline": {"bound": "hbm", "kernel": "w4a16_gemm", "achieved": round(gbs, 1),
                             "peak": PEAK["hbm"], "unit": "GB/s",
                             "frac": round(gbs / PEAK["hbm"], 4), "traffic": None,
                             "algorithmic_bytes_per_launch": nbytes},
            }
            print(json.dumps(line), flush=True)
        del layers, mems, base
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default=I.HEADLINE, choices=sorted(I.CONFIGS))
    ap.add_argument("--chunk-tokens", type=int, default=32768)
    ap.add_argument("--route", default="auto", choices=["auto", "inverse", "hessian"],
                    help="factor carrying the compensation (auto: the Hessian's own factor "
                         "where the layer allows it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-profile", action="store_true")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="run one plain streaming kernel of known size (read and write "
                         "1 GiB) before the steps, to scale rocprofv3 byte counters")
    ap.add_argument("--search", action="store_true",
                    help="choose each group's grid by the importance-weighted search")
    ap.add_argument("--w4a16", action="store_true",
                    help="measure the W4A16 product of stored 4-bit layers instead")
    ap.add_argument("--w4a16-batches", default="1,2,4,8,16,32,64")
    ap.add_argument("--w4a16-shapes", default="")
    ap.add_argument("--w4a16-iters", type=int, default=200)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(a layer's rows would shard across GPUs with one broadcast of U); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.w4a16:
        bench_w4a16(args)
        return

    import torch
    from post_weight_quantization_layer_amd import binding as B
    from post_weight_quantization_layer_amd.layer import GptqLayer

    cfg = I.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    B.lib()
    chunk = min(args.chunk_tokens, cfg.tokens)
    spans = I.token_chunks(cfg, chunk)

    # ---- inputs resident in HBM
    t0 = time.time()
    xdt = torch.bfloat16 if cfg.x_dtype == "bf16" else torch.float32
    X = torch.empty((cfg.cols, cfg.tokens), dtype=xdt, device=dev)
    for (a, n) in I.token_chunks(cfg, 8192):
        xs = I.x_chunk_storage(cfg, a, n)
        src = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16) if xs.dtype == np.uint16 \
            else torch.from_numpy(xs)
        X[:, a:a + n].copy_(src)
    W0 = torch.from_numpy(I.weight(cfg)).to(dev)
    Ws = [torch.empty_like(W0) for _ in range(args.warmup + args.steps)]
    for w in Ws:
        w.copy_(W0)
    layer = GptqLayer(cfg.rows, cfg.cols, bits=cfg.bits, group=cfg.group, block=cfg.block,
                      act_order=cfg.act_order, percdamp=cfg.percdamp, grid=cfg.grid, device=dev,
                      search=args.search, route=args.route)
    out = layer.alloc_outputs()
    packed_q = torch.empty((cfg.rows, cfg.cols * cfg.bits // 32), dtype=torch.int32, device=dev)
    packed_z = None
    if cfg.grid == "affine":
        nz = out["zero"].numel()
        packed_z = torch.empty(((nz * cfg.bits + 31) // 32,), dtype=torch.int32, device=dev)
    if args.pmc_calibration:
        a = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
    torch.cuda.synchronize()
    log(f"[bench] inputs ready in {time.time() - t0:.1f}s: X {tuple(X.shape)} {X.dtype}, "
        f"W {tuple(W0.shape)}, ws {layer.ws.numel() / 2**20:.0f} MiB")

    def step(i):
        layer.reset_hessian()
        for (a, n) in spans:
            B.gptq_hessian_accumulate(layer.H, layer.hdiag, X[:, a:a + n], n_tok=n,
                                      ld_x=X.stride(0), ws=layer.ws)
        layer.prepare()
        res = layer.quantize(Ws[i], out)
        layer.pack_codes(res.q, packed_q)
        if packed_z is not None and (out["zero"].numel() * cfg.bits) % 32 == 0:
            layer.pack_zeros(out["zero"], packed_z)

    for i in range(args.warmup):
        step(i)
        log(f"[bench] warmup step {i} done")
    # timed steps: the library's per-launch profiling events are off
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    log(f"[bench] {args.steps} steps: {ms:.3f} ms/step")
    # the same number of steps again with HIP events around every launch on
    # the launch stream, for the per-kernel split and the roofline
    if not args.no_profile:
        for i in range(args.steps):
            Ws[args.warmup + i].copy_(W0)   # the timed steps quantized these in place
        torch.cuda.synchronize()
        B.gptq_profile_reset()
        B.gptq_profile_enable(True)
        for i in range(args.steps):
            step(args.warmup + i)
        torch.cuda.synchronize()
        B.gptq_profile_enable(False)

    kernels = {}
    names = ["hessian_syrk_bf16", "hessian_fold", "hessian_syrk_f32", "hessian_diag", "prep_diag",
             "prep_rank_perm", "prep_symmetrize", "prep_gather", "chol_diag_block", "chol_trsm", "chol_near", "chol_mid", "chol_syrk",
             "trtri_gemm", "prep_rotate", "quant_gather", "quant_zero_dead", "sweep_affine",
             "sweep_q4k", "trailing_near", "trailing_group", "trailing_gemm", "quant_scatter",
             "quant_g_idx", "pack"]
    if not args.no_profile:
        for nme in names:
            n, tms = B.gptq_profile_query(nme)
            if n:
                kernels[nme] = {"launches_per_step": n / args.steps,
                                "ms_per_step": round(tms / args.steps, 4),
                                "avg_us": round(tms / n * 1e3, 2)}
    roof = None
    if kernels:
        tn = [kernels[k] for k in ("trailing_group", "trailing_gemm") if k in kernels]
        if tn:
            kernels["trailing"] = {"launches_per_step": sum(k["launches_per_step"] for k in tn),
                                   "ms_per_step": round(sum(k["ms_per_step"] for k in tn), 4)}
        work = kernel_work(cfg, chunk)
        for k, (kind_k, f) in work.items():
            if k not in kernels:
                continue
            per_step = f * (kernels[k]["launches_per_step"] if k == "hessian_syrk_bf16" else 1)
            kernels[k]["tflops"] = round(per_step / (kernels[k]["ms_per_step"] * 1e-3) / 1e12, 1)
            kernels[k]["mfma_frac"] = round(kernels[k]["tflops"] / PEAK[kind_k], 4)
        dom = "hessian_syrk_bf16"
    if kernels and dom in kernels:
        kind, per_launch = work[dom]
        avg_s = kernels[dom]["avg_us"] * 1e-6
        achieved = per_launch / avg_s / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": PEAK[kind], "unit": "TFLOP/s", "frac": round(achieved / PEAK[kind], 4),
                "traffic": measured_traffic(dom, cfg.name, chunk),
                "algorithmic_flops_per_launch": per_launch}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a bounded sample ...")
        cpu = cpu_baseline(cfg, chunk)
        log(f"[bench] oracle: {cpu['value']} ms/layer on {cpu['cores']} threads")

    line = {
        "metric": METRIC, "value": round(ms, 3), "unit": "ms", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3),
        "higher_is_better": False, "scaling": "strong", "vs_baseline": None,
        "dtype": "bf16+f32", "data": "synthetic",
        "config": {"workload": cfg.name, "rows": cfg.rows, "cols": cfg.cols,
                   "tokens": cfg.tokens, "chunk_tokens": chunk, "bits": cfg.bits,
                   "group": cfg.group, "block": cfg.block, "act_order": cfg.act_order,
                   "grid": cfg.grid, "percdamp": cfg.percdamp, "search": args.search, "route": layer.route},
        "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
