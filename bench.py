#!/usr/bin/env python3
"""Benchmark of the quantized-linear hot path on one MI355X.

One step = one pass of the whole path over synthetic inputs already resident
in HBM:
  1. forward fake-quantization (2-bit SEQ, given alpha) of the whole
     MobileLLM-125M-shaped stack -- 210 matrices, 119,439,360 weights -- in
     one grouped launch (bf16 weights + packed codes out);
  2. the straight-through backward of the same stack (dW + per-row dalpha)
     in one grouped launch;
  3. export packing (2-bit codes + bf16 alpha) of one 16384 x 16384 weight;
  4. the W2A16 GEMM on that packed weight at M = 1, 4, 16, 64, 512, each on
     its own copy of the packed weight (8 copies rotate, so the 256 MB MALL
     cannot serve repeats).
Alpha initialisation (once per run) and the per-bit-width sweep of the stack,
the 4-bit GEMM variant and a hipBLASLt bf16 GEMM are timed after the steps.

Every kernel is timed with HIP events on the stream it is launched on (torch's
current stream).  `value` is the headline metric: quantize fwd+bwd throughput
in GB/s of algorithmic bytes on the stack.  The CPU baseline is the oracle
(test infrastructure) on the same stack, timed on the host cores.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
GEMM_MS = (1, 4, 16, 64, 512)
GEMM_NK = 16384
ROTATE = 8


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip sweep / comparison GEMMs")
    return p.parse_args()


def fwd_bytes(rows, cols, cw):
    return cols * rows * (4 + 2 + cw / 8) + 4 * rows


def bwd_bytes(rows, cols):
    return cols * rows * 12 + 8 * rows


def pack_bytes(rows, cols):
    return cols * rows * (4 + 0.25) + 6 * rows


def gemm_bytes(M, N, K, bits):
    return N * K * bits / 8 + 2 * N + 2 * M * K + 2 * M * N


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the quantizer shards "
              "by rows and the GEMM by output columns with no exchange, but this build measures "
              "one GPU's share.", file=sys.stderr)
        sys.exit(2)

    import torch
    from bit_quantization_aware_amd import pq, synth

    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    dev = "cuda"
    stream = torch.cuda.current_stream()

    # ------------------------------------------------------------------ inputs
    shapes = synth.mobilellm_125m_shapes()
    mode = pq.PQ_W2_SEQ
    stack = []
    for k, (_, _, rows, cols) in enumerate(shapes):
        W = torch.from_numpy(synth.weight("mobilellm_125m", k)).to(dev)
        G = torch.from_numpy(synth.upstream_grad("mobilellm_125m", k)).to(dev)
        stack.append(dict(W=W, G=G, rows=rows, cols=cols))
    n_el = sum(m["rows"] * m["cols"] for m in stack)
    n_rows = sum(m["rows"] for m in stack)

    def make_tables(md):
        for m in stack:
            r, c = m["rows"], m["cols"]
            m["alpha"] = torch.zeros(r, dtype=torch.float32, device=dev)
            m["wq_bf16"] = torch.empty(r, c, dtype=torch.bfloat16, device=dev)
            m["codes"] = torch.empty(r, pq.pq_code_row_bytes(md, c), dtype=torch.uint8, device=dev)
            m["dW"] = torch.empty(r, c, dtype=torch.float32, device=dev)
            m["dalpha"] = torch.empty(r, dtype=torch.float32, device=dev)
            m["grad_scale"] = pq.pq_default_grad_scale(md, r, c)
        ft = pq.MatTable([{k: m[k] for k in ("W", "alpha", "wq_bf16", "codes", "rows", "cols")}
                          for m in stack])
        bt = pq.MatTable([{k: m[k] for k in ("W", "alpha", "G", "dW", "dalpha", "grad_scale",
                                            "rows", "cols")} for m in stack])
        return ft, bt

    ftab, btab = make_tables(mode)

    W16 = torch.from_numpy(synth.weight("square16k", 0)).to(dev)
    a16 = torch.zeros(GEMM_NK, dtype=torch.float32, device=dev)
    pq.pq_quantize_fwd(mode, GEMM_NK, GEMM_NK, W16, a16, pq.PQ_INIT_ALPHA, None, None, None)
    packed = [torch.empty(GEMM_NK, GEMM_NK // 4, dtype=torch.uint8, device=dev) for _ in range(ROTATE)]
    ab16 = [torch.empty(GEMM_NK, dtype=torch.bfloat16, device=dev) for _ in range(ROTATE)]
    for i in range(ROTATE):
        pq.pq_pack_w2(GEMM_NK, GEMM_NK, W16, a16, packed[i], ab16[i])
    Xs = {M: torch.from_numpy(synth.activations("square16k", 0, M, GEMM_NK).view(np.int16)).to(dev)
          .view(torch.bfloat16) for M in GEMM_MS}
    Ys = {M: torch.empty(M, GEMM_NK, dtype=torch.bfloat16, device=dev) for M in GEMM_MS}

    # alpha init of the stack (once per run), timed once after a warm launch
    pq.pq_quantize_fwd_grouped(mode, ftab, pq.PQ_INIT_ALPHA)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    pq.pq_quantize_fwd_grouped(mode, ftab, pq.PQ_INIT_ALPHA)
    e1.record(stream)
    torch.cuda.synchronize()
    init_ms = e0.elapsed_time(e1)

    kernels = ["fwd", "bwd", "pack"] + [f"gemm_m{M}" for M in GEMM_MS]

    def step(it, evs):
        evs[0].record(stream)
        pq.pq_quantize_fwd_grouped(mode, ftab, 0)
        evs[1].record(stream)
        pq.pq_quantize_bwd_grouped(mode, btab, pq.PQ_G_F32)
        evs[2].record(stream)
        r = it % ROTATE
        pq.pq_pack_w2(GEMM_NK, GEMM_NK, W16, a16, packed[r], ab16[r])
        evs[3].record(stream)
        for j, M in enumerate(GEMM_MS):
            b = (it + 1 + j) % ROTATE
            pq.pq_w2a16_gemm(M, GEMM_NK, GEMM_NK, Xs[M], packed[b], ab16[b], Ys[M])
            evs[4 + j].record(stream)

    nev = 4 + len(GEMM_MS)
    for it in range(args.warmup):
        step(it, [torch.cuda.Event(enable_timing=True) for _ in range(nev)])
    torch.cuda.synchronize()

    all_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for it in range(args.steps):
        step(args.warmup + it, all_evs[it])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    per = {k: [] for k in kernels}
    step_ms = []
    for evs in all_evs:
        for i, k in enumerate(kernels):
            per[k].append(evs[i].elapsed_time(evs[i + 1]))
        step_ms.append(evs[0].elapsed_time(evs[-1]))
    avg = {k: float(np.mean(v)) for k, v in per.items()}
    ms_per_step = float(np.mean(step_ms))

    cw = pq.CODE_BITS[mode]
    fb = sum(fwd_bytes(m["rows"], m["cols"], cw) for m in stack)
    bb = sum(bwd_bytes(m["rows"], m["cols"]) for m in stack)
    pb = pack_bytes(GEMM_NK, GEMM_NK)
    info = {
        "fwd": dict(bound="hbm", bytes=fb, ms=avg["fwd"]),
        "bwd": dict(bound="hbm", bytes=bb, ms=avg["bwd"]),
        "pack": dict(bound="hbm", bytes=pb, ms=avg["pack"]),
    }
    ridge = MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3  # flop per byte
    for M in GEMM_MS:
        by = gemm_bytes(M, GEMM_NK, GEMM_NK, 2)
        fl = 2.0 * M * GEMM_NK * GEMM_NK
        info[f"gemm_m{M}"] = dict(bound="hbm" if fl / by < ridge else "mfma", bytes=by, flops=fl,
                                  ms=avg[f"gemm_m{M}"])
    rl = {}
    for k, d in info.items():
        s = d["ms"] * 1e-3
        if d["bound"] == "hbm":
            ach = d["bytes"] / s / 1e9
            rl[k] = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(ach / HBM_PEAK_GBS, 4), ms=round(d["ms"], 5))
        else:
            ach = d["flops"] / s / 1e12
            rl[k] = dict(bound="mfma", achieved=round(ach, 1), peak=MFMA_BF16_PEAK_TFLOPS,
                         unit="TFLOP/s", frac=round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                         ms=round(d["ms"], 5))
        if k.startswith("gemm"):
            rl[k]["weight_stream_GBs"] = round(d["bytes"] / s / 1e9, 1)
            rl[k]["tflops"] = round(d["flops"] / s / 1e12, 2)
    dominant = max(info, key=lambda k: info[k]["ms"])
    per_launch_units = {"fwd": f"{n_el} weights", "bwd": f"{n_el} weights",
                        "pack": f"{GEMM_NK * GEMM_NK} weights"}
    roofline = dict(rl[dominant])
    roofline.pop("ms", None)
    roofline["kernel"] = dominant
    roofline["traffic"] = None
    roofline["units_per_launch"] = per_launch_units.get(dominant, "one GEMM call")

    qt_ms = avg["fwd"] + avg["bwd"]
    value = (fb + bb) / (qt_ms * 1e-3) / 1e9

    out = {
        "metric": "quantize fwd+bwd GB/s (% HBM peak); W2A16 GEMM TFLOP/s at 16384² (% roofline)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "MobileLLM-125M-shaped stack (30 layers x q,k,v,o 576x576, gate,up "
                        "1536x576, down 576x1536; 210 matrices, 119,439,360 fp32 weights "
                        "~N(0,0.02^2)), 2-bit SEQ fwd+bwd in one grouped launch each; plus "
                        "16384x16384 2-bit export and W2A16 GEMM at M in {1,4,16,64,512}",
            "bits": 2, "matrices": len(stack), "weights": n_el, "rows": n_rows,
            "gemm_nk": GEMM_NK, "gemm_m": list(GEMM_MS), "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": roofline,
        "kernels": rl,
        "alpha_init_ms": round(init_ms, 4),
        "wall_s_timed": round(wall, 3),
    }

    if not args.no_extras:
        out["sweep_bits"] = sweep_bits(torch, pq, stack, make_tables, stream)
        out["gemm_compare"] = gemm_compare(torch, pq, W16, a16, Xs, stream)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(shapes, fb + bb)

    print(json.dumps(out), flush=True)


def time_it(torch, stream, fn, reps):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    fn(0)
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(reps):
        fn(i + 1)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([evs[i].elapsed_time(evs[i + 1]) for i in range(reps)]))


def sweep_bits(torch, pq, stack, make_tables, stream):
    res = {}
    for md in pq.MODES:
        ft, bt = make_tables(md)
        pq.pq_quantize_fwd_grouped(md, ft, pq.PQ_INIT_ALPHA)
        f = time_it(torch, stream, lambda i: pq.pq_quantize_fwd_grouped(md, ft, 0), 10)
        b = time_it(torch, stream, lambda i: pq.pq_quantize_bwd_grouped(md, bt, pq.PQ_G_F32), 10)
        cw = pq.CODE_BITS[md]
        fb = sum(fwd_bytes(m["rows"], m["cols"], cw) for m in stack)
        bb = sum(bwd_bytes(m["rows"], m["cols"]) for m in stack)
        gbs = (fb + bb) / ((f + b) * 1e-3) / 1e9
        res[pq.MODE_NAMES[md]] = dict(fwd_ms=round(f, 4), bwd_ms=round(b, 4),
                                      fwd_GBs=round(fb / f / 1e6, 1), bwd_GBs=round(bb / b / 1e6, 1),
                                      fwdbwd_GBs=round(gbs, 1),
                                      pct_hbm_peak=round(100 * gbs / HBM_PEAK_GBS, 2))
    make_tables(pq.PQ_W2_SEQ)
    return res


def gemm_compare(torch, pq, W16, a16, Xs, stream):
    """4-bit variant of the same kernel and a hipBLASLt bf16 GEMM on the
    dequantized weight, at the same shapes (8 rotating weight copies each)."""
    N = K = GEMM_NK
    res = {}
    p4 = [torch.empty(N, K // 2, dtype=torch.uint8, device="cuda") for _ in range(ROTATE)]
    a4 = torch.zeros(N, dtype=torch.float32, device="cuda")
    pq.pq_quantize_fwd(pq.PQ_W4_LSQ, N, K, W16, a4, pq.PQ_INIT_ALPHA, None, None, None)
    ab4 = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(ROTATE)]
    for i in range(ROTATE):
        pq.pq_pack_w4(N, K, W16, a4, p4[i], ab4[i])
    wbf = [torch.empty(N, K, dtype=torch.bfloat16, device="cuda") for _ in range(ROTATE)]
    wq = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
    pq.pq_quantize_fwd(pq.PQ_W2_SEQ, N, K, W16, torch.zeros(N, device="cuda"), pq.PQ_INIT_ALPHA,
                       wq, None, None)
    for i in range(ROTATE):
        wbf[i].copy_(wq)
    del wq
    for M in GEMM_MS:
        X = Xs[M]
        Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
        t4 = time_it(torch, stream, lambda i: pq.pq_w4a16_gemm(M, N, K, X, p4[i % ROTATE],
                                                                ab4[i % ROTATE], Y), 20)
        tb = time_it(torch, stream, lambda i: torch.matmul(X, wbf[i % ROTATE].t(), out=Y), 20)
        fl = 2.0 * M * N * K
        res[f"m{M}"] = dict(w4a16_ms=round(t4, 5), w4a16_tflops=round(fl / t4 / 1e9, 2),
                            w4a16_weight_GBs=round(gemm_bytes(M, N, K, 4) / t4 / 1e6, 1),
                            bf16_hipblaslt_ms=round(tb, 5),
                            bf16_tflops=round(fl / tb / 1e9, 2))
    return res


def cpu_baseline(shapes, alg_bytes):
    """The oracle (plain C, OpenMP over rows) on the same 2-bit stack:
    one forward + backward pass over all 210 matrices."""
    import oracle as O
    from bit_quantization_aware_amd import synth

    cores = len(os.sched_getaffinity(0))
    O.set_threads(cores)
    t = 0.0
    for k in range(len(shapes)):
        W = synth.weight("mobilellm_125m", k)
        G = synth.upstream_grad("mobilellm_125m", k)
        alpha = O.alpha_init(O.SEQ2, W)
        t0 = time.perf_counter()
        O.quantize_fwd(O.SEQ2, W, alpha)
        O.quantize_bwd(O.SEQ2, W, alpha, G)
        t += time.perf_counter() - t0
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(alg_bytes / t / 1e9, 3), "unit": "GB/s", "cores": O.max_threads(),
            "kind": "oracle", "seconds": round(t, 3), "cpu": cpu,
            "sample": "one 2-bit SEQ forward + backward pass over all 210 matrices of the "
                      "MobileLLM-125M stack (the full GPU workload of steps 1-2), same "
                      "algorithmic byte count; the oracle also writes fp32 values and mask "
                      "bits the GPU step does not"}


if __name__ == "__main__":
    main()
