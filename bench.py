#!/usr/bin/env python3
"""Benchmark of the quantized-linear hot path on one MI355X.

One step = one pass of the whole path over synthetic inputs already resident
in HBM:
  1. forward fake-quantization (2-bit SEQ, given alpha) of the whole
     MobileLLM-1.5B-shaped stack -- 378 matrices, 1,473,638,400 weights with
     0.1 % outliers -- in one grouped launch (bf16 weights + packed codes out);
  2. the straight-through backward of the same stack (dW + per-row dalpha)
     in one grouped launch;
  3. the packed export of the same stack (2-bit codes in the export byte
     order + bf16 alpha) in one grouped launch;
  4. the W2A16 GEMM on one 16384 x 16384 packed weight at M = 512, 64, 16, 4,
     1, each on its own copy of the weight (8 copies rotate, so the 256 MB
     MALL cannot serve repeats), each with its caller-owned workspace.
Alpha initialisation (once per run), the MobileLLM-125M stack at every bit
width, the Llama-3-8B projections' quantizer and GEMM, the 4-bit GEMM
variant and a hipBLASLt bf16 GEMM are timed after the steps.

Every kernel is timed with HIP events on the stream it is launched on (torch's
current stream); the step's events are timing-only events without the
system-scope cache fence a default event record adds (TimingEvent).  `value` is the headline metric: quantize fwd+bwd throughput
in GB/s of algorithmic bytes on the 1.5B stack.  The CPU baseline is the
oracle (test infrastructure) on a sample of the same stack and on sampled
GEMM outputs, timed on the host cores.
"""
import argparse
import hashlib
import json
import re
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
GEMM_MS = (1, 4, 16, 64, 512)
# Order of the GEMMs inside a step.  The export pack before them leaves tens
# of MB of dirty cache lines whose write-back the next kernel pays for (about
# 8 us measured after a 1 GiB copy); the MFMA-bound M = 512 GEMM absorbs it
# with the least distortion of its own time, so it goes first.
GEMM_STEP_ORDER = (512, 64, 16, 4, 1)
GEMM_NK = 16384
ROTATE = 8
LLAMA_MS = (1, 16, 256, 4096)
# weight copies rotated per timed GEMM: enough that one pass over them
# exceeds the 256 MB last-level cache, so every launch streams from HBM
ROTATE_BYTES = 320 << 20


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    # the chip's clocks settle over the first ~20 ms of sustained load (the
    # M = 512 GEMM measured 257 us in the first step, 200 us from the 25th
    # on), so the default warm-up runs about 50 ms of steps
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true", help="skip sweep / comparison GEMMs")
    p.add_argument("--gemm-b2b-only", action="store_true",
                   help="only the back-to-back GEMM launches (for a kernel trace of them alone)")
    p.add_argument("--train-fwd-only", action="store_true",
                   help="only the training-forward measurement (for a kernel trace of it alone)")
    p.add_argument("--llama-gemm-only", action="store_true",
                   help="print only the Llama-3-8B projection GEMM measurements")
    p.add_argument("--qat-step-only", action="store_true",
                   help="only the fused QAT step measurement (for a kernel trace of it alone)")
    p.add_argument("--pmc-workload", action="store_true",
                   help="no timing: a 1 GiB copy (counter calibration), then every step kernel "
                        "three times in step order, for rocprofv3 --pmc passes")
    p.add_argument("--pmc-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="turn the two --pmc-workload counter runs into the traffic table")
    p.add_argument("--pmc-out", default=os.path.join(ROOT, "profiles", "hbm_traffic_bench_kernels.md"))
    p.add_argument("--pmc-command", default="", help="command lines recorded in the traffic table")
    p.add_argument("--mfma-summarize", metavar="PMC_DIR",
                   help="turn a --pmc-workload counter run of the MFMA counters into the MFMA table")
    p.add_argument("--mfma-out", default=os.path.join(ROOT, "profiles", "mfma_util_gemm_kernels.md"))
    return p.parse_args()


# Sources whose kernels each bench kernel runs: the traffic recorded for a
# kernel is reported only while these files are unchanged.
_QUANT_SOURCES = ("pq_quant.hip", "pq_quant_kernels.hpp", "pq_quant_mode.hip", "pq_common.hpp")
KERNEL_SOURCES = {"fwd": _QUANT_SOURCES, "bwd": _QUANT_SOURCES, "pack": _QUANT_SOURCES, "qat_step": _QUANT_SOURCES}
for _m in (1, 4, 16, 64, 512):
    KERNEL_SOURCES[f"gemm_m{_m}"] = ("pq_gemm.hip", "pq_gemm_big.hip", "pq_gemm_common.hpp", "pq_common.hpp")
CALIB_BYTES = 1 << 30   # the calibration copy reads and writes 1 GiB
# --pmc-workload: the step entries in this order, each called PMC_CALLS times
# between marker launches
PMC_KEYS = ("fwd", "bwd", "pack") + tuple(f"gemm_m{M}" for M in (512, 64, 16, 4, 1))
PMC_CALLS = 3
MARKER = "k_weight_movement"


def pmc_segments(dispatches):
    """Split [(name, counters)] of a --pmc-workload run at the marker
    launches: {key: [counters of every launch of that key's calls]}, and the
    launches before the first marker (the fused step's and the calibration
    copies)."""
    idx = [i for i, (n, _) in enumerate(dispatches) if MARKER in n]
    if len(idx) < len(PMC_KEYS) + 1:
        raise SystemExit(f"expected {len(PMC_KEYS) + 1} marker launches, found {len(idx)}")
    idx = idx[-(len(PMC_KEYS) + 1):]
    seg = {k: [c for _, c in dispatches[idx[j] + 1:idx[j + 1]]] for j, k in enumerate(PMC_KEYS)}
    return seg, dispatches[:idx[0]]


def source_sha(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "bit_quantization_aware_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(path):
    """kernel -> HBM bytes per launch, from the traffic table, for kernels
    whose sources still match the hash recorded with the counters."""
    out = {}
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return out
    for ln in lines:
        cells = [c.strip() for c in ln.strip().strip("|").split("|")]
        if len(cells) >= 6 and cells[0] in KERNEL_SOURCES:
            try:
                if cells[1] == source_sha(cells[0]):
                    out[cells[0]] = int(float(cells[5]))
            except (ValueError, OSError):
                pass
    return out


def recorded_mfma(path):
    """gemm kernel -> MFMA utilisation (fraction of the MFMA pipes' cycles
    busy over the launch), from the MFMA counter table, for kernels whose
    sources still match the recorded hash."""
    out = {}
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return out
    for ln in lines:
        cells = [c.strip() for c in ln.strip().strip("|").split("|")]
        if len(cells) >= 4 and cells[0] in KERNEL_SOURCES:
            try:
                if cells[1] == source_sha(cells[0]):
                    out[cells[0]] = float(cells[2])
            except (ValueError, OSError):
                pass
    return out


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence:
    recording it writes a timestamp without the system-scope cache write-back
    and invalidate that a default event adds (HIP documents the flag for
    this: the fence costs time and disturbs the following work, so kernels
    timed between default events look slower than they run).  Made through
    the HIP runtime this process already uses (torch's), found by its mapped
    path, so that torch's streams are valid handles for it."""
    FLAGS = 0x20000000  # hipEventDisableSystemFence
    _lib = None

    @classmethod
    def hip(cls):
        if cls._lib is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded")
            L = ctypes.CDLL(path)
            L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._lib = L
        return cls._lib

    def __init__(self):
        import ctypes
        self._c = ctypes
        self.e = ctypes.c_void_p()
        rc = self.hip().hipEventCreateWithFlags(ctypes.byref(self.e), self.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: {rc}")

    def record(self, stream):
        rc = self.hip().hipEventRecord(self.e, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord: {rc}")

    def elapsed_time(self, end):
        ms = self._c.c_float()
        rc = self.hip().hipEventElapsedTime(self._c.byref(ms), self.e, end.e)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime: {rc}")
        return float(ms.value)

    def __del__(self):
        if self._lib is not None and self.e:
            self._lib.hipEventDestroy(self.e)


def fwd_bytes(rows, cols, cw):
    return cols * rows * (4 + 2 + cw / 8) + 4 * rows


def bwd_bytes(rows, cols):
    return cols * rows * 12 + 8 * rows


def step_bytes(rows, cols, cw):
    """Fused QAT step: W, G, m, v read, W, m, v written, bf16 Wq and codes
    written; per row alpha and its two moments read and written."""
    return cols * rows * (16 + 12 + 2 + cw / 8) + 24 * rows


def pack_bytes(rows, cols):
    return cols * rows * (4 + 0.25) + 6 * rows


def gemm_bytes(M, N, K, bits):
    return N * K * bits / 8 + 2 * N + 2 * M * K + 2 * M * N


def load_pmc(d, counters):
    """[(kernel name, {counter: value summed over the dispatch's rows})] in
    dispatch order, from a rocprofv3 --pmc csv run under directory d."""
    import csv
    import glob

    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for r in csv.DictReader(open(f[0])):
        if r["Counter_Name"] not in counters:
            continue
        e = per.setdefault(int(r["Dispatch_Id"]), (r["Kernel_Name"], {}))
        e[1][r["Counter_Name"]] = e[1].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [per[k] for k in sorted(per)]


def pmc_summarize(args):
    """HBM bytes per call of each step entry from the FETCH_SIZE and
    WRITE_SIZE passes of --pmc-workload (every launch of the call summed:
    the quantizer's launches per team class, the M = 64 split-K finalize),
    each counter scaled by what it reads for the
    1 GiB copy; and the fused step's."""
    fetch = load_pmc(args.pmc_summarize[0], ("FETCH_SIZE",))
    write = load_pmc(args.pmc_summarize[1], ("WRITE_SIZE",))
    fseg, fpre = pmc_segments(fetch)
    wseg, wpre = pmc_segments(write)

    # the calibration copies: the three largest copy dispatches before the
    # first marker (the fused step measurement also clones tensors)
    def calib(seq, c):
        vals = sorted((v[c] for name, v in seq if "copy" in name.lower() and "pq::" not in name), reverse=True)
        return vals[:3] if len(vals) >= 3 else None

    cf, cw_ = calib(fpre, "FETCH_SIZE"), calib(wpre, "WRITE_SIZE")
    if not cf or not cw_:
        raise SystemExit("calibration copy dispatches not found")
    fscale = CALIB_BYTES / (np.mean(cf) * 1024.0)
    wscale = CALIB_BYTES / (np.mean(cw_) * 1024.0)
    res = {}
    for k in PMC_KEYS:
        res[k] = (sum(c["FETCH_SIZE"] for c in fseg[k]) / PMC_CALLS,
                  sum(c["WRITE_SIZE"] for c in wseg[k]) / PMC_CALLS)
    # the fused step: its last three launches before the calibration
    sf = [v["FETCH_SIZE"] for n, v in fpre if "k_qat_step<2," in n][-3:]
    sw = [v["WRITE_SIZE"] for n, v in wpre if "k_qat_step<2," in n][-3:]
    if len(sf) == 3 and len(sw) == 3:
        res["qat_step"] = (float(np.mean(sf)), float(np.mean(sw)))
    lines = [
        "# HBM traffic per launch of the bench.py step kernels (rocprofv3 PMC)",
        "",
        "Counters: `FETCH_SIZE` and `WRITE_SIZE` (KiB per dispatch), each collected in its own",
        "rocprofv3 pass over `bench.py --pmc-workload` (one MI355X). Each counter is scaled by what",
        "it reads for a plain 1 GiB device copy in the same run (1 GiB read, 1 GiB written):",
        f"FETCH scale = {fscale:.4f}, WRITE scale = {wscale:.4f}. Per call of each step entry (the mean of",
        "three calls): every launch of the call summed -- the quantizer's launch per team class, the M = 64",
        "split-K finalize. fwd, bwd and pack are the 1.5B stack's; qat_step the",
        "125M stack's fused step.",
        "`sha` is the hash of the kernel sources the counters were taken on (bench.py reports",
        "`traffic` only while it matches).",
        "",
        "Commands:",
        "```",
    ] + [c for c in args.pmc_command.split(";;") if c] + [
        "```",
        "",
        "| kernel | sha | FETCH KiB | WRITE KiB | scaled bytes (read) | scaled bytes (total) |",
        "|---|---|---|---|---|---|",
    ]
    for k, (f, w) in res.items():
        rb = f * 1024.0 * fscale
        tb = rb + w * 1024.0 * wscale
        lines.append(f"| {k} | {source_sha(k)} | {f:.0f} | {w:.0f} | {rb:.0f} | {tb:.0f} |")
    os.makedirs(os.path.dirname(args.pmc_out), exist_ok=True)
    with open(args.pmc_out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


C3 = "mobilellm_1p5b"
C2 = "mobilellm_125m"


def _gen(cfg, k):
    from bit_quantization_aware_amd import synth
    return synth.weight(cfg, k), synth.upstream_grad(cfg, k)


def build_stack(torch, pq, cfg, mode, dev, export=False):
    """Upload a stacked config's W and G (generated on the host, matrix by
    matrix from its own seed stream, 16 threads) and allocate every output of
    the fwd, bwd (and export) launches.  Returns (mats, fwd, bwd, exp) with
    the grouped descriptor tables."""
    from concurrent.futures import ThreadPoolExecutor
    from bit_quantization_aware_amd import synth

    shapes = synth.SHAPES[cfg]()
    n = len(shapes)
    mats = []
    with ThreadPoolExecutor(16) as ex:
        for c0 in range(0, n, 32):
            ks = range(c0, min(n, c0 + 32))
            for W, G in ex.map(lambda k: _gen(cfg, k), ks):
                r, c = W.shape
                m = dict(W=torch.from_numpy(W).to(dev), G=torch.from_numpy(G).to(dev), rows=r, cols=c,
                         alpha=torch.zeros(r, dtype=torch.float32, device=dev),
                         wq_bf16=torch.empty(r, c, dtype=torch.bfloat16, device=dev),
                         codes=torch.empty(r, pq.pq_code_row_bytes(mode, c), dtype=torch.uint8, device=dev),
                         dW=torch.empty(r, c, dtype=torch.float32, device=dev),
                         dalpha=torch.empty(r, dtype=torch.float32, device=dev),
                         grad_scale=pq.pq_default_grad_scale(mode, r, c))
                if export:
                    m["packed"] = torch.empty(pq.pq_packed_bytes(mode, r, c), dtype=torch.uint8, device=dev)
                    m["alpha_bf16"] = torch.empty(r, dtype=torch.bfloat16, device=dev)
                mats.append(m)
    ft = pq.MatTable([{k: m[k] for k in ("W", "alpha", "wq_bf16", "codes", "rows", "cols")} for m in mats])
    bt = pq.MatTable([{k: m[k] for k in ("W", "alpha", "G", "dW", "dalpha", "grad_scale", "rows", "cols")}
                      for m in mats])
    et = None
    if export:
        et = pq.MatTable([dict(W=m["W"], alpha=m["alpha"], codes=m["packed"], alpha_bf16=m["alpha_bf16"],
                               rows=m["rows"], cols=m["cols"]) for m in mats])
    return mats, ft, bt, et


MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU",
                 "SQ_INSTS_MFMA", "SQ_BUSY_CYCLES", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VALU")
SIMD_NUM = 1024   # 256 CUs x 4 SIMDs
XCDS = 8          # GRBM_GUI_ACTIVE comes summed over the 8 XCDs
# kernel-name parts of each GEMM of the step (M = 64 adds its split-K finalize)
GEMM_PARTS = {
    "gemm_m1": (r"k_gemm_stream<2, \d+, \d+, \d+, 1>",),
    "gemm_m4": (r"k_gemm_stream<2, \d+, \d+, \d+, 2>",),
    "gemm_m16": (r"k_gemm_stream<2, \d+, \d+, \d+, 8>",),
    "gemm_m64": (r"k_gemm_tile<2,", r"k_splitk_finalize"),
    "gemm_m512": (r"k_gemm_big2<2>",),
}


def mfma_summarize(args):
    """MFMA utilisation of the step's GEMMs from one rocprofv3 --pmc pass of
    MFMA_COUNTERS over --pmc-workload: MfmaUtil = sum over SIMDs of
    SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / XCDS * SIMD_NUM), the
    counter tool's definition (its max over XCDs taken as the per-XCD mean
    of the summed value); flops = SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512."""
    disp = load_pmc(args.mfma_summarize, MFMA_COUNTERS)
    seg, _ = pmc_segments(disp)
    rows = {}
    for key in PMC_KEYS:
        if not key.startswith("gemm"):
            continue
        tot = {c: sum(d.get(c, 0.0) for d in seg[key]) / PMC_CALLS for c in MFMA_COUNTERS}
        M = int(key.split("m")[-1])
        busy, gui = tot["SQ_VALU_MFMA_BUSY_CYCLES"], tot["GRBM_GUI_ACTIVE"] / XCDS
        mfma = tot["SQ_INSTS_MFMA"]
        rows[key] = dict(
            util=busy / (gui * SIMD_NUM) if gui else 0.0,
            flops_counted=tot["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512,
            flops_needed=2.0 * M * GEMM_NK * GEMM_NK,
            valu_per_mfma=(tot["SQ_INSTS_VALU"] - mfma) / mfma if mfma else 0.0,
            lds_per_mfma=tot["SQ_INSTS_LDS"] / mfma if mfma else 0.0,
            valu_active=tot["SQ_ACTIVE_INST_VALU"] / (gui * SIMD_NUM) if gui else 0.0,
            gui=gui)
    lines = [
        "# MFMA utilisation of the bench.py step GEMMs (16384 x 16384, 2-bit; rocprofv3 PMC)",
        "",
        "One rocprofv3 `--pmc` pass of the counters below over `bench.py --pmc-workload` (one MI355X),",
        "per call (mean of three; M = 64 adds its split-K finalize).",
        "`util` = sum over SIMDs of SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x",
        f"{SIMD_NUM} SIMDs) -- the counter tool's MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES counts 16 cycles per",
        "16x16x32 bf16 MFMA); GRBM_GUI_ACTIVE includes the launch's ramp, so short launches read low;",
        "`flops counted` = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512,",
        "`flops needed` = 2 M N K (the counted flops also hold the row sums' all-ones MFMAs, and the",
        "kernels pad M to 16-row MFMA tiles, so small M counts more);",
        "`VALU/MFMA` = (SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA, the decode and bookkeeping",
        "issued per MFMA; `LDS/MFMA` likewise; `VALU active` = SQ_ACTIVE_INST_VALU per SIMD-cycle;",
        "`GUI cycles` = GRBM_GUI_ACTIVE / 8.",
        "`sha` is the hash of the GEMM sources the counters were taken on (bench.py reports",
        "`mfma_util` per GEMM only while it matches).",
        "",
        "Command:",
        "```",
    ] + [c for c in args.pmc_command.split(";;") if c] + [
        "```",
        "",
        "| kernel | sha | util | flops counted | flops needed | VALU/MFMA | LDS/MFMA | VALU active | GUI cycles |",
        "|---|---|---|---|---|---|---|---|---|",
    ]
    for k, r in rows.items():
        lines.append(f"| {k} | {source_sha(k)} | {r['util']:.4f} | {r['flops_counted']:.4g} | "
                     f"{r['flops_needed']:.4g} | {r['valu_per_mfma']:.2f} | {r['lds_per_mfma']:.2f} | "
                     f"{r['valu_active']:.3f} | {r['gui']:.0f} |")
    os.makedirs(os.path.dirname(args.mfma_out), exist_ok=True)
    with open(args.mfma_out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    args = parse()
    if args.pmc_summarize:
        pmc_summarize(args)
        return
    if args.mfma_summarize:
        mfma_summarize(args)
        return
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
    sid = stream.cuda_stream
    mode = pq.PQ_W2_SEQ
    cw = pq.CODE_BITS[mode]

    # ------------------------------------------------------------------ inputs
    # the 125M stack: extras (bit-width sweep, fused step, training forward)
    stack, ftab, btab, _ = build_stack(torch, pq, C2, mode, dev)

    def make_tables(md):
        for m in stack:
            r, c = m["rows"], m["cols"]
            m["alpha"] = torch.zeros(r, dtype=torch.float32, device=dev)
            m["codes"] = torch.empty(r, pq.pq_code_row_bytes(md, c), dtype=torch.uint8, device=dev)
            m["grad_scale"] = pq.pq_default_grad_scale(md, r, c)
        ft = pq.MatTable([{k: m[k] for k in ("W", "alpha", "wq_bf16", "codes", "rows", "cols")}
                          for m in stack])
        bt = pq.MatTable([{k: m[k] for k in ("W", "alpha", "G", "dW", "dalpha", "grad_scale",
                                            "rows", "cols")} for m in stack])
        return ft, bt

    W16 = torch.from_numpy(synth.weight("square16k", 0)).to(dev)
    a16 = torch.zeros(GEMM_NK, dtype=torch.float32, device=dev)
    pq.pq_quantize_fwd(mode, GEMM_NK, GEMM_NK, W16, a16, pq.PQ_INIT_ALPHA, None, None, None)
    pbytes = pq.pq_packed_bytes(pq.PQ_W2_SEQ, GEMM_NK, GEMM_NK)
    packed = [torch.empty(pbytes, dtype=torch.uint8, device=dev) for _ in range(ROTATE)]
    ab16 = [torch.empty(GEMM_NK, dtype=torch.bfloat16, device=dev) for _ in range(ROTATE)]
    for i in range(ROTATE):
        pq.pq_pack_w2(GEMM_NK, GEMM_NK, W16, a16, packed[i], ab16[i])
    Xs = {M: torch.from_numpy(synth.activations("square16k", 0, M, GEMM_NK).view(np.int16)).to(dev)
          .view(torch.bfloat16) for M in GEMM_MS}
    Ys = {M: torch.empty(M, GEMM_NK, dtype=torch.bfloat16, device=dev) for M in GEMM_MS}
    # caller-owned GEMM workspaces, one per M (the library allocates nothing)
    wss = {M: pq.gemm_workspace(mode, M, GEMM_NK, GEMM_NK) for M in GEMM_MS}
    wsa = {M: ((w.data_ptr(), w.numel()) if w is not None else (0, 0)) for M, w in wss.items()}

    pq.pq_quantize_fwd_grouped(mode, ftab, pq.PQ_INIT_ALPHA)
    kernels = ["fwd", "bwd", "pack"] + [f"gemm_m{M}" for M in GEMM_STEP_ORDER]

    if args.train_fwd_only:
        print(json.dumps({"train_forward": train_forward_measure(torch, pq, stack, stream)}), flush=True)
        return

    if args.llama_gemm_only:
        print(json.dumps({"llama_gemm": llama_gemm_measure(torch, pq, synth, stream)}), flush=True)
        return

    if args.qat_step_only:
        print(json.dumps({"qat_step": qat_step_measure(torch, pq, stack, ftab, btab, stream)}), flush=True)
        return

    if args.gemm_b2b_only:
        ridge = MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3
        print(json.dumps({"gemm_back_to_back": gemm_back_to_back(torch, pq, Xs, packed, ab16, Ys, wsa, stream,
                                                                 ridge)}), flush=True)
        return

    # the 1.5B stack: the step's quantizer work
    t_up = time.perf_counter()
    big, ftab3, btab3, etab3 = build_stack(torch, pq, C3, mode, dev, export=True)
    torch.cuda.synchronize()
    upload_s = time.perf_counter() - t_up
    n_el = sum(m["rows"] * m["cols"] for m in big)
    n_rows = sum(m["rows"] for m in big)
    print(f"bench: 1.5B stack resident ({len(big)} matrices, {n_el} weights, {upload_s:.1f} s)",
          file=sys.stderr, flush=True)

    # alpha init of the stack (once per run), timed once after a warm launch
    pq.pq_quantize_fwd_grouped(mode, ftab3, pq.PQ_INIT_ALPHA)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    pq.pq_quantize_fwd_grouped(mode, ftab3, pq.PQ_INIT_ALPHA)
    e1.record(stream)
    torch.cuda.synchronize()
    init_ms = e0.elapsed_time(e1)

    if args.pmc_workload:
        # the fused step's own launches first (it runs unfused comparisons
        # too), then a 1 GiB copy for the counter calibration, then every
        # step entry three times, each entry's launches between two marker
        # launches (k_weight_movement on 64 weights, used nowhere else here)
        qat = qat_step_measure(torch, pq, stack, ftab, btab, stream, reps=3)
        print("pmc workload: qat_step", flush=True)
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        mk = torch.zeros(64, device=dev)
        mk2 = torch.zeros(8, dtype=torch.float64, device=dev)

        def marker():
            pq.pq_weight_movement(8, 8, mk, mk, mk2, mk2)
        launches = {
            "fwd": lambda: pq.pq_quantize_fwd_grouped(mode, ftab3, 0),
            "bwd": lambda: pq.pq_quantize_bwd_grouped(mode, btab3, pq.PQ_G_F32),
            "pack": lambda: pq.pq_pack_grouped(mode, etab3),
        }
        for j, M in enumerate(GEMM_MS):
            launches[f"gemm_m{M}"] = (lambda M=M, j=j: pq.pq_w2a16_gemm(
                M, GEMM_NK, GEMM_NK, Xs[M], packed[1 + j % (ROTATE - 1)], ab16[1 + j % (ROTATE - 1)], Ys[M],
                workspace=wsa[M]))
        marker()
        for k in PMC_KEYS:
            for _ in range(PMC_CALLS):
                launches[k]()
            marker()
            torch.cuda.synchronize()
            print(f"pmc workload: {k} x{PMC_CALLS}", flush=True)
        return

    def step(it, evs):
        evs[0].record(stream)
        pq.pq_quantize_fwd_grouped(mode, ftab3, 0)
        evs[1].record(stream)
        pq.pq_quantize_bwd_grouped(mode, btab3, pq.PQ_G_F32)
        evs[2].record(stream)
        pq.pq_pack_grouped(mode, etab3)
        evs[3].record(stream)
        for j, M in enumerate(GEMM_STEP_ORDER):
            b = (it + 1 + j) % ROTATE
            pq.pq_w2a16_gemm(M, GEMM_NK, GEMM_NK, Xs[M], packed[b], ab16[b], Ys[M], workspace=wsa[M])
            evs[4 + j].record(stream)

    nev = 4 + len(GEMM_STEP_ORDER)
    for it in range(args.warmup):
        step(it, [TimingEvent() for _ in range(nev)])
    torch.cuda.synchronize()

    all_evs = [[TimingEvent() for _ in range(nev)] for _ in range(args.steps)]
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

    fb = sum(fwd_bytes(m["rows"], m["cols"], cw) for m in big)
    bb = sum(bwd_bytes(m["rows"], m["cols"]) for m in big)
    pb = sum(pack_bytes(m["rows"], m["cols"]) for m in big)
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
        sec = d["ms"] * 1e-3
        if d["bound"] == "hbm":
            ach = d["bytes"] / sec / 1e9
            rl[k] = dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=round(ach / HBM_PEAK_GBS, 4), ms=round(d["ms"], 5))
        else:
            ach = d["flops"] / sec / 1e12
            rl[k] = dict(bound="mfma", achieved=round(ach, 1), peak=MFMA_BF16_PEAK_TFLOPS,
                         unit="TFLOP/s", frac=round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                         ms=round(d["ms"], 5))
        if k.startswith("gemm"):
            rl[k]["weight_stream_GBs"] = round(d["bytes"] / sec / 1e9, 1)
            rl[k]["tflops"] = round(d["flops"] / sec / 1e12, 2)
    dominant = max(info, key=lambda k: info[k]["ms"])
    per_launch_units = {"fwd": f"{n_el} weights (378 matrices)", "bwd": f"{n_el} weights (378 matrices)",
                        "pack": f"{n_el} weights (378 matrices)"}
    roofline = dict(rl[dominant])
    roofline.pop("ms", None)
    roofline["kernel"] = dominant
    traffic = recorded_traffic(args.pmc_out)
    roofline["traffic"] = traffic.get(dominant)
    for k in rl:
        rl[k]["traffic"] = traffic.get(k)
    step_traffic = traffic.get("qat_step")
    roofline["units_per_launch"] = per_launch_units.get(dominant, "one GEMM call")
    roofline["bytes_per_unit"] = {"fwd": 4 + 2 + cw / 8, "bwd": 12, "pack": 4.25}.get(dominant)
    mfma = recorded_mfma(args.mfma_out)
    for k in rl:
        if k in mfma:
            rl[k]["mfma_util"] = mfma[k]

    qt_ms = avg["fwd"] + avg["bwd"]
    value = (fb + bb) / (qt_ms * 1e-3) / 1e9
    init_bytes = fb + 4 * n_rows   # the forward's bytes (alpha written besides)

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
            "workload": "MobileLLM-1.5B-shaped stack (54 layers x q,o 1600x1600, k,v 400x1600, gate,up "
                        "4352x1600, down 1600x4352; 378 matrices, 1,473,638,400 fp32 weights ~N(0,0.02^2) "
                        "with 0.1% outliers x10), 2-bit SEQ fwd+bwd and packed export in one grouped "
                        "launch each; plus the 16384x16384 2-bit W2A16 GEMM at M in {1,4,16,64,512}",
            "bits": 2, "matrices": len(big), "weights": n_el, "rows": n_rows,
            "gemm_nk": GEMM_NK, "gemm_m": list(GEMM_MS), "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "roofline": roofline,
        "kernels": rl,
        "alpha_init": dict(ms=round(init_ms, 4), fwd_GBs=round(init_bytes / init_ms / 1e6, 1),
                           frac_of_fwd_bytes=round(init_bytes / init_ms / 1e6 / HBM_PEAK_GBS, 4)),
        "wall_s_timed": round(wall, 3),
        "upload_s": round(upload_s, 2),
    }
    del big, ftab3, btab3, etab3
    torch.cuda.empty_cache()

    if not args.no_extras:
        out["diagnostics"] = diagnostics_measure(torch, pq, W16, a16, stream)
        out["train_forward"] = train_forward_measure(torch, pq, stack, stream)
        out["qat_step"] = qat_step_measure(torch, pq, stack, ftab, btab, stream)
        out["qat_step"]["traffic"] = step_traffic
        out["gemm_back_to_back"] = gemm_back_to_back(torch, pq, Xs, packed, ab16, Ys, wsa, stream, ridge)
        # (the sweep re-allocates the 125M stack's alpha and codes: it runs
        # after every measurement that uses the first tables)
        out["mobilellm_125m"] = sweep_bits(torch, pq, stack, make_tables, stream)
        out["llama3_8b_quantizer"] = llama_quantizer_measure(torch, pq, synth, stream)
        out["gemm_compare"] = gemm_compare(torch, pq, W16, a16, Xs, stream)
        out["llama_gemm"] = llama_gemm_measure(torch, pq, synth, stream)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()

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


def diagnostics_measure(torch, pq, W16, a16, stream, reps=10):
    """Level occupancy of the 16384 x 16384 weight's codes and its movement
    against a perturbed copy: one launch each."""
    mode = pq.PQ_W2_SEQ
    N = K = GEMM_NK
    L = pq.pq_num_levels(mode)
    dev = W16.device
    codes = torch.empty(N, pq.pq_code_row_bytes(mode, K), dtype=torch.uint8, device=dev)
    pq.pq_quantize_fwd(mode, N, K, W16, a16, 0, None, None, codes)
    counts = torch.empty(N, L, dtype=torch.int32, device=dev)
    ent = torch.empty(N, dtype=torch.float64, device=dev)
    W0 = W16 + 1e-4
    d2 = torch.empty(N, dtype=torch.float64, device=dev)
    r2 = torch.empty(N, dtype=torch.float64, device=dev)
    ts = b2b_ms(torch, stream, lambda i: pq.pq_level_stats(mode, N, K, codes, counts, ent), reps)
    tm = b2b_ms(torch, stream, lambda i: pq.pq_weight_movement(N, K, W16, W0, d2, r2), reps)
    sb, mb = N * K / 4 + N * (4 * L + 8), N * K * 8 + N * 16
    out = dict(level_stats_ms=round(ts, 4), level_stats_GBs=round(sb / ts / 1e6, 1),
               level_stats_frac=round(sb / ts / 1e6 / HBM_PEAK_GBS, 4),
               movement_ms=round(tm, 4), movement_GBs=round(mb / tm / 1e6, 1),
               movement_frac=round(mb / tm / 1e6 / HBM_PEAK_GBS, 4), shape=f"{N}x{K}")
    # the pages' SEQ-vs-LSQ argument: mean level entropy (bits) of the same
    # weight under each grid, each with its own max-based alpha init
    grids = {}
    for md in (pq.PQ_W2_SEQ, pq.PQ_W2_LSQ, pq.PQ_W158_SEQ_TERNARY, pq.PQ_W158_LSQ):
        a = torch.zeros(N, dtype=torch.float32, device=dev)
        pq.pq_quantize_fwd(md, N, K, W16, a, pq.PQ_INIT_ALPHA, None, None, codes)
        cnt = torch.empty(N, pq.pq_num_levels(md), dtype=torch.int32, device=dev)
        pq.pq_level_stats(md, N, K, codes, cnt, ent)
        grids[pq.MODE_NAMES[md]] = round(float(ent.mean()), 4)
    out["mean_level_entropy_bits"] = grids
    # the forward (codes only) with and without the level statistics fused in
    tf = b2b_ms(torch, stream, lambda i: pq.pq_quantize_fwd(mode, N, K, W16, a16, 0, None, None, codes), reps)
    tfs = b2b_ms(torch, stream, lambda i: pq.pq_quantize_fwd_stats(mode, N, K, W16, a16, None, codes, counts, ent),
                 reps)
    fb = N * K * (4 + 0.25) + 4 * N
    out["fwd_codes_ms"] = round(tf, 4)
    out["fwd_codes_fused_stats_ms"] = round(tfs, 4)
    out["fwd_codes_fused_stats_frac"] = round(fb / tfs / 1e6 / HBM_PEAK_GBS, 4)
    del codes, W0
    return out


TRAIN_TOKENS = 16384  # 8 sequences x 2048 tokens (one GPU's share of the recipe's batch)


def train_forward_measure(torch, pq, stack, stream, reps=3):
    """The QAT forward of every quantized linear of the 2-bit stack at
    8 x 2048 tokens: (a) this library's forward writing only the codes in the
    export byte order, then pq_gemm_f32a per matrix (codes + fp32 alpha);
    (b) the forward writing bf16 weights, then hipBLASLt (torch.matmul) per
    matrix on them.  Three alternating passes of each; the medians are
    reported."""
    mode = pq.PQ_W2_SEQ
    dev = stack[0]["W"].device
    T = TRAIN_TOKENS
    sid = stream.cuda_stream
    xs, ys = {}, {}
    for m in stack:
        c, r = m["cols"], m["rows"]
        if c not in xs:
            xs[c] = (torch.randn(T, c, device=dev) * 0.5).to(torch.bfloat16)
        if r not in ys:
            ys[r] = torch.empty(T, r, dtype=torch.bfloat16, device=dev)
    mats = [dict(W=m["W"], alpha=m["alpha"], rows=m["rows"], cols=m["cols"],
                 codes=torch.empty(pq.pq_packed_bytes(mode, m["rows"], m["cols"]), dtype=torch.uint8, device=dev))
            for m in stack]
    ctab = pq.MatTable([{k: d[k] for k in ("W", "alpha", "codes", "rows", "cols")} for d in mats])
    btab = pq.MatTable([{k: m[k] for k in ("W", "alpha", "wq_bf16", "rows", "cols")} for m in stack])
    wss = {}
    for m in stack:
        key = (m["rows"], m["cols"])
        if key not in wss:
            wss[key] = pq.gemm_workspace(mode, T, m["rows"], m["cols"])
    wsa = {k: ((w.data_ptr(), w.numel()) if w is not None else (0, 0)) for k, w in wss.items()}
    calls = [(m["rows"], m["cols"], xs[m["cols"]].data_ptr(), d["codes"].data_ptr(), m["alpha"].data_ptr(),
              ys[m["rows"]].data_ptr(), wsa[(m["rows"], m["cols"])]) for m, d in zip(stack, mats)]

    def codes_path():
        pq.pq_quantize_fwd_grouped(mode, ctab, pq.PQ_CODES_EXPORT)
        for r, c, xp, cp, ap, yp, wa in calls:
            pq.pq_gemm_f32a(mode, T, r, c, xp, cp, ap, yp, sid, workspace=wa)

    def bf16_path():
        pq.pq_quantize_fwd_grouped(mode, btab, 0)
        for m in stack:
            torch.matmul(xs[m["cols"]], m["wq_bf16"].t(), out=ys[m["rows"]])

    a, b, pa, pb = paired_ms(lambda: b2b_ms(torch, stream, lambda i: codes_path(), reps),
                             lambda: b2b_ms(torch, stream, lambda i: bf16_path(), reps))
    fwd_c = b2b_ms(torch, stream, lambda i: pq.pq_quantize_fwd_grouped(mode, ctab, pq.PQ_CODES_EXPORT), reps)
    fwd_b = b2b_ms(torch, stream, lambda i: pq.pq_quantize_fwd_grouped(mode, btab, 0), reps)
    fl = 2.0 * T * sum(m["rows"] * m["cols"] for m in stack)
    return dict(tokens=T, codes_path_ms=round(a, 4), codes_path_tflops=round(fl / a / 1e9, 1),
                bf16_path_ms=round(b, 4), bf16_path_tflops=round(fl / b / 1e9, 1),
                fwd_codes_only_ms=round(fwd_c, 4), fwd_bf16_codes_ms=round(fwd_b, 4),
                gemm="codes: pq_gemm_f32a per matrix; bf16: torch.matmul (hipBLASLt) per matrix",
                speedup=round(b / a, 3), codes_passes_ms=[round(t, 4) for t in pa],
                bf16_passes_ms=[round(t, 4) for t in pb])


def qat_step_measure(torch, pq, stack, ftab, btab, stream, reps=10):
    """The fused QAT step (backward, AdamW on W and alpha, next forward) over
    the 2-bit stack in one grouped launch, against the same work unfused:
    this library's backward and forward launches with torch's fused AdamW
    in between (on the dW and dalpha the backward wrote)."""
    mode = pq.PQ_W2_SEQ
    dev = stack[0]["W"].device
    mats = []
    for m in stack:
        r, c = m["rows"], m["cols"]
        mats.append(dict(W=m["W"].clone(), alpha=m["alpha"].clone(), G=m["G"],
                         mW=torch.zeros(r, c, device=dev), vW=torch.zeros(r, c, device=dev),
                         m_alpha=torch.zeros(r, device=dev), v_alpha=torch.zeros(r, device=dev),
                         wq_bf16=m["wq_bf16"], codes=m["codes"], grad_scale=m["grad_scale"], rows=r, cols=c))
    table = pq.StepTable(mats)
    hps = [pq.adamw_params(t + 1) for t in range(reps + 1)]
    pq.pq_qat_step_grouped(mode, table, hps[0])
    fused = time_it(torch, stream, lambda i: pq.pq_qat_step_grouped(mode, table, hps[i]), reps)
    sb = sum(step_bytes(m["rows"], m["cols"], pq.CODE_BITS[mode]) for m in stack)
    gbs = sb / fused / 1e6

    # unfused: backward (dW, dalpha) -> torch AdamW -> forward
    params = [m["W"] for m in mats] + [m["alpha"] for m in mats]
    for m, s_ in zip(mats, stack):
        m["W"].grad = s_["dW"]
        m["alpha"].grad = s_["dalpha"]
    try:
        opt = torch.optim.AdamW(params, lr=2e-5, weight_decay=0.0, fused=True)
        kind = "torch.optim.AdamW(fused=True)"
    except (RuntimeError, TypeError):
        opt = torch.optim.AdamW(params, lr=2e-5, weight_decay=0.0, foreach=True)
        kind = "torch.optim.AdamW(foreach=True)"
    opt.step()
    bwd = time_it(torch, stream, lambda i: pq.pq_quantize_bwd_grouped(mode, btab, pq.PQ_G_F32), reps)
    adam = time_it(torch, stream, lambda i: opt.step(), reps)
    fwd = time_it(torch, stream, lambda i: pq.pq_quantize_fwd_grouped(mode, ftab, 0), reps)
    for p_ in params:
        p_.grad = None
    del opt, table, mats
    return dict(ms=round(fused, 4), bytes=int(sb), achieved_GBs=round(gbs, 1), peak_GBs=HBM_PEAK_GBS,
                frac=round(gbs / HBM_PEAK_GBS, 4), bytes_per_weight=30.25,
                unfused=dict(bwd_ms=round(bwd, 4), adamw_ms=round(adam, 4), fwd_ms=round(fwd, 4),
                             total_ms=round(bwd + adam + fwd, 4), adamw=kind, bytes_per_weight=46.25),
                speedup_vs_unfused=round((bwd + adam + fwd) / fused, 3))


def gemm_back_to_back(torch, pq, Xs, packed, ab16, Ys, wsa, stream, ridge, reps=40):
    """Each GEMM of the step launched `reps` times in a row on the rotating
    weight copies, with one event pair around the run: the kernel's rate
    without the event packets and the other kernels of the step in between
    (the in-step times above include both)."""
    res = {}
    sid = stream.cuda_stream
    pk = [p.data_ptr() for p in packed]
    ab = [a.data_ptr() for a in ab16]
    for M in GEMM_MS:
        xp, yp = Xs[M].data_ptr(), Ys[M].data_ptr()

        def run(i, M=M, xp=xp, yp=yp):
            # plain integers: the host side of a launch stays well below the
            # kernel time, so the GPU never waits for the next launch
            b = i % ROTATE
            pq.pq_w2a16_gemm(M, GEMM_NK, GEMM_NK, xp, pk[b], ab[b], yp, sid, workspace=wsa[M])
        for i in range(8):
            run(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            run(i)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        by = gemm_bytes(M, GEMM_NK, GEMM_NK, 2)
        fl = 2.0 * M * GEMM_NK * GEMM_NK
        gbs, tf = by / ms / 1e6, fl / ms / 1e9
        frac = gbs / HBM_PEAK_GBS if fl / by < ridge else tf / MFMA_BF16_PEAK_TFLOPS
        res[f"m{M}"] = dict(ms=round(ms, 5), weight_stream_GBs=round(gbs, 1), tflops=round(tf, 2),
                            frac=round(frac, 4))
    return res


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


def paired_ms(fa, fb, passes=3):
    """Two timings taken in alternating passes (a, b, a, b, ...): the medians
    and every pass.  The first pass of a shape runs on cold clocks and caches
    for both sides; the median keeps it from deciding the comparison."""
    ta, tb = [], []
    for _ in range(passes):
        ta.append(fa())
        tb.append(fb())
    return statistics.median(ta), statistics.median(tb), ta, tb


def b2b_ms(torch, stream, run, reps):
    """Mean time per launch of `reps` launches in a row, one event pair
    around them (after a few warm launches)."""
    for i in range(4):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        run(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def graph_ms(torch, run, reps, check=None):
    """Mean time per launch of `reps` launches captured in one HIP graph and
    replayed: launches a few microseconds long are then timed without the
    host's per-call cost between them.  run(i, sid) launches call i on the
    stream `sid`; `check`, if given, returns the output, which must be the
    same after the replay as after an eager call."""
    # warm launches, then capture on a side stream
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(4):
            run(i, side.cuda_stream)
    torch.cuda.synchronize()
    want = check().clone() if check else None
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for i in range(reps):
            run(i, side.cuda_stream)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    if check is not None:
        assert torch.equal(check(), want), "graph replay changed the output"
    del g
    return e0.elapsed_time(e1) / reps


def gemm_compare(torch, pq, W16, a16, Xs, stream, reps=30):
    """The other widths through the same kernels (binary in 1-bit codes, ternary
    in the 2-bit container, 3- and 4-bit LSQ in nibbles) and a hipBLASLt bf16 GEMM on the
    dequantized weight, at the same shapes: each launched back to back on 8
    rotating weight copies (the 2-bit numbers are in gemm_back_to_back)."""
    N = K = GEMM_NK
    sid = stream.cuda_stream
    res = {f"m{M}": {} for M in GEMM_MS}
    widths = (("w1", pq.PQ_W1_BINARY, 1), ("ternary", pq.PQ_W158_SEQ_TERNARY, 2), ("w3", pq.PQ_W3_LSQ, 4),
              ("w4", pq.PQ_W4_LSQ, 4))
    for name, md, cbits in widths:
        a = torch.zeros(N, dtype=torch.float32, device="cuda")
        pq.pq_quantize_fwd(md, N, K, W16, a, pq.PQ_INIT_ALPHA, None, None, None)
        pk = [torch.empty(pq.pq_packed_bytes(md, N, K), dtype=torch.uint8, device="cuda") for _ in range(ROTATE)]
        ab = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(ROTATE)]
        for i in range(ROTATE):
            pq.pq_pack(md, N, K, W16, a, pk[i], ab[i])
        pkp, abp = [t.data_ptr() for t in pk], [t.data_ptr() for t in ab]
        for M in GEMM_MS:
            xp = Xs[M].data_ptr()
            Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            yp = Y.data_ptr()
            ws = pq.gemm_workspace(md, M, N, K)
            wa = (ws.data_ptr(), ws.numel()) if ws is not None else (0, 0)
            ms = b2b_ms(torch, stream, lambda i: pq.pq_gemm(md, M, N, K, xp, pkp[i % ROTATE], abp[i % ROTATE], yp,
                                                              sid, workspace=wa), reps)
            fl = 2.0 * M * N * K
            res[f"m{M}"].update({f"{name}_ms": round(ms, 5), f"{name}_tflops": round(fl / ms / 1e9, 2),
                                 f"{name}_weight_GBs": round(gemm_bytes(M, N, K, cbits) / ms / 1e6, 1)})
        del pk, ab
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
        tb = b2b_ms(torch, stream, lambda i: torch.matmul(X, wbf[i % ROTATE].t(), out=Y), reps)
        fl = 2.0 * M * N * K
        res[f"m{M}"].update(bf16_hipblaslt_ms=round(tb, 5), bf16_tflops=round(fl / tb / 1e9, 2))
    del wbf
    return res


def llama_gemm_measure(torch, pq, synth, stream, reps=20):
    """The four Llama-3-8B projections (2-bit SEQ, exported) through the W2A16
    GEMM at M in {1, 16, 256, 4096}, next to a hipBLASLt bf16 GEMM on the
    dequantized weight.  Both rotate weight copies (ROTATE_BYTES) and run
    back to back inside one HIP graph (so that launches of a few microseconds
    are not bound by the host's per-call cost), in three alternating passes
    whose medians are reported; frac is against the weight-stream roofline
    below the ridge point and the bf16 MFMA peak above it."""
    res = {}
    ridge = MFMA_BF16_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3
    for k, (_, name, N, K) in enumerate(synth.llama3_8b_shapes()):
        W = torch.from_numpy(synth.weight("llama3_8b", k)).to("cuda")
        a = torch.zeros(N, dtype=torch.float32, device="cuda")
        wq = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
        pq.pq_quantize_fwd(pq.PQ_W2_SEQ, N, K, W, a, pq.PQ_INIT_ALPHA, wq, None, None)
        nb = pq.pq_packed_bytes(pq.PQ_W2_SEQ, N, K)
        R = max(2, -(-ROTATE_BYTES // nb))
        pk = [torch.empty(nb, dtype=torch.uint8, device="cuda") for _ in range(R)]
        ab = [torch.empty(N, dtype=torch.bfloat16, device="cuda") for _ in range(R)]
        for i in range(R):
            pq.pq_pack_w2(N, K, W, a, pk[i], ab[i])
        del W
        Rb = max(2, -(-ROTATE_BYTES // (N * K * 2)))
        wb = [wq] + [wq.clone() for _ in range(Rb - 1)]
        pkp, abp = [t.data_ptr() for t in pk], [t.data_ptr() for t in ab]
        for M in LLAMA_MS:
            X = torch.from_numpy(synth.activations("llama3_8b", k, M, K).view(np.int16)).to("cuda") \
                .view(torch.bfloat16)
            Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            xp, yp = X.data_ptr(), Y.data_ptr()
            ws = pq.gemm_workspace(pq.PQ_W2_SEQ, M, N, K)
            wa = (ws.data_ptr(), ws.numel()) if ws is not None else (0, 0)
            ms, tb, pa, pb = paired_ms(
                lambda: graph_ms(torch, lambda i, sd: pq.pq_w2a16_gemm(M, N, K, xp, pkp[i % R], abp[i % R], yp,
                                                                       sd, workspace=wa),
                                 reps, check=lambda: Y),
                lambda: graph_ms(torch, lambda i, sd: torch.matmul(X, wb[i % Rb].t(), out=Y), reps))
            fl, by = 2.0 * M * N * K, gemm_bytes(M, N, K, 2)
            gbs, tf = by / ms / 1e6, fl / ms / 1e9
            frac = gbs / HBM_PEAK_GBS if fl / by < ridge else tf / MFMA_BF16_PEAK_TFLOPS
            res[f"{name}_m{M}"] = dict(ms=round(ms, 5), tflops=round(tf, 2), weight_stream_GBs=round(gbs, 1),
                                       frac=round(frac, 4), bf16_hipblaslt_ms=round(tb, 5),
                                       speedup_vs_bf16=round(tb / ms, 2),
                                       passes_ms=[round(t, 5) for t in pa],
                                       bf16_passes_ms=[round(t, 5) for t in pb])
        del pk, ab, wb, wq
        torch.cuda.empty_cache()
    return res


def llama_quantizer_measure(torch, pq, synth, stream, reps=10):
    """The Llama-3-8B projections' quantizer: 2-bit SEQ and ternary forward
    (bf16 weights + codes, given alpha) and backward (dW + dalpha), one
    matrix per launch, back to back; GB/s of algorithmic bytes and the
    fraction of HBM peak."""
    res = {}
    for k, (_, name, N, K) in enumerate(synth.llama3_8b_shapes()):
        W = torch.from_numpy(synth.weight("llama3_8b", k)).to("cuda")
        G = torch.from_numpy(synth.upstream_grad("llama3_8b", k)).to("cuda")
        wq = torch.empty(N, K, dtype=torch.bfloat16, device="cuda")
        dW = torch.empty_like(W)
        da = torch.empty(N, dtype=torch.float32, device="cuda")
        for md, tag in ((pq.PQ_W2_SEQ, "w2_seq"), (pq.PQ_W158_SEQ_TERNARY, "ternary")):
            a = torch.zeros(N, dtype=torch.float32, device="cuda")
            codes = torch.empty(N, pq.pq_code_row_bytes(md, K), dtype=torch.uint8, device="cuda")
            pq.pq_quantize_fwd(md, N, K, W, a, pq.PQ_INIT_ALPHA, None, None, None)
            gs = pq.pq_default_grad_scale(md, N, K)
            f = b2b_ms(torch, stream, lambda i: pq.pq_quantize_fwd(md, N, K, W, a, 0, wq, None, codes), reps)
            b = b2b_ms(torch, stream, lambda i: pq.pq_quantize_bwd(md, N, K, W, a, G, pq.PQ_G_F32, gs, dW, da),
                       reps)
            fb, bb = fwd_bytes(N, K, pq.CODE_BITS[md]), bwd_bytes(N, K)
            gbs = (fb + bb) / ((f + b) * 1e-3) / 1e9
            res[f"{name}_{tag}"] = dict(fwd_ms=round(f, 4), bwd_ms=round(b, 4), fwd_GBs=round(fb / f / 1e6, 1),
                                        bwd_GBs=round(bb / b / 1e6, 1), fwdbwd_GBs=round(gbs, 1),
                                        frac=round(gbs / HBM_PEAK_GBS, 4))
        del W, G, wq, dW
        torch.cuda.empty_cache()
    return res


def cpu_baseline(reps=5, gemm_samples=4096):
    """The oracle (plain C, OpenMP over rows) on a bounded sample of the
    step's workload, on the host cores of this run:
      * quantizer: 2-bit SEQ forward + backward over layers 0 and 1 of the
        1.5B stack (14 matrices, 54,579,200 weights), the median of `reps`
        whole passes at 1 thread and at every core;
      * GEMM: the binary64 reference (the parity oracle) on `gemm_samples`
        sampled outputs of the 16384^2 2-bit GEMM at each M, every core,
        scaled to the whole call's flops."""
    import oracle as O
    from bit_quantization_aware_amd import synth

    cores = len(os.sched_getaffinity(0))
    shapes = synth.mobilellm_1p5b_shapes()
    ks = [k for k, (l, _, _, _) in enumerate(shapes) if l in (0, 1)]
    data = []
    for k in ks:
        W, G = _gen(C3, k)
        data.append((W, G, O.alpha_init(O.SEQ2, W)))
    n_el = sum(W.size for W, _, _ in data)
    alg = sum(fwd_bytes(W.shape[0], W.shape[1], 2) + bwd_bytes(W.shape[0], W.shape[1]) for W, _, _ in data)

    def one_pass():
        t0 = time.perf_counter()
        for W, G, a in data:
            O.quantize_fwd(O.SEQ2, W, a)
            O.quantize_bwd(O.SEQ2, W, a, G)
        return time.perf_counter() - t0

    legs = {}
    for name, th in (("one_thread", 1), ("all_cores", cores)):
        O.set_threads(th)
        ts = [one_pass() for _ in range(reps)]
        med = float(np.median(ts))
        legs[name] = dict(threads=O.max_threads(), median_s=round(med, 4), passes=reps,
                          GBs=round(alg / med / 1e9, 3), weights_per_s=round(n_el / med, 1))

    O.set_threads(cores)
    W = synth.weight("square16k", 0)
    a = O.alpha_init(O.SEQ2, W)
    p, ab = O.pack(O.SEQ2, W, a)
    del W
    gemm = {}
    for M in GEMM_MS:
        X = synth.activations("square16k", 0, M, GEMM_NK)
        rng = np.random.default_rng(M)
        ms, ns = rng.integers(0, M, gemm_samples), rng.integers(0, GEMM_NK, gemm_samples)
        t0 = time.perf_counter()
        O.gemm_ref_at(O.SEQ2, X, p, ab, GEMM_NK, ms, ns)
        dt = time.perf_counter() - t0
        fl = 2.0 * gemm_samples * GEMM_NK
        full = 2.0 * M * GEMM_NK * GEMM_NK
        gemm[f"m{M}"] = dict(sampled_outputs=gemm_samples, seconds=round(dt, 4), gflops=round(fl / dt / 1e9, 3),
                             full_call_s_est=round(dt * full / fl, 2))
    cpu = ""
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    return {"value": legs["all_cores"]["GBs"], "unit": "GB/s", "cores": legs["all_cores"]["threads"],
            "kind": "oracle", "cpu": cpu, "one_thread": legs["one_thread"], "all_cores": legs["all_cores"],
            "gemm_fp64_reference": gemm,
            "sample": f"2-bit SEQ forward + backward over layers 0-1 of the MobileLLM-1.5B stack "
                      f"({len(data)} matrices, {n_el} weights; same algorithmic bytes per weight as the "
                      f"GPU step), median of {reps} whole passes at 1 thread and at {cores} threads; the "
                      "oracle also writes fp32 values and mask bits the GPU step does not.  GEMM: the "
                      f"binary64 reference on {gemm_samples} sampled outputs of the 16384^2 call per M, "
                      "scaled to the call's flops"}


if __name__ == "__main__":
    main()
