"""Build libpq.so (the HIP library behind include/pq.h) in-tree for gfx950.

hipcc compiles each HIP source to an object (in parallel), then links the
shared library next to this file.  Flags:
  -ffp-contract=off      every float step stays one IEEE operation (the
                         quantizer is bit-exact by construction);
  -packed-fp32-ops off   no v_pk_*_f32 instructions are generated;
  -amdgpu-mfma-vgpr-form MFMA accumulators live in ordinary VGPRs (no copies
                         between AGPRs and VGPRs around the MFMA chains).
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpq.so")
SOURCES = ["pq_quant.hip", "pq_gemm.hip", "pq_gemm_big.hip", "pq_gemm_wres.hip", "pq_stats.hip", "pq_noalloc.hip"]
# the quantizer's kernels, one translation unit per mode (PQ_W1_BINARY .. PQ_W158_LSQ)
MODE_SOURCE = "pq_quant_mode.hip"
NUM_MODES = 7
ARCH = "gfx950"
CFLAGS = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-command-line-argument"]


def _hipcc() -> str:
    for p in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if p and os.path.exists(p):
            return p
    return "hipcc"


def _compile(unit, verbose: bool) -> str:
    src, defines, tag = unit
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + tag + ".o")
    cmd = [_hipcc(), *CFLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32-ops feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src} {' '.join(defines)}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    units = [(s, [], "") for s in SOURCES]
    units += [(MODE_SOURCE, [f"-DPQ_QUANT_MODE={m}"], f"_{m}") for m in range(NUM_MODES)]
    workers = max(1, min(len(units), os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(lambda u: _compile(u, verbose), units))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
