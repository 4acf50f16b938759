"""Thin Python binding of libpq (the C ABI in include/pq.h).

Argument marshalling only: every function here turns torch tensors into
device pointers and calls the C entry point of the same name; all of the
computation runs in libpq's HIP kernels.  Importing this module loads
``libpq.so`` and raises if it has not been built -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpq.so")

PQ_W1_BINARY, PQ_W158_SEQ_TERNARY, PQ_W2_SEQ, PQ_W3_LSQ, PQ_W4_LSQ = 0, 1, 2, 3, 4
PQ_W2_LSQ, PQ_W158_LSQ = 5, 6  # the LSQ ablation grids at 2 and 1.58 bits
MODES = (PQ_W1_BINARY, PQ_W158_SEQ_TERNARY, PQ_W2_SEQ, PQ_W3_LSQ, PQ_W4_LSQ, PQ_W2_LSQ, PQ_W158_LSQ)
MODE_NAMES = {PQ_W1_BINARY: "w1_binary", PQ_W158_SEQ_TERNARY: "w1.58_ternary",
              PQ_W2_SEQ: "w2_seq", PQ_W3_LSQ: "w3_lsq", PQ_W4_LSQ: "w4_lsq", PQ_W2_LSQ: "w2_lsq",
              PQ_W158_LSQ: "w1.58_lsq"}
CODE_BITS = {PQ_W1_BINARY: 1, PQ_W158_SEQ_TERNARY: 2, PQ_W2_SEQ: 2, PQ_W3_LSQ: 4, PQ_W4_LSQ: 4,
             PQ_W2_LSQ: 2, PQ_W158_LSQ: 2}
PQ_INIT_ALPHA = 1
PQ_G_F32, PQ_G_BF16 = 0, 1
STATUS = {0: "PQ_OK", 1: "PQ_ERR_NULL", 2: "PQ_ERR_SHAPE", 3: "PQ_ERR_MODE", 4: "PQ_ERR_ALIGN",
          5: "PQ_ERR_UNSUPPORTED", 6: "PQ_ERR_HIP", 7: "PQ_ERR_ARG"}

# Every symbol include/pq.h declares.
EXPORTS = ("pq_code_row_bytes", "pq_packed_bytes", "pq_default_grad_scale", "pq_status_str", "pq_version",
           "pq_gemm_workspace_bytes",
           "pq_quantize_fwd", "pq_quantize_bwd", "pq_pack_w2", "pq_pack_w4", "pq_w2a16_gemm",
           "pq_w4a16_gemm", "pq_quantize_fwd_grouped", "pq_quantize_bwd_grouped", "pq_qat_step",
           "pq_qat_step_grouped", "pq_pack", "pq_gemm", "pq_gemm_f32a", "pq_num_levels", "pq_level_stats",
           "pq_quantize_fwd_stats", "pq_weight_movement", "pq_pack_grouped", "pq_gemm_noalloc")


class PQError(RuntimeError):
    def __init__(self, status: int, fn: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)}")
        self.status = status


class pq_mat(ctypes.Structure):
    """Mirror of `struct pq_mat` in include/pq.h."""
    _fields_ = [("W", ctypes.c_void_p), ("alpha", ctypes.c_void_p), ("wq_bf16", ctypes.c_void_p),
                ("wq_f32", ctypes.c_void_p), ("codes", ctypes.c_void_p), ("G", ctypes.c_void_p),
                ("dW", ctypes.c_void_p), ("dalpha", ctypes.c_void_p), ("mask_bits", ctypes.c_void_p),
                ("grad_scale", ctypes.c_double), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("alpha_bf16", ctypes.c_void_p)]


class pq_adamw(ctypes.Structure):
    """Mirror of `struct pq_adamw` in include/pq.h."""
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("step", ctypes.c_int64)]


class pq_step_mat(ctypes.Structure):
    """Mirror of `struct pq_step_mat` in include/pq.h."""
    _fields_ = [("W", ctypes.c_void_p), ("alpha", ctypes.c_void_p), ("G", ctypes.c_void_p),
                ("mW", ctypes.c_void_p), ("vW", ctypes.c_void_p), ("m_alpha", ctypes.c_void_p),
                ("v_alpha", ctypes.c_void_p), ("wq_bf16", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("dalpha", ctypes.c_void_p), ("grad_scale", ctypes.c_double), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    i64, vp, u32, dbl = ctypes.c_int64, ctypes.c_void_p, ctypes.c_uint, ctypes.c_double
    i32 = ctypes.c_int
    L.pq_code_row_bytes.argtypes = [i32, i64]
    L.pq_code_row_bytes.restype = i64
    L.pq_packed_bytes.argtypes = [i32, i64, i64]
    L.pq_packed_bytes.restype = i64
    L.pq_default_grad_scale.argtypes = [i32, i64, i64]
    L.pq_default_grad_scale.restype = dbl
    L.pq_status_str.argtypes = [i32]
    L.pq_status_str.restype = ctypes.c_char_p
    L.pq_version.restype = ctypes.c_char_p
    L.pq_quantize_fwd.argtypes = [i32, i64, i64, vp, vp, u32, vp, vp, vp, vp]
    L.pq_quantize_bwd.argtypes = [i32, i64, i64, vp, vp, vp, i32, dbl, vp, vp, vp, vp]
    L.pq_pack_w2.argtypes = [i64, i64, vp, vp, vp, vp, vp]
    L.pq_pack_w4.argtypes = [i64, i64, vp, vp, vp, vp, vp]
    L.pq_gemm_workspace_bytes.argtypes = [i32, i64, i64, i64]
    L.pq_gemm_workspace_bytes.restype = i64
    L.pq_w2a16_gemm.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, i64, vp]
    L.pq_w4a16_gemm.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp, i64, vp]
    L.pq_pack.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp]
    L.pq_gemm.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, i64, vp]
    L.pq_gemm_f32a.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp, i64, vp]
    L.pq_gemm_noalloc.argtypes = [i32, i64, i64, i64, vp, vp, vp, vp, vp]
    L.pq_num_levels.argtypes = [i32]
    L.pq_num_levels.restype = i32
    L.pq_level_stats.argtypes = [i32, i64, i64, vp, vp, vp, vp]
    L.pq_quantize_fwd_stats.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, vp, vp]
    L.pq_weight_movement.argtypes = [i64, i64, vp, vp, vp, vp, vp]
    L.pq_quantize_fwd_grouped.argtypes = [i32, i32, vp, vp, u32, vp]
    L.pq_quantize_bwd_grouped.argtypes = [i32, i32, vp, vp, i32, vp]
    L.pq_pack_grouped.argtypes = [i32, i32, vp, vp, vp]
    L.pq_qat_step.argtypes = [i32, i64, i64, vp, vp, vp, i32, dbl, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.pq_qat_step_grouped.argtypes = [i32, i32, vp, vp, i32, vp, vp]
    for name in EXPORTS:
        if name not in ("pq_code_row_bytes", "pq_packed_bytes", "pq_default_grad_scale", "pq_status_str",
                        "pq_version", "pq_num_levels", "pq_gemm_workspace_bytes"):
            getattr(L, name).restype = i32
    return L


lib = _load()


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, fn: str) -> None:
    if rc != 0:
        raise PQError(rc, fn)


def pq_code_row_bytes(mode: int, cols: int) -> int:
    return int(lib.pq_code_row_bytes(mode, cols))


def pq_packed_bytes(mode: int, rows: int, cols: int) -> int:
    return int(lib.pq_packed_bytes(mode, rows, cols))


def pq_default_grad_scale(mode: int, rows: int, cols: int) -> float:
    return float(lib.pq_default_grad_scale(mode, rows, cols))


def pq_status_str(status: int) -> str:
    return lib.pq_status_str(status).decode()


def pq_version() -> str:
    return lib.pq_version().decode()


def pq_quantize_fwd(mode, rows, cols, W, alpha, flags=0, Wq_bf16=None, Wq_f32=None, codes=None,
                    stream=None) -> None:
    _check(lib.pq_quantize_fwd(mode, rows, cols, _ptr(W), _ptr(alpha), flags, _ptr(Wq_bf16),
                               _ptr(Wq_f32), _ptr(codes), _stream(stream)), "pq_quantize_fwd")


def pq_quantize_bwd(mode, rows, cols, W, alpha, G, g_dtype, grad_scale, dW, dalpha,
                    mask_bits=None, stream=None) -> None:
    _check(lib.pq_quantize_bwd(mode, rows, cols, _ptr(W), _ptr(alpha), _ptr(G), g_dtype,
                               float(grad_scale), _ptr(dW), _ptr(dalpha), _ptr(mask_bits),
                               _stream(stream)), "pq_quantize_bwd")


def pq_pack_w2(rows, cols, W, alpha, packed, alpha_bf16, stream=None) -> None:
    _check(lib.pq_pack_w2(rows, cols, _ptr(W), _ptr(alpha), _ptr(packed), _ptr(alpha_bf16),
                          _stream(stream)), "pq_pack_w2")


def pq_pack_w4(rows, cols, W, alpha, packed, alpha_bf16, stream=None) -> None:
    _check(lib.pq_pack_w4(rows, cols, _ptr(W), _ptr(alpha), _ptr(packed), _ptr(alpha_bf16),
                          _stream(stream)), "pq_pack_w4")


def pq_gemm_workspace_bytes(mode: int, M: int, N: int, K: int) -> int:
    return int(lib.pq_gemm_workspace_bytes(mode, M, N, K))


def gemm_workspace(mode: int, M: int, N: int, K: int, device="cuda") -> Optional[torch.Tensor]:
    """A device buffer of pq_gemm_workspace_bytes(mode, M, N, K) bytes (None
    when the shape needs none), allocated by torch for the caller to keep."""
    n = pq_gemm_workspace_bytes(mode, M, N, K)
    if n < 0:
        raise PQError(2, "pq_gemm_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device) if n > 0 else None


def _ws(mode, M, N, K, X, workspace, stream):
    """(pointer, size, tensor) of the caller's workspace, or of one allocated
    here from torch's caching allocator.  A buffer allocated here is marked
    as used by the launch stream, so torch hands it out again only after the
    GEMM on that stream is done with it."""
    if workspace is None:
        dev = X.device if isinstance(X, torch.Tensor) else "cuda"
        workspace = gemm_workspace(mode, M, N, K, dev)
        if workspace is None:
            return None, 0, None
        if stream is not None:
            s = torch.cuda.ExternalStream(stream) if isinstance(stream, int) else stream
            workspace.record_stream(s)
    if isinstance(workspace, tuple):        # (pointer, bytes) from a caller that keeps its own buffer
        return workspace[0], int(workspace[1]), None
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace


def pq_w2a16_gemm(M, N, K, X, packed, alpha_bf16, Y, stream=None, workspace=None) -> None:
    wp, wb, _keep = _ws(PQ_W2_SEQ, M, N, K, X, workspace, stream)
    _check(lib.pq_w2a16_gemm(M, N, K, _ptr(X), _ptr(packed), _ptr(alpha_bf16), _ptr(Y), wp, wb,
                             _stream(stream)), "pq_w2a16_gemm")


def pq_w4a16_gemm(M, N, K, X, packed, alpha_bf16, Y, stream=None, workspace=None) -> None:
    wp, wb, _keep = _ws(PQ_W4_LSQ, M, N, K, X, workspace, stream)
    _check(lib.pq_w4a16_gemm(M, N, K, _ptr(X), _ptr(packed), _ptr(alpha_bf16), _ptr(Y), wp, wb,
                             _stream(stream)), "pq_w4a16_gemm")


def pq_pack(mode, rows, cols, W, alpha, packed, alpha_bf16, stream=None) -> None:
    _check(lib.pq_pack(mode, rows, cols, _ptr(W), _ptr(alpha), _ptr(packed), _ptr(alpha_bf16),
                       _stream(stream)), "pq_pack")


def pq_gemm(mode, M, N, K, X, packed, alpha_bf16, Y, stream=None, workspace=None) -> None:
    wp, wb, _keep = _ws(mode, M, N, K, X, workspace, stream)
    _check(lib.pq_gemm(mode, M, N, K, _ptr(X), _ptr(packed), _ptr(alpha_bf16), _ptr(Y), wp, wb,
                       _stream(stream)), "pq_gemm")


def pq_gemm_f32a(mode, M, N, K, X, packed, alpha, Y, stream=None, workspace=None) -> None:
    wp, wb, _keep = _ws(mode, M, N, K, X, workspace, stream)
    _check(lib.pq_gemm_f32a(mode, M, N, K, _ptr(X), _ptr(packed), _ptr(alpha), _ptr(Y), wp, wb,
                            _stream(stream)), "pq_gemm_f32a")


PQ_NOALLOC_SCRATCH_BYTES = 32 << 20


def pq_gemm_noalloc(mode, M, N, K, X, packed, alpha_bf16, Y, stream=None) -> None:
    """pq_gemm with the library's fixed scratch instead of a workspace."""
    _check(lib.pq_gemm_noalloc(mode, M, N, K, _ptr(X), _ptr(packed), _ptr(alpha_bf16), _ptr(Y),
                               _stream(stream)), "pq_gemm_noalloc")


PQ_CODES_EXPORT = 2


def pq_num_levels(mode: int) -> int:
    return int(lib.pq_num_levels(mode))


def pq_level_stats(mode, rows, cols, codes, counts, entropy=None, stream=None) -> None:
    _check(lib.pq_level_stats(mode, rows, cols, _ptr(codes), _ptr(counts), _ptr(entropy), _stream(stream)),
           "pq_level_stats")


def pq_quantize_fwd_stats(mode, rows, cols, W, alpha, Wq_bf16, codes, counts, entropy=None,
                          stream=None) -> None:
    _check(lib.pq_quantize_fwd_stats(mode, rows, cols, _ptr(W), _ptr(alpha), _ptr(Wq_bf16), _ptr(codes),
                                     _ptr(counts), _ptr(entropy), _stream(stream)), "pq_quantize_fwd_stats")


def pq_weight_movement(rows, cols, W, W0, sq_diff, sq_ref, stream=None) -> None:
    _check(lib.pq_weight_movement(rows, cols, _ptr(W), _ptr(W0), _ptr(sq_diff), _ptr(sq_ref), _stream(stream)),
           "pq_weight_movement")


class MatTable:
    """A pq_mat[] descriptor table in host memory plus its device copy.

    Build it once per stack of matrices and pass it to the grouped calls;
    it keeps the device copy (a torch uint8 tensor) alive."""

    STRUCT = pq_mat
    POINTERS = ("W", "alpha", "wq_bf16", "wq_f32", "codes", "G", "dW", "dalpha", "mask_bits", "alpha_bf16")

    def __init__(self, mats: Sequence[dict], device="cuda"):
        n = len(mats)
        self.count = n
        self.host = (self.STRUCT * max(n, 1))()
        for i, m in enumerate(mats):
            d = self.host[i]
            for f in self.POINTERS:
                setattr(d, f, _ptr(m.get(f)))
            d.grad_scale = float(m.get("grad_scale", 0.0))
            d.rows = int(m["rows"])
            d.cols = int(m["cols"])
        raw = bytes(memoryview(self.host).cast("B"))[: n * ctypes.sizeof(self.STRUCT)]
        self.dev = torch.frombuffer(bytearray(raw) or bytearray(1), dtype=torch.uint8).to(device)

    @property
    def host_ptr(self) -> int:
        return ctypes.addressof(self.host)

    @property
    def dev_ptr(self) -> int:
        return self.dev.data_ptr()


def pq_quantize_fwd_grouped(mode, table: MatTable, flags=0, stream=None) -> None:
    _check(lib.pq_quantize_fwd_grouped(mode, table.count, table.host_ptr, table.dev_ptr, flags,
                                       _stream(stream)), "pq_quantize_fwd_grouped")


def pq_quantize_bwd_grouped(mode, table: MatTable, g_dtype=PQ_G_F32, stream=None) -> None:
    _check(lib.pq_quantize_bwd_grouped(mode, table.count, table.host_ptr, table.dev_ptr, g_dtype,
                                       _stream(stream)), "pq_quantize_bwd_grouped")


def pq_pack_grouped(mode, table: MatTable, stream=None) -> None:
    _check(lib.pq_pack_grouped(mode, table.count, table.host_ptr, table.dev_ptr, _stream(stream)),
           "pq_pack_grouped")


class StepTable(MatTable):
    """A pq_step_mat[] descriptor table (host + device copy) for the fused step."""

    STRUCT = pq_step_mat
    POINTERS = ("W", "alpha", "G", "mW", "vW", "m_alpha", "v_alpha", "wq_bf16", "codes", "dalpha")


def adamw_params(step, lr=2e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0) -> pq_adamw:
    return pq_adamw(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay), int(step))


def pq_qat_step(mode, rows, cols, W, alpha, G, g_dtype, grad_scale, mW, vW, m_alpha, v_alpha,
                hp: pq_adamw, Wq_bf16=None, codes=None, dalpha=None, stream=None) -> None:
    _check(lib.pq_qat_step(mode, rows, cols, _ptr(W), _ptr(alpha), _ptr(G), g_dtype, float(grad_scale),
                           _ptr(mW), _ptr(vW), _ptr(m_alpha), _ptr(v_alpha), ctypes.addressof(hp),
                           _ptr(Wq_bf16), _ptr(codes), _ptr(dalpha), _stream(stream)), "pq_qat_step")


def pq_qat_step_grouped(mode, table: StepTable, hp: pq_adamw, g_dtype=PQ_G_F32, stream=None) -> None:
    _check(lib.pq_qat_step_grouped(mode, table.count, table.host_ptr, table.dev_ptr, g_dtype,
                                   ctypes.addressof(hp), _stream(stream)), "pq_qat_step_grouped")
