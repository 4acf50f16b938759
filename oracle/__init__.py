"""CPU oracle for the ParetoQ quantized linear layer -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``libpq_oracle.so`` (plain C, built by
``oracle/build.py``) with numpy in/out arrays.  bf16 values are carried as
``numpy.uint16`` bit patterns.  See ``pq_oracle.c`` for the arithmetic and the
page citations of every step.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build as _build

BINARY, TERNARY, SEQ2, LSQ3, LSQ4, LSQ2, LSQ158 = 0, 1, 2, 3, 4, 5, 6
MODES = (BINARY, TERNARY, SEQ2, LSQ3, LSQ4, LSQ2, LSQ158)
CODE_BITS = {BINARY: 1, TERNARY: 2, SEQ2: 2, LSQ3: 4, LSQ4: 4, LSQ2: 2, LSQ158: 2}

_lib = None
_f32p = ctypes.POINTER(ctypes.c_float)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)
_i64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            _build()
        L = ctypes.CDLL(LIB)
        L.pqo_code_bits.argtypes = [ctypes.c_int]
        L.pqo_code_row_bytes.argtypes = [ctypes.c_int, _i64]
        L.pqo_code_row_bytes.restype = _i64
        L.pqo_clip_value.restype = ctypes.c_float
        L.pqo_bf16_rne.argtypes = [ctypes.c_float]
        L.pqo_bf16_rne.restype = ctypes.c_uint16
        L.pqo_seq2_quantize.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float, _f32p, _f32p]
        L.pqo_quantize_scalar.argtypes = [ctypes.c_int, ctypes.c_float, ctypes.c_float, _f32p, _f32p]
        L.pqo_alpha_init.argtypes = [ctypes.c_int, _i64, _i64, _f32p, _f32p]
        L.pqo_quantize_fwd.argtypes = [ctypes.c_int, _i64, _i64, _f32p, _f32p, _u16p, _f32p, _u8p]
        L.pqo_quantize_bwd.argtypes = [ctypes.c_int, _i64, _i64, _f32p, _f32p, ctypes.c_void_p,
                                       ctypes.c_int, ctypes.c_double, _f32p, _f32p, _u8p]
        L.pqo_default_grad_scale.argtypes = [ctypes.c_int, _i64, _i64]
        L.pqo_default_grad_scale.restype = ctypes.c_double
        L.pqo_pack.argtypes = [ctypes.c_int, _i64, _i64, _f32p, _f32p, _u8p, _u16p]
        L.pqo_gemm_ref.argtypes = [ctypes.c_int, _i64, _i64, _i64, _u16p, _u8p, _u16p, _f64p]
        L.pqo_gemm_ref_at.argtypes = [ctypes.c_int, _i64, _i64, _i64, _u16p, _u8p, _u16p,
                                      _i64p, _i64p, _i64, _f64p]
        L.pqo_tiled_bytes.argtypes = [_i64, _i64]
        L.pqo_tiled_bytes.restype = _i64
        L.pqo_tile_codes.argtypes = [ctypes.c_int, _i64, _i64, _u8p, _u8p]
        L.pqo_adamw.argtypes = [_i64, _f32p, _f32p, _f32p, _f32p] + [ctypes.c_double] * 5 + [_i64]
        L.pqo_qat_step.argtypes = ([ctypes.c_int, _i64, _i64, _f32p, _f32p, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_double, _f32p, _f32p, _f32p, _f32p] + [ctypes.c_double] * 5 +
                                   [_i64, _u16p, _u8p, _f32p])
        L.pqo_gemm_ref_f32a.argtypes = [ctypes.c_int, _i64, _i64, _i64, _u16p, _u8p, _f32p, _f64p]
        L.pqo_num_levels.argtypes = [ctypes.c_int]
        L.pqo_level_stats.argtypes = [ctypes.c_int, _i64, _i64, _u8p, ctypes.POINTER(ctypes.c_uint32), _f64p]
        L.pqo_weight_movement.argtypes = [_i64, _i64, _f32p, _f32p, _f64p, _f64p]
        L.pqo_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _p(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def _check(rc):
    if rc != 0:
        raise ValueError("oracle rejected its arguments")


def set_threads(n: int) -> None:
    lib().pqo_set_threads(int(n))


def max_threads() -> int:
    return int(lib().pqo_max_threads())


def code_row_bytes(mode: int, cols: int) -> int:
    return int(lib().pqo_code_row_bytes(mode, cols))


def clip_value() -> float:
    return float(lib().pqo_clip_value())


def bf16_rne(x):
    """bf16 bits (uint16) of each finite float32 in x, round-to-nearest-even."""
    x = np.asarray(x, dtype=np.float32)
    f = lib().pqo_bf16_rne
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def quantize_scalar(mode: int, w: float, alpha: float):
    """(r, q, x) for one weight: step index, binary32 fake-quant value, w/alpha."""
    q = ctypes.c_float()
    x = ctypes.c_float()
    r = lib().pqo_quantize_scalar(mode, ctypes.c_float(w), ctypes.c_float(alpha),
                                  ctypes.byref(q), ctypes.byref(x))
    return int(r), q.value, x.value


def seq2_scalar(w: float, alpha: float, clip: float):
    """2-bit SEQ formula with an explicit clip bound: (r, q)."""
    q = ctypes.c_float()
    r = lib().pqo_seq2_quantize(ctypes.c_float(w), ctypes.c_float(alpha), ctypes.c_float(clip),
                                ctypes.byref(q), None)
    return int(r), q.value


def alpha_init(mode: int, W: np.ndarray) -> np.ndarray:
    W = _c(W, np.float32)
    rows, cols = W.shape
    a = np.empty(rows, np.float32)
    _check(lib().pqo_alpha_init(mode, rows, cols, _p(W, _f32p), _p(a, _f32p)))
    return a


def quantize_fwd(mode: int, W: np.ndarray, alpha: np.ndarray):
    """Returns (wq_bf16 uint16 [rows,cols], wq_f32 [rows,cols], codes uint8 [rows,row_bytes])."""
    W = _c(W, np.float32)
    alpha = _c(alpha, np.float32)
    rows, cols = W.shape
    wq16 = np.empty((rows, cols), np.uint16)
    wq32 = np.empty((rows, cols), np.float32)
    codes = np.empty((rows, code_row_bytes(mode, cols)), np.uint8)
    _check(lib().pqo_quantize_fwd(mode, rows, cols, _p(W, _f32p), _p(alpha, _f32p),
                                  _p(wq16, _u16p), _p(wq32, _f32p), _p(codes, _u8p)))
    return wq16, wq32, codes


def default_grad_scale(mode: int, rows: int, cols: int) -> float:
    return float(lib().pqo_default_grad_scale(mode, rows, cols))


def quantize_bwd(mode: int, W: np.ndarray, alpha: np.ndarray, G: np.ndarray, grad_scale=None):
    """Returns (dW f32 [rows,cols], dalpha f32 [rows], mask_bits uint8 [rows, ceil(cols/8)]).

    G is float32, or uint16 bf16 bits."""
    W = _c(W, np.float32)
    alpha = _c(alpha, np.float32)
    G = np.ascontiguousarray(G)
    if G.dtype not in (np.float32, np.uint16):
        raise TypeError("G must be float32 or uint16 (bf16 bits)")
    rows, cols = W.shape
    if grad_scale is None:
        grad_scale = default_grad_scale(mode, rows, cols)
    dW = np.empty((rows, cols), np.float32)
    da = np.empty(rows, np.float32)
    mask = np.empty((rows, (cols + 7) // 8), np.uint8)
    _check(lib().pqo_quantize_bwd(mode, rows, cols, _p(W, _f32p), _p(alpha, _f32p),
                                  G.ctypes.data_as(ctypes.c_void_p), int(G.dtype == np.uint16),
                                  float(grad_scale), _p(dW, _f32p), _p(da, _f32p), _p(mask, _u8p)))
    return dW, da, mask


def pack(mode: int, W: np.ndarray, alpha: np.ndarray):
    """Export: (packed codes uint8 [rows, row_bytes], alpha bf16 bits uint16 [rows])."""
    W = _c(W, np.float32)
    alpha = _c(alpha, np.float32)
    rows, cols = W.shape
    packed = np.empty((rows, code_row_bytes(mode, cols)), np.uint8)
    ab = np.empty(rows, np.uint16)
    _check(lib().pqo_pack(mode, rows, cols, _p(W, _f32p), _p(alpha, _f32p),
                          _p(packed, _u8p), _p(ab, _u16p)))
    return packed, ab


ADAMW_DEFAULTS = dict(lr=2e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0)


def adamw(p, g, m, v, step, lr, beta1, beta2, eps, weight_decay):
    """AdamW on float32 arrays; returns updated copies (p, m, v)."""
    p, m, v = (np.array(a, dtype=np.float32, copy=True) for a in (p, m, v))
    g = _c(g, np.float32)
    _check(lib().pqo_adamw(p.size, _p(p, _f32p), _p(g, _f32p), _p(m, _f32p), _p(v, _f32p),
                           lr, beta1, beta2, eps, weight_decay, step))
    return p, m, v


def qat_step(mode: int, W, alpha, G, mW, vW, m_alpha, v_alpha, step, grad_scale=None,
             lr=2e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
    """Backward + AdamW + next forward.  Returns a dict of new arrays: W, alpha,
    mW, vW, m_alpha, v_alpha, wq_bf16, codes, dalpha."""
    W, alpha, mW, vW, m_alpha, v_alpha = (np.array(a, dtype=np.float32, copy=True)
                                          for a in (W, alpha, mW, vW, m_alpha, v_alpha))
    rows, cols = W.shape
    if grad_scale is None:
        grad_scale = default_grad_scale(mode, rows, cols)
    G = np.ascontiguousarray(G)
    wq = np.empty((rows, cols), np.uint16)
    codes = np.empty((rows, code_row_bytes(mode, cols)), np.uint8)
    da = np.empty(rows, np.float32)
    _check(lib().pqo_qat_step(mode, rows, cols, _p(W, _f32p), _p(alpha, _f32p),
                              G.ctypes.data_as(ctypes.c_void_p), int(G.dtype == np.uint16),
                              float(grad_scale), _p(mW, _f32p), _p(vW, _f32p), _p(m_alpha, _f32p),
                              _p(v_alpha, _f32p), lr, beta1, beta2, eps, weight_decay, step,
                              _p(wq, _u16p), _p(codes, _u8p), _p(da, _f32p)))
    return dict(W=W, alpha=alpha, mW=mW, vW=vW, m_alpha=m_alpha, v_alpha=v_alpha, wq_bf16=wq,
                codes=codes, dalpha=da)


def num_levels(mode: int) -> int:
    return int(lib().pqo_num_levels(mode))


def level_stats(mode: int, codes: np.ndarray, cols: int):
    """(counts uint32 [rows, levels], entropy float64 [rows]) of row-major codes."""
    codes = _c(codes, np.uint8)
    rows = codes.shape[0]
    counts = np.empty((rows, num_levels(mode)), np.uint32)
    ent = np.empty(rows, np.float64)
    _check(lib().pqo_level_stats(mode, rows, cols, _p(codes, _u8p),
                                 counts.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), _p(ent, _f64p)))
    return counts, ent


def weight_movement(W: np.ndarray, W0: np.ndarray):
    """(sum (W - W0)^2, sum W0^2) per row, binary64."""
    W, W0 = _c(W, np.float32), _c(W0, np.float32)
    rows, cols = W.shape
    d2, r2 = np.empty(rows, np.float64), np.empty(rows, np.float64)
    _check(lib().pqo_weight_movement(rows, cols, _p(W, _f32p), _p(W0, _f32p), _p(d2, _f64p), _p(r2, _f64p)))
    return d2, r2


def tiled_bytes(rows: int, row_bytes: int) -> int:
    return int(lib().pqo_tiled_bytes(rows, row_bytes))


def tile_codes(packed: np.ndarray, cw: int) -> np.ndarray:
    """Deployment byte order (flat uint8) of row-major rows [rows, rb] of
    cw-bit codes (2-bit codes are also reordered inside each 4-byte word)."""
    packed = _c(packed, np.uint8)
    rows, rb = packed.shape
    out = np.empty(tiled_bytes(rows, rb), np.uint8)
    _check(lib().pqo_tile_codes(cw, rows, rb, _p(packed, _u8p), _p(out, _u8p)))
    return out


def pack_tiled(mode: int, W: np.ndarray, alpha: np.ndarray):
    """Export in the deployment byte order: (tiled codes uint8 flat, alpha bf16 bits)."""
    packed, ab = pack(mode, W, alpha)
    return tile_codes(packed, CODE_BITS[mode]), ab


def gemm_ref(mode: int, X_bf16: np.ndarray, packed: np.ndarray, alpha_bf16: np.ndarray, N: int):
    """Binary64 Y [M,N] of the packed-weight GEMM."""
    X = _c(X_bf16, np.uint16)
    packed = _c(packed, np.uint8)
    ab = _c(alpha_bf16, np.uint16)
    M, K = X.shape
    Y = np.empty((M, N), np.float64)
    _check(lib().pqo_gemm_ref(mode, M, N, K, _p(X, _u16p), _p(packed, _u8p), _p(ab, _u16p),
                              _p(Y, _f64p)))
    return Y


def gemm_ref_f32a(mode: int, X_bf16: np.ndarray, packed: np.ndarray, alpha: np.ndarray, N: int):
    """Binary64 Y [M,N] with a binary32 scale per row."""
    X = _c(X_bf16, np.uint16)
    packed = _c(packed, np.uint8)
    alpha = _c(alpha, np.float32)
    M, K = X.shape
    Y = np.empty((M, N), np.float64)
    _check(lib().pqo_gemm_ref_f32a(mode, M, N, K, _p(X, _u16p), _p(packed, _u8p), _p(alpha, _f32p),
                                   _p(Y, _f64p)))
    return Y


def gemm_ref_at(mode: int, X_bf16, packed, alpha_bf16, N: int, ms, ns):
    """Binary64 Y[ms[t], ns[t]] for each t."""
    X = _c(X_bf16, np.uint16)
    packed = _c(packed, np.uint8)
    ab = _c(alpha_bf16, np.uint16)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    M, K = X.shape
    out = np.empty(len(ms), np.float64)
    _check(lib().pqo_gemm_ref_at(mode, M, N, K, _p(X, _u16p), _p(packed, _u8p), _p(ab, _u16p),
                                 _p(ms, _i64p), _p(ns, _i64p), len(ms), _p(out, _f64p)))
    return out
