"""The C ABI without a GPU: the library loads, exports every symbol that
include/pq.h declares, and rejects bad arguments on the host (nothing is
enqueued, so no device is needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def pq():
    from bit_quantization_aware_amd import pq as _pq
    return _pq


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pq_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(pq):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(pq.lib, n), n
    assert set(names) == set(pq.EXPORTS)


def test_header_constants_match_binding(pq):
    """The sizes pq.h defines are the ones the binding uses."""
    src = open(os.path.join(ROOT, "include", "pq.h")).read()
    for name, value in {"PQ_NOALLOC_SCRATCH_BYTES": pq.PQ_NOALLOC_SCRATCH_BYTES}.items():
        m = re.search(r"#define\s+" + name + r"\s+(.+)", src)
        assert m, name
        expr = re.sub(r"\(\s*int64_t\s*\)", "", m.group(1))
        assert eval(expr, {}) == value, name


def test_struct_layout(pq):
    assert ctypes.sizeof(pq.pq_mat) == 104
    assert pq.pq_mat.alpha_bf16.offset == 96
    assert ctypes.sizeof(pq.pq_step_mat) == 104
    assert ctypes.sizeof(pq.pq_adamw) == 48


def test_helpers(pq):
    assert pq.pq_code_row_bytes(pq.PQ_W2_SEQ, 64) == 16
    assert pq.pq_code_row_bytes(pq.PQ_W1_BINARY, 64) == 8
    assert pq.pq_code_row_bytes(pq.PQ_W4_LSQ, 64) == 32
    assert pq.pq_code_row_bytes(9, 64) == -1
    # export size: 64-byte groups of every row, rows rounded up to 16
    assert pq.pq_packed_bytes(pq.PQ_W2_SEQ, 16384, 16384) == 16384 * 4096
    assert pq.pq_packed_bytes(pq.PQ_W2_SEQ, 20, 576) == 3 * 32 * 64
    assert pq.pq_packed_bytes(pq.PQ_W4_LSQ, 1, 8) == 16 * 64
    assert pq.pq_packed_bytes(pq.PQ_W2_SEQ, 0, 64) == 0
    assert pq.pq_packed_bytes(pq.PQ_W1_BINARY, 16, 64) == 16 * 64          # 8 bytes of a row: one group
    assert pq.pq_packed_bytes(pq.PQ_W1_BINARY, 16384, 16384) == 32 * 16384 * 64
    assert pq.pq_packed_bytes(7, 16, 64) == -1
    assert pq.pq_packed_bytes(pq.PQ_W158_SEQ_TERNARY, 16, 1024) == 16 * 256
    assert pq.pq_packed_bytes(pq.PQ_W3_LSQ, 16, 1024) == 16 * 512
    assert pq.pq_packed_bytes(pq.PQ_W2_SEQ, 16, 12) == -1
    assert pq.pq_default_grad_scale(pq.PQ_W4_LSQ, 4, 16) == pytest.approx((4 * 16 * 7) ** -0.5)
    assert pq.pq_default_grad_scale(pq.PQ_W2_SEQ, 0, 16) == 0.0
    assert [pq.pq_num_levels(m) for m in range(7)] == [2, 3, 4, 8, 16, 4, 3] and pq.pq_num_levels(7) == -1
    assert "NULL" in pq.pq_status_str(1)
    assert "gfx950" in pq.pq_version()


A = 0x100000          # fake, 16-byte aligned device addresses: never dereferenced,
B = 0x200000          # because every call below fails validation first
MIS = 0x100004        # not 16-byte aligned


def rc(fn, *args):
    return fn(*args)


def test_fwd_argument_checks(pq):
    L = pq.lib
    assert L.pq_quantize_fwd(2, 4, 64, None, A, 0, B, None, None, None) == 1      # W NULL
    assert L.pq_quantize_fwd(2, 4, 64, A, None, 0, B, None, None, None) == 1      # alpha NULL
    assert L.pq_quantize_fwd(2, 4, 60, A, B, 0, B, None, None, None) == 2         # cols % 8
    assert L.pq_quantize_fwd(2, 4, 0, A, B, 0, B, None, None, None) == 2          # cols 0
    assert L.pq_quantize_fwd(2, -1, 64, A, B, 0, B, None, None, None) == 2        # rows < 0
    assert L.pq_quantize_fwd(7, 4, 64, A, B, 0, B, None, None, None) == 3         # mode
    assert L.pq_quantize_fwd(2, 4, 64, A, B, 4, B, None, None, None) == 3         # flag
    assert L.pq_quantize_fwd(2, 4, 64, MIS, B, 0, B, None, None, None) == 4       # align
    assert L.pq_quantize_fwd(2, 4, 64, A, B, 0, MIS, None, None, None) == 4
    assert L.pq_quantize_fwd(2, 0, 64, A, B, 0, B, None, None, None) == 0         # empty: no-op


def test_bwd_argument_checks(pq):
    L = pq.lib
    ok = (2, 4, 64, A, B, A, 0, 1.0, B, B, None, None)
    args = list(ok)
    args[5] = None
    assert L.pq_quantize_bwd(*args) == 1                                         # G NULL
    args = list(ok)
    args[9] = None
    assert L.pq_quantize_bwd(*args) == 1                                         # dalpha NULL
    args = list(ok)
    args[6] = 5
    assert L.pq_quantize_bwd(*args) == 3                                         # g dtype
    args = list(ok)
    args[7] = float("nan")
    assert L.pq_quantize_bwd(*args) == 7                                         # grad_scale
    args = list(ok)
    args[6], args[8] = 1, A
    assert L.pq_quantize_bwd(*args) == 7                                         # bf16 G aliased
    args = list(ok)
    args[5] = MIS
    assert L.pq_quantize_bwd(*args) == 4
    args = list(ok)
    args[1] = 0
    assert L.pq_quantize_bwd(*args) == 0                                         # empty


def test_pack_and_gemm_argument_checks(pq):
    L = pq.lib
    assert L.pq_pack_w2(4, 64, None, A, B, A, None) == 1
    assert L.pq_pack_w2(4, 12, A, A, B, A, None) == 2
    assert L.pq_pack_w4(4, 64, A, A, MIS, A, None) == 4
    # pq_w2a16_gemm(M, N, K, X, packed, alpha_bf16, Y, workspace, workspace_bytes, stream)
    assert L.pq_w2a16_gemm(4, 8, 64, None, A, B, A, None, 0, None) == 1
    assert L.pq_w2a16_gemm(4, 8, 60, A, A, B, A, None, 0, None) == 2
    assert L.pq_w2a16_gemm(4, 8, 72, A, A, B, A, None, 0, None) == 2                 # K % 64
    assert L.pq_w2a16_gemm(-1, 8, 64, A, A, B, A, None, 0, None) == 2
    assert L.pq_w4a16_gemm(4, 8, 64, A, MIS, B, A, None, 0, None) == 4
    assert L.pq_w2a16_gemm(0, 8, 64, A, A, B, A, None, 0, None) == 0                 # empty
    assert L.pq_w2a16_gemm(1, (1 << 24) + 16, 64, A, A, B, A, None, 0, None) == 2    # N bound
    assert L.pq_w2a16_gemm(4, 8, 64, A, A, B, A, None, -1, None) == 7                # negative size
    assert L.pq_pack_w2(0, 64, A, A, B, A, None) == 0                                # empty
    assert L.pq_pack(7, 4, 64, A, A, B, A, None) == 3                                # bad mode
    assert L.pq_gemm(7, 4, 8, 64, A, A, B, A, None, 0, None) == 3
    assert L.pq_gemm(1, 4, 8, 60, A, A, B, A, None, 0, None) == 2                    # ternary, K % 64
    assert L.pq_pack(3, 4, 60, A, A, B, A, None) == 2
    assert L.pq_gemm_f32a(2, 4, 8, 64, A, A, None, A, None, 0, None) == 1            # alpha NULL
    assert L.pq_gemm_f32a(7, 4, 8, 64, A, A, B, A, None, 0, None) == 3
    # forward with codes in the export byte order: deployable widths, codes required
    assert L.pq_quantize_fwd(7, 4, 64, A, B, 2, None, None, A, None) == 3
    assert L.pq_quantize_fwd(2, 4, 64, A, B, 2, A, None, None, None) == 1
    assert L.pq_quantize_fwd(2, 4, 64, A, B, 4, None, None, A, None) == 3            # unknown flag


def test_gemm_workspace_size_query(pq):
    """The size query follows the kernel choice: none for the weight-streaming
    path (M <= 16), split-K partials when the tiled path splits K, the
    none for the large-M 2-bit path; -1 for bad arguments."""
    q = pq.pq_gemm_workspace_bytes
    for mode in range(7):
        for M in (1, 4, 16):
            assert q(mode, M, 16384, 16384) == 0
    assert q(7, 1, 64, 64) == -1 and q(2, 1, 64, 60) == -1 and q(2, -1, 64, 64) == -1
    assert q(2, 0, 64, 64) == 0 and q(2, 64, 0, 64) == 0
    # 64 x 16384 output: 64 tiles of 64 x 256 do not fill the chip, so K is
    # split over blocks, each split writing fp32 partials [M, N]
    for mode in (2, 4):
        ws = q(mode, 64, 16384, 16384)
        assert ws > 0 and ws % (64 * 16384 * 4) == 0 and ws // (64 * 16384 * 4) >= 2
    # 1024 rows at K >= 2048: the large-M path sums the activation rows itself
    assert q(2, 1024, 8192, 2048) == 0
    assert q(2, 1100, 8200, 2112) == 0
    # a chip-filling tiled grid needs nothing
    assert q(4, 4096, 16384, 256) == 0


def test_gemm_workspace_checks(pq):
    """A shape that needs a workspace rejects a missing, misaligned or short
    one before anything is enqueued."""
    L = pq.lib
    M, N, K = 64, 16384, 16384
    ws = pq.pq_gemm_workspace_bytes(2, M, N, K)
    assert ws > 0
    assert L.pq_w2a16_gemm(M, N, K, A, A, B, A, None, 0, None) == 1                  # missing
    assert L.pq_w2a16_gemm(M, N, K, A, A, B, A, None, ws, None) == 1
    assert L.pq_w2a16_gemm(M, N, K, A, A, B, A, MIS, ws, None) == 4                  # misaligned
    assert L.pq_w2a16_gemm(M, N, K, A, A, B, A, B, ws - 16, None) == 7               # too small
    assert L.pq_gemm_f32a(2, M, N, K, A, A, B, A, None, 0, None) == 1
    assert L.pq_gemm(2, 256, 4096, 4096, A, A, B, A, None, 0, None) == 1             # tiled split-K
    assert L.pq_gemm(2, 256, 4096, 4096, A, A, B, A, B, pq.pq_gemm_workspace_bytes(2, 256, 4096, 4096) - 16,
                     None) == 7


def test_library_holds_no_allocator():
    """The GEMM sources call no device allocator and keep no per-stream cache."""
    csrc = os.path.join(ROOT, "bit_quantization_aware_amd", "csrc")
    for f in os.listdir(csrc):
        src = open(os.path.join(csrc, f)).read()
        for word in ("hipMalloc", "hipFree", "hipStreamSynchronize", "std::map", "std::mutex"):
            assert word not in src, (f, word)


def test_grouped_argument_checks(pq):
    L = pq.lib
    mats = (pq.pq_mat * 2)()
    mats[0].W, mats[0].alpha, mats[0].rows, mats[0].cols = A, B, 4, 64
    mats[1].W, mats[1].alpha, mats[1].rows, mats[1].cols = A, B, 4, 60
    h = ctypes.addressof(mats)
    assert L.pq_quantize_fwd_grouped(2, 2, h, A, 0, None) == 2                    # cols % 8
    mats[1].cols = 64
    mats[1].wq_bf16 = B
    assert L.pq_quantize_fwd_grouped(2, 2, h, A, 0, None) == 7                    # mixed outputs
    assert L.pq_quantize_fwd_grouped(2, 2, h, None, 0, None) == 7 or \
        L.pq_quantize_fwd_grouped(2, 2, h, None, 0, None) == 1
    assert L.pq_quantize_fwd_grouped(2, -1, h, A, 0, None) == 7
    assert L.pq_quantize_fwd_grouped(2, 0, None, None, 0, None) == 0              # empty stack
    assert L.pq_quantize_bwd_grouped(2, 2, h, A, 0, None) == 1                    # G NULL
    # grouped export: codes and alpha_bf16 required per matrix
    assert L.pq_pack_grouped(2, 2, h, A, None) == 1
    for m in mats:
        m.codes, m.alpha_bf16 = A, B
    assert L.pq_pack_grouped(7, 2, h, A, None) == 3                               # not deployable
    assert L.pq_pack_grouped(2, 2, h, None, None) == 1                            # no device table
    mats[1].alpha_bf16 = MIS
    assert L.pq_pack_grouped(2, 2, h, A, None) == 4
    mats[1].cols = 12
    assert L.pq_pack_grouped(2, 2, h, A, None) == 2
    assert L.pq_pack_grouped(2, 0, None, None, None) == 0                         # empty stack


def test_qat_step_argument_checks(pq):
    L = pq.lib
    hp = pq.adamw_params(1)
    H = ctypes.addressof(hp)
    ok = [2, 4, 64, A, B, A, 0, 1.0, A, B, A, B, H, None, None, None, None]
    args = list(ok)
    args[12] = None
    assert L.pq_qat_step(*args) == 1                                              # hp NULL
    args = list(ok)
    args[8] = None
    assert L.pq_qat_step(*args) == 1                                              # mW NULL
    args = list(ok)
    args[2] = 60
    assert L.pq_qat_step(*args) == 2                                              # cols % 8
    args = list(ok)
    args[0] = 7
    assert L.pq_qat_step(*args) == 3                                              # mode
    args = list(ok)
    args[9] = MIS
    assert L.pq_qat_step(*args) == 4                                              # vW aligned
    args = list(ok)
    args[7] = float("nan")
    assert L.pq_qat_step(*args) == 7                                              # grad_scale
    for field, bad in (("step", 0), ("beta1", 1.0), ("beta2", -0.1), ("eps", 0.0), ("lr", float("inf")),
                       ("weight_decay", -1.0)):
        h2 = pq.adamw_params(1)
        setattr(h2, field, bad)
        args = list(ok)
        args[12] = ctypes.addressof(h2)
        assert L.pq_qat_step(*args) == 7, field
    args = list(ok)
    args[1] = 0
    assert L.pq_qat_step(*args) == 0                                              # empty
    mats = (pq.pq_step_mat * 2)()
    for m in mats:
        m.W, m.alpha, m.G, m.mW, m.vW, m.m_alpha, m.v_alpha = A, B, A, B, A, B, A
        m.rows, m.cols, m.grad_scale = 4, 64, 1.0
    mats[1].codes = B
    assert L.pq_qat_step_grouped(2, 2, ctypes.addressof(mats), A, 0, H, None) == 7  # mixed outputs
    assert L.pq_qat_step_grouped(2, 0, None, None, 0, H, None) == 0                # empty stack


def test_diagnostics_argument_checks(pq):
    L = pq.lib
    assert L.pq_level_stats(7, 4, 64, A, B, None, None) == 3
    assert L.pq_level_stats(2, 4, 60, A, B, None, None) == 2
    assert L.pq_level_stats(2, 4, 64, None, B, None, None) == 1
    assert L.pq_level_stats(2, 0, 64, None, None, None, None) == 0               # empty
    # pq_quantize_fwd_stats(mode, rows, cols, W, alpha, Wq_bf16, codes, counts, entropy, stream)
    assert L.pq_quantize_fwd_stats(7, 4, 64, A, B, None, A, B, None, None) == 3
    assert L.pq_quantize_fwd_stats(2, 4, 60, A, B, None, A, B, None, None) == 2
    assert L.pq_quantize_fwd_stats(2, 4, 64, A, B, None, None, B, None, None) == 1   # codes required
    assert L.pq_quantize_fwd_stats(2, 4, 64, A, B, None, A, None, None, None) == 1   # counts required
    assert L.pq_quantize_fwd_stats(2, 4, 64, A, B, None, A, MIS, None, None) == 4
    assert L.pq_quantize_fwd_stats(2, 4, 64, None, B, None, A, B, None, None) == 1
    assert L.pq_quantize_fwd_stats(2, 0, 64, None, None, None, None, None, None, None) == 0  # empty
    assert L.pq_weight_movement(4, 64, A, MIS, A, B, None) == 4
    assert L.pq_weight_movement(4, 64, A, B, None, B, None) == 1
    assert L.pq_weight_movement(-1, 64, A, B, A, B, None) == 2


def test_launch_failure_reports_pq_err_hip(pq):
    """With no usable device the launch itself fails, and every entry point
    reports PQ_ERR_HIP instead of pretending success.  Runs only where no GPU
    is visible: the fake addresses below would otherwise reach a kernel."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: this check needs a host without one")
    L = pq.lib
    assert L.pq_quantize_fwd(2, 4, 64, A, B, 0, B, None, None, None) == 6
    assert L.pq_quantize_bwd(2, 4, 64, A, B, A, 0, 1.0, B, B, None, None) == 6
    assert L.pq_pack_w2(4, 64, A, A, B, A, None) == 6
    assert L.pq_w2a16_gemm(1, 64, 64, A, A, B, A, None, 0, None) == 6
    assert L.pq_w2a16_gemm(64, 16384, 16384, A, A, B, A, B, 1 << 30, None) == 6


def test_gemm_noalloc_argument_checks(pq):
    """pq_gemm_noalloc validates like pq_gemm and rejects, before anything
    is enqueued, a shape whose scratch need exceeds the library's array."""
    L = pq.lib
    assert pq.PQ_NOALLOC_SCRATCH_BYTES == 32 << 20
    assert L.pq_gemm_noalloc(7, 4, 8, 64, A, A, B, A, None) == 3                    # mode
    assert L.pq_gemm_noalloc(2, 4, 8, 60, A, A, B, A, None) == 2                    # K % 64
    assert L.pq_gemm_noalloc(2, 4, 8, 64, None, A, B, A, None) == 1                 # X NULL
    assert L.pq_gemm_noalloc(2, 4, 8, 64, A, MIS, B, A, None) == 4                  # align
    assert L.pq_gemm_noalloc(2, 0, 8, 64, A, A, B, A, None) == 0                    # empty
    assert pq.pq_gemm_workspace_bytes(2, 300, 16384, 16384) > pq.PQ_NOALLOC_SCRATCH_BYTES
    assert L.pq_gemm_noalloc(2, 300, 16384, 16384, A, A, B, A, None) == 5           # scratch too small
    assert pq.pq_gemm_workspace_bytes(2, 64, 16384, 16384) <= pq.PQ_NOALLOC_SCRATCH_BYTES
