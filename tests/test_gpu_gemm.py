"""GPU parity of the packed-weight GEMM (2-bit SEQ, ternary, 3- and 4-bit LSQ weights,
bf16 activations) against the oracle's binary64 reference, through the C ABI.

Inputs (packed codes, bf16 scales, activations) come from the oracle's own
pack on the CPU, never from the GPU path.  Bar: every checked output within
2e-2 * max(|Y_ref|, rms(Y_ref)) of the binary64 reference (the stated
tolerance), and also within 4e-3 * max(|Y_ref|, rms(Y_ref)) -- twice the
final bf16 rounding, which with the fp32 accumulation is all the error the
arithmetic makes -- so that a single misdecoded code fails even at large K.  Small cases
compare every element; the full 16384^2 and Llama-3-8B shapes compare
sampled elements the oracle computes one by one, in the launch configuration
the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle as O
from bit_quantization_aware_amd import synth

from gpu_util import dev, host

pytestmark = pytest.mark.gpu

pq = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global pq
    from bit_quantization_aware_amd import pq as _pq
    pq = _pq
    assert torch.cuda.is_available()
    O.set_threads(16)
    yield


REL = 2e-2
# Second, tighter bar on every checked output: the kernels' only roundings
# are the fp32 accumulation (products of bf16 activations and the exact
# decoded operands are exact in fp32; at K = 16384 the accumulated error
# stays near 1e-6 of the result) and the final bf16 rounding of the output
# (at most 2^-9 ~ 1.95e-3 relative).  4e-3 covers both with a factor two to
# spare, while one wrongly decoded or misplaced code moves an output by
# about |x| * alpha / 2, some 0.7 % of the rms at K = 16384 -- which the 2e-2
# bar alone would let through.
REL_TIGHT = 4e-3


def gpu_gemm(mode, X, packed, ab, N):
    """packed: the oracle's row-major code rows [N, rb]; the GPU gets them in
    the export byte order (the oracle's tile_codes)."""
    M, K = X.shape
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    tiled = O.tile_codes(packed, O.CODE_BITS[mode])
    assert tiled.size == pq.pq_packed_bytes(mode, N, K)
    if mode == O.SEQ2:
        pq.pq_w2a16_gemm(M, N, K, dev(X), dev(tiled), dev(ab), Y)
    elif mode == O.LSQ4:
        pq.pq_w4a16_gemm(M, N, K, dev(X), dev(tiled), dev(ab), Y)
    else:
        pq.pq_gemm(mode, M, N, K, dev(X), dev(tiled), dev(ab), Y)
    torch.cuda.synchronize()
    return synth.bf16_bits_to_f32(host(Y)).astype(np.float64)


def check(Y, Yref, what):
    rms = np.sqrt(np.mean(Yref ** 2)) if Yref.size else 0.0
    for rel in (REL, REL_TIGHT):
        lim = rel * np.maximum(np.abs(Yref), rms)
        bad = np.argwhere(np.abs(Y - Yref) > lim)
        assert bad.size == 0, f"{what}: {len(bad)} outside {rel} of the reference, first {bad[:4].tolist()}: " \
                              f"got {Y[tuple(bad[0])]} want {Yref[tuple(bad[0])]} (rms {rms})"


def make_case(mode, seed, M, N, K, sigma=0.02):
    rng = np.random.default_rng(seed)
    W = synth.normal_f32(rng, (N, K), sigma)
    alpha = O.alpha_init(mode, W)
    packed, ab = O.pack(mode, W, alpha)
    X = synth.to_bf16_bits(synth.normal_f32(rng, (M, K)))
    return X, packed, ab


DEPLOYABLE = [O.SEQ2, O.LSQ4, O.TERNARY, O.LSQ3, O.LSQ2, O.LSQ158, O.BINARY]


@pytest.mark.parametrize("mode", DEPLOYABLE)
@pytest.mark.parametrize("M,N,K", [(8, 256, 256), (1, 64, 64), (5, 100, 320), (16, 257, 1024),
                                   (17, 64, 128), (33, 96, 192), (64, 130, 256), (65, 128, 64),
                                   (130, 300, 384), (257, 129, 512), (64, 512, 4096),
                                   (100, 1000, 2048), (200, 260, 1600), (17, 8, 64),
                                   (16, 8192, 512), (3, 6200, 1024), (1, 12300, 256)])
def test_gemm_small_full_compare(mode, M, N, K):
    print(f"[gemm mode={mode} M={M} N={N} K={K}]", flush=True)
    X, packed, ab = make_case(mode, 7 * M + N + K, M, N, K)
    Y = gpu_gemm(mode, X, packed, ab, N)
    Yref = O.gemm_ref(mode, X, packed, ab, N)
    check(Y, Yref, f"m{mode} {M}x{N}x{K}")


def test_gemm_tiny_config_seed0():
    """The 256x256 seed-0 weight (2-bit SEQ, alpha = max|W_row|) against 8x256 activations."""
    W, _, X = synth.tiny()
    alpha = O.alpha_init(O.SEQ2, W)
    packed, ab = O.pack(O.SEQ2, W, alpha)
    Y = gpu_gemm(O.SEQ2, X, packed, ab, 256)
    check(Y, O.gemm_ref(O.SEQ2, X, packed, ab, 256), "tiny")


def test_gemm_zero_and_edge_values():
    # all-zero activations give exactly zero; extreme codes (all 0 / all 3)
    M, N, K = 3, 64, 128
    X = np.zeros((M, K), np.uint16)
    packed = np.zeros((N, K // 4), np.uint8)
    packed[1::2] = 0xFF
    ab = synth.to_bf16_bits(np.full(N, 0.5, np.float32))
    Y = gpu_gemm(O.SEQ2, X, packed, ab, N)
    assert np.all(Y == 0)
    X = synth.to_bf16_bits(np.ones((M, K), np.float32))
    Y = gpu_gemm(O.SEQ2, X, packed, ab, N)
    check(Y, O.gemm_ref(O.SEQ2, X, packed, ab, N), "edge codes")
    assert np.allclose(Y[:, 0], -0.75 * 0.5 * K) and np.allclose(Y[:, 1], 0.75 * 0.5 * K)


@pytest.mark.parametrize("M,N,K", [(1, 96, 1024), (2, 130, 2048), (4, 64, 512), (6, 64, 512), (8, 257, 1536),
                                   (12, 100, 1024), (16, 4100, 2048), (3, 9000, 512)])
def test_gemm_binary_streaming_full_compare(M, N, K):
    """1-bit codes (eight per byte) through the streaming kernel: one, two,
    four, eight and sixteen activation DMAs per 512-k group, one to four
    column tiles per block; every output."""
    print(f"[gemm binary M={M} N={N} K={K}]", flush=True)
    X, packed, ab = make_case(O.BINARY, 17 * M + N + K, M, N, K)
    Y = gpu_gemm(O.BINARY, X, packed, ab, N)
    check(Y, O.gemm_ref(O.BINARY, X, packed, ab, N), f"binary {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 64, 7680), (2, 100, 8192), (2, 1000, 16384), (1, 257, 5888),
                                   (1, 8, 16384), (2, 16, 6144)])
def test_gemm_small_m_long_k_full_compare(M, N, K):
    """One or two activation rows against long rows of weights (the decode
    shape), ragged and narrow N; every output."""
    print(f"[gemm small-M M={M} N={N} K={K}]", flush=True)
    X, packed, ab = make_case(O.SEQ2, 11 * M + N + K, M, N, K)
    Y = gpu_gemm(O.SEQ2, X, packed, ab, N)
    check(Y, O.gemm_ref(O.SEQ2, X, packed, ab, N), f"small-M {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 2, 4])
def test_gemm_wide_range_activations(M):
    """Activations spanning ten decades inside every 128-k chunk, exact zeros
    and whole zero chunks, against the binary64 reference."""
    N, K = 96, 8192
    rng = np.random.default_rng(100 + M)
    W = synth.normal_f32(rng, (N, K), 0.02)
    alpha = O.alpha_init(O.SEQ2, W)
    packed, ab = O.pack(O.SEQ2, W, alpha)
    x = rng.standard_normal((M, K)) * 10.0 ** rng.uniform(-6, 4, (M, K))
    x[:, ::7] = 0.0
    x[:, 256:512] = 0.0
    X = synth.to_bf16_bits(x.astype(np.float32))
    Y = gpu_gemm(O.SEQ2, X, packed, ab, N)
    check(Y, O.gemm_ref(O.SEQ2, X, packed, ab, N), f"wide range M={M}")


def sample_points(rng, M, N, count):
    ms = np.concatenate([[0, M - 1, 0, M - 1], rng.integers(0, M, count)])
    ns = np.concatenate([[0, 0, N - 1, N - 1], rng.integers(0, N, count)])
    return ms, ns


_C5 = {}


def c5_weights(mode):
    if mode not in _C5:
        W = synth.weight("square16k", 0)
        alpha = O.alpha_init(mode, W)
        _C5[mode] = O.pack(mode, W, alpha)
        del W
    return _C5[mode]


@pytest.mark.parametrize("mode", DEPLOYABLE)
@pytest.mark.parametrize("M", [1, 4, 16, 64, 512])
def test_gemm_16384_sampled(mode, M):
    """Full 16384 x 16384 weight at the benchmark's M values, sampled outputs."""
    N = K = 16384
    print(f"[gemm 16384^2 mode={mode} M={M}]", flush=True)
    packed, ab = c5_weights(mode)
    X = synth.activations("square16k", 0, M, K)
    Y = gpu_gemm(mode, X, packed, ab, N)
    rng = np.random.default_rng(M)
    ms, ns = sample_points(rng, M, N, 1500)
    ref = O.gemm_ref_at(mode, X, packed, ab, N, ms, ns)
    check(Y[ms, ns], ref, f"16384^2 M={M}")
    assert np.all(np.isfinite(Y))


@pytest.mark.parametrize("mode", [O.SEQ2, O.TERNARY, O.LSQ2, O.LSQ158])
@pytest.mark.parametrize("M,N,K", [(1024, 8192, 2048), (1100, 8200, 2112), (1030, 8202, 2240),
                                   (512, 16384, 2048), (600, 16200, 2176), (520, 16202, 2048)])
def test_gemm_large_m_sampled(mode, M, N, K):
    """The large-M path (64 x 128 outputs per wave, the activation row sums
    taken inside the kernel on the matrix unit), both forms: 128-row blocks (M >= 1024) and 64-row blocks whose
    two wave pairs split K (the M = 512..600 cases); ragged M and N, N not a
    multiple of 4, K with a partial last 64-byte group and, for the first
    form, an odd number of 64-k stages; 4000 sampled outputs
    plus every output of the first and last row and column against the
    binary64 reference."""
    print(f"[gemm large-M mode={mode} M={M} N={N} K={K}]", flush=True)
    X, packed, ab = make_case(mode, 13 * M + N + K, M, N, K)
    Y = gpu_gemm(mode, X, packed, ab, N)
    rng = np.random.default_rng(M + N + K + mode)
    ms, ns = sample_points(rng, M, N, 4000)
    edge_m = np.concatenate([np.zeros(N, int), np.full(N, M - 1), np.arange(M), np.arange(M)])
    edge_n = np.concatenate([np.arange(N), np.arange(N), np.zeros(M, int), np.full(M, N - 1)])
    ms, ns = np.concatenate([ms, edge_m]), np.concatenate([ns, edge_n])
    check(Y[ms, ns], O.gemm_ref_at(mode, X, packed, ab, N, ms, ns), f"large-M m{mode} {M}x{N}x{K}")


def test_gemm_large_m_full_compare():
    """One large-M case compared at every output, with the exported bf16 scale
    and with the binary32 scale of the training forward."""
    M, N, K = 1024, 8192, 2048
    X, packed, ab = make_case(O.SEQ2, 77, M, N, K)
    check(gpu_gemm(O.SEQ2, X, packed, ab, N), O.gemm_ref(O.SEQ2, X, packed, ab, N), "large-M full")
    rng = np.random.default_rng(78)
    W = synth.normal_f32(rng, (N, K), 0.02)
    alpha = O.alpha_init(O.SEQ2, W)
    packed, _ = O.pack(O.SEQ2, W, alpha)
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    pq.pq_gemm_f32a(O.SEQ2, M, N, K, dev(X), dev(O.tile_codes(packed, O.CODE_BITS[O.SEQ2])), dev(alpha), Y)
    torch.cuda.synchronize()
    Yg = synth.bf16_bits_to_f32(host(Y)).astype(np.float64)
    check(Yg, O.gemm_ref_f32a(O.SEQ2, X, packed, alpha, N), "large-M f32a full")


@pytest.mark.parametrize("M", [1, 16, 256, 4096])
def test_gemm_llama3_8b_sampled(M):
    """The four Llama-3-8B projection shapes (2-bit SEQ), sampled outputs."""
    for k, (_, name, N, K) in enumerate(synth.llama3_8b_shapes()):
        print(f"[gemm llama {name} M={M}]", flush=True)
        W = synth.weight("llama3_8b", k)
        packed, ab = O.pack(O.SEQ2, W, O.alpha_init(O.SEQ2, W))
        del W
        X = synth.activations("llama3_8b", k, M, K)
        Y = gpu_gemm(O.SEQ2, X, packed, ab, N)
        rng = np.random.default_rng(k)
        ms, ns = sample_points(rng, M, N, 800)
        check(Y[ms, ns], O.gemm_ref_at(O.SEQ2, X, packed, ab, N, ms, ns), f"{name} M={M}")


@pytest.mark.parametrize("mode", DEPLOYABLE)
@pytest.mark.parametrize("M,N,K", [(1, 96, 1024), (16, 257, 512), (64, 576, 576), (256, 1536, 576),
                                   (512, 576, 1536), (2048, 576, 576)])
def test_gemm_f32_alpha(mode, M, N, K):
    """The training forward's product: codes + the binary32 alpha (no bf16
    rounding of the scale), every output against the binary64 reference."""
    rng = np.random.default_rng(M * 3 + N + K + mode)
    W = synth.normal_f32(rng, (N, K), 0.02)
    alpha = O.alpha_init(mode, W)
    packed, _ = O.pack(mode, W, alpha)
    X = synth.to_bf16_bits(synth.normal_f32(rng, (M, K)))
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    pq.pq_gemm_f32a(mode, M, N, K, dev(X), dev(O.tile_codes(packed, O.CODE_BITS[mode])), dev(alpha), Y)
    torch.cuda.synchronize()
    Yg = synth.bf16_bits_to_f32(host(Y)).astype(np.float64)
    check(Yg, O.gemm_ref_f32a(mode, X, packed, alpha, N), f"f32a m{mode} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(64, 2048, 2048), (1024, 8192, 2048), (4, 1000, 1024)])
def test_gemm_caller_workspace_and_guards(M, N, K):
    """The workspace is the caller's: exactly pq_gemm_workspace_bytes bytes
    between canary guards, as is the output; the guards stay intact and the
    result matches the reference (split-K partials, and shapes that need no
    workspace: the large-M path and weight streaming)."""
    from gpu_util import Guarded

    X, packed, ab = make_case(O.SEQ2, 500 + M + N, M, N, K)
    nbytes = pq.pq_gemm_workspace_bytes(O.SEQ2, M, N, K)
    assert nbytes >= 0
    ws = Guarded((nbytes,), torch.uint8)
    Y = Guarded((M, N), torch.bfloat16)
    tiled = dev(O.tile_codes(packed, O.CODE_BITS[O.SEQ2]))
    pq.pq_w2a16_gemm(M, N, K, dev(X), tiled, dev(ab), Y.t, workspace=(ws.t.data_ptr() if nbytes else 0, nbytes))
    torch.cuda.synchronize()
    ws.check("workspace")
    Y.check("Y")
    Yg = synth.bf16_bits_to_f32(host(Y.t)).astype(np.float64)
    if M * N <= 1 << 20:
        check(Yg, O.gemm_ref(O.SEQ2, X, packed, ab, N), f"caller workspace {M}x{N}x{K}")
    else:
        rng = np.random.default_rng(M)
        ms, ns = sample_points(rng, M, N, 3000)
        check(Yg[ms, ns], O.gemm_ref_at(O.SEQ2, X, packed, ab, N, ms, ns), f"caller workspace {M}x{N}x{K}")


@pytest.mark.parametrize("mode", [O.SEQ2, O.LSQ4, O.BINARY])
@pytest.mark.parametrize("M,N,K", [(2100, 4000, 256), (1030, 7700, 512)])
def test_gemm_persistent_tiles_full_compare(mode, M, N, K):
    """More output tiles than the tiled launch has blocks (528 and 527
    items of 64 x 256 for 512 blocks): blocks take several tiles in turn,
    with and without the XCD order (item count a multiple of 8 or not),
    ragged last row and column tiles; every output."""
    print(f"[gemm persistent mode={mode} M={M} N={N} K={K}]", flush=True)
    assert -(-M // 64) * -(-N // 256) > 512
    X, packed, ab = make_case(mode, 31 * M + N + K + mode, M, N, K)
    Y = gpu_gemm(mode, X, packed, ab, N)
    check(Y, O.gemm_ref(mode, X, packed, ab, N), f"persistent m{mode} {M}x{N}x{K}")


def test_gemm_training_forward_shape_sampled():
    """The MobileLLM training forward's up projection at 16384 tokens from
    codes with the binary32 scale (1536 tiles of 64 x 256, runs of four row
    tiles per block of the resident-code kernel), sampled outputs against
    the binary64 reference."""
    M, N, K = 16384, 1536, 576
    rng = np.random.default_rng(4242)
    W = synth.normal_f32(rng, (N, K), 0.02)
    alpha = O.alpha_init(O.SEQ2, W)
    packed, _ = O.pack(O.SEQ2, W, alpha)
    X = synth.to_bf16_bits(synth.normal_f32(rng, (M, K)))
    Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    pq.pq_gemm_f32a(O.SEQ2, M, N, K, dev(X), dev(O.tile_codes(packed, 2)), dev(alpha), Y)
    torch.cuda.synchronize()
    Yg = synth.bf16_bits_to_f32(host(Y)).astype(np.float64)
    ms, ns = sample_points(rng, M, N, 4000)
    # every output of the first and the last 64-row tile too
    edge_m = np.repeat(np.r_[0:64, M - 64:M], N)
    edge_n = np.tile(np.arange(N), 128)
    ms, ns = np.concatenate([ms, edge_m]), np.concatenate([ns, edge_n])
    # binary64 reference with the binary32 scale, on the sampled rows only
    rows = np.unique(ms)
    Yr = O.gemm_ref_f32a(O.SEQ2, X[rows], packed, alpha, N)
    pos = {r: i for i, r in enumerate(rows)}
    ref = Yr[[pos[m] for m in ms], ns]
    check(Yg[ms, ns], ref, "training forward 16384x1536x576")


def _wres_runs(M, N):
    """(row tiles, blocks) of the resident-code launch: 64 x 256 tiles, or
    64 x 192 where those pad N less; per column tile as many runs of row
    tiles as 512 blocks allow, then as few as give the same longest run."""
    tn = 192 if -(-N // 192) * 192 < -(-N // 256) * 256 else 256
    mt, nt = -(-M // 64), -(-N // tn)
    rmax = max(1, min(mt, 512 // nt))
    runlen = -(-mt // rmax)
    return mt * nt, nt * -(-mt // runlen)


@pytest.mark.parametrize("mode,M,N,K", [(O.SEQ2, 1030, 600, 576), (O.TERNARY, 1030, 600, 576),
                                        (O.LSQ2, 1030, 600, 576), (O.LSQ158, 1030, 600, 576),
                                        (O.SEQ2, 8380, 1102, 192), (O.SEQ2, 2100, 200, 704),
                                        (O.SEQ2, 1024, 256, 64), (O.LSQ2, 3000, 515, 640),
                                        (O.SEQ2, 2048, 576, 576), (O.TERNARY, 1100, 192, 320),
                                        (O.LSQ158, 1500, 380, 704), (O.SEQ2, 1090, 190, 64),
                                        (O.LSQ2, 8300, 1150, 192)])
def test_gemm_short_k_resident_codes_full_compare(mode, M, N, K):
    """2-bit GEMMs with K <= 704 and M >= 1024 (the resident-code kernel):
    ragged last row tile, N not a multiple of 256, 16, 8 or 4 (the
    element-wise store), one K stage, the largest K, 655 tiles on 330
    blocks (runs of one and two row tiles), and the 192-column blocks of
    48-column waves (N = 576, 192, 380, 190, 1150, where they pad N less
    than 256-column ones); every output."""
    print(f"[gemm resident codes mode={mode} M={M} N={N} K={K}]", flush=True)
    tiles, nb = _wres_runs(M, N)
    if (M, N) == (8380, 1102):
        assert tiles > nb
    X, packed, ab = make_case(mode, 13 * M + N + K + mode, M, N, K)
    Y = gpu_gemm(mode, X, packed, ab, N)
    check(Y, O.gemm_ref(mode, X, packed, ab, N), f"resident codes m{mode} {M}x{N}x{K}")


def test_gemm_workspace_reused_across_shapes():
    """One workspace, sized for the largest of the shapes, through a sequence
    of GEMMs that use it differently (split-K partials of several sizes, and
    paths that use none), twice over: every result matches the
    reference, whatever the previous call left in it."""
    shapes = [(64, 2048, 2048), (1024, 8192, 2048), (1, 1024, 4096), (256, 1536, 4096), (100, 1000, 2048),
              (4, 4096, 4096)]
    need = max(pq.pq_gemm_workspace_bytes(O.SEQ2, *sh) for sh in shapes)
    ws = torch.full((need,), 0x5A, dtype=torch.uint8, device="cuda")
    cases = {sh: make_case(O.SEQ2, 700 + sum(sh), *sh) for sh in shapes}
    for rnd in range(2):
        for (M, N, K) in shapes:
            print(f"[gemm ws reuse round={rnd} M={M} N={N} K={K}]", flush=True)
            X, packed, ab = cases[(M, N, K)]
            Y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
            pq.pq_w2a16_gemm(M, N, K, dev(X), dev(O.tile_codes(packed, O.CODE_BITS[O.SEQ2])), dev(ab), Y, workspace=(ws.data_ptr(), need))
            torch.cuda.synchronize()
            Yg = synth.bf16_bits_to_f32(host(Y)).astype(np.float64)
            if M * N <= 1 << 20:
                check(Yg, O.gemm_ref(O.SEQ2, X, packed, ab, N), f"reuse {M}x{N}x{K}")
            else:
                rng = np.random.default_rng(M + rnd)
                ms, ns = sample_points(rng, M, N, 2000)
                check(Yg[ms, ns], O.gemm_ref_at(O.SEQ2, X, packed, ab, N, ms, ns), f"reuse {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(64, 2048, 2048), (1024, 8192, 2048), (16, 4096, 4096)])
def test_gemm_graph_capture_without_warmup(M, N, K):
    """The first call of a shape can be captured into a HIP graph (nothing is
    allocated or synchronised inside the call): captured before any eager
    call, replayed three times with eager work in between, every replay
    equal bit for bit to the eager result, which matches the reference."""
    X, packed, ab = make_case(O.SEQ2, 900 + M + N, M, N, K)
    Xd, tiled, abd = dev(X), dev(O.tile_codes(packed, O.CODE_BITS[O.SEQ2])), dev(ab)
    ws = pq.gemm_workspace(O.SEQ2, M, N, K)
    wsa = (ws.data_ptr(), ws.numel()) if ws is not None else (0, 0)
    Yg = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        pq.pq_w2a16_gemm(M, N, K, Xd, tiled, abd, Yg, stream=side.cuda_stream, workspace=wsa)
    torch.cuda.synchronize()
    Ye = torch.empty_like(Yg)
    pq.pq_w2a16_gemm(M, N, K, Xd, tiled, abd, Ye, workspace=wsa)
    torch.cuda.synchronize()
    for r in range(3):
        Yg.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Yg.view(torch.int16), Ye.view(torch.int16)), f"replay {r} differs from eager"
        junk = torch.randn(1 << 20, device="cuda")
        junk.mul_(2.0)
        torch.cuda.synchronize()
    Yh = synth.bf16_bits_to_f32(host(Ye)).astype(np.float64)
    rng = np.random.default_rng(N)
    ms, ns = sample_points(rng, M, N, 2000)
    check(Yh[ms, ns], O.gemm_ref_at(O.SEQ2, X, packed, ab, N, ms, ns), f"graph {M}x{N}x{K}")
    del g
