"""Pins of the CPU oracle to facts outside the oracle itself.

What each pin stands on:
  * level sets, the clip-boundary worked example and the ternary bins: the
    pages' own printed values (tests/golden/*, each with its citation);
  * nearest-level projection: exact rational arithmetic (fractions) on tiny
    random inputs -- a textbook projection onto the level set;
  * backward: torch autograd (float64) of the straight-through surrogate
    "round acts as the identity inside the clip range" -- the chain rule
    derives the gradient independently of the oracle's hand-derived formula;
  * finite differences where every weight is clipped (q is linear in alpha);
  * alpha init, GEMM and bf16 rounding: numpy / torch library routines;
  * the deployment byte order of exported codes: a numpy axis shuffle of the
    padded code rows and hand-worked positions (the layout is the library's
    own definition; the pages fix only four codes per byte);
  * AdamW: torch.optim.AdamW in float64 over five steps, and the first-step
    closed form (bias corrections cancel); the fused QAT step against the
    pinned backward, AdamW and forward called in turn.
Parity unpinned (documented readings): the 1-bit quantizer, the ternary
alpha-gradient of clipped weights, and n / Qp of the default gradient scale.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O
from bit_quantization_aware_amd import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MODE_NAMES = {"binary": O.BINARY, "ternary": O.TERNARY, "seq2": O.SEQ2, "lsq3": O.LSQ3,
              "lsq4": O.LSQ4, "lsq2": O.LSQ2, "lsq158": O.LSQ158}
F32 = np.float32
CLIP = F32(0.99)


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def levels_exact(mode):
    """Level set of a mode from the golden file, as Fractions."""
    for row in read_golden("level_sets.txt"):
        if MODE_NAMES[row[0]] == mode:
            return [Fraction(v) for v in row[1:]]
    raise KeyError(mode)


def clip_bounds(mode):
    if mode in (O.SEQ2, O.TERNARY):
        return -CLIP, CLIP
    if mode == O.LSQ3:
        return F32(-4), F32(3)
    if mode == O.LSQ4:
        return F32(-8), F32(7)
    if mode == O.LSQ2:
        return F32(-2), F32(1)
    return F32(-1), F32(1)          # binary, 1.58-bit LSQ


def r_min(mode):
    return {O.BINARY: -1, O.TERNARY: -1, O.SEQ2: -2, O.LSQ3: -4, O.LSQ4: -8, O.LSQ2: -2, O.LSQ158: -1}[mode]


def unpack_codes(codes, mode, cols):
    """Independent unpacker: LSB-first bit stream, code_bits per element."""
    cw = O.CODE_BITS[mode]
    bits = np.unpackbits(codes, axis=1, bitorder="little")[:, : cols * cw]
    bits = bits.reshape(codes.shape[0], cols, cw).astype(np.int64)
    return (bits * (1 << np.arange(cw))).sum(axis=2)


def steps_of(codes, mode, cols):
    """Step index r of each stored code (1 bit: 0 -> -1, 1 -> +1)."""
    c = unpack_codes(codes, mode, cols)
    if mode == O.BINARY:
        return 2 * c - 1
    return c + r_min(mode)


# ----------------------------------------------------------------------------
# Level sets (golden, from the pages)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("mode", O.MODES)
def test_level_sets_match_pages(mode):
    # alpha = 1: q is the level itself, exactly.
    ws = np.linspace(-10.0, 10.0, 80001, dtype=np.float32)
    W = ws.reshape(1, -1)
    _, q32, _ = O.quantize_fwd(mode, W, np.ones(1, np.float32))
    got = sorted(set(q32.ravel().tolist()))
    want = sorted(float(F32(float(v))) for v in levels_exact(mode))
    assert got == want
    # another scale: the same step indices, levels scaled by alpha
    a = F32(0.0371)
    _, q32b, codes = O.quantize_fwd(mode, (ws * a).reshape(1, -1), np.array([a], np.float32))
    lv = np.array([float(v) for v in levels_exact(mode)])
    ratio = q32b.ravel().astype(np.float64) / float(a)
    assert np.all(np.min(np.abs(ratio[:, None] - lv[None, :]), axis=1) < 1e-6)
    n_codes = len(set(unpack_codes(codes, mode, ws.size).ravel().tolist()))
    assert n_codes == len(lv)


def test_seq2_levels_in_half_steps_match_rebuttal():
    # The rebuttal prints the 2-bit SEQ grid as {-1.5,-0.5,0.5,1.5} in half-steps.
    half = [Fraction(-3, 2), Fraction(-1, 2), Fraction(1, 2), Fraction(3, 2)]
    assert [v / 2 for v in half] == levels_exact(O.SEQ2)


def test_seq2_clip_boundary_worked_example():
    for x, clip, want in read_golden("seq2_clip_boundary.txt"):
        for alpha in (1.0, 0.02, 3.5):
            r, q = O.seq2_scalar(float(x) * alpha, alpha, float(clip))
            assert q / alpha == pytest.approx(float(want), rel=1e-6), (x, clip, alpha)
    # the shipped clip constant is fl32(0.99)
    assert np.float32(O.clip_value()).view(np.uint32) == 0x3F7D70A4


def test_ternary_bins_match_rebuttal():
    bins = [(Fraction(lo), Fraction(hi), int(r)) for lo, hi, r in read_golden("ternary_bins.txt")]
    xs = np.linspace(-1.2, 1.2, 4801, dtype=np.float32)
    for x in xs:
        r, q, xo = O.quantize_scalar(O.TERNARY, float(x), 1.0)
        xc = min(max(Fraction(float(xo)), Fraction(float(-CLIP))), Fraction(float(CLIP)))
        v = Fraction(3, 2) * xc
        hits = [b for b in bins if b[0] <= v <= b[1]]
        assert hits, v
        if len(hits) == 1 and abs(v - hits[0][0]) > Fraction(1, 10**6) and \
                abs(v - hits[0][1]) > Fraction(1, 10**6):
            assert r == hits[0][2], (x, v)
    # shared edge v = +-0.5 (both closed bins contain it): ties go to index 0
    for x in (np.float32(1) / np.float32(3), -(np.float32(1) / np.float32(3))):
        assert O.quantize_scalar(O.TERNARY, float(x), 1.0)[0] == 0


# ----------------------------------------------------------------------------
# Brute force: nearest level in exact arithmetic
# ----------------------------------------------------------------------------
def nearest_index_exact(mode, x32):
    """Exact projection of the fp32 ratio x onto the clipped grid; ties to even r."""
    lo, hi = clip_bounds(mode)
    xf = Fraction(float(x32))
    if mode == O.BINARY:
        return 1 if x32 >= 0 else -1, False
    xc = min(max(xf, Fraction(float(lo))), Fraction(float(hi)))
    lv = levels_exact(mode)
    d = [abs(xc - v) for v in lv]
    best = min(d)
    idx = [i for i, v in enumerate(d) if v == best]
    rs = [i + r_min(mode) for i in idx]
    tie = len(rs) > 1
    if tie:
        rs = [r for r in rs if r % 2 == 0]
    # distance of xc to the nearest decision edge, in level-spacing units
    edges = [(lv[i] + lv[i + 1]) / 2 for i in range(len(lv) - 1)]
    near_edge = min(abs(xc - e) for e in edges) < Fraction(1, 2**21)
    return rs[0], near_edge


@pytest.mark.parametrize("mode", O.MODES)
def test_nearest_level_bruteforce(mode):
    rng = np.random.default_rng(100 + mode)
    alphas = np.array([0.02, 1.0, 3.0e-3, 7.5], np.float32)
    for a in alphas:
        W = (rng.standard_normal((4, 64)).astype(np.float32) * a * F32(1.3))
        _, _, codes = O.quantize_fwd(mode, W, np.full(4, a, np.float32))
        got = steps_of(codes, mode, 64)
        for i in range(4):
            for j in range(64):
                x32 = F32(W[i, j]) / F32(a)
                want, near_edge = nearest_index_exact(mode, x32)
                if got[i, j] != want:
                    assert near_edge, (mode, a, W[i, j], got[i, j], want)


def test_seq2_tiny_negative_and_ties():
    # Documented fp32 behaviour of the literal formula (no page prints these):
    # for -2^-26 <= x < 0, fl32(2x - 0.5) = -0.5 -> round -> 0 -> +0.25;
    # x = -2^-25 is far enough to land on -0.25.
    assert O.quantize_scalar(O.SEQ2, -(2.0 ** -26), 1.0)[0] == 0
    assert O.quantize_scalar(O.SEQ2, -(2.0 ** -25), 1.0)[0] == -1
    # exact ties of z = 2x - 0.5 go to the even step index
    assert O.quantize_scalar(O.SEQ2, -0.5, 1.0)[0] == -2     # z = -1.5 -> -2
    assert O.quantize_scalar(O.SEQ2, 0.5, 1.0)[0] == 0       # z = 0.5 -> 0
    assert O.quantize_scalar(O.SEQ2, 0.0, 1.0)[0] == 0       # z = -0.5 -> 0
    assert O.quantize_scalar(O.SEQ2, -0.0, 1.0)[0] == 0
    # LSQ: x = n + 1/2 rounds to even
    assert O.quantize_scalar(O.LSQ4, 2.5, 1.0)[0] == 2
    assert O.quantize_scalar(O.LSQ4, -3.5, 1.0)[0] == -4
    # binary: sign(+-0) = +1
    assert O.quantize_scalar(O.BINARY, -0.0, 1.0)[0] == 1


@pytest.mark.parametrize("mode", O.MODES)
def test_idempotent(mode):
    W, _ = synth.random_case(7, 16, 96)
    alpha = O.alpha_init(mode, W)
    wq16, q32, codes = O.quantize_fwd(mode, W, alpha)
    wq16b, q32b, codesb = O.quantize_fwd(mode, q32, alpha)
    assert np.array_equal(codes, codesb)
    assert np.array_equal(q32.view(np.uint32), q32b.view(np.uint32))
    assert np.array_equal(wq16, wq16b)


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(3)
    vals = [rng.standard_normal(2000).astype(np.float32) * F32(s) for s in (1e-3, 1.0, 1e5)]
    # exact ties (low half 0x8000) with even and odd kept parts, and edge values
    ties = np.array([0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000, 0x00008000,
                     0x7F7F8000, 0x00000001, 0x80000000, 0x00000000, 0x3F7FFFFF],
                    np.uint32).view(np.float32)
    x = np.concatenate(vals + [ties])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_rne(x), want)


@pytest.mark.parametrize("mode", O.MODES)
def test_fwd_bf16_is_rne_of_fp32_value(mode):
    W, _ = synth.random_case(11, 8, 64)
    wq16, q32, _ = O.quantize_fwd(mode, W, O.alpha_init(mode, W))
    want = torch.from_numpy(q32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wq16, want)


# ----------------------------------------------------------------------------
# Backward
# ----------------------------------------------------------------------------
def boundary_rich_case(seed, rows, cols, mode):
    """Weights spread past the clip range, plus exact clip-bound ratios."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((rows, cols)).astype(np.float32) * F32(0.02)
    alpha = (np.abs(W).max(axis=1) * F32(0.6)).astype(np.float32)
    if mode in (O.LSQ3, O.LSQ4):
        alpha = (alpha / F32(clip_bounds(mode)[1])).astype(np.float32)
    lo, hi = clip_bounds(mode)
    # plant exact boundary ratios: w = bound * alpha where that product is exact in fp32
    for i in range(rows):
        a = F32(2.0) ** -6
        alpha[i] = a if i % 2 == 0 else alpha[i]
        if i % 2 == 0:
            W[i, 0] = F32(hi) * a
            W[i, 1] = F32(lo) * a
    G = rng.standard_normal((rows, cols)).astype(np.float32)
    return W, alpha, G


def ste_surrogate_grad(mode, W, alpha, G, r):
    """torch float64 autograd of L = sum G*q with q = alpha * f(R), where the
    rounding R is replaced by 'identity plus a detached offset' -- the
    straight-through estimator -- and clamp provides the clip-range gate."""
    w = torch.from_numpy(W.astype(np.float64)).requires_grad_(True)
    a = torch.from_numpy(alpha.astype(np.float64)).requires_grad_(True)
    g = torch.from_numpy(G.astype(np.float64))
    rr = torch.from_numpy(r.astype(np.float64))
    lo, hi = clip_bounds(mode)
    x = w / a[:, None]
    xc = torch.clamp(x, float(lo), float(hi))
    if mode == O.SEQ2:
        u = xc * 2.0 - 0.5
        R = u + (rr - u).detach()
        q = a[:, None] * (R + 0.5) / 4.0 * 2.0
    elif mode == O.TERNARY:
        v = xc * 1.5
        R = v + (rr - v).detach()
        q = a[:, None] * R * float(np.float32(2.0 / 3.0))  # the binary32 level 2/3
    else:  # LSQ grids, and the sign binarizer as its two-level grid
        R = xc + (rr - xc).detach()
        q = a[:, None] * R
    (g * q).sum().backward()
    return w.grad.numpy(), a.grad.numpy()


@pytest.mark.parametrize("mode", O.MODES)
def test_bwd_matches_autograd_of_ste_surrogate(mode):
    W, alpha, G = boundary_rich_case(20 + mode, 12, 40, mode)
    _, _, codes = O.quantize_fwd(mode, W, alpha)
    r = steps_of(codes, mode, W.shape[1])
    dW, dalpha, mask = O.quantize_bwd(mode, W, alpha, G, grad_scale=1.0)
    wgrad, agrad = ste_surrogate_grad(mode, W, alpha, G, r)
    # alpha gradient: autograd in float64 (x = w/alpha in float64) vs the
    # oracle (x rounded to fp32, sum rounded once to fp32): rounding noise only
    noise = 1e-6 * np.abs(G.astype(np.float64)).sum(axis=1)
    assert np.all(np.abs(dalpha.astype(np.float64) - agrad) <= 1e-6 * np.abs(agrad) + noise)
    # weight gradient: G inside the clip range, 0 outside (the surrogate's slope
    # is 1 up to the binary32 constants: 1.5 * fl32(2/3) = 1 + 4.5e-8)
    assert np.allclose(dW.astype(np.float64), wgrad, rtol=1e-6, atol=0)
    assert np.array_equal(dW == 0, (wgrad == 0) | (G == 0))
    # both cases (inside and clipped) occur in this input
    inside = np.unpackbits(mask, axis=1, bitorder="little")[:, :W.shape[1]].astype(bool)
    assert inside.any() and (~inside).any()


@pytest.mark.parametrize("mode", O.MODES)
def test_mask_bounds_are_inclusive_in_fp32(mode):
    W, alpha, G = boundary_rich_case(30 + mode, 6, 24, mode)
    dW, _, mask = O.quantize_bwd(mode, W, alpha, G)
    inside = np.unpackbits(mask, axis=1, bitorder="little")[:, :24].astype(bool)
    lo, hi = clip_bounds(mode)
    x = W / np.maximum(alpha, F32(1e-5))[:, None]
    want = (x >= lo) & (x <= hi)
    assert np.array_equal(inside, want)
    # the planted exact-bound ratios are inside
    assert inside[0, 0] and inside[0, 1]
    assert np.array_equal(dW.view(np.uint32), np.where(want, G, F32(0)).view(np.uint32))


@pytest.mark.parametrize("mode", O.MODES)
def test_alpha_grad_finite_difference_when_all_clipped(mode):
    rng = np.random.default_rng(40 + mode)
    rows, cols = 5, 32
    alpha = np.full(rows, 0.01, np.float32)
    hi = float(clip_bounds(mode)[1])
    mag = rng.uniform(1.5 * max(hi, 1.0) + 1, 3 * max(hi, 1.0) + 2, (rows, cols))
    W = (np.sign(rng.standard_normal((rows, cols))) * mag * 0.01).astype(np.float32)
    G = rng.standard_normal((rows, cols)).astype(np.float32)
    _, dalpha, mask = O.quantize_bwd(mode, W, alpha, G, grad_scale=1.0)
    assert not mask.any()
    h = 1e-4

    def loss(a):
        _, q, _ = O.quantize_fwd(mode, W, np.full(rows, a, np.float32))
        return (q.astype(np.float64) * G).sum(axis=1)
    fd = (loss(0.01 + h) - loss(0.01 - h)) / (F32(0.01 + h) - F32(0.01 - h)).astype(np.float64)
    assert np.allclose(dalpha, fd, rtol=1e-3)


def test_default_grad_scale_reading():
    # Documented reading (parity unpinned): 1/sqrt(n * Qp), n = rows*cols,
    # Qp = 1, 1, 1, 3, 7 for 1, 1.58, 2, 3, 4 bits.
    for mode, qp in zip(O.MODES, (1, 1, 1, 3, 7, 1, 1)):
        assert O.default_grad_scale(mode, 64, 128) == pytest.approx((64 * 128 * qp) ** -0.5)


def test_bwd_bf16_gradient_equals_fp32_of_same_values():
    W, G = synth.random_case(5, 8, 64)
    Gb = synth.to_bf16_bits(G)
    alpha = O.alpha_init(O.SEQ2, W)
    a = O.quantize_bwd(O.SEQ2, W, alpha, Gb)
    b = O.quantize_bwd(O.SEQ2, W, alpha, synth.bf16_bits_to_f32(Gb))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ----------------------------------------------------------------------------
# alpha init
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("mode", O.MODES)
def test_alpha_init_matches_numpy(mode):
    W, _ = synth.random_case(9, 33, 200)
    W[3] = 0.0
    a = O.alpha_init(mode, W)
    amax = np.abs(W).max(axis=1)
    if mode in (O.SEQ2, O.TERNARY, O.LSQ2, O.LSQ158):   # max|w| / Qp with Qp = 1 for the LSQ ablation grids
        assert np.array_equal(a, amax)
    elif mode == O.LSQ3:
        assert np.array_equal(a, amax / F32(3))
    elif mode == O.LSQ4:
        assert np.array_equal(a, amax / F32(7))
    else:
        want = np.abs(W).astype(np.float64).mean(axis=1).astype(np.float32)
        ulp = np.spacing(want)
        assert np.all(np.abs(a - want) <= ulp)


@pytest.mark.parametrize("mode", O.MODES)
def test_seq_init_puts_row_max_outside(mode):
    # With alpha = max|w| the row's largest weight has x = +-1 exactly, beyond
    # the 0.99 clip, so its straight-through gradient is zero.
    if mode not in (O.SEQ2, O.TERNARY):
        return
    W, G = synth.random_case(13, 10, 50)
    alpha = O.alpha_init(mode, W)
    dW, _, mask = O.quantize_bwd(mode, W, alpha, G)
    j = np.abs(W).argmax(axis=1)
    inside = np.unpackbits(mask, axis=1, bitorder="little")[:, :50].astype(bool)
    assert not inside[np.arange(10), j].any()


def test_all_zero_row_is_finite():
    W = np.zeros((2, 16), np.float32)
    G = np.ones((2, 16), np.float32)
    for mode in O.MODES:
        a = O.alpha_init(mode, W)
        assert np.all(a == 0)
        wq16, q32, codes = O.quantize_fwd(mode, W, a)
        dW, da, _ = O.quantize_bwd(mode, W, a, G)
        assert np.all(np.isfinite(q32)) and np.all(np.isfinite(dW)) and np.all(np.isfinite(da))


# ----------------------------------------------------------------------------
# Packing and the GEMM reference
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("mode", O.MODES)
def test_codes_dequantize_to_forward_values(mode):
    W, _ = synth.random_case(17, 9, 72)
    alpha = O.alpha_init(mode, W)
    _, q32, codes = O.quantize_fwd(mode, W, alpha)
    assert codes.shape == (9, 72 * O.CODE_BITS[mode] // 8)
    r = steps_of(codes, mode, 72)
    steps = [-1, 1] if mode == O.BINARY else \
        list(range(r_min(mode), r_min(mode) + len(levels_exact(mode))))
    lv = {t: F32(float(v)) for t, v in zip(steps, levels_exact(mode))}
    lev = np.vectorize(lambda t: lv[t])(r).astype(np.float32)
    want = np.maximum(alpha, F32(1e-5))[:, None] * lev
    assert np.array_equal(q32.view(np.uint32), want.astype(np.float32).view(np.uint32))
    if mode == O.TERNARY:
        assert (r <= 1).all()


def test_pack_byte_layout_lsb_first():
    # 2-bit SEQ codes 0,1,2,3 (levels -0.75,-0.25,0.25,0.75) in one byte,
    # first element in the lowest bits: 0b11_10_01_00 = 0xE4.
    W = np.array([[-0.75, -0.25, 0.25, 0.75, 0.75, 0.25, -0.25, -0.75]], np.float32)
    packed, ab = O.pack(O.SEQ2, W, np.ones(1, np.float32))
    assert packed.tolist() == [[0xE4, 0x1B]]
    assert ab.tolist() == [0x3F80]
    # 4-bit LSQ: levels -8 and 7 -> codes 0 and 15, low nibble first
    W4 = np.array([[-8.0, 7.0, 0.0, 1.0]], np.float32)
    p4, _ = O.pack(O.LSQ4, W4, np.ones(1, np.float32))
    assert p4.tolist() == [[0xF0, 0x98]]
    # 1 bit: -1 -> code 0, +1 -> code 1, eight codes per byte, first code lowest
    W1 = np.array([[-1.0, 1.0, 1.0, -1.0, 1.0, 1.0, 1.0, 1.0]], np.float32)
    p1, _ = O.pack(O.BINARY, W1, np.ones(1, np.float32))
    assert p1.tolist() == [[0xF6]]


@pytest.mark.parametrize("mode", [O.SEQ2, O.LSQ4, O.TERNARY, O.LSQ3, O.BINARY])
def test_gemm_ref_is_matmul_of_dequantized_weight(mode):
    rng = np.random.default_rng(50)
    M, N, K = 5, 24, 64
    W = rng.standard_normal((N, K)).astype(np.float32) * F32(0.02)
    alpha = O.alpha_init(mode, W)
    packed, ab = O.pack(mode, W, alpha)
    X = synth.to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    Y = O.gemm_ref(mode, X, packed, ab, N)
    lev = {O.SEQ2: lambda c: (c - 1.5) / 2.0, O.LSQ4: lambda c: c - 8.0,
           O.TERNARY: lambda c: (c - 1.0) * np.float64(np.float32(2.0 / 3.0)), O.LSQ3: lambda c: c - 4.0,
           O.BINARY: lambda c: 2.0 * c - 1.0}[mode]
    Wd = lev(unpack_codes(packed, mode, K).astype(np.float64)) * \
        synth.bf16_bits_to_f32(ab).astype(np.float64)[:, None]
    want = np.matmul(synth.bf16_bits_to_f32(X).astype(np.float64), Wd.T)
    assert np.allclose(Y, want, rtol=1e-12, atol=1e-12)
    ms = rng.integers(0, M, 17)
    ns = rng.integers(0, N, 17)
    assert np.array_equal(O.gemm_ref_at(mode, X, packed, ab, N, ms, ns), Y[ms, ns])
    # binary32 scale: the same matmul with the unrounded alpha
    Wf = lev(unpack_codes(packed, mode, K).astype(np.float64)) * alpha.astype(np.float64)[:, None]
    want32 = np.matmul(synth.bf16_bits_to_f32(X).astype(np.float64), Wf.T)
    assert np.allclose(O.gemm_ref_f32a(mode, X, packed, alpha, N), want32, rtol=1e-12, atol=1e-12)


def _word_order_2bit(P):
    """The 2-bit export's reorder inside each 4-byte word, in numpy: the row
    zero-padded to whole words, its 16 codes per word split out (code i in
    bits 2i..2i+1), and byte j rebuilt from codes 2j, 8+2j, 2j+1, 9+2j."""
    rows, rb = P.shape
    rbw = -(-rb // 4) * 4
    pad = np.zeros((rows, rbw), np.uint8)
    pad[:, :rb] = P
    words = pad.reshape(rows, rbw // 4, 4).astype(np.uint32)
    w = words[..., 0] | (words[..., 1] << 8) | (words[..., 2] << 16) | (words[..., 3] << 24)
    k = [(w >> (2 * i)) & 3 for i in range(16)]
    out = np.zeros((rows, rbw // 4, 4), np.uint8)
    for j in range(4):
        out[..., j] = (k[2 * j] | (k[8 + 2 * j] << 2) | (k[2 * j + 1] << 4) | (k[9 + 2 * j] << 6)).astype(np.uint8)
    return out.reshape(rows, rbw)


def _tile_by_reshape(P, cw):
    """The deployment byte order as a numpy index shuffle: (2-bit codes:
    reorder inside each word,) pad to whole tiles and groups, then order the
    axes (group, tile, row, byte)."""
    if cw == 2:
        P = _word_order_2bit(P)
    rows, rb = P.shape
    Np, G = -(-rows // 16) * 16, -(-rb // 64)
    pad = np.zeros((Np, G * 64), np.uint8)
    pad[:rows, :rb] = P
    return pad.reshape(Np // 16, 16, G, 64).transpose(2, 0, 1, 3).reshape(-1)


@pytest.mark.parametrize("cw", [1, 2, 4])
@pytest.mark.parametrize("rows,rb", [(16, 64), (20, 144), (1, 2), (33, 16), (48, 256), (7, 200),
                                     (0, 64), (5, 0), (3, 25), (17, 66)])
def test_tile_codes_matches_axis_shuffle(rows, rb, cw):
    rng = np.random.default_rng(rows * 1000 + rb)
    P = rng.integers(0, 256, (rows, rb), dtype=np.uint8)
    T = O.tile_codes(P, cw)
    assert T.size == O.tiled_bytes(rows, rb) == -(-rb // 64) * (-(-rows // 16) * 16) * 64
    assert np.array_equal(T, _tile_by_reshape(P, cw))


def test_tile_codes_2bit_word_by_hand():
    """One row of 16 2-bit codes k_i = i mod 4 (row-major bytes 0xE4 each):
    export byte j holds k(2j), k(8+2j), k(2j+1), k(9+2j) in bits 0-1, 2-3,
    4-5, 6-7, so bytes 0..3 are 0x50, 0xFA, 0x50, 0xFA (worked out by hand:
    0x50 = 0 | 0 << 2 | 1 << 4 | 1 << 6, 0xFA = 2 | 2 << 2 | 3 << 4 | 3 << 6);
    the rest of the 64-byte group and the 15 padding rows are zero."""
    P = np.full((1, 4), 0xE4, np.uint8)
    T = O.tile_codes(P, 2)
    assert T.size == 16 * 64
    assert list(T[:4]) == [0x50, 0xFA, 0x50, 0xFA]
    assert not T[4:].any()
    # 1- and 4-bit codes keep the row-major bytes
    assert list(O.tile_codes(P, 4)[:4]) == [0xE4] * 4 and list(O.tile_codes(P, 1)[:4]) == [0xE4] * 4


def _e2m1(nib):
    """Value of an e2m1 nibble from the format's definition: sign bit 3,
    exponent bits 2-1 (bias 1), mantissa bit 0; exponent 0 is subnormal."""
    s = -1.0 if nib & 8 else 1.0
    e, m = (nib >> 1) & 3, nib & 1
    return s * (m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1))


def test_tile_codes_2bit_nibbles_decode_in_k_order():
    """What the export order is for: in each word, the nibbles of
    word & 0x33333333 (low nibble of each byte first) are the e2m1 values
    c/2 of codes k0..k7 in order, and those of (word >> 2) & 0x33333333 the
    codes k8..k15 -- checked on random rows through the oracle's tiling."""
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 4, (16, 64))
    P = np.zeros((16, 16), np.uint8)
    for i in range(64):
        P[:, i // 4] |= (codes[:, i] << (2 * (i % 4))).astype(np.uint8)
    T = O.tile_codes(P, 2)
    for r in range(16):
        row = T[r * 64:r * 64 + 16]
        for wi in range(4):
            w = int.from_bytes(bytes(row[4 * wi:4 * wi + 4]), "little")
            got = []
            for m in (w & 0x33333333, (w >> 2) & 0x33333333):
                for n in range(8):
                    got.append(_e2m1((m >> (4 * n)) & 0xF))
            assert got == [c / 2 for c in codes[r, 16 * wi:16 * wi + 16]]


def test_tile_codes_hand_positions():
    # 20 rows of 144 bytes (4-bit codes of 288 weights): 32 padded rows, 3 groups.
    P = (np.arange(20 * 144) % 251 + 1).astype(np.uint8).reshape(20, 144)
    T = O.tile_codes(P, 4)
    assert T.size == 3 * 32 * 64
    # row 17, byte 70: group 1, tile 1, tile row 1, byte 6 of the group
    assert T[((1 * 2 + 1) * 16 + 1) * 64 + 6] == P[17, 70]
    # row 0, byte 143: group 2, tile 0, tile row 0, byte 15
    assert T[(2 * 2 * 16) * 64 + 15] == P[0, 143]
    # row 19, byte 0: group 0, tile 1, tile row 3
    assert T[1024 + 3 * 64] == P[19, 0]
    # row 1, bytes 64..79 follow row 1's group-1 start: tile 0, row 1 of group 1
    assert np.array_equal(T[(1 * 2 * 16 + 1) * 64:(1 * 2 * 16 + 1) * 64 + 16], P[1, 64:80])
    # padding: bytes past the row in its last group (row 0, group 2, bytes 16..63)
    # and rows past 20 (tile 1, rows 4..15, group 0) are zero
    assert not T[(2 * 2 * 16) * 64 + 16:(2 * 2 * 16) * 64 + 64].any()
    assert not T[1024 + 4 * 64:1024 + 16 * 64].any()
    # every stored byte appears exactly once: nonzero bytes are a permutation
    assert np.count_nonzero(T) == P.size
    assert np.array_equal(np.sort(T[T != 0]), np.sort(P.reshape(-1)))


# ----------------------------------------------------------------------------
# Optimizer step (AdamW, decoupled weight decay) and the fused QAT step
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("wd", [0.0, 0.1])
def test_adamw_matches_torch_float64(wd):
    """Five AdamW steps in binary32 against torch.optim.AdamW in float64 (its
    own implementation of the published algorithm): a dropped bias
    correction, eps under the square root or weight decay folded into the
    gradient would move p by far more than the few ulps allowed."""
    rng = np.random.default_rng(77)
    n = 4096
    hp = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd)
    p = (rng.standard_normal(n) * 0.05).astype(np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    tp = torch.nn.Parameter(torch.from_numpy(p.astype(np.float64)))
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=wd, foreach=False)
    for t in range(1, 6):
        g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-6, 0, n)).astype(np.float32)
        p_prev = p
        p, m, v = O.adamw(p, g, m, v, t, **hp)
        tp.grad = torch.from_numpy(g.astype(np.float64))
        opt.step()
        ref = tp.detach().numpy()
        st = opt.state[tp]
        # binary32 roundings of p accumulate over the steps (at most ~t ulps
        # of the larger of p before and after); the update itself is exact to
        # ~1e-7 relative.  Every plausible formula slip moves p by ~lr.
        mag = np.maximum(np.abs(p_prev), np.abs(ref)).astype(np.float32)
        tol = 2 * t * np.spacing(mag) + 1e-6 * hp["lr"]
        assert np.all(np.abs(p - ref) <= tol), f"step {t}"
        mr = st["exp_avg"].numpy()  # a signed running sum: compare on its scale
        assert np.allclose(m, mr, rtol=1e-5, atol=1e-6 * np.abs(mr).max())
        assert np.allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-5, atol=0)


def test_adamw_first_step_closed_form():
    """At t = 1 from zero moments the bias corrections cancel:
    m_hat = g, v_hat = g^2, so p' = p (1 - lr wd) - lr g / (|g| + eps)."""
    rng = np.random.default_rng(78)
    n = 1000
    lr, wd, eps = 3e-3, 0.05, 1e-8
    p = rng.standard_normal(n).astype(np.float32)
    g = (rng.standard_normal(n) * 10.0 ** rng.uniform(-5, 1, n)).astype(np.float32)
    p1, m1, v1 = O.adamw(p, g, np.zeros(n), np.zeros(n), 1, lr, 0.9, 0.999, eps, wd)
    p64, g64 = p.astype(np.float64), g.astype(np.float64)
    want = p64 * (1 - lr * wd) - lr * g64 / (np.abs(g64) + eps)
    mag = np.maximum(np.abs(p64), np.abs(want)).astype(np.float32)
    assert np.all(np.abs(p1 - want) <= 2 * np.spacing(mag) + 1e-6 * lr)
    assert np.allclose(m1, 0.1 * g64, rtol=1e-6)
    assert np.allclose(v1, 0.001 * g64 * g64, rtol=1e-5)


@pytest.mark.parametrize("mode", [O.SEQ2, O.TERNARY, O.LSQ4, O.BINARY])
@pytest.mark.parametrize("g_bf16", [False, True])
def test_qat_step_is_bwd_then_adamw_then_fwd(mode, g_bf16):
    """The fused step's definition, checked against the three pinned pieces
    called one after the other."""
    rng = np.random.default_rng(79 + mode)
    rows, cols = 24, 96
    W = synth.normal_f32(rng, (rows, cols), 0.02)
    alpha = O.alpha_init(mode, W) * np.float32(0.8)
    G = synth.normal_f32(rng, (rows, cols))
    Gin = synth.to_bf16_bits(G) if g_bf16 else G
    mW = synth.normal_f32(rng, (rows, cols), 1e-3)
    vW = np.abs(synth.normal_f32(rng, (rows, cols), 1e-6))
    ma = synth.normal_f32(rng, (rows,), 1e-3)
    va = np.abs(synth.normal_f32(rng, (rows,), 1e-6))
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    out = O.qat_step(mode, W, alpha, Gin, mW, vW, ma, va, 7, **hp)
    dW, da, _ = O.quantize_bwd(mode, W, alpha, Gin)
    W1, mW1, vW1 = O.adamw(W, dW, mW, vW, 7, **hp)
    a1, ma1, va1 = O.adamw(alpha, da, ma, va, 7, **hp)
    wq1, _, codes1 = O.quantize_fwd(mode, W1, a1)
    for k, want in (("W", W1), ("mW", mW1), ("vW", vW1), ("alpha", a1), ("m_alpha", ma1),
                    ("v_alpha", va1), ("wq_bf16", wq1), ("codes", codes1), ("dalpha", da)):
        assert np.array_equal(out[k].view(np.uint8), np.ascontiguousarray(want).view(np.uint8)), k


# ----------------------------------------------------------------------------
# Diagnostics: level occupancy and weight movement
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("mode", [O.BINARY, O.TERNARY, O.SEQ2, O.LSQ3, O.LSQ4])
def test_level_stats_match_bincount_and_scipy(mode):
    import scipy.stats
    rng = np.random.default_rng(90 + mode)
    rows, cols = 40, 264
    W = synth.normal_f32(rng, (rows, cols), 0.02)
    W[3] = 0.0                       # a row with one level only (entropy 0)
    _, _, codes = O.quantize_fwd(mode, W, O.alpha_init(mode, W))
    counts, ent = O.level_stats(mode, codes, cols)
    c = unpack_codes(codes, mode, cols)
    L = {O.BINARY: 2, O.TERNARY: 3, O.SEQ2: 4, O.LSQ3: 8, O.LSQ4: 16}[mode]
    want = np.stack([np.bincount(r, minlength=L) for r in c])
    assert np.array_equal(counts, want)
    assert np.allclose(ent, [scipy.stats.entropy(r, base=2) for r in want], rtol=0, atol=1e-12)
    assert ent[3] == 0.0 and counts.sum() == rows * cols


def test_weight_movement_matches_numpy():
    rng = np.random.default_rng(95)
    W0 = synth.normal_f32(rng, (17, 333), 0.02)
    W = W0 + synth.normal_f32(rng, (17, 333), 1e-4)
    d2, r2 = O.weight_movement(W, W0)
    want_d = ((W.astype(np.float64) - W0.astype(np.float64)) ** 2).sum(axis=1)
    want_r = (W0.astype(np.float64) ** 2).sum(axis=1)
    assert np.allclose(d2, want_d, rtol=1e-13, atol=0)
    assert np.allclose(r2, want_r, rtol=1e-13, atol=0)
    z, _ = O.weight_movement(W0, W0)
    assert not z.any()


def test_seq_levels_carry_more_entropy_than_lsq():
    """[Rebuttal], part on why SEQ beats LSQ: on the same weights with each
    grid's own max-based init, SEQ's equal-width bins spread the weights over
    the levels more evenly than LSQ's grid at 2 bits ({-2,-1,0,1}) and at 1.58
    bits (LSQ's middle bin twice as wide), so the level entropy is higher."""
    rng = np.random.default_rng(97)
    W = synth.normal_f32(rng, (64, 1536), 0.02)
    ent = {}
    for mode in (O.SEQ2, O.LSQ2, O.TERNARY, O.LSQ158):
        _, _, codes = O.quantize_fwd(mode, W, O.alpha_init(mode, W))
        ent[mode] = O.level_stats(mode, codes, 1536)[1].mean()
    assert ent[O.SEQ2] > ent[O.LSQ2] + 0.1
    assert ent[O.TERNARY] > ent[O.LSQ158] + 0.1
    assert ent[O.SEQ2] <= 2.0 and ent[O.TERNARY] <= np.log2(3)
