"""GPU parity of the quantizer path (alpha init, forward, backward, export)
against the CPU oracle, through the C ABI.

Bar: codes, packing, masks, dW, alpha-init (max-based) and fake-quant values
bit-exact (0 ulp; the fp32 and bf16 outputs compared as bit patterns);
dalpha within rel 1e-5 of the oracle (both accumulate in binary64, in
different orders); the 1-bit alpha init (a binary64 mean) at <= 1 ulp.
"""
import numpy as np
import pytest
import torch

import oracle as O
from bit_quantization_aware_amd import synth

from gpu_util import assert_bits_equal, assert_rel, dev, empty_bf16, host

pytestmark = pytest.mark.gpu

pq = None  # the binding, loaded by the module fixture


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global pq
    from bit_quantization_aware_amd import pq as _pq
    pq = _pq
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    O.set_threads(16)
    yield


MODES = [O.BINARY, O.TERNARY, O.SEQ2, O.LSQ3, O.LSQ4, O.LSQ2, O.LSQ158]


def gpu_fwd(mode, W, alpha=None, init=False, want_f32=True):
    rows, cols = W.shape
    Wd = dev(W)
    ad = dev(alpha) if alpha is not None else torch.zeros(rows, dtype=torch.float32, device="cuda")
    wq = empty_bf16(rows, cols)
    wq32 = torch.empty(rows, cols, dtype=torch.float32, device="cuda") if want_f32 else None
    codes = torch.empty(rows, pq.pq_code_row_bytes(mode, cols), dtype=torch.uint8, device="cuda")
    pq.pq_quantize_fwd(mode, rows, cols, Wd, ad, pq.PQ_INIT_ALPHA if init else 0, wq, wq32, codes)
    torch.cuda.synchronize()
    return host(ad), host(wq), (host(wq32) if want_f32 else None), host(codes)


def gpu_bwd(mode, W, alpha, G, grad_scale=None, g_bf16=False, alias=False, want_mask=True):
    rows, cols = W.shape
    if grad_scale is None:
        grad_scale = pq.pq_default_grad_scale(mode, rows, cols)
    Wd, ad = dev(W), dev(alpha)
    Gd = dev(G)
    dW = Gd if alias else torch.empty(rows, cols, dtype=torch.float32, device="cuda")
    da = torch.empty(rows, dtype=torch.float32, device="cuda")
    mask = torch.empty(rows, cols // 8, dtype=torch.uint8, device="cuda") if want_mask else None
    pq.pq_quantize_bwd(mode, rows, cols, Wd, ad, Gd, pq.PQ_G_BF16 if g_bf16 else pq.PQ_G_F32,
                       grad_scale, dW, da, mask)
    torch.cuda.synchronize()
    return host(dW), host(da), (host(mask) if want_mask else None)


def check_fwd(mode, W, alpha, init, what):
    """GPU forward vs oracle.  With init, the oracle computes its own alpha
    (never the GPU's) and both must agree bit for bit -- for the 1-bit mean
    too: the reading allows 1 ulp between binary64 sums taken in different
    orders, but on these seeded inputs they round to the same binary32."""
    a_g, wq_g, wq32_g, codes_g = gpu_fwd(mode, W, alpha, init)
    if init:
        alpha = O.alpha_init(mode, W)
        assert np.all(np.abs(a_g - alpha) <= np.spacing(np.abs(alpha))), what + " alpha > 1 ulp"
        assert_bits_equal(a_g, alpha, what + " alpha")
    wq_o, wq32_o, codes_o = O.quantize_fwd(mode, W, alpha)
    assert_bits_equal(codes_g, codes_o, what + " codes")
    assert_bits_equal(wq32_g, wq32_o, what + " wq_f32")
    assert_bits_equal(wq_g, wq_o, what + " wq_bf16")
    return alpha


def check_bwd(mode, W, alpha, G, what, **kw):
    dW_g, da_g, m_g = gpu_bwd(mode, W, alpha, G, **kw)
    Gin = synth.to_bf16_bits(G) if kw.get("g_bf16") else G
    dW_o, da_o, m_o = O.quantize_bwd(mode, W, alpha, Gin, kw.get("grad_scale"))
    assert_bits_equal(m_g, m_o, what + " mask")
    assert_bits_equal(dW_g, dW_o, what + " dW")
    assert_rel(da_g, da_o, 1e-5, np.float64(1e-35), what + " dalpha")


SHAPES = [(256, 256), (37, 72), (5, 8), (3, 1600), (1, 16384), (4100, 24), (70, 4352)]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", SHAPES)
def test_fwd_bwd_parity(mode, shape):
    rows, cols = shape
    W, G = synth.random_case(1000 + rows + cols + mode, rows, cols)
    print(f"[fwd/bwd mode={mode} shape={shape}]", flush=True)
    alpha = check_fwd(mode, W, None, True, f"init m{mode} {shape}")
    # a given alpha smaller than the init value, so many weights are clipped
    alpha2 = (O.alpha_init(mode, W) * np.float32(0.7)).astype(np.float32)
    check_fwd(mode, W, alpha2, False, f"fwd m{mode} {shape}")
    check_bwd(mode, W, alpha2, G, f"bwd m{mode} {shape}")
    check_bwd(mode, W, alpha, G, f"bwd-init-alpha m{mode} {shape}")


def test_tiny_config_seed0():
    """The 256x256 seed-0 case: 2-bit SEQ, alpha = max|W_row| init, STE backward."""
    W, G, _ = synth.tiny()
    a_g, wq_g, wq32_g, codes_g = gpu_fwd(O.SEQ2, W, None, True)
    a_o = O.alpha_init(O.SEQ2, W)
    assert np.array_equal(a_o, np.abs(W).max(axis=1))
    assert_bits_equal(a_g, a_o, "alpha")
    wq_o, wq32_o, codes_o = O.quantize_fwd(O.SEQ2, W, a_o)
    assert_bits_equal(codes_g, codes_o, "codes")
    assert_bits_equal(wq_g, wq_o, "wq")
    check_bwd(O.SEQ2, W, a_o, G, "tiny bwd")


def adversarial_rows(mode):
    """Rows built to hit the edges: zero rows, exact ties, tiny negatives,
    signed zeros, exact clip bounds, subnormals, exact row maxima."""
    cols = 64
    a = np.float32(2.0 ** -4)
    lo, hi = {O.SEQ2: (-0.99, 0.99), O.TERNARY: (-0.99, 0.99), O.LSQ3: (-4, 3), O.LSQ4: (-8, 7),
              O.BINARY: (-1, 1), O.LSQ2: (-2, 1), O.LSQ158: (-1, 1)}[mode]
    rows = []
    rows.append(np.zeros(cols, np.float32))
    ties = np.array([-0.5, 0.0, 0.5, -1.5 / 1.5, 1.0 / 3.0, -1.0 / 3.0, 2.5, -3.5, 1.5, -2.5],
                    np.float32)
    r = np.resize(ties, cols).astype(np.float32) * a
    rows.append(r)
    tn = np.array([-(2.0 ** -26), -(2.0 ** -25), -0.0, 0.0, 2.0 ** -26, -(2.0 ** -24)], np.float32)
    rows.append(np.resize(tn, cols).astype(np.float32) * a)
    b = np.array([lo, hi, np.nextafter(np.float32(lo), np.float32(-9)),
                  np.nextafter(np.float32(hi), np.float32(9)), 1.0, -1.0], np.float32)
    rows.append(np.resize(b * a, cols).astype(np.float32))
    sub = np.array([1e-45, -1e-45, 1e-40, -3e-39, 1.17e-38, 0.0], np.float32)
    rows.append(np.resize(sub, cols).astype(np.float32))
    rng = np.random.default_rng(5)
    rows.append((rng.standard_normal(cols) * 0.02).astype(np.float32))
    W = np.stack(rows).astype(np.float32)
    alpha = np.full(W.shape[0], a, np.float32)
    alpha[0] = 0.0        # all-zero row with a zero scale
    alpha[4] = 1e-38      # subnormal row with a scale under the floor
    return W, alpha


@pytest.mark.parametrize("mode", MODES)
def test_adversarial_rows(mode):
    W, alpha = adversarial_rows(mode)
    G = np.random.default_rng(6).standard_normal(W.shape).astype(np.float32)
    check_fwd(mode, W, alpha, False, f"adv fwd m{mode}")
    check_fwd(mode, W, None, True, f"adv init m{mode}")
    check_bwd(mode, W, alpha, G, f"adv bwd m{mode}")


@pytest.mark.parametrize("mode", [O.SEQ2, O.TERNARY, O.LSQ4])
def test_bwd_bf16_gradient_and_aliasing(mode):
    W, G = synth.random_case(77, 96, 520)
    alpha = (O.alpha_init(mode, W) * np.float32(0.8)).astype(np.float32)
    Gb = synth.bf16_bits_to_f32(synth.to_bf16_bits(G))
    dW_g, da_g, _ = gpu_bwd(mode, W, alpha, synth.to_bf16_bits(G), g_bf16=True)
    dW_o, da_o, _ = O.quantize_bwd(mode, W, alpha, synth.to_bf16_bits(G))
    assert_bits_equal(dW_g, dW_o, "bf16 G dW")
    assert_rel(da_g, da_o, 1e-5, np.float64(1e-35), "bf16 G dalpha")
    # dW written over G in place
    dW_a, da_a, m_a = gpu_bwd(mode, W, alpha, G, alias=True)
    dW_o, da_o, m_o = O.quantize_bwd(mode, W, alpha, G)
    assert_bits_equal(dW_a, dW_o, "aliased dW")
    assert_bits_equal(m_a, m_o, "aliased mask")
    del Gb


def test_explicit_grad_scale_and_null_optionals():
    W, G = synth.random_case(78, 40, 96)
    alpha = O.alpha_init(O.LSQ3, W)
    dW_g, da_g, _ = gpu_bwd(O.LSQ3, W, alpha, G, grad_scale=0.37, want_mask=False)
    dW_o, da_o, _ = O.quantize_bwd(O.LSQ3, W, alpha, G, 0.37)
    assert_bits_equal(dW_g, dW_o, "dW")
    assert_rel(da_g, da_o, 1e-5, np.float64(1e-35), "dalpha")
    # codes only, no value outputs
    rows, cols = W.shape
    codes = torch.empty(rows, cols // 2, dtype=torch.uint8, device="cuda")
    pq.pq_quantize_fwd(O.LSQ3, rows, cols, dev(W), dev(alpha), 0, None, None, codes)
    torch.cuda.synchronize()
    assert_bits_equal(host(codes), O.quantize_fwd(O.LSQ3, W, alpha)[2], "codes only")


def test_zero_rows_is_a_no_op():
    W = torch.zeros(0, 64, device="cuda")
    a = torch.zeros(1, device="cuda")
    pq.pq_quantize_fwd(O.SEQ2, 0, 64, W if W.numel() else a, a, 0, None, None, None)
    pq.pq_quantize_bwd(O.SEQ2, 0, 64, a, a, a, 0, 1.0, None, a, None)
    torch.cuda.synchronize()


def test_deterministic_dalpha():
    W, G = synth.random_case(79, 300, 4096)
    alpha = O.alpha_init(O.SEQ2, W)
    runs = [gpu_bwd(O.SEQ2, W, alpha, G)[1] for _ in range(3)]
    assert all(np.array_equal(runs[0].view(np.uint32), r.view(np.uint32)) for r in runs)


def gpu_pack(mode, W, alpha):
    """Export on the GPU into a buffer prefilled with 0xA5, so that a byte the
    kernel does not write (padding included) shows up."""
    rows, cols = W.shape
    nbytes = pq.pq_packed_bytes(mode, rows, cols)
    packed = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    ab = empty_bf16(rows)
    if mode == O.SEQ2:
        pq.pq_pack_w2(rows, cols, dev(W), dev(alpha), packed, ab)
    elif mode == O.LSQ4:
        pq.pq_pack_w4(rows, cols, dev(W), dev(alpha), packed, ab)
    else:
        pq.pq_pack(mode, rows, cols, dev(W), dev(alpha), packed, ab)
    torch.cuda.synchronize()
    return host(packed), host(ab)


@pytest.mark.parametrize("mode", [O.SEQ2, O.LSQ4, O.TERNARY, O.LSQ3, O.BINARY])
def test_pack_matches_forward_codes(mode):
    # 333 rows (three padding rows in the last tile), 1600 columns (a partly
    # filled last 64-byte group at both widths)
    W, _ = synth.random_case(80, 333, 1600)
    alpha = O.alpha_init(mode, W)
    packed, ab = gpu_pack(mode, W, alpha)
    p_o, ab_o = O.pack(mode, W, alpha)
    assert_bits_equal(packed, O.tile_codes(p_o, O.CODE_BITS[mode]), "packed")
    assert_bits_equal(ab, ab_o, "alpha bf16")
    _, _, _, codes_fwd = gpu_fwd(mode, W, alpha, False, want_f32=False)
    assert_bits_equal(packed, O.tile_codes(codes_fwd, O.CODE_BITS[mode]), "pack == fwd codes in export order")


@pytest.mark.parametrize("mode", [O.SEQ2, O.LSQ4, O.TERNARY, O.LSQ3, O.LSQ2, O.LSQ158, O.BINARY])
@pytest.mark.parametrize("rows,cols", [(1, 8), (17, 64), (16, 1024), (4100, 264), (4096, 520), (8192, 256)])
def test_pack_export_order_shapes(mode, rows, cols):
    """Export byte order across the launch shapes: one row per block (fewer
    than 4096 rows) and one per wave, with and without the XCD row remap
    (block count a multiple of 8 or not), padding rows and partial groups."""
    rng = np.random.default_rng(rows * 7 + cols)
    W = synth.normal_f32(rng, (rows, cols), 0.02)
    alpha = O.alpha_init(mode, W)
    packed, ab = gpu_pack(mode, W, alpha)
    p_o, ab_o = O.pack(mode, W, alpha)
    assert_bits_equal(packed, O.tile_codes(p_o, O.CODE_BITS[mode]), f"packed {rows}x{cols}")
    assert_bits_equal(ab, ab_o, "alpha bf16")


# ----------------------------------------------------------------------------
# Grouped launches, as the benchmark runs them
# ----------------------------------------------------------------------------
def run_grouped(mode, mats, init):
    """mats: list of (W, G) numpy pairs.  Returns per-matrix host outputs."""
    dev_mats, descs = [], []
    for W, G in mats:
        rows, cols = W.shape
        d = dict(W=dev(W), alpha=torch.zeros(rows, dtype=torch.float32, device="cuda"),
                 wq_bf16=empty_bf16(rows, cols),
                 codes=torch.empty(rows, pq.pq_code_row_bytes(mode, cols), dtype=torch.uint8,
                                   device="cuda"),
                 G=dev(G), dW=torch.empty(rows, cols, dtype=torch.float32, device="cuda"),
                 dalpha=torch.empty(rows, dtype=torch.float32, device="cuda"),
                 mask_bits=torch.empty(rows, cols // 8, dtype=torch.uint8, device="cuda"),
                 grad_scale=pq.pq_default_grad_scale(mode, rows, cols), rows=rows, cols=cols)
        dev_mats.append(d)
    fwd_t = pq.MatTable([{k: d[k] for k in ("W", "alpha", "wq_bf16", "codes", "rows", "cols")}
                         for d in dev_mats])
    bwd_t = pq.MatTable([{k: d[k] for k in ("W", "alpha", "G", "dW", "dalpha", "mask_bits",
                                            "grad_scale", "rows", "cols")} for d in dev_mats])
    if not init:
        for d, (W, _) in zip(dev_mats, mats):
            d["alpha"].copy_(dev(O.alpha_init(mode, W)))
    pq.pq_quantize_fwd_grouped(mode, fwd_t, pq.PQ_INIT_ALPHA if init else 0)
    pq.pq_quantize_bwd_grouped(mode, bwd_t, pq.PQ_G_F32)
    torch.cuda.synchronize()
    return [{k: host(d[k]) for k in ("alpha", "wq_bf16", "codes", "dW", "dalpha", "mask_bits")}
            for d in dev_mats]


def check_grouped(mode, mats, outs, what):
    for i, ((W, G), o) in enumerate(zip(mats, outs)):
        a_o = O.alpha_init(mode, W)
        assert_bits_equal(o["alpha"], a_o, f"{what}[{i}] alpha")
        wq_o, _, codes_o = O.quantize_fwd(mode, W, a_o)
        assert_bits_equal(o["codes"], codes_o, f"{what}[{i}] codes")
        assert_bits_equal(o["wq_bf16"], wq_o, f"{what}[{i}] wq")
        dW_o, da_o, m_o = O.quantize_bwd(mode, W, a_o, G)
        assert_bits_equal(o["mask_bits"], m_o, f"{what}[{i}] mask")
        assert_bits_equal(o["dW"], dW_o, f"{what}[{i}] dW")
        assert_rel(o["dalpha"], da_o, 1e-5, np.float64(1e-35), f"{what}[{i}] dalpha")


@pytest.mark.parametrize("mode", MODES)
def test_grouped_mixed_stack(mode):
    shapes = [(576, 576), (1536, 576), (576, 1536), (3, 8), (0, 64), (129, 72), (400, 1600)]
    mats = [synth.random_case(90 + i, r, c) for i, (r, c) in enumerate(shapes)]
    print(f"[grouped mixed mode={mode}]", flush=True)
    outs = run_grouped(mode, mats, init=True)
    check_grouped(mode, mats, outs, f"mixed m{mode}")


@pytest.mark.parametrize("mode", MODES)
def test_mobilellm_125m_full_stack(mode):
    """All 210 matrices of the 125M stack in one grouped fwd and one grouped
    bwd launch (the benchmark's launch configuration), every output checked."""
    n = len(synth.mobilellm_125m_shapes())
    mats = [(synth.weight("mobilellm_125m", k), synth.upstream_grad("mobilellm_125m", k))
            for k in range(n)]
    print(f"[125M stack mode={mode}: {n} matrices]", flush=True)
    outs = run_grouped(mode, mats, init=True)
    check_grouped(mode, mats, outs, f"125M m{mode}")


def test_mobilellm_1p5b_layers_with_outliers():
    """MobileLLM-1.5B-shaped layers (hidden 1600, FFN 4352, GQA kv width 400;
    weights ~N(0, 0.02^2) with 0.1 % of them scaled by 10): the 7 matrices of
    layers 0, 27 and 53 in one grouped 2-bit fwd + bwd launch, every output
    checked, then the packed export of each matrix."""
    shapes = synth.mobilellm_1p5b_shapes()
    ks = [k for k, (l, _, _, _) in enumerate(shapes) if l in (0, 27, 53)]
    mats = [(synth.weight("mobilellm_1p5b", k), synth.upstream_grad("mobilellm_1p5b", k)) for k in ks]
    assert any(np.abs(W).max() > 0.15 for W, _ in mats), "outliers present"
    print(f"[1.5B layers 0/27/53: {len(mats)} matrices]", flush=True)
    outs = run_grouped(O.SEQ2, mats, init=True)
    check_grouped(O.SEQ2, mats, outs, "1.5B")
    for i, ((W, _), o) in enumerate(zip(mats, outs)):
        rows, cols = W.shape
        packed, ab = gpu_pack(O.SEQ2, W, o["alpha"])
        p_o, ab_o = O.pack(O.SEQ2, W, o["alpha"])
        assert_bits_equal(packed, O.tile_codes(p_o, O.CODE_BITS[O.SEQ2]), f"1.5B[{i}] packed")
        assert_bits_equal(ab, ab_o, f"1.5B[{i}] alpha bf16")


@pytest.mark.parametrize("mode", [O.SEQ2, O.TERNARY])
def test_llama3_8b_projections(mode):
    """The four Llama-3-8B projection shapes (4096x4096, 1024x4096,
    14336x4096, 4096x14336; weights ~N(0, 0.015^2)) in one grouped fwd + bwd
    launch, 2-bit SEQ and ternary, every output checked."""
    n = len(synth.llama3_8b_shapes())
    mats = [(synth.weight("llama3_8b", k), synth.upstream_grad("llama3_8b", k)) for k in range(n)]
    print(f"[Llama-3-8B projections mode={mode}]", flush=True)
    outs = run_grouped(mode, mats, init=True)
    check_grouped(mode, mats, outs, f"llama m{mode}")


BOUNDARIES = {
    O.SEQ2: [0.0, 0.5, -0.5, 0.99, -0.99, 0.25, -0.75],
    O.TERNARY: [1.0 / 3.0, -1.0 / 3.0, 0.99, -0.99, 0.0],
    O.LSQ3: [-4.0, 3.0, -3.5, 2.5, 0.5, -0.5, 1.5],
    O.LSQ4: [-8.0, 7.0, -7.5, 6.5, 0.5, -0.5, 3.5],
    O.BINARY: [1.0, -1.0, 0.0],
    O.LSQ2: [-2.0, 1.0, -1.5, -0.5, 0.5],
    O.LSQ158: [-1.0, 1.0, -0.5, 0.5, 0.0],
}


@pytest.mark.parametrize("mode", MODES)
def test_division_at_decision_boundaries(mode):
    """w / alpha is computed on the GPU as a binary64 product with 1/alpha;
    it must round exactly like the IEEE binary32 division wherever the result
    decides a code or a mask bit: weights at fl32(b * alpha) and +-3 ulps for
    every decision boundary b, over 300 log-spread scales."""
    rng = np.random.default_rng(300 + mode)
    alphas = np.exp(rng.uniform(np.log(1e-4), np.log(30.0), 300)).astype(np.float32)
    cols_raw = []
    for b in BOUNDARIES[mode]:
        w0 = (np.float32(b) * alphas).astype(np.float32)
        for k in range(-3, 4):
            w = w0.copy()
            step = np.float32(np.inf) if k > 0 else np.float32(-np.inf)
            for _ in range(abs(k)):
                w = np.nextafter(w, step).astype(np.float32)
            cols_raw.append(w)
    W = np.stack(cols_raw, axis=1).astype(np.float32)
    pad = (-W.shape[1]) % 8
    W = np.concatenate([W, np.zeros((W.shape[0], pad), np.float32)], axis=1)
    G = rng.standard_normal(W.shape).astype(np.float32)
    check_fwd(mode, W, alphas, False, f"div-boundary fwd m{mode}")
    check_bwd(mode, W, alphas, G, f"div-boundary bwd m{mode}")


@pytest.mark.parametrize("mode", [O.TERNARY, O.SEQ2, O.LSQ3, O.LSQ4, O.LSQ2, O.LSQ158, O.BINARY])
@pytest.mark.parametrize("rows,cols,init", [(333, 1600, True), (4100, 264, False), (17, 64, True),
                                            (64, 16384, False)])
def test_fwd_codes_in_export_order(mode, rows, cols, init):
    """PQ_CODES_EXPORT: the forward's codes in the export byte order (padding
    zeroed), its bf16 weights and alpha unchanged."""
    rng = np.random.default_rng(rows + cols + mode)
    W = synth.normal_f32(rng, (rows, cols), 0.02)
    alpha = None if init else O.alpha_init(mode, W) * np.float32(0.9)
    ad = dev(alpha) if alpha is not None else torch.zeros(rows, dtype=torch.float32, device="cuda")
    wq = empty_bf16(rows, cols)
    codes = torch.full((pq.pq_packed_bytes(mode, rows, cols),), 0xA5, dtype=torch.uint8, device="cuda")
    flags = pq.PQ_CODES_EXPORT | (pq.PQ_INIT_ALPHA if init else 0)
    pq.pq_quantize_fwd(mode, rows, cols, dev(W), ad, flags, wq, None, codes)
    torch.cuda.synchronize()
    a_o = O.alpha_init(mode, W) if init else alpha
    wq_o, _, codes_o = O.quantize_fwd(mode, W, a_o)
    assert_bits_equal(host(ad), a_o, "alpha")
    assert_bits_equal(host(wq), wq_o, "wq")
    assert_bits_equal(host(codes), O.tile_codes(codes_o, O.CODE_BITS[mode]), "codes (export order)")


def test_grouped_fwd_codes_in_export_order():
    """The grouped forward over MobileLLM-125M layer 0 (576- and 1536-wide
    rows) writing export-order codes only, as the training forward that feeds
    pq_gemm_f32a does."""
    mode = O.SEQ2
    shapes = synth.mobilellm_125m_shapes()
    ks = [k for k, (l, _, _, _) in enumerate(shapes) if l == 0]
    mats, Ws = [], []
    for k in ks:
        W = synth.weight("mobilellm_125m", k)
        rows, cols = W.shape
        Ws.append(W)
        mats.append(dict(W=dev(W), alpha=torch.zeros(rows, dtype=torch.float32, device="cuda"),
                         codes=torch.full((pq.pq_packed_bytes(mode, rows, cols),), 0xA5, dtype=torch.uint8,
                                          device="cuda"), rows=rows, cols=cols))
    table = pq.MatTable(mats)
    pq.pq_quantize_fwd_grouped(mode, table, pq.PQ_INIT_ALPHA | pq.PQ_CODES_EXPORT)
    torch.cuda.synchronize()
    for W, m in zip(Ws, mats):
        a_o = O.alpha_init(mode, W)
        _, _, codes_o = O.quantize_fwd(mode, W, a_o)
        assert_bits_equal(host(m["alpha"]), a_o, "alpha")
        assert_bits_equal(host(m["codes"]), O.tile_codes(codes_o, O.CODE_BITS[mode]), f"codes {W.shape}")


# ----------------------------------------------------------------------------
# The MobileLLM-1.5B stack at full size, the split of very large stacks, and
# canary guards around every output
# ----------------------------------------------------------------------------
def _gen_1p5b(k):
    return synth.weight("mobilellm_1p5b", k), synth.upstream_grad("mobilellm_1p5b", k)


@pytest.mark.timeout(900)
def test_mobilellm_1p5b_full_stack():
    """All 378 matrices of the MobileLLM-1.5B-shaped stack (1,473,638,400
    weights, 0.1 % outliers x10) through one grouped 2-bit fwd launch (alpha
    init), one grouped bwd launch and one grouped export launch -- the
    benchmark's launch configuration -- with every output of every matrix
    checked against the oracle.  The inputs are regenerated on the host from
    each matrix's seed stream for the comparison, so host memory holds one
    chunk of matrices at a time."""
    from concurrent.futures import ThreadPoolExecutor

    mode = O.SEQ2
    shapes = synth.mobilellm_1p5b_shapes()
    n = len(shapes)
    assert n == 378 and sum(r * c for _, _, r, c in shapes) == 1473638400
    print(f"[1.5B full stack: {n} matrices, upload]", flush=True)
    mats = []
    with ThreadPoolExecutor(16) as ex:
        for c0 in range(0, n, 32):
            for k, (W, G) in zip(range(c0, min(n, c0 + 32)), ex.map(_gen_1p5b, range(c0, min(n, c0 + 32)))):
                rows, cols = W.shape
                mats.append(dict(
                    W=dev(W), G=dev(G), alpha=torch.zeros(rows, dtype=torch.float32, device="cuda"),
                    wq_bf16=empty_bf16(rows, cols),
                    codes=torch.empty(rows, cols // 4, dtype=torch.uint8, device="cuda"),
                    dW=torch.empty(rows, cols, dtype=torch.float32, device="cuda"),
                    dalpha=torch.empty(rows, dtype=torch.float32, device="cuda"),
                    mask_bits=torch.empty(rows, cols // 8, dtype=torch.uint8, device="cuda"),
                    packed=torch.full((pq.pq_packed_bytes(mode, rows, cols),), 0xA5, dtype=torch.uint8,
                                      device="cuda"),
                    alpha_bf16=empty_bf16(rows), grad_scale=pq.pq_default_grad_scale(mode, rows, cols),
                    rows=rows, cols=cols))
    fwd_t = pq.MatTable([{k: d[k] for k in ("W", "alpha", "wq_bf16", "codes", "rows", "cols")} for d in mats])
    bwd_t = pq.MatTable([{k: d[k] for k in ("W", "alpha", "G", "dW", "dalpha", "mask_bits", "grad_scale",
                                            "rows", "cols")} for d in mats])
    exp_t = pq.MatTable([dict(W=d["W"], alpha=d["alpha"], codes=d["packed"], alpha_bf16=d["alpha_bf16"],
                              rows=d["rows"], cols=d["cols"]) for d in mats])
    print("[1.5B full stack: grouped fwd (init) + bwd + export]", flush=True)
    pq.pq_quantize_fwd_grouped(mode, fwd_t, pq.PQ_INIT_ALPHA)
    pq.pq_quantize_bwd_grouped(mode, bwd_t, pq.PQ_G_F32)
    pq.pq_pack_grouped(mode, exp_t)
    torch.cuda.synchronize()
    print("[1.5B full stack: checking]", flush=True)
    with ThreadPoolExecutor(4) as ex:
        for c0 in range(0, n, 16):
            ks = list(range(c0, min(n, c0 + 16)))
            for k, (W, G) in zip(ks, ex.map(_gen_1p5b, ks)):
                d = mats[k]
                a_o = O.alpha_init(mode, W)
                assert_bits_equal(host(d["alpha"]), a_o, f"1.5B[{k}] alpha")
                wq_o, _, codes_o = O.quantize_fwd(mode, W, a_o)
                assert_bits_equal(host(d["codes"]), codes_o, f"1.5B[{k}] codes")
                assert_bits_equal(host(d["wq_bf16"]), wq_o, f"1.5B[{k}] wq")
                dW_o, da_o, m_o = O.quantize_bwd(mode, W, a_o, G)
                assert_bits_equal(host(d["mask_bits"]), m_o, f"1.5B[{k}] mask")
                assert_bits_equal(host(d["dW"]), dW_o, f"1.5B[{k}] dW")
                assert_rel(host(d["dalpha"]), da_o, 1e-5, np.float64(1e-35), f"1.5B[{k}] dalpha")
                p_o, ab_o = O.pack(mode, W, a_o)
                assert_bits_equal(host(d["packed"]), O.tile_codes(p_o, O.CODE_BITS[mode]), f"1.5B[{k}] packed")
                assert_bits_equal(host(d["alpha_bf16"]), ab_o, f"1.5B[{k}] alpha bf16")
            if c0 % 64 == 0:
                print(f"[1.5B full stack: {min(n, c0 + 16)} of {n} checked]", flush=True)


@pytest.mark.parametrize("mode", [O.SEQ2, O.BINARY, O.LSQ4])
def test_grouped_stack_beyond_one_launch(mode):
    """A stack of 1000 matrices: more than one launch table holds (448 per
    launch), so the grouped calls split it into three launches; every output
    of every matrix checked, fwd with alpha init, bwd and export."""
    shapes = [(16, 64), (3, 8), (40, 136), (1, 8), (17, 72), (64, 256), (5, 16), (33, 40)]
    mats = [synth.random_case(5000 + i, *shapes[i % len(shapes)]) for i in range(1000)]
    print(f"[grouped 1000 matrices mode={mode}]", flush=True)
    outs = run_grouped(mode, mats, init=True)
    check_grouped(mode, mats, outs, f"1000-stack m{mode}")
    # the same stack through the grouped export
    dmats = []
    for W, _ in mats:
        rows, cols = W.shape
        dmats.append(dict(W=dev(W), alpha=dev(O.alpha_init(mode, W)),
                          codes=torch.full((pq.pq_packed_bytes(mode, rows, cols),), 0xA5, dtype=torch.uint8,
                                           device="cuda"), alpha_bf16=empty_bf16(rows), rows=rows, cols=cols))
    pq.pq_pack_grouped(mode, pq.MatTable(dmats))
    torch.cuda.synchronize()
    for i, ((W, _), d) in enumerate(zip(mats, dmats)):
        p_o, ab_o = O.pack(mode, W, O.alpha_init(mode, W))
        assert_bits_equal(host(d["codes"]), O.tile_codes(p_o, O.CODE_BITS[mode]), f"1000-stack[{i}] packed")
        assert_bits_equal(host(d["alpha_bf16"]), ab_o, f"1000-stack[{i}] alpha bf16")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("shape", [(37, 72), (5, 8), (4100, 24), (1, 16384), (70, 4352)])
def test_outputs_stay_inside_their_buffers(mode, shape):
    """Every fwd / bwd / export output sits between 256-byte canary guards
    (0xA5); after the calls the guards are intact and the outputs match the
    oracle (ragged rows, one row, many short rows, long rows)."""
    from gpu_util import Guarded

    rows, cols = shape
    W, G = synth.random_case(6000 + rows + cols + mode, rows, cols)
    a_o = O.alpha_init(mode, W)
    alpha = Guarded((rows,), torch.float32)
    wq = Guarded((rows, cols), torch.bfloat16)
    wq32 = Guarded((rows, cols), torch.float32)
    codes = Guarded((rows, pq.pq_code_row_bytes(mode, cols)), torch.uint8)
    pq.pq_quantize_fwd(mode, rows, cols, dev(W), alpha.t, pq.PQ_INIT_ALPHA, wq.t, wq32.t, codes.t)
    dW = Guarded((rows, cols), torch.float32)
    da = Guarded((rows,), torch.float32)
    mask = Guarded((rows, cols // 8), torch.uint8)
    pq.pq_quantize_bwd(mode, rows, cols, dev(W), dev(a_o), dev(G), pq.PQ_G_F32,
                       pq.pq_default_grad_scale(mode, rows, cols), dW.t, da.t, mask.t)
    packed = Guarded((pq.pq_packed_bytes(mode, rows, cols),), torch.uint8)
    ab = Guarded((rows,), torch.bfloat16)
    pq.pq_pack(mode, rows, cols, dev(W), dev(a_o), packed.t, ab.t)
    torch.cuda.synchronize()
    for name, g in (("alpha", alpha), ("wq_bf16", wq), ("wq_f32", wq32), ("codes", codes), ("dW", dW),
                    ("dalpha", da), ("mask", mask), ("packed", packed), ("alpha_bf16", ab)):
        g.check(f"m{mode} {shape} {name}")
    wq_o, wq32_o, codes_o = O.quantize_fwd(mode, W, a_o)
    assert_bits_equal(host(alpha.t), a_o, "alpha")
    assert_bits_equal(host(codes.t), codes_o, "codes")
    assert_bits_equal(host(wq.t), wq_o, "wq")
    assert_bits_equal(host(wq32.t), wq32_o, "wq32")
    dW_o, da_o, m_o = O.quantize_bwd(mode, W, a_o, G)
    assert_bits_equal(host(dW.t), dW_o, "dW")
    assert_bits_equal(host(mask.t), m_o, "mask")
    assert_rel(host(da.t), da_o, 1e-5, np.float64(1e-35), "dalpha")
    p_o, ab_o = O.pack(mode, W, a_o)
    assert_bits_equal(host(packed.t), O.tile_codes(p_o, O.CODE_BITS[mode]), "packed")
    assert_bits_equal(host(ab.t), ab_o, "alpha bf16")
