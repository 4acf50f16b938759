// pq_gemm.hip -- gfx950 deployment GEMM with packed low-bit weights and bf16
// activations:  Y[m, n] = bf16( alpha[n] * sum_k X[m, k] * level(code[n, k]) ).
//
// Sources (web pages, cited by title and section):
//   [News] "Meta's ParetoQ compares five bit widths and puts the accuracy
//          cliff at 1 bit" -- speed paragraph: a 2-bit-weight GEMM timed
//          against FP16 and against a 4-bit kernel at a 16384 x 16384
//          weight, where in-kernel conversion overhead decides the end-to-end
//          gain.
//   [Note] "ParetoQ, the strongest low-bit QAT I could find" -- "Paper vs.
//          code": the layer has no bias; SEQ 2-bit levels {+-1/4, +-3/4}.
//
// Design (gfx950, 64-wide waves, bf16 MFMA 16x16x32):
//  * The contraction runs on MFMA in bf16 with fp32 accumulation.  Weights
//    reach the MFMA B operand straight from packed codes, decoded in
//    registers.  2-bit codes use gfx950's fp4 -> bf16 pair convert
//    (v_cvt_scalef32_pk_bf16_fp4, scale 1): after masking, a nibble 0..3
//    reads as the fp4 value c/2, so level = (c - 1.5)/2 = c/2 - 0.75; the
//    kernel accumulates X.(c/2) on MFMA and subtracts 0.75 * rowsum(X) in
//    the epilogue.  4-bit codes use the bf16 mantissa: 0x4000 | c << 3 is
//    2 + c/8, so level = c - 8 = 8 * (v - 3).
//  * A dword of codes holds 16 (2-bit) or 8 (4-bit) consecutive k.  The
//    2-bit convert reads nibbles, so d & 0x33333333 and (d >> 2) & 0x33333333
//    give the pairs (4b, 4b+2) and (4b+1, 4b+3) of byte b; 4-bit codes pair
//    (i, i+4).  The MFMA sums over k in any order as long as A and B agree,
//    so X is staged in that same order (a fixed permutation inside each 16-
//    or 8-wide k block), and the A operand is a contiguous 16-byte LDS read.
//  * X tiles go global -> registers -> LDS (padded rows, no bank conflicts),
//    one stage ahead of the MFMA work; code tiles go global -> registers,
//    one stage ahead.  The X row sums are taken while staging.
//  * Tile shapes: see the streaming kernel below for M <= 16; the tiled
//    kernel covers larger M (MFMA-bound), with wide column tiles so the
//    activations are re-read from L2 as few times as possible.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pq_common.hpp"

// Streaming-kernel shape: waves per block and groups in flight per wave.
// Tiled kernel shapes <TM, TN, WM, WN, BK> for 16 < M <= 64 and M > 64.
#ifndef PQ_TILE_MID
#define PQ_TILE_MID 2, 1, 2, 2, 256
#endif
#ifndef PQ_TILE_BIG
#define PQ_TILE_BIG 4, 4, 2, 2, 128
#endif
#ifndef PQ_STREAM_NW
#define PQ_STREAM_NW 4
#endif
#ifndef PQ_STREAM_P
#define PQ_STREAM_P 3
#endif
#ifndef PQ_STREAM_TN
#define PQ_STREAM_TN 2
#endif

namespace pq {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}
typedef float floatx4 __attribute__((ext_vector_type(4)));

struct GemmArgs {
    const uint16_t *X;       // [M, K] bf16
    const uint8_t *packed;   // [N, K * BITS / 8]
    const uint16_t *alpha;   // [N] bf16
    uint16_t *Y;             // [M, N] bf16
    int M, N, K;
};

// Decode of one 4-bit output bf16x2 from a dword of codes: nibbles I and
// I+4 -> mantissa bits 3-6 of each half of bf16 2.0, i.e. 2 + c/8.
template <int I>
__device__ __forceinline__ uint32_t decode_pair4(uint32_t d)
{
    constexpr int sh = 4 * I - 3;
    uint32_t t;
    if constexpr (sh >= 0) t = d >> sh;
    else t = d << (-sh);
    return (t & 0x00780078u) | 0x40004000u;
}

// B operand (8 bf16) for MFMA k-step T of a stage from the lane's code dwords.
// 2-bit: dword T/2; its even codes (T even) or odd codes (T odd) as exact
// bf16 c/2 through the fp4 convert (pairs (4b, 4b+2) resp. (4b+1, 4b+3)).
// 4-bit: dword T, pairs (i, i+4).
template <int BITS, int T>
__device__ __forceinline__ bf16x8 decode_b(const uint32_t *cw)
{
    uint4 r;
    if constexpr (BITS == 2) {
        const uint32_t d = cw[T >> 1];
        const uint32_t m = ((T & 1) ? (d >> 2) : d) & 0x33333333u;
        r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m, 1.0f, 0));
        r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m, 1.0f, 1));
        r.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m, 1.0f, 2));
        r.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m, 1.0f, 3));
    } else {
        const uint32_t d = cw[T];
        r.x = decode_pair4<0>(d);
        r.y = decode_pair4<1>(d);
        r.z = decode_pair4<2>(d);
        r.w = decode_pair4<3>(d);
    }
    return __builtin_bit_cast(bf16x8, r);
}

template <int BITS, int TM, int TN, int WM, int WN, int BK>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g)
{
    static_assert(WM * WN == 4, "four waves per block");
    static_assert(BK == 128 || BK == 256, "code loads are 8- or 16-byte (2-bit) / 16- or 32-byte (4-bit) per lane");
    constexpr int BM = 16 * TM * WM;
    constexpr int BN = 16 * TN * WN;
    constexpr int KSTEPS = BK / 32;               // MFMA k-steps per stage
    constexpr int CW = BK * BITS / 128;           // code dwords per lane per tile per stage
    constexpr int CH = BITS == 2 ? 16 : 8;        // X staging chunk (elements), one permutation block
    constexpr int CPR = BK / CH;                  // chunks per X row per stage
    constexpr int NCHUNK = BM * CPR;
    constexpr int NCT = (NCHUNK + 255) / 256;     // chunks per thread
    constexpr int LDS_ROW = BK + 8;               // bf16 per LDS row (+16 bytes of padding)
    static_assert(CPR <= 64 && (64 % CPR) == 0, "a row's chunks stay inside one wave");

    __shared__ __attribute__((aligned(16))) uint16_t xs[BM * LDS_ROW];
    __shared__ float ssum[BM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int i16 = lane & 15, grp = lane >> 4;

    const int M = g.M, N = g.N, K = g.K;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int64_t row_bytes = static_cast<int64_t>(K) * BITS / 8;

    // This lane's weight rows (one per N tile) and their validity.
    const uint8_t *crow[TN];
    bool cval[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * 16 * TN + j * 16 + i16;
        cval[j] = n < N;
        crow[j] = g.packed + static_cast<int64_t>(cval[j] ? n : 0) * row_bytes;
    }

    floatx4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    float xsum[NCT];
#pragma unroll
    for (int r = 0; r < NCT; ++r) xsum[r] = 0.f;

    // Register stages: X chunks and code dwords for the next stage.
    uint4 xr[NCT][CH / 8];
    uint32_t cnext[TN][CW];
    uint32_t ccur[TN][CW];

    auto load_stage = [&](int kb) {
#pragma unroll
        for (int r = 0; r < NCT; ++r) {
            const int c = tid + 256 * r;
            const int row = c / CPR, kc = c % CPR;
            const int m = m0 + row;
            const int k = kb + kc * CH;
            const bool v = (c < NCHUNK) && (m < M) && (k < K);
            const uint4 *src = reinterpret_cast<const uint4 *>(g.X + static_cast<int64_t>(v ? m : 0) * K + (v ? k : 0));
#pragma unroll
            for (int h = 0; h < CH / 8; ++h) xr[r][h] = v ? src[h] : make_uint4(0, 0, 0, 0);
        }
        // codes: lane group grp covers k in [kb + grp*BK/4, kb + (grp+1)*BK/4)
        const int kq = kb + grp * (BK / 4);
        const bool kv = kq < K;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const bool v = kv && cval[j];
            const uint8_t *p = crow[j] + (v ? static_cast<int64_t>(kq) * BITS / 8 : 0);
            if constexpr (CW == 2) {
                const uint2 t = v ? *reinterpret_cast<const uint2 *>(p) : make_uint2(0, 0);
                cnext[j][0] = t.x;
                cnext[j][1] = t.y;
            } else {
#pragma unroll
                for (int q = 0; q < CW / 4; ++q) {
                    const uint4 t = v ? reinterpret_cast<const uint4 *>(p)[q] : make_uint4(0, 0, 0, 0);
                    cnext[j][4 * q + 0] = t.x;
                    cnext[j][4 * q + 1] = t.y;
                    cnext[j][4 * q + 2] = t.z;
                    cnext[j][4 * q + 3] = t.w;
                }
            }
        }
    };

    auto store_stage = [&]() {
#pragma unroll
        for (int r = 0; r < NCT; ++r) {
            const int c = tid + 256 * r;
            if (c < NCHUNK) {
                const int row = c / CPR, kc = c % CPR;
                uint4 o[CH / 8];
                float s = 0.f;
                if constexpr (BITS == 2) {
                    // evens then odds of the 16-wide block: [0,2,...,14, 1,3,...,15]
                    const uint32_t r8[8] = {xr[r][0].x, xr[r][0].y, xr[r][0].z, xr[r][0].w,
                                            xr[r][1].x, xr[r][1].y, xr[r][1].z, xr[r][1].w};
                    uint32_t w[8];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        w[j] = (r8[2 * j] & 0xFFFFu) | (r8[2 * j + 1] << 16);
                        w[4 + j] = (r8[2 * j] >> 16) | (r8[2 * j + 1] & 0xFFFF0000u);
                    }
#pragma unroll
                    for (int j = 0; j < 8; ++j) s += bf16_to_f32(r8[j] & 0xFFFFu) + bf16_to_f32(r8[j] >> 16);
                    o[0] = make_uint4(w[0], w[1], w[2], w[3]);
                    o[1] = make_uint4(w[4], w[5], w[6], w[7]);
                } else {
                    // [0,4,1,5,2,6,3,7]
                    const uint32_t d[4] = {xr[r][0].x, xr[r][0].y, xr[r][0].z, xr[r][0].w};
                    o[0] = make_uint4((d[0] & 0xFFFFu) | (d[2] << 16), (d[0] >> 16) | (d[2] & 0xFFFF0000u),
                                      (d[1] & 0xFFFFu) | (d[3] << 16), (d[1] >> 16) | (d[3] & 0xFFFF0000u));
#pragma unroll
                    for (int j = 0; j < 4; ++j) s += bf16_to_f32(d[j] & 0xFFFFu) + bf16_to_f32(d[j] >> 16);
                }
                xsum[r] += s;
                uint4 *dst = reinterpret_cast<uint4 *>(xs + row * LDS_ROW + kc * CH);
#pragma unroll
                for (int h = 0; h < CH / 8; ++h) dst[h] = o[h];
            }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < CW; ++q) ccur[j][q] = cnext[j][q];
    };

    auto compute_stage = [&]() {
        static_for<0, KSTEPS>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            bf16x8 a[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * 16 * TM + i * 16 + i16;
                const uint4 v = *reinterpret_cast<const uint4 *>(xs + row * LDS_ROW + grp * (BK / 4) + 8 * t);
                a[i] = __builtin_bit_cast(bf16x8, v);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const bf16x8 b = decode_b<BITS, t>(ccur[j]);
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][j], 0, 0, 0);
            }
        });
    };

    const int nstages = (K + BK - 1) / BK;
    load_stage(0);
    for (int s = 0; s < nstages; ++s) {
        __syncthreads();  // previous stage's LDS reads are done
        store_stage();
        __syncthreads();
        if (s + 1 < nstages) load_stage((s + 1) * BK);
        compute_stage();
    }

    // X row sums: reduce over the CPR lanes that staged each row.
#pragma unroll
    for (int r = 0; r < NCT; ++r) {
        float v = xsum[r];
#pragma unroll
        for (int o = 1; o < CPR; o <<= 1) v += __shfl_xor(v, o);
        const int c = tid + 256 * r;
        if (c < NCHUNK && (c % CPR) == 0) ssum[c / CPR] = v;
    }
    __syncthreads();

    // Epilogue: lane holds rows 4*grp + e of each 16x16 tile, column i16.
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * 16 * TN + j * 16 + i16;
        if (n >= N) continue;
        const float al = bf16_to_f32(g.alpha[n]);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rl = wm * 16 * TM + i * 16 + 4 * grp + e;
                const int m = m0 + rl;
                if (m >= M) continue;
                float v;
                if constexpr (BITS == 2) {
                    v = acc[i][j][e] - 0.75f * ssum[rl];
                } else {
                    v = 8.0f * (acc[i][j][e] - 3.0f * ssum[rl]);
                }
                const float y = al * v;
                const __bf16 h = static_cast<__bf16>(y);
                g.Y[static_cast<int64_t>(m) * N + n] = __builtin_bit_cast(uint16_t, h);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel for M <= 16 (decode and small batches).
//
// The weight (N*K*BITS/8 bytes) is the whole cost.  A block owns 16*TN output
// columns and its NW waves split K between them (wave w takes groups w,
// w+NW, ...), so no barrier is needed until the final reduction.  Per group
// a wave needs 16 bytes of codes per lane per tile and the group's k-slice of
// the M activation rows; both are fetched P groups ahead into registers
// (vector loads retire in order, so activations must be requested as early
// as the codes they meet).  Activations move row-contiguously, only the M
// real rows (XI = ceil(M / rows-per-load) loads), and are turned into MFMA A
// fragments through a wave-private LDS slot.  Output rows >= M come from
// stale A rows and are never stored; columns >= N read a clamped row.
//
// Decode.  2-bit: with D & 0x33333333 every nibble holds one code in its low
// two bits, the e2m1 value c/2; v_cvt_scalef32_pk_bf16_fp4 turns each byte
// into two exact bf16 (codes 4b and 4b+2), and (D >> 2) & 0x33333333 gives
// codes 4b+1, 4b+3.  level = (c - 1.5)/2 = v - 0.75.  4-bit: nibbles are
// spread into bytes and completed to bf16 128 + c (exact); level = v - 136.
// The activations are put in the matching k order (evens, then odds, of each
// 16- or 8-wide block) by byte permutes.  The row sums of X needed by the
// offsets come from one extra MFMA per k-step against an all-ones operand.
// The NW partial sums are combined in LDS in a fixed order.
// ---------------------------------------------------------------------------
template <int BITS, int NW, int P, int TN, int XI>
__global__ __launch_bounds__(64 * NW) void k_gemm_stream(GemmArgs g)
{
    static_assert(TN <= NW, "one wave finishes each tile");
    constexpr int GK = BITS == 2 ? 256 : 128;     // k per group (16 B of codes per lane per tile)
    constexpr int RPL = 512 / GK;                 // activation rows per 1 KB load (2 or 4)
    constexpr int XROW = GK + 8;                  // LDS row stride, bf16 (+16 bytes)
    constexpr int NACC = TN * 4 + 4;
    static_assert(NW * NACC * 64 * 4 <= NW * 16 * XROW * 2, "reduction fits in the X slots");

    __shared__ __attribute__((aligned(16))) uint16_t xs[NW * 16 * XROW];
    float *red = reinterpret_cast<float *>(xs);

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int i16 = lane & 15, grp = lane >> 4;
    const int M = g.M, N = g.N, K = g.K;
    const int n0 = blockIdx.x * 16 * TN;
    const int G = K / GK;
    const int64_t row_bytes = static_cast<int64_t>(K) * BITS / 8;

    typedef __attribute__((address_space(1))) const u32x4 guint4;
    guint4 *cp[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        int n = n0 + 16 * j + i16;
        n = n < N ? n : N - 1;
        cp[j] = (guint4 *)(g.packed + n * row_bytes + grp * 16);
    }
    // activation loads: lane -> (row within the load, 8-element chunk)
    const int xr_sub = lane / (64 / RPL), xr_chunk = lane % (64 / RPL);
    guint4 *xp[XI];
    int xrow_of[XI];
#pragma unroll
    for (int q = 0; q < XI; ++q) {
        int r = RPL * q + xr_sub;
        xrow_of[q] = r;
        r = r < M ? r : M - 1;
        xp[q] = (guint4 *)(g.X + static_cast<int64_t>(r) * K + xr_chunk * 8);
    }
    uint16_t *xw = xs + w * 16 * XROW;            // this wave's slot
    const int mrow = i16 < M ? i16 : M - 1;

    floatx4 acc[TN];
    floatx4 accs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    const uint4 ones_u = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
    const bf16x8 ones = __builtin_bit_cast(bf16x8, ones_u);

    uint4 cb[P][TN];
    uint4 xb[P][XI];

    // This wave's groups are w + NW*i, i < nit; each block walks them from
    // its own starting point, so at any moment the blocks read different
    // activation lines (all blocks read the same X, and in lockstep they
    // would queue on the same L2 channel).  Loads past the end read an
    // in-bounds group and their results are never used.
    const int nit = G > w ? (G - w + NW - 1) / NW : 0;
    const int rot = nit > 0 ? static_cast<int>(blockIdx.x % static_cast<unsigned>(nit)) : 0;
    auto load = [&](int it, uint4 (&c)[TN], uint4 (&x)[XI]) {
        int i = it + rot;
        i = i >= nit ? i - nit : i;
        int gi = w + NW * i;
        gi = gi < G ? gi : G - 1;
#pragma unroll
        for (int j = 0; j < TN; ++j) c[j] = __builtin_bit_cast(uint4, cp[j][gi * 4]);
#pragma unroll
        for (int q = 0; q < XI; ++q) x[q] = __builtin_bit_cast(uint4, xp[q][gi * (GK / 8)]);
    };

    auto compute = [&](const uint4 (&c)[TN], const uint4 (&x)[XI]) {
        // activations of this group -> the wave's LDS slot (row-major)
#pragma unroll
        for (int q = 0; q < XI; ++q)
            *reinterpret_cast<uint4 *>(xw + xrow_of[q] * XROW + xr_chunk * 8) = x[q];
        // Rows >= M read row M-1: with one address per lane group the LDS
        // serves the read as a broadcast.
        const uint16_t *xa = xw + mrow * XROW + grp * (GK / 4);
        if constexpr (BITS == 2) {
            uint4 ua[8];  // issue every A read of the group before the decode work
#pragma unroll
            for (int q = 0; q < 8; ++q) ua[q] = *reinterpret_cast<const uint4 *>(xa + 8 * q);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint4 u0 = ua[2 * d];
                const uint4 u1 = ua[2 * d + 1];
                const uint32_t r[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
                uint4 ae, ao;
                ae.x = (r[0] & 0xFFFFu) | (r[1] << 16);
                ae.y = (r[2] & 0xFFFFu) | (r[3] << 16);
                ae.z = (r[4] & 0xFFFFu) | (r[5] << 16);
                ae.w = (r[6] & 0xFFFFu) | (r[7] << 16);
                ao.x = (r[0] >> 16) | (r[1] & 0xFFFF0000u);
                ao.y = (r[2] >> 16) | (r[3] & 0xFFFF0000u);
                ao.z = (r[4] >> 16) | (r[5] & 0xFFFF0000u);
                ao.w = (r[6] >> 16) | (r[7] & 0xFFFF0000u);
                const bf16x8 a_e = __builtin_bit_cast(bf16x8, ae);
                const bf16x8 a_o = __builtin_bit_cast(bf16x8, ao);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const uint32_t D = d == 0 ? c[j].x : d == 1 ? c[j].y : d == 2 ? c[j].z : c[j].w;
                    const uint32_t m0 = D & 0x33333333u;
                    const uint32_t m1 = (D >> 2) & 0x33333333u;
                    uint4 be, bo;
                    be.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m0, 1.0f, 0));
                    be.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m0, 1.0f, 1));
                    be.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m0, 1.0f, 2));
                    be.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m0, 1.0f, 3));
                    bo.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m1, 1.0f, 0));
                    bo.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m1, 1.0f, 1));
                    bo.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m1, 1.0f, 2));
                    bo.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(m1, 1.0f, 3));
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_e, __builtin_bit_cast(bf16x8, be), acc[j], 0, 0, 0);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_o, __builtin_bit_cast(bf16x8, bo), acc[j], 0, 0, 0);
                }
                accs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_e, ones, accs, 0, 0, 0);
                accs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_o, ones, accs, 0, 0, 0);
            }
        } else {
            uint4 ua[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) ua[q] = *reinterpret_cast<const uint4 *>(xa + 8 * q);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint4 xv = ua[d];
                uint4 a;
                a.x = (xv.x & 0xFFFFu) | (xv.y << 16);          // x0, x2
                a.y = (xv.z & 0xFFFFu) | (xv.w << 16);          // x4, x6
                a.z = (xv.x >> 16) | (xv.y & 0xFFFF0000u);      // x1, x3
                a.w = (xv.z >> 16) | (xv.w & 0xFFFF0000u);      // x5, x7
                const bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const uint32_t D = d == 0 ? c[j].x : d == 1 ? c[j].y : d == 2 ? c[j].z : c[j].w;
                    const uint32_t lo = D & 0x0F0F0F0Fu;          // nibbles 0,2,4,6 in bytes
                    const uint32_t hi = (D >> 4) & 0x0F0F0F0Fu;   // nibbles 1,3,5,7
                    uint4 b;
                    b.x = (lo & 0xFFu) | ((lo << 8) & 0x00FF0000u) | 0x43004300u;
                    b.y = ((lo >> 16) & 0xFFu) | ((lo >> 8) & 0x00FF0000u) | 0x43004300u;
                    b.z = (hi & 0xFFu) | ((hi << 8) & 0x00FF0000u) | 0x43004300u;
                    b.w = ((hi >> 16) & 0xFFu) | ((hi >> 8) & 0x00FF0000u) | 0x43004300u;
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, b), acc[j], 0, 0, 0);
                }
                accs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, ones, accs, 0, 0, 0);
            }
        }
    };

#pragma unroll
    for (int s = 0; s < P; ++s) load(s, cb[s], xb[s]);
    // Steady state: no conditionals, so the compiler can count the loads in
    // flight and wait only for the slot being consumed.
    int base = 0;
    for (; base + P <= nit; base += P) {
        static_for<0, P>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            compute(cb[s], xb[s]);
            load(base + s + P, cb[s], xb[s]);
            // keep the scheduler from hoisting later slots' work above this
            // slot's wait (which would wait for every load in flight)
            __builtin_amdgcn_sched_barrier(0);
        });
    }
    static_for<0, P>([&](auto sc) {
        constexpr int s = decltype(sc)::value;
        if (base + s < nit) compute(cb[s], xb[s]);
    });

    // Combine the NW partial sums in LDS (fixed order); wave j < TN finishes
    // tile j for all rows.
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(w * NACC + 4 * j + e) * 64 + lane] = acc[j][e];
#pragma unroll
    for (int e = 0; e < 4; ++e) red[(w * NACC + 4 * TN + e) * 64 + lane] = accs[e];
    __syncthreads();
    if (w < TN) {
        const int j = w;
        const int n = n0 + 16 * j + i16;
        if (n < N) {
            const float al = bf16_to_f32(g.alpha[n]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 4 * grp + e;
                if (m < M) {
                    float a = 0.f, sm = 0.f;
                    for (int v = 0; v < NW; ++v) {
                        a += red[(v * NACC + 4 * j + e) * 64 + lane];
                        sm += red[(v * NACC + 4 * TN + e) * 64 + lane];
                    }
                    const float y = BITS == 2 ? al * (a - 0.75f * sm) : al * (a - 136.0f * sm);
                    const __bf16 h = static_cast<__bf16>(y);
                    g.Y[static_cast<int64_t>(m) * N + n] = __builtin_bit_cast(uint16_t, h);
                }
            }
        }
    }
}

template <int BITS, int XI>
void launch_stream(const GemmArgs &a, hipStream_t s)
{
    hipLaunchKernelGGL((k_gemm_stream<BITS, PQ_STREAM_NW, PQ_STREAM_P, PQ_STREAM_TN, XI>),
                       dim3((a.N + 16 * PQ_STREAM_TN - 1) / (16 * PQ_STREAM_TN)),
                       dim3(64 * PQ_STREAM_NW), 0, s, a);
}

template <int BITS, int TM, int TN, int WM, int WN, int BK>
void launch(const GemmArgs &a, hipStream_t s)
{
    constexpr int BM = 16 * TM * WM, BN = 16 * TN * WN;
    dim3 grid((a.N + BN - 1) / BN, (a.M + BM - 1) / BM);
    hipLaunchKernelGGL((k_gemm<BITS, TM, TN, WM, WN, BK>), grid, dim3(256), 0, s, a);
}

template <int BITS>
pq_status gemm(int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
               const void *alpha_bf16, void *Y, void *stream)
{
    if (!X || !packed || !alpha_bf16 || !Y) return PQ_ERR_NULL;
    if (M < 0 || N < 0 || K <= 0 || K % 64 != 0 || K > kMaxCols || M > INT32_MAX / 2 ||
        N > INT32_MAX / 2)
        return PQ_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(packed) || !aligned16(Y) || !aligned16(alpha_bf16))
        return PQ_ERR_ALIGN;
    if (M == 0 || N == 0) return PQ_OK;
    GemmArgs a{static_cast<const uint16_t *>(X), packed, static_cast<const uint16_t *>(alpha_bf16),
               static_cast<uint16_t *>(Y), static_cast<int>(M), static_cast<int>(N), static_cast<int>(K)};
    hipStream_t s = static_cast<hipStream_t>(stream);
    constexpr int GK = BITS == 2 ? 256 : 128;
    constexpr int RPL = 512 / GK;
    if (M <= 16 && K % GK == 0) {
        if (M <= RPL) launch_stream<BITS, 1>(a, s);
        else if (M <= 2 * RPL) launch_stream<BITS, 2>(a, s);
        else if (M <= 4 * RPL) launch_stream<BITS, 4>(a, s);
        else launch_stream<BITS, 16 / RPL>(a, s);
    } else if (M <= 16) launch<BITS, 1, 1, 1, 4, 256>(a, s);
    else if (M <= 64) launch<BITS, PQ_TILE_MID>(a, s);
    else launch<BITS, PQ_TILE_BIG>(a, s);
    return hipGetLastError() == hipSuccess ? PQ_OK : PQ_ERR_HIP;
}

}  // namespace
}  // namespace pq

extern "C" {

pq_status pq_w2a16_gemm(int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
                        const void *alpha_bf16, void *Y, void *stream)
{
    return pq::gemm<2>(M, N, K, X, packed, alpha_bf16, Y, stream);
}

pq_status pq_w4a16_gemm(int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
                        const void *alpha_bf16, void *Y, void *stream)
{
    return pq::gemm<4>(M, N, K, X, packed, alpha_bf16, Y, stream);
}

}  // extern "C"
