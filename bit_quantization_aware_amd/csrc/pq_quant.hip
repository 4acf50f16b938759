// pq_quant.hip -- gfx950 kernels and C entry points for the per-row weight
// quantizer: alpha init, forward fake-quantization, straight-through backward
// with the scale gradient, and export packing.
//
// Sources (web pages, cited by title and section):
//   [Note]     "ParetoQ, the strongest low-bit QAT I could find"
//   [Rebuttal] "ParetoQ: Improving Scaling Laws in Extremely Low-bit LLM
//              Quantization" (authors' OpenReview replies)
//   [News]     "Meta's ParetoQ compares five bit widths and puts the accuracy
//              cliff at 1 bit"
//
// Work mapping.  The whole pass is HBM-bound elementwise work with one scalar
// (alpha) and one reduction (init statistic or alpha gradient) per row.  A
// "team" of WPR wavefronts owns one row: WPR = 1 (four rows per 256-thread
// block) when the stack has enough rows to fill the chip, WPR = 4 (one row
// per block) otherwise.  Each lane handles quads of 4 consecutive weights;
// the quads of one wave instruction are contiguous, so every 128-bit load
// and every 64-bit bf16 store is fully coalesced.  1-bit codes and mask bits
// (a nibble per quad) are paired with the neighbouring lane into bytes.
// Row reductions: a butterfly over the wave (ds_bpermute), then LDS across
// the team's waves, in a fixed order, so results are run-to-run identical.
//
// Arithmetic.  Every float step gives the IEEE binary32 result of the
// definition (built with -ffp-contract=off; explicit fmas only where the
// product they absorb is exact): x = w / a correctly rounded, clamp, the SEQ
// shift, rint (v_rndne_f32, half-to-even), q = a * level with the level
// exact in binary32, bf16 by v_cvt_pk_bf16_f32 (nearest-even).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <type_traits>

#include "pq_common.hpp"

// Blocks per CU the register allocation must allow (occupancy floor).
#ifndef PQ_QUANT_FWD_MINB
#define PQ_QUANT_FWD_MINB 8
#endif
#ifndef PQ_QUANT_BWD_MINB
#define PQ_QUANT_BWD_MINB 4
#endif

namespace pq {
namespace {

// Streaming access: every weight, gradient and output is touched once, so
// loads and stores are nontemporal (they do not displace other data in L2).
template <typename P>
__device__ __forceinline__ auto ld_stream(const P *p)
{
    return __builtin_nontemporal_load(p);
}
template <typename P, typename V>
__device__ __forceinline__ void st_stream(P *p, V v)
{
    __builtin_nontemporal_store(v, p);
}

// [Note] "Paper vs. code", first bullet: clip w/alpha to +-(1 - 1e-2).
constexpr float kClip = 0.99f;
// alpha <= 1e-5 is used as 1e-5 (the pages are silent; keeps 0/0 away).
constexpr float kAlphaFloor = 1e-5f;
// [Note] "Finding 3": ternary levels are {-2/3, 0, +2/3} alpha.
constexpr float kTwoThirds = static_cast<float>(2.0 / 3.0);

template <int MODE> struct Mode;
template <> struct Mode<PQ_W1_BINARY> {
    static constexpr int cw = 1;
    static constexpr int levels = 2;
    static constexpr float lo = -1.0f, hi = 1.0f;
};
template <> struct Mode<PQ_W158_SEQ_TERNARY> {
    static constexpr int cw = 2;
    static constexpr int levels = 3;
    static constexpr float lo = -kClip, hi = kClip;
};
template <> struct Mode<PQ_W2_SEQ> {
    static constexpr int cw = 2;
    static constexpr int levels = 4;
    static constexpr float lo = -kClip, hi = kClip;
};
template <> struct Mode<PQ_W3_LSQ> {
    static constexpr int cw = 4;
    static constexpr int levels = 8;
    static constexpr float lo = -4.0f, hi = 3.0f;  // LSQ grid -2^(b-1) .. 2^(b-1)-1
};
// The LSQ grids the pages set against SEQ at 2 and 1.58 bits ([Rebuttal]).
template <> struct Mode<PQ_W2_LSQ> {
    static constexpr int cw = 2;
    static constexpr int levels = 4;
    static constexpr float lo = -2.0f, hi = 1.0f;
};
template <> struct Mode<PQ_W158_LSQ> {
    static constexpr int cw = 2;
    static constexpr int levels = 3;
    static constexpr float lo = -1.0f, hi = 1.0f;
};
template <> struct Mode<PQ_W4_LSQ> {
    static constexpr int cw = 4;
    static constexpr int levels = 16;
    static constexpr float lo = -8.0f, hi = 7.0f;
};

// x = w / a rounded to binary32, computed as RN32(RN64(w * y)) with
// y = RN64(1 / a) taken once per row.  This equals the correctly rounded
// binary32 quotient whenever |w / a| >= 2^-125: the exact quotient of two
// binary32 numbers is never a binary32 rounding midpoint and lies at a
// relative distance of at least 2^-50 from every midpoint, while the binary64
// product is within 2^-52 (relative) of it, so both round the same way.
// Below 2^-125 the two may differ in the last subnormal place.  The forward
// outputs cannot see that: for |x| <= 2^-125 every mode's rounding input is
// exactly -0.5 (SEQ 2-bit) or +-0 (ternary, LSQ), whatever x is.  The
// backward, whose alpha gradient uses x itself, re-divides such weights
// (see tiny_key).
__device__ __forceinline__ float div_fast(float w, double y)
{
    return static_cast<float>(static_cast<double>(w) * y);
}

// Key for "0 < |w| < t" with one unsigned min per weight: (bits << 1) drops
// the sign, and the -2 sends +-0 to the top of the range.
__device__ __forceinline__ uint32_t tiny_key(float w)
{
    return (__builtin_bit_cast(uint32_t, w) << 1) - 2u;
}

// One weight from its quotient x: returns the code; writes the level
// (binary32, exact).  Every step is the binary32 operation of the
// definition; an fma is used only where its single rounding equals the
// definition's (the product it absorbs is exact).
template <int MODE>
__device__ __forceinline__ uint32_t quant_x(float w, float x, float &lvl)
{
    if constexpr (MODE == PQ_W2_SEQ) {
        // [Note] "Paper vs. code", SEQ row: round(Clip(x) * k/2 - 0.5) + 0.5, k = 4.
        // xc * 2 is exact, so fma(xc, 2, -0.5) rounds xc * 2 - 0.5 once, as the
        // two-step form does; the level (r + 0.5) * 2/k = r/2 + 1/4 is exact.
        const float xc = __builtin_amdgcn_fmed3f(x, -kClip, kClip);
        const float rf = __builtin_rintf(__builtin_fmaf(xc, 2.0f, -0.5f));
        lvl = __builtin_fmaf(rf, 0.5f, 0.25f);
        return static_cast<uint32_t>(static_cast<int>(rf) + 2);
    } else if constexpr (MODE == PQ_W158_SEQ_TERNARY) {
        // [Rebuttal] 1.58-bit bullet: stretch to [-1.5, 1.5], three equal bins.
        const float xc = __builtin_amdgcn_fmed3f(x, -kClip, kClip);
        const int r = static_cast<int>(__builtin_rintf(xc * 1.5f));
        lvl = static_cast<float>(r) * kTwoThirds;
        return static_cast<uint32_t>(r + 1);
    } else if constexpr (MODE == PQ_W3_LSQ || MODE == PQ_W4_LSQ || MODE == PQ_W2_LSQ || MODE == PQ_W158_LSQ) {
        // LSQ integer grid: round(clamp(x, Qn, Qp)).
        const float xc = __builtin_amdgcn_fmed3f(x, Mode<MODE>::lo, Mode<MODE>::hi);
        const int r = static_cast<int>(__builtin_rintf(xc));
        lvl = static_cast<float>(r);
        return static_cast<uint32_t>(r - static_cast<int>(Mode<MODE>::lo));
    } else {
        // 1 bit: sign(w) with sign(0) = +1.
        const bool pos = w >= 0.0f;
        lvl = pos ? 1.0f : -1.0f;
        return pos ? 1u : 0u;
    }
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ __forceinline__ double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Team-wide reductions.  WPR == 1: the wave butterfly; WPR == 4: the four wave
// results go through LDS and are combined in wave order by every thread.
template <int WPR>
__device__ __forceinline__ float team_max(float v, float *lds4)
{
    v = wave_max(v);
    if constexpr (WPR == 1) {
        return v;
    } else {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) lds4[wave] = v;
        __syncthreads();
        float r = fmaxf(fmaxf(lds4[0], lds4[1]), fmaxf(lds4[2], lds4[3]));
        __syncthreads();
        return r;
    }
}

template <int WPR>
__device__ __forceinline__ double team_sum(double v, double *lds4)
{
    v = wave_sum(v);
    if constexpr (WPR == 1) {
        return v;
    } else {
        const int wave = threadIdx.x >> 6;
        if ((threadIdx.x & 63) == 0) lds4[wave] = v;
        __syncthreads();
        double r = ((lds4[0] + lds4[1]) + lds4[2]) + lds4[3];
        __syncthreads();
        return r;
    }
}

// Quads handled per lane per batch (loads are issued for the whole batch
// before any math, to keep U * 16 bytes per lane in flight).
constexpr int kUnroll = 4;

enum : unsigned { OUT_BF16 = 1, OUT_F32 = 2, OUT_CODES = 4, OUT_ALPHA_BF16 = 8, OUT_TILED = 16, OUT_STATS = 32 };

// Level statistics fused into the forward (OUT_STATS, single matrix): per
// row the count of each stored code [rows, levels] and its entropy in bits.
struct StatsOut {
    uint32_t *counts;
    double *entropy;
};

// Forward rows per wave: with one wave per row (launches of many short
// rows) each wave takes two rows in turn, which halves the number of waves
// to launch and retire; a team of four waves takes one row.  Codes in the
// export byte order take one row per wave, so that the rows sharing a
// 128-byte line of the export are written close together in time (with an
// earlier layout whose lines held 16-byte pieces of 8 rows, two rows per
// wave let lines leave L2 partly written: 21x the code bytes written, 2.4x
// the time).
constexpr int fwd_rows_per_wave(int wpr, bool tiled) { return wpr == 1 && !tiled ? 2 : 1; }

// Row-major codes of quad q (weights 4q .. 4q+3) from their four codes.  The
// 1-bit case pairs each even lane with its odd neighbour, so every lane of
// the wave must make this call (act only gates the store).
template <int CW>
__device__ __forceinline__ void store_codes(PQ_GLOBAL uint8_t *crow, int q, uint32_t c0, uint32_t c1, uint32_t c2,
                                            uint32_t c3, bool act, int tl)
{
    if constexpr (CW == 2) {
        if (act) crow[q] = static_cast<uint8_t>(c0 | (c1 << 2) | (c2 << 4) | (c3 << 6));
    } else if constexpr (CW == 4) {
        if (act) ((PQ_GLOBAL uint16_t *)crow)[q] = static_cast<uint16_t>(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
    } else {
        // 1 bit: a nibble per quad; the even lane takes its odd neighbour's.
        const uint32_t nib = c0 | (c1 << 1) | (c2 << 2) | (c3 << 3);
        const uint32_t hi = __shfl_down(nib, 1);
        if (act && (tl & 1) == 0) crow[q >> 1] = static_cast<uint8_t>(nib | (hi << 4));
    }
}

// Export byte order of the codes (OUT_TILED, single matrix).  The 64-byte
// groups of all rows are stored group after group; inside a group, each tile
// of 16 rows is 1 KB ordered [row of the tile][64 bytes of the row]:
//   byte kb of row n -> (kb / 64) * Np * 64 + (n / 16) * 1024
//                       + (n % 16) * 64 + kb % 64,
// Np = rows rounded up to 16.  Bytes past a row's end within its last group,
// and the rows from `rows` to Np, are zero.  A 1-KB tile is then exactly the
// deployment GEMM's MFMA operand for 16 columns and 64 code bytes, fetched
// with one contiguous load.
//
// Forward: optional alpha init, then per quad: quantize, emit bf16 / fp32 /
// codes.  OUT_ALPHA_BF16 (export) also writes bf16(alpha) per row.
// (The fused level statistics and the scale init hold more registers: their
// launches ask for half the blocks per CU rather than spill.)
template <int MODE, bool INIT, int WPR, unsigned OUTS>
__global__ __launch_bounds__(256, ((OUTS & OUT_STATS) || INIT) ? PQ_QUANT_FWD_MINB / 2 : PQ_QUANT_FWD_MINB) void k_quant_fwd(
    LaunchTable lt, StatsOut so)
{
    constexpr int RPB = 4 / WPR;
    constexpr int TEAM = 64 * WPR;
    constexpr int CW = Mode<MODE>::cw;
    constexpr int L = Mode<MODE>::levels;
    constexpr bool STATS = (OUTS & OUT_STATS) != 0;
    __shared__ float lds_f[4];
    __shared__ double lds_d[4];
    // OUT_STATS: per wave, a count of each level for each lane ([level][lane],
    // so a wave's increments of one level fall on 64 distinct banks)
    __shared__ uint32_t hist[STATS ? 4 * L * 64 : 1];

    constexpr bool TILED = (OUTS & OUT_TILED) != 0;
    static_assert(!TILED || (OUTS & OUT_CODES) != 0, "tiled export writes codes");
    const int wave = threadIdx.x >> 6;
    const int tl = (wave % WPR) * 64 + (threadIdx.x & 63);
    int b = blockIdx.x;
    if constexpr (TILED) {
        // The eight XCDs take blocks round robin; give the blocks of one XCD
        // consecutive rows, so that the 16 rows of a tile -- whose code
        // pieces share cache lines -- are written through one L2.
        const int nb = gridDim.x;
        if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
    }
    const int k = find_matrix(lt, b);
    const pq_mat m = lt.table ? lt.table[k] : lt.single;
    const int64_t cols = m.cols;
    const int nq = static_cast<int>(cols >> 2);
    constexpr int RPW = fwd_rows_per_wave(WPR, TILED);
    const int64_t row0 = static_cast<int64_t>(b - lt.block_start[k]) * (RPB * RPW) + wave / WPR;

    // One row (RPB rows per block, one after the other RPW times).
    auto one_row = [&](const int64_t row) {
        // Tiled export: this row's 64-byte slot in every tile, and the group stride.
        PQ_GLOBAL uint8_t *tbase = nullptr;
        int64_t gstride = 0, gbytes = 0;
        if constexpr (TILED) {
            const int64_t np = (m.rows + 15) & ~int64_t(15);
            gstride = np * 64;
            gbytes = (cols * CW / 8 + 63) / 64 * 64;
            tbase = (PQ_GLOBAL uint8_t *)m.codes + (row >> 4) * 1024 + (row & 15) * 64;
            if (row >= m.rows) {
                // padding row of the last tile: zero pieces in every group
                if (row < np)
                    for (int64_t p = tl; p < gbytes / 16; p += TEAM)
                        *(PQ_GLOBAL u32x4 *)(tbase + (p >> 2) * gstride + (p & 3) * 16) = u32x4{0u, 0u, 0u, 0u};
                return;
            }
        }
        if (row >= m.rows) return;  // only when WPR == 1 (RPB rows per block)
        const PQ_GLOBAL f32x4 *wr = (const PQ_GLOBAL f32x4 *)(m.W + row * cols);

        float alpha_raw;
        if constexpr (INIT) {
            // [Note] "The 2-bit recipe" table / scale-init row of "Paper vs. code".
            if constexpr (MODE == PQ_W1_BINARY) {
                double s = 0.0;
                for (int q = tl; q < nq; q += TEAM) {
                    const f32x4 v = wr[q];
                    s += static_cast<double>(fabsf(v.x));
                    s += static_cast<double>(fabsf(v.y));
                    s += static_cast<double>(fabsf(v.z));
                    s += static_cast<double>(fabsf(v.w));
                }
                s = team_sum<WPR>(s, lds_d);
                alpha_raw = static_cast<float>(s / static_cast<double>(cols));
            } else {
                float mx = 0.0f;
                for (int q = tl; q < nq; q += TEAM) {
                    const f32x4 v = wr[q];
                    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
                }
                mx = team_max<WPR>(mx, lds_f);
                if constexpr (MODE == PQ_W3_LSQ || MODE == PQ_W4_LSQ || MODE == PQ_W2_LSQ || MODE == PQ_W158_LSQ)
                    mx = mx / Mode<MODE>::hi;
                alpha_raw = mx;
            }
            if (tl == 0) m.alpha[row] = alpha_raw;
        } else {
            alpha_raw = m.alpha[row];
        }
        const float a = alpha_raw > kAlphaFloor ? alpha_raw : kAlphaFloor;
        const double y = 1.0 / static_cast<double>(a);

        if constexpr ((OUTS & OUT_ALPHA_BF16) != 0) {
            if (tl == 0) {
                __bf16 h = static_cast<__bf16>(alpha_raw);
                static_cast<uint16_t *>(m.alpha_bf16)[row] = __builtin_bit_cast(uint16_t, h);
            }
        }

        PQ_GLOBAL u32x2 *wq16 =
            (OUTS & OUT_BF16) ? (PQ_GLOBAL u32x2 *)(static_cast<uint16_t *>(m.wq_bf16) + row * cols) : nullptr;
        PQ_GLOBAL f32x4 *wq32 = (OUTS & OUT_F32) ? (PQ_GLOBAL f32x4 *)(m.wq_f32 + row * cols) : nullptr;
        PQ_GLOBAL uint8_t *crow = (OUTS & OUT_CODES) ? (PQ_GLOBAL uint8_t *)(m.codes + row * (cols * CW / 8)) : nullptr;

        uint32_t *whist = hist + (STATS ? (threadIdx.x >> 6) * L * 64 + (threadIdx.x & 63) : 0);
        if constexpr (STATS) {
#pragma unroll
            for (int l = 0; l < L; ++l) whist[l * 64] = 0u;
        }

        // One pass: kUnroll quads per lane, loads first.  GUARD only on the last.
        auto pass = [&](int base, auto guard_c) {
            constexpr bool GUARD = decltype(guard_c)::value;
            f32x4 v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int q = base + u * TEAM + tl;
                if (!GUARD || q < nq) v[u] = ld_stream(&wr[q]);
                else v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                // in the tail pass, quad slots no lane of the team owns are skipped
                if (GUARD && base + u * TEAM >= nq) break;
                const int q = base + u * TEAM + tl;
                const bool act = !GUARD || q < nq;
                float l0, l1, l2, l3;
                const uint32_t c0 = quant_x<MODE>(v[u].x, div_fast(v[u].x, y), l0);
                const uint32_t c1 = quant_x<MODE>(v[u].y, div_fast(v[u].y, y), l1);
                const uint32_t c2 = quant_x<MODE>(v[u].z, div_fast(v[u].z, y), l2);
                const uint32_t c3 = quant_x<MODE>(v[u].w, div_fast(v[u].w, y), l3);
                const float q0 = a * l0, q1 = a * l1, q2 = a * l2, q3 = a * l3;
                if constexpr (STATS) {
                    if (act) {
                        __hip_atomic_fetch_add(&whist[c0 * 64], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
                        __hip_atomic_fetch_add(&whist[c1 * 64], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
                        __hip_atomic_fetch_add(&whist[c2 * 64], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
                        __hip_atomic_fetch_add(&whist[c3 * 64], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
                    }
                }
                if constexpr ((OUTS & OUT_BF16) != 0) {
                    if (act) wq16[q] = u32x2{pack_bf16x2(q0, q1), pack_bf16x2(q2, q3)};
                }
                if constexpr ((OUTS & OUT_F32) != 0) {
                    if (act) wq32[q] = f32x4{q0, q1, q2, q3};
                }
                if constexpr (TILED && CW == 1) {
                    // 1 bit: quad q is the low or high nibble of byte q / 2 of
                    // the row; the even lane takes its odd neighbour's nibble
                    // (every lane shuffles, act only gates the store).
                    const uint32_t nib = c0 | (c1 << 1) | (c2 << 2) | (c3 << 3);
                    const uint32_t hi = __shfl_down(nib, 1);
                    PQ_GLOBAL uint8_t *d = tbase + static_cast<int64_t>(q >> 7) * gstride + ((q >> 1) & 63);
                    if (act && (tl & 1) == 0) *d = static_cast<uint8_t>(nib | (hi << 4));
                } else if constexpr (TILED) {
                    // A quad is CW / 2 code bytes, and base + u * TEAM starts a
                    // whole 64-byte group g0; the lane's byte offset from there
                    // (tl or 2 tl) splits into group and byte.
                    const int64_t g0 = (static_cast<int64_t>(base + u * TEAM) * (CW / 2)) >> 6;
                    if constexpr (CW == 2) {
                        PQ_GLOBAL uint8_t *d = tbase + (g0 + (tl >> 6)) * gstride + (tl & 63);
                        if (act) *d = static_cast<uint8_t>(c0 | (c1 << 2) | (c2 << 4) | (c3 << 6));
                    } else {
                        PQ_GLOBAL uint8_t *d =
                            tbase + (g0 + (tl >> 5)) * gstride + ((2 * tl) & 63);
                        if (act)
                            *(PQ_GLOBAL uint16_t *)d = static_cast<uint16_t>(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
                    }
                } else if constexpr ((OUTS & OUT_CODES) != 0) {
                    store_codes<CW>(crow, q, c0, c1, c2, c3, act, tl);
                }
            }
        };
        constexpr int STEP = TEAM * kUnroll;
        const int nfull = nq / STEP * STEP;
        for (int base = 0; base < nfull; base += STEP) pass(base, std::false_type{});
        if (nfull < nq) pass(nfull, std::true_type{});
        if constexpr (STATS) {
            // Counts of the row (lanes, then the team's waves, in a fixed
            // order; exact in binary64) and their entropy, as the separate
            // level-statistics kernel computes them.
            double h = 0.0;
#pragma unroll 1
            for (int l = 0; l < L; ++l) {
                const double c = team_sum<WPR>(static_cast<double>(whist[l * 64]), lds_d);
                if (tl == 0) {
                    so.counts[row * L + l] = static_cast<uint32_t>(c);
                    if (c > 0.0) {
                        const double pr = c / static_cast<double>(cols);
                        h -= pr * log2(pr);
                    }
                }
            }
            if (tl == 0 && so.entropy) so.entropy[row] = h;
        }
        if constexpr (TILED) {
            // zero the bytes of the last group past the row's end (< 64 bytes)
            const int64_t rb = cols * CW / 8;
            const int64_t kb = rb + tl;
            if (kb < gbytes) tbase[(kb >> 6) * gstride + (kb & 63)] = 0;
        }
    };
#pragma unroll 1
    for (int rr = 0; rr < RPW; ++rr) one_row(row0 + rr * RPB);
}

// Backward: per weight the forward's x and level (bit-identical), the clip
// gate, dW = inside ? G : +0, and the binary64 alpha-gradient partial
// (level - x inside, the boundary level outside).
template <int MODE, int WPR, bool GBF16, bool WDW, bool WMASK>
__global__ __launch_bounds__(256, PQ_QUANT_BWD_MINB) void k_quant_bwd(LaunchTable lt)
{
    constexpr int RPB = 4 / WPR;
    constexpr int TEAM = 64 * WPR;
    __shared__ double lds_d[4];

    const int wave = threadIdx.x >> 6;
    const int tl = (wave % WPR) * 64 + (threadIdx.x & 63);
    const int b = blockIdx.x;
    const int k = find_matrix(lt, b);
    const pq_mat m = lt.table ? lt.table[k] : lt.single;
    const int64_t row = static_cast<int64_t>(b - lt.block_start[k]) * RPB + wave / WPR;
    if (row >= m.rows) return;

    const int64_t cols = m.cols;
    const int nq = static_cast<int>(cols >> 2);
    const PQ_GLOBAL f32x4 *wr = (const PQ_GLOBAL f32x4 *)(m.W + row * cols);
    const PQ_GLOBAL f32x4 *gr32 = (const PQ_GLOBAL f32x4 *)(static_cast<const float *>(m.G) + row * cols);
    const PQ_GLOBAL u32x2 *gr16 = (const PQ_GLOBAL u32x2 *)(static_cast<const uint16_t *>(m.G) + row * cols);
    PQ_GLOBAL f32x4 *dwr = WDW ? (PQ_GLOBAL f32x4 *)(m.dW + row * cols) : nullptr;
    PQ_GLOBAL uint8_t *mrow = WMASK ? (PQ_GLOBAL uint8_t *)(m.mask_bits + row * (cols >> 3)) : nullptr;

    const float alpha_raw = m.alpha[row];
    const float a = alpha_raw > kAlphaFloor ? alpha_raw : kAlphaFloor;
    const double y = 1.0 / static_cast<double>(a);
    // |w| < a * 2^-123 covers every quotient below 2^-125 (the product is
    // rounded at most once, in the subnormal range, far from a factor of 4).
    const uint32_t tkey = tiny_key(a * 0x1p-123f);
    constexpr float lo = Mode<MODE>::lo, hi = Mode<MODE>::hi;
    double acc = 0.0;

    // The arithmetic of one quad, on W and G already in registers.  EXACT:
    // quotients by the IEEE division, else by the binary64 product.  Returns
    // the quad's mask nibble.
    auto quad = [&](const f32x4 &wq, const f32x4 &gq, int q, bool act, auto exact_c) -> uint32_t {
        constexpr bool EXACT = decltype(exact_c)::value;
        const float w4[4] = {wq.x, wq.y, wq.z, wq.w};
        const float g4[4] = {gq.x, gq.y, gq.z, gq.w};
        float d4[4];
        uint32_t nib = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float lvl;
            const float x = EXACT ? w4[e] / a : div_fast(w4[e], y);
            quant_x<MODE>(w4[e], x, lvl);
            const bool inside = (x >= lo) && (x <= hi);
            d4[e] = inside ? g4[e] : 0.0f;
            nib |= static_cast<uint32_t>(inside) << e;
            const double s = static_cast<double>(lvl) - (inside ? static_cast<double>(x) : 0.0);
            // inactive lanes loaded zeros, so their products are +0
            acc += s * static_cast<double>(g4[e]);
        }
        if constexpr (WDW) {
            if (act) st_stream(&dwr[q], f32x4{d4[0], d4[1], d4[2], d4[3]});
        }
        return nib;
    };

    // One pass: kUnroll quads per lane; all W and G loads are issued before
    // any store, so dW may overwrite G in place.  A quad holding a weight
    // with a quotient below 2^-125 (0 < |w| < a * 2^-123) takes the exact
    // body (rare); the test is one unsigned min per weight.  The mask
    // nibbles are paired across lanes after the (divergent) quad bodies.
    auto pass = [&](int base, auto guard_c) {
        constexpr bool GUARD = decltype(guard_c)::value;
        f32x4 wv[kUnroll], gv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int q = base + u * TEAM + tl;
            if (!GUARD || q < nq) {
                wv[u] = ld_stream(&wr[q]);
                if constexpr (GBF16) {
                    const u32x2 h = ld_stream(&gr16[q]);
                    gv[u] = f32x4{bf16_to_f32(h.x & 0xFFFFu), bf16_to_f32(h.x >> 16),
                                  bf16_to_f32(h.y & 0xFFFFu), bf16_to_f32(h.y >> 16)};
                } else {
                    gv[u] = ld_stream(&gr32[q]);
                }
            } else {
                wv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                gv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
        uint32_t nibs = 0;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (GUARD && base + u * TEAM >= nq) break;  // slot empty for the whole team
            const int q = base + u * TEAM + tl;
            const bool act = !GUARD || q < nq;
            const uint32_t kmin = min(min(tiny_key(wv[u].x), tiny_key(wv[u].y)),
                                      min(tiny_key(wv[u].z), tiny_key(wv[u].w)));
            uint32_t nib;
            if (__builtin_expect(kmin < tkey, 0)) nib = quad(wv[u], gv[u], q, act, std::true_type{});
            else nib = quad(wv[u], gv[u], q, act, std::false_type{});
            nibs |= nib << (4 * u);
        }
        if constexpr (WMASK) {
            // a nibble per quad; the even lane takes its odd neighbour's
            // into the high half of the byte
            const uint32_t hi = __shfl_down(nibs, 1);
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int q = base + u * TEAM + tl;
                const bool act = !GUARD || q < nq;
                if (act && (tl & 1) == 0)
                    mrow[q >> 1] = static_cast<uint8_t>(((nibs >> (4 * u)) & 0xFu) | (((hi >> (4 * u)) & 0xFu) << 4));
            }
        }
    };
    constexpr int STEP = TEAM * kUnroll;
    const int nfull = nq / STEP * STEP;
    for (int base = 0; base < nfull; base += STEP) pass(base, std::false_type{});
    if (nfull < nq) pass(nfull, std::true_type{});

    acc = team_sum<WPR>(acc, lds_d);
    if (tl == 0) m.dalpha[row] = static_cast<float>(m.grad_scale * acc);
}

// ---------------------------------------------------------------------------
// Fused QAT step: backward of the current forward, AdamW on W and alpha, and
// the next forward, one team per row.
//
// Pass A streams W, G and the two moments of W once: per weight the
// backward's x, gate and dW (bit-identical to k_quant_bwd, including the
// exact division for tiny quotients) and the alpha-gradient partial, then
// the AdamW update of w, m, v; the new w is stored with a plain store (it is
// read back in pass B, from L2), the moments with streaming stores.  The
// team's binary64 sum gives dalpha; every lane then updates alpha and its
// moments with the same binary32 operations (identical results), and lane 0
// stores them.  Pass B reads the new weights back and writes the next
// forward's bf16 weights and codes, as k_quant_fwd does.
// ---------------------------------------------------------------------------
struct AdamK {
    float b1, w1, b2, w2, s2, eps, decay, step_size;
};

// One AdamW update in the documented binary32 order (the kernels are built
// with -ffp-contract=off, so no product is fused into an add).
__device__ __forceinline__ float adam_one(const AdamK &k, float p, float g, float &m, float &v)
{
    const float mn = k.b1 * m + k.w1 * g;
    const float vn = k.b2 * v + (k.w2 * g) * g;
    const float den = __builtin_sqrtf(vn) / k.s2 + k.eps;
    const float pd = p * k.decay;
    m = mn;
    v = vn;
    return pd - (k.step_size * mn) / den;
}

// Quads per lane per pass: four streams in, so two quads keep the same bytes
// in flight as the other kernels' four, within 128 VGPRs.
constexpr int kStepUnroll = 2;

template <int MODE, int WPR, bool GBF16>
__global__ __launch_bounds__(256, PQ_QUANT_BWD_MINB) void k_qat_step(StepTable lt, AdamK ak)
{
    constexpr int RPB = 4 / WPR;
    constexpr int TEAM = 64 * WPR;
    constexpr int CW = Mode<MODE>::cw;
    __shared__ double lds_d[4];

    const int wave = threadIdx.x >> 6;
    const int tl = (wave % WPR) * 64 + (threadIdx.x & 63);
    const int b = blockIdx.x;
    const int k = find_matrix(lt, b);
    const pq_step_mat m = lt.table ? lt.table[k] : lt.single;
    const int64_t row = static_cast<int64_t>(b - lt.block_start[k]) * RPB + wave / WPR;
    if (row >= m.rows) return;

    const int64_t cols = m.cols;
    const int nq = static_cast<int>(cols >> 2);
    PQ_GLOBAL f32x4 *wr = (PQ_GLOBAL f32x4 *)(m.W + row * cols);
    const PQ_GLOBAL f32x4 *gr32 = (const PQ_GLOBAL f32x4 *)(static_cast<const float *>(m.G) + row * cols);
    const PQ_GLOBAL u32x2 *gr16 = (const PQ_GLOBAL u32x2 *)(static_cast<const uint16_t *>(m.G) + row * cols);
    PQ_GLOBAL f32x4 *mr = (PQ_GLOBAL f32x4 *)(m.mW + row * cols);
    PQ_GLOBAL f32x4 *vr = (PQ_GLOBAL f32x4 *)(m.vW + row * cols);

    const float alpha_raw = m.alpha[row];
    const float a = alpha_raw > kAlphaFloor ? alpha_raw : kAlphaFloor;
    const double y = 1.0 / static_cast<double>(a);
    const uint32_t tkey = tiny_key(a * 0x1p-123f);
    constexpr float lo = Mode<MODE>::lo, hi = Mode<MODE>::hi;
    constexpr int STEP = TEAM * kStepUnroll;
    const int nfull = nq / STEP * STEP;
    double acc = 0.0;

    // Pass A: backward + AdamW of one quad on values already in registers.
    auto quad_a = [&](f32x4 &wq, const f32x4 &gq, f32x4 &mq, f32x4 &vq, auto exact_c) {
        constexpr bool EXACT = decltype(exact_c)::value;
        float w4[4] = {wq.x, wq.y, wq.z, wq.w};
        const float g4[4] = {gq.x, gq.y, gq.z, gq.w};
        float m4[4] = {mq.x, mq.y, mq.z, mq.w};
        float v4[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float lvl;
            const float x = EXACT ? w4[e] / a : div_fast(w4[e], y);
            quant_x<MODE>(w4[e], x, lvl);
            const bool inside = (x >= lo) && (x <= hi);
            const float d = inside ? g4[e] : 0.0f;
            const double s = static_cast<double>(lvl) - (inside ? static_cast<double>(x) : 0.0);
            acc += s * static_cast<double>(g4[e]);
            w4[e] = adam_one(ak, w4[e], d, m4[e], v4[e]);
        }
        wq = f32x4{w4[0], w4[1], w4[2], w4[3]};
        mq = f32x4{m4[0], m4[1], m4[2], m4[3]};
        vq = f32x4{v4[0], v4[1], v4[2], v4[3]};
    };
    auto pass_a = [&](int base, auto guard_c) {
        constexpr bool GUARD = decltype(guard_c)::value;
        f32x4 wv[kStepUnroll], gv[kStepUnroll], mv[kStepUnroll], vv[kStepUnroll];
#pragma unroll
        for (int u = 0; u < kStepUnroll; ++u) {
            const int q = base + u * TEAM + tl;
            if (!GUARD || q < nq) {
                wv[u] = wr[q];
                if constexpr (GBF16) {
                    const u32x2 h = ld_stream(&gr16[q]);
                    gv[u] = f32x4{bf16_to_f32(h.x & 0xFFFFu), bf16_to_f32(h.x >> 16),
                                  bf16_to_f32(h.y & 0xFFFFu), bf16_to_f32(h.y >> 16)};
                } else {
                    gv[u] = ld_stream(&gr32[q]);
                }
                mv[u] = ld_stream(&mr[q]);
                vv[u] = ld_stream(&vr[q]);
            } else {
                // inactive slots: zero weight and gradient (their products
                // are +0); the moments are never stored
                wv[u] = gv[u] = mv[u] = vv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
#pragma unroll
        for (int u = 0; u < kStepUnroll; ++u) {
            if (GUARD && base + u * TEAM >= nq) break;
            const int q = base + u * TEAM + tl;
            const uint32_t kmin = min(min(tiny_key(wv[u].x), tiny_key(wv[u].y)),
                                      min(tiny_key(wv[u].z), tiny_key(wv[u].w)));
            if (__builtin_expect(kmin < tkey, 0)) quad_a(wv[u], gv[u], mv[u], vv[u], std::true_type{});
            else quad_a(wv[u], gv[u], mv[u], vv[u], std::false_type{});
            if (!GUARD || q < nq) {
                wr[q] = wv[u];
                st_stream(&mr[q], mv[u]);
                st_stream(&vr[q], vv[u]);
            }
        }
    };
    for (int base = 0; base < nfull; base += STEP) pass_a(base, std::false_type{});
    if (nfull < nq) pass_a(nfull, std::true_type{});

    // dalpha, then AdamW on alpha (same operations in every lane).
    acc = team_sum<WPR>(acc, lds_d);
    const float da = static_cast<float>(m.grad_scale * acc);
    float ma = m.m_alpha[row], va = m.v_alpha[row];
    const float alpha_new = adam_one(ak, alpha_raw, da, ma, va);
    if (tl == 0) {
        m.alpha[row] = alpha_new;
        m.m_alpha[row] = ma;
        m.v_alpha[row] = va;
        if (m.dalpha) m.dalpha[row] = da;
    }

    // Pass B: the next forward on the updated row.
    if (!m.wq_bf16 && !m.codes) return;
    const float a2 = alpha_new > kAlphaFloor ? alpha_new : kAlphaFloor;
    const double y2 = 1.0 / static_cast<double>(a2);
    PQ_GLOBAL u32x2 *wq16 = m.wq_bf16 ? (PQ_GLOBAL u32x2 *)(static_cast<uint16_t *>(m.wq_bf16) + row * cols) : nullptr;
    PQ_GLOBAL uint8_t *crow = m.codes ? (PQ_GLOBAL uint8_t *)(m.codes + row * (cols * CW / 8)) : nullptr;
    auto pass_b = [&](int base, auto guard_c) {
        constexpr bool GUARD = decltype(guard_c)::value;
        f32x4 v[kStepUnroll];
#pragma unroll
        for (int u = 0; u < kStepUnroll; ++u) {
            const int q = base + u * TEAM + tl;
            if (!GUARD || q < nq) v[u] = wr[q];
            else v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kStepUnroll; ++u) {
            if (GUARD && base + u * TEAM >= nq) break;
            const int q = base + u * TEAM + tl;
            const bool act = !GUARD || q < nq;
            float l0, l1, l2, l3;
            const uint32_t c0 = quant_x<MODE>(v[u].x, div_fast(v[u].x, y2), l0);
            const uint32_t c1 = quant_x<MODE>(v[u].y, div_fast(v[u].y, y2), l1);
            const uint32_t c2 = quant_x<MODE>(v[u].z, div_fast(v[u].z, y2), l2);
            const uint32_t c3 = quant_x<MODE>(v[u].w, div_fast(v[u].w, y2), l3);
            if (wq16 && act)
                st_stream(&wq16[q], u32x2{pack_bf16x2(a2 * l0, a2 * l1), pack_bf16x2(a2 * l2, a2 * l3)});
            if (crow) store_codes<CW>(crow, q, c0, c1, c2, c3, act, tl);
        }
    };
    for (int base = 0; base < nfull; base += STEP) pass_b(base, std::false_type{});
    if (nfull < nq) pass_b(nfull, std::true_type{});
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Rows a launch needs before one wave per row fills the chip
// (256 CUs x 4 SIMDs x 4 waves).
constexpr int64_t kWaveRowsThreshold = 4096;
// Mean row length from which a team of four waves per row is faster even
// with many rows (measured: from 4096 columns on, for fwd, bwd and export).
constexpr int64_t kTeamColsThreshold = 4096;

bool finite(double x) { return x == x && x < 1e300 && x > -1e300; }

// Widths with a deployment format: every code container (binary in 1 bit,
// ternary, 2-bit SEQ and the 2-bit LSQ grids in 2, 3- and 4-bit LSQ in 4).
bool deployable(int mode)
{
    return mode == PQ_W1_BINARY || mode == PQ_W158_SEQ_TERNARY || mode == PQ_W2_SEQ || mode == PQ_W3_LSQ ||
           mode == PQ_W4_LSQ || mode == PQ_W2_LSQ || mode == PQ_W158_LSQ;
}

int choose_wpr(int64_t total_rows, int64_t total_elems)
{
    const bool many_rows = total_rows >= kWaveRowsThreshold;
    const bool short_rows = total_elems < kTeamColsThreshold * total_rows;
    return many_rows && short_rows ? 1 : 4;
}

bool ptr_ok(const void *p) { return p == nullptr || aligned16(p); }

// One or more launches over a stack (kMaxGroup matrices each), with one
// team size for the whole stack; `fwd` launches take fwd_rows_per_wave rows
// per wave.
template <typename D, typename F>
pq_status launch_grouped(int count, const D *host, const D *dev, hipStream_t stream, bool fwd, F &&launch_one,
                         bool pad16 = false)
{
    // pad16: the launch also covers the padding rows of each matrix's last
    // 16-row tile (codes in the export byte order)
    auto rows_of = [&](int i) { return pad16 ? (host[i].rows + 15) / 16 * 16 : host[i].rows; };
    int64_t total_rows = 0, total_elems = 0;
    for (int i = 0; i < count; ++i) {
        total_rows += rows_of(i);
        total_elems += rows_of(i) * host[i].cols;
    }
    const int wpr = choose_wpr(total_rows, total_elems);
    const int rpb = (4 / wpr) * (fwd ? fwd_rows_per_wave(wpr, pad16) : 1);  // rows per block
    for (int start = 0; start < count; start += kMaxGroup) {
        const int n = count - start < kMaxGroup ? count - start : kMaxGroup;
        LaunchTableT<D> lt;
        lt.table = dev ? dev + start : nullptr;
        lt.single = host[start];
        lt.count = n;
        int64_t blocks = 0;
        for (int i = 0; i < n; ++i) {
            lt.block_start[i] = static_cast<int32_t>(blocks);
            blocks += (rows_of(start + i) + rpb - 1) / rpb;
            if (blocks > INT32_MAX) return PQ_ERR_SHAPE;
        }
        lt.block_start[n] = static_cast<int32_t>(blocks);
        if (blocks == 0) continue;
        launch_one(lt, static_cast<int>(blocks), wpr, stream);
        if (hipGetLastError() != hipSuccess) return PQ_ERR_HIP;
    }
    return PQ_OK;
}

template <int MODE, bool INIT, unsigned OUTS>
void launch_fwd_t(const LaunchTable &lt, int blocks, int wpr, hipStream_t s, StatsOut so = {})
{
    if (wpr == 1)
        hipLaunchKernelGGL((k_quant_fwd<MODE, INIT, 1, OUTS>), dim3(blocks), dim3(256), 0, s, lt, so);
    else
        hipLaunchKernelGGL((k_quant_fwd<MODE, INIT, 4, OUTS>), dim3(blocks), dim3(256), 0, s, lt, so);
}

// Forward with the fused level statistics (alpha given, codes written,
// optionally the bf16 weights).
template <int MODE>
void launch_fwd_stats_mode(bool bf16, const LaunchTable &lt, int blocks, int wpr, hipStream_t s, StatsOut so)
{
    if (bf16) launch_fwd_t<MODE, false, OUT_STATS | OUT_CODES | OUT_BF16>(lt, blocks, wpr, s, so);
    else launch_fwd_t<MODE, false, OUT_STATS | OUT_CODES>(lt, blocks, wpr, s, so);
}

void launch_fwd_stats(int mode, bool bf16, const LaunchTable &lt, int blocks, int wpr, hipStream_t s, StatsOut so)
{
    switch (mode) {
    case PQ_W1_BINARY: launch_fwd_stats_mode<PQ_W1_BINARY>(bf16, lt, blocks, wpr, s, so); break;
    case PQ_W158_SEQ_TERNARY: launch_fwd_stats_mode<PQ_W158_SEQ_TERNARY>(bf16, lt, blocks, wpr, s, so); break;
    case PQ_W2_SEQ: launch_fwd_stats_mode<PQ_W2_SEQ>(bf16, lt, blocks, wpr, s, so); break;
    case PQ_W3_LSQ: launch_fwd_stats_mode<PQ_W3_LSQ>(bf16, lt, blocks, wpr, s, so); break;
    case PQ_W2_LSQ: launch_fwd_stats_mode<PQ_W2_LSQ>(bf16, lt, blocks, wpr, s, so); break;
    case PQ_W158_LSQ: launch_fwd_stats_mode<PQ_W158_LSQ>(bf16, lt, blocks, wpr, s, so); break;
    default: launch_fwd_stats_mode<PQ_W4_LSQ>(bf16, lt, blocks, wpr, s, so); break;
    }
}

template <int MODE, bool INIT>
void launch_fwd_outs(unsigned outs, const LaunchTable &lt, int blocks, int wpr, hipStream_t s)
{
    switch (outs) {
    case 0: launch_fwd_t<MODE, INIT, 0>(lt, blocks, wpr, s); break;
    case 1: launch_fwd_t<MODE, INIT, 1>(lt, blocks, wpr, s); break;
    case 2: launch_fwd_t<MODE, INIT, 2>(lt, blocks, wpr, s); break;
    case 3: launch_fwd_t<MODE, INIT, 3>(lt, blocks, wpr, s); break;
    case 4: launch_fwd_t<MODE, INIT, 4>(lt, blocks, wpr, s); break;
    case 5: launch_fwd_t<MODE, INIT, 5>(lt, blocks, wpr, s); break;
    case 6: launch_fwd_t<MODE, INIT, 6>(lt, blocks, wpr, s); break;
    case 7: launch_fwd_t<MODE, INIT, 7>(lt, blocks, wpr, s); break;
    default:
        // codes in the export byte order
        switch (outs) {
        case OUT_CODES | OUT_TILED: launch_fwd_t<MODE, INIT, 20>(lt, blocks, wpr, s); break;
        case OUT_BF16 | OUT_CODES | OUT_TILED: launch_fwd_t<MODE, INIT, 21>(lt, blocks, wpr, s); break;
        case OUT_F32 | OUT_CODES | OUT_TILED: launch_fwd_t<MODE, INIT, 22>(lt, blocks, wpr, s); break;
        default: launch_fwd_t<MODE, INIT, 23>(lt, blocks, wpr, s); break;
        }
        break;
    }
}

template <int MODE>
void launch_fwd_mode(bool init, unsigned outs, const LaunchTable &lt, int blocks, int wpr, hipStream_t s)
{
    if (init) launch_fwd_outs<MODE, true>(outs, lt, blocks, wpr, s);
    else launch_fwd_outs<MODE, false>(outs, lt, blocks, wpr, s);
}

void launch_fwd(int mode, bool init, unsigned outs, const LaunchTable &lt, int blocks, int wpr, hipStream_t s)
{
    switch (mode) {
    case PQ_W1_BINARY: launch_fwd_mode<PQ_W1_BINARY>(init, outs, lt, blocks, wpr, s); break;
    case PQ_W158_SEQ_TERNARY: launch_fwd_mode<PQ_W158_SEQ_TERNARY>(init, outs, lt, blocks, wpr, s); break;
    case PQ_W2_SEQ: launch_fwd_mode<PQ_W2_SEQ>(init, outs, lt, blocks, wpr, s); break;
    case PQ_W3_LSQ: launch_fwd_mode<PQ_W3_LSQ>(init, outs, lt, blocks, wpr, s); break;
    case PQ_W2_LSQ: launch_fwd_mode<PQ_W2_LSQ>(init, outs, lt, blocks, wpr, s); break;
    case PQ_W158_LSQ: launch_fwd_mode<PQ_W158_LSQ>(init, outs, lt, blocks, wpr, s); break;
    default: launch_fwd_mode<PQ_W4_LSQ>(init, outs, lt, blocks, wpr, s); break;
    }
}

template <int MODE, int WPR, bool GBF16>
void launch_bwd_t(bool wdw, bool wmask, const LaunchTable &lt, int blocks, hipStream_t s)
{
    if (wdw && wmask)
        hipLaunchKernelGGL((k_quant_bwd<MODE, WPR, GBF16, true, true>), dim3(blocks), dim3(256), 0, s, lt);
    else if (wdw)
        hipLaunchKernelGGL((k_quant_bwd<MODE, WPR, GBF16, true, false>), dim3(blocks), dim3(256), 0, s, lt);
    else if (wmask)
        hipLaunchKernelGGL((k_quant_bwd<MODE, WPR, GBF16, false, true>), dim3(blocks), dim3(256), 0, s, lt);
    else
        hipLaunchKernelGGL((k_quant_bwd<MODE, WPR, GBF16, false, false>), dim3(blocks), dim3(256), 0, s, lt);
}

template <int MODE>
void launch_bwd_mode(int wpr, bool gbf, bool wdw, bool wmask, const LaunchTable &lt, int blocks, hipStream_t s)
{
    if (wpr == 1) {
        if (gbf) launch_bwd_t<MODE, 1, true>(wdw, wmask, lt, blocks, s);
        else launch_bwd_t<MODE, 1, false>(wdw, wmask, lt, blocks, s);
    } else {
        if (gbf) launch_bwd_t<MODE, 4, true>(wdw, wmask, lt, blocks, s);
        else launch_bwd_t<MODE, 4, false>(wdw, wmask, lt, blocks, s);
    }
}

void launch_bwd(int mode, int wpr, bool gbf, bool wdw, bool wmask, const LaunchTable &lt, int blocks, hipStream_t s)
{
    switch (mode) {
    case PQ_W1_BINARY: launch_bwd_mode<PQ_W1_BINARY>(wpr, gbf, wdw, wmask, lt, blocks, s); break;
    case PQ_W158_SEQ_TERNARY: launch_bwd_mode<PQ_W158_SEQ_TERNARY>(wpr, gbf, wdw, wmask, lt, blocks, s); break;
    case PQ_W2_SEQ: launch_bwd_mode<PQ_W2_SEQ>(wpr, gbf, wdw, wmask, lt, blocks, s); break;
    case PQ_W3_LSQ: launch_bwd_mode<PQ_W3_LSQ>(wpr, gbf, wdw, wmask, lt, blocks, s); break;
    case PQ_W2_LSQ: launch_bwd_mode<PQ_W2_LSQ>(wpr, gbf, wdw, wmask, lt, blocks, s); break;
    case PQ_W158_LSQ: launch_bwd_mode<PQ_W158_LSQ>(wpr, gbf, wdw, wmask, lt, blocks, s); break;
    default: launch_bwd_mode<PQ_W4_LSQ>(wpr, gbf, wdw, wmask, lt, blocks, s); break;
    }
}

unsigned fwd_outs(const pq_mat &m)
{
    return (m.wq_bf16 ? OUT_BF16 : 0u) | (m.wq_f32 ? OUT_F32 : 0u) | (m.codes ? OUT_CODES : 0u);
}

pq_status check_fwd_descs(int mode, int count, const pq_mat *host, unsigned flags, unsigned *outs)
{
    if (!valid_mode(mode)) return PQ_ERR_MODE;
    if ((flags & ~(PQ_INIT_ALPHA | PQ_CODES_EXPORT)) != 0) return PQ_ERR_MODE;
    const bool exported = (flags & PQ_CODES_EXPORT) != 0;
    if (exported && !deployable(mode)) return PQ_ERR_MODE;
    if (count < 0) return PQ_ERR_ARG;
    if (count > 0 && !host) return PQ_ERR_NULL;
    bool have_first = false;
    for (int i = 0; i < count; ++i) {
        const pq_mat &m = host[i];
        if (m.rows < 0 || !valid_cols(m.cols)) return PQ_ERR_SHAPE;
        if (m.rows == 0) continue;  // enqueues nothing; its pointers are not used
        const unsigned o = fwd_outs(m) | (exported ? OUT_TILED : 0u);
        if (exported && !m.codes) return PQ_ERR_NULL;
        if (!have_first) {
            *outs = o;
            have_first = true;
        } else if (o != *outs) {
            return PQ_ERR_ARG;  // one output set per launch
        }
        if (!m.W || !m.alpha) return PQ_ERR_NULL;
        if (!aligned16(m.W) || !ptr_ok(m.wq_bf16) || !ptr_ok(m.wq_f32) || !ptr_ok(m.codes) ||
            !ptr_ok(m.alpha))
            return PQ_ERR_ALIGN;
    }
    return PQ_OK;
}

pq_status check_bwd_descs(int mode, int count, const pq_mat *host, int g_dtype, bool *wdw, bool *wmask)
{
    if (!valid_mode(mode)) return PQ_ERR_MODE;
    if (g_dtype != PQ_G_F32 && g_dtype != PQ_G_BF16) return PQ_ERR_MODE;
    if (count < 0) return PQ_ERR_ARG;
    if (count > 0 && !host) return PQ_ERR_NULL;
    bool have_first = false;
    for (int i = 0; i < count; ++i) {
        const pq_mat &m = host[i];
        if (m.rows < 0 || !valid_cols(m.cols)) return PQ_ERR_SHAPE;
        if (m.rows == 0) continue;  // enqueues nothing; its pointers are not used
        if (!m.W || !m.alpha || !m.G || !m.dalpha) return PQ_ERR_NULL;
        if (!aligned16(m.W) || !aligned16(m.G) || !ptr_ok(m.dW) || !ptr_ok(m.mask_bits) ||
            !ptr_ok(m.alpha) || !ptr_ok(m.dalpha))
            return PQ_ERR_ALIGN;
        if (!(m.grad_scale == m.grad_scale) || m.grad_scale > 1e300 || m.grad_scale < -1e300)
            return PQ_ERR_ARG;
        if (g_dtype == PQ_G_BF16 && m.dW && static_cast<const void *>(m.dW) == m.G) return PQ_ERR_ARG;
        const bool d = m.dW != nullptr, k = m.mask_bits != nullptr;
        if (!have_first) {
            *wdw = d;
            *wmask = k;
            have_first = true;
        } else if (d != *wdw || k != *wmask) {
            return PQ_ERR_ARG;
        }
    }
    return PQ_OK;
}

template <int MODE>
void launch_step_mode(int wpr, bool gbf, const StepTable &lt, int blocks, const AdamK &k, hipStream_t s)
{
    if (wpr == 1) {
        if (gbf) hipLaunchKernelGGL((k_qat_step<MODE, 1, true>), dim3(blocks), dim3(256), 0, s, lt, k);
        else hipLaunchKernelGGL((k_qat_step<MODE, 1, false>), dim3(blocks), dim3(256), 0, s, lt, k);
    } else {
        if (gbf) hipLaunchKernelGGL((k_qat_step<MODE, 4, true>), dim3(blocks), dim3(256), 0, s, lt, k);
        else hipLaunchKernelGGL((k_qat_step<MODE, 4, false>), dim3(blocks), dim3(256), 0, s, lt, k);
    }
}

void launch_step(int mode, int wpr, bool gbf, const StepTable &lt, int blocks, const AdamK &k, hipStream_t s)
{
    switch (mode) {
    case PQ_W1_BINARY: launch_step_mode<PQ_W1_BINARY>(wpr, gbf, lt, blocks, k, s); break;
    case PQ_W158_SEQ_TERNARY: launch_step_mode<PQ_W158_SEQ_TERNARY>(wpr, gbf, lt, blocks, k, s); break;
    case PQ_W2_SEQ: launch_step_mode<PQ_W2_SEQ>(wpr, gbf, lt, blocks, k, s); break;
    case PQ_W3_LSQ: launch_step_mode<PQ_W3_LSQ>(wpr, gbf, lt, blocks, k, s); break;
    case PQ_W2_LSQ: launch_step_mode<PQ_W2_LSQ>(wpr, gbf, lt, blocks, k, s); break;
    case PQ_W158_LSQ: launch_step_mode<PQ_W158_LSQ>(wpr, gbf, lt, blocks, k, s); break;
    default: launch_step_mode<PQ_W4_LSQ>(wpr, gbf, lt, blocks, k, s); break;
    }
}


// AdamW scalars: binary64 from the hyper-parameters, rounded once.
pq_status adam_scalars(const pq_adamw *hp, AdamK *k)
{
    if (!hp) return PQ_ERR_NULL;
    const double lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2, eps = hp->eps, wd = hp->weight_decay;
    if (!finite(lr) || !finite(b1) || !finite(b2) || !finite(eps) || !finite(wd)) return PQ_ERR_ARG;
    if (hp->step < 1 || lr < 0.0 || b1 < 0.0 || b1 >= 1.0 || b2 < 0.0 || b2 >= 1.0 || eps <= 0.0 || wd < 0.0)
        return PQ_ERR_ARG;
    const double t = static_cast<double>(hp->step);
    k->b1 = static_cast<float>(b1);
    k->w1 = static_cast<float>(1.0 - b1);
    k->b2 = static_cast<float>(b2);
    k->w2 = static_cast<float>(1.0 - b2);
    k->s2 = static_cast<float>(sqrt(1.0 - pow(b2, t)));
    k->eps = static_cast<float>(eps);
    k->decay = static_cast<float>(1.0 - lr * wd);
    k->step_size = static_cast<float>(lr / (1.0 - pow(b1, t)));
    return PQ_OK;
}

pq_status check_step_descs(int mode, int count, const pq_step_mat *host, int g_dtype)
{
    if (!valid_mode(mode)) return PQ_ERR_MODE;
    if (g_dtype != PQ_G_F32 && g_dtype != PQ_G_BF16) return PQ_ERR_MODE;
    if (count < 0) return PQ_ERR_ARG;
    if (count > 0 && !host) return PQ_ERR_NULL;
    bool have_first = false, wq = false, cd = false, da = false;
    for (int i = 0; i < count; ++i) {
        const pq_step_mat &m = host[i];
        if (m.rows < 0 || !valid_cols(m.cols)) return PQ_ERR_SHAPE;
        if (m.rows == 0) continue;
        if (!m.W || !m.alpha || !m.G || !m.mW || !m.vW || !m.m_alpha || !m.v_alpha) return PQ_ERR_NULL;
        if (!aligned16(m.W) || !aligned16(m.G) || !aligned16(m.mW) || !aligned16(m.vW) ||
            !ptr_ok(m.alpha) || !ptr_ok(m.m_alpha) || !ptr_ok(m.v_alpha) || !ptr_ok(m.wq_bf16) ||
            !ptr_ok(m.codes) || !ptr_ok(m.dalpha))
            return PQ_ERR_ALIGN;
        if (!finite(m.grad_scale)) return PQ_ERR_ARG;
        const bool w = m.wq_bf16 != nullptr, c = m.codes != nullptr, d = m.dalpha != nullptr;
        if (!have_first) {
            wq = w;
            cd = c;
            da = d;
            have_first = true;
        } else if (w != wq || c != cd || d != da) {
            return PQ_ERR_ARG;
        }
    }
    return PQ_OK;
}

// Export: the forward's codes in the export byte order plus bf16(alpha), one
// launch over every matrix's rows rounded up to 16 (the padding rows of each
// last tile are written as zeros).
template <int MODE>
void launch_pack_mode(const LaunchTable &lt, int blocks, int wpr, hipStream_t s)
{
    launch_fwd_t<MODE, false, OUT_CODES | OUT_TILED | OUT_ALPHA_BF16>(lt, blocks, wpr, s);
}

pq_status check_pack_descs(int mode, int count, const pq_mat *host)
{
    if (!deployable(mode)) return PQ_ERR_MODE;
    if (count < 0) return PQ_ERR_ARG;
    if (count > 0 && !host) return PQ_ERR_NULL;
    for (int i = 0; i < count; ++i) {
        const pq_mat &m = host[i];
        if (m.rows < 0 || !valid_cols(m.cols)) return PQ_ERR_SHAPE;
        if (m.rows == 0) continue;  // enqueues nothing; its pointers are not used
        if (!m.W || !m.alpha || !m.codes || !m.alpha_bf16) return PQ_ERR_NULL;
        if (!aligned16(m.W) || !aligned16(m.alpha) || !aligned16(m.codes) || !aligned16(m.alpha_bf16))
            return PQ_ERR_ALIGN;
    }
    return PQ_OK;
}

pq_status pack_grouped(int mode, int count, const pq_mat *host, const pq_mat *dev, void *stream)
{
    return launch_grouped(
        count, host, dev, static_cast<hipStream_t>(stream), true,
        [&](const LaunchTable &lt, int blocks, int wpr, hipStream_t s) {
            switch (mode) {
            case PQ_W1_BINARY: launch_pack_mode<PQ_W1_BINARY>(lt, blocks, wpr, s); break;
            case PQ_W158_SEQ_TERNARY: launch_pack_mode<PQ_W158_SEQ_TERNARY>(lt, blocks, wpr, s); break;
            case PQ_W2_SEQ: launch_pack_mode<PQ_W2_SEQ>(lt, blocks, wpr, s); break;
            case PQ_W3_LSQ: launch_pack_mode<PQ_W3_LSQ>(lt, blocks, wpr, s); break;
            case PQ_W2_LSQ: launch_pack_mode<PQ_W2_LSQ>(lt, blocks, wpr, s); break;
            case PQ_W158_LSQ: launch_pack_mode<PQ_W158_LSQ>(lt, blocks, wpr, s); break;
            default: launch_pack_mode<PQ_W4_LSQ>(lt, blocks, wpr, s); break;
            }
        },
        true);
}

pq_status pack_common(int mode, int64_t rows, int64_t cols, const float *W,
                             const float *alpha, uint8_t *packed, void *alpha_bf16, void *stream)
{
    pq_mat m = {};
    m.W = W;
    m.alpha = const_cast<float *>(alpha);
    m.codes = packed;
    m.alpha_bf16 = alpha_bf16;
    m.rows = rows;
    m.cols = cols;
    if (!deployable(mode)) return PQ_ERR_MODE;
    if (!W || !alpha || !packed || !alpha_bf16) return PQ_ERR_NULL;
    const pq_status st = check_pack_descs(mode, 1, &m);
    if (st != PQ_OK) return st;
    return pack_grouped(mode, 1, &m, nullptr, stream);
}

}  // namespace
}  // namespace pq

using namespace pq;

extern "C" {

int64_t pq_code_row_bytes(int mode, int64_t cols)
{
    if (!valid_mode(mode) || cols <= 0) return -1;
    return (cols * code_bits(mode) + 7) / 8;
}

int64_t pq_packed_bytes(int mode, int64_t rows, int64_t cols)
{
    if (!deployable(mode) || rows < 0 || !valid_cols(cols)) return -1;
    const int64_t rb = cols * code_bits(mode) / 8;
    return (rb + 63) / 64 * ((rows + 15) / 16 * 16) * 64;
}

double pq_default_grad_scale(int mode, int64_t rows, int64_t cols)
{
    if (!valid_mode(mode) || rows <= 0 || cols <= 0) return 0.0;
    const double qp = mode == PQ_W3_LSQ ? 3.0 : (mode == PQ_W4_LSQ ? 7.0 : 1.0);
    return 1.0 / sqrt(static_cast<double>(rows) * static_cast<double>(cols) * qp);
}

const char *pq_status_str(pq_status s)
{
    switch (s) {
    case PQ_OK: return "PQ_OK";
    case PQ_ERR_NULL: return "PQ_ERR_NULL: a required pointer is NULL";
    case PQ_ERR_SHAPE: return "PQ_ERR_SHAPE: bad rows/cols/M/N/K (cols and K must be positive multiples of 8)";
    case PQ_ERR_MODE: return "PQ_ERR_MODE: unknown mode, flag or dtype";
    case PQ_ERR_ALIGN: return "PQ_ERR_ALIGN: array pointer not 16-byte aligned";
    case PQ_ERR_UNSUPPORTED: return "PQ_ERR_UNSUPPORTED";
    case PQ_ERR_HIP: return "PQ_ERR_HIP: kernel launch failed";
    case PQ_ERR_ARG: return "PQ_ERR_ARG: bad argument (descriptor table, grad_scale or aliasing)";
    }
    return "unknown pq_status";
}

const char *pq_version(void) { return "libpq 0.1 (gfx950)"; }

pq_status pq_quantize_fwd_grouped(int mode, int count, const pq_mat *descs_host,
                                  const pq_mat *descs_dev, unsigned flags, void *stream)
{
    unsigned outs = 0;
    pq_status st = check_fwd_descs(mode, count, descs_host, flags, &outs);
    if (st != PQ_OK) return st;
    if (count > 0 && !descs_dev) return PQ_ERR_NULL;
    const bool init = (flags & PQ_INIT_ALPHA) != 0;
    return launch_grouped(
        count, descs_host, descs_dev, static_cast<hipStream_t>(stream), true,
        [&](const LaunchTable &lt, int blocks, int wpr, hipStream_t s) { launch_fwd(mode, init, outs, lt, blocks, wpr, s); },
        (flags & PQ_CODES_EXPORT) != 0);
}

pq_status pq_quantize_fwd(int mode, int64_t rows, int64_t cols, const float *W, float *alpha,
                          unsigned flags, void *Wq_bf16, float *Wq_f32, uint8_t *codes,
                          void *stream)
{
    pq_mat m = {};
    m.W = W;
    m.alpha = alpha;
    m.wq_bf16 = Wq_bf16;
    m.wq_f32 = Wq_f32;
    m.codes = codes;
    m.rows = rows;
    m.cols = cols;
    unsigned outs = 0;
    pq_status st = check_fwd_descs(mode, 1, &m, flags, &outs);
    if (st != PQ_OK) return st;
    const bool init = (flags & PQ_INIT_ALPHA) != 0;
    return launch_grouped(
        1, &m, static_cast<const pq_mat *>(nullptr), static_cast<hipStream_t>(stream), true,
        [&](const LaunchTable &lt, int blocks, int wpr, hipStream_t s) { launch_fwd(mode, init, outs, lt, blocks, wpr, s); },
        (flags & PQ_CODES_EXPORT) != 0);
}

pq_status pq_quantize_fwd_stats(int mode, int64_t rows, int64_t cols, const float *W, const float *alpha,
                                void *Wq_bf16, uint8_t *codes, uint32_t *counts, double *entropy, void *stream)
{
    using namespace pq;
    pq_mat m = {};
    m.W = W;
    m.alpha = const_cast<float *>(alpha);
    m.wq_bf16 = Wq_bf16;
    m.codes = codes;
    m.rows = rows;
    m.cols = cols;
    unsigned outs = 0;
    pq_status st = check_fwd_descs(mode, 1, &m, 0u, &outs);
    if (st != PQ_OK) return st;
    if (rows == 0) return PQ_OK;
    if (!codes || !counts) return PQ_ERR_NULL;
    if (!ptr_ok(counts) || !ptr_ok(entropy)) return PQ_ERR_ALIGN;
    const StatsOut so{counts, entropy};
    return launch_grouped(1, &m, static_cast<const pq_mat *>(nullptr), static_cast<hipStream_t>(stream), true,
                          [&](const LaunchTable &lt, int blocks, int wpr, hipStream_t s) {
                              launch_fwd_stats(mode, Wq_bf16 != nullptr, lt, blocks, wpr, s, so);
                          });
}

pq_status pq_quantize_bwd_grouped(int mode, int count, const pq_mat *descs_host,
                                  const pq_mat *descs_dev, int g_dtype, void *stream)
{
    bool wdw = false, wmask = false;
    pq_status st = check_bwd_descs(mode, count, descs_host, g_dtype, &wdw, &wmask);
    if (st != PQ_OK) return st;
    if (count > 0 && !descs_dev) return PQ_ERR_NULL;
    return launch_grouped(count, descs_host, descs_dev, static_cast<hipStream_t>(stream), false,
                          [&](const LaunchTable &lt, int blocks, int wpr, hipStream_t s) {
                              launch_bwd(mode, wpr, g_dtype == PQ_G_BF16, wdw, wmask, lt, blocks, s);
                          });
}

pq_status pq_quantize_bwd(int mode, int64_t rows, int64_t cols, const float *W, const float *alpha,
                          const void *G, int g_dtype, double grad_scale, float *dW, float *dalpha,
                          uint8_t *mask_bits, void *stream)
{
    pq_mat m = {};
    m.W = W;
    m.alpha = const_cast<float *>(alpha);
    m.G = G;
    m.dW = dW;
    m.dalpha = dalpha;
    m.mask_bits = mask_bits;
    m.grad_scale = grad_scale;
    m.rows = rows;
    m.cols = cols;
    bool wdw = false, wmask = false;
    pq_status st = check_bwd_descs(mode, 1, &m, g_dtype, &wdw, &wmask);
    if (st != PQ_OK) return st;
    return launch_grouped(1, &m, static_cast<const pq_mat *>(nullptr), static_cast<hipStream_t>(stream),
                          false,
                          [&](const LaunchTable &lt, int blocks, int wpr, hipStream_t s) {
                              launch_bwd(mode, wpr, g_dtype == PQ_G_BF16, wdw, wmask, lt, blocks, s);
                          });
}

pq_status pq_pack_grouped(int mode, int count, const pq_mat *descs_host, const pq_mat *descs_dev, void *stream)
{
    const pq_status st = check_pack_descs(mode, count, descs_host);
    if (st != PQ_OK) return st;
    if (count > 0 && !descs_dev) return PQ_ERR_NULL;
    return pack_grouped(mode, count, descs_host, descs_dev, stream);
}

pq_status pq_pack(int mode, int64_t rows, int64_t cols, const float *W, const float *alpha, uint8_t *packed,
                  void *alpha_bf16, void *stream)
{
    return pack_common(mode, rows, cols, W, alpha, packed, alpha_bf16, stream);
}

pq_status pq_pack_w2(int64_t rows, int64_t cols, const float *W, const float *alpha,
                     uint8_t *packed, void *alpha_bf16, void *stream)
{
    return pack_common(PQ_W2_SEQ, rows, cols, W, alpha, packed, alpha_bf16, stream);
}

pq_status pq_pack_w4(int64_t rows, int64_t cols, const float *W, const float *alpha,
                     uint8_t *packed, void *alpha_bf16, void *stream)
{
    return pack_common(PQ_W4_LSQ, rows, cols, W, alpha, packed, alpha_bf16, stream);
}

pq_status pq_qat_step_grouped(int mode, int count, const pq_step_mat *descs_host, const pq_step_mat *descs_dev,
                              int g_dtype, const pq_adamw *hp, void *stream)
{
    pq_status st = check_step_descs(mode, count, descs_host, g_dtype);
    if (st != PQ_OK) return st;
    AdamK k;
    st = adam_scalars(hp, &k);
    if (st != PQ_OK) return st;
    if (count > 0 && !descs_dev) return PQ_ERR_NULL;
    return launch_grouped(count, descs_host, descs_dev, static_cast<hipStream_t>(stream), false,
                          [&](const StepTable &lt, int blocks, int wpr, hipStream_t s) {
                              launch_step(mode, wpr, g_dtype == PQ_G_BF16, lt, blocks, k, s);
                          });
}

pq_status pq_qat_step(int mode, int64_t rows, int64_t cols, float *W, float *alpha, const void *G, int g_dtype,
                      double grad_scale, float *mW, float *vW, float *m_alpha, float *v_alpha,
                      const pq_adamw *hp, void *Wq_bf16, uint8_t *codes, float *dalpha, void *stream)
{
    pq_step_mat m = {};
    m.W = W;
    m.alpha = alpha;
    m.G = G;
    m.mW = mW;
    m.vW = vW;
    m.m_alpha = m_alpha;
    m.v_alpha = v_alpha;
    m.wq_bf16 = Wq_bf16;
    m.codes = codes;
    m.dalpha = dalpha;
    m.grad_scale = grad_scale;
    m.rows = rows;
    m.cols = cols;
    pq_status st = check_step_descs(mode, 1, &m, g_dtype);
    if (st != PQ_OK) return st;
    AdamK k;
    st = adam_scalars(hp, &k);
    if (st != PQ_OK) return st;
    return launch_grouped(1, &m, static_cast<const pq_step_mat *>(nullptr), static_cast<hipStream_t>(stream), false,
                          [&](const StepTable &lt, int blocks, int wpr, hipStream_t s) {
                              launch_step(mode, wpr, g_dtype == PQ_G_BF16, lt, blocks, k, s);
                          });
}

}  // extern "C"
