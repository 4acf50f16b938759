// pq_quant_kernels.hpp -- gfx950 kernels of the per-row weight quantizer:
// alpha init, forward fake-quantization, straight-through backward with the
// scale gradient, export packing and the fused QAT step, with their per-mode
// launchers.  Internal header: pq_quant_mode.hip instantiates the launchers
// of one mode per translation unit (so the modes compile in parallel), and
// pq_quant.hip holds the host side and the C entry points.
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

#pragma once

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

// Level statistics fused into the forward (OUT_STATS, single matrix): per
// row the count of each stored code [rows, levels] and its entropy in bits.
struct StatsOut {
    uint32_t *counts;
    double *entropy;
};

// AdamW scalars of one step, rounded once to binary32 on the host.
struct AdamK {
    float b1, w1, b2, w2, s2, eps, decay, step_size;
};

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

// Quads handled per lane per pass, U: every load of a pass is issued before
// any math.  4, or 8 when the launch's longest row needs more than four
// quads per lane of its team, so that rows of up to 2048 columns (one wave)
// or 8192 (a team of four) are read in one pass: one round trip to HBM per
// row (measured: the MobileLLM-1.5B stack's 1600-column rows took two
// passes of four, 62.7 % of HBM peak for the forward).
constexpr int kPassNarrow = 4;
constexpr int kPassWide = 8;
// Scale init: rows of up to kInitSmall (or kInitLarge) quads per lane of the
// team -- 1536 (4352) columns with one wave per row, 6144 (17408) with four
// -- are read from HBM once and held in registers from the statistic to the
// quantization; longer rows take two passes.
constexpr int kInitSmall = 6;
constexpr int kInitLarge = 17;

enum : unsigned { OUT_BF16 = 1, OUT_F32 = 2, OUT_CODES = 4, OUT_ALPHA_BF16 = 8, OUT_TILED = 16, OUT_STATS = 32 };

// Forward rows per wave: with one wave per row (launches of many short
// rows) each wave takes two rows in turn, which halves the number of waves
// to launch and retire; a team of four waves takes one row.  Codes in the
// export byte order take one row per wave, so that the rows sharing a
// 128-byte line of the export are written close together in time (with an
// earlier layout whose lines held 16-byte pieces of 8 rows, two rows per
// wave let lines leave L2 partly written: 21x the code bytes written, 2.4x
// the time; with the current layout two rows per wave, in either order,
// still made the export 1.5-2.7x slower).
#ifndef PQ_FWD_RPW
#define PQ_FWD_RPW 2
#endif
#ifndef PQ_FWD_XCD_REMAP
#define PQ_FWD_XCD_REMAP 1
#endif
constexpr int fwd_rows_per_wave(int wpr, bool tiled) { return wpr == 1 && !tiled ? PQ_FWD_RPW : 1; }

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
// Waves per SIMD the forward's register allocation must allow: the plain
// forward keeps eight (HBM latency), five with eight-quad passes; the 1-bit
// one one fewer, for the registers of its cross-lane code gather; the fused
// statistics and the scale init with up to six quads per lane in registers
// four, and with seventeen three (a whole 4352-column row per wave: 17 KB in
// flight per wave).
constexpr int fwd_waves_per_eu(int mode, int iq, unsigned outs, int u)
{
    return iq > 6 ? (mode == PQ_W1_BINARY ? 2 : 3)
           : (iq > 0 || (outs & OUT_STATS)) ? PQ_QUANT_FWD_MINB / 2
           : u > kPassNarrow ? (mode == PQ_W1_BINARY ? 4 : 5)
           : mode == PQ_W1_BINARY ? 6 : PQ_QUANT_FWD_MINB;
}

// IQ = 0: alpha given.  IQ > 0: INIT -- alpha from the row statistic, with
// rows of up to IQ quads per lane of the team held in registers.
template <int MODE, int IQ, int WPR, unsigned OUTS, int U>
__global__ __launch_bounds__(256, fwd_waves_per_eu(MODE, IQ, OUTS, U)) void k_quant_fwd(LaunchTable lt, StatsOut so)
{
    constexpr bool INIT = IQ > 0;
    constexpr int kInitQuads = IQ > 0 ? IQ : 1;
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
    {
        // The eight XCDs take blocks round robin; give the blocks of one XCD
        // consecutive rows, so that rows whose codes share cache lines (the
        // 16 rows of an export tile; row-major code rows that are not whole
        // 128-byte lines) are written through one L2.
        const int nb = gridDim.x;
        if ((TILED || PQ_FWD_XCD_REMAP) && (nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
    }
    const int k = find_matrix(lt, b);
    const pq_mat m = lt.table ? lt.table[lt.idx[k]] : lt.single;
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

        PQ_GLOBAL u32x2 *wq16 =
            (OUTS & OUT_BF16) ? (PQ_GLOBAL u32x2 *)(static_cast<uint16_t *>(m.wq_bf16) + row * cols) : nullptr;
        PQ_GLOBAL f32x4 *wq32 = (OUTS & OUT_F32) ? (PQ_GLOBAL f32x4 *)(m.wq_f32 + row * cols) : nullptr;
        PQ_GLOBAL uint8_t *crow = (OUTS & OUT_CODES) ? (PQ_GLOBAL uint8_t *)(m.codes + row * (cols * CW / 8)) : nullptr;
        // 1-bit codes go out as dwords gathered from eight lanes when every
        // eight-quad group of the row is whole and the row's bytes start on
        // a 4-byte boundary (cols a multiple of 32; the export order's
        // 64-byte slots always do)
        const bool bits_by_dword = CW == 1 && (TILED || (cols & 31) == 0);

        uint32_t *whist = hist + (STATS ? (threadIdx.x >> 6) * L * 64 + (threadIdx.x & 63) : 0);
        if constexpr (STATS) {
#pragma unroll
            for (int l = 0; l < L; ++l) whist[l * 64] = 0u;
        }

        auto finish_row = [&]() __attribute__((always_inline)) {
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
                // zero the bytes of the last group past the row's end (< 64
                // bytes); 2-bit rows end on a whole word of the export
                const int64_t rb = CW == 2 ? (cols * CW / 8 + 3) / 4 * 4 : cols * CW / 8;
                const int64_t kb = rb + tl;
                if (kb < gbytes) tbase[(kb >> 6) * gstride + (kb & 63)] = 0;
            }
        };

        // One quad: quantize, emit every output.  `sbase` is the first quad
        // of the team-wide slot (a multiple of TEAM) that quad q belongs to;
        // every lane of the team makes this call for the slot (the 1-bit
        // gathers shuffle across lanes), `act` gates the stores.
        auto emit = [&](float a, double y, int sbase, int q, const f32x4 &v, bool act) __attribute__((always_inline)) {
            float l0, l1, l2, l3;
            const uint32_t c0 = quant_x<MODE>(v.x, div_fast(v.x, y), l0);
            const uint32_t c1 = quant_x<MODE>(v.y, div_fast(v.y, y), l1);
            const uint32_t c2 = quant_x<MODE>(v.z, div_fast(v.z, y), l2);
            const uint32_t c3 = quant_x<MODE>(v.w, div_fast(v.w, y), l3);
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
                if (act) {
                    const u32x2 hv = u32x2{pack_bf16x2(q0, q1), pack_bf16x2(q2, q3)};
                    if (lt.nt_out) st_stream(&wq16[q], hv);
                    else wq16[q] = hv;
                }
            }
            if constexpr ((OUTS & OUT_F32) != 0) {
                if (act) {
                    if (lt.nt_out) st_stream(&wq32[q], f32x4{q0, q1, q2, q3});
                    else wq32[q] = f32x4{q0, q1, q2, q3};
                }
            }
            if constexpr (CW == 1 && (OUTS & OUT_CODES) != 0) {
                // 1 bit: a nibble per quad; lanes 8j .. 8j+7 hold eight
                // consecutive quads, i.e. 4 code bytes, combined into lane
                // 8j's dword (inactive lanes contribute zeros).
                const uint32_t nib = act ? (c0 | (c1 << 1) | (c2 << 2) | (c3 << 3)) : 0u;
                const uint32_t b8 = nib | (__shfl_down(nib, 1) << 4);
                if (bits_by_dword) {
                    const uint32_t b16 = b8 | (__shfl_down(b8, 2) << 8);
                    const uint32_t b32 = b16 | (__shfl_down(b16, 4) << 16);
                    if ((tl & 7) == 0 && act) {
                        PQ_GLOBAL uint8_t *d;
                        if constexpr (TILED) d = tbase + static_cast<int64_t>(q >> 7) * gstride + ((q >> 1) & 63);
                        else d = crow + (q >> 1);
                        *(PQ_GLOBAL uint32_t *)d = b32;
                    }
                } else if (act && (tl & 1) == 0) {
                    PQ_GLOBAL uint8_t *d;
                    if constexpr (TILED) d = tbase + static_cast<int64_t>(q >> 7) * gstride + ((q >> 1) & 63);
                    else d = crow + (q >> 1);
                    *d = static_cast<uint8_t>(b8);
                }
            } else if constexpr (TILED) {
                // A quad is CW / 2 code bytes, and the slot base starts a
                // whole 64-byte group g0; the lane's byte offset from there
                // (tl or 2 tl) splits into group and byte.
                const int64_t g0 = (static_cast<int64_t>(sbase) * (CW / 2)) >> 6;
                if constexpr (CW == 2) {
                    // Four lanes' quads are one 4-byte word of the export,
                    // whose byte j holds codes 2j, 8+2j, 2j+1, 9+2j of the
                    // word's 16 (bits 0-1, 2-3, 4-5, 6-7).  Quads 0 and 2 make
                    // bytes 0-1, quads 1 and 3 bytes 2-3: each lane spreads
                    // its codes over a halfword (the word's second half one
                    // bit pair higher), adds its partner's (lane tl ^ 2) and
                    // writes byte 2 (qq & 1) + (qq >> 1).  Quads past the row
                    // end add zeros; a word holding any code of the row is
                    // written whole.
                    const int qq = tl & 3;
                    uint32_t h = act ? (c0 | (c1 << 4) | (c2 << 8) | (c3 << 12)) : 0u;
                    h <<= 2 * (qq >> 1);
                    h |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(h), 2));
                    const int wq0 = sbase + (tl & ~3);  // the word's first quad in the row
                    if (wq0 * 4 < cols) {
                        PQ_GLOBAL uint8_t *d =
                            tbase + (g0 + (tl >> 6)) * gstride + ((tl & 60) + 2 * (qq & 1) + (qq >> 1));
                        *d = static_cast<uint8_t>(h >> (8 * (qq >> 1)));
                    }
                } else {
                    PQ_GLOBAL uint8_t *d = tbase + (g0 + (tl >> 5)) * gstride + ((2 * tl) & 63);
                    if (act) *(PQ_GLOBAL uint16_t *)d = static_cast<uint16_t>(c0 | (c1 << 4) | (c2 << 8) | (c3 << 12));
                }
            } else if constexpr ((OUTS & OUT_CODES) != 0) {
                store_codes<CW>(crow, q, c0, c1, c2, c3, act, tl);
            }
        };

        // The INIT statistic of a row held in registers (zeros in the slots
        // past the row's end change neither a max nor a sum of magnitudes):
        // [Note] "The 2-bit recipe" table / scale-init row of "Paper vs.
        // code" -- max|w| (SEQ, ternary), max|w| / Qp (LSQ), mean|w| summed
        // in binary64 (1 bit).
        auto row_init_stat = [&](const f32x4 (&c)[kInitQuads]) __attribute__((always_inline)) -> float {
            if constexpr (MODE == PQ_W1_BINARY) {
                double sacc = 0.0;
#pragma unroll
                for (int u = 0; u < kInitQuads; ++u) {
                    sacc += static_cast<double>(fabsf(c[u].x));
                    sacc += static_cast<double>(fabsf(c[u].y));
                    sacc += static_cast<double>(fabsf(c[u].z));
                    sacc += static_cast<double>(fabsf(c[u].w));
                }
                sacc = team_sum<WPR>(sacc, lds_d);
                return static_cast<float>(sacc / static_cast<double>(cols));
            } else {
                float mx = 0.0f;
#pragma unroll
                for (int u = 0; u < kInitQuads; ++u)
                    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(c[u].x), fabsf(c[u].y)), fmaxf(fabsf(c[u].z), fabsf(c[u].w))));
                mx = team_max<WPR>(mx, lds_f);
                if constexpr (MODE == PQ_W3_LSQ || MODE == PQ_W4_LSQ || MODE == PQ_W2_LSQ || MODE == PQ_W158_LSQ)
                    mx = mx / Mode<MODE>::hi;
                return mx;
            }
        };

        // Scale of the row: given, or (INIT) the row statistic.  With INIT a
        // row of at most kInitQuads quads per lane is read once: its quads
        // stay in registers from the statistic to the quantization.
        float alpha_raw = 0.0f;
        if constexpr (INIT) {
            if (nq <= kInitQuads * TEAM) {
                f32x4 c[kInitQuads];
#pragma unroll
                for (int u = 0; u < kInitQuads; ++u) {
                    const int q = u * TEAM + tl;
                    c[u] = q < nq ? ld_stream(&wr[q]) : f32x4{0.f, 0.f, 0.f, 0.f};
                }
                alpha_raw = row_init_stat(c);
                if (tl == 0) m.alpha[row] = alpha_raw;
                const float a = alpha_raw > kAlphaFloor ? alpha_raw : kAlphaFloor;
                const double y = 1.0 / static_cast<double>(a);
                if constexpr ((OUTS & OUT_ALPHA_BF16) != 0) {
                    if (tl == 0) {
                        __bf16 h = static_cast<__bf16>(alpha_raw);
                        static_cast<uint16_t *>(m.alpha_bf16)[row] = __builtin_bit_cast(uint16_t, h);
                    }
                }
#pragma unroll
                for (int u = 0; u < kInitQuads; ++u) {
                    if (u * TEAM >= nq) break;  // slot empty for the whole team
                    const int q = u * TEAM + tl;
                    emit(a, y, u * TEAM, q, c[u], q < nq);
                }
                finish_row();
                return;
            }
            // longer rows: a first pass for the statistic, then the quantization pass
            if constexpr (MODE == PQ_W1_BINARY) {
                double sacc = 0.0;
                for (int q = tl; q < nq; q += TEAM) {
                    const f32x4 v = wr[q];
                    sacc += static_cast<double>(fabsf(v.x));
                    sacc += static_cast<double>(fabsf(v.y));
                    sacc += static_cast<double>(fabsf(v.z));
                    sacc += static_cast<double>(fabsf(v.w));
                }
                sacc = team_sum<WPR>(sacc, lds_d);
                alpha_raw = static_cast<float>(sacc / static_cast<double>(cols));
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

        // One pass: U quads per lane, loads first.  GUARD only on the last.
        auto pass = [&](int base, auto guard_c) {
            constexpr bool GUARD = decltype(guard_c)::value;
            f32x4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int q = base + u * TEAM + tl;
                if (!GUARD || q < nq) v[u] = ld_stream(&wr[q]);
                else v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                // in the tail pass, quad slots no lane of the team owns are skipped
                if (GUARD && base + u * TEAM >= nq) break;
                const int q = base + u * TEAM + tl;
                emit(a, y, base + u * TEAM, q, v[u], !GUARD || q < nq);
            }
        };
        constexpr int STEP = TEAM * U;
        const int nfull = nq / STEP * STEP;
        for (int base = 0; base < nfull; base += STEP) pass(base, std::false_type{});
        if (nfull < nq) pass(nfull, std::true_type{});
        finish_row();
    };
#pragma unroll 1
    for (int rr = 0; rr < RPW; ++rr) one_row(row0 + rr * RPB);
}

// Backward: per weight the forward's x and level (bit-identical), the clip
// gate, dW = inside ? G : +0, and the binary64 alpha-gradient partial
// (level - x inside, the boundary level outside).
template <int MODE, int WPR, bool GBF16, bool WDW, bool WMASK, int U>
__global__ __launch_bounds__(256, PQ_QUANT_BWD_MINB) void k_quant_bwd(LaunchTable lt)
{
    constexpr int RPB = 4 / WPR;
    constexpr int TEAM = 64 * WPR;
    __shared__ double lds_d[4];

    const int wave = threadIdx.x >> 6;
    const int tl = (wave % WPR) * 64 + (threadIdx.x & 63);
    const int b = blockIdx.x;
    const int k = find_matrix(lt, b);
    const pq_mat m = lt.table ? lt.table[lt.idx[k]] : lt.single;
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

    // One pass: U quads per lane; all W and G loads are issued before
    // any store, so dW may overwrite G in place.  A quad holding a weight
    // with a quotient below 2^-125 (0 < |w| < a * 2^-123) takes the exact
    // body (rare); the test is one unsigned min per weight.  The mask
    // nibbles are paired across lanes after the (divergent) quad bodies.
    auto pass = [&](int base, auto guard_c) {
        constexpr bool GUARD = decltype(guard_c)::value;
        f32x4 wv[U], gv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
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
        for (int u = 0; u < U; ++u) {
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
            for (int u = 0; u < U; ++u) {
                const int q = base + u * TEAM + tl;
                const bool act = !GUARD || q < nq;
                if (act && (tl & 1) == 0)
                    mrow[q >> 1] = static_cast<uint8_t>(((nibs >> (4 * u)) & 0xFu) | (((hi >> (4 * u)) & 0xFu) << 4));
            }
        }
    };
    constexpr int STEP = TEAM * U;
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
    const pq_step_mat m = lt.table ? lt.table[lt.idx[k]] : lt.single;
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

}  // namespace

// ---------------------------------------------------------------------------
// Per-mode launchers (defined and instantiated in pq_quant_mode.hip, one
// translation unit per mode).  init: 0 (alpha given) or the register depth of
// the scale init; u: quads per lane per pass; wpr: waves per row.
// ---------------------------------------------------------------------------
template <int MODE>
void launch_fwd_m(int init, unsigned outs, int u, const LaunchTable &lt, int blocks, int wpr, hipStream_t s);
template <int MODE>
void launch_fwd_stats_m(bool bf16, const LaunchTable &lt, int blocks, int wpr, hipStream_t s, StatsOut so);
template <int MODE>
void launch_pack_m(int u, const LaunchTable &lt, int blocks, int wpr, hipStream_t s);
template <int MODE>
void launch_bwd_m(int u, int wpr, bool gbf, bool wdw, bool wmask, const LaunchTable &lt, int blocks, hipStream_t s);
template <int MODE>
void launch_step_m(int wpr, bool gbf, const StepTable &lt, int blocks, const AdamK &k, hipStream_t s);

}  // namespace pq
