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
//    reach the MFMA B (or A) operand straight from packed codes, decoded in
//    registers into an exact bf16 value v; every width's level is affine in
//    the code, level = step * (c - zc), so the kernels accumulate X.v and the
//    epilogue applies level = mul * (v - off) with the X row sums:
//      2-bit container (2-bit SEQ, ternary): gfx950's fp4 -> bf16 pair
//        convert (v_cvt_scalef32_pk_bf16_fp4, scale 1) reads a masked nibble
//        0..3 as the fp4 value v = c/2; SEQ levels (c - 1.5)/2 give off =
//        0.75, mul = 1; ternary levels (c - 1) * 2/3 give off = 0.5, mul =
//        2 * 2/3.
//      4-bit container (4- and 3-bit LSQ): v = 128 + c (streaming kernel) or
//        v = 2 + c/8 (tiled kernel) from the bf16 mantissa; level = c - 8
//        (c - 4 at 3 bits).
//  * The weights are read in the export byte order (1-KB tiles of 16 rows x
//    64 code bytes, group-major) with the LDS-DMA load; the streaming kernel
//    (M <= 16) reads them exactly once, the tiled kernel (M > 16) once per
//    64-row tile of activations.  See each kernel below.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "pq_common.hpp"
#include "pq_gemm_common.hpp"

// Tiled-kernel LDS ring depth (2- and 4-bit); streaming-kernel shape: waves
// per block, groups in flight per wave and column tiles per block.
#ifndef PQ_TILE_WN
#define PQ_TILE_WN 4
#endif
#ifndef PQ_TILE_DMA_MID
#define PQ_TILE_DMA_MID 1
#endif
#ifndef PQ_TILE_P2
#define PQ_TILE_P2 4
#endif
#ifndef PQ_TILE_P4
#define PQ_TILE_P4 4
#endif
// Code fetches in the tiled kernel's LDS ring (2- and 4-bit; 1-bit keeps 2):
// with 3, two fetches of weight codes are in flight behind the one in use.
// 1: 192-column tiled blocks (four waves of 48 columns) where they pad N
// less than 256-column ones.
#ifndef PQ_TILE_NARROW
#define PQ_TILE_NARROW 1
#endif
#ifndef PQ_TILE_NCB
#define PQ_TILE_NCB 2
#endif
// Fewest K stages per split of the tiled kernel's K split.
#ifndef PQ_TILE_MIN_STAGES
#define PQ_TILE_MIN_STAGES 4
#endif
// Blocks of a tiled launch with more output tiles x splits than this many
// (a multiple of 8; two per CU): each block then takes several in turn
// (0: one block per item).
#ifndef PQ_TILE_PERSIST
#define PQ_TILE_PERSIST 512
#endif
// 1: the tiled kernel takes its row sums on the matrix unit (one MFMA per
// k-step with an all-ones A operand) instead of 4 v_dot2 per k-step; it ran
// 1-7 % faster on eight of nine shapes measured (16384^2 at M = 64..256,
// the Llama-3-8B and training-forward shapes), the ninth unchanged.
#ifndef PQ_TILE_RS_MFMA
#define PQ_TILE_RS_MFMA 1
#endif
#ifndef PQ_STREAM_NW
#define PQ_STREAM_NW 4
#endif
// 2-bit streaming configurations with at most this many activation DMAs per
// group (M <= 4) use eight waves per block, two per SIMD, so that one wave's
// decode overlaps the other's MFMAs and DMA waits (measured at 16384^2:
// M = 1 16.0 -> 14.7 us, M = 4 17.4 -> 16.1 us, with two stages in flight
// per wave instead of three); 0: none do.
#ifndef PQ_STREAM_NW8_XI
#define PQ_STREAM_NW8_XI 2
#endif
#ifndef PQ_STREAM_TN
#define PQ_STREAM_TN 4
#endif
// 2-bit streaming configurations with at least this many activation DMAs
// per group (M >= 3) take the activation row sums on the matrix unit, one
// MFMA per k-step against an all-ones operand, instead of 4 v_dot2 per DMA
// on the VALU, which bounds these launches (16384^2 back to back: M = 16
// 21.8 -> 19.1 us, M = 8 18.0 -> 16.4, M = 4 15.6 -> 15.1; M <= 2, with one
// DMA per group, keeps the 4 v_dot2).
#ifndef PQ_STREAM_RS_MFMA_XI
#define PQ_STREAM_RS_MFMA_XI 2
#endif
// 4-bit streaming kernel: column tiles per block (with one activation DMA
// per group, and with more), stages for 1, 2, 4 DMAs
#ifndef PQ_STREAM4_TN1
#define PQ_STREAM4_TN1 2
#endif
#ifndef PQ_STREAM4_TN
#define PQ_STREAM4_TN 4
#endif
#ifndef PQ_STREAM4_D1
#define PQ_STREAM4_D1 3
#endif
#ifndef PQ_STREAM4_D2
#define PQ_STREAM4_D2 3
#endif
#ifndef PQ_STREAM4_D4
#define PQ_STREAM4_D4 3
#endif
// streaming-kernel stages in flight for 1, 2, 4 and 8 activation DMAs per
// group.  Measured on the export byte order: three stages (12-15 KB per
// wave) stream faster than five or six.
#ifndef PQ_STREAM_D1
#define PQ_STREAM_D1 3
#endif
#ifndef PQ_STREAM_D2
#define PQ_STREAM_D2 3
#endif
#ifndef PQ_STREAM_D4
#define PQ_STREAM_D4 3
#endif
#ifndef PQ_STREAM_D8
#define PQ_STREAM_D8 2
#endif

namespace pq {
namespace {


// ---------------------------------------------------------------------------
// Tiled kernel for M > 16.
//
// A block owns a 64 x 256 output tile; its four waves each own 64 columns
// (4 x 4 MFMA tiles of 16 x 16), so every wave reads the whole 64-row
// activation tile and every decoded weight fragment feeds four MFMAs.  Where
// 192-column tiles pad N less (N = 576), the waves own 48 columns (4 x 3
// MFMA tiles) and the code fetches shrink to match.  K runs
// in stages of 64.  Each stage's activation tile (64 rows x 128 B) is copied
// global -> LDS by the gfx950 LDS-DMA load (global_load_lds_dwordx4), with no
// register or VALU traffic, into a ring of four stage buffers kept three
// stages ahead.  Codes are fetched the same way but one 64-byte group per
// column at a time (four stages at 2 bits, two at 4): in the export byte
// order a group of 16 columns is one contiguous 1-KB tile, so every DMA
// instruction reads 1 KB in one piece; the fetches are double-buffered.  One
// s_waitcnt plus one barrier per stage orders both rings.
//
// LDS activation layout: row r holds its eight 16-byte k-chunks with chunk c
// stored in slot c ^ xswz(r).  The DMA writes 1 KB contiguous per wave
// instruction (eight rows), so the swizzle is applied on the global side:
// the lane that fills slot s of row r fetches chunk s ^ xswz(r).
//
// Lane (i16, grp) takes k = 16 * grp + 8 * t + [0, 8) of the stage at k-step
// t, so its codes for a stage are one dword (2-bit) or two (4-bit), and the
// decode yields the eight codes in natural k order:
//   2-bit: the export orders each code word so that w0 = d & 0x33333333
//          holds codes 0..7 as fp4 nibbles in k order (low nibble of each
//          byte first) and w1 = (d >> 2) & 0x33333333 codes 8..15; the
//          fp4 -> bf16 pair converts of w0's four bytes give k-step 0 as c/2,
//          those of w1 k-step 1.
//   4-bit: byte p of d & 0x0F0F0F0F and of (d >> 4) & 0x0F0F0F0F hold codes
//          2p and 2p+1; a byte permute places them in the two bf16 halves and
//          (q << 3) | 0x40004000 makes 2 + c/8.
// Row sums of X for the level offset come from v_dot2_f32_bf16 on the A
// fragments already in registers (wave w sums row tile w).
//
// When the tile grid is too small to fill the chip, K is split over blocks;
// each split writes fp32 partials (with its own offset term) to a
// workspace and a second kernel sums the splits, scales by alpha and rounds
// to bf16.  Block order is XCD-aware: the eight XCDs take workgroups round
// robin, so consecutive tile indices are given to the blocks of one XCD and
// the m-tiles that share a weight tile share that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kTileM = 64;
// Largest K and N: the DMA loads address with 32-bit offsets from a
// wave-uniform base -- up to 64 activation rows, or one 64-byte group of all
// weight rows (N * 64 bytes).
constexpr int64_t kMaxGemmK = int64_t(1) << 24;
constexpr int64_t kMaxGemmN = int64_t(1) << 24;

struct TileArgs {
    const uint16_t *X;       // [M, K] bf16
    const uint8_t *packed;   // export byte order (see GemmArgs)
    const uint16_t *alpha;   // [N] bf16
    uint16_t *Y;             // [M, N] bf16 (single split)
    float *ws;               // [splits, M, N] fp32 partials (several splits)
    int M, N, K;
    int mtiles, ntiles, splits;
    int kps;                 // k per split, a multiple of the 64-byte group
    int64_t gstride;         // bytes per 64-byte group of all rows
    float off, mul;          // level = mul * (v - off) for the decoded operand v
    const float *alpha32;    // [N] binary32 scale, or nullptr (use alpha)
    int nfast;               // item order: column tile fastest (1) or row tile fastest (0)
};


// Tile of WN waves along N (16 JW columns each: JW = 4, or 3 where 192-column
// blocks pad N less): 64 x 16*JW*WN outputs per block.
template <int BITS, int WN, int JW = 4>
struct TileCfg {
    static constexpr int WC = 16 * JW;                   // columns per wave
    static constexpr int TN = WC * WN;                   // columns per block
    static constexpr int CB = 8 * BITS;                  // code bytes per column per stage
    static constexpr int XBYTES = kTileM * kStageK * 2;  // 8 KB
    static constexpr int CBYTES = TN * CB;               // codes of one stage
    static constexpr int SS = 64 / CB;                   // stages per code fetch (64 B per column)
    static constexpr int CSS = SS * CBYTES;              // codes of one fetch
    static constexpr int P = BITS == 2 ? PQ_TILE_P2 : PQ_TILE_P4;  // activation ring depth
    static constexpr int XI = 8 / WN;                    // activation DMAs per wave per stage
    static constexpr int NC = JW;                        // code DMAs per wave per fetch
    static constexpr int NCB = BITS == 1 ? 2 : PQ_TILE_NCB;  // code fetches in the ring
    static constexpr int LDS = P * XBYTES + NCB * CSS;
    static_assert(WN == 4, "block width: the epilogue stages 2 KB per wave in one 8-KB slot");
    static_assert(JW == 3 || JW == 4, "48 or 64 columns per wave");
    static_assert(NC * WN * 1024 == CSS, "one fetch is NC 1-KB DMAs per wave");
    static_assert(P >= 3, "activation ring depth");
    static_assert(NCB == 2 || NCB == 3, "code ring depth");
};



// 1-bit decode: the eight codes of byte b (first code lowest) spread to the
// eight nibbles of a word, each nibble 2 * code: the e2m1 value of the code
// (0 or 1.0), so the fp4 -> bf16 pair converts of bytes 0..3 give codes
// 0..7 in order.
__device__ __forceinline__ uint32_t spread_bits_fp4(uint32_t b)
{
    uint32_t x = (b | (b << 12)) & 0x000F000Fu;
    x = (x | (x << 6)) & 0x03030303u;
    x = (x | (x << 3)) & 0x11111111u;
    return x << 1;
}

template <int BITS, int P, int WN, int JW>
__global__ __launch_bounds__(64 * WN, 8 / WN) void k_gemm_tile(TileArgs g)
{
    using C = TileCfg<BITS, WN, JW>;
    constexpr int WC = C::WC;
    static_assert(P >= 3, "ring depth");
    // LDS: P activation stages, then NCB code fetches.  Between items,
    // activation slot P - 1 stages the outputs: the next item's prologue
    // fills slots 0 .. P-2 only, and its first refill of slot P - 1 comes
    // after a barrier that every wave reaches past its epilogue.
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS];
    __shared__ float ssum[kTileM];
    constexpr int XR = 0;                 // activation region
    constexpr int CR = P * C::XBYTES;     // code region
    constexpr int NCB = C::NCB;
    static_assert(C::LDS + kTileM * 4 <= 80 * 1024, "two blocks per CU");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i16 = lane & 15, grp = lane >> 4;

    // Work items (m-tile, n-tile, split); the block takes items blockIdx.x,
    // blockIdx.x + gridDim.x, ...  With the item count and the grid multiples
    // of 8, item i is remapped so that consecutive indices -- the m-tiles
    // sharing a weight tile, or with g.nfast the n-tiles sharing a row
    // tile -- fall to one XCD (the eight XCDs take workgroups round robin, so
    // all of a block's items stay on its XCD).
    const int nitems = g.mtiles * g.ntiles * g.splits;
    const int nb = gridDim.x;
    const bool remap = (nitems & 7) == 0 && (nb & 7) == 0;
    const int M = g.M, N = g.N, K = g.K;
    constexpr int NC = C::NC;
    constexpr int SS = C::SS;
    const int cpiece = lane >> 4;
    const int cstage = (16 * cpiece) / C::CB, cwithin = (16 * cpiece) % C::CB;

    // The current item: its tile, K range and DMA sources (a wave-uniform
    // base, advanced per stage, plus a fixed per-lane byte offset; rows >= M
    // and columns >= N read row M-1 / N-1).  Code DMAs: one fetch covers SS
    // stages of the block's columns, one 64-byte group of each.  DMA i of
    // wave w brings columns 16 (NC w + i) .. +15, which is one 1-KB tile of
    // the export order: lane l reads the 16-byte piece l >> 4 of column
    // l & 15 (tile offset 64 (l & 15) + 16 (l >> 4)) and it lands as
    // [piece][16 columns][16 B] in LDS.
    int m0 = 0, n0 = 0, split = 0, kbeg = 0, ns = 0;
    int64_t g_first = 0;
    const uint8_t *xbase = nullptr;
    uint32_t xoff[C::XI], ccol[NC];
    auto setup = [&](int item) {
        int t = remap ? (item & 7) * (nitems >> 3) + (item >> 3) : item;
        int mt, nt;
        if (g.nfast) {
            nt = t % g.ntiles;
            t /= g.ntiles;
            mt = t % g.mtiles;
            split = t / g.mtiles;
        } else {
            mt = t % g.mtiles;
            t /= g.mtiles;
            nt = t % g.ntiles;
            split = t / g.ntiles;
        }
        m0 = mt * kTileM;
        n0 = nt * C::TN;
        kbeg = split * g.kps;
        ns = (min(K, kbeg + g.kps) - kbeg) / kStageK;
        xbase = reinterpret_cast<const uint8_t *>(g.X + static_cast<int64_t>(m0) * K + kbeg);
#pragma unroll
        for (int q = 0; q < C::XI; ++q) {
            const int r = 8 * (C::XI * w + q) + (lane >> 3);
            const int c = (lane & 7) ^ xswz(r);
            xoff[q] = static_cast<uint32_t>(static_cast<int64_t>(min(m0 + r, M - 1) - m0) * K * 2 + 16 * c);
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int cl = min(n0 + 16 * (NC * w + i) + (lane & 15), N - 1);
            ccol[i] = static_cast<uint32_t>((cl >> 4) * 1024 + (cl & 15) * 64);
        }
        g_first = kbeg / (SS * kStageK);  // the split starts a group
    };
    const uint32_t lds_base = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t *)lds));

    // Activation DMA of stage st (clamped to the last stage, so that every
    // iteration issues the same loads) into ring slot `slot`.
    auto issue_x = [&](int st, int slot) {
        const uint8_t *xs = xbase + min(st, ns - 1) * (kStageK * 2);
#pragma unroll
        for (int q = 0; q < C::XI; ++q)
            dma16(xs, xoff[q], lds_base + XR + slot * C::XBYTES + (C::XI * w + q) * 1024);
    };
    // Code DMA of fetch G (group g_first + G) into buffer `buf` (G mod NCB);
    // a lane whose stage lies past the split's end re-reads the last stage
    // (in bounds, never used), which lies in the same group or, for a fetch
    // wholly past the end, in the split's last group.
    auto issue_c = [&](int G, int buf) {
        const int st = min(G * SS + cstage, ns - 1);
        const uint8_t *cb = g.packed + (g_first + min(G, (ns - 1) / SS)) * g.gstride;
        const uint32_t po = static_cast<uint32_t>((((st % SS) * C::CB + cwithin) >> 4) * 16);
#pragma unroll
        for (int i = 0; i < NC; ++i)
            dma16<PQ_NT_TILE>(cb, ccol[i] + po, lds_base + CR + buf * C::CSS + (NC * w + i) * 1024);
    };

    floatx4 acc[4][JW];
    float rs = 0.f;
    floatx4 accrs = floatx4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 ones8 = __builtin_bit_cast(bf16x8, uint4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);

    // Loop-invariant per-lane LDS addresses; a[i] is row tile (i + w) & 3 so
    // that a[0] is the tile whose row sums this wave keeps.
    const int swz = xswz(i16);
    const uint8_t *xa[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int T = 0; T < 2; ++T)
            xa[i][T] = lds + XR + (16 * ((i + w) & 3) + i16) * 128 + (((2 * grp + T) ^ swz) << 4);
    // Code reads: the wave's column 16j + i16 is in DMA block NC w + j; 2-bit
    // lanes take dword grp of the stage's 16-byte piece, 4-bit lanes bytes
    // 8 (grp & 1) of piece 2 (stage) + (grp >> 1).
    const uint8_t *ca = lds + CR + (NC * w) * 1024 + i16 * 16 +
                        (BITS == 1 ? 2 * grp : BITS == 2 ? 4 * grp : 8 * (grp & 1) + 256 * (grp >> 1));

    // Fragments of one stage: A for both k-steps and the code words.
    struct Frag {
        uint4 a[2][4];
        uint32_t d[JW][BITS == 4 ? 2 : 1];
    };
    // Fragments of stage st, with PH = st mod U known at compile time
    // (activation slot PH mod P, code buffer (PH / SS) mod NCB, stage PH mod SS).
    auto read_frags = [&](auto ph_c, Frag &f) {
        constexpr int PH = decltype(ph_c)::value;
        constexpr int SLOT = PH % P;
        constexpr int CBUF = (PH / C::SS) % NCB;
        constexpr int CST = PH % C::SS;
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            // stage CST's bytes: 8, 16 or 32 per column, in the 16-byte pieces
            const uint8_t *p = ca + CBUF * C::CSS + j * 1024 +
                               (C::CB == 8 ? (CST >> 1) * 256 + (CST & 1) * 8 : CST * (C::CB == 16 ? 256 : 512));
            if constexpr (BITS == 1) {
                f.d[j][0] = *reinterpret_cast<const uint16_t *>(p);
            } else if constexpr (BITS == 2) {
                f.d[j][0] = *reinterpret_cast<const uint32_t *>(p);
            } else {
                const uint2 v = *reinterpret_cast<const uint2 *>(p);
                f.d[j][0] = v.x;
                f.d[j][1] = v.y;
            }
        }
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                f.a[T][i] = *reinterpret_cast<const uint4 *>(xa[i][T] + SLOT * C::XBYTES);
    };
    auto mma = [&](const Frag &f, auto &&between) {
        // 2 bits: the code word's masked nibbles are its codes 0..7 (w0)
        // and 8..15 (w1) in k order, one k-step each (the export's word order)
        uint32_t w0[JW], w1[JW];
        if constexpr (BITS == 2) {
#pragma unroll
            for (int j = 0; j < JW; ++j) {
                const uint32_t x = f.d[j][0];
                w0[j] = x & 0x33333333u;
                w1[j] = (x >> 2) & 0x33333333u;
            }
        }
        static_for<0, 2>([&](auto tc) {
            constexpr int T = decltype(tc)::value;
#pragma unroll
            for (int j = 0; j < JW; ++j) {
                uint4 b;
                if constexpr (BITS == 1) {
                    const uint32_t x = spread_bits_fp4((f.d[j][0] >> (8 * T)) & 0xFFu);
                    b.x = fp4x2_to_bf16x2<0>(x);
                    b.y = fp4x2_to_bf16x2<1>(x);
                    b.z = fp4x2_to_bf16x2<2>(x);
                    b.w = fp4x2_to_bf16x2<3>(x);
                } else if constexpr (BITS == 2) {
                    const uint32_t wt = T == 0 ? w0[j] : w1[j];
                    b.x = fp4x2_to_bf16x2<0>(wt);
                    b.y = fp4x2_to_bf16x2<1>(wt);
                    b.z = fp4x2_to_bf16x2<2>(wt);
                    b.w = fp4x2_to_bf16x2<3>(wt);
                } else {
                    const uint32_t x = f.d[j][T];
                    const uint32_t lo = x & 0x0F0F0F0Fu;
                    const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;
                    b.x = (__builtin_amdgcn_perm(hi, lo, 0x0C040C00u) << 3) | 0x40004000u;
                    b.y = (__builtin_amdgcn_perm(hi, lo, 0x0C050C01u) << 3) | 0x40004000u;
                    b.z = (__builtin_amdgcn_perm(hi, lo, 0x0C060C02u) << 3) | 0x40004000u;
                    b.w = (__builtin_amdgcn_perm(hi, lo, 0x0C070C03u) << 3) | 0x40004000u;
                }
                const bf16x8 bv = __builtin_bit_cast(bf16x8, b);
                // Weights as the MFMA A operand: the lane's outputs are four
                // consecutive columns n of one row m.
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, __builtin_bit_cast(bf16x8, f.a[T][i]),
                                                                         acc[i][j], 0, 0, 0);
            }
            const uint4 aw = f.a[T][0];
            if constexpr (PQ_TILE_RS_MFMA != 0) {
                // row m = 16 w + i16 of the tile, summed over the k-step
                accrs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, __builtin_bit_cast(bf16x8, aw), accrs, 0, 0, 0);
            } else {
                rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, aw.x), ones2, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, aw.y), ones2, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, aw.z), ones2, rs, false);
                rs = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, aw.w), ones2, rs, false);
            }
            if constexpr (T == 0) {
                __builtin_amdgcn_sched_barrier(0);
                between();
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };

    // Pipeline.  Activation DMAs run P - 1 stages ahead; code fetch G + NCB
    // is issued in the last iteration that reads fetch G's buffer (after its
    // barrier), (NCB - 1) SS stages before it is needed.  Iteration s waits for
    // stage s + 1 (and its codes), passes the barrier, refills, reads stage
    // s + 1's fragments and multiplies stage s.  The wait count of each
    // unrolled phase comes from tile_wait: the DMAs issued after the newer of
    // the two it needs may stay in flight.
    //
    // A block with several items issues the next item's prologue DMAs as soon
    // as the current item's ring is free (after the row-sum barrier), then
    // writes the current item's outputs, so the next item's first loads are
    // in flight during the epilogue.  The prologue wait stays correct with
    // those stores outstanding: the loads retire in order among themselves,
    // so at most (P - 2) XI + (NCB - 1) NC operations outstanding still
    // means that code fetch 0 and activation stage 0 have landed.
    constexpr int U = lcm_int(P, NCB * C::SS);   // unroll: phases of slots and buffers
    static_assert(U % P == 0 && U % (NCB * C::SS) == 0, "unroll covers both rings");
    Frag fr[2];
    auto prologue = [&]() {
        issue_c(0, 0);
#pragma unroll
        for (int st = 0; st < P - 1; ++st) issue_x(st, st);
#pragma unroll
        for (int G = 1; G < NCB; ++G) issue_c(G, G);
    };
    int item = blockIdx.x;
    setup(item);
    prologue();
    for (;;) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JW; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
    rs = 0.f;
    accrs = floatx4{0.f, 0.f, 0.f, 0.f};
    // activation stage 0 and code fetch 0 landed
    wait_vmcnt<(P - 2) * C::XI + (NCB - 1) * NC>();
    block_barrier();
    read_frags(std::integral_constant<int, 0>{}, fr[0]);
    auto step = [&](int s, auto pc) {
        constexpr int p = decltype(pc)::value;  // s mod U
        constexpr bool code_now = ((p + 1) % C::SS) == 0;
        // The code refill below overwrites the buffer that holds stage s's
        // codes, read in the previous iteration: those reads (long since
        // issued) complete before the barrier.
        wait_lgkmcnt0();
        wait_vmcnt<tile_wait(p, P, C::SS, C::XI, NC, U, NCB)>();
        block_barrier();
        // A wave just released from the barrier issues at raised priority
        // until its refill is out: its fragment reads, first MFMAs and DMAs
        // then go ahead of the other block's wave on the same SIMD, which is
        // in the middle of its own MFMAs (measured: M = 512 at 16384^2,
        // 218 -> 206 us back to back; M = 256, 123 -> 114 us).
        __builtin_amdgcn_s_setprio(1);
        auto refill = [&]() {
            issue_x(s + P - 1, (p + P - 1) % P);
            if constexpr (code_now) issue_c((s + 1) / C::SS + NCB - 1, ((p + 1) / C::SS + NCB - 1) % NCB);
        };
        if (PQ_TILE_DMA_MID == 0) refill();
        read_frags(std::integral_constant<int, (p + 1) % U>{}, fr[(p + 1) & 1]);
        // Keep the scheduler from hoisting work on the fragments just
        // requested (which would wait on them) into this step's MFMAs.
        __builtin_amdgcn_sched_barrier(0);
        // The refill goes between the two k-steps' MFMAs, so that the waves
        // leaving the barrier together do not all queue on the vector memory
        // unit before their first MFMA.
        mma(fr[p & 1], [&]() {
            if (PQ_TILE_DMA_MID != 0) refill();
            __builtin_amdgcn_s_setprio(0);
        });
        __builtin_amdgcn_sched_barrier(0);
    };
    int s = 0;
    for (; s + U <= ns; s += U) {
        static_for<0, U>([&](auto pc) { step(s + decltype(pc)::value, pc); });
    }
    // Tail (fewer than U stages left); s is a multiple of U.
    static_for<0, U - 1>([&](auto pc) {
        if (s + decltype(pc)::value < ns) step(s + decltype(pc)::value, pc);
    });
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    // every wave's DMAs have landed and its reads are done: slot P - 1 is free
    block_barrier();

    // Row sums: combine the four k-groups, publish row 16w + i16 (from the
    // matrix unit every lane of column i16 holds the whole sum).
    if constexpr (PQ_TILE_RS_MFMA != 0) {
        rs = accrs[0];
    } else {
        rs += __shfl_xor(rs, 16);
        rs += __shfl_xor(rs, 32);
    }
    if (grp == 0 && w < 4) ssum[16 * w + i16] = rs;
    __syncthreads();

    // One split: this item's per-column scales, loaded and waited for while
    // no DMA is in flight (a wait for them later would also wait for the
    // next item's first loads).
    float al[JW][4];
    if (g.splits == 1) {
        load_col_scales<JW>(g.alpha, g.alpha32, n0 + WC * w + 4 * grp, N, al);
        wait_vmcnt<0>();
    }

    // The next item's prologue, into the ring every wave is done with.
    const int e_m0 = m0, e_n0 = n0, e_split = split;
    const int next = item + nb;
    if (next < nitems) {
        setup(next);
        prologue();
    }

    // Epilogue: acc[i][j][e] is row e_m0 + 16 * ((i + w) & 3) + i16, column
    // e_n0 + WC w + 16j + 4grp + e; four lanes hold a row's WC columns in
    // 8-byte pieces.  One split: each wave passes its rows through 2 KB of
    // slot P - 1, 16 rows at a time, so that every store instruction writes
    // 16 bytes per lane and eight whole 128-byte row segments (16-byte
    // chunks XOR-swizzled by row for the LDS banks).  Several splits: fp32
    // partials, 16 bytes per lane as held.
    if (g.splits == 1) {
        uint8_t *stg = lds + XR + (P - 1) * C::XBYTES + w * 2048;
        const int nw = e_n0 + WC * w + 8 * (lane & 7);   // this lane's 8 output columns
        const bool lane_cols = (lane & 7) < 2 * JW;
        const bool vec8 = (N & 7) == 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rt = (i + w) & 3;
            const float sr = g.off * ssum[16 * rt + i16];
#pragma unroll
            for (int j = 0; j < JW; ++j) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = g.mul * (acc[i][j][e] - sr);
                const int ch = (2 * j + (grp >> 1)) ^ (i16 & 7);
                *reinterpret_cast<u32x2 *>(stg + i16 * 128 + ch * 16 + (grp & 1) * 8) =
                    u32x2{pack_bf16x2(al[j][0] * v[0], al[j][1] * v[1]), pack_bf16x2(al[j][2] * v[2], al[j][3] * v[3])};
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = (lane >> 3) + 8 * h;
                const uint4 d = *reinterpret_cast<const uint4 *>(stg + r * 128 + (((lane & 7) ^ (r & 7)) << 4));
                const int m = e_m0 + 16 * rt + r;
                if (lane_cols && m < M && nw < N) {
                    uint16_t *y = g.Y + static_cast<int64_t>(m) * N + nw;
                    if (vec8) {
                        *reinterpret_cast<uint4 *>(y) = d;
                    } else {
                        const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            if (nw + e < N) y[e] = static_cast<uint16_t>(dw[e >> 1] >> (16 * (e & 1)));
                    }
                }
            }
        }
    } else {
        const bool vec = (N & 3) == 0;
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const int n = e_n0 + WC * w + 16 * j + 4 * grp;
            if (n >= N) continue;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rl = 16 * ((i + w) & 3) + i16;
                const int m = e_m0 + rl;
                if (m >= M) continue;
                const float sr = g.off * ssum[rl];
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = g.mul * (acc[i][j][e] - sr);
                float *dst = g.ws + static_cast<int64_t>(e_split) * M * N + static_cast<int64_t>(m) * N + n;
                if (vec) {
                    *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) dst[e] = v[e];
                }
            }
        }
    }
    if (next >= nitems) break;
    item = next;
    }
}

// Sum of the split-K partials, scaled by alpha and rounded to bf16.  Four
// consecutive elements of the flattened [M, N] output per thread.
__global__ __launch_bounds__(256) void k_splitk_finalize(const float *ws, const uint16_t *alpha, const float *alpha32,
                                                         uint16_t *Y, int64_t total, int N, int splits)
{
    const int64_t i0 = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (i0 >= total) return;
    if (i0 + 4 <= total) {
        f32x4 s = *reinterpret_cast<const f32x4 *>(ws + i0);
        for (int k = 1; k < splits; ++k) s += *reinterpret_cast<const f32x4 *>(ws + k * total + i0);
        uint32_t o[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t e = i0 + 2 * h;
            const float a0 = col_scale(alpha, alpha32, static_cast<int>(e % N));
            const float a1 = col_scale(alpha, alpha32, static_cast<int>((e + 1) % N));
            o[h] = pack_bf16x2(a0 * s[2 * h], a1 * s[2 * h + 1]);
        }
        *reinterpret_cast<u32x2 *>(Y + i0) = u32x2{o[0], o[1]};
    } else {
        for (int64_t e = i0; e < total; ++e) {
            float s = 0.f;
            for (int k = 0; k < splits; ++k) s += ws[k * total + e];
            const __bf16 h = static_cast<__bf16>(col_scale(alpha, alpha32, static_cast<int>(e % N)) * s);
            Y[e] = __builtin_bit_cast(uint16_t, h);
        }
    }
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel for M <= 16 (decode and small batches).
//
// The weight (N*K*BITS/8 bytes, read once) is the whole cost, and HBM gives
// its rate only with tens of KB in flight per CU (about 50-60 KB measured
// best; more slows the stream down).  A block owns TN column
// tiles of 16 and its NW waves share K out by groups (256 k at 2 bits, 128
// at 4: 64 bytes of each weight row), wave w taking groups w, w + NW, ....
// In the export byte order a group of all rows is one contiguous run, so at
// any moment the blocks of the whole grid, which walk the groups in the same
// order, read one window of consecutive addresses: each DMA 1 KB, each block
// TN KB, the grid one run per group.  Every wave streams its groups through a
// private LDS ring of D stages with the LDS-DMA load
// (global_load_lds_dwordx4, no registers used): per group one 1-KB DMA per
// column tile (lane (i16, grp) fetches bytes 16*grp .. 16*grp+15 of the
// group's 64 in row i16) and ceil(M / RPL) 1-KB DMAs of activations, so up to
// D * (TN + XI) KB per wave are in flight.  The ring is private to the wave:
// a stage waits on the wave's own s_waitcnt only, and the block meets at a
// barrier once, to add the NW partial sums.
//
// LDS.  A code block is read back by the lane that fetched each 16 bytes,
// which is that lane's MFMA B fragment for the decode below.  An activation
// DMA holds RPL rows interleaved in 16-byte chunks (lane l fetches chunk
// l / RPL of row RPL*q + l % RPL) and consecutive DMAs sit 16*RPL bytes
// further apart than their size, so the 16 rows one A-operand read touches
// fall on distinct banks.  Rows >= M are fetched as row M - 1; their outputs
// are never stored.  Columns >= N read a clamped row.
//
// Decode.  2-bit: with D & 0x33333333 every nibble holds one code in its low
// two bits, the e2m1 value c/2; v_cvt_scalef32_pk_bf16_fp4 turns each byte
// into two exact bf16, and the export's word order makes the four bytes
// codes 0..7 of the word in k order and those of (D >> 2) & 0x33333333
// codes 8..15, so the activation chunks are used as loaded.
// level = (c - 1.5)/2 = v - 0.75.  4-bit: nibbles are spread into bytes and
// completed to bf16 128 + c (exact); level = v - 136, and the activations
// are put in the matching k order (evens, then odds, of each 8-wide block)
// by byte permutes.  The row sums of X needed by the
// offsets are taken with v_dot2 on the chunk each lane fetched.  The NW
// partial sums are combined in LDS in a fixed order.
// ---------------------------------------------------------------------------
template <int BITS>
struct StreamGeom {
    static constexpr int GK = 512 / BITS;             // k per group (64 bytes of a row)
    static constexpr int RPL = 512 / GK;              // activation rows per 1-KB DMA
    static constexpr int XQS = 1024 + 16 * RPL;       // LDS stride of the activation DMAs
};

template <int BITS, int TN, int NW, int D, int XI>
__global__ __launch_bounds__(64 * NW) void k_gemm_stream(GemmArgs g)
{
    using SG = StreamGeom<BITS>;
    constexpr int GK = SG::GK, RPL = SG::RPL, XQS = SG::XQS;
    constexpr int SLOT = TN * 1024 + XI * XQS;  // one stage: codes, then activations
    constexpr int WLDS = D * SLOT;              // one wave's ring
    constexpr int NACC = TN * 4;
    constexpr int PER_STAGE = TN + XI;          // DMAs per stage
    static_assert(D >= 1 && D * PER_STAGE < 64, "DMAs in flight fit the vmcnt counter");
    static_assert(NW * WLDS + NW * 16 * 4 <= 160 * 1024, "LDS");
    static_assert(NACC * 64 * 4 <= WLDS, "partial sums fit in the wave's ring");
    static_assert(TN <= NW, "one wave finishes each tile");
    static_assert(RPL * XI <= 16 + RPL - 1, "at most 16 activation rows");

    __shared__ __attribute__((aligned(16))) uint8_t lds[NW * WLDS];
    __shared__ float rsum[NW][16];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i16 = lane & 15, grp = lane >> 4;
    const int M = g.M, N = g.N, K = g.K;
    const int n0 = blockIdx.x * 16 * TN;
    const int G = K / GK;
    // This wave's groups are w, w + NW, w + 2 NW, ...: at any moment the
    // block's waves read neighbouring 64-byte pieces of the same rows.
    const int nit = G > w ? (G - w + NW - 1) / NW : 0;

    // DMA sources: a wave-uniform base plus a 32-bit per-lane offset (the
    // host bounds K and N so that every offset fits).  Code tile j of group
    // gi is the 1 KB at gi * gstride + (n0 / 16 + j) * 1024, row r's 64 bytes
    // at 64 r in it: lane (i16, grp) fetches bytes 16 grp .. 16 grp + 15 of
    // row i16, which land at 16 * lane in LDS.  Tiles past the last one
    // re-read it (their outputs are not stored).
    const int last_tile = (N - 1) >> 4;
    uint32_t coff[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j)
        coff[j] = static_cast<uint32_t>(min((n0 >> 4) + j, last_tile) * 1024 + i16 * 64 + grp * 16);
    uint32_t xoff[XI];
#pragma unroll
    for (int q = 0; q < XI; ++q) {
        const int r = min(RPL * q + lane % RPL, M - 1);
        xoff[q] = static_cast<uint32_t>((static_cast<int64_t>(r) * K + (lane / RPL) * 8) * 2);
    }
    const uint32_t ring = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t *)lds)) + w * WLDS;
    const uint8_t *wring = lds + w * WLDS;

    auto issue = [&](int it, int slot) __attribute__((always_inline)) {
        const uint32_t gi = static_cast<uint32_t>(w + NW * it);
        const uint32_t sb = ring + slot * SLOT;
        const uint8_t *cb = g.packed + static_cast<int64_t>(gi) * g.gstride;
#pragma unroll
        for (int j = 0; j < TN; ++j) dma16<PQ_NT_STREAM>(cb, coff[j], sb + j * 1024);
#pragma unroll
        for (int q = 0; q < XI; ++q) dma16(g.X, xoff[q] + gi * (GK * 2), sb + TN * 1024 + q * XQS);
    };

    floatx4 acc[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);
    float rsx[XI];
#pragma unroll
    for (int q = 0; q < XI; ++q) rsx[q] = 0.f;
    constexpr bool RSM = BITS == 2 && XI >= PQ_STREAM_RS_MFMA_XI;  // row sums on the matrix unit
    floatx4 accr = floatx4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 ones8 = __builtin_bit_cast(bf16x8, uint4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    // A-operand row of this lane; rows >= M repeat row M - 1 (an LDS broadcast).
    const int mrow = i16 < M ? i16 : M - 1;
    const int aoff = TN * 1024 + (mrow / RPL) * XQS + (mrow % RPL) * 16;

    auto compute = [&](int slot) __attribute__((always_inline)) {
        const uint8_t *sp = wring + slot * SLOT;
        uint4 c[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) c[j] = *reinterpret_cast<const uint4 *>(sp + j * 1024 + lane * 16);
#pragma unroll
        for (int q = 0; q < (RSM ? 0 : XI); ++q) {
            const uint4 v = *reinterpret_cast<const uint4 *>(sp + TN * 1024 + q * XQS + lane * 16);
            rsx[q] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.x), ones2, rsx[q], false);
            rsx[q] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.y), ones2, rsx[q], false);
            rsx[q] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.z), ones2, rsx[q], false);
            rsx[q] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, v.w), ones2, rsx[q], false);
        }
        // chunk ch of the lane's row sits at aoff + ch * 16 * RPL
        const uint8_t *xa = sp + aoff;
        if constexpr (BITS == 1) {
            // k = 128 grp + [0, 128): chunks 16 grp .. 16 grp + 15; code byte t
            // of the lane's 16 holds k = 128 grp + 8 t + [0, 8), first lowest
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(xa + (16 * grp + t) * 16));
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const uint32_t Dw = (t >> 2) == 0 ? c[j].x : (t >> 2) == 1 ? c[j].y : (t >> 2) == 2 ? c[j].z : c[j].w;
                    const uint32_t x = spread_bits_fp4((Dw >> (8 * (t & 3))) & 0xFFu);
                    uint4 b;
                    b.x = fp4x2_to_bf16x2<0>(x);
                    b.y = fp4x2_to_bf16x2<1>(x);
                    b.z = fp4x2_to_bf16x2<2>(x);
                    b.w = fp4x2_to_bf16x2<3>(x);
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, b), acc[j], 0, 0, 0);
                }
            }
        } else if constexpr (BITS == 2) {
            uint4 ua[8];  // k = 64 * grp + [0, 64): chunks 8 * grp .. 8 * grp + 7
#pragma unroll
            for (int q = 0; q < 8; ++q) ua[q] = *reinterpret_cast<const uint4 *>(xa + (8 * grp + q) * 32);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                // code word d holds k = 64 grp + 16 d + [0, 16): its low
                // nibbles k .. k + 7, its high ones k + 8 .. k + 15, in k
                // order (the export's word order), matching chunks 2d, 2d + 1
                const bf16x8 a_e = __builtin_bit_cast(bf16x8, ua[2 * d]);
                const bf16x8 a_o = __builtin_bit_cast(bf16x8, ua[2 * d + 1]);
                if constexpr (RSM) {
                    accr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_e, ones8, accr, 0, 0, 0);
                    accr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_o, ones8, accr, 0, 0, 0);
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const uint32_t Dw = d == 0 ? c[j].x : d == 1 ? c[j].y : d == 2 ? c[j].z : c[j].w;
                    const uint32_t m0 = Dw & 0x33333333u;
                    const uint32_t m1 = (Dw >> 2) & 0x33333333u;
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
            }
        } else {
            uint4 ua[4];  // k = 32 * grp + [0, 32): chunks 4 * grp .. 4 * grp + 3
#pragma unroll
            for (int q = 0; q < 4; ++q) ua[q] = *reinterpret_cast<const uint4 *>(xa + (4 * grp + q) * 64);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint4 xv = ua[d];
                uint4 a;
                a.x = __builtin_amdgcn_perm(xv.y, xv.x, 0x05040100u);  // x0, x2
                a.y = __builtin_amdgcn_perm(xv.w, xv.z, 0x05040100u);  // x4, x6
                a.z = __builtin_amdgcn_perm(xv.y, xv.x, 0x07060302u);  // x1, x3
                a.w = __builtin_amdgcn_perm(xv.w, xv.z, 0x07060302u);  // x5, x7
                const bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const uint32_t Dw = d == 0 ? c[j].x : d == 1 ? c[j].y : d == 2 ? c[j].z : c[j].w;
                    const uint32_t lo = Dw & 0x0F0F0F0Fu;          // nibbles 0,2,4,6 in bytes
                    const uint32_t hi = (Dw >> 4) & 0x0F0F0F0Fu;   // nibbles 1,3,5,7
                    uint4 b;
                    b.x = (lo & 0xFFu) | ((lo << 8) & 0x00FF0000u) | 0x43004300u;
                    b.y = ((lo >> 16) & 0xFFu) | ((lo >> 8) & 0x00FF0000u) | 0x43004300u;
                    b.z = (hi & 0xFFu) | ((hi << 8) & 0x00FF0000u) | 0x43004300u;
                    b.w = ((hi >> 16) & 0xFFu) | ((hi >> 8) & 0x00FF0000u) | 0x43004300u;
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, b), acc[j], 0, 0, 0);
                }
            }
        }
    };

    // Prologue: the first min(D, nit) stages.  Steady state: stage s is
    // consumed when at most D - 1 later stages are still in flight, and its
    // slot is refilled with stage s + D once its LDS reads have returned.
    // The last stages drain with exact counts.
    const int npro = min(D, nit);
    for (int s = 0; s < npro; ++s) issue(s, s);
    int s = 0, slot = 0;
    for (; s + D < nit; ++s) {
        wait_vmcnt<(D - 1) * PER_STAGE>();
        compute(slot);
        wait_lgkmcnt0();
        issue(s + D, slot);
        slot = slot + 1 == D ? 0 : slot + 1;
    }
    static_for<0, D>([&](auto tc) {
        constexpr int r = D - 1 - decltype(tc)::value;  // stages issued after this one
        const int st = nit - 1 - r;
        if (st >= s) {
            wait_vmcnt<r * PER_STAGE>();
            compute(st % D);
        }
    });

    // Combine the NW partial sums in LDS (fixed order); wave j < TN finishes
    // tile j for all rows.
    __syncthreads();
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(w * NACC + 4 * j + e) * 64 + lane] = acc[j][e];
    // Row sums: reduce over the lanes that fetched chunks of the same row
    // (on the matrix unit: lane (0, grp) holds rows 4 grp .. 4 grp + 3).
    if constexpr (RSM) {
        if (i16 == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) rsum[w][4 * grp + e] = accr[e];
        }
    }
#pragma unroll
    for (int q = 0; q < (RSM ? 0 : XI); ++q) {
        float v = rsx[q];
#pragma unroll
        for (int o = RPL; o < 64; o <<= 1) v += __shfl_xor(v, o);
        const int r = RPL * q + lane % RPL;
        if (lane < RPL && r < 16) rsum[w][r] = v;
    }
    __syncthreads();
    if (w < TN) {
        const int j = w;
        const int n = n0 + 16 * j + i16;
        if (n < N) {
            const float al = col_scale(g.alpha, g.alpha32, n);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = 4 * grp + e;
                if (m < M) {
                    float a = 0.f, sm = 0.f;
                    for (int v = 0; v < NW; ++v) {
                        a += red[(v * NACC + 4 * j + e) * 64 + lane];
                        sm += rsum[v][m];
                    }
                    const float y = al * (g.mul * (a - g.off * sm));
                    const __bf16 h = static_cast<__bf16>(y);
                    g.Y[static_cast<int64_t>(m) * N + n] = __builtin_bit_cast(uint16_t, h);
                }
            }
        }
    }
}

// Streaming-kernel shapes by activation DMAs per group (XI): column tiles
// per block, waves per block, stages in flight.  The 4-bit decode costs
// about twice the VALU work per weight byte, so with few activation rows
// 4-bit blocks take fewer column tiles and the chip runs two per CU.
template <int BITS, int XI>
struct StreamCfg {
    // 1 bit: 16 activation DMAs of one row each (M up to 16) leave LDS for two tiles
    static constexpr int TN = BITS == 1 ? (XI == 16 ? 2 : PQ_STREAM_TN)
                              : BITS == 2 ? PQ_STREAM_TN : (XI == 1 ? PQ_STREAM4_TN1 : PQ_STREAM4_TN);
    static constexpr bool NW8 = BITS == 2 && XI <= PQ_STREAM_NW8_XI;
    static constexpr int NW = NW8 ? 8 : PQ_STREAM_NW;
    static constexpr int D = BITS == 1 ? (XI <= 4 ? 3 : 2)
                             : BITS == 2 ? (NW8 ? 2 : XI == 1 ? PQ_STREAM_D1 : XI == 2 ? PQ_STREAM_D2 : XI <= 4 ? PQ_STREAM_D4 : PQ_STREAM_D8)
                                       : (XI == 1 ? PQ_STREAM4_D1 : XI == 2 ? PQ_STREAM4_D2 : PQ_STREAM4_D4);
};

// Column tiles per block for N: the configured width while it still gives
// about 3/4 of a block per CU, else half of it, down to one tile.  A block
// streams its columns' codes at the rate of its waves' DMAs in flight, so a
// narrow N spread over more, narrower blocks reads faster (N = 4096, M = 1:
// 5.7 us with four tiles per block, 4.1 with one); at 16384 columns four
// tiles measured best (one tile: 19.7 us against 15.9).
constexpr int kStreamMinBlocks = 192;

template <int BITS, int XI, int TN>
void launch_stream_tn(const GemmArgs &a, hipStream_t s)
{
    using C = StreamCfg<BITS, XI>;
    if constexpr (TN > 1) {
        if ((a.N + 16 * TN - 1) / (16 * TN) < kStreamMinBlocks) {
            launch_stream_tn<BITS, XI, TN / 2>(a, s);
            return;
        }
    }
    hipLaunchKernelGGL((k_gemm_stream<BITS, TN, C::NW, C::D, XI>), dim3((a.N + 16 * TN - 1) / (16 * TN)),
                       dim3(64 * C::NW), 0, s, a);
}

template <int BITS, int XI>
void launch_stream(const GemmArgs &a, hipStream_t s)
{
    launch_stream_tn<BITS, XI, StreamCfg<BITS, XI>::TN>(a, s);
}

constexpr int kNumCU = 256;  // MI355X / MI350X compute units

// Estimated time (us) of a tiled launch with `splits` K splits, from
// measurements at 16384^2 and the Llama-3-8B shapes: blocks run in rounds of
// up to two per CU; one stage of a block takes about 0.56 us alone on its CU
// and 0.78 us beside a second block, plus about 3 us of pipeline fill and
// epilogue per round; a split adds its fp32 partials, written and read back
// at about 5 TB/s, and the finalize launch.
double tile_cost(int64_t tiles, int stages, int splits, int64_t M, int64_t N)
{
    const int64_t blocks = tiles * splits;
    const int per_cu = blocks > kNumCU ? 2 : 1;
    const int64_t rounds = (blocks + per_cu * kNumCU - 1) / (per_cu * kNumCU);
    const int sps = (stages + splits - 1) / splits;
    double t = static_cast<double>(rounds) * (sps * (per_cu == 1 ? 0.56 : 0.78) + 3.0);
    if (splits > 1) t += 2.0 + static_cast<double>(splits) * static_cast<double>(M) * static_cast<double>(N) * 8.0 / 5e6;
    return t;
}

// How a GEMM of one shape runs, and the workspace it needs: the plan is a
// pure function of (width, M, N, K), so the size query and the launch agree.
struct GemmPlan {
    enum Path { STREAM, TILE, BIG, WRES } path = STREAM;
    int jw = 4;          // TILE: 16-column tiles per wave (3: 192-column blocks)
    int splits = 1;      // TILE: K splits
    int sps = 0;         // TILE: stages per split (whole 64-byte groups)
    int64_t ws = 0;      // workspace bytes (0: none)
};


// Tiled path: the K split of least estimated time, each split keeping at
// least PQ_TILE_MIN_STAGES stages.
template <int BITS>
void plan_tile(int64_t M, int64_t N, int64_t K, GemmPlan &p)
{
    constexpr int kMinStages = PQ_TILE_MIN_STAGES;
    using C = TileCfg<BITS, PQ_TILE_WN>;
    // 192-column blocks where they pad N less than 256-column ones
    p.jw = PQ_TILE_NARROW && (N + 191) / 192 * 192 < (N + C::TN - 1) / C::TN * C::TN ? 3 : 4;
    const int64_t tn = 16 * p.jw * PQ_TILE_WN;
    const int64_t mtiles = (M + kTileM - 1) / kTileM;
    const int64_t ntiles = (N + tn - 1) / tn;
    const int64_t tiles = mtiles * ntiles;
    const int stages = static_cast<int>(K / kStageK);
    int splits = 1;
    double best = tile_cost(tiles, stages, 1, M, N);
    for (int sp = 2; sp <= std::min(64, stages / kMinStages); ++sp) {
        const double c = tile_cost(tiles, stages, sp, M, N);
        if (c < best) {
            best = c;
            splits = sp;
        }
    }
    // stages per split: whole 64-byte groups, so every split starts a group
    const int sps = ((stages + splits - 1) / splits + C::SS - 1) / C::SS * C::SS;
    splits = (stages + sps - 1) / sps;
    p.path = GemmPlan::TILE;
    p.splits = splits;
    p.sps = sps;
    p.ws = splits > 1 ? static_cast<int64_t>(splits) * M * N * 4 : 0;
}

template <int BITS>
GemmPlan plan_gemm(int64_t M, int64_t N, int64_t K)
{
    constexpr int GK = 512 / BITS;
    GemmPlan p;
    if (M <= 16 && K % GK == 0) {
        p.path = GemmPlan::STREAM;
    } else if (gemm_big_takes(BITS, M, N, K)) {
        p.path = GemmPlan::BIG;
    } else if (gemm_wres_takes(BITS, M, N, K)) {
        p.path = GemmPlan::WRES;
    } else {
        plan_tile<BITS>(M, N, K, p);
    }
    return p;
}

template <int BITS, int JW>
pq_status launch_tile(const GemmArgs &a, const GemmPlan &p, float *ws, hipStream_t s)
{
    using C = TileCfg<BITS, PQ_TILE_WN, JW>;
    const int mtiles = (a.M + kTileM - 1) / kTileM;
    const int ntiles = (a.N + C::TN - 1) / C::TN;
    // the tile kernel's 4-bit operand is 2 + c/8 (the stream kernel's 128 + c)
    const float off = BITS != 4 ? a.off : 2.0f + (a.off - 128.0f) / 8.0f;
    const float mul = BITS != 4 ? a.mul : 8.0f * a.mul;
    // Item order: the blocks of one XCD take consecutive items and share its
    // L2.  Row tile fastest, each XCD reads the activations of all rows
    // (up to 8 copies, one per XCD, or one per column tile if fewer) and a
    // share of the codes; column tile fastest, the other way round.  Take
    // the order of fewer HBM bytes.
    const double xb = 2.0 * a.M * a.K, cb = static_cast<double>(a.N) * a.K * BITS / 8.0;
    const int nfast = std::min(8, mtiles) * cb + xb < cb + std::min(8, ntiles) * xb;
    TileArgs t{a.X, a.packed, a.alpha, a.Y, ws, a.M, a.N, a.K, mtiles, ntiles, p.splits, p.sps * kStageK,
               a.gstride, off, mul, a.alpha32, nfast};
    const int64_t total = static_cast<int64_t>(a.M) * a.N;
    const int64_t items = static_cast<int64_t>(mtiles) * ntiles * p.splits;
    if (items > INT32_MAX) return PQ_ERR_SHAPE;
    // More items than two blocks per CU: persistent blocks, each taking
    // items in turn with the next item's first loads under the epilogue.
    const int64_t blocks = PQ_TILE_PERSIST > 0 && items > PQ_TILE_PERSIST ? PQ_TILE_PERSIST : items;
    hipLaunchKernelGGL((k_gemm_tile<BITS, C::P, PQ_TILE_WN, JW>), dim3(static_cast<unsigned>(blocks)), dim3(64 * PQ_TILE_WN),
                       0, s, t);
    if (p.splits > 1) {
        const int64_t threads = (total + 3) / 4;
        hipLaunchKernelGGL(k_splitk_finalize, dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0, s,
                           t.ws, a.alpha, a.alpha32, a.Y, total, a.N, p.splits);
    }
    return PQ_OK;
}

// Level of a stored code as level = step * (c - zc): the code of level 0
// and the step between levels, per width ([Note] "Finding 3" level sets).
struct LevelMap {
    int bits;
    float zc, step;
};

bool level_map(int mode, LevelMap *lm)
{
    switch (mode) {
    case PQ_W158_SEQ_TERNARY: *lm = {2, 1.0f, static_cast<float>(2.0 / 3.0)}; return true;
    case PQ_W2_SEQ: *lm = {2, 1.5f, 0.5f}; return true;
    case PQ_W3_LSQ: *lm = {4, 4.0f, 1.0f}; return true;
    case PQ_W4_LSQ: *lm = {4, 8.0f, 1.0f}; return true;
    case PQ_W2_LSQ: *lm = {2, 2.0f, 1.0f}; return true;    // the ablation grids ([Rebuttal])
    case PQ_W158_LSQ: *lm = {2, 1.0f, 1.0f}; return true;
    case PQ_W1_BINARY: *lm = {1, 0.5f, 2.0f}; return true;  // level 2c - 1
    default: return false;
    }
}

bool gemm_shape_ok(int64_t M, int64_t N, int64_t K)
{
    return M >= 0 && N >= 0 && K > 0 && K % 64 == 0 && K <= kMaxGemmK && M <= INT32_MAX / 2 && N <= kMaxGemmN;
}

int64_t gemm_ws_bytes(int bits, int64_t M, int64_t N, int64_t K)
{
    if (M == 0 || N == 0) return 0;
    if (bits == 1) return plan_gemm<1>(M, N, K).ws;
    if (bits == 2) return plan_gemm<2>(M, N, K).ws;
    return plan_gemm<4>(M, N, K).ws;
}

template <int BITS>
pq_status gemm(int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
               const void *alpha_bf16, void *Y, void *workspace, int64_t ws_bytes, void *stream,
               const LevelMap &lm, const float *alpha32 = nullptr)
{
    if (!X || !packed || (!alpha_bf16 && !alpha32) || !Y) return PQ_ERR_NULL;
    if (!gemm_shape_ok(M, N, K)) return PQ_ERR_SHAPE;
    if (!aligned16(X) || !aligned16(packed) || !aligned16(Y) || (alpha_bf16 && !aligned16(alpha_bf16)) ||
        (alpha32 && !aligned16(alpha32)))
        return PQ_ERR_ALIGN;
    if (ws_bytes < 0) return PQ_ERR_ARG;
    if (M == 0 || N == 0) return PQ_OK;
    const GemmPlan plan = plan_gemm<BITS>(M, N, K);
    if (plan.ws > 0) {
        if (!workspace) return PQ_ERR_NULL;
        if (!aligned16(workspace)) return PQ_ERR_ALIGN;
        if (ws_bytes < plan.ws) return PQ_ERR_ARG;
    }
    GemmArgs a{static_cast<const uint16_t *>(X), packed, static_cast<const uint16_t *>(alpha_bf16),
               static_cast<uint16_t *>(Y), static_cast<int>(M), static_cast<int>(N), static_cast<int>(K),
               (N + 15) / 16 * 16 * 64,
               // the stream kernel's operand: c (1 bit), c / 2 (2 bits), 128 + c (4 bits); all exact
               BITS == 1 ? lm.zc : BITS == 2 ? lm.zc / 2.0f : 128.0f + lm.zc,
               BITS == 1 ? lm.step : BITS == 2 ? 2.0f * lm.step : lm.step, alpha32};
    hipStream_t s = static_cast<hipStream_t>(stream);
    constexpr int GK = 512 / BITS;
    constexpr int RPL = 512 / GK;
    if (plan.path == GemmPlan::STREAM) {
        if (M <= RPL) launch_stream<BITS, 1>(a, s);
        else if (M <= 2 * RPL) launch_stream<BITS, 2>(a, s);
        else if (M <= 4 * RPL) launch_stream<BITS, 4>(a, s);
        else if (BITS == 1 && M <= 8) launch_stream<BITS, (BITS == 1 ? 8 : 4)>(a, s);
        else launch_stream<BITS, 16 / RPL>(a, s);
    } else if (plan.path == GemmPlan::BIG) {
        const pq_status sb = launch_gemm_big(a, s);
        if (sb != PQ_OK) return sb;
    } else if (plan.path == GemmPlan::WRES) {
        const pq_status sw = launch_gemm_wres(a, s);
        if (sw != PQ_OK) return sw;
    } else {
        const pq_status st = plan.jw == 3 ? launch_tile<BITS, 3>(a, plan, static_cast<float *>(workspace), s)
                                          : launch_tile<BITS, 4>(a, plan, static_cast<float *>(workspace), s);
        if (st != PQ_OK) return st;
    }
    return hipGetLastError() == hipSuccess ? PQ_OK : PQ_ERR_HIP;
}

pq_status gemm_dispatch(int mode, int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
                        const void *alpha_bf16, const float *alpha32, void *Y, void *workspace, int64_t ws_bytes,
                        void *stream)
{
    LevelMap lm;
    if (!level_map(mode, &lm)) return PQ_ERR_MODE;
    if (lm.bits == 1) return gemm<1>(M, N, K, X, packed, alpha_bf16, Y, workspace, ws_bytes, stream, lm, alpha32);
    if (lm.bits == 2) return gemm<2>(M, N, K, X, packed, alpha_bf16, Y, workspace, ws_bytes, stream, lm, alpha32);
    return gemm<4>(M, N, K, X, packed, alpha_bf16, Y, workspace, ws_bytes, stream, lm, alpha32);
}

}  // namespace

int64_t gemm_workspace_need(int mode, int64_t M, int64_t N, int64_t K)
{
    LevelMap lm;
    if (!level_map(mode, &lm) || !gemm_shape_ok(M, N, K)) return -1;
    return gemm_ws_bytes(lm.bits, M, N, K);
}

pq_status gemm_run(int mode, int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
                   const void *alpha_bf16, void *Y, void *workspace, int64_t workspace_bytes, void *stream)
{
    return gemm_dispatch(mode, M, N, K, X, packed, alpha_bf16, nullptr, Y, workspace, workspace_bytes, stream);
}

}  // namespace pq

extern "C" {

int64_t pq_gemm_workspace_bytes(int mode, int64_t M, int64_t N, int64_t K)
{
    pq::LevelMap lm;
    if (!pq::level_map(mode, &lm) || !pq::gemm_shape_ok(M, N, K)) return -1;
    return pq::gemm_ws_bytes(lm.bits, M, N, K);
}

pq_status pq_gemm(int mode, int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
                  const void *alpha_bf16, void *Y, void *workspace, int64_t workspace_bytes, void *stream)
{
    return pq::gemm_dispatch(mode, M, N, K, X, packed, alpha_bf16, nullptr, Y, workspace, workspace_bytes, stream);
}

pq_status pq_gemm_f32a(int mode, int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
                       const float *alpha, void *Y, void *workspace, int64_t workspace_bytes, void *stream)
{
    if (!alpha) {
        pq::LevelMap lm;
        return pq::level_map(mode, &lm) ? PQ_ERR_NULL : PQ_ERR_MODE;
    }
    return pq::gemm_dispatch(mode, M, N, K, X, packed, nullptr, alpha, Y, workspace, workspace_bytes, stream);
}

pq_status pq_w2a16_gemm(int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
                        const void *alpha_bf16, void *Y, void *workspace, int64_t workspace_bytes, void *stream)
{
    return pq_gemm(PQ_W2_SEQ, M, N, K, X, packed, alpha_bf16, Y, workspace, workspace_bytes, stream);
}

pq_status pq_w4a16_gemm(int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
                        const void *alpha_bf16, void *Y, void *workspace, int64_t workspace_bytes, void *stream)
{
    return pq_gemm(PQ_W4_LSQ, M, N, K, X, packed, alpha_bf16, Y, workspace, workspace_bytes, stream);
}

}  // extern "C"
