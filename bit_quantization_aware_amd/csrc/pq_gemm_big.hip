// pq_gemm_big.hip -- the W2A16 GEMM for large M (gfx950): 2-bit codes in the
// export byte order x bf16 activations, 128 x 256 output tiles.
//
// Sources (web pages, cited by title and section):
//   [News] "ParetoQ ... 2-bit kernel" news item -- speed paragraph: the 2-bit
//          weights are used packed by the deployed kernel.
//   [Note] "ParetoQ, the strongest low-bit QAT I could find" -- "Finding 3"
//          (the level sets) and "Paper vs. code" (no bias in the layer).
//
// The tiled kernel of pq_gemm.hip gives each wave a 64 x 64 output tile: per
// 32 MFMAs a wave reads the 64 x 64 activation tile from LDS, decodes 16
// weight columns, sums its rows and passes a barrier.  With M in the
// thousands there are enough output tiles for wider ones: here the 4 waves
// of a block own 64 x 128 outputs each (2 x 2 waves, 4 x 8 MFMA tiles of
// 16 x 16), so every activation fragment read from LDS feeds 8 MFMAs instead
// of 4, and the activation row sums come from 4 extra MFMAs per stage
// against an all-ones operand; two blocks share a CU
// (80 KB of LDS each, 234 VGPRs per lane).  The waves' two halves split
// either the block's rows (128-row blocks) or K (64-row blocks, for M too
// small to give every CU two 128-row blocks); see BigCfg.  A 128 x 128 wave
// tile (256 accumulators per lane, one wave per SIMD) was slower: its
// accumulators no longer fit beside the fragments and moved between AGPRs
// and VGPRs.
//
// Per iteration (one K stage of 64 over 128 rows, or two over 64 rows) the
// block's activations (16 KB) go global -> LDS by the LDS-DMA load into a
// ring of four slots kept three iterations ahead, with the tiled kernel's
// XOR swizzle of 16-byte chunks; the codes come 32 bytes per column (two
// stages) per fetch into a double buffer, two column tiles of the export
// order per 1-KB DMA.  One s_waitcnt plus one barrier per iteration order
// both rings (the wait counts from the shared pipeline model).  Within an
// iteration the wave reads its next k-step's activation fragments and the
// next iteration's code words while its MFMAs on the current ones run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pq_common.hpp"
#include "pq_gemm_common.hpp"

// Smallest M and K, and fewest block tiles, for which the large-M kernel
// runs; elsewhere the tiled kernel of pq_gemm.hip, whose 64 x 256 tiles or K
// split fill the chip better and which needs no row-sum pass (16384^2 at
// M = 512, 256 tiles here: 228 us against 205; N = 1024, K = 4096 at
// M = 4096, 128 tiles: 78 us against 48; the MobileLLM-125M training
// forward, K of 576 and 1536: 10.1 ms against 7.4).
#ifndef PQ_BIG_MIN_M
#define PQ_BIG_MIN_M 1024
#endif
#ifndef PQ_BIG_MIN_K
#define PQ_BIG_MIN_K 2048
#endif
#ifndef PQ_BIG_MIN_TILES
#define PQ_BIG_MIN_TILES 256
#endif
// The K-split form (KH = 2): smallest M and fewest 64 x 256 tiles.
#ifndef PQ_BIG_KH2_MIN_M
#define PQ_BIG_KH2_MIN_M 512
#endif
#ifndef PQ_BIG_KH2_MIN_TILES
#define PQ_BIG_KH2_MIN_TILES 512
#endif

namespace pq {
namespace {

constexpr int kWaveM = 64;                          // rows per wave
constexpr int kRT = kWaveM / 16;                    // MFMA row tiles per wave
constexpr int kBigN = 256;                          // block columns
constexpr int kBigP = 4;                            // activation ring slots
constexpr int kBigXBytes = 2 * kWaveM * kStageK * 2;  // one slot: two halves of 64 rows x 128 B
constexpr int kBigXI = kBigXBytes / 4096;           // activation DMAs per wave per slot
constexpr int kBigNC = 2;                           // code DMAs per wave per fetch
constexpr int kBigCBytes = kBigN * 16 * 2;          // one fetch: 2 stages x 16 B per column
constexpr int kBigLds = kBigP * kBigXBytes + 2 * kBigCBytes;
constexpr int kBigU = 4;                            // unrolled phases: ring slot and code buffer
static_assert(kBigXI * 4 * 1024 == kBigXBytes, "one slot is XI 1-KB DMAs per wave");
static_assert(kBigNC * 4 * 1024 == kBigCBytes, "one fetch is NC 1-KB DMAs per wave");

// Two ways to use the 4 waves (2 x 2, each 64 rows x 128 columns of output):
// KH = 1 splits the block's 128 rows in two, every iteration one K stage,
// the two halves of a ring slot holding the two row halves; KH = 2 gives
// the block 64 rows and splits K, every iteration two K stages (one per
// half of the slot, each wave pair taking one), the two partial sums added
// through LDS at the end.  KH = 2 doubles the blocks for the same M, so a
// 16384^2 GEMM at M = 512 keeps two blocks on every CU.
template <int KH>
struct BigCfg {
    static constexpr int BM = KH == 1 ? 2 * kWaveM : kWaveM;  // block rows
    static constexpr int SS = KH == 1 ? 2 : 1;                // iterations per code fetch
    static_assert(kBigU % kBigP == 0 && kBigU % (2 * SS) == 0, "unroll covers both rings");
};
// DMA byte offsets from the tile's first row stay below 2^32.
constexpr int64_t kBigMaxK = int64_t(1) << 22;

template <int KH>
__global__ __launch_bounds__(256, 2) void k_gemm_big2(GemmArgs g, int mtiles)
{
    using C = BigCfg<KH>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kBigLds];
    constexpr int XR = 0;
    constexpr int CR = kBigP * kBigXBytes;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w >> 1, wn = w & 1;  // the wave's half (rows or K) and 128-column half
    const int i16 = lane & 15, grp = lane >> 4;

    // Block -> (m-tile, n-tile); consecutive indices on one XCD, m fastest,
    // so the m-tiles sharing a weight tile share that XCD's L2.
    int t = blockIdx.x;
    const int nb = gridDim.x;
    if ((nb & 7) == 0) t = (t & 7) * (nb >> 3) + (t >> 3);
    const int mt = t % mtiles;
    const int nt = t / mtiles;
    const int M = g.M, N = g.N, K = g.K;
    const int m0 = mt * C::BM, n0 = nt * kBigN;
    const int ns = K / kStageK;
    const int nit = ns / KH;  // iterations (K a multiple of 128 when KH = 2)

    // Activation DMAs: wave w, DMA q fills slot rows 8 (XI w + q) .. + 7,
    // in half h = (XI w + q) / 64 rows; lane l fills chunk slot l & 7 of slot
    // row r with chunk (l & 7) ^ xswz(r).  The half is row half h of the
    // stage (KH = 1) or rows 0..63 of the iteration's stage h (KH = 2).  Rows
    // >= M read row M - 1 (their outputs are not stored).
    const uint8_t *xbase = reinterpret_cast<const uint8_t *>(g.X + static_cast<int64_t>(m0) * K);
    uint32_t xoff[kBigXI];
#pragma unroll
    for (int q = 0; q < kBigXI; ++q) {
        const int r = 8 * (kBigXI * w + q) + (lane >> 3);
        const int h = r / kWaveM;
        const int c = (lane & 7) ^ xswz(r);
        const int rg = KH == 1 ? r : r - h * kWaveM;
        xoff[q] = static_cast<uint32_t>(static_cast<int64_t>(min(m0 + rg, M - 1) - m0) * K * 2 +
                                        (KH == 1 ? 0 : h * kStageK * 2) + 16 * c);
    }
    // Code DMAs: DMA d = NC w + i of a fetch covers block column tiles 2d and
    // 2d + 1 (16 columns each); lane l takes tile 2d + (l >> 5), the fetch's
    // stage (l >> 4) & 1, column l & 15: 16 bytes at 64 column + 16 piece of
    // the 1-KB export tile, landing at LDS [tile][stage][column][16 B].
    // Column tiles past the last one re-read it.
    const int last_tile = (N - 1) >> 4;
    const int cst = (lane >> 4) & 1;
    uint32_t ccol[kBigNC];
#pragma unroll
    for (int i = 0; i < kBigNC; ++i) {
        const int tb = 2 * (kBigNC * w + i) + (lane >> 5);
        ccol[i] = static_cast<uint32_t>(min((n0 >> 4) + tb, last_tile) * 1024 + (lane & 15) * 64);
    }
    const uint32_t lds_base = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t *)lds));

    auto issue_x = [&](int it, int slot) __attribute__((always_inline)) {
        const uint8_t *xs = xbase + min(KH * it, ns - KH) * (kStageK * 2);
#pragma unroll
        for (int q = 0; q < kBigXI; ++q)
            dma16(xs, xoff[q], lds_base + XR + slot * kBigXBytes + (kBigXI * w + q) * 1024);
    };
    // Code fetch F: stages 2F, 2F + 1 (clamped to the last stage, which is in
    // the same 64-byte group as 2F, or for a fetch wholly past the end the
    // last group) into buffer F & 1.
    auto issue_c = [&](int F) __attribute__((always_inline)) {
        const int st0 = min(2 * F, ns - 1);
        const int st = min(2 * F + cst, ns - 1);
        const uint8_t *cb = g.packed + static_cast<int64_t>(st0 >> 2) * g.gstride;
        const uint32_t po = static_cast<uint32_t>((st & 3) * 16);
#pragma unroll
        for (int i = 0; i < kBigNC; ++i)
            dma16<PQ_NT_BIG>(cb, ccol[i] + po, lds_base + CR + (F & 1) * kBigCBytes + (kBigNC * w + i) * 1024);
    };

    floatx4 acc[kRT][8];
#pragma unroll
    for (int i = 0; i < kRT; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // LDS read addresses.  Activation fragment of row tile i, k-step T: slot
    // row wm*64 + 16 i + i16 (the wave's half), chunk 2 grp + T (swizzled);
    // code word of the wave's column tile j at stage-in-fetch p: dword grp of
    // column i16.
    const int swz = xswz(i16);
    const uint8_t *xa0 = lds + XR + (wm * kWaveM + i16) * 128 + (((2 * grp) ^ swz) << 4);
    const uint8_t *xa1 = lds + XR + (wm * kWaveM + i16) * 128 + (((2 * grp + 1) ^ swz) << 4);
    const uint8_t *ca = lds + CR + (wn * 8) * 512 + i16 * 16 + grp * 4 + (KH == 2 ? wm * 256 : 0);

    auto read_a = [&](auto slot_c, auto t_c, uint4 (&a)[kRT]) __attribute__((always_inline)) {
        constexpr int SLOT = decltype(slot_c)::value;
        constexpr int T = decltype(t_c)::value;
        const uint8_t *base = (T == 0 ? xa0 : xa1) + SLOT * kBigXBytes;
#pragma unroll
        for (int i = 0; i < kRT; ++i) a[i] = *reinterpret_cast<const uint4 *>(base + i * 16 * 128);
    };
    auto read_c = [&](auto ph_c, uint32_t (&d)[8]) __attribute__((always_inline)) {
        constexpr int PH = decltype(ph_c)::value;  // iteration mod U
        constexpr int BUF = (PH / C::SS) & 1;
        constexpr int P = KH == 1 ? PH % 2 : 0;  // KH = 2: the wave's stage, in ca
#pragma unroll
        for (int j = 0; j < 8; ++j)
            d[j] = *reinterpret_cast<const uint32_t *>(ca + BUF * kBigCBytes + j * 512 + P * 256);
    };
    // Activation row sums for the level offset, on the matrix unit: of the
    // two waves sharing a row half, column half WN sums row tiles 2 WN and
    // 2 WN + 1 of every k-step with an all-ones A operand (4 MFMAs per stage
    // beside 64); accrs[ii] is row tile 2 WN + ii of the wave's rows.
    floatx4 accrs[2];
    accrs[0] = accrs[1] = floatx4{0.f, 0.f, 0.f, 0.f};
    const bf16x8 ones8 = __builtin_bit_cast(bf16x8, uint4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

    // MFMAs of one k-step: weights (16 columns) as the A operand, so each
    // lane ends with four consecutive columns of one row.
    auto mma = [&](auto t_c, const uint4 (&a)[kRT], const uint32_t (&d)[8], auto wn_c) __attribute__((always_inline)) {
        constexpr int T = decltype(t_c)::value;
        {
            constexpr int WN = decltype(wn_c)::value;
#pragma unroll
            for (int ii = 0; ii < 2; ++ii)
                accrs[ii] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, __builtin_bit_cast(bf16x8, a[2 * WN + ii]),
                                                                    accrs[ii], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            // the code word's masked nibbles: codes 0..7 (k-step 0) and
            // 8..15 (k-step 1) in k order (the export's word order)
            const uint32_t wt = T == 0 ? d[j] & 0x33333333u : (d[j] >> 2) & 0x33333333u;
            uint4 b;
            b.x = fp4x2_to_bf16x2<0>(wt);
            b.y = fp4x2_to_bf16x2<1>(wt);
            b.z = fp4x2_to_bf16x2<2>(wt);
            b.w = fp4x2_to_bf16x2<3>(wt);
            const bf16x8 bv = __builtin_bit_cast(bf16x8, b);
#pragma unroll
            for (int i = 0; i < kRT; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, __builtin_bit_cast(bf16x8, a[i]), acc[i][j],
                                                                     0, 0, 0);
        }
    };

    // The pipeline, instantiated once per column half (the row tiles a wave
    // sums are then a compile-time choice and its MFMA sequence stays
    // unbranched).
    auto pipeline = [&](auto wn_c) __attribute__((always_inline)) {
    // Prologue: code fetch 0, activation stages 0 .. P - 2, code fetch 1
    // (the issue order the wait model assumes); stage 0 and fetch 0 landed.
    // code fetches first when each iteration has its own (KH = 2; see the
    // step below), so that the wait model's order holds from the start
    constexpr int CF = C::SS == 1 ? 1 : 0;
    issue_c(0);
    if constexpr (CF) issue_c(1);
#pragma unroll
    for (int it = 0; it < kBigP - 1; ++it) issue_x(it, it);
    if constexpr (!CF) issue_c(1);
    // activation stage 0 and code fetch 0 landed: the DMAs issued after stage
    // 0 may stay in flight (stages 1 .. P-2, and code fetch 1 unless it went
    // first)
    wait_vmcnt<(kBigP - 2) * kBigXI + (CF ? 0 : kBigNC)>();
    block_barrier();
    uint4 a0[kRT], a1[kRT];
    uint32_t dc[2][8];
    read_a(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{}, a0);
    read_c(std::integral_constant<int, 0>{}, dc[0]);

    // Iteration s: wait for stage s + 1 (and its codes), barrier, refill the
    // slot of stage s - 1 and, every second stage, the code buffer of the
    // fetch before last; then the two k-steps of stage s, each reading the
    // next k-step's fragments first.  Every LDS read of a ring slot or code
    // buffer is complete before the barrier that precedes its refill.
    //
    // With one code fetch per iteration (KH = 2) the fetch an iteration
    // needs is issued one iteration ahead; issued after that iteration's
    // activation stage it would be the newest DMA, and every wait would be
    // for all of them (vmcnt 0).  Issued before it, one activation stage
    // stays in flight across each wait.
    auto step = [&](int s, auto pc) __attribute__((always_inline)) {
        constexpr int p = decltype(pc)::value;  // s mod U
        constexpr bool code_now = ((p + 1) % C::SS) == 0;
        wait_lgkmcnt0();
        wait_vmcnt<tile_wait(p, kBigP, C::SS, kBigXI, kBigNC, kBigU, 2, CF)>();
        block_barrier();
        __builtin_amdgcn_s_setprio(1);
        if constexpr (code_now && CF) issue_c((s + 1) / C::SS + 1);
        issue_x(s + kBigP - 1, (p + kBigP - 1) % kBigP);
        if constexpr (code_now && !CF) issue_c((s + 1) / C::SS + 1);
        // k-step 0 of stage s (a0), reading k-step 1 (a1)
        read_a(std::integral_constant<int, p % kBigP>{}, std::integral_constant<int, 1>{}, a1);
        __builtin_amdgcn_sched_barrier(0);
        mma(std::integral_constant<int, 0>{}, a0, dc[p & 1], wn_c);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
        // k-step 1 of stage s (a1), reading stage s + 1's k-step 0 and codes
        read_a(std::integral_constant<int, (p + 1) % kBigP>{}, std::integral_constant<int, 0>{}, a0);
        read_c(std::integral_constant<int, (p + 1) % kBigU>{}, dc[(p + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        mma(std::integral_constant<int, 1>{}, a1, dc[p & 1], wn_c);
        __builtin_amdgcn_sched_barrier(0);
    };
    int s = 0;
    for (; s + kBigU <= nit; s += kBigU) {
        static_for<0, kBigU>([&](auto pc) __attribute__((always_inline)) { step(s + decltype(pc)::value, pc); });
    }
    static_for<0, kBigU - 1>([&](auto pc) __attribute__((always_inline)) {
        if (s + decltype(pc)::value < nit) step(s + decltype(pc)::value, pc);
    });
    };
    if (wn == 0) pipeline(std::integral_constant<int, 0>{});
    else pipeline(std::integral_constant<int, 1>{});
    wait_vmcnt<0>();
    // The row sums to LDS, past the K-half buffer below (the ring is free
    // once every wave is here).
    float *rsl = reinterpret_cast<float *>(lds) + 2 * (kRT * 8 * 4 * 64);
    __syncthreads();
    if (grp == 0) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) rsl[w * kWaveM + 16 * (2 * wn + ii) + i16] = accrs[ii][0];
    }
    if constexpr (KH == 1) __syncthreads();
    if constexpr (KH == 2) {
        // Add the second K half's sums to the first's through LDS (the ring
        // is free: every DMA has landed and, after the barrier, every read).
        __syncthreads();
        float *red = reinterpret_cast<float *>(lds) + wn * (kRT * 8 * 4 * 64) + lane;
        if (wm == 1) {
#pragma unroll
            for (int i = 0; i < kRT; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) red[((i * 8 + j) * 4 + e) * 64] = acc[i][j][e];
        }
        __syncthreads();
        if (wm == 1) return;
#pragma unroll
        for (int i = 0; i < kRT; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][e] += red[((i * 8 + j) * 4 + e) * 64];
    }

    // Epilogue: acc[i][j][e] is row m0 + wm*kWaveM (KH = 1) + 16 i + i16, column
    // n0 + wn*128 + 16 j + 4 grp + e; four lanes hold a row's 128 columns in
    // 8-byte pieces.  Each wave writes its 64 x 128 outputs to 16 KB of LDS
    // and reads them back by rows, so that every store instruction writes 16
    // bytes per lane and four whole 256-byte row segments (16-byte chunks
    // XOR-swizzled by row for the LDS banks).  The staging area is the ring
    // below the row sums (KH = 1), or the wave's own K-half buffer, already
    // read (KH = 2).
    uint8_t *stg = lds + (KH == 1 ? w * 16384 : wn * (kRT * 8 * 4 * 64 * 4));
    float sr[kRT];
#pragma unroll
    for (int i = 0; i < kRT; ++i) {
        const int r = 16 * i + i16;
        // the row's sum: from the wave of its row half that owns row tile
        // i (KH = 1), or the two K halves' owners added (KH = 2)
        const float rsum = KH == 1 ? rsl[(2 * wm + (i >> 1)) * kWaveM + r]
                                   : rsl[(i >> 1) * kWaveM + r] + rsl[(2 + (i >> 1)) * kWaveM + r];
        sr[i] = g.off * rsum;
    }
    // the per-column scales of each column tile, its four loads issued
    // before any of them is used
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float al[1][4];
        load_col_scales<1>(g.alpha, g.alpha32, n0 + wn * 128 + 16 * j + 4 * grp, N, al);
#pragma unroll
        for (int i = 0; i < kRT; ++i) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = al[0][e] * (g.mul * (acc[i][j][e] - sr[i]));
            const int r = 16 * i + i16;
            const int ch = (2 * j + (grp >> 1)) ^ i16;
            *reinterpret_cast<u32x2 *>(stg + r * 256 + ch * 16 + (grp & 1) * 8) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
    }
    const int nw = n0 + wn * 128 + 8 * (lane & 15);   // this lane's 8 output columns
    const bool vec8 = (N & 7) == 0;
#pragma unroll
    for (int h = 0; h < 16; ++h) {
        const int r = (lane >> 4) + 4 * h;
        const uint4 d = *reinterpret_cast<const uint4 *>(stg + r * 256 + (((lane & 15) ^ (r & 15)) << 4));
        const int m = m0 + (KH == 1 ? wm * kWaveM : 0) + r;
        if (m < M && nw < N) {
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

// Which form takes a GEMM: 0 none, 1 or 2 the KH above.
int big_form(int bits, int64_t M, int64_t N, int64_t K)
{
    if (bits != 2 || K < PQ_BIG_MIN_K || K > kBigMaxK) return 0;
    const int64_t nt = (N + kBigN - 1) / kBigN;
    const int64_t t1 = (M + 2 * kWaveM - 1) / (2 * kWaveM) * nt;
    const int64_t t2 = (M + kWaveM - 1) / kWaveM * nt;
    if (M >= PQ_BIG_MIN_M && t1 >= PQ_BIG_MIN_TILES && t1 <= INT32_MAX) return 1;
    if (M >= PQ_BIG_KH2_MIN_M && K % (2 * kStageK) == 0 && t2 >= PQ_BIG_KH2_MIN_TILES && t2 <= INT32_MAX) return 2;
    return 0;
}

}  // namespace

bool gemm_big_takes(int bits, int64_t M, int64_t N, int64_t K) { return big_form(bits, M, N, K) != 0; }

pq_status launch_gemm_big(const GemmArgs &a, hipStream_t s)
{
    const int form = big_form(2, a.M, a.N, a.K);
    const int ntiles = (a.N + kBigN - 1) / kBigN;
    if (form == 1) {
        const int mtiles = (a.M + BigCfg<1>::BM - 1) / BigCfg<1>::BM;
        hipLaunchKernelGGL(k_gemm_big2<1>, dim3(static_cast<unsigned>(mtiles * ntiles)), dim3(256), 0, s, a, mtiles);
    } else if (form == 2) {
        const int mtiles = (a.M + BigCfg<2>::BM - 1) / BigCfg<2>::BM;
        hipLaunchKernelGGL(k_gemm_big2<2>, dim3(static_cast<unsigned>(mtiles * ntiles)), dim3(256), 0, s, a, mtiles);
    } else {
        return PQ_ERR_SHAPE;
    }
    return hipGetLastError() == hipSuccess ? PQ_OK : PQ_ERR_HIP;
}

}  // namespace pq
