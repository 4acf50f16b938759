// pq_gemm_wres.hip -- the W2A16 GEMM for short K and many rows (gfx950):
// 2-bit codes in the export byte order x bf16 activations, with the block's
// weight codes resident in LDS and its activations streamed across all of
// its row tiles.
//
// Sources (web pages, cited by title and section):
//   [News] "ParetoQ ... 2-bit kernel" news item -- speed paragraph: the 2-bit
//          weights are used packed by the deployed kernel.
//   [Note] "ParetoQ, the strongest low-bit QAT I could find" -- "Finding 3"
//          (the level sets) and "Paper vs. code" (no bias in the layer).
//
// The QAT forward of a small model multiplies many tokens by short-K
// weights (MobileLLM-125M: K = 576 for six of its seven projections, at
// 16384 tokens).  The tiled kernel of pq_gemm.hip gives such a GEMM 64 x 256
// output tiles of only 9 K stages each, every one with its own pipeline
// fill, and writes each tile's outputs in 8-byte pieces.  Here a block owns
// one 256-column tile and a run of consecutive 64-row tiles:
//   - its codes for the whole K (16 bytes per column per stage, 4 KB per
//     stage, at most kWresMaxStages stages) are fetched once into LDS and
//     stay there;
//   - its activation stages, row tile after row tile, form one stream
//     through a ring of four 8-KB slots kept three stages ahead by the
//     LDS-DMA load, so the next row tile's first stages land while the
//     current one finishes, and the wait before each stage is one constant;
//   - when a row tile's last stage is done the waves combine its row sums
//     and write its outputs through LDS as whole 128-byte row segments,
//     inside the stream;
//   - the blocks of one run of row tiles (one per column tile) are
//     neighbours on one XCD, so each activation row is read from HBM about
//     once and from that XCD's L2 by the others.
// The fragment layout, decode, row sums on the matrix unit, LDS swizzle and
// output arithmetic are those of the tiled kernel, so both give the same
// sums in the same order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "pq_common.hpp"
#include "pq_gemm_common.hpp"

// Largest K, in 64-k stages, whose codes stay resident (4 KB per stage):
// with the 32-KB ring and the row sums, 11 keep two blocks on a CU.
#ifndef PQ_WRES_MAX_STAGES
#define PQ_WRES_MAX_STAGES 11
#endif
// 1: 192-column blocks (four waves of 48 columns) where they pad N less.
#ifndef PQ_WRES_NARROW
#define PQ_WRES_NARROW 1
#endif
// Fewest rows for which this kernel takes a 2-bit GEMM.
#ifndef PQ_WRES_MIN_M
#define PQ_WRES_MIN_M 1024
#endif

namespace pq {
namespace {

constexpr int kWresTM = 64;                          // rows per tile
constexpr int kWresN = 256;                          // block columns: 4 waves x 64 (or x 48)
constexpr int kWresP = 4;                            // activation ring slots
constexpr int kWresXBytes = kWresTM * kStageK * 2;   // 8 KB per slot
constexpr int kWresXI = kWresXBytes / (4 * 1024);    // activation DMAs per wave per stage
constexpr int kWresCStage = kWresN * 16;             // codes of one stage, 16 B per column
constexpr int kWresMaxStages = PQ_WRES_MAX_STAGES;
constexpr int kWresLds = kWresP * kWresXBytes + kWresMaxStages * kWresCStage;
constexpr int kWresBlocks = 512;                     // two per CU
static_assert(kWresXI * 4 * 1024 == kWresXBytes, "one slot is XI 1-KB DMAs per wave");
static_assert(kWresLds + kWresTM * 4 <= 80 * 1024, "two blocks per CU");

// JW: 16-column MFMA tiles per wave, 4 (256-column blocks) or 3 (192).
template <int JW>
__global__ __launch_bounds__(256, 2) void k_gemm_wres(GemmArgs g, int mtiles, int ntiles)
{
    static_assert(JW == 3 || JW == 4, "48 or 64 columns per wave");
    constexpr int P = kWresP, XI = kWresXI;
    constexpr int WC = 16 * JW, TN = 4 * WC;   // columns per wave, per block
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kWresLds];
    __shared__ float ssum[kWresTM];
    constexpr int XR = 0;                   // activation ring
    constexpr int CR = P * kWresXBytes;     // resident codes, [stage][wave][64 columns][16 B]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i16 = lane & 15, grp = lane >> 4;
    const int M = g.M, N = g.N, K = g.K;
    const int ns = K / kStageK;

    // The block's work: column tile nt, row tiles [mt0, mt0 + nseg).  The
    // grid holds ntiles blocks per run of row tiles, column tile fastest, and
    // consecutive block indices go to one XCD (the XCDs take workgroups
    // round robin), so the blocks reading the same rows share its L2 copy.
    const int nb = gridDim.x;
    int b = blockIdx.x;
    if ((nb & 7) == 0) b = (b & 7) * (nb >> 3) + (b >> 3);
    const int runs = nb / ntiles;
    const int nt = b % ntiles, run = b / ntiles;
    const int mt0 = static_cast<int>(static_cast<int64_t>(run) * mtiles / runs);
    const int nseg = static_cast<int>(static_cast<int64_t>(run + 1) * mtiles / runs) - mt0;

    const uint32_t lds_base = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) uint8_t *)lds));

    // Activation DMA q of wave w fills slot rows 8 (XI w + q) .. + 7; lane l
    // fills chunk slot l & 7 of row r with chunk (l & 7) ^ xswz(r).  Rows
    // >= M read row M - 1 (their outputs are not stored).
    int xr[XI];
    uint32_t xfull[XI];
#pragma unroll
    for (int q = 0; q < XI; ++q) {
        xr[q] = 8 * (XI * w + q) + (lane >> 3);
        xfull[q] = static_cast<uint32_t>(xr[q] * K * 2 + 16 * ((lane & 7) ^ xswz(xr[q])));
    }

    // LDS read addresses.  a[i] is row tile (i + w) & 3, so a[0] is the tile
    // whose row sums this wave keeps; the code word of the wave's column
    // 16 j + i16 at stage st is dword grp of its 16 bytes (1 KB per wave and
    // stage, the last 16 columns unused when JW = 3).
    const int swz = xswz(i16);
    const uint8_t *xa[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int T = 0; T < 2; ++T)
            xa[i][T] = lds + XR + (16 * ((i + w) & 3) + i16) * 128 + (((2 * grp + T) ^ swz) << 4);
    const uint8_t *ca = lds + CR + w * 1024 + i16 * 16 + 4 * grp;

    struct Frag {
        uint4 a[2][4];
        uint32_t d[JW];
    };
    auto read_frags = [&](auto slot_c, int kst, Frag &f) __attribute__((always_inline)) {
        constexpr int SLOT = decltype(slot_c)::value;
        const uint8_t *cp = ca + kst * kWresCStage;
#pragma unroll
        for (int j = 0; j < JW; ++j) f.d[j] = *reinterpret_cast<const uint32_t *>(cp + j * 256);
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                f.a[T][i] = *reinterpret_cast<const uint4 *>(xa[i][T] + SLOT * kWresXBytes);
    };

    floatx4 acc[4][JW];
    floatx4 accrs;
    const bf16x8 ones8 = __builtin_bit_cast(bf16x8, uint4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    auto clear_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < JW; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
        accrs = floatx4{0.f, 0.f, 0.f, 0.f};
    };
    // One stage: the code word's masked nibbles are its codes 0..7 (k-step 0)
    // and 8..15 (k-step 1) in k order (the export's word order); the weights
    // are the MFMA A operand, so a lane's outputs are four consecutive
    // columns of one row.
    auto mma = [&](const Frag &f, auto &&between) __attribute__((always_inline)) {
        uint32_t w0[JW], w1[JW];
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            w0[j] = f.d[j] & 0x33333333u;
            w1[j] = (f.d[j] >> 2) & 0x33333333u;
        }
        static_for<0, 2>([&](auto tc) {
            constexpr int T = decltype(tc)::value;
#pragma unroll
            for (int j = 0; j < JW; ++j) {
                const uint32_t wt = T == 0 ? w0[j] : w1[j];
                uint4 bw;
                bw.x = fp4x2_to_bf16x2<0>(wt);
                bw.y = fp4x2_to_bf16x2<1>(wt);
                bw.z = fp4x2_to_bf16x2<2>(wt);
                bw.w = fp4x2_to_bf16x2<3>(wt);
                const bf16x8 bv = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv, __builtin_bit_cast(bf16x8, f.a[T][i]),
                                                                         acc[i][j], 0, 0, 0);
            }
            // rows 16 w + i16 of the tile, summed over the k-step
            accrs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, __builtin_bit_cast(bf16x8, f.a[T][0]), accrs, 0, 0, 0);
            if constexpr (T == 0) {
                __builtin_amdgcn_sched_barrier(0);
                between();
                __builtin_amdgcn_sched_barrier(0);
            }
        });
    };

    {
        const int T = nseg * ns;
        const int n0 = nt * TN;

        // Per-column scales of the tile, the same for all its row tiles:
        // loaded before any DMA and waited for here, so that no wait for
        // them (which would also wait for every DMA in flight) lands in the
        // stream.  Columns >= N read column N - 1 and get 0.
        float al[JW][4];
        load_col_scales<JW>(g.alpha, g.alpha32, n0 + WC * w + 4 * grp, N, al);
        wait_vmcnt<0>();

        // Resident codes: per stage one DMA per wave, lane l fetching the
        // stage's 16 bytes of the wave's column l (piece st & 3 of group
        // st >> 2 of its export tile).  Columns >= N re-read column N - 1;
        // with JW = 3 lanes 48..63 fetch unused pieces.
        {
            const int cl = min(n0 + WC * w + lane, N - 1);
            const uint32_t coff = static_cast<uint32_t>((cl >> 4) * 1024 + (cl & 15) * 64);
            for (int st = 0; st < ns; ++st)
                dma16<PQ_NT_WRES>(g.packed + static_cast<int64_t>(st >> 2) * g.gstride, coff + (st & 3) * 16,
                      lds_base + CR + st * kWresCStage + w * 1024);
        }

        // Issue cursor of the activation stream: row tile im of the stream,
        // stage ik; past the stream's end the last stage is issued again (in
        // bounds, never read), so that every step issues the same DMAs.
        int im = 0, ik = 0, issued = 0;
        uint32_t xo[XI];
        auto set_rows = [&]() __attribute__((always_inline)) {
            const int m0 = (mt0 + im) * kWresTM;
            if (m0 + kWresTM <= M) {
#pragma unroll
                for (int q = 0; q < XI; ++q) xo[q] = xfull[q];
            } else {
#pragma unroll
                for (int q = 0; q < XI; ++q)
                    xo[q] = static_cast<uint32_t>((min(m0 + xr[q], M - 1) - m0) * K * 2 +
                                                  16 * ((lane & 7) ^ xswz(xr[q])));
            }
        };
        set_rows();
        auto issue_x = [&](int slot) __attribute__((always_inline)) {
            const int m0 = (mt0 + im) * kWresTM;
            const uint8_t *xs = reinterpret_cast<const uint8_t *>(g.X + static_cast<int64_t>(m0) * K + ik * kStageK);
#pragma unroll
            for (int q = 0; q < XI; ++q)
                dma16(xs, xo[q], lds_base + XR + slot * kWresXBytes + (XI * w + q) * 1024);
            if (issued + 1 < T) {
                ++issued;
                if (++ik == ns) {
                    ik = 0;
                    ++im;
                    set_rows();
                }
            }
        };
#pragma unroll
        for (int st = 0; st < P - 1; ++st) issue_x(st);

        clear_acc();
        // the codes and activation stage 0 landed
        wait_vmcnt<(P - 2) * XI>();
        block_barrier();
        Frag fr[2];
        read_frags(std::integral_constant<int, 0>{}, 0, fr[0]);

        // Compute cursor: row tile mc, stage kc of the stage being multiplied.
        int mc = 0, kc = 0;
        // Row tile mc is complete: publish its row sums, write its outputs,
        // clear the accumulators.  acc[i][j][e] is row 16 ((i + w) & 3) + i16
        // of the tile, the wave's column 16 j + 4 grp + e: four lanes hold a
        // row's WC columns in 8-byte pieces.  Each wave passes its rows
        // through 2 KB of the slot of the stage just multiplied (free until
        // the next step refills it), 16 rows at a time, so that every store
        // instruction writes 16 bytes per lane and eight whole 128-byte row
        // segments; the 16-byte chunks are XOR-swizzled by row so that both
        // the writes and the reads spread over the LDS banks.
        auto finish_tile = [&](auto slot_c) __attribute__((always_inline)) {
            constexpr int SLOT = decltype(slot_c)::value;
            if (grp == 0) ssum[16 * w + i16] = accrs[0];
            __syncthreads();
            const int m0 = (mt0 + mc) * kWresTM;
            uint8_t *stg = lds + XR + SLOT * kWresXBytes + w * 2048;
            const int nw = n0 + WC * w + 8 * (lane & 7);   // this lane's 8 output columns
            const bool lane_cols = (lane & 7) < 2 * JW;
            const bool vec = (N & 7) == 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rt = (i + w) & 3;
                const float sr = g.off * ssum[16 * rt + i16];
#pragma unroll
                for (int j = 0; j < JW; ++j) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = al[j][e] * (g.mul * (acc[i][j][e] - sr));
                    const int ch = (2 * j + (grp >> 1)) ^ (i16 & 7);
                    *reinterpret_cast<u32x2 *>(stg + i16 * 128 + ch * 16 + (grp & 1) * 8) =
                        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
                }
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = (lane >> 3) + 8 * h;
                    const uint4 d = *reinterpret_cast<const uint4 *>(stg + r * 128 + (((lane & 7) ^ (r & 7)) << 4));
                    const int m = m0 + 16 * rt + r;
                    if (lane_cols && m < M && nw < N) {
                        uint16_t *y = g.Y + static_cast<int64_t>(m) * N + nw;
                        if (vec) {
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
            clear_acc();
        };
        // Step t (phase p = t mod 4): wait for stage t + 1, refill the slot
        // of stage t - 1 with stage t + P - 1, read stage t + 1's fragments,
        // multiply stage t.  ssum is rewritten only a stage barrier after
        // every wave has read it.
        auto step = [&](auto pc) __attribute__((always_inline)) {
            constexpr int p = decltype(pc)::value;
            const int kn = kc + 1 == ns ? 0 : kc + 1;
            wait_lgkmcnt0();
            wait_vmcnt<(P - 3) * XI>();
            block_barrier();
            __builtin_amdgcn_s_setprio(1);
            read_frags(std::integral_constant<int, (p + 1) % P>{}, kn, fr[(p + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            mma(fr[p & 1], [&]() {
                issue_x((p + P - 1) % P);
                __builtin_amdgcn_s_setprio(0);
            });
            __builtin_amdgcn_sched_barrier(0);
            if (kc + 1 == ns) {
                finish_tile(std::integral_constant<int, p>{});
                ++mc;
            }
            kc = kn;
        };
        static_assert(P == 4, "the unrolled loop covers the ring's phases and the fragment double buffer");
        int t = 0;
        for (; t + 4 <= T; t += 4) {
            step(std::integral_constant<int, 0>{});
            step(std::integral_constant<int, 1>{});
            step(std::integral_constant<int, 2>{});
            step(std::integral_constant<int, 3>{});
        }
        if (t < T) step(std::integral_constant<int, 0>{});
        if (t + 1 < T) step(std::integral_constant<int, 1>{});
        if (t + 2 < T) step(std::integral_constant<int, 2>{});
    }
}

}  // namespace

bool gemm_wres_takes(int bits, int64_t M, int64_t N, int64_t K)
{
    if (bits != 2 || M < PQ_WRES_MIN_M || K > static_cast<int64_t>(kWresMaxStages) * kStageK) return false;
    const int64_t items = (M + kWresTM - 1) / kWresTM * ((N + 191) / 192);
    return items <= INT32_MAX;
}

pq_status launch_gemm_wres(const GemmArgs &a, hipStream_t s)
{
    if (!gemm_wres_takes(2, a.M, a.N, a.K)) return PQ_ERR_SHAPE;
    const int mtiles = (a.M + kWresTM - 1) / kWresTM;
    // 192-column blocks where they pad N less than 256-column ones (N = 576:
    // three tiles either way, no idle columns)
    const bool narrow = PQ_WRES_NARROW && (a.N + 191) / 192 * 192 < (a.N + kWresN - 1) / kWresN * kWresN;
    const int tn = narrow ? 192 : kWresN;
    const int ntiles = (a.N + tn - 1) / tn;
    // Runs per column tile: as many as two blocks per CU allow, then as few
    // as give the same longest run (the runs differ by at most a row tile).
    const int64_t rmax = std::max<int64_t>(1, std::min<int64_t>(mtiles, kWresBlocks / ntiles));
    const int64_t runlen = (mtiles + rmax - 1) / rmax;
    const int64_t blocks = ntiles * ((mtiles + runlen - 1) / runlen);
    if (blocks > INT32_MAX) return PQ_ERR_SHAPE;
    if (narrow)
        hipLaunchKernelGGL(k_gemm_wres<3>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a, mtiles, ntiles);
    else
        hipLaunchKernelGGL(k_gemm_wres<4>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a, mtiles, ntiles);
    return hipGetLastError() == hipSuccess ? PQ_OK : PQ_ERR_HIP;
}

}  // namespace pq
