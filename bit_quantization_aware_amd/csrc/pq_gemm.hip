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
//    registers: a 2-bit code c is placed in the mantissa of the bf16 2.0
//    (0x4000 | c << 5 = 2 + c/2), one shift and one and-or per two codes.
//    Since level = (c - 1.5)/2 = v - 2.75, the kernel accumulates X.v on
//    MFMA and subtracts 2.75 * rowsum(X) in the epilogue.  4-bit nibbles use
//    0x4000 | c << 3 = 2 + c/8, level = c - 8 = 8v - 24.
//  * A dword of codes holds 16 (2-bit) or 8 (4-bit) consecutive k; the decode
//    pairs codes (i, i+8) (resp. (i, i+4)) into one bf16x2.  The MFMA sums
//    over k in any order as long as A and B agree, so X is staged into LDS
//    in that same pair order (a fixed permutation inside each 16- or 8-wide
//    k block), and the A operand is a contiguous 16-byte LDS read.
//  * X tiles go global -> registers -> LDS (padded rows, no bank conflicts),
//    one stage ahead of the MFMA work; code tiles go global -> registers,
//    one stage ahead.  The X row sums are taken while staging.
//  * Tile shapes: small M streams the weight (16 x 64 block tile, deep K
//    stages); large M is MFMA-bound (128 x 128 block tile).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pq_common.hpp"

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

// Decode of one output bf16x2 from a dword of codes.
template <int BITS, int I>
__device__ __forceinline__ uint32_t decode_pair(uint32_t d)
{
    if constexpr (BITS == 2) {
        // codes I and I+8 -> mantissa bits 5-6 of each half
        constexpr int sh = 2 * I - 5;
        const uint32_t t = sh >= 0 ? (d >> sh) : (d << (-sh));
        return (t & 0x00600060u) | 0x40004000u;
    } else {
        // nibbles I and I+4 -> mantissa bits 3-6 of each half
        constexpr int sh = 4 * I - 3;
        const uint32_t t = sh >= 0 ? (d >> sh) : (d << (-sh));
        return (t & 0x00780078u) | 0x40004000u;
    }
}

// B operand (8 bf16) for MFMA k-step T of a stage from the lane's code dwords.
template <int BITS, int T>
__device__ __forceinline__ bf16x8 decode_b(const uint32_t *cw)
{
    uint4 r;
    if constexpr (BITS == 2) {
        const uint32_t d = cw[T >> 1];
        constexpr int h = (T & 1) * 4;
        r.x = decode_pair<2, h + 0>(d);
        r.y = decode_pair<2, h + 1>(d);
        r.z = decode_pair<2, h + 2>(d);
        r.w = decode_pair<2, h + 3>(d);
    } else {
        const uint32_t d = cw[T];
        r.x = decode_pair<4, 0>(d);
        r.y = decode_pair<4, 1>(d);
        r.z = decode_pair<4, 2>(d);
        r.w = decode_pair<4, 3>(d);
    }
    return __builtin_bit_cast(bf16x8, r);
}

template <int BITS, int TM, int TN, int WM, int WN, int BK>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g)
{
    static_assert(WM * WN == 4, "four waves per block");
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
                    // [0,8,1,9,...,7,15]: o[2j] = (x[2j'], x[8+2j']) pairs from d_j and e_j
                    const uint32_t d[4] = {xr[r][0].x, xr[r][0].y, xr[r][0].z, xr[r][0].w};
                    const uint32_t e[4] = {xr[r][1].x, xr[r][1].y, xr[r][1].z, xr[r][1].w};
                    uint32_t w[8];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        w[2 * j] = (d[j] & 0xFFFFu) | (e[j] << 16);
                        w[2 * j + 1] = (d[j] >> 16) | (e[j] & 0xFFFF0000u);
                        s += bf16_to_f32(d[j] & 0xFFFFu) + bf16_to_f32(d[j] >> 16);
                        s += bf16_to_f32(e[j] & 0xFFFFu) + bf16_to_f32(e[j] >> 16);
                    }
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
                    v = acc[i][j][e] - 2.75f * ssum[rl];
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
    if (M <= 16) launch<BITS, 1, 1, 1, 4, 256>(a, s);
    else if (M <= 64) launch<BITS, 2, 1, 2, 2, 256>(a, s);
    else launch<BITS, 4, 4, 2, 2, 128>(a, s);
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
