// pq_stats.hip -- gfx950 kernels and C entry points for the layer's
// diagnostics: per-row level occupancy of the stored codes (counts and their
// entropy) and the per-row movement of the shadow weights from a reference.
//
// Sources (web pages, cited by title and section):
//   [Note]     "ParetoQ, the strongest low-bit QAT I could find" -- "Finding
//              3" (the level sets) and "QAT versus PTQ" (QAT compensates for
//              the quantizer instead of reconstructing the weights).
//   [Rebuttal] "ParetoQ: Improving Scaling Laws in Extremely Low-bit LLM
//              Quantization" -- why SEQ's balanced levels beat LSQ's at 2 bits
//              and below (how the weights spread over the levels).
//
// Both are row reductions over HBM-bound streams: one wave per row, four rows
// per 256-thread block, sums in a fixed-order wave butterfly (run-to-run
// identical results).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "pq_common.hpp"

namespace pq {
namespace {

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ double wave_sum_f64(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Codes equal to l among the 32 / CW fields of a word: XOR with l in every
// field makes the matching fields zero; OR-folding each field into its low
// bit and counting the low bits that stay clear counts them.
template <int CW>
__device__ __forceinline__ uint32_t count_equal(uint32_t d, uint32_t l, uint32_t valid_fields_mask)
{
    if constexpr (CW == 1) {
        const uint32_t ones = __builtin_popcount(d & valid_fields_mask);
        return l ? ones : __builtin_popcount(valid_fields_mask) - ones;
    } else {
        constexpr uint32_t kLow = CW == 2 ? 0x55555555u : 0x11111111u;
        uint32_t x = d ^ (l * kLow);
        x |= x >> 1;
        if constexpr (CW == 4) x |= x >> 2;
        return __builtin_popcount(~x & kLow & valid_fields_mask);
    }
}

// Level occupancy of one row of row-major codes (CW bits each, LSB first).
// Each lane takes 16-byte pieces lane, lane + 64, ... of the row (32-bit
// words, or bytes, when the rows are not 16- or 4-byte aligned) and counts
// each level with a few bit operations and a popcount per word.
template <int CW, int L>
__global__ __launch_bounds__(256) void k_level_stats(const uint8_t *codes, int64_t rows, int64_t cols,
                                                     uint32_t *counts, double *entropy)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const int64_t rb = cols * CW / 8;
    const uint8_t *cr = codes + row * rb;
    uint32_t c[L];
#pragma unroll
    for (int l = 0; l < L; ++l) c[l] = 0;
    if ((rb & 15) == 0 && (reinterpret_cast<uintptr_t>(codes) & 15) == 0) {
        // 16-byte loads, several in flight per lane
        const u32x4 *qr = reinterpret_cast<const u32x4 *>(cr);
#pragma unroll 4
        for (int64_t i = lane; i < rb / 16; i += 64) {
            const u32x4 d = __builtin_nontemporal_load(&qr[i]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int l = 0; l < L; ++l) c[l] += count_equal<CW>(d[e], static_cast<uint32_t>(l), 0xFFFFFFFFu);
        }
    } else if ((rb & 3) == 0 && (reinterpret_cast<uintptr_t>(codes) & 3) == 0) {
        const uint32_t *wr = reinterpret_cast<const uint32_t *>(cr);
        for (int64_t i = lane; i < rb / 4; i += 64) {
            const uint32_t d = __builtin_nontemporal_load(&wr[i]);
#pragma unroll
            for (int l = 0; l < L; ++l) c[l] += count_equal<CW>(d, static_cast<uint32_t>(l), 0xFFFFFFFFu);
        }
    } else {
        for (int64_t b = lane; b < rb; b += 64) {
            const uint32_t d = cr[b];
#pragma unroll
            for (int l = 0; l < L; ++l) c[l] += count_equal<CW>(d, static_cast<uint32_t>(l), 0xFFu);
        }
    }
#pragma unroll
    for (int l = 0; l < L; ++l) c[l] = wave_sum_u32(c[l]);
    if (lane == 0) {
        double h = 0.0;
#pragma unroll
        for (int l = 0; l < L; ++l) {
            counts[row * L + l] = c[l];
            if (c[l]) {
                const double p = static_cast<double>(c[l]) / static_cast<double>(cols);
                h -= p * log2(p);
            }
        }
        if (entropy) entropy[row] = h;
    }
}

// sum_j (W - W0)^2 and sum_j W0^2 per row, binary64.
__global__ __launch_bounds__(256) void k_weight_movement(const float *W, const float *W0, int64_t rows,
                                                         int64_t cols, double *sq_diff, double *sq_ref)
{
    const int lane = threadIdx.x & 63;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const PQ_GLOBAL f32x4 *w = (const PQ_GLOBAL f32x4 *)(W + row * cols);
    const PQ_GLOBAL f32x4 *w0 = (const PQ_GLOBAL f32x4 *)(W0 + row * cols);
    const int64_t nq = cols >> 2;
    double d2 = 0.0, r2 = 0.0;
    for (int64_t q = lane; q < nq; q += 64) {
        const f32x4 a = __builtin_nontemporal_load(&w[q]);
        const f32x4 b = __builtin_nontemporal_load(&w0[q]);
        const float av[4] = {a.x, a.y, a.z, a.w};
        const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double d = static_cast<double>(av[e]) - static_cast<double>(bv[e]);
            const double r = static_cast<double>(bv[e]);
            d2 += d * d;
            r2 += r * r;
        }
    }
    d2 = wave_sum_f64(d2);
    r2 = wave_sum_f64(r2);
    if (lane == 0) {
        sq_diff[row] = d2;
        sq_ref[row] = r2;
    }
}

int num_levels(int mode)
{
    switch (mode) {
    case PQ_W1_BINARY: return 2;
    case PQ_W158_SEQ_TERNARY: return 3;
    case PQ_W2_SEQ: return 4;
    case PQ_W3_LSQ: return 8;
    case PQ_W4_LSQ: return 16;
    case PQ_W2_LSQ: return 4;
    case PQ_W158_LSQ: return 3;
    default: return -1;
    }
}

}  // namespace
}  // namespace pq

extern "C" {

int pq_num_levels(int mode) { return pq::num_levels(mode); }

pq_status pq_level_stats(int mode, int64_t rows, int64_t cols, const uint8_t *codes, uint32_t *counts,
                         double *entropy, void *stream)
{
    using namespace pq;
    if (!valid_mode(mode)) return PQ_ERR_MODE;
    if (rows < 0 || !valid_cols(cols)) return PQ_ERR_SHAPE;
    if (rows == 0) return PQ_OK;
    if (!codes || !counts) return PQ_ERR_NULL;
    const int64_t blocks = (rows + 3) / 4;
    if (blocks > INT32_MAX) return PQ_ERR_SHAPE;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const dim3 g(static_cast<unsigned>(blocks)), b(256);
    switch (mode) {
    case PQ_W1_BINARY: hipLaunchKernelGGL((k_level_stats<1, 2>), g, b, 0, s, codes, rows, cols, counts, entropy); break;
    case PQ_W158_SEQ_TERNARY:
        hipLaunchKernelGGL((k_level_stats<2, 3>), g, b, 0, s, codes, rows, cols, counts, entropy);
        break;
    case PQ_W2_SEQ: hipLaunchKernelGGL((k_level_stats<2, 4>), g, b, 0, s, codes, rows, cols, counts, entropy); break;
    case PQ_W3_LSQ: hipLaunchKernelGGL((k_level_stats<4, 8>), g, b, 0, s, codes, rows, cols, counts, entropy); break;
    case PQ_W2_LSQ: hipLaunchKernelGGL((k_level_stats<2, 4>), g, b, 0, s, codes, rows, cols, counts, entropy); break;
    case PQ_W158_LSQ: hipLaunchKernelGGL((k_level_stats<2, 3>), g, b, 0, s, codes, rows, cols, counts, entropy); break;
    default: hipLaunchKernelGGL((k_level_stats<4, 16>), g, b, 0, s, codes, rows, cols, counts, entropy); break;
    }
    return hipGetLastError() == hipSuccess ? PQ_OK : PQ_ERR_HIP;
}

pq_status pq_weight_movement(int64_t rows, int64_t cols, const float *W, const float *W0, double *sq_diff,
                             double *sq_ref, void *stream)
{
    using namespace pq;
    if (rows < 0 || !valid_cols(cols)) return PQ_ERR_SHAPE;
    if (rows == 0) return PQ_OK;
    if (!W || !W0 || !sq_diff || !sq_ref) return PQ_ERR_NULL;
    if (!aligned16(W) || !aligned16(W0)) return PQ_ERR_ALIGN;
    const int64_t blocks = (rows + 3) / 4;
    if (blocks > INT32_MAX) return PQ_ERR_SHAPE;
    hipLaunchKernelGGL(k_weight_movement, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), W, W0, rows, cols, sq_diff, sq_ref);
    return hipGetLastError() == hipSuccess ? PQ_OK : PQ_ERR_HIP;
}

}  // extern "C"
