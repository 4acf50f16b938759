// pq_common.hpp -- internal helpers shared by the libpq HIP sources
// (argument checks, bf16 packing, launch tables).  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pq.h"

namespace pq {

// Global-memory (address space 1) pointers: descriptors are loaded from
// memory, so without this the compiler could only emit flat accesses.
#define PQ_GLOBAL __attribute__((address_space(1)))
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline bool valid_mode(int mode) { return mode >= PQ_W1_BINARY && mode <= PQ_W158_LSQ; }

inline int code_bits(int mode)
{
    switch (mode) {
    case PQ_W1_BINARY: return 1;
    case PQ_W158_SEQ_TERNARY: return 2;
    case PQ_W2_SEQ: return 2;
    case PQ_W3_LSQ: return 4;
    case PQ_W4_LSQ: return 4;
    case PQ_W2_LSQ: return 2;
    case PQ_W158_LSQ: return 2;
    default: return -1;
    }
}

// Largest accepted cols / K: keeps every per-row quad index in 32 bits.
constexpr int64_t kMaxCols = int64_t(1) << 30;

inline bool valid_cols(int64_t cols) { return cols > 0 && cols % 8 == 0 && cols <= kMaxCols; }

// Two fp32 -> packed bf16x2, round to nearest-even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16)
{
    return __builtin_bit_cast(float, bits16 << 16);
}

// Launch table for the quantizer kernels: one launch covers `count` matrices;
// launch entry k is descriptor idx[k] of the table and owns blocks
// [block_start[k], block_start[k+1]).  It travels in the kernel-argument
// segment, so the per-block lookup is a few scalar-cache hits.
constexpr int kMaxGroup = 448;

template <typename D>
struct LaunchTableT {
    const D *table;  // device descriptors, or nullptr -> use `single`
    D single;
    int count;
    int32_t block_start[kMaxGroup + 1];
    int16_t idx[kMaxGroup];
    int nt_out;      // forward: write the outputs with nontemporal stores
};
using LaunchTable = LaunchTableT<pq_mat>;
using StepTable = LaunchTableT<pq_step_mat>;

template <typename D>
__device__ __forceinline__ int find_matrix(const LaunchTableT<D> &lt, int b)
{
    int lo = 0, hi = lt.count - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (lt.block_start[mid] <= b) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

}  // namespace pq
