// pq_gemm_common.hpp -- internal pieces shared by the GEMM sources: the
// launch arguments, the LDS-DMA load and its ordering primitives, the
// activation swizzle and the DMA-pipeline wait model.  Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pq_common.hpp"

namespace pq {

struct GemmArgs {
    const uint16_t *X;       // [M, K] bf16
    const uint8_t *packed;   // export byte order: [groups][N / 16 tiles][1 KB]
    const uint16_t *alpha;   // [N] bf16
    uint16_t *Y;             // [M, N] bf16
    int M, N, K;
    int64_t gstride;         // bytes per 64-byte group of all rows (Np * 64)
    float off, mul;          // level = mul * (v - off) for the decoded operand v
    const float *alpha32;    // [N] binary32 scale, or nullptr (use alpha)
};

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Per-column scale: binary32 (the training forward's alpha) when given, else
// the exported bf16 scale.
__device__ __forceinline__ float col_scale(const uint16_t *a16, const float *a32, int n)
{
    return a32 ? a32[n] : bf16_to_f32(a16[n]);
}

// Per-column scales of a lane's output columns: out[j][e] for column
// n0 + 16 j + e (j < J, e < 4), 0 past N.  All loads are issued, from the
// binary32 or the bf16 array (a uniform choice), before any is used, so
// they cost one round trip instead of one each.
template <int J>
__device__ __forceinline__ void load_col_scales(const uint16_t *a16, const float *a32, int n0, int N,
                                                float (&out)[J][4])
{
    if (a32) {
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) out[j][e] = a32[min(n0 + 16 * j + e, N - 1)];
    } else {
#pragma unroll
        for (int j = 0; j < J; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) out[j][e] = bf16_to_f32(a16[min(n0 + 16 * j + e, N - 1)]);
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n0 + 16 * j + e >= N) out[j][e] = 0.f;
}

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


// K per pipeline stage of the tiled kernels.
constexpr int kStageK = 64;

constexpr int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }
constexpr int lcm_int(int a, int b) { return a / gcd_int(a, b) * b; }

// Activation LDS swizzle: chunk c of tile row r sits in slot c ^ xswz(r).
// Rows 0-7 (and 8-15) get distinct slots and rows r, r + 8 differ in the
// slot's low bit, so the 16 rows one A-operand read touches are spread over
// all banks whether the LDS serves 8 or 16 lanes of a 16-byte read per clock.
__device__ __forceinline__ int xswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// DMA bookkeeping of the tiled kernels' pipelines, evaluated at compile
// time, for a ring of P activation stages and NCB code fetches of SS stages.
// Issue order: code fetch 0, activation stages 0 .. P-2, code fetches
// 1 .. NCB-1 (with CF = 1: all code fetches first); then iteration j issues
// activation stage j + P - 1 and, when (j + 1) % SS == 0, code fetch
// (j + 1) / SS + NCB - 1 (after the activation stage, or before it when
// CF = 1).  Iteration s needs activation stage
// s + 1 and code fetch (s + 1) / SS landed; loads retire in order, so the
// largest safe vmcnt is the number of DMA instructions issued after the
// newer of the two.  Issue "times" only order the events.
constexpr int tile_t_x(int k, int P, int NCB, int CF = 0)
{
    return k <= P - 2 ? (CF ? NCB + k : 1 + k) : P + NCB - 1 + 2 * (k - P + 1) + CF;
}
constexpr int tile_t_c(int F, int P, int SS, int NCB, int CF = 0)
{
    return F == 0 ? 0 : F < NCB ? (CF ? F : P + F - 1) : P + NCB + 2 * ((F - NCB + 1) * SS - 1) - CF;
}
constexpr int tile_wait_at(int s, int P, int SS, int XI, int NC, int NCB, int CF = 0)
{
    const int a = tile_t_x(s + 1, P, NCB, CF), b = tile_t_c((s + 1) / SS, P, SS, NCB, CF);
    const int newest = a > b ? a : b;
    int n = 0;
    for (int st = 0; st < P - 1; ++st)
        if ((CF ? NCB + st : 1 + st) > newest) n += XI;
    for (int F = 1; F < NCB; ++F)
        if ((CF ? F : P + F - 1) > newest) n += NC;
    for (int j = 0; j < s; ++j) {
        if (P + NCB - 1 + 2 * j + CF > newest) n += XI;
        if ((j + 1) % SS == 0 && P + NCB + 2 * j - CF > newest) n += NC;
    }
    return n;
}
// The wait of unrolled phase p: the smallest safe count over the iterations
// s = p, p + U, ... (the first ones included; steady state is reached well
// within the range scanned).
constexpr int tile_wait(int p, int P, int SS, int XI, int NC, int U, int NCB = 2, int CF = 0)
{
    int best = 1 << 30;
    for (int s = p; s < 4 * U + 2 * P + 2 * NCB * SS; s += U) {
        const int w = tile_wait_at(s, P, SS, XI, NC, NCB, CF);
        best = w < best ? w : best;
    }
    return best;
}

// One LDS-DMA load: every lane fetches 16 bytes at `base + off` (`base`
// wave-uniform, in SGPRs) and the wave's 64 results land contiguously at LDS
// byte address `lds_addr` (via M0).  Issued from asm so that the compiler,
// which cannot tell the ring slots apart, does not wait for every DMA before
// each LDS read; the kernel orders the ring itself with s_waitcnt vmcnt and
// s_barrier.  The instruction writes no VGPRs.
//
// NT marks the load non-temporal: the weight codes, which a GEMM reads once,
// then take no room in the caches from data that is reused.  Above all they
// do not displace dirty lines that earlier kernels left in the memory-side
// last-level cache, which would have to be written back to HBM during the
// GEMM.  After a 1 GB copy, a 16384^2 GEMM with one activation row took
// 20.3 us with plain loads and 15.1 us with non-temporal ones (14.4-14.5 us
// in both cases back to back, with nothing dirty); with 16 rows 23.1 and
// 20.6 us.
// Non-temporal code loads, per GEMM kernel (1: on).  On in the streaming
// kernel only.  The other kernels measured slower with them, 3-8 % back to
// back, and no faster after a large write: 16384^2 at 512 rows 201 us
// against 187; 4096 x 4096 x 4096 100 against 95; 16384 rows of K = 576,
// N = 576 through the resident-code kernel 21.6 against 20.4.
#ifndef PQ_NT_STREAM
#define PQ_NT_STREAM 1
#endif
#ifndef PQ_NT_TILE
#define PQ_NT_TILE 0
#endif
#ifndef PQ_NT_BIG
#define PQ_NT_BIG 0
#endif
#ifndef PQ_NT_WRES
#define PQ_NT_WRES 0
#endif

template <bool NT = false>
__device__ __forceinline__ void dma16(const void *base, uint32_t off, uint32_t lds_addr)
{
    // M0 is saved and restored around the load, so the compiler's own use
    // of it (if any) is undisturbed; one wait state separates the M0 write
    // from the LDS-DMA that reads it.
    uint32_t saved;
    if constexpr (NT) {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %3\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %2 nt\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"(off), "s"(base), "s"(lds_addr)
            : "memory");
    } else {
        asm volatile(
            "s_mov_b32 %0, m0\n\t"
            "s_mov_b32 m0, %3\n\t"
            "s_nop 0\n\t"
            "global_load_lds_dwordx4 %1, %2\n\t"
            "s_mov_b32 m0, %0"
            : "=&s"(saved)
            : "v"(off), "s"(base), "s"(lds_addr)
            : "memory");
    }
}

__device__ __forceinline__ void block_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
// The empty asm with a memory clobber keeps the compiler from moving LDS
// reads of DMA-filled buffers above the wait (LDS loads cannot fault, so it
// would otherwise be free to hoist them).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    asm volatile("" ::: "memory");
}

// s_waitcnt lgkmcnt(0): every LDS access of the wave has completed.
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
    asm volatile("" ::: "memory");
}

template <int SEL>
__device__ __forceinline__ uint32_t fp4x2_to_bf16x2(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL));
}

}  // namespace

// pq_gemm with a given workspace (pq_gemm.hip), and the workspace bytes a
// shape needs (-1 for an unknown mode or a rejected shape).
pq_status gemm_run(int mode, int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
                   const void *alpha_bf16, void *Y, void *workspace, int64_t workspace_bytes, void *stream);
int64_t gemm_workspace_need(int mode, int64_t M, int64_t N, int64_t K);

// Large-M 2-bit path (pq_gemm_big.hip): whether it takes a GEMM of this
// shape, and its launch (no workspace).
bool gemm_big_takes(int bits, int64_t M, int64_t N, int64_t K);
pq_status launch_gemm_big(const GemmArgs &a, hipStream_t s);

// Short-K, many-row 2-bit path with resident codes (pq_gemm_wres.hip):
// whether it takes a GEMM of this shape, and its launch (no workspace).
bool gemm_wres_takes(int bits, int64_t M, int64_t N, int64_t K);
pq_status launch_gemm_wres(const GemmArgs &a, hipStream_t s);

}  // namespace pq
