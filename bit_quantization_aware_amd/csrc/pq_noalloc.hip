// pq_noalloc.hip -- pq_gemm_noalloc: the packed-weight GEMM for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid device allocation).  The GEMM kernels that need
// scratch -- split-K partial sums -- use a fixed array
// inside the library instead of a caller's workspace.
//
// The array lives in this file as a device variable.  Its host-side name is
// only a stand-in for the registered symbol, never a device address: the
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and kept per device, and only that address reaches the
// kernels.  Each GPU has its own copy of the array, which it holds until the
// process ends and which keeps the contents of the last call.  No part of
// the scratch needs to start at zero (every kernel that reads it reads only
// what the same call wrote first), so nothing is cleared.  Calls that
// overlap on one GPU -- on different streams, or from different threads --
// share the array and race on it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "pq_common.hpp"
#include "pq_gemm_common.hpp"

// Largest scratch a call may need: 32 MiB (the split-K partials of a
// 64 x 16384 output in eight splits); PQ_NOALLOC_SCRATCH_BYTES in pq.h.
static_assert(PQ_NOALLOC_SCRATCH_BYTES == (32 << 20), "header and library agree");

static __device__ __align__(256) uint8_t scratch[PQ_NOALLOC_SCRATCH_BYTES];

namespace pq {
namespace {

constexpr int64_t kScratchBytes = PQ_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];

// The current device's address of `scratch`, looked up on the first call
// made with that device current.  Two threads racing on the first call both
// store the same address.
pq_status scratch_address(void **out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return PQ_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return PQ_ERR_UNSUPPORTED;
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PQ_ERR_HIP;
        g_scratch_addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return PQ_OK;
}

}  // namespace
}  // namespace pq

extern "C" {

pq_status pq_gemm_noalloc(int mode, int64_t M, int64_t N, int64_t K, const void *X, const uint8_t *packed,
                          const void *alpha_bf16, void *Y, void *stream)
{
    const int64_t need = pq::gemm_workspace_need(mode, M, N, K);
    if (need < 0) {
        // the same status pq_gemm gives for these arguments
        return pq::gemm_run(mode, M, N, K, X, packed, alpha_bf16, Y, nullptr, 0, stream);
    }
    if (need > pq::kScratchBytes) return PQ_ERR_UNSUPPORTED;
    void *ws = nullptr;
    if (need > 0 && X && packed && alpha_bf16 && Y) {
        const pq_status st = pq::scratch_address(&ws);
        if (st != PQ_OK) return st;
    }
    return pq::gemm_run(mode, M, N, K, X, packed, alpha_bf16, Y, ws, need, stream);
}

}  // extern "C"
