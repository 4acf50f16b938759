// pq_quant_mode.hip -- the quantizer's kernel launchers for one mode,
// PQ_QUANT_MODE (a pq_mode value given on the compiler command line): the
// build compiles this file once per mode, so the seven modes' kernels are
// instantiated in separate translation units that compile in parallel.

#include "pq_quant_kernels.hpp"

#ifndef PQ_QUANT_MODE
#error "compile with -DPQ_QUANT_MODE=<pq_mode value>"
#endif

namespace pq {
namespace {

template <int MODE, int IQ, unsigned OUTS, int U>
void launch_fwd_t(const LaunchTable &lt, int blocks, int wpr, hipStream_t s, StatsOut so = {})
{
    if (wpr == 1)
        hipLaunchKernelGGL((k_quant_fwd<MODE, IQ, 1, OUTS, U>), dim3(blocks), dim3(256), 0, s, lt, so);
    else
        hipLaunchKernelGGL((k_quant_fwd<MODE, IQ, 4, OUTS, U>), dim3(blocks), dim3(256), 0, s, lt, so);
}

template <int MODE, int INIT, int U>
void launch_fwd_outs(unsigned outs, const LaunchTable &lt, int blocks, int wpr, hipStream_t s)
{
    switch (outs) {
    case 0: launch_fwd_t<MODE, INIT, 0, U>(lt, blocks, wpr, s); break;
    case 1: launch_fwd_t<MODE, INIT, 1, U>(lt, blocks, wpr, s); break;
    case 2: launch_fwd_t<MODE, INIT, 2, U>(lt, blocks, wpr, s); break;
    case 3: launch_fwd_t<MODE, INIT, 3, U>(lt, blocks, wpr, s); break;
    case 4: launch_fwd_t<MODE, INIT, 4, U>(lt, blocks, wpr, s); break;
    case 5: launch_fwd_t<MODE, INIT, 5, U>(lt, blocks, wpr, s); break;
    case 6: launch_fwd_t<MODE, INIT, 6, U>(lt, blocks, wpr, s); break;
    case 7: launch_fwd_t<MODE, INIT, 7, U>(lt, blocks, wpr, s); break;
    // codes in the export byte order
    case OUT_CODES | OUT_TILED: launch_fwd_t<MODE, INIT, 20, U>(lt, blocks, wpr, s); break;
    case OUT_BF16 | OUT_CODES | OUT_TILED: launch_fwd_t<MODE, INIT, 21, U>(lt, blocks, wpr, s); break;
    case OUT_F32 | OUT_CODES | OUT_TILED: launch_fwd_t<MODE, INIT, 22, U>(lt, blocks, wpr, s); break;
    default: launch_fwd_t<MODE, INIT, 23, U>(lt, blocks, wpr, s); break;
    }
}

template <int MODE, int WPR, bool GBF16, int U>
void launch_bwd_t(bool wdw, bool wmask, const LaunchTable &lt, int blocks, hipStream_t s)
{
    if (wdw && wmask)
        hipLaunchKernelGGL((k_quant_bwd<MODE, WPR, GBF16, true, true, U>), dim3(blocks), dim3(256), 0, s, lt);
    else if (wdw)
        hipLaunchKernelGGL((k_quant_bwd<MODE, WPR, GBF16, true, false, U>), dim3(blocks), dim3(256), 0, s, lt);
    else if (wmask)
        hipLaunchKernelGGL((k_quant_bwd<MODE, WPR, GBF16, false, true, U>), dim3(blocks), dim3(256), 0, s, lt);
    else
        hipLaunchKernelGGL((k_quant_bwd<MODE, WPR, GBF16, false, false, U>), dim3(blocks), dim3(256), 0, s, lt);
}

template <int MODE, int U>
void launch_bwd_u(int wpr, bool gbf, bool wdw, bool wmask, const LaunchTable &lt, int blocks, hipStream_t s)
{
    if (wpr == 1) {
        if (gbf) launch_bwd_t<MODE, 1, true, U>(wdw, wmask, lt, blocks, s);
        else launch_bwd_t<MODE, 1, false, U>(wdw, wmask, lt, blocks, s);
    } else {
        if (gbf) launch_bwd_t<MODE, 4, true, U>(wdw, wmask, lt, blocks, s);
        else launch_bwd_t<MODE, 4, false, U>(wdw, wmask, lt, blocks, s);
    }
}

}  // namespace

template <int MODE>
void launch_fwd_m(int init, unsigned outs, int u, const LaunchTable &lt, int blocks, int wpr, hipStream_t s)
{
    // the scale init reads whole rows into registers; its fallback passes
    // for longer rows keep the narrow width
    if (init == kInitLarge) launch_fwd_outs<MODE, kInitLarge, kPassNarrow>(outs, lt, blocks, wpr, s);
    else if (init > 0) launch_fwd_outs<MODE, kInitSmall, kPassNarrow>(outs, lt, blocks, wpr, s);
    else if (u > kPassNarrow) launch_fwd_outs<MODE, 0, kPassWide>(outs, lt, blocks, wpr, s);
    else launch_fwd_outs<MODE, 0, kPassNarrow>(outs, lt, blocks, wpr, s);
}

template <int MODE>
void launch_fwd_stats_m(bool bf16, const LaunchTable &lt, int blocks, int wpr, hipStream_t s, StatsOut so)
{
    if (bf16) launch_fwd_t<MODE, 0, OUT_STATS | OUT_CODES | OUT_BF16, kPassNarrow>(lt, blocks, wpr, s, so);
    else launch_fwd_t<MODE, 0, OUT_STATS | OUT_CODES, kPassNarrow>(lt, blocks, wpr, s, so);
}

template <int MODE>
void launch_pack_m(int u, const LaunchTable &lt, int blocks, int wpr, hipStream_t s)
{
    constexpr unsigned O = OUT_CODES | OUT_TILED | OUT_ALPHA_BF16;
    if (u > kPassNarrow) launch_fwd_t<MODE, 0, O, kPassWide>(lt, blocks, wpr, s);
    else launch_fwd_t<MODE, 0, O, kPassNarrow>(lt, blocks, wpr, s);
}

template <int MODE>
void launch_bwd_m(int u, int wpr, bool gbf, bool wdw, bool wmask, const LaunchTable &lt, int blocks, hipStream_t s)
{
    if (u > kPassNarrow) launch_bwd_u<MODE, kPassWide>(wpr, gbf, wdw, wmask, lt, blocks, s);
    else launch_bwd_u<MODE, kPassNarrow>(wpr, gbf, wdw, wmask, lt, blocks, s);
}

template <int MODE>
void launch_step_m(int wpr, bool gbf, const StepTable &lt, int blocks, const AdamK &k, hipStream_t s)
{
    if (wpr == 1) {
        if (gbf) hipLaunchKernelGGL((k_qat_step<MODE, 1, true>), dim3(blocks), dim3(256), 0, s, lt, k);
        else hipLaunchKernelGGL((k_qat_step<MODE, 1, false>), dim3(blocks), dim3(256), 0, s, lt, k);
    } else {
        if (gbf) hipLaunchKernelGGL((k_qat_step<MODE, 4, true>), dim3(blocks), dim3(256), 0, s, lt, k);
        else hipLaunchKernelGGL((k_qat_step<MODE, 4, false>), dim3(blocks), dim3(256), 0, s, lt, k);
    }
}

template void launch_fwd_m<PQ_QUANT_MODE>(int, unsigned, int, const LaunchTable &, int, int, hipStream_t);
template void launch_fwd_stats_m<PQ_QUANT_MODE>(bool, const LaunchTable &, int, int, hipStream_t, StatsOut);
template void launch_pack_m<PQ_QUANT_MODE>(int, const LaunchTable &, int, int, hipStream_t);
template void launch_bwd_m<PQ_QUANT_MODE>(int, int, bool, bool, bool, const LaunchTable &, int, hipStream_t);
template void launch_step_m<PQ_QUANT_MODE>(int, bool, const StepTable &, int, const AdamK &, hipStream_t);

}  // namespace pq
