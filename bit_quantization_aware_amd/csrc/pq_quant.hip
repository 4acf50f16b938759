// pq_quant.hip -- host side and C entry points of the per-row weight
// quantizer: alpha init, forward fake-quantization, straight-through backward
// with the scale gradient, export packing and the fused QAT step.  The
// kernels and their arithmetic are in pq_quant_kernels.hpp; their launchers
// are instantiated per mode in pq_quant_mode.hip.
//
// Sources (web pages, cited by title and section):
//   [Note]     "ParetoQ, the strongest low-bit QAT I could find"
//   [Rebuttal] "ParetoQ: Improving Scaling Laws in Extremely Low-bit LLM
//              Quantization" (authors' OpenReview replies)
//   [News]     "Meta's ParetoQ compares five bit widths and puts the accuracy
//              cliff at 1 bit"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "pq_quant_kernels.hpp"

namespace pq {
namespace {


// Rows a launch needs before one wave per row fills the chip
// (256 CUs x 4 SIMDs x 4 waves).
constexpr int64_t kWaveRowsThreshold = 4096;
// Mean row length from which a team of four waves per row is faster even
// with many rows (measured: from 4096 columns on, for fwd, bwd and export).
// Weights per grouped launch from which the forward's outputs are written
// nontemporally (512 Mi weights: 2 GB of fp32 input).
constexpr int64_t kNtStoreElems = int64_t(1) << 29;
#ifndef PQ_TEAM_COLS
#define PQ_TEAM_COLS 4096
#endif
constexpr int64_t kTeamColsThreshold = PQ_TEAM_COLS;

bool finite(double x) { return x == x && x < 1e300 && x > -1e300; }

// Widths with a deployment format: every code container (binary in 1 bit,
// ternary, 2-bit SEQ and the 2-bit LSQ grids in 2, 3- and 4-bit LSQ in 4).
bool deployable(int mode)
{
    return mode == PQ_W1_BINARY || mode == PQ_W158_SEQ_TERNARY || mode == PQ_W2_SEQ || mode == PQ_W3_LSQ ||
           mode == PQ_W4_LSQ || mode == PQ_W2_LSQ || mode == PQ_W158_LSQ;
}

bool ptr_ok(const void *p) { return p == nullptr || aligned16(p); }

// Waves per row of one matrix: a team of four for long rows, or for every
// matrix of a launch too small to fill the chip with one wave per row; one
// wave per row otherwise.
int matrix_wpr(int64_t cols, bool few_rows) { return few_rows || cols >= kTeamColsThreshold ? 4 : 1; }

// Quads per lane per pass for rows of `cols` columns and a team of wpr
// waves: four when that covers the row in one pass, else eight (rows of up
// to 2048 columns with one wave, 8192 with four, in one pass).
// The export reads four bytes per weight and writes a quarter byte: its
// narrow passes at full occupancy measured faster than wide ones (1.5B stack:
// 5128 against 4905 GB/s).
#ifndef PQ_PACK_PASS_WIDE
#define PQ_PACK_PASS_WIDE 0
#endif
#ifndef PQ_QUANT_PASS_WIDE
#define PQ_QUANT_PASS_WIDE 1
#endif
int pass_width(int64_t cols, int wpr)
{
    return cols / 4 > static_cast<int64_t>(kPassNarrow) * 64 * wpr ? kPassWide : kPassNarrow;
}

// Launches over a stack: its matrices split by team size (one wave per row,
// or four), each class in launches of up to kMaxGroup matrices whose table
// maps launch entries to descriptor indices.  A class takes the pass width
// of the rows that hold most of its weights (`wide` = false: always narrow):
// a second launch per width measured slower where one width holds most of
// the weights (the 125M stack: 73 against 71 % of HBM peak), and one width
// per class fits the 1.5B stack, whose classes each have one row length.
// launch_one(lt, blocks, wpr, u, max_cols, stream) starts one launch; `fwd`
// launches take fwd_rows_per_wave rows per wave.
template <typename D, typename F>
pq_status launch_grouped(int count, const D *host, const D *dev, hipStream_t stream, bool fwd, F &&launch_one,
                         bool pad16 = false, bool wide = true)
{
    // pad16: the launch also covers the padding rows of each matrix's last
    // 16-row tile (codes in the export byte order)
    auto rows_of = [&](int i) { return pad16 ? (host[i].rows + 15) / 16 * 16 : host[i].rows; };
    int64_t total_rows = 0, total_elems = 0;
    for (int i = 0; i < count; ++i) {
        total_rows += rows_of(i);
        total_elems += rows_of(i) * host[i].cols;
    }
    const bool few_rows = total_rows < kWaveRowsThreshold;
    // Stacks of several GB stream the forward's bf16 weights out with
    // nontemporal stores: nothing of them stays in the 256 MB MALL anyway,
    // and the 1.5B stack's forward measured 5375 -> 5691 GB/s; smaller
    // launches (the 125M stack, single Llama-3-8B projections) measured
    // 2-7 % faster with plain stores.
    const int nt_out = total_elems >= kNtStoreElems ? 1 : 0;
    for (int wpr : {1, 4}) {
        auto member = [&](int i) { return rows_of(i) > 0 && matrix_wpr(host[i].cols, few_rows) == wpr; };
        int64_t by_width[2] = {0, 0};  // weights whose rows want the narrow / wide pass
        for (int i = 0; i < count; ++i)
            if (member(i)) by_width[pass_width(host[i].cols, wpr) == kPassWide] += rows_of(i) * host[i].cols;
        const int u = wide && by_width[1] > by_width[0] ? kPassWide : kPassNarrow;
        const int rpb = (4 / wpr) * (fwd ? fwd_rows_per_wave(wpr, pad16) : 1);  // rows per block
        int i = 0;
        while (i < count) {
            LaunchTableT<D> lt;
            lt.table = dev;
            lt.count = 0;
            lt.nt_out = nt_out;
            int64_t blocks = 0, max_cols = 0;
            for (; i < count && lt.count < kMaxGroup; ++i) {
                if (!member(i)) continue;
                if (lt.count == 0) lt.single = host[i];
                lt.idx[lt.count] = static_cast<int16_t>(i);
                lt.block_start[lt.count] = static_cast<int32_t>(blocks);
                blocks += (rows_of(i) + rpb - 1) / rpb;
                if (blocks > INT32_MAX) return PQ_ERR_SHAPE;
                if (host[i].cols > max_cols) max_cols = host[i].cols;
                ++lt.count;
            }
            if (lt.count == 0) continue;
            lt.block_start[lt.count] = static_cast<int32_t>(blocks);
            launch_one(lt, static_cast<int>(blocks), wpr, u, max_cols, stream);
            if (hipGetLastError() != hipSuccess) return PQ_ERR_HIP;
        }
    }
    return PQ_OK;
}

#define PQ_MODE_SWITCH(mode, CALL)                                     \
    switch (mode) {                                                    \
    case PQ_W1_BINARY: CALL(PQ_W1_BINARY); break;                      \
    case PQ_W158_SEQ_TERNARY: CALL(PQ_W158_SEQ_TERNARY); break;        \
    case PQ_W2_SEQ: CALL(PQ_W2_SEQ); break;                            \
    case PQ_W3_LSQ: CALL(PQ_W3_LSQ); break;                            \
    case PQ_W2_LSQ: CALL(PQ_W2_LSQ); break;                            \
    case PQ_W158_LSQ: CALL(PQ_W158_LSQ); break;                        \
    default: CALL(PQ_W4_LSQ); break;                                   \
    }

void launch_fwd(int mode, int init, unsigned outs, int u, const LaunchTable &lt, int blocks, int wpr, hipStream_t s)
{
#define PQ_CALL(M) launch_fwd_m<M>(init, outs, u, lt, blocks, wpr, s)
    PQ_MODE_SWITCH(mode, PQ_CALL)
#undef PQ_CALL
}

void launch_fwd_stats(int mode, bool bf16, const LaunchTable &lt, int blocks, int wpr, hipStream_t s, StatsOut so)
{
#define PQ_CALL(M) launch_fwd_stats_m<M>(bf16, lt, blocks, wpr, s, so)
    PQ_MODE_SWITCH(mode, PQ_CALL)
#undef PQ_CALL
}

void launch_bwd(int mode, int u, int wpr, bool gbf, bool wdw, bool wmask, const LaunchTable &lt, int blocks,
                hipStream_t s)
{
#define PQ_CALL(M) launch_bwd_m<M>(u, wpr, gbf, wdw, wmask, lt, blocks, s)
    PQ_MODE_SWITCH(mode, PQ_CALL)
#undef PQ_CALL
}

void launch_step(int mode, int wpr, bool gbf, const StepTable &lt, int blocks, const AdamK &k, hipStream_t s)
{
#define PQ_CALL(M) launch_step_m<M>(wpr, gbf, lt, blocks, k, s)
    PQ_MODE_SWITCH(mode, PQ_CALL)
#undef PQ_CALL
}

void launch_pack(int mode, int u, const LaunchTable &lt, int blocks, int wpr, hipStream_t s)
{
#define PQ_CALL(M) launch_pack_m<M>(u, lt, blocks, wpr, s)
    PQ_MODE_SWITCH(mode, PQ_CALL)
#undef PQ_CALL
}

// Register depth of the scale init for rows of up to max_cols columns and a
// team of wpr waves.
int init_depth(int64_t max_cols, int wpr)
{
    const int64_t per_lane = (max_cols / 4 + 64 * wpr - 1) / (64 * wpr);
    return per_lane <= kInitSmall ? kInitSmall : kInitLarge;
}

unsigned fwd_outs(const pq_mat &m)
{
    return (m.wq_bf16 ? OUT_BF16 : 0u) | (m.wq_f32 ? OUT_F32 : 0u) | (m.codes ? OUT_CODES : 0u);
}

pq_status check_fwd_descs(int mode, int count, const pq_mat *host, unsigned flags, unsigned *outs)
{
    if (!valid_mode(mode)) return PQ_ERR_MODE;
    if ((flags & ~(PQ_INIT_ALPHA | PQ_CODES_EXPORT)) != 0) return PQ_ERR_MODE;
    const bool exported = (flags & PQ_CODES_EXPORT) != 0;
    if (exported && !deployable(mode)) return PQ_ERR_MODE;
    if (count < 0) return PQ_ERR_ARG;
    if (count > 0 && !host) return PQ_ERR_NULL;
    bool have_first = false;
    for (int i = 0; i < count; ++i) {
        const pq_mat &m = host[i];
        if (m.rows < 0 || !valid_cols(m.cols)) return PQ_ERR_SHAPE;
        if (m.rows == 0) continue;  // enqueues nothing; its pointers are not used
        const unsigned o = fwd_outs(m) | (exported ? OUT_TILED : 0u);
        if (exported && !m.codes) return PQ_ERR_NULL;
        if (!have_first) {
            *outs = o;
            have_first = true;
        } else if (o != *outs) {
            return PQ_ERR_ARG;  // one output set per launch
        }
        if (!m.W || !m.alpha) return PQ_ERR_NULL;
        if (!aligned16(m.W) || !ptr_ok(m.wq_bf16) || !ptr_ok(m.wq_f32) || !ptr_ok(m.codes) ||
            !ptr_ok(m.alpha))
            return PQ_ERR_ALIGN;
    }
    return PQ_OK;
}

pq_status check_bwd_descs(int mode, int count, const pq_mat *host, int g_dtype, bool *wdw, bool *wmask)
{
    if (!valid_mode(mode)) return PQ_ERR_MODE;
    if (g_dtype != PQ_G_F32 && g_dtype != PQ_G_BF16) return PQ_ERR_MODE;
    if (count < 0) return PQ_ERR_ARG;
    if (count > 0 && !host) return PQ_ERR_NULL;
    bool have_first = false;
    for (int i = 0; i < count; ++i) {
        const pq_mat &m = host[i];
        if (m.rows < 0 || !valid_cols(m.cols)) return PQ_ERR_SHAPE;
        if (m.rows == 0) continue;  // enqueues nothing; its pointers are not used
        if (!m.W || !m.alpha || !m.G || !m.dalpha) return PQ_ERR_NULL;
        if (!aligned16(m.W) || !aligned16(m.G) || !ptr_ok(m.dW) || !ptr_ok(m.mask_bits) ||
            !ptr_ok(m.alpha) || !ptr_ok(m.dalpha))
            return PQ_ERR_ALIGN;
        if (!(m.grad_scale == m.grad_scale) || m.grad_scale > 1e300 || m.grad_scale < -1e300)
            return PQ_ERR_ARG;
        if (g_dtype == PQ_G_BF16 && m.dW && static_cast<const void *>(m.dW) == m.G) return PQ_ERR_ARG;
        const bool d = m.dW != nullptr, k = m.mask_bits != nullptr;
        if (!have_first) {
            *wdw = d;
            *wmask = k;
            have_first = true;
        } else if (d != *wdw || k != *wmask) {
            return PQ_ERR_ARG;
        }
    }
    return PQ_OK;
}

// AdamW scalars: binary64 from the hyper-parameters, rounded once.
pq_status adam_scalars(const pq_adamw *hp, AdamK *k)
{
    if (!hp) return PQ_ERR_NULL;
    const double lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2, eps = hp->eps, wd = hp->weight_decay;
    if (!finite(lr) || !finite(b1) || !finite(b2) || !finite(eps) || !finite(wd)) return PQ_ERR_ARG;
    if (hp->step < 1 || lr < 0.0 || b1 < 0.0 || b1 >= 1.0 || b2 < 0.0 || b2 >= 1.0 || eps <= 0.0 || wd < 0.0)
        return PQ_ERR_ARG;
    const double t = static_cast<double>(hp->step);
    k->b1 = static_cast<float>(b1);
    k->w1 = static_cast<float>(1.0 - b1);
    k->b2 = static_cast<float>(b2);
    k->w2 = static_cast<float>(1.0 - b2);
    k->s2 = static_cast<float>(sqrt(1.0 - pow(b2, t)));
    k->eps = static_cast<float>(eps);
    k->decay = static_cast<float>(1.0 - lr * wd);
    k->step_size = static_cast<float>(lr / (1.0 - pow(b1, t)));
    return PQ_OK;
}

pq_status check_step_descs(int mode, int count, const pq_step_mat *host, int g_dtype)
{
    if (!valid_mode(mode)) return PQ_ERR_MODE;
    if (g_dtype != PQ_G_F32 && g_dtype != PQ_G_BF16) return PQ_ERR_MODE;
    if (count < 0) return PQ_ERR_ARG;
    if (count > 0 && !host) return PQ_ERR_NULL;
    bool have_first = false, wq = false, cd = false, da = false;
    for (int i = 0; i < count; ++i) {
        const pq_step_mat &m = host[i];
        if (m.rows < 0 || !valid_cols(m.cols)) return PQ_ERR_SHAPE;
        if (m.rows == 0) continue;
        if (!m.W || !m.alpha || !m.G || !m.mW || !m.vW || !m.m_alpha || !m.v_alpha) return PQ_ERR_NULL;
        if (!aligned16(m.W) || !aligned16(m.G) || !aligned16(m.mW) || !aligned16(m.vW) ||
            !ptr_ok(m.alpha) || !ptr_ok(m.m_alpha) || !ptr_ok(m.v_alpha) || !ptr_ok(m.wq_bf16) ||
            !ptr_ok(m.codes) || !ptr_ok(m.dalpha))
            return PQ_ERR_ALIGN;
        if (!finite(m.grad_scale)) return PQ_ERR_ARG;
        const bool w = m.wq_bf16 != nullptr, c = m.codes != nullptr, d = m.dalpha != nullptr;
        if (!have_first) {
            wq = w;
            cd = c;
            da = d;
            have_first = true;
        } else if (w != wq || c != cd || d != da) {
            return PQ_ERR_ARG;
        }
    }
    return PQ_OK;
}

// Export: the forward's codes in the export byte order plus bf16(alpha), one
// launch over every matrix's rows rounded up to 16 (the padding rows of each
// last tile are written as zeros).
pq_status check_pack_descs(int mode, int count, const pq_mat *host)
{
    if (!deployable(mode)) return PQ_ERR_MODE;
    if (count < 0) return PQ_ERR_ARG;
    if (count > 0 && !host) return PQ_ERR_NULL;
    for (int i = 0; i < count; ++i) {
        const pq_mat &m = host[i];
        if (m.rows < 0 || !valid_cols(m.cols)) return PQ_ERR_SHAPE;
        if (m.rows == 0) continue;  // enqueues nothing; its pointers are not used
        if (!m.W || !m.alpha || !m.codes || !m.alpha_bf16) return PQ_ERR_NULL;
        if (!aligned16(m.W) || !aligned16(m.alpha) || !aligned16(m.codes) || !aligned16(m.alpha_bf16))
            return PQ_ERR_ALIGN;
    }
    return PQ_OK;
}

pq_status pack_grouped(int mode, int count, const pq_mat *host, const pq_mat *dev, void *stream)
{
    return launch_grouped(
        count, host, dev, static_cast<hipStream_t>(stream), true,
        [&](const LaunchTable &lt, int blocks, int wpr, int u, int64_t, hipStream_t s) {
            launch_pack(mode, u, lt, blocks, wpr, s);
        },
        true, PQ_PACK_PASS_WIDE != 0);
}

pq_status pack_common(int mode, int64_t rows, int64_t cols, const float *W,
                             const float *alpha, uint8_t *packed, void *alpha_bf16, void *stream)
{
    pq_mat m = {};
    m.W = W;
    m.alpha = const_cast<float *>(alpha);
    m.codes = packed;
    m.alpha_bf16 = alpha_bf16;
    m.rows = rows;
    m.cols = cols;
    if (!deployable(mode)) return PQ_ERR_MODE;
    if (!W || !alpha || !packed || !alpha_bf16) return PQ_ERR_NULL;
    const pq_status st = check_pack_descs(mode, 1, &m);
    if (st != PQ_OK) return st;
    return pack_grouped(mode, 1, &m, nullptr, stream);
}

}  // namespace
}  // namespace pq

using namespace pq;

extern "C" {

int64_t pq_code_row_bytes(int mode, int64_t cols)
{
    if (!valid_mode(mode) || cols <= 0) return -1;
    return (cols * code_bits(mode) + 7) / 8;
}

int64_t pq_packed_bytes(int mode, int64_t rows, int64_t cols)
{
    if (!deployable(mode) || rows < 0 || !valid_cols(cols)) return -1;
    const int64_t rb = cols * code_bits(mode) / 8;
    return (rb + 63) / 64 * ((rows + 15) / 16 * 16) * 64;
}

double pq_default_grad_scale(int mode, int64_t rows, int64_t cols)
{
    if (!valid_mode(mode) || rows <= 0 || cols <= 0) return 0.0;
    const double qp = mode == PQ_W3_LSQ ? 3.0 : (mode == PQ_W4_LSQ ? 7.0 : 1.0);
    return 1.0 / sqrt(static_cast<double>(rows) * static_cast<double>(cols) * qp);
}

const char *pq_status_str(pq_status s)
{
    switch (s) {
    case PQ_OK: return "PQ_OK";
    case PQ_ERR_NULL: return "PQ_ERR_NULL: a required pointer is NULL";
    case PQ_ERR_SHAPE: return "PQ_ERR_SHAPE: bad rows/cols/M/N/K (cols and K must be positive multiples of 8)";
    case PQ_ERR_MODE: return "PQ_ERR_MODE: unknown mode, flag or dtype";
    case PQ_ERR_ALIGN: return "PQ_ERR_ALIGN: array pointer not 16-byte aligned";
    case PQ_ERR_UNSUPPORTED: return "PQ_ERR_UNSUPPORTED";
    case PQ_ERR_HIP: return "PQ_ERR_HIP: kernel launch failed";
    case PQ_ERR_ARG: return "PQ_ERR_ARG: bad argument (descriptor table, grad_scale or aliasing)";
    }
    return "unknown pq_status";
}

const char *pq_version(void) { return "libpq 0.1 (gfx950)"; }

pq_status pq_quantize_fwd_grouped(int mode, int count, const pq_mat *descs_host,
                                  const pq_mat *descs_dev, unsigned flags, void *stream)
{
    unsigned outs = 0;
    pq_status st = check_fwd_descs(mode, count, descs_host, flags, &outs);
    if (st != PQ_OK) return st;
    if (count > 0 && !descs_dev) return PQ_ERR_NULL;
    const bool init = (flags & PQ_INIT_ALPHA) != 0;
    return launch_grouped(
        count, descs_host, descs_dev, static_cast<hipStream_t>(stream), true,
        [&](const LaunchTable &lt, int blocks, int wpr, int u, int64_t max_cols, hipStream_t s) {
            launch_fwd(mode, init ? init_depth(max_cols, wpr) : 0, outs, u, lt, blocks, wpr, s);
        },
        (flags & PQ_CODES_EXPORT) != 0, PQ_QUANT_PASS_WIDE != 0);
}

pq_status pq_quantize_fwd(int mode, int64_t rows, int64_t cols, const float *W, float *alpha,
                          unsigned flags, void *Wq_bf16, float *Wq_f32, uint8_t *codes,
                          void *stream)
{
    pq_mat m = {};
    m.W = W;
    m.alpha = alpha;
    m.wq_bf16 = Wq_bf16;
    m.wq_f32 = Wq_f32;
    m.codes = codes;
    m.rows = rows;
    m.cols = cols;
    unsigned outs = 0;
    pq_status st = check_fwd_descs(mode, 1, &m, flags, &outs);
    if (st != PQ_OK) return st;
    const bool init = (flags & PQ_INIT_ALPHA) != 0;
    return launch_grouped(
        1, &m, static_cast<const pq_mat *>(nullptr), static_cast<hipStream_t>(stream), true,
        [&](const LaunchTable &lt, int blocks, int wpr, int u, int64_t max_cols, hipStream_t s) {
            launch_fwd(mode, init ? init_depth(max_cols, wpr) : 0, outs, u, lt, blocks, wpr, s);
        },
        (flags & PQ_CODES_EXPORT) != 0, PQ_QUANT_PASS_WIDE != 0);
}

pq_status pq_quantize_fwd_stats(int mode, int64_t rows, int64_t cols, const float *W, const float *alpha,
                                void *Wq_bf16, uint8_t *codes, uint32_t *counts, double *entropy, void *stream)
{
    using namespace pq;
    pq_mat m = {};
    m.W = W;
    m.alpha = const_cast<float *>(alpha);
    m.wq_bf16 = Wq_bf16;
    m.codes = codes;
    m.rows = rows;
    m.cols = cols;
    unsigned outs = 0;
    pq_status st = check_fwd_descs(mode, 1, &m, 0u, &outs);
    if (st != PQ_OK) return st;
    if (rows == 0) return PQ_OK;
    if (!codes || !counts) return PQ_ERR_NULL;
    if (!ptr_ok(counts) || !ptr_ok(entropy)) return PQ_ERR_ALIGN;
    const StatsOut so{counts, entropy};
    return launch_grouped(1, &m, static_cast<const pq_mat *>(nullptr), static_cast<hipStream_t>(stream), true,
                          [&](const LaunchTable &lt, int blocks, int wpr, int, int64_t, hipStream_t s) {
                              launch_fwd_stats(mode, Wq_bf16 != nullptr, lt, blocks, wpr, s, so);
                          });
}

pq_status pq_quantize_bwd_grouped(int mode, int count, const pq_mat *descs_host,
                                  const pq_mat *descs_dev, int g_dtype, void *stream)
{
    bool wdw = false, wmask = false;
    pq_status st = check_bwd_descs(mode, count, descs_host, g_dtype, &wdw, &wmask);
    if (st != PQ_OK) return st;
    if (count > 0 && !descs_dev) return PQ_ERR_NULL;
    return launch_grouped(count, descs_host, descs_dev, static_cast<hipStream_t>(stream), false,
                          [&](const LaunchTable &lt, int blocks, int wpr, int u, int64_t, hipStream_t s) {
                              launch_bwd(mode, u, wpr, g_dtype == PQ_G_BF16, wdw, wmask, lt, blocks, s);
                          },
                          false, PQ_QUANT_PASS_WIDE != 0);
}

pq_status pq_quantize_bwd(int mode, int64_t rows, int64_t cols, const float *W, const float *alpha,
                          const void *G, int g_dtype, double grad_scale, float *dW, float *dalpha,
                          uint8_t *mask_bits, void *stream)
{
    pq_mat m = {};
    m.W = W;
    m.alpha = const_cast<float *>(alpha);
    m.G = G;
    m.dW = dW;
    m.dalpha = dalpha;
    m.mask_bits = mask_bits;
    m.grad_scale = grad_scale;
    m.rows = rows;
    m.cols = cols;
    bool wdw = false, wmask = false;
    pq_status st = check_bwd_descs(mode, 1, &m, g_dtype, &wdw, &wmask);
    if (st != PQ_OK) return st;
    return launch_grouped(1, &m, static_cast<const pq_mat *>(nullptr), static_cast<hipStream_t>(stream),
                          false,
                          [&](const LaunchTable &lt, int blocks, int wpr, int u, int64_t, hipStream_t s) {
                              launch_bwd(mode, u, wpr, g_dtype == PQ_G_BF16, wdw, wmask, lt, blocks, s);
                          },
                          false, PQ_QUANT_PASS_WIDE != 0);
}

pq_status pq_pack_grouped(int mode, int count, const pq_mat *descs_host, const pq_mat *descs_dev, void *stream)
{
    const pq_status st = check_pack_descs(mode, count, descs_host);
    if (st != PQ_OK) return st;
    if (count > 0 && !descs_dev) return PQ_ERR_NULL;
    return pack_grouped(mode, count, descs_host, descs_dev, stream);
}

pq_status pq_pack(int mode, int64_t rows, int64_t cols, const float *W, const float *alpha, uint8_t *packed,
                  void *alpha_bf16, void *stream)
{
    return pack_common(mode, rows, cols, W, alpha, packed, alpha_bf16, stream);
}

pq_status pq_pack_w2(int64_t rows, int64_t cols, const float *W, const float *alpha,
                     uint8_t *packed, void *alpha_bf16, void *stream)
{
    return pack_common(PQ_W2_SEQ, rows, cols, W, alpha, packed, alpha_bf16, stream);
}

pq_status pq_pack_w4(int64_t rows, int64_t cols, const float *W, const float *alpha,
                     uint8_t *packed, void *alpha_bf16, void *stream)
{
    return pack_common(PQ_W4_LSQ, rows, cols, W, alpha, packed, alpha_bf16, stream);
}

pq_status pq_qat_step_grouped(int mode, int count, const pq_step_mat *descs_host, const pq_step_mat *descs_dev,
                              int g_dtype, const pq_adamw *hp, void *stream)
{
    pq_status st = check_step_descs(mode, count, descs_host, g_dtype);
    if (st != PQ_OK) return st;
    AdamK k;
    st = adam_scalars(hp, &k);
    if (st != PQ_OK) return st;
    if (count > 0 && !descs_dev) return PQ_ERR_NULL;
    return launch_grouped(count, descs_host, descs_dev, static_cast<hipStream_t>(stream), false,
                          [&](const StepTable &lt, int blocks, int wpr, int, int64_t, hipStream_t s) {
                              launch_step(mode, wpr, g_dtype == PQ_G_BF16, lt, blocks, k, s);
                          },
                          false, false);
}

pq_status pq_qat_step(int mode, int64_t rows, int64_t cols, float *W, float *alpha, const void *G, int g_dtype,
                      double grad_scale, float *mW, float *vW, float *m_alpha, float *v_alpha,
                      const pq_adamw *hp, void *Wq_bf16, uint8_t *codes, float *dalpha, void *stream)
{
    pq_step_mat m = {};
    m.W = W;
    m.alpha = alpha;
    m.G = G;
    m.mW = mW;
    m.vW = vW;
    m.m_alpha = m_alpha;
    m.v_alpha = v_alpha;
    m.wq_bf16 = Wq_bf16;
    m.codes = codes;
    m.dalpha = dalpha;
    m.grad_scale = grad_scale;
    m.rows = rows;
    m.cols = cols;
    pq_status st = check_step_descs(mode, 1, &m, g_dtype);
    if (st != PQ_OK) return st;
    AdamK k;
    st = adam_scalars(hp, &k);
    if (st != PQ_OK) return st;
    return launch_grouped(1, &m, static_cast<const pq_step_mat *>(nullptr), static_cast<hipStream_t>(stream), false,
                          [&](const StepTable &lt, int blocks, int wpr, int, int64_t, hipStream_t s) {
                              launch_step(mode, wpr, g_dtype == PQ_G_BF16, lt, blocks, k, s);
                          },
                          false, false);
}

}  // extern "C"
