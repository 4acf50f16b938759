/*
 * pq_oracle.c -- plain, slow, CPU reference ("the oracle") for the ParetoQ
 * quantized linear layer: alpha init, forward fake-quantization at
 * 1 / 1.58 / 2 / 3 / 4 bits, the straight-through backward with the per-row
 * scale gradient, 2-bit / 4-bit export packing (and the deployment byte
 * order of the exported codes) and the packed-weight GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or constant with the GPU library, and the GPU library never
 * calls it.
 *
 * Sources (web pages, cited by title and section):
 *   [Note]     "ParetoQ, the strongest low-bit QAT I could find"
 *              (sections "QAT versus PTQ", "Finding 3", "The 2-bit recipe,
 *              in full", "Paper vs. code").
 *   [Rebuttal] "ParetoQ: Improving Scaling Laws in Extremely Low-bit LLM
 *              Quantization" (the authors' OpenReview replies; part
 *              "Regarding more discussion on why SEQ is better than LSQ").
 *   [News]     "Meta's ParetoQ compares five bit widths and puts the accuracy
 *              cliff at 1 bit" (speed and storage paragraphs).
 *   [Abstract] "ParetoQ: Scaling Laws in Extremely Low-bit LLM Quantization".
 *
 * Arithmetic: every float expression below is one IEEE binary32 operation
 * rounded to nearest-even.  Build with -O2 -ffp-contract=off, no fast-math, on
 * x86-64 SSE (no x87 excess precision, no flush-to-zero).  Sums that the
 * method leaves to the implementation are taken in binary64, sequentially in
 * column order.
 *
 * Parity unpinned (no page fixes them; each is a documented reading):
 *   - the 1-bit quantizer as a whole (the pages name the width only);
 *   - the ternary alpha-gradient value for clipped weights (+-2/3);
 *   - n and Qp of the 1/sqrt(n*Qp) gradient scale (only the default value).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Bit-width modes, in the order the pages list the widths ([Abstract]). */
enum {
    PQO_W1_BINARY = 0,        /* 1 bit                                   */
    PQO_W158_SEQ_TERNARY = 1, /* 1.58 bit, SEQ                           */
    PQO_W2_SEQ = 2,           /* 2 bit, SEQ                              */
    PQO_W3_LSQ = 3,           /* 3 bit, LSQ integer grid                 */
    PQO_W4_LSQ = 4,           /* 4 bit, LSQ integer grid                 */
    /* The LSQ grids the pages set against SEQ at 2 and 1.58 bits ([Rebuttal],
     * part on why SEQ beats LSQ): the ablation, not the recipe. */
    PQO_W2_LSQ = 5,           /* 2 bit, LSQ levels {-2, -1, 0, 1}        */
    PQO_W158_LSQ = 6          /* 1.58 bit, LSQ levels {-1, 0, 1}         */
};

/* [Note] "Paper vs. code", first bullet: the shipped clip is 1 - 1e-2, which
 * removes the fifth level (+1.25 alpha) that clipping to +-1 would create. */
static const float CLIP_SHIPPED = 0.99f;
/* Guard against alpha <= 0 (the pages are silent): divide by max(alpha, 1e-5). */
static const float ALPHA_FLOOR = 1e-5f;
/* [Note] "Finding 3": ternary SEQ levels are {-2/3, 0, +2/3} alpha. */
static const float TWO_THIRDS = (float)(2.0 / 3.0);

static int valid_mode(int mode) { return mode >= PQO_W1_BINARY && mode <= PQO_W158_LSQ; }

/* Bits per stored code: 1 for binary, 2 for ternary and 2-bit SEQ (the
 * [News] storage paragraph notes ternary is often kept as 2-bit integers),
 * a 4-bit nibble for 3- and 4-bit LSQ. */
int pqo_code_bits(int mode)
{
    switch (mode) {
    case PQO_W1_BINARY: return 1;
    case PQO_W158_SEQ_TERNARY: return 2;
    case PQO_W2_SEQ: return 2;
    case PQO_W3_LSQ: return 4;
    case PQO_W4_LSQ: return 4;
    case PQO_W2_LSQ: return 2;
    case PQO_W158_LSQ: return 2;
    }
    return -1;
}

/* LSQ integer grid [Note] "Finding 3": levels -2^(b-1) .. 2^(b-1)-1, so
 * {-2, -1, 0, 1} at 2 bits ([Rebuttal], 2-bit bullet); at 1.58 bits LSQ
 * scales the weight to [-1, 1] and rounds onto {-1, 0, 1} ([Rebuttal],
 * 1.58-bit bullet). */
static int is_lsq(int mode)
{
    return mode == PQO_W3_LSQ || mode == PQO_W4_LSQ || mode == PQO_W2_LSQ || mode == PQO_W158_LSQ;
}
static float lsq_qn(int mode)
{
    switch (mode) {
    case PQO_W158_LSQ: return -1.0f;
    case PQO_W2_LSQ: return -2.0f;
    case PQO_W3_LSQ: return -4.0f;
    default: return -8.0f;
    }
}
static float lsq_qp(int mode)
{
    switch (mode) {
    case PQO_W158_LSQ: return 1.0f;
    case PQO_W2_LSQ: return 1.0f;
    case PQO_W3_LSQ: return 3.0f;
    default: return 7.0f;
    }
}

/* Smallest step index r of each grid; the stored code is r - r_min. */
static int r_min_of(int mode)
{
    switch (mode) {
    case PQO_W1_BINARY: return -1;
    case PQO_W158_SEQ_TERNARY: return -1;
    case PQO_W2_SEQ: return -2;
    default: return (int)lsq_qn(mode);
    }
}

/* Stored code of step index r: offset-binary r - r_min on the multi-level
 * grids; for the two 1-bit levels -1, +1 the code is 0, 1. */
static unsigned code_of(int mode, int r)
{
    if (mode == PQO_W1_BINARY) return r > 0 ? 1u : 0u;
    return (unsigned)(r - r_min_of(mode));
}

static int step_of_code(int mode, unsigned code)
{
    if (mode == PQO_W1_BINARY) return code ? 1 : -1;
    return (int)code + r_min_of(mode);
}

float pqo_clip_value(void) { return CLIP_SHIPPED; }

/* bf16 round-to-nearest-even of a finite binary32 value: keep the top 16
 * bits, adding half an ulp of the result (plus one if the kept part is odd). */
uint16_t pqo_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

float pqo_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ---------------------------------------------------------------------------
 * One weight through the quantizer.  Returns the step index r and writes the
 * fake-quantized binary32 value q (before the bf16 cast) and x = w / alpha.
 * ------------------------------------------------------------------------- */

/* 2-bit SEQ, [Note] "Paper vs. code" (SEQ formula row):
 *   q = alpha * (round(Clip(w/alpha) * k/2 - 0.5) + 0.5) / k * 2,  k = 4,
 * with round = half-to-even and the clip bound `clip` (0.99 as shipped; the
 * test suite also evaluates the literal +-1 of the paper's equation). */
int pqo_seq2_quantize(float w, float alpha, float clip, float *q_out, float *x_out)
{
    float a = alpha > ALPHA_FLOOR ? alpha : ALPHA_FLOOR;
    float x = w / a;                          /* w / alpha               */
    float xc = fmaxf(x, -clip);               /* Clip(., -clip, clip)    */
    xc = fminf(xc, clip);
    float z = xc * 2.0f;                      /* * k/2 with k = 4        */
    z = z - 0.5f;                             /* - 0.5                   */
    float rf = rintf(z);                      /* round half-to-even      */
    int r = (int)rf;
    float t = (float)r + 0.5f;                /* + 0.5                   */
    float q = a * t;                          /* alpha * (...)           */
    q = q / 4.0f;                             /* / k                     */
    q = q * 2.0f;                             /* * 2                     */
    if (q_out) *q_out = q;
    if (x_out) *x_out = x;
    return r;
}

/* Ternary SEQ, [Rebuttal] 1.58-bit bullet: the clipped ratio is stretched to
 * [-1.5, 1.5] and cut into three equal-width bins [-1.5,-0.5], [-0.5,0.5],
 * [0.5,1.5] -> -1, 0, +1 (ties at +-0.5 go to the even index 0); the level of
 * bin r is r * 2/3 of alpha ([Note] "Finding 3"). */
static int ternary_quantize(float w, float alpha, float *q_out, float *x_out)
{
    float a = alpha > ALPHA_FLOOR ? alpha : ALPHA_FLOOR;
    float x = w / a;
    float xc = fmaxf(x, -CLIP_SHIPPED);
    xc = fminf(xc, CLIP_SHIPPED);
    float v = xc * 1.5f;                      /* stretch to [-1.5, 1.5]  */
    float rf = rintf(v);                      /* nearest bin centre      */
    int r = (int)rf;
    float level = (float)r * TWO_THIRDS;      /* -2/3, 0, +2/3           */
    float q = a * level;
    if (q_out) *q_out = q;
    if (x_out) *x_out = x;
    return r;
}

/* LSQ: q = alpha * round(clamp(w/alpha, Qn, Qp)) on the integer grid
 * ([Note] "Finding 3"; the dispatch row of "Paper vs. code" sends 3 and 4
 * bits to LSQ; the 2- and 1.58-bit grids are the [Rebuttal]'s ablation). */
static int lsq_quantize(int mode, float w, float alpha, float *q_out, float *x_out)
{
    float a = alpha > ALPHA_FLOOR ? alpha : ALPHA_FLOOR;
    float x = w / a;
    float xc = fmaxf(x, lsq_qn(mode));
    xc = fminf(xc, lsq_qp(mode));
    float rf = rintf(xc);
    int r = (int)rf;
    float q = a * (float)r;
    if (q_out) *q_out = q;
    if (x_out) *x_out = x;
    return r;
}

/* 1 bit: q = alpha * sign(w), sign(0) taken as +1 so exactly two levels exist.
 * The pages give the width only; this is the sign / mean-|W| binarizer of
 * XNOR-Net, which [Rebuttal] cites as binary prior work. */
static int binary_quantize(float w, float alpha, float *q_out, float *x_out)
{
    float a = alpha > ALPHA_FLOOR ? alpha : ALPHA_FLOOR;
    float x = w / a;
    int r = (w >= 0.0f) ? 1 : -1;
    float q = a * (float)r;
    if (q_out) *q_out = q;
    if (x_out) *x_out = x;
    return r;
}

int pqo_quantize_scalar(int mode, float w, float alpha, float *q_out, float *x_out)
{
    switch (mode) {
    case PQO_W1_BINARY: return binary_quantize(w, alpha, q_out, x_out);
    case PQO_W158_SEQ_TERNARY: return ternary_quantize(w, alpha, q_out, x_out);
    case PQO_W2_SEQ: return pqo_seq2_quantize(w, alpha, CLIP_SHIPPED, q_out, x_out);
    case PQO_W3_LSQ:
    case PQO_W4_LSQ:
    case PQO_W2_LSQ:
    case PQO_W158_LSQ: return lsq_quantize(mode, w, alpha, q_out, x_out);
    }
    return 0;
}

/* Level of step index r in units of alpha, as a binary64 value. */
static double level_of(int mode, int r)
{
    switch (mode) {
    case PQO_W2_SEQ: return ((double)r + 0.5) / 2.0;        /* +-0.25, +-0.75 */
    case PQO_W158_SEQ_TERNARY: return (double)((float)r * TWO_THIRDS);
    default: return (double)r;                               /* LSQ, binary    */
    }
}

/* Write `code` (cw bits) as element j of a row's LSB-first bit stream. */
static void put_code(uint8_t *row, int64_t j, int cw, unsigned code)
{
    int64_t bit = j * cw;
    row[bit >> 3] |= (uint8_t)((code & ((1u << cw) - 1u)) << (bit & 7));
}

static unsigned get_code(const uint8_t *row, int64_t j, int cw)
{
    int64_t bit = j * cw;
    return (row[bit >> 3] >> (bit & 7)) & ((1u << cw) - 1u);
}

int64_t pqo_code_row_bytes(int mode, int64_t cols)
{
    return (cols * pqo_code_bits(mode) + 7) / 8;
}

void pqo_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int pqo_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------------------
 * alpha initialisation, per output row.
 *   2-bit SEQ and ternary: max|w| ([Note] "The 2-bit recipe" table and the
 *   scale-init row of "Paper vs. code").
 *   LSQ: max|w| / Qp, Qp = 2^(b-1) - 1 (3 at 3 bits, 7 at 4, 1 for the
 *   2-bit and the 1.58-bit LSQ grids), one binary32 division (same row).
 *   1 bit: mean|w|, summed in binary64 in column order, divided in binary64,
 *   rounded once to binary32.
 * Returns 0, or -1 on a bad argument.
 * ------------------------------------------------------------------------- */
int pqo_alpha_init(int mode, int64_t rows, int64_t cols, const float *W, float *alpha)
{
    if (!valid_mode(mode) || rows < 0 || cols <= 0 || !W || !alpha) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        const float *w = W + i * cols;
        if (mode == PQO_W1_BINARY) {
            double s = 0.0;
            for (int64_t j = 0; j < cols; ++j) s += (double)fabsf(w[j]);
            alpha[i] = (float)(s / (double)cols);
        } else {
            float m = 0.0f;
            for (int64_t j = 0; j < cols; ++j) {
                float v = fabsf(w[j]);
                if (v > m) m = v;
            }
            if (is_lsq(mode)) m = m / lsq_qp(mode);
            alpha[i] = m;
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Forward.  For every weight: the mode's quantizer above; the binary32 value
 * is cast to bf16 (round to nearest-even) because the layer casts the
 * fake-quantized weight to the activation dtype ([Note] "Paper vs. code",
 * last bullet).  Outputs are optional (NULL skips them):
 *   wq_bf16 [rows, cols] bf16 bits, wq_f32 [rows, cols], codes [rows,
 *   code_row_bytes] (code_of above), LSB-first.
 * ------------------------------------------------------------------------- */
int pqo_quantize_fwd(int mode, int64_t rows, int64_t cols, const float *W,
                     const float *alpha, uint16_t *wq_bf16, float *wq_f32,
                     uint8_t *codes)
{
    if (!valid_mode(mode) || rows < 0 || cols <= 0 || !W || !alpha) return -1;
    const int cw = pqo_code_bits(mode);
    const int64_t rb = pqo_code_row_bytes(mode, cols);
    if (codes) memset(codes, 0, (size_t)(rows * rb));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < cols; ++j) {
            float q;
            int r = pqo_quantize_scalar(mode, W[i * cols + j], alpha[i], &q, NULL);
            if (wq_bf16) wq_bf16[i * cols + j] = pqo_bf16_rne(q);
            if (wq_f32) wq_f32[i * cols + j] = q;
            if (codes) put_code(codes + i * rb, j, cw, code_of(mode, r));
        }
    }
    return 0;
}

/* Qp used in the 1/sqrt(n * Qp) scale of the alpha gradient ([Note]
 * "Paper vs. code", LSQ-gradient row): 2^(b-1) - 1 for 3 and 4 bits,
 * floored at 1 for the widths where that count is below one. */
static double grad_qp(int mode)
{
    switch (mode) {
    case PQO_W3_LSQ: return 3.0;
    case PQO_W4_LSQ: return 7.0;
    case PQO_W2_LSQ: return 1.0;
    case PQO_W158_LSQ: return 1.0;
    default: return 1.0;
    }
}

/* Default gradient scale 1/sqrt(n * Qp), n = number of weights in the matrix
 * (LSQ's count of the weights the scale serves). */
double pqo_default_grad_scale(int mode, int64_t rows, int64_t cols)
{
    return 1.0 / sqrt((double)rows * (double)cols * grad_qp(mode));
}

/* ---------------------------------------------------------------------------
 * Backward.  G is dL/d(fake-quantized weight), binary32 (g_is_bf16 = 0) or
 * bf16 bits (g_is_bf16 = 1).  Per weight, with x = w / alpha:
 *   inside = x lies in the clip range, bounds included: [-0.99, 0.99] for SEQ
 *            and ternary, [Qn, Qp] for LSQ, [-1, 1] for 1 bit;
 *   dW     = G where inside, exactly +0 elsewhere ([Note] "QAT versus PTQ"
 *            and the STE paragraph of "The 2-bit recipe, in full");
 *   s      = d q / d alpha with round() (sign() at 1 bit) passed straight
 *            through: level - x inside; the boundary level (the level of the
 *            clipped value) outside, which keeps a gradient flowing to alpha
 *            from clipped weights (same paragraph);
 *   dalpha = grad_scale * sum_j s * G, summed in binary64, rounded once
 *            ([Note] "Paper vs. code", LSQ-gradient row).
 * mask_bits (optional) gets `inside` per weight, LSB-first, ceil(cols/8)
 * bytes per row.
 * ------------------------------------------------------------------------- */
int pqo_quantize_bwd(int mode, int64_t rows, int64_t cols, const float *W,
                     const float *alpha, const void *G, int g_is_bf16,
                     double grad_scale, float *dW, float *dalpha,
                     uint8_t *mask_bits)
{
    if (!valid_mode(mode) || rows < 0 || cols <= 0 || !W || !alpha || !G) return -1;
    const int64_t mb = (cols + 7) / 8;
    if (mask_bits) memset(mask_bits, 0, (size_t)(rows * mb));
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            int64_t e = i * cols + j;
            float g = g_is_bf16 ? pqo_bf16_to_f32(((const uint16_t *)G)[e])
                                : ((const float *)G)[e];
            float x;
            int r = pqo_quantize_scalar(mode, W[e], alpha[i], NULL, &x);
            int inside;
            double s;
            if (mode == PQO_W1_BINARY) {
                /* sign(w) plays the part of round(): level - x inside
                 * [-1, 1], the boundary level sign(w) outside. */
                inside = (x >= -1.0f) && (x <= 1.0f);
                if (inside) s = (double)r - (double)x;
                else s = (double)r;
            } else if (is_lsq(mode)) {
                float qn = lsq_qn(mode), qp = lsq_qp(mode);
                inside = (x >= qn) && (x <= qp);
                if (inside) s = (double)r - (double)x;
                else s = (x < qn) ? (double)qn : (double)qp;
            } else {
                inside = (x >= -CLIP_SHIPPED) && (x <= CLIP_SHIPPED);
                /* Outside, r is the index of the clipped value, so level_of(r)
                 * is the boundary level +-0.75 (2 bit) or +-2/3 (ternary). */
                if (inside) s = level_of(mode, r) - (double)x;
                else s = level_of(mode, r);
            }
            if (dW) dW[e] = inside ? g : 0.0f;
            if (mask_bits && inside) mask_bits[i * mb + (j >> 3)] |= (uint8_t)(1u << (j & 7));
            acc += s * (double)g;
        }
        if (dalpha) dalpha[i] = (float)(grad_scale * acc);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Export: the codes the forward emits for W and the per-row scale rounded to
 * bf16.  Memory savings exist only after such an export ([Note] "Paper vs.
 * code", last bullet).  Widths with a 2-bit container (ternary, 2-bit SEQ;
 * ternary is commonly held in 2-bit integers, [News] storage paragraph) or a
 * 4-bit one (3- and 4-bit LSQ).
 * ------------------------------------------------------------------------- */
/* Widths with an export: every code container (1-bit codes eight per byte,
 * 2-bit four per byte, 4-bit two per byte). */
static int deployable(int mode)
{
    return mode == PQO_W1_BINARY || mode == PQO_W158_SEQ_TERNARY || mode == PQO_W2_SEQ || mode == PQO_W3_LSQ ||
           mode == PQO_W4_LSQ || mode == PQO_W2_LSQ || mode == PQO_W158_LSQ;
}

int pqo_pack(int mode, int64_t rows, int64_t cols, const float *W, const float *alpha,
             uint8_t *packed, uint16_t *alpha_bf16)
{
    if (!deployable(mode)) return -1;
    if (pqo_quantize_fwd(mode, rows, cols, W, alpha, NULL, NULL, packed) != 0) return -1;
    if (alpha_bf16)
        for (int64_t i = 0; i < rows; ++i) alpha_bf16[i] = pqo_bf16_rne(alpha[i]);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Optimizer step.  The recipe trains W and the per-row scale alpha with AdamW
 * at weight decay 0 ([Note] "The 2-bit recipe, in full", optimizer row); the
 * pages give no formula, so this is AdamW as published (Adam moments with
 * bias correction, weight decay decoupled from the gradient), in this
 * binary32 order, one rounding per operation:
 *   m'  = b1 * m + (1 - b1) * g
 *   v'  = b2 * v + ((1 - b2) * g) * g
 *   den = sqrt(v') / sqrt(1 - b2^t) + eps
 *   p'  = p * (1 - lr * wd) - (lr / (1 - b1^t)) * m' / den
 * The scalars b1, 1 - b1, b2, 1 - b2, sqrt(1 - b2^t), eps, 1 - lr * wd and
 * lr / (1 - b1^t) are computed in binary64 from the hyper-parameters and
 * rounded once to binary32.  t >= 1 is the step number.
 * ------------------------------------------------------------------------- */
typedef struct {
    float b1, w1, b2, w2, s2, eps, decay, step_size;
} adam_k;

static adam_k adam_scalars(double lr, double b1, double b2, double eps, double wd, int64_t t)
{
    adam_k k;
    k.b1 = (float)b1;
    k.w1 = (float)(1.0 - b1);
    k.b2 = (float)b2;
    k.w2 = (float)(1.0 - b2);
    k.s2 = (float)sqrt(1.0 - pow(b2, (double)t));
    k.eps = (float)eps;
    k.decay = (float)(1.0 - lr * wd);
    k.step_size = (float)(lr / (1.0 - pow(b1, (double)t)));
    return k;
}

static float adam_one(const adam_k *k, float p, float g, float *m, float *v)
{
    const float mn = k->b1 * *m + k->w1 * g;
    const float vn = k->b2 * *v + (k->w2 * g) * g;
    const float den = sqrtf(vn) / k->s2 + k->eps;
    const float pd = p * k->decay;
    *m = mn;
    *v = vn;
    return pd - (k->step_size * mn) / den;
}

static int adam_args_ok(double lr, double b1, double b2, double eps, double wd, int64_t t)
{
    return t >= 1 && lr >= 0.0 && lr < 1e30 && b1 >= 0.0 && b1 < 1.0 && b2 >= 0.0 && b2 < 1.0 &&
           eps > 0.0 && eps < 1e30 && wd >= 0.0 && wd < 1e30;
}

/* AdamW on n parameters p with gradients g and moments m, v (all updated in
 * place except g). */
int pqo_adamw(int64_t n, float *p, const float *g, float *m, float *v, double lr, double b1,
              double b2, double eps, double wd, int64_t t)
{
    if (n < 0 || !adam_args_ok(lr, b1, b2, eps, wd, t)) return -1;
    const adam_k k = adam_scalars(lr, b1, b2, eps, wd, t);
    for (int64_t i = 0; i < n; ++i) p[i] = adam_one(&k, p[i], g[i], &m[i], &v[i]);
    return 0;
}

/* One QAT step of a quantized linear layer, as three steps of its definition
 * in order: the straight-through backward of the current forward
 * (pqo_quantize_bwd: dW and dalpha from W, alpha and G), AdamW on W (with
 * dW) and on alpha (with dalpha, its own moments), then the next forward's
 * fake-quantization of the updated W with the updated alpha
 * (pqo_quantize_fwd).  W, alpha and the four moment arrays are updated in
 * place; wq_bf16, codes and dalpha_out are optional outputs. */
int pqo_qat_step(int mode, int64_t rows, int64_t cols, float *W, float *alpha, const void *G,
                 int g_is_bf16, double grad_scale, float *mW, float *vW, float *m_alpha,
                 float *v_alpha, double lr, double b1, double b2, double eps, double wd,
                 int64_t t, uint16_t *wq_bf16, uint8_t *codes, float *dalpha_out)
{
    if (!valid_mode(mode) || rows < 0 || cols <= 0 || !W || !alpha || !G || !mW || !vW ||
        !m_alpha || !v_alpha || !adam_args_ok(lr, b1, b2, eps, wd, t))
        return -1;
    float *dW = (float *)malloc((size_t)(rows * cols) * sizeof(float) + 1);
    float *da = (float *)malloc((size_t)rows * sizeof(float) + 1);
    if (!dW || !da) {
        free(dW);
        free(da);
        return -1;
    }
    int rc = pqo_quantize_bwd(mode, rows, cols, W, alpha, G, g_is_bf16, grad_scale, dW, da, NULL);
    if (rc == 0) rc = pqo_adamw(rows * cols, W, dW, mW, vW, lr, b1, b2, eps, wd, t);
    if (rc == 0) rc = pqo_adamw(rows, alpha, da, m_alpha, v_alpha, lr, b1, b2, eps, wd, t);
    if (rc == 0) rc = pqo_quantize_fwd(mode, rows, cols, W, alpha, wq_bf16, NULL, codes);
    if (rc == 0 && dalpha_out) memcpy(dalpha_out, da, (size_t)rows * sizeof(float));
    free(dW);
    free(da);
    return rc;
}

/* ---------------------------------------------------------------------------
 * Diagnostics the pages argue with: how the weights of a row spread over the
 * levels (the level occupancy behind the SEQ-vs-LSQ argument of [Rebuttal]
 * and [Note] "Finding 3") and how far training moved the weights from their
 * starting point ([Note] "QAT versus PTQ": QAT compensates rather than
 * reconstructs).
 *   counts[i, c]  number of weights of row i stored with code c, c = 0 ..
 *                 levels - 1 (codes are offset-binary: code c is level c);
 *   entropy[i]    -sum_c p_c log2 p_c, p_c = counts[i, c] / cols, binary64;
 *   sq_diff[i]    sum_j (W[i,j] - W0[i,j])^2 and sq_ref[i] = sum_j W0[i,j]^2,
 *                 each difference and square a binary64 operation, summed
 *                 in column order.
 * ------------------------------------------------------------------------- */
int pqo_num_levels(int mode)
{
    switch (mode) {
    case PQO_W1_BINARY: return 2;
    case PQO_W158_SEQ_TERNARY: return 3;
    case PQO_W2_SEQ: return 4;
    case PQO_W3_LSQ: return 8;
    case PQO_W4_LSQ: return 16;
    case PQO_W2_LSQ: return 4;
    case PQO_W158_LSQ: return 3;
    default: return -1;
    }
}

int pqo_level_stats(int mode, int64_t rows, int64_t cols, const uint8_t *codes, uint32_t *counts,
                    double *entropy)
{
    if (!valid_mode(mode) || rows < 0 || cols <= 0 || !codes || !counts) return -1;
    const int L = pqo_num_levels(mode), cw = pqo_code_bits(mode);
    const int64_t rb = pqo_code_row_bytes(mode, cols);
    for (int64_t i = 0; i < rows; ++i) {
        uint32_t *c = counts + i * L;
        for (int l = 0; l < L; ++l) c[l] = 0;
        for (int64_t j = 0; j < cols; ++j) {
            const unsigned code = get_code(codes + i * rb, j, cw);
            if ((int)code >= L) return -1;
            c[code] += 1;
        }
        if (entropy) {
            double h = 0.0;
            for (int l = 0; l < L; ++l)
                if (c[l]) {
                    const double p = (double)c[l] / (double)cols;
                    h -= p * log2(p);
                }
            entropy[i] = h;
        }
    }
    return 0;
}

int pqo_weight_movement(int64_t rows, int64_t cols, const float *W, const float *W0, double *sq_diff,
                        double *sq_ref)
{
    if (rows < 0 || cols <= 0 || !W || !W0 || !sq_diff || !sq_ref) return -1;
    for (int64_t i = 0; i < rows; ++i) {
        double d2 = 0.0, r2 = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            const double d = (double)W[i * cols + j] - (double)W0[i * cols + j];
            const double r = (double)W0[i * cols + j];
            d2 += d * d;
            r2 += r * r;
        }
        sq_diff[i] = d2;
        sq_ref[i] = r2;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Deployment layout of the exported codes.  The pages fix only what a packed
 * 2-bit weight holds (four codes per byte and a bf16 scale per row, [News]
 * storage and speed paragraphs); the byte order the deployed GEMM reads is
 * this library's own, defined here from the row-major code rows that the
 * forward emits (rb bytes per row, cw-bit codes, first code lowest):
 *
 * 1. (2-bit codes only) inside each 4-byte word of a row -- 16 codes
 *    k0 .. k15, code ki in bits 2i .. 2i+1 of the little-endian word, the
 *    row's bytes zero-padded to a whole word -- byte j (j = 0 .. 3) of the
 *    export word holds
 *        k(2j) in bits 0-1, k(8+2j) in bits 2-3,
 *        k(2j+1) in bits 4-5, k(9+2j) in bits 6-7,
 *    so that masking the word with 0x33333333 leaves codes k0 .. k7 in its
 *    eight nibbles in k order (low nibble of each byte first), and masking
 *    it shifted right by 2 leaves k8 .. k15.  1- and 4-bit codes keep the
 *    row-major bytes.
 * 2. the bytes are then placed group by group:
 *    groups   g = 0 .. G-1,  G  = ceil(rb / 64)   (64 bytes of every row)
 *    tiles    t = 0 .. Np/16-1, Np = rows rounded up to a multiple of 16
 *    row r = 0 .. 15 of the tile, byte e = 0 .. 63 of the row's group
 *    tiled[((g * (Np/16) + t) * 16 + r) * 64 + e]
 *        = row[16 t + r] byte 64 g + e  (after step 1)
 *    when the row 16 t + r < rows and the byte lies within the row (rb
 *    bytes; for 2-bit codes rb rounded up to a whole word), else 0.
 * So every 64-byte group of all rows is one contiguous run (group-major),
 * inside it each tile of 16 rows is 1 KB, and inside a tile each row's 64
 * bytes are contiguous.  Size: G * Np * 64 bytes.
 * ------------------------------------------------------------------------- */
int64_t pqo_tiled_bytes(int64_t rows, int64_t rb)
{
    if (rows < 0 || rb < 0) return -1;
    return ((rb + 63) / 64) * ((rows + 15) / 16 * 16) * 64;
}

/* Step 1 for one word of 2-bit codes. */
static uint32_t export_word2(uint32_t w)
{
    uint32_t out = 0;
    for (int j = 0; j < 4; ++j) {
        const uint32_t b = ((w >> (2 * (2 * j))) & 3u) | (((w >> (2 * (8 + 2 * j))) & 3u) << 2) |
                           (((w >> (2 * (2 * j + 1))) & 3u) << 4) | (((w >> (2 * (9 + 2 * j))) & 3u) << 6);
        out |= b << (8 * j);
    }
    return out;
}

int pqo_tile_codes(int cw, int64_t rows, int64_t rb, const uint8_t *rowmajor, uint8_t *tiled)
{
    if (rows < 0 || rb < 0 || (cw != 1 && cw != 2 && cw != 4)) return -1;
    const int64_t G = (rb + 63) / 64, T = (rows + 15) / 16;
    const int64_t rbw = cw == 2 ? (rb + 3) / 4 * 4 : rb;  /* bytes the row covers in the export */
    uint8_t *row = (uint8_t *)calloc((size_t)(G * 64 > 0 ? G * 64 : 1), 1);
    if (!row) return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int r = 0; r < 16; ++r) {
            const int64_t n = 16 * t + r;
            memset(row, 0, (size_t)(G * 64));
            if (n < rows) {
                memcpy(row, rowmajor + n * rb, (size_t)rb);
                if (cw == 2)
                    for (int64_t c = 0; c < rbw; c += 4) {
                        const uint32_t w = (uint32_t)row[c] | ((uint32_t)row[c + 1] << 8) |
                                           ((uint32_t)row[c + 2] << 16) | ((uint32_t)row[c + 3] << 24);
                        const uint32_t e = export_word2(w);
                        for (int b = 0; b < 4; ++b) row[c + b] = (uint8_t)(e >> (8 * b));
                    }
            }
            for (int64_t g = 0; g < G; ++g)
                for (int e = 0; e < 64; ++e) {
                    const int64_t c = 64 * g + e;
                    tiled[((g * T + t) * 16 + r) * 64 + e] = c < rbw ? row[c] : 0;
                }
        }
    free(row);
    return 0;
}

/* Dequantized level of a stored code, in units of alpha. */
static double code_level(int mode, unsigned code)
{
    return level_of(mode, step_of_code(mode, code));
}

/* ---------------------------------------------------------------------------
 * Deployment GEMM reference, binary64: Y[m,n] = sum_k X[m,k] * alpha[n] *
 * level(code[n,k]) -- a plain matmul of the activations with the dequantized
 * packed weight (the deployed layer of the [News] speed paragraph, whose
 * 2-bit-weight kernel is timed against FP16 and 4-bit GEMMs; the layer has no
 * bias, [Note] "Paper vs. code").  X is [M,K] bf16 bits, packed is
 * [N, code_row_bytes(K)], alpha_bf16 is [N].
 * pqo_gemm_ref fills all of Y [M,N]; pqo_gemm_ref_at only the listed (m, n).
 * ------------------------------------------------------------------------- */
static double gemm_one(int mode, int64_t K, const uint16_t *xrow, const uint8_t *crow,
                       double a)
{
    const int cw = pqo_code_bits(mode);
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double w = a * code_level(mode, get_code(crow, k, cw));
        acc += (double)pqo_bf16_to_f32(xrow[k]) * w;
    }
    return acc;
}

int pqo_gemm_ref(int mode, int64_t M, int64_t N, int64_t K, const uint16_t *X,
                 const uint8_t *packed, const uint16_t *alpha_bf16, double *Y)
{
    if (!deployable(mode)) return -1;
    const int64_t rb = pqo_code_row_bytes(mode, K);
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            Y[m * N + n] = gemm_one(mode, K, X + m * K, packed + n * rb,
                                    (double)pqo_bf16_to_f32(alpha_bf16[n]));
    return 0;
}

/* The same product with a binary32 scale per row (the training forward's
 * alpha, before any export rounding): Y[m,n] = sum_k X[m,k] * alpha[n] *
 * level(code[n,k]) in binary64. */
int pqo_gemm_ref_f32a(int mode, int64_t M, int64_t N, int64_t K, const uint16_t *X,
                      const uint8_t *packed, const float *alpha, double *Y)
{
    if (!deployable(mode)) return -1;
    const int64_t rb = pqo_code_row_bytes(mode, K);
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            Y[m * N + n] = gemm_one(mode, K, X + m * K, packed + n * rb, (double)alpha[n]);
    return 0;
}

int pqo_gemm_ref_at(int mode, int64_t M, int64_t N, int64_t K, const uint16_t *X,
                    const uint8_t *packed, const uint16_t *alpha_bf16,
                    const int64_t *ms, const int64_t *ns, int64_t count, double *out)
{
    if (!deployable(mode)) return -1;
    const int64_t rb = pqo_code_row_bytes(mode, K);
    for (int64_t t = 0; t < count; ++t)
        if (ms[t] < 0 || ms[t] >= M || ns[t] < 0 || ns[t] >= N) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < count; ++t)
        out[t] = gemm_one(mode, K, X + ms[t] * K, packed + ns[t] * rb,
                          (double)pqo_bf16_to_f32(alpha_bf16[ns[t]]));
    return 0;
}
