/*
 * pq.h -- C ABI of libpq, the gfx950 (MI355X) implementation of the ParetoQ
 * quantized linear layer: per-row fake-quantization of fp32 shadow weights at
 * 1 / 1.58 / 2 / 3 / 4 bits, its straight-through backward with the learned
 * per-row scale's gradient, 2-bit (and 4-bit) export packing, and the
 * packed-weight x bf16-activation GEMM used at deployment.
 *
 * Sources (web pages, cited by title and section):
 *   [Note]     "ParetoQ, the strongest low-bit QAT I could find" -- sections
 *              "QAT versus PTQ", "Finding 3", "The 2-bit recipe, in full",
 *              "Paper vs. code".
 *   [Rebuttal] "ParetoQ: Improving Scaling Laws in Extremely Low-bit LLM
 *              Quantization" -- authors' replies, part on why SEQ beats LSQ.
 *   [News]     "Meta's ParetoQ compares five bit widths and puts the accuracy
 *              cliff at 1 bit" -- speed and storage paragraphs.
 *   [Abstract] "ParetoQ: Scaling Laws in Extremely Low-bit LLM Quantization".
 *
 * Conventions shared by every entry point
 *   Memory     Every array argument is a DEVICE pointer owned by the caller;
 *              the library keeps no pointer after the call returns and never
 *              allocates or frees device memory: the GEMM's scratch (split-K
 *              partial sums) is a caller-owned
 *              workspace sized by pq_gemm_workspace_bytes.  The one
 *              exception is pq_gemm_noalloc, whose scratch is a fixed array
 *              inside the library (see there).  Arrays are row-major and
 *              contiguous
 *              (leading dimension = cols), except the exported codes of
 *              pq_pack_w2 / pq_pack_w4 (the export byte order below).  Weight matrices are [out, in]:
 *              a "row" is one output channel, the unit the scale alpha
 *              belongs to ([Note] "Paper vs. code": one learned scale per
 *              row, shape (rows, 1)).
 *   Streams    `stream` is a hipStream_t (NULL = the null stream).  Calls only
 *              enqueue work on it and return, without waiting on the host;
 *              results are ready when the stream is.  Apart from
 *              pq_gemm_noalloc's scratch the library holds no global mutable
 *              state, so calls from several host threads are safe, and every
 *              call can be captured into a HIP graph (including its first
 *              call).
 *   bf16       bf16 arrays are passed as void* and hold IEEE bfloat16 bit
 *              patterns; every cast to bf16 rounds to nearest-even.
 *   Errors     Arguments are checked on the host before anything is enqueued:
 *              a NULL required pointer -> PQ_ERR_NULL; rows, cols, M, N or K
 *              negative, cols not a positive multiple of 8, K not a
 *              positive multiple of 64 or above 2^24, or N above 2^24 ->
 *              PQ_ERR_SHAPE; an
 *              unknown mode,
 *              flag or dtype -> PQ_ERR_MODE; an array pointer not 16-byte
 *              aligned -> PQ_ERR_ALIGN; a bad descriptor table or grad_scale
 *              -> PQ_ERR_ARG.  A failed launch -> PQ_ERR_HIP.  On any error
 *              nothing is enqueued.  Zero rows (or M = 0 / N = 0) is valid
 *              and enqueues nothing; the array pointers of such an empty
 *              matrix are not checked or used.
 *   Inputs     Weights, scales and gradients must be finite (not checked;
 *              outputs are unspecified otherwise).  A scale alpha <= 1e-5 is
 *              used as 1e-5 in the arithmetic (and stored unchanged), so an
 *              all-zero row gives finite outputs.
 */
#ifndef PQ_H_
#define PQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pq_status {
    PQ_OK = 0,
    PQ_ERR_NULL = 1,
    PQ_ERR_SHAPE = 2,
    PQ_ERR_MODE = 3,
    PQ_ERR_ALIGN = 4,
    PQ_ERR_UNSUPPORTED = 5,
    PQ_ERR_HIP = 6,
    PQ_ERR_ARG = 7
} pq_status;

/* Bit widths of the unified framework ([Abstract]: 1, 1.58, 2, 3, 4 bits).
 * SEQ at 1.58 and 2 bits, LSQ at 3 and 4 bits ([Note] "Paper vs. code",
 * dispatch row); the two LSQ grids the pages set against SEQ at 2 and 1.58
 * bits ([Rebuttal], part on why SEQ beats LSQ) are the ablation modes 5 and
 * 6.  Level sets, in units of alpha:
 *   PQ_W1_BINARY         {-1, +1}            sign(w), sign(0) = +1
 *   PQ_W158_SEQ_TERNARY  {-2/3, 0, +2/3}     ([Note] "Finding 3"; bins of
 *                                             [Rebuttal], 1.58-bit bullet)
 *   PQ_W2_SEQ            {-3/4,-1/4,1/4,3/4} ([Note] "Finding 3" and the SEQ
 *                                             formula row of "Paper vs. code")
 *   PQ_W3_LSQ            {-4 .. 3}           ([Note] "Finding 3": integer grid)
 *   PQ_W4_LSQ            {-8 .. 7}
 *   PQ_W2_LSQ            {-2, -1, 0, 1}      ([Rebuttal], 2-bit bullet)
 *   PQ_W158_LSQ          {-1, 0, 1}          (weights scaled to [-1, 1];
 *                                             [Rebuttal], 1.58-bit bullet)
 * LSQ clips x to [Qn, Qp] (the set's ends) and rounds half-to-even.
 * Stored codes: 1 bit for binary (0 -> -1, 1 -> +1); 2 bits for ternary and
 * 2-bit SEQ (code = step + 1 resp. step + 2, so ternary never stores 3; the
 * [News] storage paragraph notes ternary is commonly held in 2-bit integers);
 * a 4-bit nibble for 3- and 4-bit LSQ (code = step + 2^(b-1)); 2 bits for
 * the ablation grids (code = step - Qn).  Codes are a bit stream
 * per row, first element in the lowest bits of the first byte. */
typedef enum pq_mode {
    PQ_W1_BINARY = 0,
    PQ_W158_SEQ_TERNARY = 1,
    PQ_W2_SEQ = 2,
    PQ_W3_LSQ = 3,
    PQ_W4_LSQ = 4,
    PQ_W2_LSQ = 5,
    PQ_W158_LSQ = 6
} pq_mode;

/* pq_quantize_fwd flag: compute alpha from the row first and store it
 * ([Note] "The 2-bit recipe" table and the scale-init row of "Paper vs.
 * code": alpha = max|w| for SEQ and ternary, max|w| / Qp for LSQ with
 * Qp = 2^(b-1)-1, i.e. 3, 7, and 1 for both ablation grids;
 * mean|w| for 1 bit, summed in binary64). */
#define PQ_INIT_ALPHA 1u

/* pq_quantize_fwd flag: write `codes` in the export byte order of
 * pq_pack_w2 (pq_packed_bytes(mode, rows, cols) bytes, padding zeroed)
 * instead of row-major, so that the next GEMM can read them directly (the
 * training forward through pq_gemm_f32a, with no bf16 weights written or
 * read).  Deployable widths only (else PQ_ERR_MODE); codes must then be
 * non-NULL. */
#define PQ_CODES_EXPORT 2u

/* Upstream-gradient dtypes for pq_quantize_bwd. */
#define PQ_G_F32 0
#define PQ_G_BF16 1

/* Bytes per row of the code array of `mode` for `cols` weights
 * (cols * code_bits / 8), or -1 for a bad mode / cols. */
int64_t pq_code_row_bytes(int mode, int64_t cols);

/* Default alpha-gradient scale 1/sqrt(n * Qp) with n = rows * cols and
 * Qp = 1, 1, 1, 3, 7 for 1, 1.58, 2, 3, 4 bits ([Note] "Paper vs. code",
 * LSQ-gradient row: LSQ's 1/sqrt(n * Qp)).  Returns 0 for a bad argument. */
double pq_default_grad_scale(int mode, int64_t rows, int64_t cols);

/* Human-readable name of a status code (static string). */
const char *pq_status_str(pq_status s);

/* Library version string (static). */
const char *pq_version(void);

/*
 * pq_quantize_fwd -- forward fake-quantization of one weight matrix.
 * Every training step re-quantizes the fp32 shadow weights ([Note] "QAT
 * versus PTQ"); per weight w of row i, with a = max(alpha[i], 1e-5):
 *   x = w / a (IEEE division), clipped to [-0.99, 0.99] for SEQ / ternary
 *   ([Note] "Paper vs. code", first bullet) or to [Qn, Qp] for LSQ, rounded
 *   half-to-even onto the mode's grid; q = a * level; Wq = bf16(q), the cast
 *   to the activation dtype ([Note] "Paper vs. code", last bullet).
 *
 *   mode      pq_mode
 *   rows,cols W is [rows, cols] fp32; cols a positive multiple of 8
 *   W         in   [rows, cols] fp32 shadow weights
 *   alpha     in   [rows] fp32 per-row scale; with PQ_INIT_ALPHA it is OUT:
 *                  written with the row statistic, then used
 *   flags     0, PQ_INIT_ALPHA and/or PQ_CODES_EXPORT
 *   Wq_bf16   out  [rows, cols] bf16 fake-quantized weights, or NULL
 *   Wq_f32    out  [rows, cols] the same values before the bf16 cast, or NULL
 *   codes     out  [rows, pq_code_row_bytes(mode, cols)] packed codes, or NULL
 *   stream    hipStream_t
 */
pq_status pq_quantize_fwd(int mode, int64_t rows, int64_t cols, const float *W,
                          float *alpha, unsigned flags, void *Wq_bf16, float *Wq_f32,
                          uint8_t *codes, void *stream);

/*
 * pq_quantize_bwd -- straight-through backward of pq_quantize_fwd.
 * Per weight (same a and x as the forward, bit for bit):
 *   inside = x within the clip range, bounds included ([-0.99, 0.99] SEQ and
 *            ternary, [Qn, Qp] LSQ, [-1, 1] binary);
 *   dW     = G inside, exactly +0 outside -- the rounding is treated as the
 *            identity inside the range and the clamp is flat outside ([Note]
 *            "QAT versus PTQ" and the gradient paragraph of "The 2-bit
 *            recipe, in full");
 *   dalpha = grad_scale * sum_j s_j * G_j per row, with s = level - x inside
 *            and s = the boundary level outside (clipped weights still feed
 *            the scale), accumulated in binary64 and rounded once ([Note]
 *            "Paper vs. code", LSQ-gradient row).
 *   The boundary level is +-0.75 at 2-bit SEQ, +-fl32(2/3) for ternary (the
 *   level of the clipped value), Qn or Qp for the LSQ grids.  For 1 bit,
 *   sign(w) plays the part of the rounding, so the same rule reads
 *   s = sign(w) - x inside |x| <= 1 and s = sign(w) outside (sign(+-0) = +1).
 *   The pages name no binary gradient; this uniform reading is the library's
 *   own, and an alternative (s = sign(w) everywhere, the derivative of
 *   q = alpha * sign(w)) would change dalpha on every binary row.  The
 *   ternary outside value and the default grad_scale carry readings the
 *   pages do not pin either.
 *
 *   W, alpha   in   as in the forward (alpha is the value the forward used)
 *   G          in   [rows, cols] dL/dWq, fp32 (PQ_G_F32) or bf16 (PQ_G_BF16)
 *   g_dtype    PQ_G_F32 or PQ_G_BF16
 *   grad_scale the alpha-gradient scale; pass pq_default_grad_scale(...)
 *              for LSQ's 1/sqrt(n*Qp); must be finite
 *   dW         out  [rows, cols] fp32, or NULL; may alias G when g_dtype is
 *                   PQ_G_F32 (each element is read before it is written)
 *   dalpha     out  [rows] fp32
 *   mask_bits  out  [rows, cols/8] the `inside` bit per weight, first weight
 *                   in the lowest bit, or NULL
 */
pq_status pq_quantize_bwd(int mode, int64_t rows, int64_t cols, const float *W,
                          const float *alpha, const void *G, int g_dtype,
                          double grad_scale, float *dW, float *dalpha,
                          uint8_t *mask_bits, void *stream);

/*
 * Export byte order.  The exported codes are the forward's code rows
 * (pq_quantize_fwd `codes`: rb = cols * b / 8 bytes per row, eight 1-bit,
 * four 2-bit or two 4-bit codes per byte, first code lowest), reordered for
 * the deployment GEMM, which reads 16 rows x 64 bytes as one MFMA operand
 * ([News] speed paragraph: the 2-bit kernel consumes packed weights; the
 * pages fix four codes per byte and a bf16 scale per row, not a byte order):
 * 1. 2-bit codes only: each 4-byte word of a row (16 codes k0 .. k15, code
 *    ki in bits 2i .. 2i+1 of the little-endian word; the row zero-padded to
 *    whole words, rbw = rb rounded up to 4) is rewritten so that its byte j
 *    holds k(2j) in bits 0-1, k(8+2j) in bits 2-3, k(2j+1) in bits 4-5 and
 *    k(9+2j) in bits 6-7: masked with 0x33333333 the word's nibbles are
 *    codes k0 .. k7 in order (low nibble of each byte first), and shifted
 *    right by 2 and masked, k8 .. k15.  1- and 4-bit rows keep their bytes
 *    (rbw = rb).
 * 2. With Np = rows rounded up to a multiple of 16 and G = ceil(rb / 64):
 *    byte c of row n (c < rbw, n < rows) is stored at
 *      (c / 64) * Np * 64 + (n / 16) * 1024 + (n % 16) * 64 + c % 64,
 *    i.e. group-major runs of 64 bytes of every row, each 16-row tile 1 KB
 *    ordered [row][64 bytes].  Every other byte (rows rows .. Np - 1,
 *    bytes rbw .. 64 G - 1 of a row) is written as 0.  Total size
 *    G * Np * 64 bytes = pq_packed_bytes(mode, rows, cols).
 */
int64_t pq_packed_bytes(int mode, int64_t rows, int64_t cols);

/* Widths with a deployment format ("deployable" below): PQ_W1_BINARY in a
 * 1-bit container (eight codes per byte), PQ_W158_SEQ_TERNARY, PQ_W2_SEQ,
 * PQ_W2_LSQ and PQ_W158_LSQ in a 2-bit container, PQ_W3_LSQ and PQ_W4_LSQ
 * in a 4-bit one
 * (ternary is commonly held in 2-bit integers, [News] storage paragraph).
 * pq_packed_bytes returns -1 for a bad mode. */

/*
 * pq_pack_w2 -- export a 2-bit SEQ layer for deployment: the forward's codes
 * (the bytes of pq_quantize_fwd(PQ_W2_SEQ, ...) codes, bit for bit) in the
 * export byte order, and the scale rounded to bf16.  Memory savings exist
 * only after export ([Note] "Paper vs. code", last bullet); the deployed
 * GEMM consumes this format ([News] speed paragraph).
 *   W          in   [rows, cols] fp32, cols a positive multiple of 8
 *   alpha      in   [rows] fp32
 *   packed     out  pq_packed_bytes(PQ_W2_SEQ, rows, cols) bytes, export
 *                   byte order (above); every byte is written
 *   alpha_bf16 out  [rows] bf16
 */
pq_status pq_pack_w2(int64_t rows, int64_t cols, const float *W, const float *alpha,
                     uint8_t *packed, void *alpha_bf16, void *stream);

/* pq_pack -- the export of any deployable width (the same contract as
 * pq_pack_w2, with the width's code container); an other mode ->
 * PQ_ERR_MODE.  pq_pack_w2 is pq_pack(PQ_W2_SEQ, ...), pq_pack_w4
 * pq_pack(PQ_W4_LSQ, ...). */
pq_status pq_pack(int mode, int64_t rows, int64_t cols, const float *W, const float *alpha,
                  uint8_t *packed, void *alpha_bf16, void *stream);

/* pq_pack_w4 -- the 4-bit LSQ counterpart of pq_pack_w2 (two codes per byte,
 * low nibble first; pq_packed_bytes(PQ_W4_LSQ, rows, cols) bytes in the
 * export byte order), feeding pq_w4a16_gemm, the 4-bit comparison point of
 * the [News] speed paragraph. */
pq_status pq_pack_w4(int64_t rows, int64_t cols, const float *W, const float *alpha,
                     uint8_t *packed, void *alpha_bf16, void *stream);

/*
 * pq_gemm_workspace_bytes -- device workspace, in bytes, that the GEMM entry
 * points below need for this width and shape: 0 when the kernels chosen for
 * the shape use none, -1 for an unknown mode or a shape they reject.  The
 * kernel choice is a fixed function of (mode, M, N, K), so the value is the
 * same for every call with these arguments:
 *   M <= 16 (weight streaming): none;
 *   larger M with 64 x 256 (or 64 x 192) output tiles: when there are too
 *     few tiles to fill the chip, K is split over blocks, each split writes
 *     fp32 partial sums [splits, M, N] and a second kernel adds them in
 *     split order -- splits * M * N * 4 bytes; otherwise none;
 *   large M at 2-bit widths (K >= 2048; M >= 1024, or M >= 512 when N gives
 *     at least 512 tiles of 64 x 256): none (the kernel sums the activation
 *     rows for the level offset itself);
 *   short K at 2-bit widths (K <= 704, M >= 1024; the codes of a column
 *     tile stay in LDS): none.
 */
int64_t pq_gemm_workspace_bytes(int mode, int64_t M, int64_t N, int64_t K);

/*
 * pq_w2a16_gemm -- deployment GEMM with packed 2-bit SEQ weights and bf16
 * activations ([News] speed paragraph: 2-bit-weight kernel against FP16 and
 * 4-bit weights at a 16384 x 16384 weight; the layer has no bias, [Note]
 * "Paper vs. code"):
 *   Y[m, n] = bf16( alpha_bf16[n] * sum_k X[m, k] * level(code[n, k]) )
 * with level(c) = (c - 1.5) / 2, fp32 accumulation.
 *   M, N, K    X is [M, K]; K a positive multiple of 64 (so every packed
 *              row is a whole number of 16-byte pieces) and at most 2^24,
 *              0 <= N <= 2^24 (the kernels address up to 64 activation rows
 *              or one 64-byte group of all weight rows with 32-bit offsets);
 *              M >= 0
 *   X          in   [M, K] bf16 activations
 *   packed     in   pq_packed_bytes(PQ_W2_SEQ, N, K) bytes from pq_pack_w2
 *                   (export byte order; the padding bytes are never used)
 *   alpha_bf16 in   [N] bf16
 *   Y          out  [M, N] bf16
 *   workspace  scratch device memory of at least
 *              pq_gemm_workspace_bytes(PQ_W2_SEQ, M, N, K) bytes, 16-byte
 *              aligned, owned by the caller; its contents on entry do not
 *              matter and on return are unspecified.  May be NULL when that
 *              size is 0.  Two calls in flight at once (on different
 *              streams) need different workspaces.
 *   workspace_bytes  the size of `workspace` (>= 0)
 * Errors as above, and: workspace needed but NULL -> PQ_ERR_NULL; not
 * 16-byte aligned -> PQ_ERR_ALIGN; workspace_bytes too small or negative ->
 * PQ_ERR_ARG.
 * Caches: with M <= 16 the weight codes are read as non-temporal (streaming)
 * loads, so that they neither displace other data nor force dirty lines out
 * of the last-level cache; a later call on the same weight should not count
 * on finding them cached.  Larger M reads them with ordinary loads.
 */
pq_status pq_w2a16_gemm(int64_t M, int64_t N, int64_t K, const void *X,
                        const uint8_t *packed, const void *alpha_bf16, void *Y,
                        void *workspace, int64_t workspace_bytes, void *stream);

/* pq_w4a16_gemm -- the same GEMM on pq_pack_w4 weights
 * (pq_packed_bytes(PQ_W4_LSQ, N, K) bytes), level(c) = c - 8. */
pq_status pq_w4a16_gemm(int64_t M, int64_t N, int64_t K, const void *X,
                        const uint8_t *packed, const void *alpha_bf16, void *Y,
                        void *workspace, int64_t workspace_bytes, void *stream);

/* pq_gemm -- the same GEMM for any deployable width, on pq_pack(mode, ...)
 * weights, with the width's levels ([Note] "Finding 3"): ternary
 * (c - 1) * fl32(2/3), 2-bit SEQ (c - 1.5) / 2, 3-bit LSQ c - 4, 4-bit LSQ
 * c - 8, and the ablation grids c - 2 (2-bit LSQ) and c - 1 (1.58-bit LSQ);
 * an other mode -> PQ_ERR_MODE.  These are the widths whose accuracy
 * and storage the pages compare ([News] speed and storage paragraphs).
 * Workspace as pq_w2a16_gemm, sized by pq_gemm_workspace_bytes(mode, ...). */
pq_status pq_gemm(int mode, int64_t M, int64_t N, int64_t K, const void *X,
                  const uint8_t *packed, const void *alpha_bf16, void *Y,
                  void *workspace, int64_t workspace_bytes, void *stream);

/* pq_gemm_f32a -- pq_gemm with the binary32 scale of training (alpha [N]
 * fp32, as pq_quantize_fwd keeps it) instead of the exported bf16 one: the
 * QAT forward's linear layer computed from the codes, Y = bf16(alpha[n] *
 * sum_k X[m,k] * level(code[n,k])), with the codes written by
 * pq_quantize_fwd(..., PQ_CODES_EXPORT, ...).  It reads 1/8 or 1/4 of the
 * bytes of the fake-quantized bf16 weights and never materialises them; the
 * forward's own Wq = bf16(alpha * level) rounds each weight to bf16 first,
 * so the two differ by that rounding (relative 2^-9 per weight).  Errors
 * and workspace as pq_gemm; alpha NULL -> PQ_ERR_NULL. */
pq_status pq_gemm_f32a(int mode, int64_t M, int64_t N, int64_t K, const void *X,
                       const uint8_t *packed, const float *alpha, void *Y,
                       void *workspace, int64_t workspace_bytes, void *stream);

/*
 * pq_gemm_noalloc -- pq_gemm for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, kernels and results as pq_gemm, without the
 * workspace: the scratch the kernels need (split-K partial sums;
 * pq_gemm_workspace_bytes of the shape) is a fixed array of
 * PQ_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, looked up
 * on the first call made on that GPU and held until the process ends.  The
 * call allocates nothing and never waits on the host.
 *   A shape whose scratch need exceeds PQ_NOALLOC_SCRATCH_BYTES ->
 *   PQ_ERR_UNSUPPORTED, with nothing enqueued (use pq_gemm with a workspace).
 *   Other errors as pq_gemm.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (no part of it needs to start at zero): calls that overlap on one
 * GPU (on different streams, or from different host threads) race on it and
 * must be serialised by the caller.
 */
#define PQ_NOALLOC_SCRATCH_BYTES (((int64_t)32) << 20)
pq_status pq_gemm_noalloc(int mode, int64_t M, int64_t N, int64_t K, const void *X,
                          const uint8_t *packed, const void *alpha_bf16, void *Y, void *stream);

/*
 * Grouped launches: one kernel launch over a whole stack of matrices (for
 * example every projection of every layer of a model), since a training step
 * re-quantizes all of them with the same mode.
 *
 * pq_mat describes one matrix.  The caller fills an array of them twice --
 * in host memory (checked and used for launch sizing) and an identical copy
 * in device memory (read by the kernels); the two must hold the same values.
 * Unused fields may be NULL.  Any count >= 0 is accepted (large stacks are
 * split over several launches internally).
 */
typedef struct pq_mat {
    const float *W;       /* [rows, cols] fp32                             */
    float *alpha;         /* [rows] fp32 (in; out with PQ_INIT_ALPHA)      */
    void *wq_bf16;        /* fwd out [rows, cols] bf16, or NULL            */
    float *wq_f32;        /* fwd out [rows, cols] fp32, or NULL            */
    uint8_t *codes;       /* fwd out codes, or NULL                        */
    const void *G;        /* bwd in [rows, cols] (dtype per call)          */
    float *dW;            /* bwd out [rows, cols] fp32, or NULL            */
    float *dalpha;        /* bwd out [rows] fp32                           */
    uint8_t *mask_bits;   /* bwd out [rows, cols/8], or NULL               */
    double grad_scale;    /* bwd alpha-gradient scale for this matrix      */
    int64_t rows;
    int64_t cols;         /* positive multiple of 8                        */
    void *alpha_bf16;     /* export out [rows] bf16 (pq_pack_grouped)      */
} pq_mat;

/* Forward over `count` matrices; per matrix exactly pq_quantize_fwd.
 * descs_host / descs_dev: identical pq_mat[count] in host / device memory. */
pq_status pq_quantize_fwd_grouped(int mode, int count, const pq_mat *descs_host,
                                  const pq_mat *descs_dev, unsigned flags, void *stream);

/* Backward over `count` matrices; per matrix exactly pq_quantize_bwd with
 * that entry's grad_scale. */
pq_status pq_quantize_bwd_grouped(int mode, int count, const pq_mat *descs_host,
                                  const pq_mat *descs_dev, int g_dtype, void *stream);

/* Export over `count` matrices in one launch; per matrix exactly
 * pq_pack(mode, rows, cols, W, alpha, codes, alpha_bf16): `codes` receives
 * pq_packed_bytes(mode, rows, cols) bytes in the export byte order and
 * `alpha_bf16` the [rows] bf16 scales (the export of a whole model, [Note]
 * "Paper vs. code", last bullet: savings exist only after export). */
pq_status pq_pack_grouped(int mode, int count, const pq_mat *descs_host,
                          const pq_mat *descs_dev, void *stream);

/*
 * Fused QAT step: the straight-through backward of the current forward,
 * AdamW on W and alpha, and the next forward's fake-quantization, in one
 * pass over each row.  The recipe trains the shadow weights and the per-row
 * scale with AdamW at weight decay 0 and a cosine-decayed learning rate
 * ([Note] "The 2-bit recipe, in full", optimizer and learning-rate rows);
 * the pages give no update formula, so this is AdamW as published, with
 * decoupled weight decay, computed in binary32 in this order, one rounding
 * per operation (g = dW for W, g = dalpha for alpha):
 *   m'  = b1 * m + (1 - b1) * g
 *   v'  = b2 * v + ((1 - b2) * g) * g
 *   den = sqrt(v') / sqrt(1 - b2^t) + eps
 *   p'  = p * (1 - lr * wd) - (lr / (1 - b1^t)) * m' / den
 * where b1, 1 - b1, b2, 1 - b2, sqrt(1 - b2^t), eps, 1 - lr * wd and
 * lr / (1 - b1^t) are computed in binary64 on the host and rounded once to
 * binary32.  dW and dalpha are exactly pq_quantize_bwd's (from W, alpha and
 * G before the update); the outputs Wq / codes are exactly
 * pq_quantize_fwd's for the updated W and alpha.
 */
typedef struct pq_adamw {
    double lr;            /* this step's learning rate (the schedule is the caller's) */
    double beta1, beta2;  /* in [0, 1) */
    double eps;           /* > 0 */
    double weight_decay;  /* >= 0 (the recipe uses 0) */
    int64_t step;         /* t >= 1, for the bias corrections */
} pq_adamw;

/* One matrix of a fused step (grouped launches, as pq_mat). */
typedef struct pq_step_mat {
    float *W;             /* in/out [rows, cols] fp32 shadow weights        */
    float *alpha;         /* in/out [rows] fp32 scale                       */
    const void *G;        /* in [rows, cols] dL/dWq (dtype per call)        */
    float *mW;            /* in/out [rows, cols] first moment of W          */
    float *vW;            /* in/out [rows, cols] second moment of W         */
    float *m_alpha;       /* in/out [rows] first moment of alpha            */
    float *v_alpha;       /* in/out [rows] second moment of alpha           */
    void *wq_bf16;        /* out [rows, cols] next forward's bf16, or NULL  */
    uint8_t *codes;       /* out [rows, pq_code_row_bytes] codes, or NULL   */
    float *dalpha;        /* out [rows] this step's alpha gradient, or NULL */
    double grad_scale;    /* the alpha-gradient scale, as pq_quantize_bwd   */
    int64_t rows;
    int64_t cols;         /* positive multiple of 8                         */
} pq_step_mat;

/*
 * pq_qat_step -- the fused step on one matrix.  W, alpha and the four moment
 * arrays are updated in place; G is read only.  Wq_bf16, codes and dalpha
 * are optional outputs (NULL skips them).  hp is a host pointer read during
 * the call.  Errors as the other entry points; hp NULL -> PQ_ERR_NULL; a
 * hyper-parameter out of its range (or a non-finite one), or a non-finite
 * grad_scale -> PQ_ERR_ARG.  Weights, moments and gradients must be finite.
 */
pq_status pq_qat_step(int mode, int64_t rows, int64_t cols, float *W, float *alpha,
                      const void *G, int g_dtype, double grad_scale, float *mW, float *vW,
                      float *m_alpha, float *v_alpha, const pq_adamw *hp, void *Wq_bf16,
                      uint8_t *codes, float *dalpha, void *stream);

/* The fused step over `count` matrices in one launch; per matrix exactly
 * pq_qat_step.  descs_host / descs_dev: identical pq_step_mat[count] in host
 * / device memory; every entry must use the same set of optional outputs. */
pq_status pq_qat_step_grouped(int mode, int count, const pq_step_mat *descs_host,
                              const pq_step_mat *descs_dev, int g_dtype, const pq_adamw *hp,
                              void *stream);

/*
 * Diagnostics.  How the weights of each row spread over the levels -- the
 * level occupancy behind the SEQ-vs-LSQ argument ([Rebuttal], part on why
 * SEQ beats LSQ; [Note] "Finding 3" level sets) -- and how far training
 * moved the shadow weights from a reference ([Note] "QAT versus PTQ": QAT
 * compensates for the quantizer rather than reconstructing the weights).
 *
 * pq_num_levels -- levels of a mode (2, 3, 4, 8, 16 for 1, 1.58, 2, 3, 4
 * bits; 4 and 3 for the 2- and 1.58-bit LSQ grids), -1 for a bad mode.
 *
 * pq_level_stats -- from the forward's row-major codes ([rows,
 * pq_code_row_bytes(mode, cols)]): counts [rows, pq_num_levels(mode)] u32,
 * counts[i, c] = weights of row i stored with code c (code c is level c,
 * lowest first), and optionally entropy [rows] f64, -sum_c p_c log2 p_c with
 * p_c = counts[i, c] / cols (binary64; 0 for a row on one level).  Reads
 * 1/8 .. 1/2 byte per weight.
 *
 * pq_quantize_fwd_stats -- the forward of pq_quantize_fwd (alpha given, no
 * init) with the level statistics of pq_level_stats taken in the same pass,
 * from the codes as they are made: codes [rows, pq_code_row_bytes] are
 * written (required), Wq_bf16 [rows, cols] optionally (NULL: not written),
 * counts [rows, pq_num_levels(mode)] u32 (required) and entropy [rows] f64
 * (optional) as pq_level_stats defines them.  All pointers 16-byte aligned.
 * Errors as pq_quantize_fwd; codes or counts NULL -> PQ_ERR_NULL.
 *
 * pq_weight_movement -- sq_diff[i] = sum_j (W[i,j] - W0[i,j])^2 and
 * sq_ref[i] = sum_j W0[i,j]^2 per row, each difference and square in
 * binary64, summed in a fixed order (run-to-run identical); the relative
 * movement of a matrix is sqrt(sum sq_diff / sum sq_ref).  W, W0 fp32
 * [rows, cols] (16-byte aligned), outputs f64 [rows].
 */
int pq_num_levels(int mode);
pq_status pq_level_stats(int mode, int64_t rows, int64_t cols, const uint8_t *codes,
                         uint32_t *counts, double *entropy, void *stream);
pq_status pq_quantize_fwd_stats(int mode, int64_t rows, int64_t cols, const float *W,
                                const float *alpha, void *Wq_bf16, uint8_t *codes,
                                uint32_t *counts, double *entropy, void *stream);
pq_status pq_weight_movement(int64_t rows, int64_t cols, const float *W, const float *W0,
                             double *sq_diff, double *sq_ref, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PQ_H_ */
