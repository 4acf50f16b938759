/* Exercise every entry point of the CPU oracle on small ragged inputs, for
 * a build under AddressSanitizer and UndefinedBehaviorSanitizer (host code
 * only): any out-of-bounds access, use of uninitialised heap, signed
 * overflow or bad shift in the oracle aborts the run.  Prints "ok" and
 * returns 0 when every call succeeds. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int pqo_code_bits(int mode);
int64_t pqo_code_row_bytes(int mode, int64_t cols);
int pqo_alpha_init(int mode, int64_t rows, int64_t cols, const float *W, float *alpha);
int pqo_quantize_fwd(int mode, int64_t rows, int64_t cols, const float *W, const float *alpha,
                     uint16_t *wq_bf16, float *wq_f32, uint8_t *codes);
double pqo_default_grad_scale(int mode, int64_t rows, int64_t cols);
int pqo_quantize_bwd(int mode, int64_t rows, int64_t cols, const float *W, const float *alpha,
                     const void *G, int g_is_bf16, double grad_scale, float *dW, float *dalpha,
                     uint8_t *mask_bits);
int pqo_pack(int mode, int64_t rows, int64_t cols, const float *W, const float *alpha,
             uint8_t *packed, uint16_t *alpha_bf16);
int pqo_qat_step(int mode, int64_t rows, int64_t cols, float *W, float *alpha, const void *G,
                 int g_is_bf16, double grad_scale, float *mW, float *vW, float *m_alpha,
                 float *v_alpha, double lr, double b1, double b2, double eps, double wd,
                 int64_t t, uint16_t *wq_bf16, uint8_t *codes, float *dalpha_out);
int pqo_num_levels(int mode);
int pqo_level_stats(int mode, int64_t rows, int64_t cols, const uint8_t *codes, uint32_t *counts,
                    double *entropy);
int pqo_weight_movement(int64_t rows, int64_t cols, const float *W, const float *W0, double *sq_diff,
                        double *sq_ref);
int64_t pqo_tiled_bytes(int64_t rows, int64_t rb);
int pqo_tile_codes(int cw, int64_t rows, int64_t rb, const uint8_t *rowmajor, uint8_t *tiled);
int pqo_gemm_ref(int mode, int64_t M, int64_t N, int64_t K, const uint16_t *X, const uint8_t *packed,
                 const uint16_t *alpha_bf16, double *Y);
int pqo_gemm_ref_f32a(int mode, int64_t M, int64_t N, int64_t K, const uint16_t *X,
                      const uint8_t *packed, const float *alpha, double *Y);
int pqo_gemm_ref_at(int mode, int64_t M, int64_t N, int64_t K, const uint16_t *X,
                    const uint8_t *packed, const uint16_t *alpha_bf16, const int64_t *ms,
                    const int64_t *ns, int64_t count, double *out);

static uint64_t state = 0x9E3779B97F4A7C15ull;

static double uniform(void)
{
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return (double)(state >> 11) / 9007199254740992.0;
}

static float randn(void)
{
    double s = 0.0;
    for (int i = 0; i < 12; ++i) s += uniform();
    return (float)(s - 6.0);
}

/* Exactly-sized heap arrays, so that the sanitizer sees any access past them. */
#define ALLOC(T, n) ((T *)malloc((size_t)(n) * sizeof(T) + ((n) == 0)))

#define CHECK(call)                                                  \
    do {                                                             \
        if ((call) != 0) {                                           \
            fprintf(stderr, "failed: %s (mode %d, %lld x %lld)\n", #call, mode, (long long)rows, (long long)cols); \
            return 1;                                                \
        }                                                            \
    } while (0)

static int one_case(int mode, int64_t rows, int64_t cols, int g_bf16)
{
    const int64_t n = rows * cols, rb = pqo_code_row_bytes(mode, cols), mb = (cols + 7) / 8;
    float *W = ALLOC(float, n), *G = ALLOC(float, n), *alpha = ALLOC(float, rows);
    uint16_t *Gh = ALLOC(uint16_t, n), *wq = ALLOC(uint16_t, n), *ab = ALLOC(uint16_t, rows);
    float *wq32 = ALLOC(float, n), *dW = ALLOC(float, n), *da = ALLOC(float, rows);
    uint8_t *codes = ALLOC(uint8_t, rows * rb), *mask = ALLOC(uint8_t, rows * mb);
    for (int64_t i = 0; i < n; ++i) {
        W[i] = 0.02f * randn();
        G[i] = randn();
        uint32_t b;
        memcpy(&b, &G[i], 4);
        Gh[i] = (uint16_t)(b >> 16);
    }
    if (rows > 0) W[0] = -0.0f;
    CHECK(pqo_alpha_init(mode, rows, cols, W, alpha));
    CHECK(pqo_quantize_fwd(mode, rows, cols, W, alpha, wq, wq32, codes));
    CHECK(pqo_quantize_bwd(mode, rows, cols, W, alpha, g_bf16 ? (const void *)Gh : (const void *)G, g_bf16,
                           pqo_default_grad_scale(mode, rows, cols), dW, da, mask));
    const int L = pqo_num_levels(mode);
    uint32_t *counts = ALLOC(uint32_t, rows * L);
    double *ent = ALLOC(double, rows), *d2 = ALLOC(double, rows), *r2 = ALLOC(double, rows);
    CHECK(pqo_level_stats(mode, rows, cols, codes, counts, ent));
    CHECK(pqo_weight_movement(rows, cols, W, wq32, d2, r2));
    /* export and GEMM (every mode has a deployment container) */
    CHECK(pqo_pack(mode, rows, cols, W, alpha, codes, ab));
    const int64_t tb = pqo_tiled_bytes(rows, rb);
    uint8_t *tiled = ALLOC(uint8_t, tb);
    CHECK(pqo_tile_codes(pqo_code_bits(mode), rows, rb, codes, tiled));
    const int64_t M = 3;
    uint16_t *X = ALLOC(uint16_t, M * cols);
    for (int64_t i = 0; i < M * cols; ++i) X[i] = Gh[i % (n > 0 ? n : 1)];
    double *Y = ALLOC(double, M * rows), *Y2 = ALLOC(double, M * rows), *Ys = ALLOC(double, 4);
    if (cols % 64 == 0) {
        CHECK(pqo_gemm_ref(mode, M, rows, cols, X, codes, ab, Y));
        CHECK(pqo_gemm_ref_f32a(mode, M, rows, cols, X, codes, alpha, Y2));
        int64_t ms[4] = {0, M - 1, 1, 2}, ns[4] = {0, rows - 1, rows / 2, rows - 1};
        CHECK(pqo_gemm_ref_at(mode, M, rows, cols, X, codes, ab, ms, ns, 4, Ys));
    }
    /* one fused step from zero moments */
    float *mW = ALLOC(float, n), *vW = ALLOC(float, n), *ma = ALLOC(float, rows), *va = ALLOC(float, rows);
    memset(mW, 0, (size_t)n * 4);
    memset(vW, 0, (size_t)n * 4);
    memset(ma, 0, (size_t)rows * 4);
    memset(va, 0, (size_t)rows * 4);
    CHECK(pqo_qat_step(mode, rows, cols, W, alpha, G, 0, pqo_default_grad_scale(mode, rows, cols), mW, vW, ma,
                       va, 1e-3, 0.9, 0.999, 1e-8, 0.01, 1, wq, codes, da));
    free(W); free(G); free(alpha); free(Gh); free(wq); free(ab); free(wq32); free(dW); free(da);
    free(codes); free(mask); free(counts); free(ent); free(d2); free(r2); free(tiled); free(X);
    free(Y); free(Y2); free(Ys); free(mW); free(vW); free(ma); free(va);
    return 0;
}

int main(void)
{
    static const int64_t shapes[][2] = {{1, 8}, {3, 8}, {5, 64}, {17, 72}, {16, 128}, {33, 192}, {2, 1600}};
    for (int mode = 0; mode < 7; ++mode)
        for (size_t s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
            for (int gb = 0; gb < 2; ++gb)
                if (one_case(mode, shapes[s][0], shapes[s][1], gb) != 0) return 1;
    printf("ok\n");
    return 0;
}
