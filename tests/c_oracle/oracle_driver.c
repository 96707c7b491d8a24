/* Drives every entry point of the plain-C oracle (oracle/lmh_oracle.c) on
 * small, ragged, seeded inputs.  tests/test_oracle_sanitized.py builds it
 * together with the oracle under gcc's address and undefined-behaviour
 * sanitizers, so an out-of-bounds access, a use of freed memory or undefined
 * arithmetic anywhere in the oracle fails the build's run.  The checks here
 * are only what holds at any size (return codes, range of the codes, pack and
 * unpack round trips, top-K order); the oracle's values are pinned by the
 * other tests. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int orc_quantize(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t G,
                 int scale_dtype, const double* ratios, int nratios, int8_t* q_out,
                 uint16_t* s_out, int8_t* pick_out);
int orc_quantize_asym(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t G,
                      int scale_dtype, uint8_t* n_out, uint16_t* s_out, uint8_t* z_out);
int64_t orc_packed_bytes(int64_t V, int64_t K, int bits, int64_t G);
int orc_pack(const int8_t* q, const uint16_t* s, int64_t V, int64_t K, int bits, int64_t G,
             uint8_t* out);
int orc_unpack(const uint8_t* blob, int64_t V, int64_t K, int bits, int64_t G, int8_t* q,
               uint16_t* s);
int64_t orc_packed_bytes_zp(int64_t V, int64_t K, int bits, int64_t G);
int orc_pack_zp(const uint8_t* n, const uint16_t* s, const uint8_t* z, int64_t V, int64_t K,
                int bits, int64_t G, uint8_t* out);
int orc_unpack_zp(const uint8_t* blob, int64_t V, int64_t K, int bits, int64_t G, uint8_t* n,
                  uint16_t* s, uint8_t* z);
int orc_logits(const void* x, int x_dtype, int64_t M, const int8_t* q, const uint16_t* s,
               int scale_dtype, int64_t V, int64_t K, int64_t G, const float* bias,
               const int64_t* rows, int64_t nrows, double* y);
int orc_logits_zp(const void* x, int x_dtype, int64_t M, const uint8_t* n, const uint16_t* s,
                  const uint8_t* z, int scale_dtype, int64_t V, int64_t K, int64_t G,
                  const float* bias, const int64_t* rows, int64_t nrows, double* y);
int orc_embed(const int8_t* q, const uint16_t* s, int scale_dtype, int64_t V, int64_t K,
              int64_t G, const int32_t* ids, int64_t T, int out_dtype, void* out);
int orc_embed_zp(const uint8_t* n, const uint16_t* s, const uint8_t* z, int scale_dtype,
                 int64_t V, int64_t K, int64_t G, const int32_t* ids, int64_t T, int out_dtype,
                 void* out);
int orc_dense_logits(const void* x, int x_dtype, int64_t M, const void* w, int w_dtype, int64_t V,
                     int64_t K, const int64_t* rows, int64_t nrows, double* y);
int orc_topk(const float* y, int64_t V, int topk, int64_t* idx);
int orc_topk_rescore(const float* y, int64_t ldy, int64_t M, int64_t V, int topk, const void* x,
                     int x_dtype, const void* w, int w_dtype, int64_t K, int64_t* idx_out,
                     double* val_out, int64_t* top1_out);
uint16_t orc_f32_to_f16(float f);
uint16_t orc_f32_to_bf16(float f);
void orc_f32_to_f16_array(const float* in, int64_t n, uint16_t* out);
void orc_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out);
void orc_f16_to_f32_array(const uint16_t* in, int64_t n, float* out);
void orc_bf16_to_f32_array(const uint16_t* in, int64_t n, float* out);

enum { F32 = 0, F16 = 1, BF16 = 2 };

static int failures = 0;
#define CHECK(c, ...)                                      \
    do {                                                   \
        if (!(c)) {                                        \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                  \
            fprintf(stderr, "\n");                         \
            ++failures;                                    \
        }                                                  \
    } while (0)

/* xorshift64*, uniform in [-1, 1) */
static uint64_t rng = 0x9E3779B97F4A7C15ull;
static float urand(void) {
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (float)((double)((rng * 2685821657736338717ull) >> 11) / 4503599627370496.0 - 1.0);
}

/* V x K weights of type w_dtype (exact sizes: every buffer malloc'd to its
 * length, so the sanitizer sees any read past it); rows 0 and V - 1 zero */
static void* make_weights(int64_t V, int64_t K, int w_dtype) {
    float* f = malloc((size_t)(V * K) * sizeof(float));
    for (int64_t i = 0; i < V * K; ++i) f[i] = 0.02f * urand();
    for (int64_t k = 0; k < K; ++k) f[k] = f[(V - 1) * K + k] = 0.0f;
    f[K + 3] = 0.5f; /* an outlier */
    if (w_dtype == F32) return f;
    uint16_t* h = malloc((size_t)(V * K) * sizeof(uint16_t));
    if (w_dtype == F16) orc_f32_to_f16_array(f, V * K, h);
    else orc_f32_to_bf16_array(f, V * K, h);
    free(f);
    return h;
}

static void* make_x(int64_t M, int64_t K, int x_dtype) {
    float* f = malloc((size_t)(M * K) * sizeof(float));
    for (int64_t i = 0; i < M * K; ++i) f[i] = urand();
    if (x_dtype == F32) return f;
    uint16_t* h = malloc((size_t)(M * K) * sizeof(uint16_t));
    if (x_dtype == F16) orc_f32_to_f16_array(f, M * K, h);
    else orc_f32_to_bf16_array(f, M * K, h);
    free(f);
    return h;
}

static void run_symmetric(int64_t V, int64_t K, int bits, int64_t G, int w_dtype, int sdt,
                          int nratios) {
    static const double ratios[5] = {1.0, 0.95, 0.9, 0.85, 0.8};
    const int64_t NG = K / G, M = 3;
    void* w = make_weights(V, K, w_dtype);
    int8_t* q = malloc((size_t)(V * K));
    uint16_t* s = malloc((size_t)(V * NG) * sizeof(uint16_t));
    int8_t* pick = malloc((size_t)(V * NG));
    CHECK(orc_quantize(w, w_dtype, V, K, bits, G, sdt, ratios, nratios, q, s, pick) == 0,
          "quantize V=%lld K=%lld bits=%d G=%lld", (long long)V, (long long)K, bits, (long long)G);
    const int qlo = bits == 4 ? -8 : -128, qhi = bits == 4 ? 7 : 127;
    for (int64_t i = 0; i < V * K; ++i) CHECK(q[i] >= qlo && q[i] <= qhi, "code range");
    for (int64_t i = 0; i < V * NG; ++i) CHECK(pick[i] >= 0 && pick[i] < nratios, "pick range");

    const int64_t nb = orc_packed_bytes(V, K, bits, G);
    CHECK(nb > 0, "packed bytes");
    uint8_t* blob = malloc((size_t)nb);
    CHECK(orc_pack(q, s, V, K, bits, G, blob) == 0, "pack");
    int8_t* q2 = malloc((size_t)(V * K));
    uint16_t* s2 = malloc((size_t)(V * NG) * sizeof(uint16_t));
    CHECK(orc_unpack(blob, V, K, bits, G, q2, s2) == 0, "unpack");
    CHECK(memcmp(q, q2, (size_t)(V * K)) == 0, "codes round trip");
    CHECK(memcmp(s, s2, (size_t)(V * NG) * sizeof(uint16_t)) == 0, "scales round trip");

    for (int xdt = F16; xdt <= BF16; ++xdt) {
        void* x = make_x(M, K, xdt);
        float* bias = malloc((size_t)V * sizeof(float));
        for (int64_t v = 0; v < V; ++v) bias[v] = 0.1f * urand();
        double* y = malloc((size_t)(M * V) * sizeof(double));
        CHECK(orc_logits(x, xdt, M, q, s, sdt, V, K, G, bias, NULL, V, y) == 0, "logits");
        for (int64_t m = 0; m < M; ++m) CHECK(y[m * V] == (double)bias[0], "zero row gives its bias");
        const int64_t rows[3] = {V - 1, 0, V / 2};
        double* yr = malloc((size_t)(M * 3) * sizeof(double));
        CHECK(orc_logits(x, xdt, M, q, s, sdt, V, K, G, NULL, rows, 3, yr) == 0, "logits rows");
        /* dense logits and top-K rescoring against the unquantized weights */
        double* yd = malloc((size_t)(M * V) * sizeof(double));
        CHECK(orc_dense_logits(x, xdt, M, w, w_dtype, V, K, NULL, V, yd) == 0, "dense logits");
        float* yf = malloc((size_t)(M * V) * sizeof(float));
        for (int64_t i = 0; i < M * V; ++i) yf[i] = (float)y[i];
        const int topk = 5;
        int64_t* idx = malloc((size_t)topk * sizeof(int64_t));
        CHECK(orc_topk(yf, V, topk, idx) == 0, "topk");
        for (int i = 0; i + 1 < topk; ++i) CHECK(yf[idx[i]] >= yf[idx[i + 1]], "topk order");
        int64_t* idx2 = malloc((size_t)(M * topk) * sizeof(int64_t));
        double* val = malloc((size_t)(M * topk) * sizeof(double));
        int64_t* top1 = malloc((size_t)M * sizeof(int64_t));
        if (w_dtype != F32) {
            CHECK(orc_topk_rescore(yf, V, M, V, topk, x, xdt, w, w_dtype, K, idx2, val, top1) == 0,
                  "topk rescore");
            for (int64_t m = 0; m < M; ++m) CHECK(top1[m] >= 0 && top1[m] < V, "top1 range");
        }
        /* embedding rows, in each output type */
        int32_t ids[4] = {0, (int32_t)(V - 1), 1, (int32_t)(V / 3)};
        for (int odt = F32; odt <= BF16; ++odt) {
            void* e = malloc((size_t)(4 * K) * (odt == F32 ? 4 : 2));
            CHECK(orc_embed(q, s, sdt, V, K, G, ids, 4, odt, e) == 0, "embed");
            free(e);
        }
        free(x), free(bias), free(y), free(yr), free(yd), free(yf), free(idx), free(idx2), free(val),
            free(top1);
    }
    free(w), free(q), free(s), free(pick), free(blob), free(q2), free(s2);
}

static void run_asym(int64_t V, int64_t K, int bits, int64_t G, int w_dtype, int sdt) {
    const int64_t NG = K / G, M = 2;
    void* w = make_weights(V, K, w_dtype);
    uint8_t* n = malloc((size_t)(V * K));
    uint16_t* s = malloc((size_t)(V * NG) * sizeof(uint16_t));
    uint8_t* z = malloc((size_t)(V * NG));
    CHECK(orc_quantize_asym(w, w_dtype, V, K, bits, G, sdt, n, s, z) == 0, "quantize zp");
    const int qr = bits == 4 ? 15 : 255;
    for (int64_t i = 0; i < V * K; ++i) CHECK(n[i] <= qr, "zp code range");
    const int64_t nb = orc_packed_bytes_zp(V, K, bits, G);
    uint8_t* blob = malloc((size_t)nb);
    CHECK(orc_pack_zp(n, s, z, V, K, bits, G, blob) == 0, "pack zp");
    uint8_t* n2 = malloc((size_t)(V * K));
    uint16_t* s2 = malloc((size_t)(V * NG) * sizeof(uint16_t));
    uint8_t* z2 = malloc((size_t)(V * NG));
    CHECK(orc_unpack_zp(blob, V, K, bits, G, n2, s2, z2) == 0, "unpack zp");
    CHECK(memcmp(n, n2, (size_t)(V * K)) == 0 && memcmp(z, z2, (size_t)(V * NG)) == 0 &&
              memcmp(s, s2, (size_t)(V * NG) * sizeof(uint16_t)) == 0,
          "zp round trip");
    void* x = make_x(M, K, F16);
    double* y = malloc((size_t)(M * V) * sizeof(double));
    CHECK(orc_logits_zp(x, F16, M, n, s, z, sdt, V, K, G, NULL, NULL, V, y) == 0, "logits zp");
    for (int64_t m = 0; m < M; ++m) CHECK(y[m * V] == 0.0, "zero row gives zero");
    int32_t ids[3] = {(int32_t)(V - 1), 0, 2};
    void* e = malloc((size_t)(3 * K) * 2);
    CHECK(orc_embed_zp(n, s, z, sdt, V, K, G, ids, 3, F16, e) == 0, "embed zp");
    free(w), free(n), free(s), free(z), free(blob), free(n2), free(s2), free(z2), free(x), free(y),
        free(e);
}

int main(void) {
    /* ragged row counts (not multiples of 64), both code widths, groups
     * shorter than, equal to and longer than a superchunk, one scale per row */
    const int64_t Vs[2] = {67, 130};
    for (int vi = 0; vi < 2; ++vi) {
        const int64_t V = Vs[vi];
        run_symmetric(V, 256, 4, 64, F32, F16, 1);
        run_symmetric(V, 256, 4, 256, BF16, BF16, 5);
        run_symmetric(V, 256, 8, 32, F16, F16, 5);
        run_symmetric(V, 384, 8, 128, BF16, F16, 1);
        run_symmetric(V, 128, 4, 128, F16, BF16, 5);
        run_asym(V, 256, 4, 64, F32, F16);
        run_asym(V, 128, 8, 128, BF16, BF16);
    }
    /* argument errors are reported, not acted on */
    CHECK(orc_pack(NULL, NULL, 64, 128, 4, 64, NULL) != 0, "null arguments rejected");
    CHECK(orc_topk(NULL, 10, 3, NULL) != 0, "null top-K rejected");
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: all entry points ran clean\n");
    return 0;
}
