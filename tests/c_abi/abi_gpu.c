/* The C ABI from plain C on the GPU: a small head quantized, packed (two
 * steps and fused), and its logits computed by every kernel path, using only
 * the HIP runtime's C API for memory.  Checks: the fused blob equals the
 * two-step blob byte for byte; the register-fed, LDS-staged and
 * activation-resident kernels give identical bits; every path lies within the
 * fp32 summation bound (K + K/G + 16) 2^-24 sum|x q s| of the exact sum,
 * taken in double from the codes and scales the library returned. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lmhead.h"

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__);      \
            return 1;                                                     \
        }                                                                 \
    } while (0)
#define HIPCHECK(c) CHECK((c) == hipSuccess)

enum { V = 200, K = 512, G = 64, M = 3, NG = K / G };

static double half_value(uint16_t h) {
    const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    const double v = e == 0 ? ldexp(m, -24) : ldexp(m + 1024, e - 25);
    return s ? -v : v;
}

/* fp16 bits of v, which must be zero or a normal fp16 value exactly */
static uint16_t half_bits(double v) {
    if (v == 0) return 0;
    const uint16_t sgn = v < 0 ? 0x8000 : 0;
    int E;
    const double f = frexp(fabs(v), &E); /* |v| = f 2^E, f in [0.5, 1) */
    return (uint16_t)(sgn | ((E + 14) << 10) | (int)((2 * f - 1) * 1024));
}

int main(void) {
    static float w[V * K];
    static uint16_t xh[M * K];
    static double xd[M * K];
    uint32_t state = 12345u;
    for (int i = 0; i < V * K; ++i) { /* a seeded LCG, values in [-0.05, 0.05) */
        state = state * 1664525u + 1013904223u;
        w[i] = (float)(((double)(state >> 8) / 16777216.0 - 0.5) * 0.1);
    }
    for (int i = 0; i < M * K; ++i) { /* x = k / 8, k in [-32, 32]: exact in fp16 */
        state = state * 1664525u + 1013904223u;
        xd[i] = (double)((int)(state >> 26) - 32) / 8.0;
        xh[i] = half_bits(xd[i]);
    }
    const size_t nb = lmhead_packed_bytes(V, K, 4, G);
    CHECK(nb > 0);
    void *dw, *dq, *ds, *dblob, *dfused, *dx, *dy;
    HIPCHECK(hipMalloc(&dw, sizeof(w)));
    HIPCHECK(hipMalloc(&dq, (size_t)V * K));
    HIPCHECK(hipMalloc(&ds, (size_t)V * NG * 2));
    HIPCHECK(hipMalloc(&dblob, nb));
    HIPCHECK(hipMalloc(&dfused, nb));
    HIPCHECK(hipMalloc(&dx, sizeof(xh)));
    HIPCHECK(hipMalloc(&dy, (size_t)6 * M * V * 4));
    HIPCHECK(hipMemcpy(dw, w, sizeof(w), hipMemcpyHostToDevice));
    HIPCHECK(hipMemcpy(dx, xh, sizeof(xh), hipMemcpyHostToDevice));

    CHECK(lmhead_quantize(dw, LMH_F32, V, K, 4, G, LMH_F16, LMH_CLIP_RTN, (int8_t*)dq, ds, NULL) ==
          LMH_OK);
    CHECK(lmhead_pack((const int8_t*)dq, ds, V, K, 4, G, dblob, NULL) == LMH_OK);
    CHECK(lmhead_quantize_pack(dw, LMH_F32, K, V, K, 4, G, LMH_F16, LMH_CLIP_RTN, 0, V, dfused,
                               NULL) == LMH_OK);
    /* paths 0 (automatic) .. 5 into six output buffers */
    for (int p = 0; p <= 5; ++p)
        CHECK(lmhead_logits_path(dx, LMH_F16, M, dblob, V, K, 4, G, LMH_F16, NULL,
                                 (float*)dy + (size_t)p * M * V, V, NULL, 0, p, NULL) == LMH_OK);
    HIPCHECK(hipDeviceSynchronize());

    static int8_t q[V * K];
    static uint16_t s[V * NG];
    static unsigned char blob[1 << 20], fused[1 << 20];
    static float y[6 * M * V];
    CHECK(nb <= sizeof(blob));
    HIPCHECK(hipMemcpy(q, dq, sizeof(q), hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(s, ds, sizeof(s), hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(blob, dblob, nb, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(fused, dfused, nb, hipMemcpyDeviceToHost));
    HIPCHECK(hipMemcpy(y, dy, sizeof(y), hipMemcpyDeviceToHost));
    CHECK(memcmp(blob, fused, nb) == 0);
    for (int i = 0; i < V * K; ++i) CHECK(q[i] >= -8 && q[i] <= 7);
    /* the register-fed (2), LDS-staged (3) and activation-resident (4) kernels agree bit for bit */
    CHECK(memcmp(y + 2 * M * V, y + 3 * M * V, sizeof(float) * M * V) == 0);
    CHECK(memcmp(y + 2 * M * V, y + 4 * M * V, sizeof(float) * M * V) == 0);
    for (int m = 0; m < M; ++m)
        for (int v = 0; v < V; ++v) {
            double exact = 0, mag = 0;
            for (int k = 0; k < K; ++k) {
                const double t = xd[m * K + k] * q[v * K + k] * half_value(s[v * NG + k / G]);
                exact += t;
                mag += fabs(t);
            }
            const double bound = (K + K / G + 16) * ldexp(1.0, -24) * mag + 1e-30;
            for (int p = 0; p <= 5; ++p) CHECK(fabs(y[(p * M + m) * V + v] - exact) <= bound);
        }
    hipFree(dw); hipFree(dq); hipFree(ds); hipFree(dblob); hipFree(dfused); hipFree(dx); hipFree(dy);
    printf("c gpu abi ok\n");
    return 0;
}
