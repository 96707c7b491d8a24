/* The C ABI from plain C (no GPU needed): the header compiles as C, the
 * library links, and sizes, the automatic kernel choice and argument
 * validation answer as include/lmhead.h documents -- before any device work. */
#include <stdio.h>
#include <string.h>

#include "lmhead.h"

#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) {                                                       \
            fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__);      \
            return 1;                                                     \
        }                                                                 \
    } while (0)

int main(void) {
    const size_t V = 151936, K = 1024;
    CHECK(lmhead_abi_version() == 2);
    /* 151936 x 1024 int4 g64: codes V*K/2, fp16 scales V*(K/64)*2, zero points V*(K/64) */
    CHECK(lmhead_packed_bytes(V, K, 4, 64) == V * K / 2 + V * (K / 64) * 2);
    CHECK(lmhead_packed_bytes(V, K, 4 | LMH_ZP, 64) == V * K / 2 + V * (K / 64) * 3);
    CHECK(lmhead_packed_bytes(V, K, 8, 128) == V * K + V * (K / 128) * 2);
    CHECK(lmhead_packed_bytes(100, 100, 4, 64) == 0); /* K not a whole number of superchunks */
    int path = -1;
    CHECK(lmhead_logits_auto_path_x(1, 1024, 4, 64, LMH_F16, &path) == LMH_OK && path == 1);
    CHECK(lmhead_logits_auto_path_x(2, 1024, 4, 64, LMH_F16, &path) == LMH_OK && path == 5);
    CHECK(lmhead_logits_auto_path_x(2, 1024, 4, 64, LMH_BF16, &path) == LMH_OK && path == 1);
    CHECK(lmhead_logits_auto_path_x(256, 1024, 4, 64, LMH_F16, &path) == LMH_OK && path == 4);
    CHECK(lmhead_logits_auto_path(256, 1024, 4, 64, &path) == LMH_OK && path == 4);
    path = -1;
    CHECK(lmhead_logits_auto_path(0, 1024, 4, 64, &path) == LMH_E_SHAPE && path == -1);
    CHECK(lmhead_logits_auto_path_x(1, 1024, 4, 64, LMH_F32, &path) == LMH_E_DTYPE);
    /* validation runs before any device work: no x for a nonempty request */
    float y[64];
    CHECK(lmhead_logits(NULL, LMH_F16, 1, (const void*)y, 64, 128, 4, 64, LMH_F16, NULL, y, 64,
                        NULL, 0, NULL) == LMH_E_NULL);
    CHECK(lmhead_logits(y, LMH_F16, 0, y, 64, 128, 4, 64, LMH_F16, NULL, y, 64, NULL, 0, NULL) ==
          LMH_OK); /* M = 0: nothing to do */
    CHECK(lmhead_quantize(NULL, LMH_F32, 64, 100, 4, 64, LMH_F16, LMH_CLIP_RTN, NULL, NULL, NULL) ==
          LMH_E_SHAPE);
    CHECK(strncmp(lmhead_status_string(LMH_E_SHAPE), "LMH_E_SHAPE", 11) == 0);
    CHECK(strstr(lmhead_status_string(1234), "unknown") != NULL);
    printf("c host abi ok\n");
    return 0;
}
