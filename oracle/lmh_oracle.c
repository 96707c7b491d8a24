/*
 * lmh_oracle.c -- the oracle for the weight-only-quantized LM-head path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file: only the tests, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no source, header, table or constant
 * generator with the GPU library.
 *
 * What it computes, and where that is defined:
 *   - 16-bit float codecs (IEEE-754 binary16 and bfloat16, round to nearest,
 *     ties to even), written from the format definitions;
 *   - the load-time quantizer: symmetric per-group round-to-nearest, optionally
 *     with the least-squared-error clip-ratio search, the scale rounded to the
 *     16-bit scale type before q is chosen (page "radiance_lmhead_int4.py":
 *     docstring "How" paragraph, module constants, quantize_int4_rows);
 *   - the asymmetric variant: unsigned codes with a per-group zero point
 *     (reading R21: plain min/max round-to-nearest, zero kept exact), its
 *     packed form (an extra zero-point region), logits and embedding rows;
 *   - the packed blob layout (our own gfx950 layout; the byte-level definition
 *     is in include/lmhead.h and restated in the comments below);
 *   - logits y[m,v] = sum_k x[m,k] * q[v,k] * s[v,k/G] (+ bias[v]), exact
 *     products, fp64 sums (vLLM PR #48870 "Fused WNA16 GEMM for tied quantized
 *     lm_head logits", Purpose: the fused dequant-GEMM computes the same logits
 *     as dequantize-then-F.linear);
 *   - embedding rows q[v,k] * s[v,k/G] gathered by token id from the same
 *     quantized table (same page, Purpose: the tied embedding's table serves
 *     both the input lookup and the lm_head);
 *   - dense logits x * W_ref^T in fp64 (the unquantized control, same page,
 *     review comment point 1);
 *   - top-K selection and exact rescoring of the K rows from the unquantized
 *     weight (same page, review comment point 2).
 *
 * Arithmetic rules: fp32 steps are IEEE single precision (build with
 * -O2 -ffp-contract=off, never -ffast-math); fp64 sums are sequential in
 * ascending index order.  Everything is single-threaded and unblocked.
 *
 * Readings of the pages that are not stated there (referred to below, in
 * oracle/__init__.py and in the tests by these tags):
 *   R1 an all-zero group gets scale 0 and q = 0 (the page clamps the scale to
 *      1e-8 instead; the logits are 0 either way);
 *   R2 the scale floor is 1e-8f for bf16 scales and 2^-24 (smallest fp16
 *      subnormal) for fp16 scales, so a non-zero group never gets scale 0;
 *   R3 int8 uses qmax = 127, qmin = -128; int4 uses qmax = 7, qmin = -8;
 *   R4 the clip-search error is accumulated in fp64, k ascending, one fused
 *      multiply-add per element (the page sums in fp32 in torch's unspecified
 *      order);
 *   R5 top-K order is value descending, then index ascending; the top-1 after
 *      rescoring is the first maximum of the whole scattered vector;
 *   R7 the scale is fl32(amax * fl32(r / qmax)), the page's literal form;
 *   R21 the asymmetric form: the pages name it (a per-group zero point in place
 *      of the module's fixed nibble offset 8; an asymmetric lm_head checkpoint)
 *      but give no quantizer for it, so it is plain min/max round-to-nearest
 *      over [min(0, min w), max(0, max w)] with the scale rules of R2/R7 and a
 *      rounded, clamped zero point; no clip search.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2

#define ORC_OK 0
#define ORC_EARG 1

/* ------------------------------------------------------------------------ */
/* 16-bit binary floating point formats.                                      */
/* A format with `mb` stored mantissa bits and exponent bias `bias` encodes   */
/*   exp field e in [1, 2*bias]: (-1)^s * 2^(e - bias) * (1 + m / 2^mb)       */
/*   exp field 0:               (-1)^s * 2^(1 - bias) * (m / 2^mb)            */
/*   exp field 2*bias+1:        infinity (m == 0) or NaN (m != 0).            */
/* binary16: mb = 10, bias = 15.  bfloat16: mb = 7, bias = 127.               */
/* ------------------------------------------------------------------------ */

static uint16_t enc16(float f, int mb, int bias) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    int emax_field = 2 * bias + 1; /* all-ones exponent field */
    uint16_t inf_bits = (uint16_t)(sign | (emax_field << mb));
    if (isnan(f)) return (uint16_t)(inf_bits | (1u << (mb - 1))); /* quiet NaN */
    if (isinf(f)) return inf_bits;
    double x = fabs((double)f); /* exact: every float is a double */
    if (x == 0.0) return sign;
    int E;
    (void)frexp(x, &E); /* x = f * 2^E, f in [0.5, 1) */
    int e = E - 1;      /* x in [2^e, 2^(e+1)) */
    int emin = 1 - bias;
    int qexp = (e < emin) ? (emin - mb) : (e - mb); /* weight of the last mantissa bit */
    double n = ldexp(x, -qexp);                      /* exact (power-of-two scaling) */
    double r = rint(n);                              /* nearest integer, ties to even */
    if (e < emin) {
        /* subnormal range: field = r (r == 2^mb lands exactly on the smallest normal) */
        return (uint16_t)(sign | (uint16_t)r);
    }
    if (r == ldexp(1.0, mb + 1)) { /* mantissa carried into the next binade */
        r = ldexp(1.0, mb);
        e += 1;
    }
    int ef = e + bias;
    if (ef >= emax_field) return inf_bits;
    return (uint16_t)(sign | (ef << mb) | ((uint32_t)r - (1u << mb)));
}

static double dec16(uint16_t h, int mb, int bias) {
    int s = (h >> 15) & 1;
    int ef = (h >> mb) & ((1 << (15 - mb)) - 1);
    int m = h & ((1 << mb) - 1);
    double v;
    if (ef == 0)
        v = ldexp((double)m, 1 - bias - mb);
    else if (ef == 2 * bias + 1)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)((1 << mb) + m), ef - bias - mb);
    return s ? -v : v;
}

uint16_t orc_f32_to_f16(float f) { return enc16(f, 10, 15); }
uint16_t orc_f32_to_bf16(float f) { return enc16(f, 7, 127); }
float orc_f16_to_f32(uint16_t h) { return (float)dec16(h, 10, 15); }
float orc_bf16_to_f32(uint16_t h) { return (float)dec16(h, 7, 127); }

/* array forms of the codecs (for sweeping many values in the checks) */
void orc_f32_to_f16_array(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_f16(in[i]);
}
void orc_f32_to_bf16_array(const float* in, int64_t n, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(in[i]);
}
void orc_f16_to_f32_array(const uint16_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f32(in[i]);
}
void orc_bf16_to_f32_array(const uint16_t* in, int64_t n, float* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f32(in[i]);
}

static double load_as_double(const void* p, int dtype, int64_t i) {
    switch (dtype) {
    case ORC_F32: return (double)((const float*)p)[i];
    case ORC_F16: return dec16(((const uint16_t*)p)[i], 10, 15);
    case ORC_BF16: return dec16(((const uint16_t*)p)[i], 7, 127);
    default: return NAN;
    }
}

static float scale_round(float s32, int scale_dtype) {
    /* round to the scale type, then widen back (exact) */
    if (scale_dtype == ORC_F16) return orc_f16_to_f32(orc_f32_to_f16(s32));
    return orc_bf16_to_f32(orc_f32_to_bf16(s32));
}

static uint16_t scale_bits(float s, int scale_dtype) {
    return scale_dtype == ORC_F16 ? orc_f32_to_f16(s) : orc_f32_to_bf16(s);
}

/* ------------------------------------------------------------------------ */
/* Quantizer.                                                                 */
/* For every row v and group g of G consecutive columns:                      */
/*   amax = max |w|;  amax == 0 -> s = 0, q = 0 (R1).                         */
/*   for each clip ratio r (RTN: {1.0}; MSE: 1.0, 0.95, 0.9, 0.85, 0.8):      */
/*     s = round16( max( fl32(amax * fl32(r / qmax)), floor ) )   (R2, R7)    */
/*     q_k = clamp( rint( fl32(w_k / s) ), qmin, qmax )            (R3)       */
/*     err = sum_k (q_k * s - w_k)^2 in fp64, k ascending, fma      (R4)       */
/*   keep the first ratio whose err is strictly smaller than every earlier.   */
/* `ratios` may be any list; the page's two modes are the lists above.        */
/* pick_out (nullable) receives the index of the chosen ratio per group.      */
/* ------------------------------------------------------------------------ */
int orc_quantize(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t G,
                 int scale_dtype, const double* ratios, int nratios, int8_t* q_out,
                 uint16_t* s_out, int8_t* pick_out) {
    if (!w || !q_out || !s_out || !ratios || nratios < 1) return ORC_EARG;
    if (bits != 4 && bits != 8) return ORC_EARG;
    if (G <= 0 || K % G != 0 || V < 0) return ORC_EARG;
    if (scale_dtype != ORC_F16 && scale_dtype != ORC_BF16) return ORC_EARG;
    const int qmax = (bits == 4) ? 7 : 127;
    const int qmin = (bits == 4) ? -8 : -128;
    const float floor_s = (scale_dtype == ORC_BF16) ? 1e-8f : (float)ldexp(1.0, -24);
    const int64_t NG = K / G;
    float* blk = (float*)malloc((size_t)G * sizeof(float));
    int8_t* qtry = (int8_t*)malloc((size_t)G);
    if (!blk || !qtry) {
        free(blk);
        free(qtry);
        return ORC_EARG;
    }
    for (int64_t v = 0; v < V; ++v) {
        for (int64_t g = 0; g < NG; ++g) {
            const int64_t base = v * K + g * G;
            float amax = 0.0f;
            for (int64_t k = 0; k < G; ++k) {
                blk[k] = (float)load_as_double(w, w_dtype, base + k); /* exact widening */
                float a = fabsf(blk[k]);
                if (a > amax) amax = a;
            }
            int8_t* qdst = q_out + base;
            if (amax == 0.0f) { /* R1 */
                memset(qdst, 0, (size_t)G);
                s_out[v * NG + g] = 0;
                if (pick_out) pick_out[v * NG + g] = 0;
                continue;
            }
            double best_err = 0.0;
            float best_s = 0.0f;
            int best_i = -1;
            for (int i = 0; i < nratios; ++i) {
                float c = (float)(ratios[i] / (double)qmax);
                float s32 = amax * c;
                if (s32 < floor_s) s32 = floor_s;
                float s = scale_round(s32, scale_dtype);
                double err = 0.0;
                for (int64_t k = 0; k < G; ++k) {
                    float t = blk[k] / s;
                    float r = rintf(t);
                    if (r < (float)qmin) r = (float)qmin;
                    if (r > (float)qmax) r = (float)qmax;
                    qtry[k] = (int8_t)r;
                    double d = (double)qtry[k] * (double)s - (double)blk[k];
                    err = fma(d, d, err);
                }
                if (best_i < 0 || err < best_err) {
                    best_err = err;
                    best_s = s;
                    best_i = i;
                    memcpy(qdst, qtry, (size_t)G);
                }
            }
            s_out[v * NG + g] = scale_bits(best_s, scale_dtype);
            if (pick_out) pick_out[v * NG + g] = (int8_t)best_i;
        }
    }
    free(blk);
    free(qtry);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Asymmetric (zero-point) quantizer.  The module page keeps the constant its */
/* kernel subtracts from every code (ZP_BIAS = 8 with HAS_ZP off, so the      */
/* symmetric code is q + 8) and another page lists an asymmetric ("symFalse") */
/* lm_head checkpoint; a per-group zero point z replaces that constant:       */
/*     w ~ (n - z) * s,   n, z unsigned in [0, qr],  qr = 15 (int4) / 255.   */
/* The pages give no asymmetric quantizer; the plain min/max round-to-nearest */
/* one is used (reading R21), with zero kept exactly representable:          */
/*   lo = min(0, min w), hi = max(0, max w); lo == hi (all zero): s = z = n = 0;*/
/*   s = round16( max( fl32( fl32(hi - lo) * fl32(1 / qr) ), floor ) )        */
/*   z = clamp( rint( fl32(-lo / s) ), 0, qr )                                */
/*   n_k = clamp( rint( fl32(w_k / s) ) + z, 0, qr )                          */
/* with the floor and the 16-bit rounding of the symmetric quantizer (R2).    */
/* ------------------------------------------------------------------------ */
int orc_quantize_asym(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t G,
                      int scale_dtype, uint8_t* n_out, uint16_t* s_out, uint8_t* z_out) {
    if (!w || !n_out || !s_out || !z_out) return ORC_EARG;
    if (bits != 4 && bits != 8) return ORC_EARG;
    if (G <= 0 || K % G != 0 || V < 0) return ORC_EARG;
    if (scale_dtype != ORC_F16 && scale_dtype != ORC_BF16) return ORC_EARG;
    const int qr = (bits == 4) ? 15 : 255;
    const float c = (float)(1.0 / (double)qr);
    const float floor_s = (scale_dtype == ORC_BF16) ? 1e-8f : (float)ldexp(1.0, -24);
    const int64_t NG = K / G;
    for (int64_t v = 0; v < V; ++v) {
        for (int64_t g = 0; g < NG; ++g) {
            const int64_t base = v * K + g * G;
            float lo = 0.0f, hi = 0.0f;
            for (int64_t k = 0; k < G; ++k) {
                const float x = (float)load_as_double(w, w_dtype, base + k);
                if (x < lo) lo = x;
                if (x > hi) hi = x;
            }
            uint8_t* nd = n_out + base;
            if (hi == lo) { /* all zero */
                memset(nd, 0, (size_t)G);
                s_out[v * NG + g] = 0;
                z_out[v * NG + g] = 0;
                continue;
            }
            float s32 = (hi - lo) * c;
            if (s32 < floor_s) s32 = floor_s;
            const float s = scale_round(s32, scale_dtype);
            float zf = rintf(-lo / s);
            if (zf < 0.0f) zf = 0.0f;
            if (zf > (float)qr) zf = (float)qr;
            for (int64_t k = 0; k < G; ++k) {
                const float x = (float)load_as_double(w, w_dtype, base + k);
                float n = rintf(x / s) + zf;
                if (n < 0.0f) n = 0.0f;
                if (n > (float)qr) n = (float)qr;
                nd[k] = (uint8_t)n;
            }
            s_out[v * NG + g] = scale_bits(s, scale_dtype);
            z_out[v * NG + g] = (uint8_t)zf;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Packed blob.                                                               */
/* Rows are grouped in blocks of 64 (the last block is padded with q = 0,     */
/* s = 0).  A row of one block is cut into superchunks of `span` columns     */
/* (128 for int4, 64 for int8); each superchunk is 4 slots of 16 bytes.       */
/* Weight byte offset of (block b, superchunk c, slot t, row r in block):     */
/*     (((b * NC + c) * 4 + t) * 64 + r) * 16,   NC = K / span.               */
/* int4: the slot holds 4 little-endian 32-bit words j = 0..3; word j holds   */
/*   columns 128c + 32j + 8t + i, i = 0..7; column i sits in nibble           */
/*   position p (bits 4p..4p+3) with i = (p < 4) ? 2p : 2(p - 4) + 1;         */
/*   the stored nibble is q + 8.                                              */
/* int8: word j holds columns 64c + 32(j >> 1) + 8t + 4(j & 1) + i,           */
/*   i = 0..3, in byte i; the stored byte is q + 128.                         */
/* Scales follow the weights (at byte V_pad * K * bits / 8), 16-bit each,     */
/* element offset (b * NG + g) * 64 + r, NG = K / G.                          */
/* ------------------------------------------------------------------------ */
static int layout_ok(int64_t V, int64_t K, int bits, int64_t G) {
    if (V < 1 || K < 1 || G < 1) return 0;
    if (bits != 4 && bits != 8) return 0;
    int64_t span = (bits == 4) ? 128 : 64;
    if (K % span != 0 || K % G != 0 || G % 32 != 0) return 0;
    return 1;
}

int64_t orc_packed_bytes(int64_t V, int64_t K, int bits, int64_t G) {
    if (!layout_ok(V, K, bits, G)) return -1;
    int64_t vpad = (V + 63) / 64 * 64;
    return vpad * K * bits / 8 + vpad * (K / G) * 2;
}

/* byte offset and nibble/byte position of element (v, k) */
static void elem_pos(int64_t v, int64_t k, int64_t K, int bits, int64_t* byte_off, int* shift) {
    int64_t b = v / 64, r = v % 64;
    if (bits == 4) {
        int64_t NC = K / 128;
        int64_t c = k / 128, w = k % 128;
        int64_t j = w / 32, t = (w % 32) / 8, i = w % 8;
        int p = (i % 2 == 0) ? (int)(i / 2) : (int)(4 + i / 2);
        int64_t slot_off = (((b * NC + c) * 4 + t) * 64 + r) * 16;
        *byte_off = slot_off + j * 4 + p / 2;
        *shift = (p % 2) * 4;
    } else {
        int64_t NC = K / 64;
        int64_t c = k / 64, w = k % 64;
        int64_t hj = w / 32, t = (w % 32) / 8, h = (w % 8) / 4, i = w % 4;
        int64_t j = hj * 2 + h;
        int64_t slot_off = (((b * NC + c) * 4 + t) * 64 + r) * 16;
        *byte_off = slot_off + j * 4 + i;
        *shift = 0;
    }
}

int orc_pack(const int8_t* q, const uint16_t* s, int64_t V, int64_t K, int bits, int64_t G,
             uint8_t* out) {
    if (!q || !s || !out || !layout_ok(V, K, bits, G)) return ORC_EARG;
    int64_t vpad = (V + 63) / 64 * 64, NG = K / G;
    int64_t wbytes = vpad * K * bits / 8;
    /* padding: q = 0 everywhere, scale 0 */
    memset(out, bits == 4 ? 0x88 : 0x80, (size_t)wbytes);
    memset(out + wbytes, 0, (size_t)(vpad * NG * 2));
    for (int64_t v = 0; v < V; ++v) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t off;
            int sh;
            elem_pos(v, k, K, bits, &off, &sh);
            int qq = q[v * K + k];
            if (bits == 4) {
                uint8_t nib = (uint8_t)(qq + 8) & 0xF;
                out[off] = (uint8_t)((out[off] & ~(0xF << sh)) | (nib << sh));
            } else {
                out[off] = (uint8_t)(qq + 128);
            }
        }
        for (int64_t g = 0; g < NG; ++g) {
            int64_t e = ((v / 64) * NG + g) * 64 + v % 64;
            uint16_t sv = s[v * NG + g];
            out[wbytes + 2 * e] = (uint8_t)(sv & 0xFF);
            out[wbytes + 2 * e + 1] = (uint8_t)(sv >> 8);
        }
    }
    return ORC_OK;
}

int orc_unpack(const uint8_t* blob, int64_t V, int64_t K, int bits, int64_t G, int8_t* q,
               uint16_t* s) {
    if (!blob || !q || !s || !layout_ok(V, K, bits, G)) return ORC_EARG;
    int64_t vpad = (V + 63) / 64 * 64, NG = K / G;
    int64_t wbytes = vpad * K * bits / 8;
    for (int64_t v = 0; v < V; ++v) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t off;
            int sh;
            elem_pos(v, k, K, bits, &off, &sh);
            if (bits == 4)
                q[v * K + k] = (int8_t)(((blob[off] >> sh) & 0xF) - 8);
            else
                q[v * K + k] = (int8_t)((int)blob[off] - 128);
        }
        for (int64_t g = 0; g < NG; ++g) {
            int64_t e = ((v / 64) * NG + g) * 64 + v % 64;
            s[v * NG + g] = (uint16_t)(blob[wbytes + 2 * e] | (blob[wbytes + 2 * e + 1] << 8));
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* ------------------------------------------------------------------------ */
/* Packed blob of the zero-point form: the codes n are stored as they are     */
/* (nibble n, byte n), the scales as above, and after the scales one byte per */
/* (row, group) holds z, at byte offset (b * NG + g) * 64 + 4 * (r mod 16) +  */
/* (r div 16) of that region (a lane that owns rows r, r + 16, r + 32, r + 48 */
/* of a block reads its four zero points as one 32-bit word).  Padding rows:  */
/* n = 0, s = 0, z = 0.                                                       */
/* ------------------------------------------------------------------------ */
int64_t orc_packed_bytes_zp(int64_t V, int64_t K, int bits, int64_t G) {
    if (!layout_ok(V, K, bits, G)) return -1;
    int64_t vpad = (V + 63) / 64 * 64;
    return vpad * K * bits / 8 + vpad * (K / G) * 3;
}

static int64_t zp_off(int64_t v, int64_t g, int64_t NG) {
    const int64_t r = v % 64;
    return ((v / 64) * NG + g) * 64 + 4 * (r % 16) + r / 16;
}

int orc_pack_zp(const uint8_t* n, const uint16_t* s, const uint8_t* z, int64_t V, int64_t K,
                int bits, int64_t G, uint8_t* out) {
    if (!n || !s || !z || !out || !layout_ok(V, K, bits, G)) return ORC_EARG;
    int64_t vpad = (V + 63) / 64 * 64, NG = K / G;
    int64_t wbytes = vpad * K * bits / 8, sbytes = vpad * NG * 2;
    memset(out, 0, (size_t)(wbytes + sbytes + vpad * NG));
    for (int64_t v = 0; v < V; ++v) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t off;
            int sh;
            elem_pos(v, k, K, bits, &off, &sh);
            int nn = n[v * K + k];
            if (bits == 4)
                out[off] = (uint8_t)((out[off] & ~(0xF << sh)) | ((nn & 0xF) << sh));
            else
                out[off] = (uint8_t)nn;
        }
        for (int64_t g = 0; g < NG; ++g) {
            int64_t e = ((v / 64) * NG + g) * 64 + v % 64;
            uint16_t sv = s[v * NG + g];
            out[wbytes + 2 * e] = (uint8_t)(sv & 0xFF);
            out[wbytes + 2 * e + 1] = (uint8_t)(sv >> 8);
            out[wbytes + sbytes + zp_off(v, g, NG)] = z[v * NG + g];
        }
    }
    return ORC_OK;
}

int orc_unpack_zp(const uint8_t* blob, int64_t V, int64_t K, int bits, int64_t G, uint8_t* n,
                  uint16_t* s, uint8_t* z) {
    if (!blob || !n || !s || !z || !layout_ok(V, K, bits, G)) return ORC_EARG;
    int64_t vpad = (V + 63) / 64 * 64, NG = K / G;
    int64_t wbytes = vpad * K * bits / 8, sbytes = vpad * NG * 2;
    for (int64_t v = 0; v < V; ++v) {
        for (int64_t k = 0; k < K; ++k) {
            int64_t off;
            int sh;
            elem_pos(v, k, K, bits, &off, &sh);
            n[v * K + k] = (bits == 4) ? (uint8_t)((blob[off] >> sh) & 0xF) : blob[off];
        }
        for (int64_t g = 0; g < NG; ++g) {
            int64_t e = ((v / 64) * NG + g) * 64 + v % 64;
            s[v * NG + g] = (uint16_t)(blob[wbytes + 2 * e] | (blob[wbytes + 2 * e + 1] << 8));
            z[v * NG + g] = blob[wbytes + sbytes + zp_off(v, g, NG)];
        }
    }
    return ORC_OK;
}

/* Logits of the zero-point form: y[m, j] = sum_k x[m,k] * ((n[v,k] - z[v,g]) */
/* * s[v,g]) + bias[v], v = rows[j], exact products, fp64 sums k ascending.   */
int orc_logits_zp(const void* x, int x_dtype, int64_t M, const uint8_t* n, const uint16_t* s,
                  const uint8_t* z, int scale_dtype, int64_t V, int64_t K, int64_t G,
                  const float* bias, const int64_t* rows, int64_t nrows, double* y) {
    if (!x || !n || !s || !z || !y || G <= 0 || K % G != 0) return ORC_EARG;
    if (!rows && nrows != V) return ORC_EARG;
    const int64_t NG = K / G;
    const int sb = (scale_dtype == ORC_F16) ? 10 : 7, sbias = (scale_dtype == ORC_F16) ? 15 : 127;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < nrows; ++j) {
            int64_t v = rows ? rows[j] : j;
            if (v < 0 || v >= V) return ORC_EARG;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = load_as_double(x, x_dtype, m * K + k);
                int64_t g = k / G;
                double wv = ((double)n[v * K + k] - (double)z[v * NG + g]) *
                            dec16(s[v * NG + g], sb, sbias);
                acc += xv * wv;
            }
            if (bias) acc += (double)bias[v];
            y[m * nrows + j] = acc;
        }
    }
    return ORC_OK;
}

/* Embedding rows of the zero-point form: out[t, k] = (n[v,k] - z[v,g]) *    */
/* s[v,g], rounded once to out_dtype; ids outside [0, V) give zero rows.      */
int orc_embed_zp(const uint8_t* n, const uint16_t* s, const uint8_t* z, int scale_dtype,
                 int64_t V, int64_t K, int64_t G, const int32_t* ids, int64_t T, int out_dtype,
                 void* out) {
    if (!n || !s || !z || !ids || !out || G <= 0 || K % G != 0 || T < 0) return ORC_EARG;
    if (scale_dtype != ORC_F16 && scale_dtype != ORC_BF16) return ORC_EARG;
    if (out_dtype != ORC_F32 && out_dtype != ORC_F16 && out_dtype != ORC_BF16) return ORC_EARG;
    const int64_t NG = K / G;
    const int sb = (scale_dtype == ORC_F16) ? 10 : 7, sbias = (scale_dtype == ORC_F16) ? 15 : 127;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t v = ids[t];
        for (int64_t k = 0; k < K; ++k) {
            double p = 0.0;
            if (v >= 0 && v < V)
                p = ((double)n[v * K + k] - (double)z[v * NG + k / G]) *
                    dec16(s[v * NG + k / G], sb, sbias);
            const float f = (float)p; /* exact: the product fits in fp32 */
            if (out_dtype == ORC_F32)
                ((float*)out)[t * K + k] = f;
            else if (out_dtype == ORC_F16)
                ((uint16_t*)out)[t * K + k] = enc16(f, 10, 15);
            else
                ((uint16_t*)out)[t * K + k] = enc16(f, 7, 127);
        }
    }
    return ORC_OK;
}

/* Logits from the canonical quantized form (q int8 [V,K], s 16-bit [V,K/G]):*/
/*   y[m, j] = sum_k x[m,k] * (q[v,k] * s[v, k/G]) + bias[v],  v = rows[j],   */
/* every operand widened exactly to fp64, the sum taken k ascending.          */
/* rows == NULL means all V rows (then nrows must equal V).                   */
/* ------------------------------------------------------------------------ */
int orc_logits(const void* x, int x_dtype, int64_t M, const int8_t* q, const uint16_t* s,
               int scale_dtype, int64_t V, int64_t K, int64_t G, const float* bias,
               const int64_t* rows, int64_t nrows, double* y) {
    if (!x || !q || !s || !y || G <= 0 || K % G != 0) return ORC_EARG;
    if (!rows && nrows != V) return ORC_EARG;
    const int64_t NG = K / G;
    const int sb = (scale_dtype == ORC_F16) ? 10 : 7, sbias = (scale_dtype == ORC_F16) ? 15 : 127;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < nrows; ++j) {
            int64_t v = rows ? rows[j] : j;
            if (v < 0 || v >= V) return ORC_EARG;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double xv = load_as_double(x, x_dtype, m * K + k);
                double wv = (double)q[v * K + k] * dec16(s[v * NG + k / G], sb, sbias);
                acc += xv * wv;
            }
            if (bias) acc += (double)bias[v];
            y[m * nrows + j] = acc;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Embedding rows from the canonical quantized form:                          */
/*   out[t, k] = q[v,k] * s[v, k/G],  v = ids[t],                             */
/* the product exact (at most 8 + 11 significant bits), then rounded once to  */
/* out_dtype (fp32: unchanged; fp16/bf16: nearest, ties to even).  An id      */
/* outside [0, V) gives a row of zeros.  The packed table of a tied head is    */
/* also the input-embedding table, so the lookup dequantizes its rows (vLLM   */
/* PR #48870, Purpose: the quantized embedding serves the input lookup and     */
/* is reused as the tied lm_head).                                            */
/* ------------------------------------------------------------------------ */
int orc_embed(const int8_t* q, const uint16_t* s, int scale_dtype, int64_t V, int64_t K,
              int64_t G, const int32_t* ids, int64_t T, int out_dtype, void* out) {
    if (!q || !s || !ids || !out || G <= 0 || K % G != 0 || T < 0) return ORC_EARG;
    if (scale_dtype != ORC_F16 && scale_dtype != ORC_BF16) return ORC_EARG;
    if (out_dtype != ORC_F32 && out_dtype != ORC_F16 && out_dtype != ORC_BF16) return ORC_EARG;
    const int64_t NG = K / G;
    const int sb = (scale_dtype == ORC_F16) ? 10 : 7, sbias = (scale_dtype == ORC_F16) ? 15 : 127;
    for (int64_t t = 0; t < T; ++t) {
        const int64_t v = ids[t];
        for (int64_t k = 0; k < K; ++k) {
            double p = 0.0;
            if (v >= 0 && v < V) p = (double)q[v * K + k] * dec16(s[v * NG + k / G], sb, sbias);
            const float f = (float)p; /* exact: the product fits in fp32 */
            if (out_dtype == ORC_F32)
                ((float*)out)[t * K + k] = f;
            else if (out_dtype == ORC_F16)
                ((uint16_t*)out)[t * K + k] = enc16(f, 10, 15);
            else
                ((uint16_t*)out)[t * K + k] = enc16(f, 7, 127);
        }
    }
    return ORC_OK;
}

/* Dense logits y[m, j] = sum_k x[m,k] * W[v,k], v = rows[j], in fp64. */
int orc_dense_logits(const void* x, int x_dtype, int64_t M, const void* w, int w_dtype, int64_t V,
                     int64_t K, const int64_t* rows, int64_t nrows, double* y) {
    if (!x || !w || !y) return ORC_EARG;
    if (!rows && nrows != V) return ORC_EARG;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < nrows; ++j) {
            int64_t v = rows ? rows[j] : j;
            if (v < 0 || v >= V) return ORC_EARG;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += load_as_double(x, x_dtype, m * K + k) * load_as_double(w, w_dtype, v * K + k);
            y[m * nrows + j] = acc;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Top-K of one row: the K largest values, value descending then index        */
/* ascending (R5).  Plain selection: K passes over the row.                   */
/* ------------------------------------------------------------------------ */
static int before(float a, int64_t ia, float b, int64_t ib) {
    return a > b || (a == b && ia < ib);
}

int orc_topk(const float* y, int64_t V, int topk, int64_t* idx) {
    if (!y || !idx || topk < 1 || topk > V) return ORC_EARG;
    for (int t = 0; t < topk; ++t) {
        int64_t best = -1;
        for (int64_t v = 0; v < V; ++v) {
            int taken = 0;
            for (int u = 0; u < t; ++u)
                if (idx[u] == v) {
                    taken = 1;
                    break;
                }
            if (taken) continue;
            if (best < 0 || before(y[v], v, y[best], best)) best = v;
        }
        idx[t] = best;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Top-K exact rescoring (R5).  For each row m of the given logits y[M, ldy]: */
/*   I = top-K of y[m, 0..V);  for v in I: y'[v] = sum_k x[m,k] W[v,k] (fp64) */
/*   every other position keeps y[m, v];  top1 = first maximum of y'.         */
/* idx_out[m, t] = I in top-K order; val_out[m, t] = y'[I[t]];               */
/* top1_out[m] = the argmax.                                                  */
/* ------------------------------------------------------------------------ */
int orc_topk_rescore(const float* y, int64_t ldy, int64_t M, int64_t V, int topk, const void* x,
                     int x_dtype, const void* w, int w_dtype, int64_t K, int64_t* idx_out,
                     double* val_out, int64_t* top1_out) {
    if (!y || !x || !w || !idx_out || !val_out || !top1_out) return ORC_EARG;
    if (topk < 1 || topk > V || ldy < V) return ORC_EARG;
    for (int64_t m = 0; m < M; ++m) {
        const float* row = y + m * ldy;
        int64_t* I = idx_out + m * topk;
        int rc = orc_topk(row, V, topk, I);
        if (rc) return rc;
        for (int t = 0; t < topk; ++t) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += load_as_double(x, x_dtype, m * K + k) * load_as_double(w, w_dtype, I[t] * K + k);
            val_out[m * topk + t] = acc;
        }
        /* argmax of the scattered vector: rescored values at I, y elsewhere */
        int64_t best = -1;
        double bestv = 0.0;
        for (int64_t v = 0; v < V; ++v) {
            double val = (double)row[v];
            for (int t = 0; t < topk; ++t)
                if (I[t] == v) {
                    val = val_out[m * topk + t];
                    break;
                }
            if (best < 0 || val > bestv) {
                best = v;
                bestv = val;
            }
        }
        top1_out[m] = best;
    }
    return ORC_OK;
}

/* Algorithmic bytes of one logits call: packed weight, scales, x (16-bit), */
/* fp32 logits.  (Used by the byte-accounting checks and the benchmark.)    */
int64_t orc_algorithmic_bytes(int64_t M, int64_t V, int64_t K, int bits, int64_t G) {
    return V * K * bits / 8 + V * (K / G) * 2 + M * K * 2 + M * V * 4;
}
