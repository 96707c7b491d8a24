/*
 * lmhead.h -- C ABI of liblmhead.so: weight-only-quantized LM-head logits on
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes, for a language-model head whose weight W[V, K] is
 * stored as symmetric int4 (q in [-8, 7]) or int8 (q in [-128, 127]) codes with
 * one fp16/bf16 scale per group of G input columns,
 *
 *     y[m, v] = sum_k x[m, k] * q[v, k] * s[v, k / G]   (+ bias[v])
 *
 * straight from the packed codes, never forming the dense weight (vLLM PR
 * #48870 "Fused WNA16 GEMM for tied quantized lm_head logits", Purpose: a fused
 * dequant-GEMM in place of dequantize-then-F.linear).  Around it sit the
 * load-time quantizer (page "radiance_lmhead_int4.py", docstring "How"
 * paragraph and quantize_int4_rows), the packer into this library's own
 * layout, and the top-K exact rescoring step (vLLM PR #48870, review comment,
 * point 2).
 *
 * Conventions for every entry point
 *   - All data pointers are DEVICE pointers (hipMalloc'd or torch CUDA/HIP
 *     tensors) unless stated otherwise; the caller allocates and owns every
 *     buffer, including workspaces.  The library never allocates, frees or
 *     copies between host and device.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work
 *     is enqueued on it and the call returns without synchronising.
 *   - Every argument is validated on the host before anything is launched; on
 *     an error nothing is enqueued and the status says why.  A launch the HIP
 *     runtime rejects returns LMH_E_HIP.  No exception crosses the ABI.
 *   - Inputs must be finite; NaN/Inf inputs give unspecified (but memory-safe)
 *     results.
 *   - Data pointers must be 16-byte aligned unless stated otherwise.
 *   - M == 0 or V == 0 is a valid empty call: LMH_OK, nothing launched.
 *   - Calls are thread-safe; concurrent calls on different streams are fine.
 *
 * dtype codes: LMH_F32 = 0, LMH_F16 = 1 (IEEE binary16), LMH_BF16 = 2.
 *
 * Packed blob layout (lmhead_pack writes it, lmhead_logits reads it)
 *   span  = 128 columns for int4, 64 for int8;  NC = K / span;  NG = K / G.
 *   Rows are taken in blocks of 64 (NB = ceil(V/64), V_pad = 64*NB); rows
 *   V..V_pad-1 are padding with q = 0 and scale 0.
 *   Weight region, byte offset of the 16-byte slot for
 *     (block b, superchunk c, slot t in 0..3, row r in 0..63):
 *         (((b*NC + c)*4 + t)*64 + r) * 16
 *   int4: the slot is four little-endian 32-bit words j = 0..3; word j holds
 *     columns 128c + 32j + 8t + i, i = 0..7, as unsigned nibbles q + 8; the
 *     nibble at bits 4p..4p+3 holds column i = 2p for p < 4 and i = 2(p-4)+1
 *     for p >= 4 (even columns in the low half-word, odd in the high one).
 *   int8: word j holds columns 64c + 32(j>>1) + 8t + 4(j&1) + i, i = 0..3, in
 *     byte i, as unsigned bytes q + 128.
 *   Scale region, starting at byte V_pad*K*bits/8: 16-bit scales (fp16 or
 *     bf16 bit patterns), element offset (b*NG + g)*64 + r.
 *   Total size: V_pad*K*bits/8 + V_pad*NG*2 bytes (lmhead_packed_bytes).
 *
 * Zero-point (asymmetric) heads: `bits | LMH_ZP`
 *   The module page keeps a constant that its kernel subtracts from every
 *   nibble (ZP_BIAS = 8, with its HAS_ZP switch off), and the vLLM PR's page
 *   lists an asymmetric ("symFalse") quantized lm_head checkpoint: in that
 *   form each row and group has its own zero point z in place of the fixed 8,
 *       w[v, k] ~ (n[v, k] - z[v, g]) * s[v, g],   g = k / G,
 *   with unsigned codes n and z in [0, qr], qr = 15 (int4) or 255 (int8), so
 *       y[m, v] = sum_k x[m, k] * (n[v, k] - z[v, g]) * s[v, g]  (+ bias[v]).
 *   Passing bits | LMH_ZP (LMH_ZP = 0x10) to lmhead_packed_bytes,
 *   lmhead_quantize_pack, lmhead_embed and every logits entry point selects
 *   that form; lmhead_quantize_zp and lmhead_pack_zp are its codes-mode
 *   quantizer and packer.  Its blob differs from the symmetric one in three
 *   points: codes are stored as they are (nibble n, byte n; padding rows 0),
 *   and after the scale region a zero-point region of V_pad*NG bytes holds z
 *   for (block b, group g, row r) at byte offset
 *         (b*NG + g)*64 + 4*(r % 16) + r / 16
 *   (one 32-bit word holds the zero points of rows r, r+16, r+32, r+48: the
 *   rows one MFMA lane unpacks); padding rows have z = 0.  Total size:
 *   V_pad*K*bits/8 + V_pad*NG*3 bytes.  A symmetric head is the special case
 *   z = 8 (int4) / 128 (int8), n = q + 8 / q + 128.
 *   Why: a lane that owns a row reads one 16-byte slot per 32 (int8: 16)
 *   columns, 64 consecutive rows read 1 KiB contiguously, and the same slot,
 *   read by 16 rows x 4 slots, is exactly one 16x16x32 MFMA B-operand tile
 *   for each of its 32-column words.
 *
 * Supported shapes: bits in {4, 8}; K % span == 0; G % 32 == 0; K % G == 0;
 * G divides the span or is a multiple of it (int4: G in {32, 64} or a
 * multiple of 128; int8: G = 32 or a multiple of 64); K <= 65536; V < 2^31;
 * M <= 65535; ceil(V/256) * ceil(M/16) < 2^30 (else LMH_E_UNSUPPORTED).
 */
#ifndef LMHEAD_H
#define LMHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    LMH_OK = 0,
    LMH_E_NULL = 1,        /* a required pointer is NULL */
    LMH_E_SHAPE = 2,       /* a size is out of range or sizes disagree */
    LMH_E_DTYPE = 3,       /* a dtype code is not allowed for that argument */
    LMH_E_ALIGN = 4,       /* a pointer is not 16-byte aligned */
    LMH_E_UNSUPPORTED = 5, /* a valid request this build does not implement */
    LMH_E_WORKSPACE = 6,   /* workspace missing or smaller than required */
    LMH_E_HIP = 7,         /* the HIP runtime reported an error */
    LMH_E_SCRATCH = 8      /* more than the allocation-free entry point's scratch */
};

enum { LMH_F32 = 0, LMH_F16 = 1, LMH_BF16 = 2 };
enum { LMH_CLIP_RTN = 0, LMH_CLIP_MSE = 1 };
enum { LMH_ZP = 0x10 }; /* OR'd into `bits`: the zero-point (asymmetric) form */

/* Human-readable name of a status code (static storage; never NULL). */
const char* lmhead_status_string(int status);

/* ABI version of this header; bumped when any signature or the layout changes. */
int lmhead_abi_version(void);

/*
 * lmhead_packed_bytes -- size in bytes of the packed blob for a V x K head
 * (bits may carry LMH_ZP), or 0 if the shape is not supported.  Host-only;
 * launches nothing.
 */
size_t lmhead_packed_bytes(int64_t V, int64_t K, int bits, int64_t group);

/*
 * lmhead_quantize -- load-time symmetric per-group quantizer.
 *   Defined by page "radiance_lmhead_int4.py" (docstring "How" paragraph;
 *   module constants CLIP_RATIOS, QMAX, ZP_BIAS; quantize_int4_rows), extended
 *   to int8 and to fp16 scales.  For each row v and group g of G columns:
 *     amax = max |w|; amax == 0 gives s = 0 and q = 0 for the group;
 *     for each clip ratio r (RTN: 1.0 only; MSE: 1.0, 0.95, 0.9, 0.85, 0.8):
 *       s_r = to16( max( fl32(amax * fl32(r / qmax)), floor ) ), floor = 1e-8
 *             for bf16 scales and 2^-24 for fp16 scales, to16 = round to the
 *             scale type, nearest-even;
 *       q_r = clamp( rint( fl32(w / s_r) ), qmin, qmax )  (IEEE division,
 *             ties to even);
 *       err_r = sum over k ascending of (q_r*s_r - w)^2, fp64, one fused
 *             multiply-add per element;
 *     keep the first r whose err_r is strictly smaller than all earlier ones.
 *   qmax/qmin = 7/-8 (int4) or 127/-128 (int8).  Results are bit-exact
 *   (deterministic, no atomics).
 *   w      [V, K] row-major, w_dtype LMH_F32 / LMH_F16 / LMH_BF16.
 *   q_out  [V, K] int8 row-major (the code q itself, not biased).
 *   s_out  [V, K/G] 16-bit scale bit patterns, scale_dtype LMH_F16 / LMH_BF16.
 *   clip   LMH_CLIP_RTN or LMH_CLIP_MSE.
 *   Shape rules: G % 32 == 0 and K % G == 0 (the packing span is not needed);
 *   V * K < 2^40 (else LMH_E_SHAPE); ceil(V/64) * (K/G) <= 2^26 - 32 (one
 *   wavefront per 64 rows and group; else LMH_E_UNSUPPORTED).
 *   A scale that overflows the scale type is a precondition violation.
 */
int lmhead_quantize(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t group,
                    int scale_dtype, int clip, int8_t* q_out, void* s_out, void* stream);

/*
 * lmhead_pack -- write the packed blob (layout above) from the canonical
 *   codes q [V, K] int8 and scales s [V, K/G] (16-bit patterns).  Codes outside
 *   [qmin, qmax] are a precondition violation.  Deterministic: the same input
 *   gives the same bytes (packing twice is harmless).
 *   packed_out must hold lmhead_packed_bytes(V, K, bits, group) bytes.
 */
int lmhead_pack(const int8_t* q, const void* s, int64_t V, int64_t K, int bits, int64_t group,
                void* packed_out, void* stream);

/*
 * lmhead_quantize_zp -- load-time quantizer of the zero-point form (see
 *   "Zero-point heads" above).  The pages name that form but give no
 *   quantizer for it; this one is plain per-group min/max round-to-nearest
 *   over the group's range widened to include zero, so that w = 0 is exactly
 *   representable (n = z).  For each row v and group g of G columns:
 *     lo = min(0, min w), hi = max(0, max w); lo == hi (all zero) gives
 *       s = 0, z = 0 and n = 0 for the group;
 *     s = to16( max( fl32( fl32(hi - lo) * fl32(1 / qr) ), floor ) ), with
 *       floor and to16 as for lmhead_quantize;
 *     z = clamp( rint( fl32(-lo / s) ), 0, qr );
 *     n = clamp( rint( fl32(w / s) ) + z, 0, qr )   (IEEE division, ties to
 *       even).
 *   No clip search.  Bit-exact, deterministic.
 *   w      [V, K] row-major, w_dtype LMH_F32 / LMH_F16 / LMH_BF16.
 *   n_out  [V, K] uint8 codes, row-major.
 *   s_out  [V, K/G] 16-bit scale bit patterns, scale_dtype LMH_F16 / LMH_BF16.
 *   z_out  [V, K/G] uint8 zero points, row-major (any alignment).
 *   bits   4 or 8 (LMH_ZP may be set; it is implied).  Shape rules as for
 *          lmhead_quantize.
 */
int lmhead_quantize_zp(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t group,
                       int scale_dtype, uint8_t* n_out, void* s_out, uint8_t* z_out,
                       void* stream);

/*
 * lmhead_pack_zp -- write the zero-point blob (layout above) from the codes
 *   n [V, K] uint8, scales s [V, K/G] (16-bit patterns) and zero points
 *   z [V, K/G] uint8 (any alignment).  Codes or zero points above qr are a
 *   precondition violation.  packed_out must hold
 *   lmhead_packed_bytes(V, K, bits | LMH_ZP, group) bytes.  Deterministic.
 */
int lmhead_pack_zp(const uint8_t* n, const void* s, const uint8_t* z, int64_t V, int64_t K,
                   int bits, int64_t group, void* packed_out, void* stream);

/*
 * lmhead_quantize_pack -- the quantizer and the packer fused: rows
 *   [row0, row0 + rows) of a V x K head go straight from the unquantized
 *   weight into their place in the packed blob, with no int8 copy of the
 *   codes in between.  Page "radiance_lmhead_int4.py" quantizes the head in
 *   row chunks at load time to bound the transient memory (module constant
 *   CHUNK_ROWS; RadianceLMHeadInt4.process_weights_after_loading); the same
 *   page's quantize_int4_rows defines the arithmetic, which is exactly that
 *   of lmhead_quantize above.
 *   Calling it over chunks that cover [0, V) in any order writes the same
 *   bytes as lmhead_pack(lmhead_quantize(w)) for the whole head.
 *   w          rows row0 .. row0+rows-1 of the head, row-major with row stride
 *              ldw elements (ldw >= K, ldw % 8 == 0), w_dtype LMH_F32 /
 *              LMH_F16 / LMH_BF16.  w[0] is row row0.
 *   row0       multiple of 64; rows >= 0; row0 + rows <= V; rows is a
 *              multiple of 64 unless row0 + rows == V (the last chunk, which
 *              also writes the zero padding rows of the final block).
 *   packed_out the whole blob of the V x K head (lmhead_packed_bytes); only
 *              the blocks of this chunk are written, other bytes are left
 *              as they are.
 *   clip, scale_dtype, bits, group as for lmhead_quantize; layout rules as
 *   for lmhead_pack.  With bits | LMH_ZP the arithmetic is that of
 *   lmhead_quantize_zp and the blob the zero-point one (clip must be
 *   LMH_CLIP_RTN, else LMH_E_UNSUPPORTED).  rows == 0 is a valid empty call.
 *   ceil(rows/64) * (K / max(G, span)) <= 2^26 - 32 (one wavefront per 64
 *   rows and superchunk or group; else LMH_E_UNSUPPORTED).  Deterministic.
 */
int lmhead_quantize_pack(const void* w, int w_dtype, int64_t ldw, int64_t V, int64_t K, int bits,
                         int64_t group, int scale_dtype, int clip, int64_t row0, int64_t rows,
                         void* packed_out, void* stream);

/*
 * lmhead_embed -- the input-embedding lookup of a tied head, read from the
 *   same packed blob the logits use:
 *       out[t, k] = q[id, k] * s[id, k / G],   id = ids[t],
 *   (zero-point heads, bits | LMH_ZP: (n[id, k] - z[id, k / G]) * s[id, k / G]),
 *   the product exact, rounded once to out_dtype (LMH_F32: exact; LMH_F16 /
 *   LMH_BF16: nearest, ties to even; an fp16 result beyond its range becomes
 *   +-inf).  vLLM PR #48870, Purpose: the quantized embedding table that
 *   serves the input lookup is the one reused as the tied lm_head (that PR
 *   keeps a second, gather-format copy; this layout serves both).
 *   ids     [T] int32 token ids, device memory, 4-byte aligned.  An id outside
 *           [0, V) yields a row of zeros (never an out-of-bounds read).
 *   packed  blob of lmhead_pack / lmhead_quantize_pack for this (V, K, bits,
 *           group); scale_dtype as it was quantized with.
 *   out     [T, ldo] row-major, out_dtype LMH_F32 / LMH_F16 / LMH_BF16;
 *           ldo >= K and each row 16-byte aligned (ldo % 4 == 0 for fp32,
 *           % 8 for 16-bit).  Columns K..ldo-1 are not written.
 *   T == 0 is a valid empty call.  Deterministic.
 */
int lmhead_embed(const int32_t* ids, int64_t T, const void* packed, int64_t V, int64_t K, int bits,
                 int64_t group, int scale_dtype, void* out, int out_dtype, int64_t ldo,
                 void* stream);

/*
 * lmhead_logits_workspace_bytes -- device workspace that lmhead_logits may
 *   need for M rows of x: 0 for fp16 x; for bf16 x, room for x converted to
 *   fp16 with a per-row power-of-two scale (M*K*2 and M*4 bytes, each rounded
 *   up to a multiple of 256), which only the MFMA kernels use (the GEMV,
 *   M <= 2 by default, converts bf16 rows itself and needs none).
 */
size_t lmhead_logits_workspace_bytes(int64_t M, int64_t K, int x_dtype);

/*
 * lmhead_logits -- y[m, v] = sum_k x[m,k] * q[v,k] * s[v,k/G] (+ bias[v]).
 *   The fused weight-only-quantized logits of vLLM PR #48870 (Purpose; perf
 *   table: W4-g64 / W8-g128 heads at M = 1, 32, 256), read straight from the
 *   packed blob.  The codes q enter the arithmetic exactly; each group's
 *   partial sum is accumulated in fp32 and multiplied by its scale in fp32.
 *   x       [M, K] row-major, x_dtype LMH_F16 or LMH_BF16 (bf16 rows are
 *           converted to fp16 with an exact power-of-two row scale: inside the
 *           GEMV, and for the MFMA kernels by a first kernel into the
 *           workspace).
 *   packed  the blob for (V, K, bits, group, scale_dtype).
 *   bias    [V] fp32 or NULL.
 *   y       [M, ldy] fp32 row-major, ldy >= V; columns V..ldy-1 are not
 *           written.  Needs only 4-byte alignment.
 *   workspace / ws_bytes: at least lmhead_logits_workspace_bytes(M, K, x_dtype)
 *           when x is bf16 and an MFMA kernel runs (M > 2 by default), else
 *           ignored (may be NULL/0); a missing or short one is LMH_E_WORKSPACE.
 *   M = 1 runs a GEMV with one lane per vocabulary row (K split over up to 8
 *   waves per 64-row block), and so does M = 2 with bf16 x or K > 2048;
 *   larger M (and two fp16 rows of K <= 2048) runs a 16x16x32 fp16 MFMA
 *   kernel (its code unpacking is shared by all activation rows), chosen
 *   from measurements: for M = 2 (fp16 x) and 3..16 with K <= 2048 the
 *   split-K one (path 5);
 *   beyond, for K <= 1024 and G >= 64, the activation-resident one from
 *   M = 33 on (int4 heads: from M = 17 on), else the LDS-staged one; for
 *   K > 1024 the register-fed one for M = 25..32, else the LDS-staged one
 *   (see lmhead_logits_path).  The register-fed, LDS-staged and
 *   activation-resident kernels run the same per-group MFMA chains and fp32
 *   scale FMAs in the same order, so they give bit-identical results; the
 *   split-K kernel and the GEMV add the same exact terms in another
 *   association (within fp32 rounding of them).  The result does not depend
 *   on the stream, on timing or on other calls.
 *   Zero-point heads (bits | LMH_ZP) run the same kernels with each row's
 *   per-group zero point subtracted from its codes while they are unpacked
 *   (n - z is exact in fp16), so the arithmetic is otherwise the same.
 */
int lmhead_logits(const void* x, int x_dtype, int64_t M, const void* packed, int64_t V, int64_t K,
                  int bits, int64_t group, int scale_dtype, const float* bias, float* y,
                  int64_t ldy, void* workspace, size_t ws_bytes, void* stream);

/*
 * lmhead_logits_path -- lmhead_logits with the kernel chosen by the caller:
 *   path 0 = automatic (exactly lmhead_logits), 1 = the lane-per-row GEMV
 *   (M <= 4, else LMH_E_UNSUPPORTED), 2 = the MFMA kernel with B operands
 *   loaded straight into registers (any M), 3 = the MFMA kernel with every
 *   operand staged in LDS by direct global-to-LDS loads (any M; 32 or 64
 *   activation rows per workgroup), 4 = the activation-resident MFMA kernel
 *   (a 32-row (M <= 32) or 64-row activation tile held in LDS for the
 *   workgroup's life, weights streamed through registers; K <= 1024, else
 *   LMH_E_UNSUPPORTED), 5 = the split-K MFMA kernel (a 64-row block split
 *   along K over up to 8 waves, every load of a wave issued up front, the
 *   waves' partial tiles added in wave order through LDS; M <= 16, else
 *   LMH_E_UNSUPPORTED).  Paths 2-4 give bit-identical results; path 5 adds
 *   the same per-group products and scale FMAs, but its K partial sums
 *   associate differently (as the GEMV's do), so it agrees with them to
 *   within fp32 rounding.  All
 *   kernels compute the same function; this entry point exists to test and
 *   time each of them on the same shapes.
 */
int lmhead_logits_path(const void* x, int x_dtype, int64_t M, const void* packed, int64_t V,
                       int64_t K, int bits, int64_t group, int scale_dtype, const float* bias,
                       float* y, int64_t ldy, void* workspace, size_t ws_bytes, int path,
                       void* stream);

/*
 * lmhead_logits_auto_path_x -- the kernel lmhead_logits (path 0) runs for a
 *   head of the given shape and activation type, as a lmhead_logits_path
 *   number (1..5), in *path.  Host only: no device work, no GPU needed.
 *   M >= 1; K, bits (4 or 8, optionally | LMH_ZP), group and x_dtype (LMH_F16
 *   or LMH_BF16) as for lmhead_logits.  Returns LMH_OK, LMH_E_NULL (path
 *   NULL), LMH_E_SHAPE, LMH_E_DTYPE or LMH_E_UNSUPPORTED (invalid shape,
 *   type or width, as lmhead_logits would report); *path is written only on
 *   LMH_OK.  The choice depends on M, K, the code width, G and, at M = 2
 *   only, on x_dtype (bf16 rows stay on the GEMV, which needs no workspace).
 */
int lmhead_logits_auto_path_x(int64_t M, int64_t K, int bits, int64_t group, int x_dtype,
                              int* path);

/* lmhead_logits_auto_path -- lmhead_logits_auto_path_x for fp16 activations. */
int lmhead_logits_auto_path(int64_t M, int64_t K, int bits, int64_t group, int* path);

/*
 * lmhead_logits_typed -- lmhead_logits_path with the output type chosen by
 *   the caller: y_dtype LMH_F32 (exactly lmhead_logits_path), LMH_F16 or
 *   LMH_BF16.  The arithmetic is unchanged; the final fp32 value (after the
 *   bias and the bf16 row exponent) is rounded once to the 16-bit type,
 *   nearest even; an fp16 value beyond its range becomes +-inf.  16-bit
 *   logits halve the output bytes (M * V * 2), which at large M are the
 *   largest single cost of the call; the rounding adds up to 2^-11 (fp16) or
 *   2^-8 (bf16) of |y| to the error (vLLM's logits leave the head in the
 *   activation dtype).  y needs 2-byte alignment for 16-bit types.
 */
int lmhead_logits_typed(const void* x, int x_dtype, int64_t M, const void* packed, int64_t V,
                        int64_t K, int bits, int64_t group, int scale_dtype, const float* bias,
                        void* y, int y_dtype, int64_t ldy, void* workspace, size_t ws_bytes,
                        int path, void* stream);

/*
 * lmhead_dense_logits -- y[m, v] = sum_k x[m,k] * W[v,k] with an unquantized
 *   16-bit weight: the bandwidth control of the fp16 logits GEMV (vLLM PR
 *   #48870, review comment, point 1).  fp32 accumulation.
 *   x [M, K] and W [V, K] row-major, both LMH_F16 or both LMH_BF16; K % 8 == 0.
 *   y [M, ldy] fp32, ldy >= V (4-byte alignment).  M <= 4.
 */
int lmhead_dense_logits(const void* x, int x_dtype, int64_t M, const void* w, int w_dtype,
                        int64_t V, int64_t K, float* y, int64_t ldy, void* stream);

/*
 * lmhead_topk_workspace_bytes -- device workspace lmhead_topk_rescore needs.
 */
size_t lmhead_topk_workspace_bytes(int64_t M, int64_t V, int topk);

/*
 * lmhead_topk_rescore -- exact rescoring of the top-K quantized logits (vLLM
 *   PR #48870, review comment, point 2: the K largest quantized logits of a row
 *   are overwritten by exact dot products with the unquantized weight rows).
 *   For each row m of y [M, ldy] (fp32, in/out):
 *     I = the topk largest of y[m, 0..V), ordered by value descending, then
 *         index ascending;
 *     for v in I: y[m, v] = sum_k x[m,k] * w_ref[v,k] in fp32 (fixed
 *         summation order; error within gamma_K * sum |x w|);
 *     idx_out[m, t] = I[t]  (int32), val_out[m, t] = the new y[m, I[t]];
 *     top1_out[m] = the first (lowest-index) maximum of the updated row.
 *   x [M, K] LMH_F16 or LMH_BF16; w_ref [V, K] LMH_F16, LMH_BF16 or LMH_F32,
 *   row-major (only the topk selected rows are read).  1 <= topk <= 64,
 *   topk <= V and V <= 2097152 (LMH_E_UNSUPPORTED beyond).  Any of idx_out /
 *   val_out / top1_out may be NULL.  Alignment: x 2 bytes, w_ref and y
 *   4 bytes, workspace 16 bytes.
 *   workspace: at least lmhead_topk_workspace_bytes(M, V, topk) bytes; its
 *   contents on entry do not matter.
 *   Deterministic: the selection is unique under the order (-0 equals +0)
 *   and every sum has a fixed order.  NaN logits rank below every number;
 *   the result is then still memory-safe but otherwise unspecified.
 */
int lmhead_topk_rescore(const void* x, int x_dtype, int64_t M, const void* w_ref, int w_dtype,
                        int64_t V, int64_t K, float* y, int64_t ldy, int topk, int32_t* idx_out,
                        float* val_out, int32_t* top1_out, void* workspace, size_t ws_bytes,
                        void* stream);

/*
 * lmhead_logits_topk_workspace_bytes -- device workspace lmhead_logits_topk
 *   needs (0 for invalid arguments).
 */
size_t lmhead_logits_topk_workspace_bytes(int64_t M, int64_t V, int64_t K, int x_dtype, int topk);

/*
 * lmhead_logits_topk -- the quantized logits and exact top-K rescoring in one
 *   call (vLLM PR #48870, review comment, point 2: top-K of the quantized
 *   logits, those K rows recomputed exactly from the unquantized weight).
 *   Result: exactly that of lmhead_logits followed by lmhead_topk_rescore on
 *   the same y -- idx_out, val_out, top1_out and, when y is given, y with the
 *   rescored values scattered in.  y [M, ldy] fp32 may be NULL: the logits
 *   then live in the workspace only.  Arguments otherwise as for
 *   lmhead_logits and lmhead_topk_rescore (same shape rules, alignment,
 *   dtypes and V <= 2097152); topk 1..64, topk <= V.
 *   One activation row (M = 1, the decode case) with topk <= 16 and at most
 *   4096 row blocks (V <= 262144) takes a fused path: the GEMV itself writes
 *   each 64-row block's sorted top-(topk+1) list of its fp32 logits, and one
 *   merge kernel selects and rescores -- no second pass over the logits, and
 *   with y NULL the logits are never stored.  The result is the same.
 *   workspace: at least lmhead_logits_topk_workspace_bytes(M, V, K, x_dtype,
 *   topk) bytes, 16-byte aligned; contents on entry do not matter.
 */
int lmhead_logits_topk(const void* x, int x_dtype, int64_t M, const void* packed, int64_t V,
                       int64_t K, int bits, int64_t group, int scale_dtype, const float* bias,
                       const void* w_ref, int w_dtype, int topk, float* y, int64_t ldy,
                       int32_t* idx_out, float* val_out, int32_t* top1_out, void* workspace,
                       size_t ws_bytes, void* stream);

/*
 * lmhead_logits_topk_noalloc -- lmhead_logits_topk for callers that cannot
 *   allocate device memory: code under HIP graph capture, tight serving
 *   loops, harnesses that forbid hipMalloc.  Same arguments, result and
 *   rules as lmhead_logits_topk, without the workspace: the call uses a
 *   16 MiB scratch array inside the library instead (one per GPU, held until
 *   the process ends; its device address is looked up on the call's first use
 *   of a device, which must be the current device).  Calls no hipMalloc,
 *   hipFree or other allocating routine.  A call whose working set -- the
 *   workspace bytes it actually uses, i.e. the lmhead_logits_topk workspace
 *   without the logits region when y is given or the fused one-row path runs
 *   -- exceeds the scratch returns LMH_E_SCRATCH before any launch.  The
 *   scratch keeps the last call's contents (none of it needs clearing); every
 *   call on one GPU shares it, so calls that may overlap on one GPU (other
 *   streams, other host threads) race and must be serialised by the caller.
 */
int lmhead_logits_topk_noalloc(const void* x, int x_dtype, int64_t M, const void* packed,
                               int64_t V, int64_t K, int bits, int64_t group, int scale_dtype,
                               const float* bias, const void* w_ref, int w_dtype, int topk,
                               float* y, int64_t ldy, int32_t* idx_out, float* val_out,
                               int32_t* top1_out, void* stream);

/*
 * lmhead_stream_read -- a measurement aid, not part of the logits path: reads
 *   `bytes` bytes at src (one pass, 16-byte loads, nothing stored except by
 *   chance into sink) -- the practical HBM read rate a logits kernel that
 *   reads the same bytes is measured against.  bytes % 16 == 0; src 16-byte
 *   aligned; sink >= 1024 bytes, 4-byte aligned, contents afterwards
 *   undefined.  bytes == 0 is a valid empty call.
 */
int lmhead_stream_read(const void* src, size_t bytes, void* sink, void* stream);

/*
 * lmhead_stream_mix -- a measurement aid, not part of the logits path: reads
 *   read_bytes bytes at src once and writes write_bytes bytes at dst once
 *   (16-byte accesses; each 256-thread workgroup reads 16 KiB and then writes
 *   its share) -- the practical HBM rate for a logits call's mix of weight
 *   reads and logit writes beyond one activation row, where the writes are a
 *   large part of the bytes.  dst receives a function of the words read:
 *   thread t of workgroup b writes words b*W*256 + 256*i + t (i < W,
 *   W = ceil((write_bytes/16) / (256 * number of workgroups)), number of
 *   workgroups = max(1, ceil(read_bytes / 16384))) with the XOR of the words
 *   b*1024 + 256*j + t (j < 4) it read, plus i in the first 32-bit lane;
 *   only words below the ends are accessed.  Both sizes multiples of 16 (else
 *   LMH_E_SHAPE), both pointers 16-byte aligned (LMH_E_ALIGN); a pointer
 *   whose size is 0 may be NULL; both 0 is a valid empty call.
 */
int lmhead_stream_mix(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                      void* stream);

/*
 * lmhead_mfma_ceiling -- a measurement aid, not part of the logits path: the
 *   practical rate of the 16x16x32 fp16 MFMA (the instruction of the MFMA
 *   logits kernels) on a grid of one 16-wave workgroup per CU, each wave
 *   running `rounds` rounds of 8 independent MFMA chains on register
 *   operands (no memory traffic), and with valu_per_mfma = 2 or 4 as many
 *   independent fp32 FMAs beside each MFMA (the scale FMAs of a G-column
 *   group are 128 / G per MFMA) -- how much the VALU work of a kernel adds
 *   to its MFMA time.  rounds in [1, 2^31 - 1] (else LMH_E_SHAPE);
 *   valu_per_mfma 0, 2 or 4 (else LMH_E_UNSUPPORTED); sink (device, not
 *   NULL) receives one float per thread, 256 * 1024 floats, contents
 *   undefined.  lmhead_mfma_ceiling_mfmas(rounds) is the number of MFMAs one
 *   call issues (each 16 * 16 * 32 * 2 flops), 0 for rounds out of range.
 */
int lmhead_mfma_ceiling(int64_t rounds, int valu_per_mfma, float* sink, void* stream);
int64_t lmhead_mfma_ceiling_mfmas(int64_t rounds);

#ifdef __cplusplus
}
#endif

#endif /* LMHEAD_H */
