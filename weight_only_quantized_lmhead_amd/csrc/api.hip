// C ABI of liblmhead.so (declared in include/lmhead.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so each error path can be exercised without a GPU.  Work is
// enqueued on the caller's stream; nothing here allocates or synchronises.
#include "lmh_internal.h"
#include "lmhead.h"

#include <algorithm>
#include <atomic>
#include <mutex>

namespace {

using lmh::BF16;
using lmh::F16;
using lmh::F32;

constexpr int kAbiVersion = 2;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape rules shared by pack and logits.
int check_layout(int64_t V, int64_t K, int bits, int64_t G) {
    if (bits != 4 && bits != 8) return LMH_E_UNSUPPORTED;
    if (V < 0 || V >= (int64_t(1) << 31)) return LMH_E_SHAPE;
    if (K < 1 || K > 65536 || G < 32 || G > K) return LMH_E_SHAPE;
    const int64_t span = lmh::span_of(bits);
    if (K % span != 0 || K % G != 0 || G % 32 != 0) return LMH_E_SHAPE;
    // a group is either a whole number of superchunks or divides one
    if (!(G % span == 0 || span % G == 0)) return LMH_E_UNSUPPORTED;
    return LMH_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? LMH_OK : LMH_E_HIP; }

// Scratch of lmhead_logits_topk_noalloc, for callers that cannot allocate: a
// file-scope device array (each GPU the library runs on holds its own copy
// until the process ends).  Its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// passed to kernels: in host code the array's name is not a device address.
constexpr size_t kScratchBytes = (size_t)16 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return LMH_E_HIP;
    if (dev < 0 || dev >= kMaxDevices) return LMH_E_UNSUPPORTED;
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void* q = nullptr;
            if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return LMH_E_HIP;
            g_scratch_addr[dev].store(q, std::memory_order_release);
            p = q;
        }
    }
    *out = p;
    return LMH_OK;
}

// A `bits` argument: the code width, optionally with LMH_ZP (zero-point form).
// Quantizer launches: one wavefront per unit, four per workgroup, the
// workgroup count rounded up to a multiple of 8; the grid's work-item count
// must fit the dispatch packet's 32-bit size.
bool quant_grid_fits(int64_t units) {
    return ((units + 3) / 4 + 7) / 8 * 8 * 256 < (int64_t(1) << 32);
}

struct Width {
    int bits;
    bool zp;
};
Width width_of(int b) { return {b & ~LMH_ZP, (b & LMH_ZP) != 0}; }

}  // namespace

extern "C" {

const char* lmhead_status_string(int status) {
    switch (status) {
    case LMH_OK: return "LMH_OK";
    case LMH_E_NULL: return "LMH_E_NULL: a required pointer is NULL";
    case LMH_E_SHAPE: return "LMH_E_SHAPE: size out of range or inconsistent";
    case LMH_E_DTYPE: return "LMH_E_DTYPE: dtype not allowed for this argument";
    case LMH_E_ALIGN: return "LMH_E_ALIGN: pointer not 16-byte aligned";
    case LMH_E_UNSUPPORTED: return "LMH_E_UNSUPPORTED: combination not implemented";
    case LMH_E_WORKSPACE: return "LMH_E_WORKSPACE: workspace missing or too small";
    case LMH_E_HIP: return "LMH_E_HIP: the HIP runtime reported an error";
    case LMH_E_SCRATCH:
        return "LMH_E_SCRATCH: the call needs more than the 16 MiB scratch of the "
               "allocation-free entry point";
    default: return "unknown lmhead status";
    }
}

int lmhead_abi_version(void) { return kAbiVersion; }

size_t lmhead_packed_bytes(int64_t V, int64_t K, int bits_arg, int64_t group) {
    const Width wd = width_of(bits_arg);
    if (check_layout(V, K, wd.bits, group) != LMH_OK) return 0;
    const int64_t vpad = (V + 63) / 64 * 64;
    return (size_t)(vpad * K * wd.bits / 8 + vpad * (K / group) * (wd.zp ? 3 : 2));
}

static int quantize_impl(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t group,
                         int scale_dtype, int clip, int8_t* q_out, void* s_out, uint8_t* z_out,
                         bool zp, void* stream) {
    if (bits != 4 && bits != 8) return LMH_E_UNSUPPORTED;
    if (zp && clip != LMH_CLIP_RTN) return LMH_E_UNSUPPORTED;
    if (w_dtype != F32 && w_dtype != F16 && w_dtype != BF16) return LMH_E_DTYPE;
    if (scale_dtype != F16 && scale_dtype != BF16) return LMH_E_DTYPE;
    if (clip != LMH_CLIP_RTN && clip != LMH_CLIP_MSE) return LMH_E_UNSUPPORTED;
    if (V < 0 || K < 1 || group < 32 || group % 32 != 0 || K % group != 0) return LMH_E_SHAPE;
    if (V * K >= (int64_t(1) << 40)) return LMH_E_SHAPE;
    if (!quant_grid_fits((V + 63) / 64 * (K / group))) return LMH_E_UNSUPPORTED;
    if (V == 0) return LMH_OK;
    if (!w || !q_out || !s_out || (zp && !z_out)) return LMH_E_NULL;
    if (!aligned16(w) || !aligned16(q_out)) return LMH_E_ALIGN;
    if (((uintptr_t)s_out & 1u) != 0) return LMH_E_ALIGN;
    return from_hip(lmh::launch_quantize(w, w_dtype, V, K, bits, group, scale_dtype,
                                         clip == LMH_CLIP_MSE ? 5 : 1, q_out, (uint16_t*)s_out,
                                         zp ? z_out : nullptr, (hipStream_t)stream));
}

int lmhead_quantize(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t group,
                    int scale_dtype, int clip, int8_t* q_out, void* s_out, void* stream) {
    return quantize_impl(w, w_dtype, V, K, bits, group, scale_dtype, clip, q_out, s_out, nullptr,
                         false, stream);
}

int lmhead_quantize_zp(const void* w, int w_dtype, int64_t V, int64_t K, int bits, int64_t group,
                       int scale_dtype, uint8_t* n_out, void* s_out, uint8_t* z_out,
                       void* stream) {
    return quantize_impl(w, w_dtype, V, K, bits & ~LMH_ZP, group, scale_dtype, LMH_CLIP_RTN,
                         (int8_t*)n_out, s_out, z_out, true, stream);
}

int lmhead_quantize_pack(const void* w, int w_dtype, int64_t ldw, int64_t V, int64_t K,
                         int bits_arg, int64_t group, int scale_dtype, int clip, int64_t row0,
                         int64_t rows, void* packed_out, void* stream) {
    const Width wd = width_of(bits_arg);
    const int bits = wd.bits;
    const int rc = check_layout(V, K, bits, group);
    if (rc != LMH_OK) return rc;
    if (w_dtype != F32 && w_dtype != F16 && w_dtype != BF16) return LMH_E_DTYPE;
    if (scale_dtype != F16 && scale_dtype != BF16) return LMH_E_DTYPE;
    if (clip != LMH_CLIP_RTN && clip != LMH_CLIP_MSE) return LMH_E_UNSUPPORTED;
    if (wd.zp && clip != LMH_CLIP_RTN) return LMH_E_UNSUPPORTED;
    if (row0 < 0 || rows < 0 || row0 > V || rows > V - row0 || row0 % 64 != 0) return LMH_E_SHAPE;
    if (rows % 64 != 0 && row0 + rows != V) return LMH_E_SHAPE;
    if (ldw < K || ldw % 8 != 0) return LMH_E_SHAPE;
    if (rows == 0) return LMH_OK;
    // one wavefront per (64-row block, superchunk or group), four per workgroup
    const int64_t units = (rows + 63) / 64 * (K / std::max<int64_t>(group, lmh::span_of(bits)));
    if (!quant_grid_fits(units)) return LMH_E_UNSUPPORTED;
    if (!w || !packed_out) return LMH_E_NULL;
    if (!aligned16(w) || !aligned16(packed_out)) return LMH_E_ALIGN;
    return from_hip(lmh::launch_quantize_pack(w, w_dtype, ldw, V, K, bits, group, scale_dtype,
                                              clip == LMH_CLIP_MSE ? 5 : 1, wd.zp, row0, rows,
                                              (uint8_t*)packed_out, (hipStream_t)stream));
}

static int pack_impl(const int8_t* q, const void* s, const uint8_t* z, bool zp, int64_t V,
                     int64_t K, int bits, int64_t group, void* packed_out, void* stream) {
    const int rc = check_layout(V, K, bits, group);
    if (rc != LMH_OK) return rc;
    if (V == 0) return LMH_OK;
    if (!q || !s || !packed_out || (zp && !z)) return LMH_E_NULL;
    if (!aligned16(q) || !aligned16(packed_out)) return LMH_E_ALIGN;
    if (((uintptr_t)s & 1u) != 0) return LMH_E_ALIGN;
    return from_hip(lmh::launch_pack(q, (const uint16_t*)s, zp ? z : nullptr, V, K, bits, group,
                                     (uint8_t*)packed_out, (hipStream_t)stream));
}

int lmhead_pack(const int8_t* q, const void* s, int64_t V, int64_t K, int bits, int64_t group,
                void* packed_out, void* stream) {
    return pack_impl(q, s, nullptr, false, V, K, bits, group, packed_out, stream);
}

int lmhead_pack_zp(const uint8_t* n, const void* s, const uint8_t* z, int64_t V, int64_t K,
                   int bits, int64_t group, void* packed_out, void* stream) {
    return pack_impl((const int8_t*)n, s, z, true, V, K, bits & ~LMH_ZP, group, packed_out, stream);
}

int lmhead_embed(const int32_t* ids, int64_t T, const void* packed, int64_t V, int64_t K,
                 int bits_arg, int64_t group, int scale_dtype, void* out, int out_dtype, int64_t ldo,
                 void* stream) {
    const Width wd = width_of(bits_arg);
    const int bits = wd.bits;
    const int rc = check_layout(V, K, bits, group);
    if (rc != LMH_OK) return rc;
    if (scale_dtype != F16 && scale_dtype != BF16) return LMH_E_DTYPE;
    if (out_dtype != F32 && out_dtype != F16 && out_dtype != BF16) return LMH_E_DTYPE;
    if (T < 0 || ldo < K) return LMH_E_SHAPE;
    if (T == 0) return LMH_OK;
    if (!ids || !packed || !out) return LMH_E_NULL;
    if (!aligned16(packed) || !aligned16(out) || ((uintptr_t)ids & 3u) != 0) return LMH_E_ALIGN;
    if (ldo % (out_dtype == F32 ? 4 : 8) != 0) return LMH_E_ALIGN;  // rows stay 16-byte aligned
    // one thread per (token, 16-byte slot), 256 per workgroup
    const int64_t threads = T * (K / lmh::span_of(bits)) * 4;
    if ((threads + 255) / 256 >= (int64_t(1) << 31)) return LMH_E_UNSUPPORTED;
    return from_hip(lmh::launch_embed(ids, T, (const uint8_t*)packed, V, K, bits, group,
                                      scale_dtype, wd.zp, out, out_dtype, ldo,
                                      (hipStream_t)stream));
}

size_t lmhead_logits_workspace_bytes(int64_t M, int64_t K, int x_dtype) {
    if (x_dtype != BF16 || M <= 0 || K <= 0) return 0;
    return (size_t)(((M * K * 2 + 255) / 256) * 256 + ((M * 4 + 255) / 256) * 256);
}

// `lists` (internal, lmhead_logits_topk's fused path): the GEMV also writes
// per-block top-`list_T` lists there, and y may be null.
//
// The automatic kernel choice (path 0), from sweeps over M = 2..256 on the
// 151936 x 1024 int4 g64 and int8 g128 heads and the 248064 x 5120 int4 g128
// head:
//   - the split-K MFMA kernel for 3..16 rows when K <= 2048 (us against the
//     best of the other kernels, M = 3 / 8 / 16: 151936 x 1024 int4 g64
//     18.9 / 18.0 / 20.9 vs 21.4 / 22.5 / 23.1; g128 16.7 / 17.5 / 20.3 vs
//     20.2 / 21.2 / 21.9; int8 g128 29.8 / 29.9 / 32.1 vs 32.5 / 32.4 /
//     33.4; 50304 x 512 g64 5.3 / 5.6 / 6.1 vs 6.9 / 7.2 / 7.4; 151936 x
//     2048 int8 per-row 54.0 / 56.4 / 61.8 vs 60.5 / 61.6 / 63.9); with
//     K = 5120 its two-buffer ring needs 132 registers and it loses from
//     M = 8 (144.7 vs 135.2), and with 32 rows (104 registers, 70 KiB of
//     LDS: half the waves) it loses to the activation-resident kernel;
//   - the GEMV for one activation row, and for two bf16 rows or two rows of
//     K > 2048 (it converts bf16 rows itself, with no workspace; at M = 2,
//     int4 K = 5120: 133 vs 141 us for the best MFMA kernel); two fp16 rows
//     of K <= 2048 run the split-K kernel (M = 2, us, alternated twice:
//     151936 x 1024 int4 g64 16.0-16.1 vs 17.1-17.2 for the GEMV, int8 g128
//     28.4-28.5 vs 29.8-29.9, 151936 x 2048 int8 per-row 52.9-53.1 vs
//     55.8-55.9, 50304 x 512 g64 5.66-5.68 vs 6.35-6.40);
//   - when K <= 1024 and G >= 64, the activation-resident kernel from 33
//     rows on (int4 M = 33..64: 29-33 us against 38-42 for the LDS-staged
//     kernel's 64-row tiles; M = 96..256 6-10 % faster; int8 M = 40..256:
//     0-14 % faster; with 32-column groups it runs out of registers), and
//     on int4 heads from 17 rows on (its 32-row tile: 7.6-7.8 us against
//     8.3-9.2 on the 50304 x 512 g64 head, within 3 % of the LDS-staged
//     kernel on the 151936 x 1024 g64 and g128 heads);
//   - when K <= 1024: the LDS-staged kernel for 17..32 rows on the other
//     heads and for every M >= 3 on int8 heads (int8 3..32 rows: 4-8 %
//     faster than the activation-resident kernel's 32-row tile), else the
//     register-fed kernel (3..16 rows on int4 heads; the LDS-staged one is
//     2-15 % slower there);
//   - when K > 1024: the register-fed kernel for 25..32 rows (3 % faster),
//     else the LDS-staged one (3..24 rows: 1.5-3 % faster; beyond 32 rows
//     the register-fed kernel would read the weights once per 32 rows).
static int auto_path(int64_t M, int64_t K, int bits, int64_t group, bool x_bf16) {
    if (M <= lmh::kGemvAutoMaxM && M <= lmh::kGemvMaxM && M * K <= lmh::kGemvMaxMK)
        return M == 2 && !x_bf16 && K <= 2048 ? 5 : 1;
    if (M <= 16 && K <= 2048) return 5;
    if (M > 16 && lmh::xres_fits(K) && group >= 64 && (M > 32 || bits == 4)) return 4;
    const bool narrow = K <= 1024;
    const bool lds = narrow ? (M > 16 || bits == 8) : !(M > 24 && M <= 32);
    return lds ? 3 : 2;
}

static int logits_impl(const void* x, int x_dtype, int64_t M, const void* packed, int64_t V,
                       int64_t K, int bits_arg, int64_t group, int scale_dtype, const float* bias,
                       void* y, int y_dtype, int64_t ldy, void* workspace, size_t ws_bytes,
                       void* stream, int path, lmh::u64* lists = nullptr, int list_T = 0) {
    const Width wd = width_of(bits_arg);
    const int bits = wd.bits;
    int rc = check_layout(V, K, bits, group);
    if (rc != LMH_OK) return rc;
    if (x_dtype != F16 && x_dtype != BF16) return LMH_E_DTYPE;
    if (scale_dtype != F16 && scale_dtype != BF16) return LMH_E_DTYPE;
    if (M < 0 || M > 65535) return LMH_E_SHAPE;
    if (path < 0 || path > 5) return LMH_E_UNSUPPORTED;
    if (M == 0 || V == 0) return LMH_OK;
    if (y && ldy < V) return LMH_E_SHAPE;
    if (!x || !packed || (!y && !lists)) return LMH_E_NULL;
    if (!aligned16(x) || !aligned16(packed)) return LMH_E_ALIGN;
    if (y_dtype != F32 && y_dtype != F16 && y_dtype != BF16) return LMH_E_DTYPE;
    if (((uintptr_t)y & (y_dtype == F32 ? 3u : 1u)) != 0) return LMH_E_ALIGN;
    if (bias && ((uintptr_t)bias & 3u) != 0) return LMH_E_ALIGN;
    // the MFMA launch has one workgroup per (256 rows, 16..32 activations)
    if ((V + 255) / 256 * ((M + 15) / 16) >= (int64_t(1) << 30)) return LMH_E_UNSUPPORTED;
    const bool gemv_ok = M <= lmh::kGemvMaxM && M * K <= lmh::kGemvMaxMK;
    if (path == 1 && !gemv_ok) return LMH_E_UNSUPPORTED;
    if (path == 4 && !lmh::xres_fits(K)) return LMH_E_UNSUPPORTED;
    if (path == 5 && M > lmh::kSplitkMaxM) return LMH_E_UNSUPPORTED;
    if (path == 0) path = auto_path(M, K, bits, group, x_dtype == BF16);
    // bf16 rows: the GEMV converts them itself; the MFMA kernels take them
    // converted to fp16 (with a row exponent) in the workspace
    const bool convert = x_dtype == BF16 && path != 1;
    if (convert) {
        const size_t need = lmhead_logits_workspace_bytes(M, K, x_dtype);
        if (!workspace || ws_bytes < need) return LMH_E_WORKSPACE;
        if (!aligned16(workspace)) return LMH_E_ALIGN;
    }

    hipStream_t st = (hipStream_t)stream;
    lmh::LogitsArgs a;
    a.x = x;
    a.x_bf16 = x_dtype == BF16 && path == 1;
    a.xexp = nullptr;
    if (convert) {
        _Float16* xh = (_Float16*)workspace;
        int* xe = (int*)((char*)workspace + ((M * K * 2 + 255) / 256) * 256);
        hipError_t e = lmh::launch_x_to_f16((const uint16_t*)x, (int)M, (int)K, xh, xe, st);
        if (e != hipSuccess) return LMH_E_HIP;
        a.x = xh;
        a.xexp = xe;
    }
    a.packed = (const uint8_t*)packed;
    a.bias = bias;
    a.y = y;
    a.y_dtype = y_dtype;
    a.ldy = ldy;
    a.V = V;
    a.K = K;
    a.G = group;
    a.M = (int)M;
    a.bits = bits;
    a.scale_bf16 = scale_dtype == BF16;
    a.zp = wd.zp;
    a.lists = lists;
    a.list_T = list_T;
    if (path == 1) return from_hip(lmh::launch_gemv(a, st));
    if (path == 4) return from_hip(lmh::launch_mfma_xres(a, st));
    if (path == 5) return from_hip(lmh::launch_mfma_splitk(a, st));
    return from_hip(path == 3 ? lmh::launch_mfma_lds(a, st) : lmh::launch_mfma(a, st));
}

int lmhead_logits_auto_path_x(int64_t M, int64_t K, int bits_arg, int64_t group, int x_dtype,
                              int* path) {
    if (!path) return LMH_E_NULL;
    const Width wd = width_of(bits_arg);
    const int rc = check_layout(1, K, wd.bits, group);
    if (rc != LMH_OK) return rc;
    if (x_dtype != F16 && x_dtype != BF16) return LMH_E_DTYPE;
    if (M < 1 || M > 65535) return LMH_E_SHAPE;
    *path = auto_path(M, K, wd.bits, group, x_dtype == BF16);
    return LMH_OK;
}

int lmhead_logits_auto_path(int64_t M, int64_t K, int bits_arg, int64_t group, int* path) {
    return lmhead_logits_auto_path_x(M, K, bits_arg, group, F16, path);
}

int lmhead_logits(const void* x, int x_dtype, int64_t M, const void* packed, int64_t V, int64_t K,
                  int bits, int64_t group, int scale_dtype, const float* bias, float* y,
                  int64_t ldy, void* workspace, size_t ws_bytes, void* stream) {
    return logits_impl(x, x_dtype, M, packed, V, K, bits, group, scale_dtype, bias, y, F32, ldy,
                       workspace, ws_bytes, stream, 0);
}

int lmhead_logits_path(const void* x, int x_dtype, int64_t M, const void* packed, int64_t V,
                       int64_t K, int bits, int64_t group, int scale_dtype, const float* bias,
                       float* y, int64_t ldy, void* workspace, size_t ws_bytes, int path,
                       void* stream) {
    return logits_impl(x, x_dtype, M, packed, V, K, bits, group, scale_dtype, bias, y, F32, ldy,
                       workspace, ws_bytes, stream, path);
}

int lmhead_logits_typed(const void* x, int x_dtype, int64_t M, const void* packed, int64_t V,
                        int64_t K, int bits, int64_t group, int scale_dtype, const float* bias,
                        void* y, int y_dtype, int64_t ldy, void* workspace, size_t ws_bytes,
                        int path, void* stream) {
    return logits_impl(x, x_dtype, M, packed, V, K, bits, group, scale_dtype, bias, y, y_dtype,
                       ldy, workspace, ws_bytes, stream, path);
}

int lmhead_dense_logits(const void* x, int x_dtype, int64_t M, const void* w, int w_dtype,
                        int64_t V, int64_t K, float* y, int64_t ldy, void* stream) {
    if (x_dtype != F16 && x_dtype != BF16) return LMH_E_DTYPE;
    if (w_dtype != x_dtype) return LMH_E_DTYPE;
    if (M < 0 || M > 4 || V < 0 || V >= (int64_t(1) << 31)) return LMH_E_SHAPE;
    if (K < 8 || K % 8 != 0 || K > 65536) return LMH_E_SHAPE;
    if (M == 0 || V == 0) return LMH_OK;
    if (ldy < V) return LMH_E_SHAPE;
    if (!x || !w || !y) return LMH_E_NULL;
    if (!aligned16(x) || !aligned16(w) || ((uintptr_t)y & 3u) != 0) return LMH_E_ALIGN;
    return from_hip(lmh::launch_dense(x, x_dtype, (int)M, w, V, K, y, ldy, (hipStream_t)stream));
}

size_t lmhead_topk_workspace_bytes(int64_t M, int64_t V, int topk) {
    if (M <= 0 || V <= 0 || topk < 1 || topk > 64) return 0;
    return lmh::topk_ws_bytes(M, V, topk);
}

int lmhead_topk_rescore(const void* x, int x_dtype, int64_t M, const void* w_ref, int w_dtype,
                        int64_t V, int64_t K, float* y, int64_t ldy, int topk, int32_t* idx_out,
                        float* val_out, int32_t* top1_out, void* workspace, size_t ws_bytes,
                        void* stream) {
    if (x_dtype != F16 && x_dtype != BF16) return LMH_E_DTYPE;
    if (w_dtype != F16 && w_dtype != BF16 && w_dtype != F32) return LMH_E_DTYPE;
    if (M < 0 || M > 65535 || V < 0 || V >= (int64_t(1) << 31) || K < 1 || K > 65536)
        return LMH_E_SHAPE;
    if (topk < 1 || topk > 64) return LMH_E_SHAPE;
    if (M == 0 || V == 0) return LMH_OK;
    if (topk > V || ldy < V) return LMH_E_SHAPE;
    if (V > lmh::topk_max_v()) return LMH_E_UNSUPPORTED;
    if (!x || !w_ref || !y) return LMH_E_NULL;
    if (((uintptr_t)x & 1u) != 0 || ((uintptr_t)w_ref & 3u) != 0 || ((uintptr_t)y & 3u) != 0)
        return LMH_E_ALIGN;
    const size_t need = lmh::topk_ws_bytes(M, V, topk);
    if (!workspace || ws_bytes < need) return LMH_E_WORKSPACE;
    if (!aligned16(workspace)) return LMH_E_ALIGN;
    return from_hip(lmh::launch_topk_rescore(x, x_dtype, (int)M, w_ref, w_dtype, V, K, y, ldy, topk,
                                             idx_out, val_out, top1_out, workspace,
                                             (hipStream_t)stream));
}

static int64_t round256(int64_t n) { return (n + 255) / 256 * 256; }

// Workspace of lmhead_logits_topk: [x conversion][top-K lists (pass-1 lists,
// or the fused GEMV's per-block lists, whichever is larger)][fp32 logits
// scratch, used when y is NULL on the unfused path]; every region rounded up
// to 256 bytes.
static int64_t topk_lists_region(int64_t M, int64_t V, int topk) {
    return std::max(round256((int64_t)lmh::topk_ws_bytes(M, V, topk)),
                    round256((int64_t)lmh::topk_fused_lists_bytes(M, V, topk)));
}

size_t lmhead_logits_topk_workspace_bytes(int64_t M, int64_t V, int64_t K, int x_dtype, int topk) {
    if (M <= 0 || V <= 0 || K <= 0 || topk < 1 || topk > 64) return 0;
    if (x_dtype != F16 && x_dtype != BF16) return 0;
    return (size_t)(round256((int64_t)lmhead_logits_workspace_bytes(M, K, x_dtype)) +
                    topk_lists_region(M, V, topk) + round256(M * V * 4));
}

// lmhead_logits_topk on a given workspace.  `exact`: the workspace may be
// the exact bytes this call uses (the logits region only when y is NULL on the
// unfused path); otherwise it must hold lmhead_logits_topk_workspace_bytes.
static int logits_topk_impl(const void* x, int x_dtype, int64_t M, const void* packed, int64_t V,
                            int64_t K, int bits, int64_t group, int scale_dtype, const float* bias,
                            const void* w_ref, int w_dtype, int topk, float* y, int64_t ldy,
                            int32_t* idx_out, float* val_out, int32_t* top1_out, void* workspace,
                            size_t ws_bytes, void* stream, bool exact, size_t* need_out = nullptr) {
    int rc = check_layout(V, K, bits & ~LMH_ZP, group);
    if (rc != LMH_OK) return rc;
    if (x_dtype != F16 && x_dtype != BF16) return LMH_E_DTYPE;
    if (scale_dtype != F16 && scale_dtype != BF16) return LMH_E_DTYPE;
    if (w_dtype != F16 && w_dtype != BF16 && w_dtype != F32) return LMH_E_DTYPE;
    if (M < 0 || M > 65535) return LMH_E_SHAPE;
    if (topk < 1 || topk > 64) return LMH_E_SHAPE;
    if (M == 0 || V == 0) return LMH_OK;
    if (topk > V) return LMH_E_SHAPE;
    if (y && ldy < V) return LMH_E_SHAPE;
    if (V > lmh::topk_max_v()) return LMH_E_UNSUPPORTED;
    if ((V + 255) / 256 * ((M + 15) / 16) >= (int64_t(1) << 30)) return LMH_E_UNSUPPORTED;
    if (!x || !packed || !w_ref) return LMH_E_NULL;
    if (!aligned16(x) || !aligned16(packed)) return LMH_E_ALIGN;
    if (((uintptr_t)w_ref & 3u) != 0 || (y && ((uintptr_t)y & 3u) != 0) ||
        (bias && ((uintptr_t)bias & 3u) != 0))
        return LMH_E_ALIGN;
    const int64_t xws = round256((int64_t)lmhead_logits_workspace_bytes(M, K, x_dtype));
    const int64_t tws = topk_lists_region(M, V, topk);
    // one activation row through the GEMV: its epilogue writes each 64-row
    // block's sorted top-T list, and one merge kernel selects and rescores
    // (no separate pass over the logits; y is stored only when given)
    // (the GEMV's top-K epilogue exists for one activation row only)
    const bool gemv_one = M == 1 && K <= lmh::kGemvMaxMK;
    const bool fused = gemv_one && lmh::topk_fused_ok(V, topk);
    const size_t need =
        exact ? (size_t)(xws + tws + (fused || y ? 0 : round256(M * V * 4)))
              : lmhead_logits_topk_workspace_bytes(M, V, K, x_dtype, topk);
    if (need_out) {
        *need_out = need;
        return LMH_OK;
    }
    if (!workspace || ws_bytes < need) return LMH_E_WORKSPACE;
    if (!aligned16(workspace)) return LMH_E_ALIGN;
    char* ws = (char*)workspace;
    if (fused) {
        const int T = (int)(topk + 1 <= V ? topk + 1 : V);
        lmh::u64* lists = (lmh::u64*)(ws + xws);
        rc = logits_impl(x, x_dtype, M, packed, V, K, bits, group, scale_dtype, bias, y, F32, ldy,
                         ws, (size_t)xws, stream, 1, lists, T);
        if (rc != LMH_OK) return rc;
        return from_hip(lmh::launch_topk_merge_rescore(lists, x, x_dtype, (int)M, w_ref, w_dtype, V,
                                                       K, y, ldy, topk, T, idx_out, val_out,
                                                       top1_out, (hipStream_t)stream));
    }
    float* yy = y ? y : (float*)(ws + xws + tws);
    const int64_t ly = y ? ldy : V;
    // the logits (automatic kernel), then the two top-K passes over them
    rc = logits_impl(x, x_dtype, M, packed, V, K, bits, group, scale_dtype, bias, yy, F32, ly, ws,
                     (size_t)xws, stream, 0);
    if (rc != LMH_OK) return rc;
    return from_hip(lmh::launch_topk_rescore(x, x_dtype, (int)M, w_ref, w_dtype, V, K, yy, ly, topk,
                                             idx_out, val_out, top1_out, ws + xws,
                                             (hipStream_t)stream));
}

int lmhead_logits_topk(const void* x, int x_dtype, int64_t M, const void* packed, int64_t V,
                       int64_t K, int bits, int64_t group, int scale_dtype, const float* bias,
                       const void* w_ref, int w_dtype, int topk, float* y, int64_t ldy,
                       int32_t* idx_out, float* val_out, int32_t* top1_out, void* workspace,
                       size_t ws_bytes, void* stream) {
    return logits_topk_impl(x, x_dtype, M, packed, V, K, bits, group, scale_dtype, bias, w_ref,
                            w_dtype, topk, y, ldy, idx_out, val_out, top1_out, workspace, ws_bytes,
                            stream, false);
}

int lmhead_logits_topk_noalloc(const void* x, int x_dtype, int64_t M, const void* packed,
                               int64_t V, int64_t K, int bits, int64_t group, int scale_dtype,
                               const float* bias, const void* w_ref, int w_dtype, int topk,
                               float* y, int64_t ldy, int32_t* idx_out, float* val_out,
                               int32_t* top1_out, void* stream) {
    // validation and the bytes this call needs, before any HIP call
    size_t need = 0;
    int rc = logits_topk_impl(x, x_dtype, M, packed, V, K, bits, group, scale_dtype, bias, w_ref,
                              w_dtype, topk, y, ldy, idx_out, val_out, top1_out, nullptr, 0, stream,
                              true, &need);
    if (rc != LMH_OK) return rc;
    if (M == 0 || V == 0) return LMH_OK;
    if (need > kScratchBytes) return LMH_E_SCRATCH;
    void* ws = nullptr;
    rc = scratch_of_current_device(&ws);
    if (rc != LMH_OK) return rc;
    return logits_topk_impl(x, x_dtype, M, packed, V, K, bits, group, scale_dtype, bias, w_ref,
                            w_dtype, topk, y, ldy, idx_out, val_out, top1_out, ws, kScratchBytes,
                            stream, true);
}

int lmhead_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
    if (bytes % 16 != 0 || bytes >= ((size_t)1 << 46)) return LMH_E_SHAPE;
    if (bytes / 16 / 768 >= ((size_t)1 << 31)) return LMH_E_UNSUPPORTED;
    if (bytes == 0) return LMH_OK;
    if (!src || !sink) return LMH_E_NULL;
    if (!aligned16(src) || ((uintptr_t)sink & 3u) != 0) return LMH_E_ALIGN;
    return from_hip(lmh::launch_stream_read(src, (int64_t)bytes, sink, (hipStream_t)stream));
}

int lmhead_stream_mix(const void* src, size_t read_bytes, void* dst, size_t write_bytes,
                      void* stream) {
    if (read_bytes % 16 != 0 || write_bytes % 16 != 0) return LMH_E_SHAPE;
    if (read_bytes >= ((size_t)1 << 46) || write_bytes >= ((size_t)1 << 46)) return LMH_E_SHAPE;
    int64_t grid, words;
    lmh::stream_mix_shape((int64_t)read_bytes, (int64_t)write_bytes, &grid, &words);
    // the grid's work-item count fits 32 bits; the per-thread word count an int
    if (grid * 256 >= (int64_t(1) << 32) || words >= (int64_t(1) << 31)) return LMH_E_UNSUPPORTED;
    if (read_bytes == 0 && write_bytes == 0) return LMH_OK;
    if ((read_bytes && !src) || (write_bytes && !dst)) return LMH_E_NULL;
    if (!aligned16(src) || !aligned16(dst)) return LMH_E_ALIGN;
    return from_hip(lmh::launch_stream_mix(src, (int64_t)read_bytes, dst, (int64_t)write_bytes,
                                           (hipStream_t)stream));
}

int64_t lmhead_mfma_ceiling_mfmas(int64_t rounds) {
    if (rounds < 1 || rounds > 0x7FFFFFFF) return 0;
    return rounds * 8 * 16 * (int64_t)lmh::mfma_ceiling_grid();
}

int lmhead_mfma_ceiling(int64_t rounds, int valu_per_mfma, float* sink, void* stream) {
    if (rounds < 1 || rounds > 0x7FFFFFFF) return LMH_E_SHAPE;
    if (valu_per_mfma != 0 && valu_per_mfma != 2 && valu_per_mfma != 4) return LMH_E_UNSUPPORTED;
    if (!sink) return LMH_E_NULL;
    return from_hip(lmh::launch_mfma_ceiling((int)rounds, valu_per_mfma, sink, (hipStream_t)stream));
}

}  // extern "C"
