// libmxfp4 C ABI: argument validation, device check, dispatch to the kernels.
// Every check runs before any launch and fails loudly with a status code and
// a thread-local detail message; there is no fallback path (the page
// "primus_turbo_mxfp4_local.py" turns mis-dispatch into a hard init-time error
// for the same reason: silent fallbacks hid wrong layouts and lost speed).

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "mx_internal.h"

namespace {

thread_local char g_last_error[512] = "";

mx_status fail(mx_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device cache of the gfx950 check: 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];

// The architecture name that replaces the device query (a test aid, set by
// mx_set_device_arch_override); empty = query the device.
char g_arch_override[64] = "";
std::atomic<bool> g_has_override{false};

bool arch_is_gfx950(const char *name) {
    // "gfx950" possibly followed by target features (":sramecc+:xnack-")
    return std::strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':');
}

int query_supported(int dev) {
    if (g_has_override.load(std::memory_order_acquire)) return arch_is_gfx950(g_arch_override) ? 1 : 0;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    return arch_is_gfx950(prop.gcnArchName) ? 1 : 0;
}

mx_status check_device() {
    if (g_has_override.load(std::memory_order_acquire)) {
        if (!arch_is_gfx950(g_arch_override))
            return fail(MX_ERR_DEVICE_UNSUPPORTED, "device is %s, not gfx950 (MI355X) (architecture override)",
                        g_arch_override);
        return MX_SUCCESS;
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(MX_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(MX_ERR_DEVICE_UNSUPPORTED, "device index %d out of range", dev);
    int v = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        v = query_supported(dev) ? 1 : 2;
        g_dev_ok[dev].store(v, std::memory_order_relaxed);
    }
    if (v != 1) return fail(MX_ERR_DEVICE_UNSUPPORTED, "device %d is not gfx950 (MI355X)", dev);
    return MX_SUCCESS;
}

mx_status check_launch(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(MX_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
    return MX_SUCCESS;
}

mx_status check_opts(const mx_quant_opts *o, const char *which) {
    if (!o) return MX_SUCCESS;
    if (o->use_2d_block > 1 || o->use_sr > 1)
        return fail(MX_ERR_INVALID_ARGUMENT, "%s options: use_2d_block and use_sr must be 0 or 1", which);
    if (o->rht != 0 && o->use_2d_block)
        return fail(MX_ERR_UNSUPPORTED, "%s options: rht is not combined with use_2d_block", which);
    return MX_SUCCESS;
}

mx::DirOpts to_dir(const mx_quant_opts *o) {
    mx::DirOpts d{};
    if (o) {
        d.use_2d = o->use_2d_block;
        d.use_sr = o->use_sr;
        d.key0 = (uint32_t)o->seed;
        d.key1 = (uint32_t)(o->seed >> 32);
        d.tensor_id = o->tensor_id;
        d.index_base = o->index_base;
        d.rht = o->rht;
    }
    return d;
}

mx_status check_layout(mx_layout layout) {
    if (layout != MX_LAYOUT_CANONICAL && layout != MX_LAYOUT_TILED)
        return fail(MX_ERR_UNSUPPORTED, "unknown layout %d (valid: MX_LAYOUT_CANONICAL=0, MX_LAYOUT_TILED=1)",
                    (int)layout);
    return MX_SUCCESS;
}

mx_status validate_x(const void *x, int64_t M, int64_t N, int64_t ldx) {
    if (M < 0 || N < 0) return fail(MX_ERR_INVALID_ARGUMENT, "negative shape M=%lld N=%lld", (long long)M, (long long)N);
    if (ldx < N || ldx < 1) return fail(MX_ERR_INVALID_ARGUMENT, "ldx=%lld must be >= max(N, 1)=%lld", (long long)ldx, (long long)N);
    if (!x) return fail(MX_ERR_INVALID_ARGUMENT, "x is NULL");
    if (!aligned16(x)) return fail(MX_ERR_MISALIGNED, "x must be 16-byte aligned");
    if (ldx % 8) return fail(MX_ERR_MISALIGNED, "ldx=%lld must be a multiple of 8", (long long)ldx);
    return MX_SUCCESS;
}

mx_status validate_out(const void *q, const void *s, const char *name) {
    if (!q || !s) return fail(MX_ERR_INVALID_ARGUMENT, "%s output pointer is NULL", name);
    if (!aligned16(q) || !aligned16(s)) return fail(MX_ERR_MISALIGNED, "%s outputs must be 16-byte aligned", name);
    return MX_SUCCESS;
}

// The GEMM kernels address each operand blob with 32-bit buffer offsets: a
// tiled blob of `rows` rows must stay below 2 GiB.  row_bytes is one row's
// data bytes along the padded K.
mx_status check_blob_limit(const char *name, const char *which, int64_t rows, int64_t row_bytes) {
    const int64_t bytes = mx::cdiv(rows, 16) * 16 * row_bytes;
    if (bytes >= (int64_t(1) << 31))
        return fail(MX_ERR_UNSUPPORTED,
                    "%s: operand %s blob is %lld bytes; operand blobs are addressed with 32-bit offsets and must "
                    "stay below 2 GiB (split the product along M, N or K)",
                    name, which, (long long)bytes);
    return MX_SUCCESS;
}

#define MX_TRY(expr)                     \
    do {                                 \
        mx_status _st = (expr);          \
        if (_st != MX_SUCCESS) return _st; \
    } while (0)

}  // namespace

extern "C" {

mx_status mx_blob_bytes(int64_t rows, int64_t length, mx_layout layout, size_t *data_bytes,
                        size_t *scale_bytes) {
    if (rows < 0 || length < 0) return fail(MX_ERR_INVALID_ARGUMENT, "negative blob shape");
    MX_TRY(check_layout(layout));
    const int64_t Lp = mx::padded(length);
    int64_t db, sb;
    if (layout == MX_LAYOUT_CANONICAL) {
        db = rows * (Lp / 2);
        sb = rows * (Lp / 32);
    } else {
        const int64_t r16 = mx::cdiv(rows, 16) * 16;
        db = r16 * (Lp / 2);
        sb = r16 * mx::cdiv(Lp, 512) * 16;
    }
    if (data_bytes) *data_bytes = (size_t)db;
    if (scale_bytes) *scale_bytes = (size_t)sb;
    return MX_SUCCESS;
}

mx_status mx_quantize_rowwise(const void *x, int64_t M, int64_t N, int64_t ldx, const mx_quant_opts *opts,
                              mx_layout layout, void *q, void *s, hipStream_t stream) {
    MX_TRY(validate_x(x, M, N, ldx));
    MX_TRY(check_opts(opts, "row"));
    MX_TRY(check_layout(layout));
    MX_TRY(validate_out(q, s, "row-wise"));
    if (M == 0 || N == 0) return MX_SUCCESS;
    MX_TRY(check_device());
    mx::QuantArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.M = M; a.N = N; a.ldx = ldx;
    a.M_pad = mx::padded(M); a.N_pad = mx::padded(N);
    a.row = to_dir(opts);
    a.q_row = static_cast<uint8_t *>(q);
    a.s_row = static_cast<uint8_t *>(s);
    return check_launch(mx::launch_quantize(a, false, layout, stream),
                        "mx_quantize_rowwise");
}

mx_status mx_quantize_dual(const void *x, int64_t M, int64_t N, int64_t ldx, const mx_quant_opts *row_opts,
                           const mx_quant_opts *col_opts, mx_layout layout, void *q_row, void *s_row,
                           void *q_col, void *s_col, hipStream_t stream) {
    MX_TRY(validate_x(x, M, N, ldx));
    MX_TRY(check_opts(row_opts, "row"));
    MX_TRY(check_opts(col_opts, "col"));
    MX_TRY(check_layout(layout));
    MX_TRY(validate_out(q_row, s_row, "row-wise"));
    MX_TRY(validate_out(q_col, s_col, "column-wise"));
    if (M == 0 || N == 0) return MX_SUCCESS;
    MX_TRY(check_device());
    mx::QuantArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.M = M; a.N = N; a.ldx = ldx;
    a.M_pad = mx::padded(M); a.N_pad = mx::padded(N);
    a.row = to_dir(row_opts);
    a.col = to_dir(col_opts);
    a.sr_pairs = (N % 16 == 0 && a.row.index_base % 16 == 0 && a.col.index_base % 16 == 0) ? 1u : 0u;
    a.q_row = static_cast<uint8_t *>(q_row);
    a.s_row = static_cast<uint8_t *>(s_row);
    a.q_col = static_cast<uint8_t *>(q_col);
    a.s_col = static_cast<uint8_t *>(s_col);
    return check_launch(mx::launch_quantize(a, true, layout, stream),
                        "mx_quantize_dual");
}

mx_status mx_quantize_dual_mul(const void *x, const void *g, int64_t M, int64_t N, int64_t ldx, int64_t ldg,
                               const mx_quant_opts *row_opts, const mx_quant_opts *col_opts, mx_layout layout,
                               void *q_row, void *s_row, void *q_col, void *s_col, hipStream_t stream) {
    const bool dual = q_col || s_col;
    MX_TRY(validate_x(x, M, N, ldx));
    if (!g) return fail(MX_ERR_INVALID_ARGUMENT, "g is NULL");
    if (ldg < N || ldg < 1) return fail(MX_ERR_INVALID_ARGUMENT, "ldg=%lld must be >= max(N, 1)", (long long)ldg);
    if (!aligned16(g)) return fail(MX_ERR_MISALIGNED, "g must be 16-byte aligned");
    if (ldg % 8) return fail(MX_ERR_MISALIGNED, "ldg=%lld must be a multiple of 8", (long long)ldg);
    MX_TRY(check_opts(row_opts, "row"));
    if (row_opts && row_opts->rht) return fail(MX_ERR_UNSUPPORTED, "row options: rht is not combined with the prologue");
    if (dual) {
        MX_TRY(check_opts(col_opts, "col"));
        if (col_opts && col_opts->rht)
            return fail(MX_ERR_UNSUPPORTED, "col options: rht is not combined with the prologue");
    }
    MX_TRY(check_layout(layout));
    MX_TRY(validate_out(q_row, s_row, "row-wise"));
    if (dual) MX_TRY(validate_out(q_col, s_col, "column-wise"));
    if (M == 0 || N == 0) return MX_SUCCESS;
    MX_TRY(check_device());
    mx::QuantArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.g = static_cast<const uint16_t *>(g);
    a.M = M; a.N = N; a.ldx = ldx; a.ldg = ldg;
    a.M_pad = mx::padded(M); a.N_pad = mx::padded(N);
    a.row = to_dir(row_opts);
    if (dual) a.col = to_dir(col_opts);
    a.sr_pairs = (dual && N % 16 == 0 && a.row.index_base % 16 == 0 && a.col.index_base % 16 == 0) ? 1u : 0u;
    a.q_row = static_cast<uint8_t *>(q_row);
    a.s_row = static_cast<uint8_t *>(s_row);
    a.q_col = static_cast<uint8_t *>(q_col);
    a.s_col = static_cast<uint8_t *>(s_col);
    return check_launch(mx::launch_quantize_mul(a, dual, layout, stream),
                        "mx_quantize_dual_mul");
}

mx_status mx_fp6_blob_bytes(int64_t rows, int64_t length, mx_layout layout, size_t *data_bytes,
                            size_t *scale_bytes) {
    if (rows < 0 || length < 0) return fail(MX_ERR_INVALID_ARGUMENT, "negative blob shape");
    MX_TRY(check_layout(layout));
    const int64_t Lp = mx::padded(length);
    const int64_t r = layout == MX_LAYOUT_CANONICAL ? rows : mx::cdiv(rows, 16) * 16;
    if (data_bytes) *data_bytes = (size_t)(r * (Lp * 3 / 4));
    if (scale_bytes) *scale_bytes = (size_t)(layout == MX_LAYOUT_CANONICAL ? r * (Lp / 32) : r * mx::cdiv(Lp, 512) * 16);
    return MX_SUCCESS;
}

namespace {
mx_status check_fp6_fmt(int fmt, const char *which) {
    if (fmt != MX_FP6_E2M3 && fmt != MX_FP6_E3M2)
        return fail(MX_ERR_UNSUPPORTED, "%s element format %d (valid: MX_FP6_E2M3=2, MX_FP6_E3M2=3)", which, fmt);
    return MX_SUCCESS;
}
mx_status check_fp6_opts(const mx_quant_opts *o, const char *which) {
    MX_TRY(check_opts(o, which));
    if (o && o->rht) return fail(MX_ERR_UNSUPPORTED, "%s options: rht is not available for MXFP6", which);
    return MX_SUCCESS;
}
}  // namespace

mx_status mx_quantize_fp6(const void *x, int64_t M, int64_t N, int64_t ldx, int row_fmt,
                          const mx_quant_opts *row_opts, int col_fmt, const mx_quant_opts *col_opts,
                          mx_layout layout, void *q_row, void *s_row, void *q_col, void *s_col, hipStream_t stream) {
    const bool dual = q_col || s_col;
    MX_TRY(validate_x(x, M, N, ldx));
    MX_TRY(check_fp6_fmt(row_fmt, "row"));
    MX_TRY(check_fp6_opts(row_opts, "row"));
    if (dual) {
        MX_TRY(check_fp6_fmt(col_fmt, "col"));
        MX_TRY(check_fp6_opts(col_opts, "col"));
    }
    MX_TRY(check_layout(layout));
    MX_TRY(validate_out(q_row, s_row, "row-wise"));
    if (dual) MX_TRY(validate_out(q_col, s_col, "column-wise"));
    if (M == 0 || N == 0) return MX_SUCCESS;
    MX_TRY(check_device());
    mx::QuantArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.M = M; a.N = N; a.ldx = ldx;
    a.M_pad = mx::padded(M); a.N_pad = mx::padded(N);
    a.row = to_dir(row_opts);
    a.row.fmt = (uint32_t)row_fmt;
    if (dual) {
        a.col = to_dir(col_opts);
        a.col.fmt = (uint32_t)col_fmt;
    }
    a.sr_pairs = (dual && N % 16 == 0 && a.row.index_base % 16 == 0 && a.col.index_base % 16 == 0) ? 1u : 0u;
    a.q_row = static_cast<uint8_t *>(q_row);
    a.s_row = static_cast<uint8_t *>(s_row);
    a.q_col = static_cast<uint8_t *>(q_col);
    a.s_col = static_cast<uint8_t *>(s_col);
    return check_launch(mx::launch_quantize_fp6(a, dual, layout, stream),
                        "mx_quantize_fp6");
}

namespace {

mx_status gemm_common(const char *name, int transA, int transB, int64_t M, int64_t N, int64_t K, const void *A,
                      const void *A_scale, const void *B, const void *B_scale, mx_layout layout, mx_dtype out_dtype,
                      const void *bias, bool want_bias, void *C, int64_t ldc, hipStream_t stream, int fp6_a = 0,
                      int fp6_b = 0) {
    if (transA != 0 || transB != 1)
        return fail(MX_ERR_UNSUPPORTED,
                    "transA=%d transB=%d: only transA=0, transB=1 (C = A . B^T, both operands K-contiguous) "
                    "is supported; quantize the other direction instead of transposing",
                    transA, transB);
    if (M < 0 || N < 0 || K < 0)
        return fail(MX_ERR_INVALID_ARGUMENT, "negative shape M=%lld N=%lld K=%lld", (long long)M, (long long)N,
                    (long long)K);
    MX_TRY(check_layout(layout));
    if (layout != MX_LAYOUT_TILED)
        return fail(MX_ERR_UNSUPPORTED, "%s reads MX_LAYOUT_TILED blobs only", name);
    if (out_dtype != MX_BF16 && out_dtype != MX_F32)
        return fail(MX_ERR_UNSUPPORTED, "out_dtype %d (valid: MX_BF16=0, MX_F32=1)", (int)out_dtype);
    if (ldc < N || ldc < 1) return fail(MX_ERR_INVALID_ARGUMENT, "ldc=%lld must be >= max(N, 1)", (long long)ldc);
    if (!C) return fail(MX_ERR_INVALID_ARGUMENT, "C is NULL");
    if (K > 0 && (!A || !A_scale || !B || !B_scale))
        return fail(MX_ERR_INVALID_ARGUMENT, "operand pointer is NULL");
    if (want_bias && !bias) return fail(MX_ERR_INVALID_ARGUMENT, "bias is NULL");
    if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(A_scale) || !aligned16(B) || !aligned16(B_scale))) ||
        (want_bias && !aligned16(bias)))
        return fail(MX_ERR_MISALIGNED, "operands, bias and C must be 16-byte aligned");
    if (ldc % 8) return fail(MX_ERR_MISALIGNED, "ldc=%lld must be a multiple of 8", (long long)ldc);
    {
        const int64_t K_pad = mx::padded(K);
        MX_TRY(check_blob_limit(name, "A", M, fp6_a ? K_pad / 4 * 3 : K_pad / 2));
        MX_TRY(check_blob_limit(name, "B", N, fp6_b ? K_pad / 4 * 3 : K_pad / 2));
    }
    if (M == 0 || N == 0) return MX_SUCCESS;
    MX_TRY(check_device());
    if (fp6_a)
        return check_launch(mx::launch_gemm_fp6(M, N, K, fp6_a, static_cast<const uint8_t *>(A),
                                                static_cast<const uint8_t *>(A_scale), fp6_b,
                                                static_cast<const uint8_t *>(B), static_cast<const uint8_t *>(B_scale),
                                                out_dtype, C, ldc, stream),
                            name);
    return check_launch(mx::launch_gemm(M, N, K, static_cast<const uint8_t *>(A),
                                        static_cast<const uint8_t *>(A_scale), static_cast<const uint8_t *>(B),
                                        static_cast<const uint8_t *>(B_scale),
                                        want_bias ? static_cast<const uint16_t *>(bias) : nullptr, out_dtype, C,
                                        ldc, stream),
                        name);
}

}  // namespace

mx_status mx_gemm_a4w4(int transA, int transB, int64_t M, int64_t N, int64_t K, const void *A,
                       const void *A_scale, const void *B, const void *B_scale, mx_layout layout,
                       mx_dtype out_dtype, void *C, int64_t ldc, hipStream_t stream) {
    return gemm_common("mx_gemm_a4w4", transA, transB, M, N, K, A, A_scale, B, B_scale, layout, out_dtype, nullptr,
                       false, C, ldc, stream);
}

mx_status mx_gemm_a4w4_bias(int transA, int transB, int64_t M, int64_t N, int64_t K, const void *A,
                            const void *A_scale, const void *B, const void *B_scale, mx_layout layout,
                            mx_dtype out_dtype, const void *bias, void *C, int64_t ldc, hipStream_t stream) {
    return gemm_common("mx_gemm_a4w4_bias", transA, transB, M, N, K, A, A_scale, B, B_scale, layout, out_dtype,
                       bias, true, C, ldc, stream);
}

mx_status mx_gemm_fp6(int transA, int transB, int64_t M, int64_t N, int64_t K, int fmt_a, const void *A,
                      const void *A_scale, int fmt_b, const void *B, const void *B_scale, mx_layout layout,
                      mx_dtype out_dtype, void *C, int64_t ldc, hipStream_t stream) {
    MX_TRY(check_fp6_fmt(fmt_a, "A"));
    MX_TRY(check_fp6_fmt(fmt_b, "B"));
    return gemm_common("mx_gemm_fp6", transA, transB, M, N, K, A, A_scale, B, B_scale, layout, out_dtype, nullptr,
                       false, C, ldc, stream, fmt_a, fmt_b);
}

mx_status mx_fp8_blob_bytes(int64_t rows, int64_t length, mx_layout layout, size_t *bytes) {
    if (rows < 0 || length < 0) return fail(MX_ERR_INVALID_ARGUMENT, "negative blob shape");
    MX_TRY(check_layout(layout));
    const int64_t r = layout == MX_LAYOUT_TILED ? mx::cdiv(rows, 16) * 16 : rows;
    if (bytes) *bytes = (size_t)(r * mx::padded(length));
    return MX_SUCCESS;
}

mx_status mx_quantize_fp8_tw(const void *x, int64_t M, int64_t N, int64_t ldx, mx_layout layout, void *q_row,
                             void *q_col, float *info, hipStream_t stream) {
    MX_TRY(validate_x(x, M, N, ldx));
    MX_TRY(check_layout(layout));
    if (!q_row && !q_col) return fail(MX_ERR_INVALID_ARGUMENT, "q_row and q_col are both NULL");
    if (!info) return fail(MX_ERR_INVALID_ARGUMENT, "info is NULL");
    if ((q_row && !aligned16(q_row)) || (q_col && !aligned16(q_col)) || !aligned16(info))
        return fail(MX_ERR_MISALIGNED, "outputs and info must be 16-byte aligned");
    if (M == 0 || N == 0) return MX_SUCCESS;
    MX_TRY(check_device());
    return check_launch(mx::launch_quantize_fp8(static_cast<const uint16_t *>(x), M, N, ldx, layout,
                                                static_cast<uint8_t *>(q_row), static_cast<uint8_t *>(q_col), info,
                                                stream),
                        "mx_quantize_fp8_tw");
}

mx_status mx_gemm_f8_tw(int transA, int transB, int64_t M, int64_t N, int64_t K, const void *A,
                        const float *a_scale_inv, const void *B, const float *b_scale_inv, mx_layout layout,
                        mx_dtype out_dtype, void *C, int64_t ldc, hipStream_t stream) {
    if (transA != 0 || transB != 1)
        return fail(MX_ERR_UNSUPPORTED, "transA=%d transB=%d: only transA=0, transB=1 (C = A . B^T) is supported",
                    transA, transB);
    if (M < 0 || N < 0 || K < 0)
        return fail(MX_ERR_INVALID_ARGUMENT, "negative shape M=%lld N=%lld K=%lld", (long long)M, (long long)N,
                    (long long)K);
    MX_TRY(check_layout(layout));
    if (layout != MX_LAYOUT_TILED) return fail(MX_ERR_UNSUPPORTED, "mx_gemm_f8_tw reads MX_LAYOUT_TILED blobs only");
    if (out_dtype != MX_BF16 && out_dtype != MX_F32)
        return fail(MX_ERR_UNSUPPORTED, "out_dtype %d (valid: MX_BF16=0, MX_F32=1)", (int)out_dtype);
    if (ldc < N || ldc < 1) return fail(MX_ERR_INVALID_ARGUMENT, "ldc=%lld must be >= max(N, 1)", (long long)ldc);
    if (!C) return fail(MX_ERR_INVALID_ARGUMENT, "C is NULL");
    if (K > 0 && (!A || !B || !a_scale_inv || !b_scale_inv))
        return fail(MX_ERR_INVALID_ARGUMENT, "operand or scale pointer is NULL");
    if (!aligned16(C) || (K > 0 && (!aligned16(A) || !aligned16(B))))
        return fail(MX_ERR_MISALIGNED, "operands and C must be 16-byte aligned");
    if (ldc % 8) return fail(MX_ERR_MISALIGNED, "ldc=%lld must be a multiple of 8", (long long)ldc);
    MX_TRY(check_blob_limit("mx_gemm_f8_tw", "A", M, mx::padded(K)));
    MX_TRY(check_blob_limit("mx_gemm_f8_tw", "B", N, mx::padded(K)));
    if (M == 0 || N == 0) return MX_SUCCESS;
    MX_TRY(check_device());
    return check_launch(mx::launch_gemm_fp8(M, N, K, static_cast<const uint8_t *>(A), a_scale_inv,
                                            static_cast<const uint8_t *>(B), b_scale_inv, out_dtype, C, ldc,
                                            stream),
                        "mx_gemm_f8_tw");
}

mx_status mx_layout_convert(int to_tiled, int64_t rows, int64_t length, const void *q_src, const void *s_src,
                            void *q_dst, void *s_dst, hipStream_t stream) {
    if (rows < 0 || length < 0) return fail(MX_ERR_INVALID_ARGUMENT, "negative blob shape");
    if (!q_src || !s_src || !q_dst || !s_dst) return fail(MX_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (!aligned16(q_src) || !aligned16(q_dst) || !aligned16(s_src) || !aligned16(s_dst))
        return fail(MX_ERR_MISALIGNED, "data and scale pointers must be 16-byte aligned");
    if (rows == 0 || length == 0) return MX_SUCCESS;
    MX_TRY(check_device());
    return check_launch(mx::launch_layout_convert(to_tiled != 0, rows, length, static_cast<const uint8_t *>(q_src),
                                                  static_cast<const uint8_t *>(s_src), static_cast<uint8_t *>(q_dst),
                                                  static_cast<uint8_t *>(s_dst), stream),
                        "mx_layout_convert");
}

mx_status mx_dequantize(const void *q, const void *s, int64_t rows, int64_t length, mx_layout layout,
                        void *out_f32, int64_t ldo, hipStream_t stream) {
    if (rows < 0 || length < 0) return fail(MX_ERR_INVALID_ARGUMENT, "negative blob shape");
    MX_TRY(check_layout(layout));
    if (ldo < length || ldo < 1) return fail(MX_ERR_INVALID_ARGUMENT, "ldo must be >= max(length, 1)");
    if (!q || !s || !out_f32) return fail(MX_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (rows == 0 || length == 0) return MX_SUCCESS;
    MX_TRY(check_device());
    return check_launch(mx::launch_dequantize(static_cast<const uint8_t *>(q), static_cast<const uint8_t *>(s),
                                              rows, length, layout, static_cast<float *>(out_f32), ldo,
                                              stream),
                        "mx_dequantize");
}

mx_status mx_measure_mfma(int fmt_a, int fmt_b, const void *operands, int workgroups, int64_t iters, float *out,
                          hipStream_t stream) {
    if (fmt_a < 0 || fmt_a > 4 || fmt_b < 0 || fmt_b > 4)
        return fail(MX_ERR_UNSUPPORTED, "element formats %d, %d (valid: 0 E4M3, 1 E5M2, 2 E2M3, 3 E3M2, 4 E2M1)",
                    fmt_a, fmt_b);
    if (!operands || !out) return fail(MX_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (workgroups < 1 || iters < 1)
        return fail(MX_ERR_INVALID_ARGUMENT, "workgroups=%d and iters=%lld must be >= 1", workgroups,
                    (long long)iters);
    if (!aligned16(operands) || !aligned16(out))
        return fail(MX_ERR_MISALIGNED, "operands and out must be 16-byte aligned");
    MX_TRY(check_device());
    return check_launch(mx::launch_measure_mfma(fmt_a, fmt_b, operands, workgroups, iters, out,
                                                stream),
                        "mx_measure_mfma");
}

int mx_device_supported(int device) {
    if (device < 0 || device >= kMaxDevices) return 0;
    return query_supported(device);
}

mx_status mx_set_device_arch_override(const char *arch) {
    if (!arch) {
        g_has_override.store(false, std::memory_order_release);
        return MX_SUCCESS;
    }
    if (std::strlen(arch) >= sizeof g_arch_override)
        return fail(MX_ERR_INVALID_ARGUMENT, "architecture name longer than %d characters",
                    (int)sizeof g_arch_override - 1);
    g_has_override.store(false, std::memory_order_release);
    std::snprintf(g_arch_override, sizeof g_arch_override, "%s", arch);
    g_has_override.store(true, std::memory_order_release);
    return MX_SUCCESS;
}

const char *mx_status_string(mx_status status) {
    switch (status) {
        case MX_SUCCESS: return "MX_SUCCESS";
        case MX_ERR_INVALID_ARGUMENT: return "MX_ERR_INVALID_ARGUMENT";
        case MX_ERR_MISALIGNED: return "MX_ERR_MISALIGNED";
        case MX_ERR_UNSUPPORTED: return "MX_ERR_UNSUPPORTED";
        case MX_ERR_DEVICE_UNSUPPORTED: return "MX_ERR_DEVICE_UNSUPPORTED";
        case MX_ERR_HIP: return "MX_ERR_HIP";
    }
    return "MX_ERR_UNKNOWN";
}

const char *mx_last_error(void) { return g_last_error; }

}  // extern "C"
