// C ABI of libw8a8.so: argument validation, then one launch on the caller's
// stream. Declarations and argument contracts are in include/w8a8.h.
//
// Every check runs on the host before any HIP call, so a rejected call
// touches no device state. Failures return a nonzero status, as the pages'
// TensorRT plugin does with its library status (Paddle sparse_fc PR #41770,
// spmm_plugin.cu enqueue hunk).
#include "w8a8.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstring>

#include "common.hpp"
#include "launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// A C caller may pass any int for an enum parameter, but in C++ reading an
// enum object whose value lies outside its enumerators' range is undefined:
// selectors are read as the int they are, then validated.
template <typename E>
int selector(const E *e) {
    static_assert(sizeof(E) == sizeof(int), "C enums are int-sized here");
    int v;
    std::memcpy(&v, e, sizeof v);
    return v;
}

w8a8_status hip_status(hipError_t e) {
    if (e == hipSuccess) return W8A8_OK;
    g_last_hip_error = static_cast<int>(e);
    return W8A8_ERR_HIP;
}

// K checks shared by every entry: positive multiple of 16, int32-safe.
w8a8_status check_k(int64_t K) {
    if (K <= 0 || K % 16 != 0) return W8A8_ERR_SHAPE;
    if (K > W8A8_MAX_K) return W8A8_ERR_K_OVERFLOW;
    return W8A8_OK;
}

// Sizes the kernels index with 32-bit integers.
bool too_big(int64_t M, int64_t N) { return M > INT_MAX / 2 || N > INT_MAX / 2; }

template <typename T>
w8a8_status quantize_entry(const T *x, int64_t M, int64_t K, int8_t *xq, float *x_scale,
                           void *stream,
                           hipError_t (*launch)(const T *, int64_t, int, int8_t *, float *,
                                                hipStream_t)) {
    if (M < 0) return W8A8_ERR_SHAPE;
    if (w8a8_status s = check_k(K)) return s;
    if (M == 0) return W8A8_OK;
    if (M > INT_MAX) return W8A8_ERR_SHAPE;  // grid.x: at least one row per workgroup
    if (!x || !xq || !x_scale) return W8A8_ERR_NULL;
    if (misaligned(x) || misaligned(xq) || misaligned(x_scale)) return W8A8_ERR_ALIGN;
    return hip_status(launch(x, M, (int)K, xq, x_scale, static_cast<hipStream_t>(stream)));
}

}  // namespace

namespace w8a8 {

int device_cu_count() {
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

}  // namespace w8a8

extern "C" {

w8a8_status w8a8_quantize_rows(const void *x_bf16, int64_t M, int64_t K, int8_t *xq,
                               float *x_scale, void *stream) {
    return quantize_entry<uint16_t>(static_cast<const uint16_t *>(x_bf16), M, K, xq, x_scale,
                                    stream, w8a8::launch_quantize_rows_bf16);
}

w8a8_status w8a8_quantize_rows_f32(const float *x, int64_t M, int64_t K, int8_t *xq,
                                   float *x_scale, void *stream) {
    return quantize_entry<float>(x, M, K, xq, x_scale, stream, w8a8::launch_quantize_rows_f32);
}

w8a8_status w8a8_gemm(const int8_t *xq, const float *x_scale, int64_t M, const int8_t *wq,
                      const float *w_scale, int64_t N, int64_t K, void *out,
                      w8a8_out_dtype out_dtype, void *stream) {
    if (M < 0 || N <= 0 || N % 16 != 0 || too_big(M, N)) return W8A8_ERR_SHAPE;
    if (w8a8_status s = check_k(K)) return s;
    const int od = selector(&out_dtype);
    if (od != W8A8_OUT_BF16 && od != W8A8_OUT_I32) return W8A8_ERR_DTYPE;
    if ((M + 127) / 128 > INT_MAX / ((N + 127) / 128)) return W8A8_ERR_SHAPE;  // grid.x
    if (M == 0) return W8A8_OK;
    if (!xq || !x_scale || !wq || !w_scale || !out) return W8A8_ERR_NULL;
    if (misaligned(xq) || misaligned(x_scale) || misaligned(wq) || misaligned(w_scale) ||
        misaligned(out))
        return W8A8_ERR_ALIGN;
    return hip_status(w8a8::launch_gemm(xq, x_scale, (int)M, wq, w_scale, (int)N, (int)K, out,
                                        od == W8A8_OUT_I32,
                                        static_cast<hipStream_t>(stream)));
}

w8a8_status w8a8_gemm_addmm(const int8_t *xq, const float *x_scale, int64_t M, const int8_t *wq,
                            const float *w_scale, int64_t N, int64_t K, const float *bias,
                            float alpha, float beta, void *out, void *stream) {
    if (M < 0 || N <= 0 || N % 16 != 0 || too_big(M, N)) return W8A8_ERR_SHAPE;
    if (w8a8_status s = check_k(K)) return s;
    if (!std::isfinite(alpha) || !std::isfinite(beta)) return W8A8_ERR_VALUE;
    if ((M + 127) / 128 > INT_MAX / ((N + 127) / 128)) return W8A8_ERR_SHAPE;  // grid.x
    if (M == 0) return W8A8_OK;
    if (!xq || !x_scale || !wq || !w_scale || !out) return W8A8_ERR_NULL;
    if (!bias && beta != 0.0f) return W8A8_ERR_NULL;
    if (misaligned(xq) || misaligned(x_scale) || misaligned(wq) || misaligned(w_scale) ||
        misaligned(out) || (bias && misaligned(bias)))
        return W8A8_ERR_ALIGN;
    const w8a8::Addmm am{bias, alpha, beta};
    return hip_status(w8a8::launch_gemm(xq, x_scale, (int)M, wq, w_scale, (int)N, (int)K, out,
                                        false, static_cast<hipStream_t>(stream), &am));
}

w8a8_status w8a8_fused_linear(const void *x_bf16, int64_t M, int64_t K, const int8_t *wq,
                              const float *w_scale, int64_t N, const float *bias, float alpha,
                              float beta, void *out, void *stream) {
    if (M < 0 || M > W8A8_FUSED_MAX_M || N <= 0 || N % 16 != 0 || too_big(M, N))
        return W8A8_ERR_SHAPE;
    if (w8a8_status s = check_k(K)) return s;
    if (!std::isfinite(alpha) || !std::isfinite(beta)) return W8A8_ERR_VALUE;
    if (M == 0) return W8A8_OK;
    if (!x_bf16 || !wq || !w_scale || !out) return W8A8_ERR_NULL;
    if (!bias && beta != 0.0f) return W8A8_ERR_NULL;
    if (misaligned(x_bf16) || misaligned(wq) || misaligned(w_scale) || misaligned(out) ||
        (bias && misaligned(bias)))
        return W8A8_ERR_ALIGN;
    const w8a8::Addmm am{bias, alpha, beta};
    return hip_status(w8a8::launch_linear_decode(static_cast<const uint16_t *>(x_bf16), (int)M, wq,
                                                 w_scale, (int)N, (int)K, out,
                                                 static_cast<hipStream_t>(stream), am));
}

w8a8_status w8a8_bsr_gemm(const int8_t *xq, const float *x_scale, int64_t M, int64_t K,
                          const int32_t *crow, const int32_t *col, const int8_t *values,
                          int64_t nnzb, int64_t bs, const float *w_scale, int64_t N, void *out,
                          w8a8_out_dtype out_dtype, void *stream) {
    if (bs != 64) return W8A8_ERR_BLOCKSIZE;
    if (M < 0 || N <= 0 || N % bs != 0 || K % bs != 0 || nnzb < 0 || too_big(M, N))
        return W8A8_ERR_SHAPE;
    if (w8a8_status s = check_k(K)) return s;
    if (nnzb > (N / bs) * (K / bs)) return W8A8_ERR_SHAPE;
    const int od = selector(&out_dtype);
    if (od != W8A8_OUT_BF16 && od != W8A8_OUT_I32) return W8A8_ERR_DTYPE;
    if ((M + 127) / 128 > INT_MAX / (N / bs)) return W8A8_ERR_SHAPE;  // grid.x
    if (M == 0) return W8A8_OK;
    if (!xq || !x_scale || !crow || !w_scale || !out) return W8A8_ERR_NULL;
    if (nnzb > 0 && (!col || !values)) return W8A8_ERR_NULL;
    if (misaligned(xq) || misaligned(x_scale) || misaligned(crow) || misaligned(w_scale) ||
        misaligned(out) || (nnzb > 0 && (misaligned(col) || misaligned(values))))
        return W8A8_ERR_ALIGN;
    return hip_status(w8a8::launch_bsr_gemm(xq, x_scale, (int)M, (int)K, crow, col, values,
                                            (int)nnzb, w_scale, (int)N, out,
                                            od == W8A8_OUT_I32,
                                            static_cast<hipStream_t>(stream)));
}

w8a8_status w8a8_bsr_gemm_addmm(const int8_t *xq, const float *x_scale, int64_t M, int64_t K,
                                const int32_t *crow, const int32_t *col, const int8_t *values,
                                int64_t nnzb, int64_t bs, const float *w_scale, int64_t N,
                                const float *bias, float alpha, float beta, void *out,
                                void *stream) {
    if (bs != 64) return W8A8_ERR_BLOCKSIZE;
    if (M < 0 || N <= 0 || N % bs != 0 || K % bs != 0 || nnzb < 0 || too_big(M, N))
        return W8A8_ERR_SHAPE;
    if (w8a8_status s = check_k(K)) return s;
    if (nnzb > (N / bs) * (K / bs)) return W8A8_ERR_SHAPE;
    if (!std::isfinite(alpha) || !std::isfinite(beta)) return W8A8_ERR_VALUE;
    if ((M + 127) / 128 > INT_MAX / (N / bs)) return W8A8_ERR_SHAPE;  // grid.x
    if (M == 0) return W8A8_OK;
    if (!xq || !x_scale || !crow || !w_scale || !out) return W8A8_ERR_NULL;
    if (nnzb > 0 && (!col || !values)) return W8A8_ERR_NULL;
    if (!bias && beta != 0.0f) return W8A8_ERR_NULL;
    if (misaligned(xq) || misaligned(x_scale) || misaligned(crow) || misaligned(w_scale) ||
        misaligned(out) || (nnzb > 0 && (misaligned(col) || misaligned(values))) ||
        (bias && misaligned(bias)))
        return W8A8_ERR_ALIGN;
    const w8a8::Addmm am{bias, alpha, beta};
    return hip_status(w8a8::launch_bsr_gemm(xq, x_scale, (int)M, (int)K, crow, col, values,
                                            (int)nnzb, w_scale, (int)N, out, false,
                                            static_cast<hipStream_t>(stream), &am));
}

w8a8_status w8a8_compress24(const int8_t *wq, int64_t N, int64_t K, int8_t *values,
                            uint32_t *meta, void *stream) {
    if (N < 0 || K <= 0 || K % 128 != 0 || N > INT_MAX / 2 || K > INT_MAX / 2) return W8A8_ERR_SHAPE;
    if (N == 0) return W8A8_OK;
    if (N * (K / 32) > (int64_t)UINT_MAX * 256 / 2) return W8A8_ERR_SHAPE;  // grid.x
    if (!wq || !values || !meta) return W8A8_ERR_NULL;
    if (misaligned(wq) || misaligned(values) || misaligned(meta)) return W8A8_ERR_ALIGN;
    return hip_status(w8a8::launch_compress24(wq, (int)N, (int)K, values, meta,
                                              static_cast<hipStream_t>(stream)));
}

w8a8_status w8a8_sparse24_gemm(const int8_t *xq, const float *x_scale, int64_t M,
                               const int8_t *values, const uint32_t *meta, const float *w_scale,
                               int64_t N, int64_t K, void *out, w8a8_out_dtype out_dtype,
                               void *stream) {
    if (M < 0 || N <= 0 || N % 16 != 0 || K % 128 != 0 || too_big(M, N)) return W8A8_ERR_SHAPE;
    if (w8a8_status s = check_k(K)) return s;
    const int od = selector(&out_dtype);
    if (od != W8A8_OUT_BF16 && od != W8A8_OUT_I32) return W8A8_ERR_DTYPE;
    if ((M + 127) / 128 > INT_MAX / ((N + 255) / 256)) return W8A8_ERR_SHAPE;  // grid.x
    if (M == 0) return W8A8_OK;
    if (!xq || !x_scale || !values || !meta || !w_scale || !out) return W8A8_ERR_NULL;
    if (misaligned(xq) || misaligned(x_scale) || misaligned(values) || misaligned(meta) ||
        misaligned(w_scale) || misaligned(out))
        return W8A8_ERR_ALIGN;
    return hip_status(w8a8::launch_sparse24_gemm(xq, x_scale, (int)M, values, meta, w_scale,
                                                 (int)N, (int)K, out, od == W8A8_OUT_I32,
                                                 static_cast<hipStream_t>(stream)));
}

// W4A16 shape rules shared by both entry points.
static w8a8_status w4a16_shape(int64_t N, int64_t K, int64_t G) {
    if (N <= 0 || N % 16 != 0 || K <= 0 || K % 128 != 0 || G <= 0 || G % 32 != 0 || K % G != 0 ||
        N > INT_MAX / 2 || K > INT_MAX / 2 || N * K / 8 > (int64_t)UINT_MAX * 256 / 2)
        return W8A8_ERR_SHAPE;
    return W8A8_OK;
}

static bool misaligned2(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 1u) != 0; }

w8a8_status w4a16_dequant(const uint8_t *wq4, const void *scales, const void *zeros, int64_t N,
                          int64_t K, int64_t group_size, w4a16_codes codes, w4a16_dtype dtype,
                          void *w, void *stream) {
    if (w8a8_status s = w4a16_shape(N, K, group_size)) return s;
    const int cs = selector(&codes), dt = selector(&dtype);
    if (cs != W4A16_CODES_U4 && cs != W4A16_CODES_S4) return W8A8_ERR_DTYPE;
    if (dt != W4A16_BF16 && dt != W4A16_F16) return W8A8_ERR_DTYPE;
    if (!wq4 || !scales || !zeros || !w) return W8A8_ERR_NULL;
    if (misaligned(wq4) || misaligned(w) || misaligned2(scales) || misaligned2(zeros))
        return W8A8_ERR_ALIGN;
    return hip_status(w4a16::launch_dequant(wq4, static_cast<const uint16_t *>(scales),
                                            static_cast<const uint16_t *>(zeros), (int)N, (int)K,
                                            (int)group_size, cs == W4A16_CODES_S4,
                                            dt == W4A16_F16, static_cast<uint16_t *>(w),
                                            static_cast<hipStream_t>(stream)));
}

w8a8_status w4a16_gemm(const void *x, int64_t M, const uint8_t *wq4, const void *scales,
                       const void *zeros, int64_t N, int64_t K, int64_t group_size,
                       w4a16_codes codes, w4a16_dtype dtype, void *out, void *stream) {
    if (M < 0 || M > INT_MAX / 2) return W8A8_ERR_SHAPE;
    if (w8a8_status s = w4a16_shape(N, K, group_size)) return s;
    const int cs = selector(&codes), dt = selector(&dtype);
    if (cs != W4A16_CODES_U4 && cs != W4A16_CODES_S4) return W8A8_ERR_DTYPE;
    if (dt != W4A16_BF16 && dt != W4A16_F16) return W8A8_ERR_DTYPE;
    if ((M + 63) / 64 > INT_MAX / ((N + 63) / 64)) return W8A8_ERR_SHAPE;  // grid.x
    if (M == 0) return W8A8_OK;
    if (!x || !wq4 || !scales || !zeros || !out) return W8A8_ERR_NULL;
    if (misaligned(x) || misaligned(wq4) || misaligned(out) || misaligned2(scales) ||
        misaligned2(zeros))
        return W8A8_ERR_ALIGN;
    return hip_status(w4a16::launch_gemm(static_cast<const uint16_t *>(x), (int)M, wq4,
                                         static_cast<const uint16_t *>(scales),
                                         static_cast<const uint16_t *>(zeros), (int)N, (int)K,
                                         (int)group_size, cs == W4A16_CODES_S4,
                                         dt == W4A16_F16, static_cast<uint16_t *>(out),
                                         static_cast<hipStream_t>(stream)));
}

const char *w8a8_status_string(int status) {
    switch (status) {
        case W8A8_OK: return "ok";
        case W8A8_ERR_NULL: return "a required pointer is NULL";
        case W8A8_ERR_SHAPE: return "a size is out of range or not a required multiple";
        case W8A8_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
        case W8A8_ERR_K_OVERFLOW: return "K exceeds the int32-safe bound (128*128*K < 2^31)";
        case W8A8_ERR_BLOCKSIZE: return "BSR block size must be 64";
        case W8A8_ERR_DTYPE: return "unknown output dtype";
        case W8A8_ERR_HIP: return "HIP launch error (see w8a8_last_hip_error)";
        case W8A8_ERR_VALUE: return "alpha or beta is not finite";
        default: return "unknown status";
    }
}

int w8a8_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
