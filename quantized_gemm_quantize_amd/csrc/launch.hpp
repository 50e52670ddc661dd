// Internal kernel launchers behind the C ABI (w8a8_abi.cpp). Arguments are
// already validated when these run; each returns the HIP error of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

hipError_t launch_quantize_rows_bf16(const uint16_t *x, int64_t M, int K, int8_t *xq, float *xs,
                                     hipStream_t stream);
hipError_t launch_quantize_rows_f32(const float *x, int64_t M, int K, int8_t *xq, float *xs,
                                    hipStream_t stream);

struct Addmm;

// Dense GEMM: picks the weight-streaming kernel for M <= 64, the LDS-tiled
// MFMA kernel otherwise. With am non-null (bf16 output only) the epilogue is
// alpha * (acc * sa * sb) + beta * bias.
hipError_t launch_gemm(const int8_t *xq, const float *xs, int M, const int8_t *wq, const float *ws,
                       int N, int K, void *out, bool out_i32, hipStream_t stream,
                       const Addmm *am = nullptr);

// Single-launch linear for M <= 64: quantize_rows of bf16 X fused into the
// weight-streaming GEMM, epilogue as launch_gemm's with am.
hipError_t launch_linear_decode(const uint16_t *x, int M, const int8_t *wq, const float *ws, int N,
                                int K, void *out, hipStream_t stream, const Addmm &am);

// 2:4 weights: compression of an int8 [N,K] weight (K % 64 == 0) into values
// [N,K/2] and meta [N,K/32], and the GEMM on the compressed weight.
hipError_t launch_compress24(const int8_t *wq, int N, int K, int8_t *values, uint32_t *meta,
                             hipStream_t stream);
hipError_t launch_sparse24_gemm(const int8_t *xq, const float *xs, int M, const int8_t *values,
                                const uint32_t *meta, const float *ws, int N, int K, void *out,
                                bool out_i32, hipStream_t stream);

// Compute units of the current device (queried once per device).
int device_cu_count();

// Block-sparse GEMM; am (bf16 output only) selects the addmm epilogue.
hipError_t launch_bsr_gemm(const int8_t *xq, const float *xs, int M, int K, const int32_t *crow,
                           const int32_t *col, const int8_t *values, int nnzb, const float *ws,
                           int N, void *out, bool out_i32, hipStream_t stream,
                           const Addmm *am = nullptr);

}  // namespace w8a8

namespace w4a16 {

// W4A16 (16-bit values as uint16_t bit patterns: bf16, or binary16 when f16):
// standalone dequantization of packed 4-bit weights [N,K/2] (u4, or s4 when
// s4) with scales/zeros [N,K/G] into w [N,K], and the fused dequant GEMM
// out [M,N] = round(x [M,K] . w^T).
hipError_t launch_dequant(const uint8_t *wq4, const uint16_t *scales, const uint16_t *zeros, int N,
                          int K, int G, bool s4, bool f16, uint16_t *w, hipStream_t stream);
hipError_t launch_gemm(const uint16_t *x, int M, const uint8_t *wq4, const uint16_t *scales,
                       const uint16_t *zeros, int N, int K, int G, bool s4, bool f16,
                       uint16_t *out, hipStream_t stream);

}  // namespace w4a16
