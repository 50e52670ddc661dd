// Weight-streaming int8 GEMM for small M (M <= 64, decode-sized batches).
//
// At M = 16 every W byte is used for just 16 multiply-adds, so the kernel is
// bound by reading W [N,K] from HBM once (pytorch/ao PR #153 notes that fused
// dequant GEMMs aimed at compute-bound M > 16 do not serve this memory-bound
// inference case). Shape of the kernel:
//  - one workgroup per 16 output channels; its KSPLIT wavefronts split K, so
//    every wavefront issues all of its 16-byte W loads up front and the whole
//    weight matrix is in flight at once across the chip;
//  - v_mfma_i32_16x16x64_i8: lane l holds W row (l % 16) and activation row
//    (l % 16) of each 16-row block, 16 bytes of K at offset 16 * (l / 16) of
//    every 64-byte K step, for both operands;
//  - the K-split partial int32 tiles are summed in LDS (never in HBM), then
//    scaled, rounded to bf16 and stored: the same fused epilogue as the tiled
//    kernel.
#include "common.hpp"
#include "launch.hpp"

namespace w8a8 {
namespace {

constexpr int kUnroll = 8;   // K steps whose loads are issued together

template <int MT, int KSPLIT, bool OUT_I32, bool ADDMM>
__global__ __launch_bounds__(KSPLIT *kWave) void gemm_decode_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ sa, const int8_t *__restrict__ B,
    const float *__restrict__ sb, void *__restrict__ out, int M, int N, int K,
    int steps_per_wave, Addmm am) {
    __shared__ int red[KSPLIT][MT][4][kWave];

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int n0 = blockIdx.x * 16;
    const int r16 = lane & 15, kgrp = lane >> 4;
    const int8_t *brow = B + (int64_t)(n0 + r16) * K + kgrp * 16;
    const int8_t *arow[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) arow[mb] = A + (int64_t)min(mb * 16 + r16, M - 1) * K + kgrp * 16;

    v4i acc[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) acc[mb] = v4i{};

    const int total_steps = (K + 63) / 64;
    const int s_begin = wave * steps_per_wave;
    const int s_end = min(s_begin + steps_per_wave, total_steps);
    const v4i zero = v4i{};
    for (int s = s_begin; s < s_end; s += kUnroll) {
        v4i b[kUnroll], a[MT][kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int k = (s + u) * 64;
            const bool ok = (s + u < s_end) && (k + kgrp * 16 < K);
            b[u] = ok ? *reinterpret_cast<const v4i *>(brow + k) : zero;
#pragma unroll
            for (int mb = 0; mb < MT; ++mb) a[mb][u] = ok ? *reinterpret_cast<const v4i *>(arow[mb] + k) : zero;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int mb = 0; mb < MT; ++mb) acc[mb] = mfma_16x16x64(a[mb][u], b[u], acc[mb]);
    }

#pragma unroll
    for (int mb = 0; mb < MT; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][mb][r][lane] = acc[mb][r];
    __syncthreads();

    // one output element per thread: row i, column j of 16x16 tile mb sits in
    // lane j + 16 * (i / 4), element i % 4
    for (int e = threadIdx.x; e < MT * 256; e += KSPLIT * kWave) {
        const int mb = e >> 8, i = (e >> 4) & 15, j = e & 15;
        const int m = mb * 16 + i;
        if (m >= M) continue;
        const int l = j + 16 * (i >> 2), r = i & 3;
        int sum = 0;
#pragma unroll
        for (int w = 0; w < KSPLIT; ++w) sum += red[w][mb][r][l];
        const int n = n0 + j;
        if constexpr (OUT_I32) {
            static_cast<int32_t *>(out)[(int64_t)m * N + n] = sum;
        } else {
            const float v =
                addmm<ADDMM>((float)sum * sa[m] * sb[n], am, ADDMM && am.bias ? am.bias[n] : 0.0f);
            static_cast<__bf16 *>(out)[(int64_t)m * N + n] = (__bf16)v;
        }
    }
}

template <int MT>
hipError_t launch_mt(const int8_t *xq, const float *xs, int M, const int8_t *wq, const float *ws,
                     int N, int K, void *out, bool out_i32, hipStream_t stream, const Addmm *am) {
    constexpr int KSPLIT = 8;
    const int total_steps = (K + 63) / 64;
    const int steps_per_wave = (total_steps + KSPLIT - 1) / KSPLIT;
    const dim3 grid((unsigned)(N / 16)), block(KSPLIT * kWave);
    const Addmm a = am ? *am : Addmm{nullptr, 1.0f, 0.0f};
    if (out_i32)
        gemm_decode_kernel<MT, KSPLIT, true, false>
            <<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, steps_per_wave, a);
    else if (am)
        gemm_decode_kernel<MT, KSPLIT, false, true>
            <<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, steps_per_wave, a);
    else
        gemm_decode_kernel<MT, KSPLIT, false, false>
            <<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, steps_per_wave, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_decode(const int8_t *xq, const float *xs, int M, const int8_t *wq,
                              const float *ws, int N, int K, void *out, bool out_i32,
                              hipStream_t stream, const Addmm *am) {
    switch ((M + 15) / 16) {
        case 1: return launch_mt<1>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
        case 2: return launch_mt<2>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
        case 3: return launch_mt<3>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
        default: return launch_mt<4>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
    }
}

}  // namespace w8a8
