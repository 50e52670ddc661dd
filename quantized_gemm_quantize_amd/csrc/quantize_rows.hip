// Dynamic per-row int8 quantization: one wavefront per row.
//
//   s = fl32(absmax / 127);  q = clamp(rint(fl32(x / s)), -127, 127)
//
// (absmax / 127 scale: Paddle sparse_fc PR #41770, spmm_plugin.cu weight-scale
// hunk; clamp before the cast: vLLM csrc/quantization log, FP8 clamp commit.)
//
// The pass is HBM bound (2 or 4 bytes in, 1 byte out per element): each lane
// moves 16 input bytes per load, the wave reduces the absmax with cross-lane
// shuffles, and rows of up to 4096 elements stay in registers so the input is
// read once.
//
// Exact division, cheaply. The quantized value must equal rint of the
// correctly rounded binary32 quotient x / s. Per element we form
// t = fl(x * r) with r = fl(1 / s) (one IEEE division per row); |x/s| <= 127
// (1 + 2^-23), so |t - fl(x/s)| <= 127 * 1.5 * 2^-23 < 2^-15. When t is more
// than 2^-14 away from the nearest half-integer, rint(t) == rint(fl(x/s)) and
// t decides; otherwise (about 1 element in 8000) the element takes the full
// IEEE division. Rows whose scale is subnormal (1/s would overflow) always
// divide. The vLLM log's inverted-scale trick alone would not be exact: it
// moves about one element per 4096-wide row across a rounding boundary.
#include "common.hpp"
#include "launch.hpp"

namespace w8a8 {
namespace {

constexpr int kRowsPerBlock = 4;  // one row per wave, 4 waves per workgroup
constexpr int kMaxRegChunks = 8;  // rows up to 8 * 64 * 8 = 4096 elements stay in registers

// 8 consecutive inputs -> float (bf16 widening is exact).
__device__ __forceinline__ void load8(const uint16_t *p, float v[8]) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
    v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
}

__device__ __forceinline__ void load8(const float *p, float v[8]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// Non-negative floats order like their bit patterns, so the absmax is an
// unsigned max over the wave.
__device__ __forceinline__ float wave_absmax(uint32_t bits) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = __shfl_xor(bits, off, kWave);
        bits = bits > o ? bits : o;
    }
    return __uint_as_float(bits);
}

struct RowScale {
    float s;     // fl32(absmax / 127)
    float r;     // fl32(1 / s) when fast
    bool fast;   // s is a normal number: the reciprocal test applies
};

__device__ __forceinline__ RowScale row_scale(float absmax) {
    RowScale rs;
    rs.s = absmax / 127.0f;  // IEEE division
    rs.fast = rs.s >= 0x1p-126f;
    rs.r = rs.fast ? 1.0f / rs.s : 0.0f;
    return rs;
}

__device__ __forceinline__ int quantize1(float x, const RowScale &rs) {
    float q;
    if (rs.fast) {
        const float t = x * rs.r;
        const float k = __builtin_rintf(t);
        q = (__builtin_fabsf(t - k) < 0.5f - 0x1p-14f) ? k : __builtin_rintf(x / rs.s);
    } else {
        q = rs.s == 0.0f ? 0.0f : __builtin_rintf(x / rs.s);
    }
    q = __builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f);
    return (int)q;
}

__device__ __forceinline__ uint2 quantize8(const float v[8], const RowScale &rs) {
    uint32_t w[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t b0 = (uint32_t)quantize1(v[4 * h + 0], rs) & 0xFFu;
        const uint32_t b1 = (uint32_t)quantize1(v[4 * h + 1], rs) & 0xFFu;
        const uint32_t b2 = (uint32_t)quantize1(v[4 * h + 2], rs) & 0xFFu;
        const uint32_t b3 = (uint32_t)quantize1(v[4 * h + 3], rs) & 0xFFu;
        w[h] = b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    }
    return make_uint2(w[0], w[1]);
}

// NCH > 0: the row (at most NCH * 512 elements) is held in registers.
// NCH == 0: any K; the row is read twice (the second read hits the L2).
template <typename T, int NCH>
__global__ __launch_bounds__(kRowsPerBlock * kWave) void quantize_rows_kernel(
    const T *__restrict__ x, int64_t M, int K, int8_t *__restrict__ xq, float *__restrict__ xs) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x / kWave);
    if (row >= M) return;  // uniform per wave
    const T *xr = x + row * K;
    int8_t *qr = xq + row * K;
    const int nch = K >> 3;  // 8-element chunks (K % 16 == 0)
    uint32_t bits = 0;
    if constexpr (NCH > 0) {
        float v[NCH][8];
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = c * kWave + lane;
            if (ch < nch) {
                load8(xr + ch * 8, v[c]);
#pragma unroll
                for (int e = 0; e < 8; ++e) bits = max(bits, abs_bits(v[c][e]));
            }
        }
        const RowScale rs = row_scale(wave_absmax(bits));
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = c * kWave + lane;
            if (ch < nch) *reinterpret_cast<uint2 *>(qr + ch * 8) = quantize8(v[c], rs);
        }
        if (lane == 0) xs[row] = rs.s;
    } else {
        for (int ch = lane; ch < nch; ch += kWave) {
            float v[8];
            load8(xr + ch * 8, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) bits = max(bits, abs_bits(v[e]));
        }
        const RowScale rs = row_scale(wave_absmax(bits));
        for (int ch = lane; ch < nch; ch += kWave) {
            float v[8];
            load8(xr + ch * 8, v);
            *reinterpret_cast<uint2 *>(qr + ch * 8) = quantize8(v, rs);
        }
        if (lane == 0) xs[row] = rs.s;
    }
}

template <typename T>
hipError_t launch_quantize(const T *x, int64_t M, int K, int8_t *xq, float *xs, hipStream_t stream) {
    const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock));
    const dim3 block(kRowsPerBlock * kWave);
    const int chunks_per_lane = ((K >> 3) + kWave - 1) / kWave;
    switch (chunks_per_lane) {
#define W8A8_Q_CASE(n) \
    case n: quantize_rows_kernel<T, n><<<grid, block, 0, stream>>>(x, M, K, xq, xs); break;
        W8A8_Q_CASE(1)
        W8A8_Q_CASE(2)
        W8A8_Q_CASE(3)
        W8A8_Q_CASE(4)
        W8A8_Q_CASE(5)
        W8A8_Q_CASE(6)
        W8A8_Q_CASE(7)
        W8A8_Q_CASE(8)
#undef W8A8_Q_CASE
        default:
            static_assert(kMaxRegChunks == 8, "switch covers 1..kMaxRegChunks");
            quantize_rows_kernel<T, 0><<<grid, block, 0, stream>>>(x, M, K, xq, xs);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows_bf16(const uint16_t *x, int64_t M, int K, int8_t *xq, float *xs,
                                     hipStream_t stream) {
    return launch_quantize<uint16_t>(x, M, K, xq, xs, stream);
}

hipError_t launch_quantize_rows_f32(const float *x, int64_t M, int K, int8_t *xq, float *xs,
                                    hipStream_t stream) {
    return launch_quantize<float>(x, M, K, xq, xs, stream);
}

}  // namespace w8a8
