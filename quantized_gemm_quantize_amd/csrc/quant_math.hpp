// Element arithmetic of the dynamic per-row quantization, shared by the
// quantize kernel and the fused small-M linear:
//
//   s = fl32(absmax / 127);  q = clamp(rint(fl32(x / s)), -127, 127)
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
//
// Rounding and the byte in one add: for |t| < 2^22, m = fl(t + 1.5 * 2^23)
// rounds t to the nearest integer, ties to even, and the low byte of m's bit
// pattern is that integer in two's complement. |t| <= 127 here, so the clamp
// of the definition never binds on this path.
//
// Every translation unit that includes this is compiled with correctly
// rounded binary32 division and without FP contraction.
#pragma once

#include "common.hpp"

namespace w8a8 {

constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kTieGuard = 0.5f - 0x1p-14f;

// The absmax of 8 packed bf16 folded into `amax`, kept as the bit pattern of
// a non-negative float (such floats order like their bit patterns).
__device__ __forceinline__ void absmax8(uint4 u, uint32_t &amax) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const uint32_t a = w[h] & 0x7FFF7FFFu;
        const uint32_t lo = a & 0xFFFFu, hi = a >> 16;
        amax = max(amax, max(lo, hi) << 16);
    }
}

// 8 packed bf16 -> float (exact).
__device__ __forceinline__ void widen8(uint4 u, float v[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        v[2 * h] = bf16_lo(w[h]);
        v[2 * h + 1] = bf16_hi(w[h]);
    }
}

// 16 bytes, with the streaming hint (load16_stream) when STREAM.
template <bool STREAM>
__device__ __forceinline__ uint4 load16(const void *p) {
    if constexpr (STREAM) return load16_stream(p);
    return *reinterpret_cast<const uint4 *>(p);
}

// 8 consecutive inputs -> float, and their absmax folded into `amax`.
// STREAM: the input is read only this once (see load16_stream).
template <bool STREAM>
__device__ __forceinline__ void load8(const uint16_t *p, float v[8], uint32_t &amax) {
    const uint4 u = load16<STREAM>(p);
    widen8(u, v);
    absmax8(u, amax);
}

template <bool STREAM>
__device__ __forceinline__ void load8(const float *p, float v[8], uint32_t &amax) {
    const float4 a = __builtin_bit_cast(float4, load16<STREAM>(p));
    const float4 b = __builtin_bit_cast(float4, load16<STREAM>(p + 4));
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    float m = __uint_as_float(amax);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
    amax = __float_as_uint(m);
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

// The byte of rint(fl(x / s)) clamped to [-127, 127], by IEEE division
// (s > 0).
__device__ __forceinline__ uint32_t quantize_div(float x, float s) {
    const float q = __builtin_fminf(__builtin_fmaxf(x / s, -127.0f), 127.0f);
    return __float_as_uint(q + kMagic) & 0xFFu;
}

__device__ __forceinline__ uint32_t pack4(uint32_t b0, uint32_t b1, uint32_t b2, uint32_t b3) {
    return (b0 & 0xFFu) | ((b1 & 0xFFu) << 8) | ((b2 & 0xFFu) << 16) | (b3 << 24);
}

// The divisor as seen inside a rarely taken branch. An IEEE division is one
// instruction to the optimizer but about fifteen once expanded, so left alone
// the compiler computes the fallback's divisions ahead of the branch and every
// element pays for them. Passing the divisor through an empty volatile asm
// statement inside the branch makes the divisions depend on a value that only
// exists there: they stay behind the branch.
__device__ __forceinline__ float branch_local(float s) {
    asm volatile("" : "+v"(s));
    return s;
}

// 8 values -> 8 int8 codes (two packed words). The fallback is branched per
// element: element e takes the division only when some lane of the wavefront
// has its element e near a tie (about 64 / 8000 of the time), instead of all
// eight elements whenever any of them is (about 8 x 64 / 8000): 2048 rows of
// 4096 N(0, 2) values quantize in 7.7 us instead of 9.0 us.
__device__ __forceinline__ uint2 quantize8(const float v[8], const RowScale &rs) {
    uint32_t b[8];
    if (rs.fast) {
        bool near_tie[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float t = v[e] * rs.r;
            const float m = t + kMagic;
            const float k = m - kMagic;  // rint(t), exact
            near_tie[e] = __builtin_fabsf(t - k) >= kTieGuard;
            b[e] = __float_as_uint(m);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (near_tie[e]) b[e] = quantize_div(v[e], branch_local(rs.s));
    } else if (rs.s != 0.0f) {  // subnormal scale: 1 / s would overflow
        const float s = branch_local(rs.s);
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = quantize_div(v[e], s);
    } else {  // all-zero row
#pragma unroll
        for (int e = 0; e < 8; ++e) b[e] = 0;
    }
    return make_uint2(pack4(b[0], b[1], b[2], b[3]), pack4(b[4], b[5], b[6], b[7]));
}

}  // namespace w8a8
