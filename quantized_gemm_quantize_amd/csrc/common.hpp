// Device-side building blocks shared by the W8A8 kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;   // CDNA wavefront width
constexpr int kXcds = 8;    // MI355X: 8 accelerator complex dies, 32 CUs each

// int8 MFMA, 32x32 output tile, K = 32 per instruction (16 int8 per lane per
// operand). Output layout (lane l, element r of the v16i):
//   column = l % 32, row = 8 * (r / 4) + 4 * (l / 32) + r % 4.
__device__ __forceinline__ v16i mfma_32x32x32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// int8 MFMA, 16x16 output tile, K = 64 per instruction. Output layout
// (lane l, element r of the v4i): column = l % 16, row = 4 * (l / 16) + r.
__device__ __forceinline__ v4i mfma_16x16x64(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Two floats -> two bf16 (round to nearest even; v_cvt_pk_bf16_f32 on gfx950),
// packed into one 32-bit word, first value in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    v2f f = {lo, hi};
    v2bf b = __builtin_convertvector(f, v2bf);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Map the hardware dispatch order (workgroup i runs on XCD i % 8) to a tile
// order in which every XCD owns one contiguous range of tiles, so tiles that
// share operand rows land in the same L2. A bijection on [0, tiles).
__device__ __forceinline__ int xcd_contiguous(int pid, int tiles) {
    const int q = tiles / kXcds, r = tiles % kXcds;
    const int xcd = pid % kXcds, idx = pid / kXcds;
    const int base = xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q;
    return base + idx;
}

// Dequantization of an int32 accumulator, acc * sa * sb, without an
// intermediate that overflows or underflows where the result does not: each
// scale is split once into a significand in [0.5, 1) and a power of two
// (v_frexp_*), the int32 is multiplied by the two significands (two fp32
// roundings, no overflow: |acc| < 2^31) and the exponents are applied last
// with one v_ldexp_f32 (exact unless the result is subnormal or overflows).
// The result is within 2^-23 (relative) of the exact product, far inside one
// bf16 ulp (2^-8). A left-to-right (acc * sa) * sb would overflow to inf for
// rows of magnitude ~1e37 whose exact output is a finite bf16.
struct SplitScale {
    float f;  // significand, [0.5, 1), or 0
    int e;    // power of two
};

__device__ __forceinline__ SplitScale split_scale(float s) {
    return SplitScale{__builtin_amdgcn_frexp_mantf(s), __builtin_amdgcn_frexp_expf(s)};
}

__device__ __forceinline__ float dequant(int acc, SplitScale a, SplitScale b) {
    return __builtin_amdgcn_ldexpf((float)acc * a.f * b.f, a.e + b.e);
}

// A scale that is 0 or in [2^-40, 2^40]. When both scales of an output are
// tame, the plain left-to-right (acc * sa) * sb stays in the fp32 normal
// range for every int32 acc (|acc * sa| <= 2^71, the product <= 2^111, both
// >= 2^-80 unless zero), so its three roundings (int32 -> fp32, two products)
// keep it within 2^-22 of the exact value: the cheaper form applies. Kernels
// whose epilogue is arithmetic-heavy take it when every scale a wavefront
// touches is tame (a wave-uniform vote) and the split form otherwise.
__device__ __forceinline__ bool tame_scale(float s) {
    const uint32_t u = __float_as_uint(s);
    return u == 0 || u - 0x2B800000u <= 0x53800000u - 0x2B800000u;
}

__device__ __forceinline__ bool wave_all(bool p) { return __builtin_amdgcn_ballot_w64(!p) == 0; }

// LDS poisoning, for the debug build compiled with -DW8A8_LDS_POISON: every
// kernel fills its LDS arrays with a fixed byte pattern (0xA5) and meets at a
// barrier before its first LDS access. A read of LDS that the launch has not
// written then returns the pattern instead of what an earlier launch left
// there, which can be the right data when the same inputs run twice; the
// poisoned build must give bit-identical outputs. In the normal build both
// calls compile to nothing.
template <typename T>
__device__ __forceinline__ void lds_poison(T &array) {
#ifdef W8A8_LDS_POISON
    static_assert(sizeof(T) % 4 == 0, "LDS arrays are whole words");
    uint32_t *w = reinterpret_cast<uint32_t *>(&array);
    for (int i = threadIdx.x; i < (int)(sizeof(T) / 4); i += blockDim.x) w[i] = 0xA5A5A5A5u;
#else
    (void)array;
#endif
}

__device__ __forceinline__ void lds_poison_done() {
#ifdef W8A8_LDS_POISON
    __syncthreads();
#endif
}

// addmm epilogue of the GEMMs (bf16 output): out[m, n] = bf16(alpha * (acc *
// sa[m] * sb[n]) + beta * bias[n]); no bias term when bias is null.
struct Addmm {
    const float *bias;
    float alpha, beta;
};

template <bool ADDMM>
__device__ __forceinline__ float addmm(float v, const Addmm &am, float b) {
    if constexpr (ADDMM) {
        v = am.alpha * v;
        if (am.bias) v = v + am.beta * b;
    }
    return v;
}

// Workgroup barrier without a memory fence, for kernels whose loads go
// straight to LDS: this wavefront's vector-memory operations up to the last N
// have completed and its LDS operations are done, then all wavefronts meet.
// (A release fence would wait for every load in flight, including those of
// later pipeline stages.) The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
template <int N>
__device__ __forceinline__ void vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Workgroup barrier that waits for this wavefront's LDS operations only
// (lgkmcnt(0)); outstanding vector-memory stores are left to drain.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16-byte load with the nontemporal (streaming) hint, for data read exactly
// once (the row quantization's input, the M-small kernels' weights): the hint
// keeps it from displacing reused lines (activations, codes) in the caches.
// Measured: row quantization of 2048 x 4096 bf16 9.0 -> 7.3 us; the M = 16
// weight-streaming GEMM (K = N = 4096) 5.86 -> 5.54 us.
__device__ __forceinline__ uint4 load16_stream(const void *p) {
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p)));
}

// The cache-policy operand of global_load_lds (direct-to-LDS) that sets the
// same nontemporal bit.
constexpr int kLdsLoadStream = 2;

// 16-byte streaming (nontemporal) store.
__device__ __forceinline__ void store16_nt(void *p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(v4i, v), reinterpret_cast<v4i *>(p));
}

}  // namespace w8a8
