// W4A16: asymmetric group-wise 4-bit weights, bf16 activations (pytorch/ao
// PR #153, fused HQQ quantization GEMM: u4 weights upcast to bf16, scaled and
// shifted group-wise by bf16 scales and zero points, then multiplied with the
// bf16 activations; quantization along K).
//
//   w[n,k] = bf16(bf16(q[n,k] - z[n,g]) * s[n,g]),  g = k / G
//   out[m,n] = bf16(sum_k x[m,k] * w[n,k])           (fp32 accumulation)
//
// Packing: byte j of weight row n holds q[n,2j] in its low nibble and
// q[n,2j+1] in its high nibble (the pages' simple row interleave: no tiling or
// reordering of the weight). q - z is exact in fp32 (q <= 15, z a bf16), and
// so is the product of two bf16 values, so each bf16() below is one
// round-to-nearest-even of the exact value, as in the elementwise bf16
// arithmetic it stands for, and the dequantized weights are bit-exact.
#include "common.hpp"
#include "launch.hpp"

namespace w4a16 {
namespace {

using w8a8::kWave;
using w8a8::pack_bf16x2;
using w8a8::bf16_lo;
using w8a8::bf16_hi;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_float(uint16_t bits) {
    return __uint_as_float((uint32_t)bits << 16);
}

// 8 codes (code e in bits 4e .. 4e+3) -> 8 bf16 weights, packed 2 per word.
__device__ __forceinline__ uint4 dequant8(uint32_t packed, float s, float z) {
    const uint32_t even = packed & 0x0F0F0F0Fu, odd = (packed >> 4) & 0x0F0F0F0Fu;
    float d[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        d[2 * b] = (float)((even >> (8 * b)) & 0xFFu) - z;
        d[2 * b + 1] = (float)((odd >> (8 * b)) & 0xFFu) - z;
    }
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const uint32_t shifted = pack_bf16x2(d[2 * h], d[2 * h + 1]);   // bf16(q - z)
        o[h] = pack_bf16x2(bf16_lo(shifted) * s, bf16_hi(shifted) * s);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// One thread per 8 weights: w [N,K] bf16.
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t *__restrict__ wq4,
                                                       const uint16_t *__restrict__ scales,
                                                       const uint16_t *__restrict__ zeros,
                                                       int64_t words, int K, int G,
                                                       uint4 *__restrict__ w) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= words) return;
    const int64_t k8 = t * 8;                    // first column of the 8, row-major
    const int64_t n = k8 / K;
    const int k = (int)(k8 % K);
    const int64_t gi = n * (K / G) + k / G;
    w[t] = dequant8(wq4[t], bf16_to_float(scales[gi]), bf16_to_float(zeros[gi]));
}

// Weight-streaming W4A16 GEMM for M <= 64: one workgroup per 16 output
// channels, K split over 8 wavefronts in 128-column chunks, partials summed in
// LDS. v_mfma_f32_16x16x32_bf16 takes the dequantized weights first, so a
// lane ends with 4 consecutive channels of one activation row. Within a chunk
// lane quarter q takes columns [32q, 32q+32): one 16-byte load of 32 codes and
// 64 contiguous activation bytes per row block, fed to the MFMA as 4 K steps
// of 8 columns (the same permutation of K on both operands).
constexpr int kSplit = 8;

template <int MT>
__global__ __launch_bounds__(kSplit *kWave) void w4a16_decode_kernel(
    const uint16_t *__restrict__ X, const uint8_t *__restrict__ wq4,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ out, int M, int N, int K, int G, int chunks_per_wave) {
    __shared__ float red[kSplit][MT][4][kWave];

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int n0 = blockIdx.x * 16;
    const int r16 = lane & 15, q = lane >> 4;
    const int n = n0 + r16;
    const uint8_t *wrow = wq4 + (int64_t)n * (K / 2) + 16 * q;
    const uint16_t *srow = scales + (int64_t)n * (K / G), *zrow = zeros + (int64_t)n * (K / G);
    const uint16_t *xrow[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) xrow[mb] = X + (int64_t)min(mb * 16 + r16, M - 1) * K + 32 * q;

    const int chunks = K / 128;
    const int c_begin = wave * chunks_per_wave;
    const int c_end = min(c_begin + chunks_per_wave, chunks);

    v4f acc[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) acc[mb] = v4f{};
    for (int c = c_begin; c < c_end; ++c) {
        const uint4 codes = *reinterpret_cast<const uint4 *>(wrow + 64 * c);
        const int g = (128 * c + 32 * q) / G;
        const float s = bf16_to_float(srow[g]), z = bf16_to_float(zrow[g]);
        uint4 xv[MT][4];
#pragma unroll
        for (int mb = 0; mb < MT; ++mb)
#pragma unroll
            for (int t = 0; t < 4; ++t) xv[mb][t] = *reinterpret_cast<const uint4 *>(xrow[mb] + 128 * c + 8 * t);
        const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const v8bf a = __builtin_bit_cast(v8bf, dequant8(cw[t], s, z));
#pragma unroll
            for (int mb = 0; mb < MT; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    a, __builtin_bit_cast(v8bf, xv[mb][t]), acc[mb], 0, 0, 0);
        }
    }

#pragma unroll
    for (int mb = 0; mb < MT; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][mb][r][lane] = acc[mb][r];
    __syncthreads();

    // one output per thread: channel ch of row j of row block mb sits in lane
    // j + 16 * (ch / 4), element ch % 4; the K-split partials add in fp32
    for (int e = threadIdx.x; e < MT * 256; e += kSplit * kWave) {
        const int mb = e >> 8, j = (e >> 4) & 15, ch = e & 15;
        const int m = mb * 16 + j;
        if (m >= M) continue;
        const int l = j + 16 * (ch >> 2), r = ch & 3;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < kSplit; ++w) sum += red[w][mb][r][l];
        out[(int64_t)m * N + n0 + ch] = (uint16_t)(pack_bf16x2(sum, 0.0f) & 0xFFFFu);
    }
}

template <int MT>
hipError_t launch_decode_mt(const uint16_t *x, int M, const uint8_t *wq4, const uint16_t *scales,
                            const uint16_t *zeros, int N, int K, int G, uint16_t *out,
                            hipStream_t stream) {
    const int chunks_per_wave = (K / 128 + kSplit - 1) / kSplit;
    w4a16_decode_kernel<MT><<<dim3((unsigned)(N / 16)), dim3(kSplit * kWave), 0, stream>>>(
        x, wq4, scales, zeros, out, M, N, K, G, chunks_per_wave);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const uint8_t *wq4, const uint16_t *scales, const uint16_t *zeros, int N,
                          int K, int G, uint16_t *w, hipStream_t stream) {
    const int64_t words = (int64_t)N * K / 8;
    dequant_kernel<<<dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream>>>(
        reinterpret_cast<const uint32_t *>(wq4), scales, zeros, words, K, G,
        reinterpret_cast<uint4 *>(w));
    return hipGetLastError();
}

hipError_t launch_gemm(const uint16_t *x, int M, const uint8_t *wq4, const uint16_t *scales,
                       const uint16_t *zeros, int N, int K, int G, uint16_t *out,
                       hipStream_t stream) {
    switch ((M + 15) / 16) {
        case 1: return launch_decode_mt<1>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        case 2: return launch_decode_mt<2>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        case 3: return launch_decode_mt<3>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        case 4: return launch_decode_mt<4>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        default: return hipErrorNotSupported;
    }
}

}  // namespace w4a16
