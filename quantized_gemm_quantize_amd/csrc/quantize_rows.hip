// Dynamic per-row int8 quantization.
//
//   s = fl32(absmax / 127);  q = clamp(rint(fl32(x / s)), -127, 127)
//
// (absmax / 127 scale: Paddle sparse_fc PR #41770, spmm_plugin.cu weight-scale
// hunk; clamp before the cast: vLLM csrc/quantization log, FP8 clamp commit.)
//
// The pass is HBM bound (2 or 4 bytes in, 1 byte out per element). A row is
// split over WPR wavefronts (several for long rows, so a short batch still
// fills the chip); every lane moves 16 input bytes per load, the absmax is
// reduced across lanes with shuffles and across the row's wavefronts through
// LDS, and rows of up to NCH*64*8*WPR elements stay in registers so the input
// is read once (with the streaming hint, as nothing reads it again).
//
// The element arithmetic (exact division on multiplies, rounding, the byte)
// is in quant_math.hpp.
#include <algorithm>
#include <type_traits>

#include "launch.hpp"
#include "quant_math.hpp"

namespace w8a8 {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kMaxRegChunks = 8;     // chunks of 8 elements held per lane

__device__ __forceinline__ uint32_t wave_max(uint32_t bits) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = __shfl_xor(bits, off, kWave);
        bits = bits > o ? bits : o;
    }
    return bits;
}

// Row m is handled by WPR consecutive wavefronts; wavefront w of the row takes
// the 8-element chunks w*64 + lane + c*64*WPR (so the row's wavefronts read
// consecutive kilobytes). NCH > 0: at most NCH chunks per lane, held in
// registers. NCH == 0: any K, the row is read twice (the second read hits L2).
template <typename T, int NCH, int WPR>
__global__ __launch_bounds__(kThreads) void quantize_rows_kernel(
    const T *__restrict__ x, int64_t M, int K, int8_t *__restrict__ xq, float *__restrict__ xs) {
    constexpr int kRowsPerBlock = kWavesPerBlock / WPR;
    __shared__ uint32_t red[kWavesPerBlock];
    lds_poison(red);
    lds_poison_done();
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int sub = wave % WPR;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + wave / WPR;
    const bool live = row < M;  // uniform per wavefront
    const T *xr = x + (live ? row : 0) * K;
    int8_t *qr = xq + (live ? row : 0) * K;
    const int nch = K >> 3;  // 8-element chunks (K % 16 == 0)
    const int first = sub * kWave + lane, stride = kWave * WPR;

    uint32_t amax = 0;
    float v[NCH > 0 ? NCH : 1][8];
    if constexpr (NCH > 0) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = first + c * stride;
            if (live && ch < nch) load8<true>(xr + ch * 8, v[c], amax);
        }
    } else {
        // read twice: the second pass should find the row in L2
        for (int ch = first; live && ch < nch; ch += stride) load8<false>(xr + ch * 8, v[0], amax);
    }
    amax = wave_max(amax);
    if constexpr (WPR > 1) {
        if (lane == 0) red[wave] = amax;
        __syncthreads();
        const int base = (wave / WPR) * WPR;
#pragma unroll
        for (int w = 0; w < WPR; ++w) amax = max(amax, red[base + w]);
    }
    if (!live) return;
    const RowScale rs = row_scale(__uint_as_float(amax));
    if constexpr (NCH > 0) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = first + c * stride;
            if (ch < nch) *reinterpret_cast<uint2 *>(qr + ch * 8) = quantize8(v[c], rs);
        }
    } else {
        for (int ch = first; ch < nch; ch += stride) {
            uint32_t unused = 0;
            load8<false>(xr + ch * 8, v[0], unused);
            *reinterpret_cast<uint2 *>(qr + ch * 8) = quantize8(v[0], rs);
        }
    }
    if (sub == 0 && lane == 0) xs[row] = rs.s;
}

// Persistent variant for bf16 rows held in registers, taken for rows split
// over two or four wavefronts. With more row groups than workgroups (PIPE),
// workgroup b runs through the row groups b, b + G, b + 2G, ... (G =
// gridDim.x) and issues the loads of the next group before it reduces,
// quantizes and stores the current one, so its stores overlap its next loads
// (16448 x 5120, two wavefronts per row: 53.8 -> 51.1 us against one
// workgroup per row group). When every workgroup owns exactly one row group
// (!PIPE: 2048 x 4096, 16 x 4096) it holds one register set, 44 VGPRs instead
// of 80, so all its wavefronts are resident at once (2048 x 4096: 7.70 ->
// 7.37 us). Loads are clamped into the input (a chunk past the row repeats the
// row's last chunk, a row past M repeats row M - 1): they never branch, and
// what they bring past the row or past M is not stored. With one wavefront
// per row the pipelined form measured slower than one workgroup per row group
// (38400 x 1024: 25.7 -> 28.4 us), so those keep the plain kernel.
constexpr int kPersistBlocksPerCU = 16;

template <int NCH, int WPR, bool PIPE>
__global__ __launch_bounds__(kThreads) void quantize_rows_persistent(
    const uint16_t *__restrict__ x, int64_t M, int K, int8_t *__restrict__ xq,
    float *__restrict__ xs) {
    constexpr int kRowsPerBlock = kWavesPerBlock / WPR;
    __shared__ uint32_t red[2][kWavesPerBlock];  // by iteration parity
    lds_poison(red);
    lds_poison_done();
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int sub = wave % WPR;
    const int nch = K >> 3;
    const int first = sub * kWave + lane, stride = kWave * WPR;
    const int64_t groups = (M + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t G = gridDim.x;

    auto load_raw = [&](int64_t g, uint4 (&u)[NCH]) {
        const int64_t row = min(g * kRowsPerBlock + wave / WPR, M - 1);
        const uint16_t *xr = x + row * K;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            u[c] = load16_stream(xr + 8 * min(first + c * stride, nch - 1));
    };
    auto process = [&](int64_t g, const uint4 (&u)[NCH], int parity) {
        const int64_t row = g * kRowsPerBlock + wave / WPR;
        const bool live = row < M;  // uniform per wavefront
        uint32_t amax = 0;
#pragma unroll
        for (int c = 0; c < NCH; ++c) absmax8(u[c], amax);  // repeated chunks change nothing
        amax = wave_max(amax);
        if constexpr (WPR > 1) {
            if (lane == 0) red[parity][wave] = amax;
            __syncthreads();
            const int base = (wave / WPR) * WPR;
#pragma unroll
            for (int w = 0; w < WPR; ++w) amax = max(amax, red[parity][base + w]);
        }
        if (!live) return;
        const RowScale rs = row_scale(__uint_as_float(amax));
        int8_t *qr = xq + row * K;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int ch = first + c * stride;
            if (ch < nch) {
                float v[8];
                widen8(u[c], v);
                *reinterpret_cast<uint2 *>(qr + ch * 8) = quantize8(v, rs);
            }
        }
        if (sub == 0 && lane == 0) xs[row] = rs.s;
    };

    // two register sets, alternating (a copy between them would wait for the
    // load); every wavefront of the workgroup runs the same iterations, so the
    // barriers inside process() are reached by all
    // (the guards are uniform: a workgroup never fetches a group it will not
    // process)
    int64_t g = blockIdx.x;
    if constexpr (!PIPE) {
        // one row group per workgroup (G >= groups): a single register set, so
        // the kernel stays within 64 VGPRs and every wavefront is resident
        uint4 ua[NCH];
        load_raw(g, ua);
        process(g, ua, 0);
        return;
    }
    uint4 ua[NCH], ub[NCH];
    load_raw(g, ua);
    for (; g < groups; g += 2 * G) {
        if (g + G < groups) load_raw(g + G, ub);
        process(g, ua, 0);
        if (g + G >= groups) break;
        if (g + 2 * G < groups) load_raw(g + 2 * G, ua);
        process(g + G, ub, 1);
    }
}

template <typename T, int WPR>
hipError_t launch_wpr(const T *x, int64_t M, int K, int8_t *xq, float *xs, hipStream_t stream) {
    constexpr int kRowsPerBlock = kWavesPerBlock / WPR;
    const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock)), block(kThreads);
    const int chunks_per_lane = ((K >> 3) + kWave * WPR - 1) / (kWave * WPR);
    constexpr bool kPersist = std::is_same<T, uint16_t>::value && WPR >= 2;
    const int64_t groups = (M + kRowsPerBlock - 1) / kRowsPerBlock;
    const dim3 pgrid((unsigned)std::min<int64_t>(groups, (int64_t)kPersistBlocksPerCU * device_cu_count()));
    switch (chunks_per_lane) {
#define W8A8_Q_CASE(n)                                                                       \
    case n:                                                                                  \
        if constexpr (kPersist) {                                                            \
            if (groups <= (int64_t)pgrid.x)                                                  \
                quantize_rows_persistent<n, WPR, false><<<pgrid, block, 0, stream>>>(        \
                    reinterpret_cast<const uint16_t *>(x), M, K, xq, xs);                    \
            else                                                                             \
                quantize_rows_persistent<n, WPR, true><<<pgrid, block, 0, stream>>>(         \
                    reinterpret_cast<const uint16_t *>(x), M, K, xq, xs);                    \
        } else                                                                               \
            quantize_rows_kernel<T, n, WPR><<<grid, block, 0, stream>>>(x, M, K, xq, xs);     \
        break;
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
            quantize_rows_kernel<T, 0, WPR><<<grid, block, 0, stream>>>(x, M, K, xq, xs);
    }
    return hipGetLastError();
}

// Four wavefronts per row while that still leaves at least 8192 wavefronts
// and each lane 2+ chunks; otherwise the fewest wavefronts per row (1, 2 or
// 4) that hold the row in registers, so it is read once.
template <typename T>
hipError_t launch_quantize(const T *x, int64_t M, int K, int8_t *xq, float *xs, hipStream_t stream) {
    if (M < 8192 && K >= 4 * kWave * 8 * 2) return launch_wpr<T, 4>(x, M, K, xq, xs, stream);
    if (K <= kWave * 8 * kMaxRegChunks) return launch_wpr<T, 1>(x, M, K, xq, xs, stream);
    if (K <= 2 * kWave * 8 * kMaxRegChunks) return launch_wpr<T, 2>(x, M, K, xq, xs, stream);
    return launch_wpr<T, 4>(x, M, K, xq, xs, stream);
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
