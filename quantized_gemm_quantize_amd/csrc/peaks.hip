// On-device reference rates for the benchmark (not part of the W8A8 path):
// the int8 MFMA issue rate and the HBM streaming read and write rates that the
// kernels' roofline fractions are also quoted against, measured on the same
// GPU in the same run as the kernels, since MI355X's clock under int8 MFMA
// load is power-limited below the nominal peak's 2.4 GHz.
//
// peaks_mfma_i8: each wavefront runs `iters` rounds of 8 independent
//   v_mfma_i32_32x32x32_i8 on register operands (8 accumulators, so the issue
//   never waits on a result); 65536 ops each. The operands are varied per lane
//   so the multipliers toggle as under real data.
// peaks_mfma_bf16: the same with v_mfma_f32_32x32x16_bf16 (32768 flops each;
//   operands are finite bf16 values in [1, 2) whose mantissas vary per lane).
// peaks_read: every thread reads 16-byte chunks, grid-stride, with the
//   nontemporal hint (as the kernels that read their weights once do), and
//   folds them into one word per thread (written once, so the loads cannot be
//   dropped).
// peaks_write: every thread writes 16-byte chunks, grid-stride, with streaming
//   stores (as the GEMM epilogues do).
// peaks_operand_stream: the large-M GEMM's operand stream alone (256 x 128
//   tiles in its tile order, 128-byte K stages through a 3-stage direct-to-LDS
//   ring with its counted waits and one barrier per stage; no fragment reads,
//   MFMAs or epilogue): the time that kernel's loads take by themselves.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_loop(int iters, int *sink, uint64_t *clk) {
    const int lane = threadIdx.x & 63;
    // the shader clock over the loop: s_memtime counts core clocks, s_memrealtime
    // the constant 100 MHz reference (workgroup 0, first wavefront)
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    v4i a = {lane * 0x01030507 + 0x11, lane * 0x0f0d0b09 + 0x2b, lane ^ 0x5a5a5a5a, ~lane * 0x01010101};
    v4i b = {lane * 0x07050301 + 0x3d, lane ^ 0x3c3c3c3c, lane * 0x090b0d0f + 0x47, lane * 0x13171d1f};
    v16i acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = v16i{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, acc[i], 0, 0, 0);
        a = a ^ (v4i){it, it, it, it};  // keeps the operands varied, off the MFMA's critical path
    }
    int s = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s ^= acc[i][e];
    if (s == 0x7fffffff) sink[blockIdx.x] = s;  // practically never: keeps the loop alive
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        clk[0] = c1 - c0;
        clk[1] = r1 - r0;
    }
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_loop_bf16(int iters, int *sink, uint64_t *clk) {
    const int lane = threadIdx.x & 63;
    const uint64_t c0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
    // 8 bf16 per operand: exponent of 1.0 (0x3F80), mantissa bits from the lane
    v4i a = {0x3F803F80 | (lane * 0x00130017 & 0x007F007F), 0x3F803F80 | (lane * 0x001D0005 & 0x007F007F),
             0x3F803F80 | ((lane ^ 0x55) * 0x00070003 & 0x007F007F), 0x3F803F80 | (~lane & 0x007F007F)};
    v4i b = {0x3F803F80 | (lane * 0x000B0029 & 0x007F007F), 0x3F803F80 | ((lane ^ 0x33) & 0x007F007F),
             0x3F803F80 | (lane * 0x00250011 & 0x007F007F), 0x3F803F80 | (lane * 0x0003001F & 0x007F007F)};
    v16f acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = v16f{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b),
                                                             acc[i], 0, 0, 0);
        const int m = it & 0x007F;
        a = a ^ (v4i){m, m << 16, m, m << 16};  // mantissa bits only: the operands stay in [1, 2)
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][e];
    if (s == -1.0f) sink[blockIdx.x] = 1;  // never (every product is positive): keeps the loop alive
    const uint64_t c1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        clk[0] = c1 - c0;
        clk[1] = r1 - r0;
    }
}

__global__ __launch_bounds__(256) void read_loop(const uint4 *__restrict__ p, int64_t n16,
                                                 uint32_t *__restrict__ sink) {
    uint32_t s = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p + i));
        s ^= (uint32_t)(v.x ^ v.y ^ v.z ^ v.w);
    }
    if (s == 0x9e3779b9u) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// A [rows, 4096] byte matrix read the way the M-small GEMM reads its weight:
// workgroup b takes rows 16b .. 16b+15, its wavefront w the 1 KB column slice
// [1024 w, +1024), and every lane issues all 16 of its 16-byte loads (8 rows x
// 128 bytes per instruction) before using any of them.
__global__ __launch_bounds__(256) void read_rows(const int8_t *__restrict__ p, uint32_t *__restrict__ sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int8_t *base = p + (int64_t)blockIdx.x * 16 * 4096 + 1024 * wave + 16 * (lane & 7);
    v4i v[16];
#pragma unroll
    for (int q = 0; q < 16; ++q)
        v[q] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(
            base + (int64_t)(8 * (q & 1) + (lane >> 3)) * 4096 + 128 * (q >> 1)));
    v4i a = v[0];
#pragma unroll
    for (int q = 1; q < 16; ++q) a ^= v[q];
    const uint32_t s = (uint32_t)(a.x ^ a.y ^ a.z ^ a.w);
    if (s == 0x9e3779b9u) sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// Wait until at most N vector-memory operations are outstanding, then meet the
// workgroup at a barrier.
template <int N>
__device__ __forceinline__ void vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A [M, K] and B [N, K] int8 (M % 256 == 0, N % 128 == 0, K % 128 == 0),
// one workgroup of 4 wavefronts per 256 x 128 tile. Tile order: each XCD
// (workgroup i runs on XCD i % 8) owns a contiguous range of tiles, taken in
// groups of 4 tile rows. A stage is 384 rows x 128 bytes: load l of wavefront
// w fills 16-byte slots 64 (w + 4 l) .. of the stage, 8 rows x 128 bytes
// (chunk c of row r lands at slot 8 r + (c ^ (r % 8) ^ ((r / 8) % 2))). Stage
// s + 2 is issued before stage s + 1 is awaited.
__global__ __launch_bounds__(256, 1) void operand_stream(const int8_t *__restrict__ A,
                                                         const int8_t *__restrict__ B, int K,
                                                         int tiles_m, int tiles_n, uint32_t *sink) {
    constexpr int BM = 256, BN = 128, STAGE = (BM + BN) * 8, A_LD = BM / 32, NLD = (BM + BN) / 32;
    __shared__ uint4 lds[3 * STAGE];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int tiles = tiles_m * tiles_n;
    const int q = tiles / 8, r = tiles % 8, xcd = blockIdx.x % 8, idx = blockIdx.x / 8;
    const int t = (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
    const int per_group = 4 * tiles_n, first_m = (t / per_group) * 4;
    const int gsize = min(tiles_m - first_m, 4);
    const int m0 = (first_m + (t % per_group) % gsize) * BM, n0 = ((t % per_group) / gsize) * BN;
    const int row = 8 * wave + (lane >> 3);  // + 32 l
    const int kc = (lane & 7) ^ (row & 7) ^ ((row >> 3) & 1);
    const int8_t *src[NLD];
#pragma unroll
    for (int l = 0; l < NLD; ++l)
        src[l] = l < A_LD ? A + (int64_t)(m0 + row + 32 * l) * K + 16 * kc
                          : B + (int64_t)(n0 + row + 32 * (l - A_LD)) * K + 16 * kc;
    const int nk = K / 128;
    auto issue = [&](int s) {
        uint4 *dst = lds + (s % 3) * STAGE;
        const int k0 = 128 * min(s, nk - 1);  // stages past the last reload the last
#pragma unroll
        for (int l = 0; l < NLD; ++l)
            __builtin_amdgcn_global_load_lds((global_void *)(src[l] + k0), (lds_void *)(dst + 64 * (wave + 4 * l)),
                                             16, 0, 0);
    };
    issue(0);
    issue(1);
    vm_barrier<NLD>();
    for (int s = 0; s < nk; ++s) {
        issue(s + 2);
        vm_barrier<NLD>();
    }
    vm_barrier<0>();
    const uint32_t v = reinterpret_cast<const uint32_t *>(lds)[threadIdx.x];
    if (v == 0x9e3779b9u) sink[blockIdx.x * blockDim.x + threadIdx.x] = v;
}

__global__ __launch_bounds__(256) void write_loop(uint4 *__restrict__ p, int64_t n16, uint32_t v) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
        typedef int v4 __attribute__((ext_vector_type(4)));
        __builtin_nontemporal_store((v4){(int)v, (int)i, (int)v, (int)i}, reinterpret_cast<v4 *>(p + i));
    }
}

}  // namespace

extern "C" {

// workgroups: launched workgroups of 256 threads; the ops are
// workgroups * 4 * iters * 8 * 65536. sink: at least `workgroups` ints.
// clk[0], clk[1]: core clocks and 100 MHz reference ticks over workgroup 0's
// loop (their ratio is the shader clock under int8 MFMA load).
int peaks_mfma_i8(int workgroups, int iters, int *sink, uint64_t *clk, void *stream) {
    if (workgroups <= 0 || iters <= 0 || !sink || !clk) return -1;
    mfma_loop<<<workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, sink, clk);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

// As peaks_mfma_i8, with bf16 operands: the flops are workgroups * 4 * iters * 8 * 32768.
int peaks_mfma_bf16(int workgroups, int iters, int *sink, uint64_t *clk, void *stream) {
    if (workgroups <= 0 || iters <= 0 || !sink || !clk) return -1;
    mfma_loop_bf16<<<workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, sink, clk);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

// bytes: a multiple of 16; sink: at least workgroups * 256 words.
int peaks_read(const void *buf, int64_t bytes, int workgroups, uint32_t *sink, void *stream) {
    if (bytes <= 0 || bytes % 16 || workgroups <= 0 || !buf || !sink) return -1;
    read_loop<<<workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const uint4 *>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

// rows: a positive multiple of 16 (rows of 4096 bytes); sink: at least
// rows / 16 * 256 words.
int peaks_read_rows(const void *buf, int rows, uint32_t *sink, void *stream) {
    if (rows <= 0 || rows % 16 || !buf || !sink) return -1;
    read_rows<<<rows / 16, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const int8_t *>(buf),
                                                                         sink);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

// a: [M, K], b: [N, K] int8; M a positive multiple of 256, N of 128, K of 128;
// sink: at least (M / 256) * (N / 128) * 256 words.
int peaks_operand_stream(const void *a, const void *b, int M, int N, int K, uint32_t *sink, void *stream) {
    if (!a || !b || !sink || M <= 0 || N <= 0 || K <= 0 || M % 256 || N % 128 || K % 128) return -1;
    const int tm = M / 256, tn = N / 128;
    operand_stream<<<tm * tn, 256, 0, static_cast<hipStream_t>(stream)>>>(
        static_cast<const int8_t *>(a), static_cast<const int8_t *>(b), K, tm, tn, sink);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

int peaks_write(void *buf, int64_t bytes, int workgroups, void *stream) {
    if (bytes <= 0 || bytes % 16 || workgroups <= 0 || !buf) return -1;
    write_loop<<<workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<uint4 *>(buf),
                                                                       bytes / 16, 0x5bd1e995u);
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
