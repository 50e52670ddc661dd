// W4A16: asymmetric group-wise 4-bit weights, bf16 activations (pytorch/ao
// PR #153, fused HQQ quantization GEMM: u4 weights upcast to bf16, scaled and
// shifted group-wise by bf16 scales and zero points, then multiplied with the
// bf16 activations; quantization along K).
//
//   w[n,k] = bf16(bf16(q[n,k] - z[n,g]) * s[n,g]),  g = k / G
//   out[m,n] = bf16(sum_k x[m,k] * w[n,k])           (fp32 accumulation)
//
// Packing: byte j of weight row n holds code c[n,2j] in its low nibble and
// c[n,2j+1] in its high nibble (the pages' simple row interleave: no tiling or
// reordering of the weight). q = c for unsigned codes (u4, 0..15) and the
// 4-bit two's complement of c for signed ones (s4, -8..7): the page's kernel
// takes both. q - z is exact in fp32 (q <= 15, z a bf16), and
// so is the product of two bf16 values, so each bf16() below is one
// round-to-nearest-even of the exact value, as in the elementwise bf16
// arithmetic it stands for, and the dequantized weights are bit-exact.
#include "common.hpp"
#include "launch.hpp"

namespace w4a16 {

// Wait until at most n vector-memory operations of this wavefront are
// outstanding (vmcnt(n); expcnt and lgkmcnt left alone).
#define W4A16_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
namespace {

using w8a8::kWave;
using w8a8::pack_bf16x2;
using w8a8::bf16_lo;
using w8a8::bf16_hi;
using w8a8::load16_stream;

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_float(uint16_t bits) {
    return __uint_as_float((uint32_t)bits << 16);
}

// The 16-bit format of activations, scales, zeros, weights and outputs: bf16,
// or IEEE binary16 with F16 (the page's kernel takes either). Conversions from
// fp32 round to nearest even, subnormals kept.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

template <bool F16>
__device__ __forceinline__ float h_to_float(uint16_t bits) {
    if constexpr (F16)
        return (float)__builtin_bit_cast(_Float16, bits);
    else
        return bf16_to_float(bits);
}

template <bool F16>
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    if constexpr (F16)
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
    else
        return pack_bf16x2(lo, hi);
}

template <bool F16>
__device__ __forceinline__ float h_lo(uint32_t w) {
    if constexpr (F16)
        return h_to_float<true>((uint16_t)(w & 0xFFFFu));
    else
        return bf16_lo(w);
}

template <bool F16>
__device__ __forceinline__ float h_hi(uint32_t w) {
    if constexpr (F16)
        return h_to_float<true>((uint16_t)(w >> 16));
    else
        return bf16_hi(w);
}

// MFMAs on 8 packed 16-bit values per lane (weights first), fp32 accumulation.
template <bool F16>
__device__ __forceinline__ v4f mfma16x16x32(uint4 a, uint4 b, v4f c) {
    if constexpr (F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a),
                                                      __builtin_bit_cast(v8h, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a),
                                                       __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

// 8 codes (code e in bits 4e .. 4e+3) -> 8 bf16 weights, packed 2 per word.
// S4: signed codes. c ^ 8 is q + 8 in 0..15, converted like an unsigned code;
// subtracting 8 is exact, so q - z still takes a single rounding. F16: the
// roundings and the result are binary16 instead of bf16.
template <bool S4, bool F16>
__device__ __forceinline__ uint4 dequant8(uint32_t packed, float s, float z) {
    if constexpr (S4) packed ^= 0x88888888u;
    uint32_t even = packed & 0x0F0F0F0Fu, odd = (packed >> 4) & 0x0F0F0F0Fu;
    // opaque to the optimizer: each code then converts with one
    // v_cvt_f32_ubyteN instead of a bit-field extract and a conversion
    asm volatile("" : "+v"(even), "+v"(odd));
    float d[8];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        float qe = (float)((even >> (8 * b)) & 0xFFu), qo = (float)((odd >> (8 * b)) & 0xFFu);
        if constexpr (S4) {
            qe -= 8.0f;
            qo -= 8.0f;
        }
        d[2 * b] = qe - z;
        d[2 * b + 1] = qo - z;
    }
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const uint32_t shifted = pack_h2<F16>(d[2 * h], d[2 * h + 1]);   // bf16(q - z)
        o[h] = pack_h2<F16>(h_lo<F16>(shifted) * s, h_hi<F16>(shifted) * s);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// One thread per 8 weights: w [N,K] bf16.
template <bool S4, bool F16>
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
    w[t] = dequant8<S4, F16>(wq4[t], h_to_float<F16>(scales[gi]), h_to_float<F16>(zeros[gi]));
}

// Weight-streaming W4A16 GEMM for M <= 64: one workgroup per 16 output
// channels, K split over 8 wavefronts in 128-column chunks, partials summed in
// LDS. v_mfma_f32_16x16x32_bf16 takes the dequantized weights first, so a
// lane ends with 4 consecutive channels of one activation row. Within a chunk
// lane quarter q takes columns [32q, 32q+32): one 16-byte load of 32 codes and
// 64 contiguous activation bytes per row block, fed to the MFMA as 4 K steps
// of 8 columns (the same permutation of K on both operands).
constexpr int kSplit = 8;

template <int MT, bool S4, bool F16>
__global__ __launch_bounds__(kSplit *kWave) void w4a16_decode_kernel(
    const uint16_t *__restrict__ X, const uint8_t *__restrict__ wq4,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ out, int M, int N, int K, int G, int chunks_per_wave) {
    __shared__ float red[kSplit][MT][4][kWave];
    w8a8::lds_poison(red);
    w8a8::lds_poison_done();

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
        const uint4 codes = load16_stream(wrow + 64 * c);
        const int g = (128 * c + 32 * q) / G;
        const float s = h_to_float<F16>(srow[g]), z = h_to_float<F16>(zrow[g]);
        uint4 xv[MT][4];
#pragma unroll
        for (int mb = 0; mb < MT; ++mb)
#pragma unroll
            for (int t = 0; t < 4; ++t) xv[mb][t] = *reinterpret_cast<const uint4 *>(xrow[mb] + 128 * c + 8 * t);
        const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint4 a = dequant8<S4, F16>(cw[t], s, z);
#pragma unroll
            for (int mb = 0; mb < MT; ++mb)
                acc[mb] = mfma16x16x32<F16>(a, xv[mb][t], acc[mb]);
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
        out[(int64_t)m * N + n0 + ch] = (uint16_t)(pack_h2<F16>(sum, 0.0f) & 0xFFFFu);
    }
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// Weight-streaming W4A16 GEMM for M <= 16 and K a multiple of 4096, with the
// activations moved global -> LDS by 16-byte direct-to-LDS loads. At M = 16
// every workgroup reads all 16 x K bf16 activations, four times the bytes of
// its weight codes; loaded straight into the MFMA fragment layout (lane
// quarter q takes 16-byte pieces 64 bytes apart) each load instruction
// touched 32 cache lines a quarter used. Here one load instruction fills 64
// LDS slots with 4 rows x 256 bytes of a 128-column chunk (8 whole lines).
// Slot p of a row holds the row's 16-byte piece p ^ row, so the fragment
// reads of the 16 lanes of a quarter (16 rows, one piece) hit 16 distinct
// bank groups. Wavefront w takes chunks 4w .. 4w+3 of every 4096-column
// block, issues all their loads at once (activations, codes, scale, zero per
// chunk) and multiplies each chunk as soon as its loads have landed (vector
// loads complete in order); each wavefront touches only its own LDS region.
// Rows past M are read from row M - 1 and never stored.
template <bool S4, bool F16>
__global__ __launch_bounds__(kSplit *kWave) void w4a16_decode_lds_kernel(
    const uint16_t *__restrict__ X, const uint8_t *__restrict__ wq4,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ out, int M, int N, int K, int G) {
    constexpr int kCpw = 4;                          // chunks per wavefront per block
    constexpr int kBlockCols = kSplit * kCpw * 128;  // 4096 columns per block
    constexpr int kChunkSlots = 16 * 16;             // 16 rows x 256 bytes
    constexpr int kLoadsPerChunk = 7;                // 4 activation loads, codes, scale, zero
    static_assert(kLoadsPerChunk * kCpw < 64, "vmcnt range");
    // one LDS array per chunk position: the compiler then knows which loads in
    // flight a fragment read may depend on, and waits for those only (with one
    // array it waits for every direct-to-LDS load before the first read)
    __shared__ uint4 lds0[kSplit * kChunkSlots], lds1[kSplit * kChunkSlots],
        lds2[kSplit * kChunkSlots], lds3[kSplit * kChunkSlots];
    __shared__ float red[kSplit][4][kWave];
    w8a8::lds_poison(lds0);
    w8a8::lds_poison(lds1);
    w8a8::lds_poison(lds2);
    w8a8::lds_poison(lds3);
    w8a8::lds_poison(red);
    w8a8::lds_poison_done();

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int n0 = blockIdx.x * 16;
    const int r16 = lane & 15, q = lane >> 4;
    const int n = n0 + r16;
    const uint8_t *wrow = wq4 + (int64_t)n * (K / 2) + 16 * q;
    const uint16_t *srow = scales + (int64_t)n * (K / G), *zrow = zeros + (int64_t)n * (K / G);
    // load i of a chunk: row 4 i + lane / 16, slot lane % 16 <- piece (lane % 16) ^ row
    const uint16_t *xsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * i + (lane >> 4);
        xsrc[i] = X + (int64_t)min(row, M - 1) * K + 8 * ((lane & 15) ^ row);
    }
    uint4 *const region[kCpw] = {lds0 + wave * kChunkSlots, lds1 + wave * kChunkSlots,
                                 lds2 + wave * kChunkSlots, lds3 + wave * kChunkSlots};

    v4f acc = v4f{};
    for (int kb = 0; kb < K; kb += kBlockCols) {
        const int c0 = (kb >> 7) + wave * kCpw;
        uint4 codes[kCpw];
        uint16_t sv[kCpw], zv[kCpw];
#pragma unroll
        for (int j = 0; j < kCpw; ++j) {
            const int c = c0 + j;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_global_load_lds((global_void *)(xsrc[i] + 128 * c),
                                                 (lds_void *)(region[j] + 64 * i), 16, 0, 0);
            codes[j] = load16_stream(wrow + 64 * c);
            const int g = (128 * c + 32 * q) / G;
            sv[j] = srow[g];
            zv[j] = zrow[g];
            __builtin_amdgcn_sched_barrier(0);  // chunk by chunk, in this order
        }
#pragma unroll
        for (int j = 0; j < kCpw; ++j) {
            if (j == 0) W4A16_WAIT_VM(kLoadsPerChunk * (kCpw - 1));
            else if (j == 1) W4A16_WAIT_VM(kLoadsPerChunk * (kCpw - 2));
            else if (j == 2) W4A16_WAIT_VM(kLoadsPerChunk * (kCpw - 3));
            else W4A16_WAIT_VM(0);
            asm volatile("" ::: "memory");
            // nothing of this chunk (the dequantization of its codes included)
            // moves above its wait, nor below the next chunk's
            __builtin_amdgcn_sched_barrier(0);
            const float s = h_to_float<F16>(sv[j]), z = h_to_float<F16>(zv[j]);
            const uint32_t cw[4] = {codes[j].x, codes[j].y, codes[j].z, codes[j].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint4 b = region[j][16 * r16 + ((4 * q + t) ^ r16)];
                acc = mfma16x16x32<F16>(dequant8<S4, F16>(cw[t], s, z), b, acc);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // every fragment of this block was read (the MFMAs consumed them)
        // before the next block's loads refill the region
    }

#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    // one output per thread: channel ch of row j sits in lane j + 16 * (ch / 4),
    // element ch % 4; the K-split partials add in fp32 in wavefront order
    if (threadIdx.x >= 256) return;
    const int j = threadIdx.x >> 4, ch = threadIdx.x & 15;
    if (j >= M) return;
    const int l = j + 16 * (ch >> 2), r = ch & 3;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kSplit; ++w) sum += red[w][r][l];
    out[(int64_t)j * N + n0 + ch] = (uint16_t)(pack_h2<F16>(sum, 0.0f) & 0xFFFFu);
}

template <int MT, bool S4, bool F16>
hipError_t launch_decode_mt(const uint16_t *x, int M, const uint8_t *wq4, const uint16_t *scales,
                            const uint16_t *zeros, int N, int K, int G, uint16_t *out,
                            hipStream_t stream) {
    const int chunks_per_wave = (K / 128 + kSplit - 1) / kSplit;
    w4a16_decode_kernel<MT, S4, F16><<<dim3((unsigned)(N / 16)), dim3(kSplit * kWave), 0, stream>>>(
        x, wq4, scales, zeros, out, M, N, K, G, chunks_per_wave);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LDS-tiled W4A16 GEMM for M > 64: BM x BN tile per workgroup of 8 wavefronts
// in two roles, K advancing 64 columns per stage. Wavefronts 0-3 (2 x 2 or
// 4 x 1 over the tile, v_mfma_f32_32x32x16_bf16, weights first) move the
// activations global -> LDS with direct-to-LDS 16-byte loads through a ring of
// 4 stages (issued 3 stages ahead) and run the MFMAs. Wavefronts 4-7 load the
// weight codes of a stage into registers 2 stages ahead and dequantize them
// once per workgroup into one of two bf16 weight buffers in LDS a stage before
// they are used (the dequant arithmetic per weight is shared by the tile's BM
// rows). Each SIMD holds one wavefront of each role, so one's MFMAs and the
// other's dequantization overlap; a single role doing both took about the sum
// of the two per stage. Rows of 64 bf16 are 128 bytes, chunk c of row r at
// slot c ^ (r % 8) ^ ((r / 8) % 2), as in the int8 kernel. Each role waits
// only for its own loads of the stage that must be complete (counted
// vector-memory waits, no fence), then both meet at the stage barrier: loads
// of later stages stay in flight across it. Both roles pass the same barriers
// (one after the prologue, one per stage, two at the end).
typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int BM, int BN, int WAVES_M, bool S4, bool F16>
__global__ __launch_bounds__(512, 1) void w4a16_tiled_kernel(
    const uint16_t *__restrict__ X, const uint8_t *__restrict__ wq4,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ out, int M, int N, int K, int G, int tiles_m, int tiles_n) {
    constexpr int WAVES_N = 4 / WAVES_M;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, TM = WM / 32, TN = WN / 32;
    constexpr int XS = BM * 8, WS = BN * 8;                    // 16-byte slots per buffer
    constexpr int XBUF = 4, WBUF = 2;
    constexpr int XLD = XS / 256;                              // activation loads per wavefront
    constexpr int CODES = BN * 64 / 256;                       // weight codes per thread per stage
    constexpr int NC = 3;                                      // code loads per stage: codes, scale, zero
    // a thread's codes lie in one group: CODES consecutive columns starting at a
    // multiple of CODES, and G is a multiple of 32
    static_assert(CODES == 32 || CODES == 16, "16 or 8 bytes of codes per thread");
    static_assert(WM * WN * 2 * 4 <= (XBUF * XS + WBUF * WS) * 16, "bf16 tile fits in LDS");
    static_assert(TM >= 1 && TN >= 1 && 2 * XLD < 64, "wavefront tiles and the vmcnt range");
    __shared__ uint4 lds[XBUF * XS + WBUF * WS];
    w8a8::lds_poison(lds);
    w8a8::lds_poison_done();

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    // mwave: the wavefront's place among the four that multiply; ct: the
    // thread's place among the 256 that dequantize
    const int wave = tid / kWave, mwave = wave & 3, ct = tid & 255;
    const bool math = wave < 4;  // uniform per wavefront
    const int wm = mwave / WAVES_N, wn = mwave % WAVES_N;
    const int tiles = tiles_m * tiles_n;
    const int t = w8a8::xcd_contiguous(blockIdx.x, tiles);
    constexpr int kGroup = 4;
    const int per_group = kGroup * tiles_n;
    const int first_m = (t / per_group) * kGroup;
    const int gsize = min(tiles_m - first_m, kGroup);
    const int m0 = (first_m + (t % per_group) % gsize) * BM;
    const int n0 = ((t % per_group) / gsize) * BN;
    const int nk = K / 64;
    const int last = nk - 1;
    auto xbuf = [&](int j) { return lds + (j % XBUF) * XS; };
    auto wbuf = [&](int j) { return lds + XBUF * XS + (j % WBUF) * WS; };

    // The loops are straight-line: stages past the last are loaded from the
    // last stage (in bounds) into buffers that are never read again, and the
    // last dequantization writes a weight buffer last read two stages earlier.
    // So every wait is for a fixed count (the loads of the 2 stages issued
    // after the one that must be complete).
    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};
    if (math) {
        // activation loads: load l of this wavefront fills slots 64 (mwave + 4 l) ..
        const uint16_t *xsrc[XLD];
        {
            const int row = 8 * mwave + (lane >> 3);
            const int kc = (lane & 7) ^ swz(row);
#pragma unroll
            for (int l = 0; l < XLD; ++l)
                xsrc[l] = X + (int64_t)min(m0 + row + 32 * l, M - 1) * K + 8 * kc;
        }
        auto load_x = [&](int j, uint4 *__restrict__ buf) {
#pragma unroll
            for (int l = 0; l < XLD; ++l)
                __builtin_amdgcn_global_load_lds((global_void *)(xsrc[l] + 64 * j),
                                                 (lds_void *)(buf + 64 * (mwave + 4 * l)), 16, 0, 0);
        };
        const int frag_row = lane & 31, kh = lane >> 5;
        const int fswz = swz(frag_row);
        // the MFMAs of a stage; the fragment reads of step u + 1 go out right
        // after the first MFMA of step u (two fragment sets), so they overlap
        // that step's other MFMAs
        auto compute = [&](const uint4 *__restrict__ xb, const uint4 *__restrict__ wb) {
            uint4 xa[2][TM], wf[2][TN];
            auto read = [&](int u, uint4 (&xr)[TM], uint4 (&wr)[TN]) {
                const int c = (2 * u + kh) ^ fswz;
#pragma unroll
                for (int i = 0; i < TM; ++i) xr[i] = xb[(wm * WM + 32 * i + frag_row) * 8 + c];
#pragma unroll
                for (int q = 0; q < TN; ++q) wr[q] = wb[(wn * WN + 32 * q + frag_row) * 8 + c];
            };
            auto mma = [&](int u, int i, int q) {
                acc[i][q] = F16 ? __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                      __builtin_bit_cast(v8h, wf[u & 1][q]),
                                      __builtin_bit_cast(v8h, xa[u & 1][i]), acc[i][q], 0, 0, 0)
                                : __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                      __builtin_bit_cast(v8bf, wf[u & 1][q]),
                                      __builtin_bit_cast(v8bf, xa[u & 1][i]), acc[i][q], 0, 0, 0);
            };
            read(0, xa[0], wf[0]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                __builtin_amdgcn_sched_barrier(0);
                mma(u, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (u < 3) read(u + 1, xa[(u + 1) & 1], wf[(u + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int q = 0; q < TN; ++q)
                        if (i + q > 0) mma(u, i, q);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        // activations of stages 0..2 in flight; at each barrier the stage to
        // be read next has landed (this wavefront's loads) and been
        // dequantized (the other role's stores). The buffers a step touches
        // are distinct, and the restrict qualifiers say so (after inlining the
        // accesses carry alias scopes, so the fragment reads need not wait for
        // the direct-to-LDS loads landing in another buffer).
        load_x(0, xbuf(0));
        __builtin_amdgcn_sched_barrier(0);
        load_x(min(1, last), xbuf(1));
        __builtin_amdgcn_sched_barrier(0);
        load_x(min(2, last), xbuf(2));
        __builtin_amdgcn_sched_barrier(0);
        w8a8::vm_barrier<2 * XLD>();
        auto step = [&](int s, uint4 *__restrict__ xnew, const uint4 *__restrict__ xcur,
                        const uint4 *__restrict__ wcur) {
            load_x(min(s + 3, last), xnew);
            __builtin_amdgcn_sched_barrier(0);
            compute(xcur, wcur);
            w8a8::vm_barrier<2 * XLD>();
        };
        int s = 0;
        for (; s + 4 <= nk; s += 4) {
            step(s, xbuf(s + 3), xbuf(s), wbuf(s));
            step(s + 1, xbuf(s + 4), xbuf(s + 1), wbuf(s + 1));
            step(s + 2, xbuf(s + 5), xbuf(s + 2), wbuf(s + 2));
            step(s + 3, xbuf(s + 6), xbuf(s + 3), wbuf(s + 3));
        }
        for (; s < nk; ++s) step(s, xbuf(s + 3), xbuf(s), wbuf(s));
    } else {
        // weight codes: thread ct dequantizes columns [CODES * part, +CODES)
        // of tile row wr
        constexpr int PARTS = 64 / CODES;
        const int wr = ct / PARTS, part = ct % PARTS;
        const int64_t wn_row = min(n0 + wr, N - 1);
        const uint8_t *wsrc = wq4 + wn_row * (K / 2) + part * (CODES / 2);
        const uint16_t *ssrc = scales + wn_row * (K / G), *zsrc = zeros + wn_row * (K / G);
        struct Codes {
            uint32_t c[CODES / 8];
            uint16_t s, z;
        };
        auto load_codes = [&](int j, Codes &c) {
            const uint8_t *src = wsrc + 32 * j;
            if constexpr (CODES == 32) {
                const uint4 v = *reinterpret_cast<const uint4 *>(src);
                c.c[0] = v.x; c.c[1] = v.y; c.c[2] = v.z; c.c[3] = v.w;
            } else {
                const uint2 v = *reinterpret_cast<const uint2 *>(src);
                c.c[0] = v.x; c.c[1] = v.y;
            }
            const int g = (64 * j + part * CODES) / G;
            c.s = ssrc[g];
            c.z = zsrc[g];
        };
        auto dequant_into = [&](const Codes &c, uint4 *__restrict__ wb) {
            const float sf = h_to_float<F16>(c.s), zf = h_to_float<F16>(c.z);
#pragma unroll
            for (int i = 0; i < CODES / 8; ++i)
                wb[wr * 8 + ((part * (CODES / 8) + i) ^ swz(wr))] = dequant8<S4, F16>(c.c[i], sf, zf);
        };
        // codes of stages 0..2 in flight, stage 0 dequantized; iteration s
        // loads stage s + 3 into the set that held stage s (dequantized an
        // iteration earlier) and dequantizes stage s + 1 into the weight
        // buffer last read two stages earlier. Stage j's codes live in set
        // j % 3; unrolling by 3 keeps that rotation free of register copies (a
        // copy would wait for the load).
        Codes c0, c1, c2;
        load_codes(0, c0);
        __builtin_amdgcn_sched_barrier(0);
        load_codes(min(1, last), c1);
        __builtin_amdgcn_sched_barrier(0);
        load_codes(min(2, last), c2);
        __builtin_amdgcn_sched_barrier(0);
        W4A16_WAIT_VM(2 * NC);
        __builtin_amdgcn_sched_barrier(0);
        dequant_into(c0, wbuf(0));
        w8a8::vm_barrier<2 * NC>();
        auto step = [&](int s, Codes &into, const Codes &deq, uint4 *__restrict__ wnext) {
            load_codes(min(s + 3, last), into);
            __builtin_amdgcn_sched_barrier(0);
            // stage s + 1 has landed once at most the loads of stages s + 2
            // and s + 3 are outstanding; no use of it moves above the wait
            W4A16_WAIT_VM(2 * NC);
            __builtin_amdgcn_sched_barrier(0);
            dequant_into(deq, wnext);
            w8a8::vm_barrier<2 * NC>();
        };
        int s = 0;
        for (; s + 3 <= nk; s += 3) {
            step(s, c0, c1, wbuf(s + 1));
            step(s + 1, c1, c2, wbuf(s + 2));
            step(s + 2, c2, c0, wbuf(s + 3));
        }
        if (s < nk) { step(s, c0, c1, wbuf(s + 1)); ++s; }
        if (s < nk) { step(s, c1, c2, wbuf(s + 1)); ++s; }
    }
    // no load may still be landing in LDS when the epilogue reuses it
    w8a8::vm_barrier<0>();

    // epilogue (the multiplying wavefronts): tile (i, j), element r of a lane:
    // activation row i*32 + lane%32 of the wavefront's sub-tile, channel
    // j*32 + 8*(r/4) + 4*kh + r%4; the wavefront's WM x WN bf16 sub-tile is
    // staged in LDS (16-byte chunks of a row permuted by the row), then stored
    // as whole 16-byte row pieces
    constexpr int CH = WN / 8, PM = CH < 8 ? CH - 1 : 7;
    uint2 *st8 = reinterpret_cast<uint2 *>(lds) + mwave * (WM * WN / 4);
    const int frag_row = lane & 31, kh = lane >> 5;
    if (math) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int ml = i * 32 + frag_row;
                    const v16f &a = acc[i][j];
                    const uint32_t lo = pack_h2<F16>(a[4 * g], a[4 * g + 1]);
                    const uint32_t hi = pack_h2<F16>(a[4 * g + 2], a[4 * g + 3]);
                    st8[(ml * CH + ((j * 4 + g) ^ (ml & PM))) * 2 + kh] = make_uint2(lo, hi);
                }
    }
    __syncthreads();
    if (!math) return;
    const int mw0 = m0 + wm * WM, nw0 = n0 + wn * WN;
    const uint4 *st16 = reinterpret_cast<const uint4 *>(st8);
#pragma unroll
    for (int it = 0; it < WM * CH / kWave; ++it) {
        const int q = it * kWave + lane;
        const int ml = q / CH, cc = q % CH;
        const int m = mw0 + ml, n = nw0 + cc * 8;
        if (m < M && n < N)
            w8a8::store16_nt(out + (int64_t)m * N + n, st16[ml * CH + (cc ^ (ml & PM))]);
    }
}

template <int BM, int BN, int WAVES_M, bool S4, bool F16>
hipError_t launch_tiled(const uint16_t *x, int M, const uint8_t *wq4, const uint16_t *scales,
                        const uint16_t *zeros, int N, int K, int G, uint16_t *out,
                        hipStream_t stream) {
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    w4a16_tiled_kernel<BM, BN, WAVES_M, S4, F16>
        <<<dim3((unsigned)(tiles_m * tiles_n)), dim3(512), 0, stream>>>(
        x, wq4, scales, zeros, out, M, N, K, G, tiles_m, tiles_n);
    return hipGetLastError();
}

template <bool S4, bool F16>
hipError_t launch_dequant_codes(const uint8_t *wq4, const uint16_t *scales, const uint16_t *zeros,
                                int N, int K, int G, uint16_t *w, hipStream_t stream) {
    const int64_t words = (int64_t)N * K / 8;
    dequant_kernel<S4, F16><<<dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream>>>(
        reinterpret_cast<const uint32_t *>(wq4), scales, zeros, words, K, G,
        reinterpret_cast<uint4 *>(w));
    return hipGetLastError();
}

template <bool S4, bool F16>
hipError_t launch_gemm_codes(const uint16_t *x, int M, const uint8_t *wq4, const uint16_t *scales,
                             const uint16_t *zeros, int N, int K, int G, uint16_t *out,
                             hipStream_t stream) {
    if (M <= 16 && K % 4096 == 0) {
        w4a16_decode_lds_kernel<S4, F16><<<dim3((unsigned)(N / 16)), dim3(kSplit * kWave), 0, stream>>>(
            x, wq4, scales, zeros, out, M, N, K, G);
        return hipGetLastError();
    }
    switch ((M + 15) / 16) {
        case 1: return launch_decode_mt<1, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        case 2: return launch_decode_mt<2, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        case 3: return launch_decode_mt<3, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        case 4: return launch_decode_mt<4, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        default: break;
    }
    // The largest tile that still gives every CU a workgroup: a tile's time is
    // set by its K loop (its activation stream and stage barriers), so larger
    // tiles share it over more outputs but leave CUs idle below 256 tiles
    // (N = K = 4096: M = 2048 256 x 128, 80 us; M = 1024 256 x 64, 50 us;
    // M = 512 128 x 64, 32 us; M = 128 and 256 64 x 64, 26-27 us). Taller
    // tiles first: a column more costs every row tile a dequantization.
    auto tiles = [&](long bm, long bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    const long fill = w8a8::device_cu_count();
    if (tiles(256, 128) >= fill)
        return launch_tiled<256, 128, 2, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
    if (tiles(256, 64) >= fill)
        return launch_tiled<256, 64, 4, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
    if (tiles(128, 64) >= fill)
        return launch_tiled<128, 64, 4, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
    return launch_tiled<64, 64, 2, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
}

}  // namespace

hipError_t launch_dequant(const uint8_t *wq4, const uint16_t *scales, const uint16_t *zeros, int N,
                          int K, int G, bool s4, bool f16, uint16_t *w, hipStream_t stream) {
    if (f16)
        return s4 ? launch_dequant_codes<true, true>(wq4, scales, zeros, N, K, G, w, stream)
                  : launch_dequant_codes<false, true>(wq4, scales, zeros, N, K, G, w, stream);
    return s4 ? launch_dequant_codes<true, false>(wq4, scales, zeros, N, K, G, w, stream)
              : launch_dequant_codes<false, false>(wq4, scales, zeros, N, K, G, w, stream);
}

hipError_t launch_gemm(const uint16_t *x, int M, const uint8_t *wq4, const uint16_t *scales,
                       const uint16_t *zeros, int N, int K, int G, bool s4, bool f16,
                       uint16_t *out, hipStream_t stream) {
    if (f16)
        return s4 ? launch_gemm_codes<true, true>(x, M, wq4, scales, zeros, N, K, G, out, stream)
                  : launch_gemm_codes<false, true>(x, M, wq4, scales, zeros, N, K, G, out, stream);
    return s4 ? launch_gemm_codes<true, false>(x, M, wq4, scales, zeros, N, K, G, out, stream)
              : launch_gemm_codes<false, false>(x, M, wq4, scales, zeros, N, K, G, out, stream);
}

}  // namespace w4a16
