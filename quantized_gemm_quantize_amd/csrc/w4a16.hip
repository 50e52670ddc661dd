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
// LDS-tiled W4A16 GEMM for M > 64: BM x BN tile per workgroup of 4 wavefronts
// (2 x 2, v_mfma_f32_32x32x16_bf16, weights first), K advancing 64 columns
// per stage. Activations move global -> LDS with direct-to-LDS 16-byte loads
// through a ring of 4 stages (issued 3 stages ahead); the weight codes of a
// stage are loaded into registers 2 stages ahead, dequantized once per
// workgroup into one of two bf16 weight buffers in LDS a stage before they
// are used, and read there by every wavefront of the tile (the dequant
// arithmetic per weight is shared by the tile's BM rows). The dequantization
// of stage s + 1 is interleaved with the MFMAs of stage s, so the vector ALU
// and the matrix cores work at once. Rows of 64 bf16 are 128 bytes, chunk c of
// row r at slot c ^ (r % 8) ^ ((r / 8) % 2), as in the int8 kernel. Barriers
// wait only for the stage that must be complete (counted vector-memory waits,
// no fence): loads of later stages stay in flight across them.
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <int BM, int BN, int WAVES_M, bool S4, bool F16>
__global__ __launch_bounds__(256, 1) void w4a16_tiled_kernel(
    const uint16_t *__restrict__ X, const uint8_t *__restrict__ wq4,
    const uint16_t *__restrict__ scales, const uint16_t *__restrict__ zeros,
    uint16_t *__restrict__ out, int M, int N, int K, int G, int tiles_m, int tiles_n) {
    constexpr int WAVES_N = 4 / WAVES_M;
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N, TM = WM / 32, TN = WN / 32;
    constexpr int XS = BM * 8, WS = BN * 8;                    // 16-byte slots per buffer
    constexpr int XBUF = 4, WBUF = 2;
    constexpr int XLD = XS / 256;                              // activation loads per wavefront
    constexpr int CODES = BN * 64 / 256;                       // weight codes per thread per stage
    constexpr int CLD = CODES == 64 ? 2 : 1;                   // 16-byte code loads (or one 8-byte)
    constexpr int NLD = XLD + CLD + 2;                         // + codes, scale, zero
    static_assert(CODES == 64 || CODES == 32 || CODES == 16, "32, 16 or 8 bytes of codes per thread");
    static_assert(WM * WN * 2 * 4 <= (XBUF * XS + WBUF * WS) * 16, "bf16 tile fits in LDS");
    static_assert(TM >= 1 && TN >= 1 && 2 * NLD < 64, "wavefront tiles and the vmcnt range");
    __shared__ uint4 lds[XBUF * XS + WBUF * WS];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int tiles = tiles_m * tiles_n;
    const int t = w8a8::xcd_contiguous(blockIdx.x, tiles);
    constexpr int kGroup = 4;
    const int per_group = kGroup * tiles_n;
    const int first_m = (t / per_group) * kGroup;
    const int gsize = min(tiles_m - first_m, kGroup);
    const int m0 = (first_m + (t % per_group) % gsize) * BM;
    const int n0 = ((t % per_group) / gsize) * BN;
    const int nk = K / 64;

    // activation loads: load l of this wavefront fills slots 64 (wave + 4 l) ..
    const uint16_t *xsrc[XLD];
    {
        const int row = 8 * wave + (lane >> 3);
        const int kc = (lane & 7) ^ swz(row);
#pragma unroll
        for (int l = 0; l < XLD; ++l) xsrc[l] = X + (int64_t)min(m0 + row + 32 * l, M - 1) * K + 8 * kc;
    }
    // weight codes: thread tid dequantizes columns [CODES * part, +CODES) of tile row wr
    constexpr int PARTS = 64 / CODES;
    const int wr = tid / PARTS, part = tid % PARTS;
    const int64_t wn_row = min(n0 + wr, N - 1);
    const uint8_t *wsrc = wq4 + wn_row * (K / 2) + part * (CODES / 2);
    const uint16_t *ssrc = scales + wn_row * (K / G), *zsrc = zeros + wn_row * (K / G);

    struct Codes {
        uint32_t c[CODES / 8];
        uint16_t s, z;
    };
    auto load_codes = [&](int j, Codes &c) {
        const uint8_t *src = wsrc + 32 * j;
        if constexpr (CODES == 64) {
            const uint4 v = *reinterpret_cast<const uint4 *>(src);
            const uint4 u = *reinterpret_cast<const uint4 *>(src + 16);
            c.c[0] = v.x; c.c[1] = v.y; c.c[2] = v.z; c.c[3] = v.w;
            c.c[4] = u.x; c.c[5] = u.y; c.c[6] = u.z; c.c[7] = u.w;
        } else if constexpr (CODES == 32) {
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
    auto xbuf = [&](int j) { return lds + (j % XBUF) * XS; };
    auto wbuf = [&](int j) { return lds + XBUF * XS + (j % WBUF) * WS; };
    // word i of a thread's codes, dequantized into its weight buffer slot
    auto store_word = [&](const Codes &c, int i, uint4 *__restrict__ wb) {
        wb[wr * 8 + ((part * (CODES / 8) + i) ^ swz(wr))] =
            dequant8<S4, F16>(c.c[i], h_to_float<F16>(c.s), h_to_float<F16>(c.z));
    };
    auto load_x = [&](int j, uint4 *__restrict__ buf) {
#pragma unroll
        for (int l = 0; l < XLD; ++l)
            __builtin_amdgcn_global_load_lds((global_void *)(xsrc[l] + 64 * j),
                                             (lds_void *)(buf + 64 * (wave + 4 * l)), 16, 0, 0);
    };

    const int frag_row = lane & 31, kh = lane >> 5;
    const int fswz = swz(frag_row);
    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v16f{};
    // the MFMAs on buffers xb, wb, with the dequantization of `next` into weight
    // buffer `nb` interleaved between the 4 K steps
    auto compute = [&](const uint4 *__restrict__ xb, const uint4 *__restrict__ wb,
                       const Codes &next, uint4 *__restrict__ nb) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int c = (2 * u + kh) ^ fswz;
            uint4 xa[TM], wf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                xa[i] = xb[(wm * WM + 32 * i + frag_row) * 8 + c];
#pragma unroll
            for (int q = 0; q < TN; ++q)
                wf[q] = wb[(wn * WN + 32 * q + frag_row) * 8 + c];
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int q = 0; q < TN; ++q)
                    acc[i][q] = F16 ? __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                          __builtin_bit_cast(v8h, wf[q]), __builtin_bit_cast(v8h, xa[i]),
                                          acc[i][q], 0, 0, 0)
                                    : __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                          __builtin_bit_cast(v8bf, wf[q]), __builtin_bit_cast(v8bf, xa[i]),
                                          acc[i][q], 0, 0, 0);
            // this step's share of the code words (one or two; none in the
            // last steps when there are only two)
            constexpr int WPS = CODES / 8 > 4 ? CODES / 32 : 1;
#pragma unroll
            for (int i = 0; i < WPS; ++i)
                if (u * WPS + i < CODES / 8) store_word(next, u * WPS + i, nb);
        }
    };

    // The loop body is straight-line: stages past the last are loaded from the
    // last stage (in bounds) into buffers that are never read again, and the
    // last dequantization writes a weight buffer last read two stages earlier.
    // So every barrier waits for a fixed count (the loads of the 2 stages issued
    // after the one that must be complete) and the compiler's own waits before
    // the dequantization are exact.
    const int last = nk - 1;
    // prologue: activations and codes of stages 0..2 in flight, stage 0
    // dequantized; then stage 0 landed everywhere
    Codes c0, c1, c2;
    load_x(0, xbuf(0));
    __builtin_amdgcn_sched_barrier(0);
    load_codes(0, c0);
    __builtin_amdgcn_sched_barrier(0);
    load_x(min(1, last), xbuf(1));
    __builtin_amdgcn_sched_barrier(0);
    load_codes(min(1, last), c1);
    __builtin_amdgcn_sched_barrier(0);
    load_x(min(2, last), xbuf(2));
    __builtin_amdgcn_sched_barrier(0);
    load_codes(min(2, last), c2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < CODES / 8; ++i) store_word(c0, i, wbuf(0));
    w8a8::vm_barrier<2 * NLD>();
    // iteration s: issue stage s+3 (activations, codes into the registers that
    // held stage s's codes, dequantized an iteration earlier), compute stage s
    // while dequantizing stage s+1 (loaded two iterations earlier), then wait
    // for stage s+1. Stage j's codes live in set j % 3; unrolling by 3 keeps
    // that rotation free of register copies (a copy would wait for the load).
    // The four buffers an iteration touches are distinct, and the restrict
    // qualifiers say so: after inlining the accesses carry alias scopes, so the
    // weight-buffer stores need not wait for the activation loads still landing
    // in another buffer.
    auto iteration = [&](int s, Codes &into, const Codes &deq, uint4 *__restrict__ xnew,
                         const uint4 *__restrict__ xcur, const uint4 *__restrict__ wcur,
                         uint4 *__restrict__ wnext) {
        load_x(min(s + 3, last), xnew);
        __builtin_amdgcn_sched_barrier(0);
        load_codes(min(s + 3, last), into);
        __builtin_amdgcn_sched_barrier(0);
        // Stage s+1, whose codes compute() dequantizes, has landed once at most
        // the loads of stages s+2 and s+3 are outstanding. Said explicitly:
        // the compiler's own wait analysis loses count of one code set across
        // the unrolled loop and would otherwise drain every load in flight.
        W4A16_WAIT_VM(2 * NLD);
        __builtin_amdgcn_sched_barrier(0);  // no use of a loaded value moves above the wait
        compute(xcur, wcur, deq, wnext);
        w8a8::vm_barrier<2 * NLD>();
    };
#define W4A16_ITER(S, INTO, DEQ) \
    iteration(S, INTO, DEQ, xbuf((S) + 3), xbuf(S), wbuf(S), wbuf((S) + 1))
    int s = 0;
    for (; s + 3 <= nk; s += 3) {
        W4A16_ITER(s, c0, c1);
        W4A16_ITER(s + 1, c1, c2);
        W4A16_ITER(s + 2, c2, c0);
    }
    if (s < nk) { W4A16_ITER(s, c0, c1); ++s; }
    if (s < nk) { W4A16_ITER(s, c1, c2); ++s; }
#undef W4A16_ITER
    // no load may still be landing in LDS when the epilogue reuses it
    w8a8::vm_barrier<0>();

    // epilogue: tile (i, j), element r of a lane: activation row i*32 + lane%32
    // of the wavefront's sub-tile, channel j*32 + 8*(r/4) + 4*kh + r%4; the
    // wavefront's WM x WN bf16 sub-tile is staged in LDS (16-byte chunks of a
    // row permuted by the row), then stored as whole 16-byte row pieces
    constexpr int CH = WN / 8, PM = CH < 8 ? CH - 1 : 7;
    uint2 *st8 = reinterpret_cast<uint2 *>(lds) + wave * (WM * WN / 4);
    const int mw0 = m0 + wm * WM, nw0 = n0 + wn * WN;
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
    __syncthreads();
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
    w4a16_tiled_kernel<BM, BN, WAVES_M, S4, F16><<<dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, stream>>>(
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
    switch ((M + 15) / 16) {
        case 1: return launch_decode_mt<1, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        case 2: return launch_decode_mt<2, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        case 3: return launch_decode_mt<3, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        case 4: return launch_decode_mt<4, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
        default: break;
    }
    // 256 x 64 tiles (4 wavefronts along M: half the dequantization per output
    // of 128 x 128, measured faster at M = 1024) when they fill the chip, then
    // 128 x 64 (also 4 wavefronts along M), else 64 x 64
    const long t256 = (long)((M + 255) / 256) * ((N + 63) / 64);
    const long t128 = (long)((M + 127) / 128) * ((N + 63) / 64);
    if (t256 >= 256) return launch_tiled<256, 64, 4, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
    if (t128 >= 256) return launch_tiled<128, 64, 4, S4, F16>(x, M, wq4, scales, zeros, N, K, G, out, stream);
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
