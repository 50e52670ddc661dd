// 2:4 semi-structured int8 weights on gfx950's sparse MFMA.
//
// In every group of 4 consecutive weights along K at most two are nonzero (the
// pages' cuSPARSELt route: Paddle sparse_fc PR #41770 runs FC weights already
// pruned to 2:4; pytorch/ao PR #821 composes that path with int8 dynamic
// quantization and asks for i8i8 -> bf16 output so the int32 product is never
// materialized). The sparse MFMA multiplies a 2:4 operand stored compressed --
// two values and two 2-bit positions per group -- at twice the dense rate.
//
// Storage (the library's own, see include/w8a8.h): per weight row and 64-column
// step the 16 groups are listed in the order 0-3, 8-11, 4-7, 12-15; values hold
// the two kept weights of each listed group (lower position first), meta one
// nibble p0 | p1 << 2 per listed group, eight per 32-bit word. That order is
// the sparse operand's lane layout: for v_smfmac_i32_32x32x64_i8, lane half h
// of weight row n takes the 16 value bytes and the index word of list half h
// of the step (groups 4h..4h+3 and 8+4h..8+4h+3), against activation bytes
// [32h, 32h+32) of the step in the other operand; v_smfmac_i32_16x16x128_i8
// takes, in lane quarter q, list half q / 2 of 64-column step q % 2 against
// activation bytes [32q, 32q+32) of its 128 columns. So every operand fragment
// is one contiguous 16-byte load plus one 32-bit index. The arrays are
// K-block-major ([K/128][N][64] values, [K/128][N][4] index words): the
// pieces of one 128-column block for consecutive rows are contiguous, so a
// tile of rows loads whole cache lines (per row and block there are only 64
// value bytes and 16 index bytes).
#include "common.hpp"
#include "launch.hpp"

namespace w8a8 {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));

// s_waitcnt on the vector-memory counter only
template <int N>
__device__ __forceinline__ void wait_vm_s24() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ v4i smfmac_16x16x128(v4i a, v8i b, v4i c, int idx) {
    return __builtin_amdgcn_smfmac_i32_16x16x128_i8(a, b, c, idx, 0, 0);
}

__device__ __forceinline__ int mag(int v) { return v < 0 ? -v : v; }

// The group's kept positions p0 < p1 as the nibble p0 | p1 << 2, and its kept
// values (lower position first) packed in the low 16 bits: the two largest
// |w|, equal magnitudes in position order.
__device__ __forceinline__ void keep_two(uint32_t grp, uint32_t &nib, uint32_t &vals) {
    int w[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) w[p] = (int)(int8_t)(grp >> (8 * p));
    int first = 0;
#pragma unroll
    for (int p = 1; p < 4; ++p)
        if (mag(w[p]) > mag(w[first])) first = p;
    int second = first == 0 ? 1 : 0;
#pragma unroll
    for (int p = 0; p < 4; ++p)
        if (p != first && p > second && mag(w[p]) > mag(w[second])) second = p;
    const int p0 = min(first, second), p1 = max(first, second);
    nib = (uint32_t)(p0 | (p1 << 2));
    vals = ((uint32_t)w[p0] & 0xFFu) | (((uint32_t)w[p1] & 0xFFu) << 8);
}

// One thread per (128-column block, row, 64-column step, list half), in
// storage order: reads the 32 weights of its 8 groups (columns [16h, 16h+16)
// and [32+16h, 32+16h+16) of the step), writes 16 value bytes and one index
// word.
__global__ __launch_bounds__(256) void compress24_kernel(const int8_t *__restrict__ w,
                                                          int64_t chunks, int N, int K,
                                                          int8_t *__restrict__ values,
                                                          uint32_t *__restrict__ meta) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= chunks) return;
    const int h = (int)(t & 1), sub = (int)((t >> 1) & 1);
    const int64_t bn = t >> 2;                 // block * N + row
    const int64_t n = bn % N, blk = bn / N;
    const int8_t *row = w + n * K + 128 * blk + 64 * sub + 16 * h;
    const uint4 lo = *reinterpret_cast<const uint4 *>(row);        // groups 4h .. 4h+3
    const uint4 hi = *reinterpret_cast<const uint4 *>(row + 32);   // groups 8+4h .. 8+4h+3
    const uint32_t grp[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t word = 0, v[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t nib, vals;
        keep_two(grp[i], nib, vals);
        word |= nib << (4 * i);
        v[i >> 1] |= vals << (16 * (i & 1));
    }
    reinterpret_cast<uint4 *>(values)[t] = make_uint4(v[0], v[1], v[2], v[3]);
    meta[t] = word;
}

// Weight-streaming 2:4 GEMM for M <= 64: the shape of the dense M-small kernel
// (one workgroup per 16 output channels, K split over 8 wavefronts, partials
// summed in LDS, fused epilogue), with v_smfmac_i32_16x16x128_i8 taking the
// compressed weights as its sparse operand: half the weight bytes of the dense
// kernel per output. The weight operand comes first, so lane l ends with
// output channels 4 (l / 16) .. +3 of activation row l % 16.
constexpr int kSplit = 8;
constexpr int kUnroll = 4;   // 128-column steps whose loads are issued together

template <int MT, bool OUT_I32>
__global__ __launch_bounds__(kSplit *kWave) void sparse24_decode_kernel(
    const int8_t *__restrict__ X, const float *__restrict__ sx, const int8_t *__restrict__ V,
    const uint32_t *__restrict__ Meta, const float *__restrict__ sw, void *__restrict__ out,
    int M, int N, int K, int steps_per_wave) {
    __shared__ int red[kSplit][MT][4][kWave];
    lds_poison(red);
    lds_poison_done();

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int n0 = blockIdx.x * 16;
    const int r16 = lane & 15, q = lane >> 4;
    // lane quarter q = 2 * half + sub takes list half `half` of 64-column step
    // `sub` of each 128-column block: 16 value bytes at 32 * sub + 16 * half
    // of the row's 64, index word 2 * sub + half of its 4
    const int half = q >> 1, sub = q & 1;
    const int nblk = K / 128;
    const int8_t *vrow = V + (int64_t)(n0 + r16) * 64 + 32 * sub + 16 * half;
    const uint32_t *mrow = Meta + (int64_t)(n0 + r16) * 4 + 2 * sub + half;
    const int64_t vstride = (int64_t)N * 64, mstride = (int64_t)N * 4;   // per block
    const int8_t *xrow[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) xrow[mb] = X + (int64_t)min(mb * 16 + r16, M - 1) * K;

    const int s_begin = wave * steps_per_wave;
    const int s_end = min(s_begin + steps_per_wave, nblk);

    v4i acc[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) acc[mb] = v4i{};
    // Loads past the wavefront's blocks read block nblk - 1 (in bounds) and
    // are masked: a zero weight operand cancels whatever activation bytes
    // its partner lanes hold, so only the weight side needs the mask.
    for (int s = s_begin; s < s_end; s += kUnroll) {
        v4i a[kUnroll];
        int idx[kUnroll];
        v8i b[MT][kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int blk = min(s + u, nblk - 1);
            const v4i av = __builtin_bit_cast(v4i, load16_stream(vrow + blk * vstride));
            a[u] = s + u < s_end ? av : v4i{};
            idx[u] = (int)mrow[blk * mstride];
#pragma unroll
            for (int mb = 0; mb < MT; ++mb)
                b[mb][u] = *reinterpret_cast<const v8i *>(xrow[mb] + 128 * blk + 32 * q);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int mb = 0; mb < MT; ++mb) acc[mb] = smfmac_16x16x128(a[u], b[mb][u], acc[mb], idx[u]);
    }

#pragma unroll
    for (int mb = 0; mb < MT; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][mb][r][lane] = acc[mb][r];
    __syncthreads();

    // one output per thread: channel c (0..15) of row j of row block mb sits in
    // lane j + 16 * (c / 4), element c % 4
    for (int e = threadIdx.x; e < MT * 256; e += kSplit * kWave) {
        const int mb = e >> 8, j = (e >> 4) & 15, c = e & 15;
        const int m = mb * 16 + j;
        if (m >= M) continue;
        const int l = j + 16 * (c >> 2), r = c & 3;
        int sum = 0;
#pragma unroll
        for (int w = 0; w < kSplit; ++w) sum += red[w][mb][r][l];
        const int n = n0 + c;
        if constexpr (OUT_I32)
            static_cast<int32_t *>(out)[(int64_t)m * N + n] = sum;
        else
            static_cast<__bf16 *>(out)[(int64_t)m * N + n] =
                (__bf16)dequant(sum, split_scale(sx[m]), split_scale(sw[n]));
    }
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// The same for M <= 16 and K >= 4096, with the activations moved
// global -> LDS. Each workgroup reads all 16 x K activation bytes, twice the
// bytes of its compressed weights; loaded straight into the operand layout
// (32 bytes per lane, 16 rows x 4 pieces per instruction) each load touched
// 16 half-used lines. Here one direct-to-LDS instruction fills 64 slots with 8
// rows x 128 bytes of a block (8 whole lines); slot p of a row holds its
// 16-byte piece p ^ (row / 2), so the two fragment reads of the 16 lanes of a
// quarter (rows 0..15, one piece each) hit 16 distinct bank groups. Wavefront
// w takes blocks 4w .. 4w+3 of every 4096-column K block and issues all their
// loads at once (activations, values, index word per block), each block
// multiplied after its own wait; one LDS array per block position, so the
// compiler's waits match these (see the dense M-small kernel). Rows past M
// are read from row M - 1 and never stored; blocks past K (a ragged last K
// block) load the last block again and multiply zero values.
template <bool OUT_I32>
__global__ __launch_bounds__(kSplit *kWave) void sparse24_decode_lds_kernel(
    const int8_t *__restrict__ X, const float *__restrict__ sx, const int8_t *__restrict__ V,
    const uint32_t *__restrict__ Meta, const float *__restrict__ sw, void *__restrict__ out,
    int M, int N, int K) {
    constexpr int kBpw = 4;                        // blocks per wavefront per K block
    constexpr int kKBlock = kSplit * kBpw * 128;   // 4096 columns
    constexpr int kBlockSlots = 16 * 8;            // 16 rows x 128 bytes
    constexpr int kLoadsPerBlock = 4;              // 2 activation loads, values, index word
    __shared__ uint4 b0[kSplit * kBlockSlots], b1[kSplit * kBlockSlots], b2[kSplit * kBlockSlots],
        b3[kSplit * kBlockSlots];
    __shared__ int red[kSplit][4][kWave];
    lds_poison(b0);
    lds_poison(b1);
    lds_poison(b2);
    lds_poison(b3);
    lds_poison(red);
    lds_poison_done();

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int n0 = blockIdx.x * 16;
    const int r16 = lane & 15, q = lane >> 4;
    const int half = q >> 1, sub = q & 1;
    const int8_t *vrow = V + (int64_t)(n0 + r16) * 64 + 32 * sub + 16 * half;
    const uint32_t *mrow = Meta + (int64_t)(n0 + r16) * 4 + 2 * sub + half;
    const int64_t vstride = (int64_t)N * 64, mstride = (int64_t)N * 4;   // per block
    // activation load h of a block: row 8 h + lane / 8, slot lane % 8 <- piece (lane % 8) ^ (row / 2)
    const int8_t *xsrc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 8 * h + (lane >> 3);
        xsrc[h] = X + (int64_t)min(row, M - 1) * K + 16 * ((lane & 7) ^ (row >> 1));
    }
    uint4 *const region[kBpw] = {b0 + wave * kBlockSlots, b1 + wave * kBlockSlots,
                                 b2 + wave * kBlockSlots, b3 + wave * kBlockSlots};
    // fragment: lane (r16, q) takes pieces 2q and 2q + 1 of row r16
    const int f0 = 8 * r16 + ((2 * q) ^ (r16 >> 1)), f1 = 8 * r16 + ((2 * q + 1) ^ (r16 >> 1));

    const int nblk = K / 128;
    v4i acc = v4i{};
    for (int kb = 0; kb < K; kb += kKBlock) {
        const int blk0 = (kb >> 7) + wave * kBpw;
        v4i a[kBpw];
        int idx[kBpw];
#pragma unroll
        for (int j = 0; j < kBpw; ++j) {
            const int blk = min(blk0 + j, nblk - 1);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                __builtin_amdgcn_global_load_lds((global_void *)(xsrc[h] + 128 * blk),
                                                 (lds_void *)(region[j] + 64 * h), 16, 0, 0);
            a[j] = __builtin_bit_cast(v4i, load16_stream(vrow + blk * vstride));
            idx[j] = (int)mrow[blk * mstride];
            __builtin_amdgcn_sched_barrier(0);  // block by block, in this order
        }
#pragma unroll
        for (int j = 0; j < kBpw; ++j) {
            if (j == 0) wait_vm_s24<kLoadsPerBlock * (kBpw - 1)>();
            else if (j == 1) wait_vm_s24<kLoadsPerBlock * (kBpw - 2)>();
            else if (j == 2) wait_vm_s24<kLoadsPerBlock * (kBpw - 3)>();
            else wait_vm_s24<0>();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            // a block past K multiplies zero values (a select, not a branch:
            // see the W4A16 kernel)
            const v4i av = blk0 + j < nblk ? a[j] : v4i{};
            const uint4 lo = region[j][f0], hi = region[j][f1];
            const v8i b = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z,
                           (int)hi.w};
            acc = smfmac_16x16x128(av, b, acc, idx[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // every fragment of this block was read before the next block's
        // loads refill the regions (the MFMAs consumed them)
    }

#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();
    // one output per thread: channel c of row j sits in lane j + 16 * (c / 4), element c % 4
    if (threadIdx.x >= 256) return;
    const int j = threadIdx.x >> 4, c = threadIdx.x & 15;
    if (j >= M) return;
    const int l = j + 16 * (c >> 2), r = c & 3;
    int sum = 0;
#pragma unroll
    for (int w = 0; w < kSplit; ++w) sum += red[w][r][l];
    const int n = n0 + c;
    if constexpr (OUT_I32)
        static_cast<int32_t *>(out)[(int64_t)j * N + n] = sum;
    else
        static_cast<__bf16 *>(out)[(int64_t)j * N + n] =
            (__bf16)dequant(sum, split_scale(sx[j]), split_scale(sw[n]));
}

template <int MT>
hipError_t launch_decode_mt(const int8_t *xq, const float *xs, int M, const int8_t *values,
                            const uint32_t *meta, const float *ws, int N, int K, void *out,
                            bool out_i32, hipStream_t stream) {
    const int steps_per_wave = (K / 128 + kSplit - 1) / kSplit;   // 128-column blocks
    const dim3 grid((unsigned)(N / 16)), block(kSplit * kWave);
    if (out_i32)
        sparse24_decode_kernel<MT, true><<<grid, block, 0, stream>>>(xq, xs, values, meta, ws, out,
                                                                      M, N, K, steps_per_wave);
    else
        sparse24_decode_kernel<MT, false><<<grid, block, 0, stream>>>(xq, xs, values, meta, ws, out,
                                                                       M, N, K, steps_per_wave);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// LDS-tiled 2:4 GEMM for larger M: a workgroup of 4 wavefronts (2 x 2) computes
// a 128-row x 256-channel tile with v_smfmac_i32_32x32x64_i8 (weights as the
// sparse operand), K advancing 128 columns per stage through a ring of 4 LDS
// stages filled with direct-to-LDS 16-byte loads, as the dense tiled kernel
// does. The compressed weight is half the bytes of the dense one, so the tile
// is wide in channels: per stage 16 KB of activations and 20 KB of weights,
// and the 144 KB ring keeps three stages in flight (the loop is bound by how
// many operand bytes are on their way from L2, not by the MFMAs).
//
// Stage layout (16-byte slots): activations, 128 rows x 8 slots, chunk c of
// row r at slot c ^ (r % 8) ^ ((r / 8) % 2) (bank-conflict-free fragment
// reads, as in the dense kernel); the weights' 64 value bytes per row, 256
// rows x 4 slots, chunk c of row r at slot c ^ ((r / 2) % 4) (the same: 8
// consecutive rows reading one chunk hit 8 distinct 16-byte bank groups); the
// weights' 4 index words per row, 256 slots. In the K-block-major storage a
// block's pieces of the tile's 256 weight rows are contiguous (16 KB of
// values, 4 KB of index words), so every 64-lane load moves whole cache
// lines. Each wavefront issues 4 + 4 + 1 loads per stage.
//
// Per 64-column step a lane reads, for each 32-row activation tile, the two
// slots holding bytes [32 h, 32 h + 32) of the step (h = lane / 32), and for
// each 32-channel weight tile the value slot of list half h and its index
// word. Fragments of the next step are read while the current step's MFMAs run.
constexpr int kTBM = 128, kTBN = 256, kTStages = 4;
constexpr int kTThreads = 256;
constexpr int kTXSlots = kTBM * 8, kTVSlots = kTBN * 4, kTMSlots = kTBN;
constexpr int kTStage = kTXSlots + kTVSlots + kTMSlots;   // 16-byte slots per stage
constexpr int kTXLd = kTXSlots / (64 * 4);                // loads per wavefront per stage
constexpr int kTVLd = kTVSlots / (64 * 4);
constexpr int kTMLd = kTMSlots / (64 * 4);
constexpr int kTNld = kTXLd + kTVLd + kTMLd;
constexpr int kTWM = 64, kTWN = 128;                      // wavefront sub-tile
constexpr int kTTM = kTWM / 32, kTTN = kTWN / 32;
static_assert(kTXLd * 256 == kTXSlots && kTVLd * 256 == kTVSlots && kTMLd * 256 == kTMSlots,
              "whole runs per wavefront");
static_assert(kTBM * kTBN * 2 <= kTStages * kTStage * 16, "bf16 tile fits in the stage buffers");


__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int vswz(int row) { return (row >> 1) & 3; }

__device__ __forceinline__ v16i smfmac_32x32x64(v4i a, v8i b, v16i c, int idx) {
    return __builtin_amdgcn_smfmac_i32_32x32x64_i8(a, b, c, idx, 0, 0);
}

struct TFrag {
    v8i x[kTTM];
    v4i w[kTTN];
    int idx[kTTN];
};

template <bool OUT_I32>
__global__ __launch_bounds__(kTThreads, 1) void sparse24_tiled_kernel(
    const int8_t *__restrict__ X, const float *__restrict__ sx, const int8_t *__restrict__ V,
    const uint32_t *__restrict__ Meta, const float *__restrict__ sw, void *__restrict__ out,
    int M, int N, int K, int tiles_m, int tiles_n) {
    __shared__ uint4 lds[kTStages * kTStage];
    lds_poison(lds);
    lds_poison_done();
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;

    // tile order: XCD-contiguous, then groups of 4 tile rows
    const int tiles = tiles_m * tiles_n;
    const int t = xcd_contiguous(blockIdx.x, tiles);
    constexpr int kGroup = 4;
    const int per_group = kGroup * tiles_n;
    const int first_m = (t / per_group) * kGroup;
    const int gsize = min(tiles_m - first_m, kGroup);
    const int m0 = (first_m + (t % per_group) % gsize) * kTBM;
    const int n0 = ((t % per_group) / gsize) * kTBN;
    const int nk = K / 128;

    // per-lane sources of this wavefront's loads (stage 0; stage j adds j * inc)
    const int8_t *xsrc[kTXLd];
    {
        const int row = 8 * wave + (lane >> 3);
        const int kc = (lane & 7) ^ swz(row);
#pragma unroll
        for (int l = 0; l < kTXLd; ++l)
            xsrc[l] = X + (int64_t)min(m0 + row + 32 * l, M - 1) * K + 16 * kc;
    }
    const int8_t *vsrc[kTVLd];
#pragma unroll
    for (int l = 0; l < kTVLd; ++l) {
        const int slot = 64 * (wave + 4 * l) + lane;
        const int row = slot >> 2, c = (slot & 3) ^ vswz(row);
        vsrc[l] = V + (int64_t)min(n0 + row, N - 1) * 64 + 16 * c;
    }
    const uint32_t *msrc = Meta + (int64_t)min(n0 + 64 * wave + lane, N - 1) * 4;
    static_assert(kTMLd == 1, "one index-word load per wavefront");
    const int64_t vstride = (int64_t)N * 64, mstride = (int64_t)N * 4;   // per block
    auto load_stage = [&](int j, uint4 *buf) {
#pragma unroll
        for (int l = 0; l < kTXLd; ++l)
            __builtin_amdgcn_global_load_lds((global_void *)(xsrc[l] + 128 * j),
                                             (lds_void *)(buf + 64 * (wave + 4 * l)), 16, 0, 0);
#pragma unroll
        for (int l = 0; l < kTVLd; ++l)
            __builtin_amdgcn_global_load_lds((global_void *)(vsrc[l] + j * vstride),
                                             (lds_void *)(buf + kTXSlots + 64 * (wave + 4 * l)), 16,
                                             0, 0);
        __builtin_amdgcn_global_load_lds((global_void *)(msrc + j * mstride),
                                         (lds_void *)(buf + kTXSlots + kTVSlots + 64 * wave), 16, 0,
                                         0);
    };

    const int frag_row = lane & 31, half = lane >> 5;
    const int xrow0 = wm * kTWM + frag_row, wrow0 = wn * kTWN + frag_row;
    const int fswz = swz(frag_row);
    auto read_frags = [&](const uint4 *buf, int step, TFrag &f) {
        const int c0 = (4 * step + 2 * half) ^ fswz, c1 = (4 * step + 2 * half + 1) ^ fswz;
#pragma unroll
        for (int i = 0; i < kTTM; ++i) {
            const int r = xrow0 + 32 * i;   // r % 16 == frag_row % 16: same swizzle
            const v4i lo = __builtin_bit_cast(v4i, buf[r * 8 + c0]);
            const v4i hi = __builtin_bit_cast(v4i, buf[r * 8 + c1]);
            f.x[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        const uint4 *vb = buf + kTXSlots, *mb = buf + kTXSlots + kTVSlots;
        const int vc = (2 * step + half) ^ vswz(frag_row);   // (r / 2) % 4 == (frag_row / 2) % 4
#pragma unroll
        for (int j = 0; j < kTTN; ++j) {
            const int r = wrow0 + 32 * j;
            f.w[j] = __builtin_bit_cast(v4i, vb[r * 4 + vc]);
            f.idx[j] = reinterpret_cast<const int *>(mb + r)[2 * step + half];
        }
    };

    v16i acc[kTTM][kTTN];
#pragma unroll
    for (int i = 0; i < kTTM; ++i)
#pragma unroll
        for (int j = 0; j < kTTN; ++j) acc[i][j] = v16i{};
    // One step's MFMAs on fragments f, with `reads` (the next step's fragment
    // reads) issued right after the first one: the wait before that first MFMA
    // (the compiler waits for all LDS reads) then finds reads issued a whole
    // step earlier, and the new reads land while the other MFMAs run.
    auto mma_then_read = [&](const TFrag &f, auto &&reads) {
        acc[0][0] = smfmac_32x32x64(f.w[0], f.x[0], acc[0][0], f.idx[0]);
        __builtin_amdgcn_sched_barrier(0);
        reads();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 1; q < kTTM * kTTN; ++q) {
            const int i = q / kTTN, j = q % kTTN;
            acc[i][j] = smfmac_32x32x64(f.w[j], f.x[i], acc[i][j], f.idx[j]);
        }
        __builtin_amdgcn_sched_barrier(0);
    };

    auto stage_buf = [&](int j) { return lds + (j % kTStages) * kTStage; };
    // barrier after which stage j has landed for every wavefront, when `later`
    // stages were issued after it (their loads may stay in flight)
    auto stage_landed = [&](int later) {
        static_assert(kTStages <= 4, "waits below cover up to 2 later stages");
        if (later >= 2)
            vm_barrier<2 * kTNld>();
        else if (later == 1)
            vm_barrier<kTNld>();
        else
            vm_barrier<0>();
    };
    // prologue: stages 0 .. kTStages-2 in flight, stage 0 landed everywhere
    const int pre = min(kTStages - 1, nk);
    for (int j = 0; j < pre; ++j) load_stage(j, stage_buf(j));
    stage_landed(pre - 1);
    TFrag f0, f1;
    read_frags(stage_buf(0), 0, f0);
    for (int s = 0; s < nk; ++s) {
        const uint4 *cur = stage_buf(s);
        // the buffer refilled here was last read in stage s - 1, before its barrier
        if (s + kTStages - 1 < nk) load_stage(s + kTStages - 1, stage_buf(s + kTStages - 1));
        __builtin_amdgcn_sched_barrier(0);
        mma_then_read(f0, [&] { read_frags(cur, 1, f1); });
        // the next stage has landed from this wavefront (only stages issued
        // after it may still be in flight) and its reads of this stage are
        // done; after the barrier both hold for every wavefront. (On the last
        // stage the reads below fetch a stale buffer, in bounds and unused.)
        stage_landed(min(kTStages - 2, nk - 2 - s));
        mma_then_read(f1, [&] { read_frags(stage_buf(s + 1), 0, f0); });
    }
    __syncthreads();  // all fragment reads done before the epilogue reuses LDS

    // tile (i, j), element r of a lane: activation row i*32 + lane%32 of the
    // wavefront's sub-tile, channel j*32 + 8*(r/4) + 4*half + r%4
    const int mw0 = m0 + wm * kTWM, nw0 = n0 + wn * kTWN;
    if constexpr (OUT_I32) {
#pragma unroll
        for (int i = 0; i < kTTM; ++i) {
            const int m = mw0 + i * 32 + frag_row;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < kTTN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = nw0 + j * 32 + 8 * g + 4 * half;
                    if (n < N)
                        __builtin_nontemporal_store(
                            v4i{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                acc[i][j][4 * g + 3]},
                            reinterpret_cast<v4i *>(static_cast<int32_t *>(out) + (int64_t)m * N + n));
                }
        }
    } else {
        // stage the wavefront's 64 x 128 bf16 sub-tile in LDS (16-byte chunks of
        // a row permuted by row % 8), then store whole 16-byte row pieces
        constexpr int CH = kTWN / 8;
        uint2 *st8 = reinterpret_cast<uint2 *>(lds) + wave * (kTWM * kTWN / 4);
        float sxv[kTTM];
        bool rows_tame = true;
#pragma unroll
        for (int i = 0; i < kTTM; ++i) {
            sxv[i] = sx[min(mw0 + i * 32 + frag_row, M - 1)];
            rows_tame = rows_tame && tame_scale(sxv[i]);
        }
#pragma unroll
        for (int j = 0; j < kTTN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = min(nw0 + j * 32 + 8 * g + 4 * half, N - 4);
                const float4 w = *reinterpret_cast<const float4 *>(sw + n);
                // the plain product when the wavefront's scales are all tame
                const bool cheap = wave_all(rows_tame && tame_scale(w.x) && tame_scale(w.y) &&
                                            tame_scale(w.z) && tame_scale(w.w));
#pragma unroll
                for (int i = 0; i < kTTM; ++i) {
                    const int ml = i * 32 + frag_row;
                    const v16i &a = acc[i][j];
                    float v[4];
                    if (cheap) {
                        v[0] = (float)a[4 * g] * sxv[i] * w.x;
                        v[1] = (float)a[4 * g + 1] * sxv[i] * w.y;
                        v[2] = (float)a[4 * g + 2] * sxv[i] * w.z;
                        v[3] = (float)a[4 * g + 3] * sxv[i] * w.w;
                    } else {
                        const SplitScale x = split_scale(sxv[i]);
                        v[0] = dequant(a[4 * g], x, split_scale(w.x));
                        v[1] = dequant(a[4 * g + 1], x, split_scale(w.y));
                        v[2] = dequant(a[4 * g + 2], x, split_scale(w.z));
                        v[3] = dequant(a[4 * g + 3], x, split_scale(w.w));
                    }
                    const uint32_t lo = pack_bf16x2(v[0], v[1]);
                    const uint32_t hi = pack_bf16x2(v[2], v[3]);
                    st8[(ml * CH + ((j * 4 + g) ^ (ml & 7))) * 2 + half] = make_uint2(lo, hi);
                }
            }
        __syncthreads();
        const uint4 *st16 = reinterpret_cast<const uint4 *>(st8);
#pragma unroll
        for (int it = 0; it < kTWM * CH / kWave; ++it) {
            const int q = it * kWave + lane;
            const int ml = q / CH, cc = q % CH;
            const int m = mw0 + ml, n = nw0 + cc * 8;
            const uint4 v = st16[ml * CH + (cc ^ (ml & 7))];
            if (m < M && n < N) store16_nt(static_cast<__bf16 *>(out) + (int64_t)m * N + n, v);
        }
    }
}

}  // namespace

hipError_t launch_compress24(const int8_t *wq, int N, int K, int8_t *values, uint32_t *meta,
                             hipStream_t stream) {
    const int64_t chunks = (int64_t)N * (K / 32);   // 16-byte value pieces = index words
    const dim3 grid((unsigned)((chunks + 255) / 256)), block(256);
    compress24_kernel<<<grid, block, 0, stream>>>(wq, chunks, N, K, values, meta);
    return hipGetLastError();
}

hipError_t launch_sparse24_gemm(const int8_t *xq, const float *xs, int M, const int8_t *values,
                                const uint32_t *meta, const float *ws, int N, int K, void *out,
                                bool out_i32, hipStream_t stream) {
    if (M <= 16 && K >= 4096) {
        const dim3 grid((unsigned)(N / 16)), block(kSplit * kWave);
        if (out_i32)
            sparse24_decode_lds_kernel<true><<<grid, block, 0, stream>>>(xq, xs, values, meta, ws, out, M, N, K);
        else
            sparse24_decode_lds_kernel<false><<<grid, block, 0, stream>>>(xq, xs, values, meta, ws, out, M, N, K);
        return hipGetLastError();
    }
    switch ((M + 15) / 16) {
        case 1: return launch_decode_mt<1>(xq, xs, M, values, meta, ws, N, K, out, out_i32, stream);
        case 2: return launch_decode_mt<2>(xq, xs, M, values, meta, ws, N, K, out, out_i32, stream);
        case 3: return launch_decode_mt<3>(xq, xs, M, values, meta, ws, N, K, out, out_i32, stream);
        case 4: return launch_decode_mt<4>(xq, xs, M, values, meta, ws, N, K, out, out_i32, stream);
        default: break;
    }
    const int tiles_m = (M + kTBM - 1) / kTBM, tiles_n = (N + kTBN - 1) / kTBN;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kTThreads);
    if (out_i32)
        sparse24_tiled_kernel<true><<<grid, block, 0, stream>>>(xq, xs, values, meta, ws, out, M, N,
                                                                K, tiles_m, tiles_n);
    else
        sparse24_tiled_kernel<false><<<grid, block, 0, stream>>>(xq, xs, values, meta, ws, out, M,
                                                                 N, K, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace w8a8
