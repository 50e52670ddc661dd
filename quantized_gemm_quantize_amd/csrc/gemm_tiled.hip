// LDS-tiled int8 MFMA GEMM with the dequant epilogue fused (large M).
//
//   out[m,n] = bf16( (sum_k A[m,k] * B[n,k]) * sa[m] * sb[n] )
//
// A = xq [M,K] row-major, B = wq [N,K]: both operands K-contiguous, the int8
// layout that needs no transpose (triton issue #634, layout answer). The int32
// accumulators live in the MFMA result registers and are scaled and rounded to
// bf16 in registers before the only store, so the int32 matrix never reaches
// HBM (pytorch/ao PR #821, fused-dequant paragraph; "move scaling operations to
// bsr_dense_addmm kernel" item).
//
// Shape of the kernel (gfx950):
//  - a workgroup of 4 wavefronts computes a BM x BN tile; each wavefront owns a
//    (BM/WAVES_M) x (BN/WAVES_N) sub-tile of 32x32 v_mfma_i32_32x32x32_i8 tiles;
//  - K advances 128 bytes per stage. Every thread moves 16-byte chunks with
//    buffer loads into registers, then into one of two LDS stages; with two
//    register sets the loads for stage k+2 are in flight while stage k feeds
//    the MFMAs and stage k+1 waits in registers.
//    Buffer loads return zero past the end of the tile's rows, which handles
//    ragged M and N without branches; a chunk past K is pointed out of range;
//  - LDS rows are 128 bytes; chunk c of row r sits at slot
//    c ^ (r % 8) ^ ((r / 8) % 2), so 16 consecutive lanes reading the same
//    chunk of 16 consecutive rows hit 16 distinct 16-byte bank groups;
//  - the MFMA takes the weight fragment as its first operand, so each lane
//    ends with 4 consecutive output channels of one row: the epilogue scales
//    them, packs 4 bf16 into 8 bytes and stages the tile in LDS, from where
//    every store is a full 16-byte piece of a contiguous output row;
//  - tiles are assigned XCD-contiguously, then in groups of 8 tile rows, so
//    concurrently running tiles share A and B rows in the same L2.
#include "common.hpp"
#include "launch.hpp"

namespace w8a8 {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 128;          // K bytes per stage
constexpr int kCPR = kBK / 16;    // 16-byte chunks per tile row
constexpr int kRowsPerPass = kThreads / kCPR;  // 32 tile rows per load pass
constexpr int kGroupM = 8;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format (gfx9 family)
constexpr int kOutOfRange = 0x40000000; // offset past every tile buffer: loads return 0

// bank-group swizzle of a 128-byte LDS row
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const int8_t *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(base), (short)0, bytes, kRsrcWord3);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voffset) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, 0, 0));
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool OUT_I32>
__global__ __launch_bounds__(kThreads, 1) void gemm_tiled_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ sa, const int8_t *__restrict__ B,
    const float *__restrict__ sb, void *__restrict__ out, int M, int N, int K, int tiles_m,
    int tiles_n) {
    static_assert(WAVES_M * WAVES_N == kThreads / kWave, "4 wavefronts");
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int A_LD = BM / kRowsPerPass, B_LD = BN / kRowsPerPass;
    constexpr int STAGE = (BM + BN) * kCPR;  // uint4 slots per stage
    static_assert(BM * BN * 2 <= 2 * STAGE * 16, "bf16 tile fits in the stage buffers");
    __shared__ uint4 lds[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // tile coordinates
    const int tiles = tiles_m * tiles_n;
    const int t = xcd_contiguous(blockIdx.x, tiles);
    const int per_group = kGroupM * tiles_n;
    const int first_m = (t / per_group) * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int m0 = (first_m + (t % per_group) % gsize) * BM;
    const int n0 = ((t % per_group) / gsize) * BN;

    const __amdgpu_buffer_rsrc_t ra_rsrc = tile_rsrc(A + (int64_t)m0 * K, min(BM, M - m0) * K);
    const __amdgpu_buffer_rsrc_t rb_rsrc = tile_rsrc(B + (int64_t)n0 * K, min(BN, N - n0) * K);

    // this thread loads chunk kc of tile rows lrow + 32 * i
    const int kc = tid % kCPR, lrow = tid / kCPR;
    const int voff0 = lrow * K + kc * 16;
    const int slot0 = lrow * kCPR + (kc ^ swz(lrow));  // + 256 * i (32 rows keep the swizzle)

    // two register sets: the loads for stage k+2 are issued while stage k is
    // multiplied, so each load has two stages of MFMA work to arrive
    uint4 ra0[A_LD], rb0[B_LD], ra1[A_LD], rb1[B_LD];
    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

    const int nk = (K + kBK - 1) / kBK;
    // fragment reads: lanes 0-31 take the first 16 bytes of each 32-byte K step,
    // lanes 32-63 the second, for both operands
    const int frag_row = lane & 31, half = lane >> 5;
    const int a_frag = (wm * WM + frag_row) * kCPR;
    const int b_frag = BM * kCPR + (wn * WN + frag_row) * kCPR;
    const int fswz = swz(frag_row);

    // Tile t walks its K stages starting at stage t % nk (integer sums do not
    // depend on the order): rows of one tile sit a power-of-two stride apart,
    // so without the rotation every concurrently running tile would read the
    // same K offset, i.e. the same L2 channel.
    const int rot = t % nk;
#define W8A8_GLOAD(RA, RB, j)                                                       \
    {                                                                               \
        int ks_ = (j) + rot;                                                        \
        if (ks_ >= nk) ks_ -= nk;                                                   \
        const int koff = ((j) < nk && kc * 16 + ks_ * kBK < K) ? ks_ * kBK : kOutOfRange; \
        _Pragma("unroll") for (int i = 0; i < A_LD; ++i)                            \
            RA[i] = buffer_load16(ra_rsrc, voff0 + i * kRowsPerPass * K + koff);     \
        _Pragma("unroll") for (int i = 0; i < B_LD; ++i)                            \
            RB[i] = buffer_load16(rb_rsrc, voff0 + i * kRowsPerPass * K + koff);     \
    }
#define W8A8_LSTORE(RA, RB, stage)                                                  \
    {                                                                               \
        uint4 *s_ = lds + (stage) * STAGE + slot0;                                  \
        _Pragma("unroll") for (int i = 0; i < A_LD; ++i) s_[i * kThreads] = RA[i];  \
        _Pragma("unroll") for (int i = 0; i < B_LD; ++i)                            \
            s_[BM * kCPR + i * kThreads] = RB[i];                                   \
    }
#define W8A8_FRAGS(F, S, kk)                                                        \
    {                                                                               \
        const int c_ = ((kk) * 2 + half) ^ fswz;                                    \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                              \
            xa[F][i] = __builtin_bit_cast(v4i, S[a_frag + i * 32 * kCPR + c_]);     \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                              \
            wb[F][j] = __builtin_bit_cast(v4i, S[b_frag + j * 32 * kCPR + c_]);     \
    }
    // MFMA slots of one stage: (TM*TN) per K step, 4 K steps. Memory work per
    // stage: A_LD+B_LD buffer loads, 3 x (TM+TN) fragment reads, A_LD+B_LD
    // LDS writes. Loads go one per MFMA in the first half, reads one per MFMA
    // through the first three K steps, writes one per MFMA in the second half.
    constexpr int NMF = 4 * TM * TN, NLD = A_LD + B_LD, NRD = 3 * (TM + TN);
#define W8A8_SCHEDULE()                                                             \
    {                                                                               \
        _Pragma("unroll") for (int q = 0; q < NMF; ++q) {                           \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      \
            if (q < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);         \
            if (q < NLD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);         \
            if (q >= NMF - NLD) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);  \
        }                                                                           \
    }
    // One stage: the fragments of K step kk+1 are read while step kk multiplies,
    // the global loads for two stages ahead and the LDS writes of the stage
    // after next are spread one per MFMA. A wavefront issues in order, so a
    // burst of buffer loads would hold the MFMAs behind a full address queue;
    // the scheduling-group barriers below fix the interleaving.
#define W8A8_STAGE(stage, RA_NEXT, RB_NEXT, j_next, RA_ST, RB_ST, st_stage)          \
    {                                                                               \
        const uint4 *S = lds + (stage) * STAGE;                                     \
        __builtin_amdgcn_sched_barrier(0);                                          \
        W8A8_GLOAD(RA_NEXT, RB_NEXT, j_next)                                        \
        _Pragma("unroll") for (int kk = 0; kk < kCPR / 2; ++kk) {                   \
            if (kk + 1 < kCPR / 2) W8A8_FRAGS((kk + 1) & 1, S, kk + 1)              \
            _Pragma("unroll") for (int i = 0; i < TM; ++i)                          \
                _Pragma("unroll") for (int j = 0; j < TN; ++j)                      \
                    acc[i][j] = mfma_32x32x32(wb[kk & 1][j], xa[kk & 1][i], acc[i][j]); \
        }                                                                           \
        W8A8_LSTORE(RA_ST, RB_ST, st_stage)                                         \
        W8A8_SCHEDULE()                                                             \
        __builtin_amdgcn_sched_barrier(0);                                          \
        __syncthreads();                                                            \
        W8A8_FRAGS(0, (lds + (st_stage) * STAGE), 0)                                \
    }
    // Stages alternate between LDS buffers 0/1 and register sets 0/1. Loads of
    // stages past K return zeros (out-of-range offsets) and land in a buffer
    // no one reads, so the loop body needs no branches.
    v4i xa[2][TM], wb[2][TN];
    W8A8_GLOAD(ra0, rb0, 0)
    W8A8_GLOAD(ra1, rb1, 1)
    W8A8_LSTORE(ra0, rb0, 0)
    __syncthreads();
    W8A8_FRAGS(0, lds, 0)
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        W8A8_STAGE(0, ra0, rb0, kt + 2, ra1, rb1, 1)
        W8A8_STAGE(1, ra1, rb1, kt + 3, ra0, rb0, 0)
    }
    if (kt < nk) {
        const uint4 *S = lds;
#pragma unroll
        for (int kk = 0; kk < kCPR / 2; ++kk) {
            if (kk > 0) W8A8_FRAGS(0, S, kk)
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma_32x32x32(wb[0][j], xa[0][i], acc[i][j]);
        }
    }
#undef W8A8_GLOAD
#undef W8A8_LSTORE
#undef W8A8_FRAGS
#undef W8A8_STAGE
#undef W8A8_SCHEDULE

    // Tile (i, j), element r of a lane: row m = i*32 + lane%32 of the wave's
    // sub-tile, channel n = j*32 + 8*(r/4) + 4*half + r%4.
    const int mw0 = m0 + wm * WM, nw0 = n0 + wn * WN;
    if constexpr (OUT_I32) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = mw0 + i * 32 + frag_row;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = nw0 + j * 32 + 8 * g + 4 * half;
                    if (n < N)
                        *reinterpret_cast<v4i *>(static_cast<int32_t *>(out) + (int64_t)m * N + n) =
                            v4i{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                acc[i][j][4 * g + 3]};
                }
        }
    } else {
        // stage the wave's WM x WN bf16 sub-tile in LDS (row-major, 16-byte
        // chunks of a row permuted by row % 8), then store whole 16-byte pieces
        constexpr int CH = WN / 8;  // 16-byte chunks per staged row
        static_assert(CH >= 8, "the row-chunk permutation needs 8 chunks per row");
        uint2 *st8 = reinterpret_cast<uint2 *>(lds) + wave * (WM * WN / 4);
        float swv[TN][4][4];
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = min(nw0 + j * 32 + 8 * g + 4 * half, N - 4);
                const float4 v = *reinterpret_cast<const float4 *>(sb + n);
                swv[j][g][0] = v.x; swv[j][g][1] = v.y; swv[j][g][2] = v.z; swv[j][g][3] = v.w;
            }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int ml = i * 32 + frag_row;
            const float sxv = sa[min(mw0 + ml, M - 1)];
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const v16i &a = acc[i][j];
                    const uint32_t lo = pack_bf16x2((float)a[4 * g] * sxv * swv[j][g][0],
                                                    (float)a[4 * g + 1] * sxv * swv[j][g][1]);
                    const uint32_t hi = pack_bf16x2((float)a[4 * g + 2] * sxv * swv[j][g][2],
                                                    (float)a[4 * g + 3] * sxv * swv[j][g][3]);
                    const int chunk = (j * 4 + g) ^ (ml & 7);
                    st8[(ml * CH + chunk) * 2 + half] = make_uint2(lo, hi);
                }
        }
        __syncthreads();
        const uint4 *st16 = reinterpret_cast<const uint4 *>(st8);
#pragma unroll
        for (int it = 0; it < WM * CH / kWave; ++it) {
            const int q = it * kWave + lane;
            const int ml = q / CH, cc = q % CH;
            const int m = mw0 + ml, n = nw0 + cc * 8;
            const uint4 v = st16[ml * CH + (cc ^ (ml & 7))];
            if (m < M && n < N)
                *reinterpret_cast<uint4 *>(static_cast<__bf16 *>(out) + (int64_t)m * N + n) = v;
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N>
hipError_t launch_cfg(const int8_t *xq, const float *xs, int M, const int8_t *wq, const float *ws,
                      int N, int K, void *out, bool out_i32, hipStream_t stream) {
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kThreads);
    if (out_i32)
        gemm_tiled_kernel<BM, BN, WAVES_M, WAVES_N, true>
            <<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, tiles_m, tiles_n);
    else
        gemm_tiled_kernel<BM, BN, WAVES_M, WAVES_N, false>
            <<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_decode(const int8_t *xq, const float *xs, int M, const int8_t *wq,
                              const float *ws, int N, int K, void *out, bool out_i32,
                              hipStream_t stream);

hipError_t launch_gemm(const int8_t *xq, const float *xs, int M, const int8_t *wq, const float *ws,
                       int N, int K, void *out, bool out_i32, hipStream_t stream) {
    if (M <= 64) return launch_gemm_decode(xq, xs, M, wq, ws, N, K, out, out_i32, stream);
    // Enough 256x256 tiles to fill 256 CUs several times over: the big tile
    // halves LDS traffic per MFMA. Otherwise 256x128 (or 128x128) tiles.
    const long t256 = (long)((M + 255) / 256) * ((N + 255) / 256);
    const long t128 = (long)((M + 255) / 256) * ((N + 127) / 128);
    if (t256 >= 4 * 256) return launch_cfg<256, 256, 2, 2>(xq, xs, M, wq, ws, N, K, out, out_i32, stream);
    if (t128 >= 256) return launch_cfg<256, 128, 2, 2>(xq, xs, M, wq, ws, N, K, out, out_i32, stream);
    return launch_cfg<128, 128, 2, 2>(xq, xs, M, wq, ws, N, K, out, out_i32, stream);
}

}  // namespace w8a8
