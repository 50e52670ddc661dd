// Block-sparse (BSR, 64x64 blocks) int8 GEMM with the fused dequant epilogue.
//
// The weight arrives as the raw crow/col/values arrays of a BSR matrix
// (pytorch/ao PR #821: the custom op over crow_indices, col_indices and values;
// 64x64 blocks from the bsr_dense_addmm warning). Each workgroup owns a
// 128-row slab of X and one block row (64 output channels) and walks only the
// stored blocks of that block row: for block j it multiplies X[:, 64 col[j] :
// +64] by values[j]^T with two K=32 MFMA steps. Block rows without stored
// blocks still write their +0 outputs.
//
// At 10% block density the kernel is bound by writing the bf16 output, so the
// result tile is staged in LDS and leaves as full 128-byte rows of 16-byte
// stores; the result is written in its final [M,N] row-major layout, with no
// transposed copy (pytorch/ao PR #821, the two .t().contiguous() removals).
// Tiles are ordered so that each XCD works through whole X slabs, reading each
// slab into its L2 once for all 80 block rows.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace w8a8 {
namespace {

constexpr int kBS = 64;       // block size
constexpr int kBM = 128;      // rows of X per workgroup
constexpr int kThreads = 256; // 4 wavefronts x 32 rows

template <bool OUT_I32>
__global__ __launch_bounds__(kThreads) void bsr_gemm_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ sa, const int32_t *__restrict__ crow,
    const int32_t *__restrict__ col, const int8_t *__restrict__ values, int nnzb,
    const float *__restrict__ sb, void *__restrict__ out, int M, int N, int K, int slabs,
    int block_rows) {
    using OutT = typename std::conditional<OUT_I32, int32_t, __bf16>::type;
    __shared__ __attribute__((aligned(16))) OutT tile[kBM * kBS];

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int t = xcd_contiguous(blockIdx.x, slabs * block_rows);
    const int slab = t / block_rows, br = t % block_rows;
    const int m0 = slab * kBM;
    const int frag_row = lane & 31, half = lane >> 5;

    const int8_t *arow = A + (int64_t)min(m0 + wave * 32 + frag_row, M - 1) * K + half * 16;
    v16i acc[2] = {v16i{}, v16i{}};

    // indices are trusted for values but clamped for addresses
    int j0 = crow[br], j1 = crow[br + 1];
    j0 = max(0, min(j0, nnzb));
    j1 = max(j0, min(j1, nnzb));
    const int kblocks = K / kBS;
    for (int j = j0; j < j1; ++j) {
        const int cb = max(0, min(col[j], kblocks - 1));
        const int8_t *blk = values + (int64_t)j * kBS * kBS + half * 16;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const v4i a = *reinterpret_cast<const v4i *>(arow + cb * kBS + kk * 32);
            const v4i b0 = *reinterpret_cast<const v4i *>(blk + frag_row * kBS + kk * 32);
            const v4i b1 = *reinterpret_cast<const v4i *>(blk + (32 + frag_row) * kBS + kk * 32);
            acc[0] = mfma_32x32x32(a, b0, acc[0]);
            acc[1] = mfma_32x32x32(a, b1, acc[1]);
        }
    }

    // scale in registers, stage the tile in LDS
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
        const int c = tn * 32 + frag_row;
        const float sbv = OUT_I32 ? 0.0f : sb[br * kBS + c];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rl = wave * 32 + 8 * (r / 4) + 4 * half + (r % 4);
            if constexpr (OUT_I32) {
                tile[rl * kBS + c] = acc[tn][r];
            } else {
                const int row = min(m0 + rl, M - 1);
                tile[rl * kBS + c] = (__bf16)((float)acc[tn][r] * sa[row] * sbv);
            }
        }
    }
    __syncthreads();

    // 16-byte row-contiguous stores of the [128 x 64] tile
    constexpr int kPerChunk = 16 / sizeof(OutT);
    constexpr int kChunksPerRow = kBS / kPerChunk;
    constexpr int kChunks = kBM * kChunksPerRow;
    const uint4 *src = reinterpret_cast<const uint4 *>(tile);
    for (int q = threadIdx.x; q < kChunks; q += kThreads) {
        const int rl = q / kChunksPerRow, cc = q % kChunksPerRow;
        const int row = m0 + rl;
        if (row >= M) continue;
        OutT *dst = static_cast<OutT *>(out) + (int64_t)row * N + br * kBS + cc * kPerChunk;
        *reinterpret_cast<uint4 *>(dst) = src[q];
    }
}

}  // namespace

hipError_t launch_bsr_gemm(const int8_t *xq, const float *xs, int M, int K, const int32_t *crow,
                           const int32_t *col, const int8_t *values, int nnzb, const float *ws,
                           int N, void *out, bool out_i32, hipStream_t stream) {
    const int slabs = (M + kBM - 1) / kBM, block_rows = N / kBS;
    const dim3 grid((unsigned)(slabs * block_rows)), block(kThreads);
    if (out_i32)
        bsr_gemm_kernel<true><<<grid, block, 0, stream>>>(xq, xs, crow, col, values, nnzb, ws, out,
                                                          M, N, K, slabs, block_rows);
    else
        bsr_gemm_kernel<false><<<grid, block, 0, stream>>>(xq, xs, crow, col, values, nnzb, ws,
                                                           out, M, N, K, slabs, block_rows);
    return hipGetLastError();
}

}  // namespace w8a8
