// Block-sparse (BSR, 64x64 blocks) int8 GEMM with the fused dequant epilogue.
//
// The weight arrives as the raw crow/col/values arrays of a BSR matrix
// (pytorch/ao PR #821: the custom op over crow_indices, col_indices and values;
// 64x64 blocks from the bsr_dense_addmm warning). An output tile is a 256-row
// slab of X times one block row (64 output channels); it walks only the
// stored blocks of its block row: block j multiplies X[:, 64 col[j] : +64] by
// values[j]^T, two K=32 MFMA steps per 32x32 tile. Block rows without stored
// blocks still write their +0 outputs.
//
// At 10% block density a tile holds about two blocks, and the kernel is bound
// by its output write (2 bytes per output against about 0.2 bytes of X). A
// workgroup per tile would pay one full load latency per tile and then sit
// idle through its store. So the kernel is persistent and wave-specialised:
//  - a workgroup runs through a list of tiles; its block loads form one
//    stream across tile boundaries, kept STAGES - 1 blocks ahead in a ring of
//    LDS buffers, so the loads of the next tiles are in flight while a tile's
//    outputs are scaled and stored;
//  - 4 producer wavefronts only issue direct-to-LDS loads (64 rows of X and
//    16 rows of the weight block each, plus the tile's scales), so their
//    vector-memory counter holds loads only and a counted wait names exactly
//    the blocks that must have landed;
//  - 4 consumer wavefronts only read LDS, multiply (64 rows each: 2x2
//    v_mfma_i32_32x32x32_i8 tiles) and store; they never wait on a memory
//    counter, so their stores drain in the background;
//  - one workgroup barrier per block: the block has landed, and the buffer of
//    the previous block may be refilled;
//  - the epilogue stages each consumer's rows through a private LDS region,
//    32 rows x 128 bytes at a time, and stores whole 128-byte lines with
//    16-byte streaming (nontemporal) stores, in the final [M, N] layout
//    (pytorch/ao PR #821, the two .t().contiguous() removals); streaming
//    stores keep the output from evicting X from L2;
//  - LDS rows are 64 bytes; chunk c of row r sits at slot c ^ ((r / 2) % 4),
//    so 8 consecutive lanes reading one chunk of 8 consecutive rows touch 8
//    distinct 16-byte bank groups;
//  - the workgroups of one XCD walk a contiguous tile range side by side:
//    the ~8 block rows that read one X block find it in that XCD's L2, and
//    their stores land in adjacent 128-byte pieces of the same output rows
//    (scattered 128-byte pieces cost the write path about 10%);
//  - the addmm variant (alpha, beta, a per-channel bias) reads the tile's 64
//    bias values with scalar loads in the consumers' epilogue: no LDS (the
//    budget of two workgroups per CU is spent) and no vector-memory wait in
//    the consumers; block rows without stored blocks then write
//    bf16(alpha * 0 + beta * bias[n]) through the same epilogue;
//  - measured and not kept: 8 consumers of 32 rows each
//    (more store streams, but more barrier and LDS traffic) and equal-work
//    contiguous tile runs (better balance, scattered stores).
#include <numeric>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace w8a8 {
namespace {

constexpr int kBS = 64;          // block size
constexpr int kBM = 256;         // rows of X per tile
constexpr int kMathWaves = 4;    // consumers, kRowsPerMath rows each
constexpr int kLoadWaves = 4;    // producers
constexpr int kThreads = (kMathWaves + kLoadWaves) * kWave;
constexpr int kRowSlots = 4;     // 16-byte slots per 64-byte LDS row
constexpr int kStages = 3;       // ring depth
constexpr int kRowsPerMath = kBM / kMathWaves;  // 32: one 32-row MFMA tile
constexpr int kTM = kRowsPerMath / 32;
static_assert(kTM >= 1 && kRowsPerMath % 32 == 0, "whole 32-row MFMA tiles per consumer");

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

__device__ __forceinline__ int bswz(int row) { return (row >> 1) & 3; }
__device__ __forceinline__ int oswz(int row) { return (row >> 1) & 7; }

// One ring buffer, in 16-byte slots: the tile's 256 rows of X for the block
// (64 per producer), the 64 rows of the weight block, the tile's 256 row
// scales and its 64 channel scales.
constexpr int kXSlots = kBM * kRowSlots;                 // 16 KB
constexpr int kWSlots = kBS * kRowSlots;                 // 4 KB
constexpr int kSaSlots = kBM * 4 / 16;                   // 1 KB
constexpr int kSbSlots = kBS * 4 / 16;                   // 256 B
constexpr int kWOff = kXSlots, kSaOff = kWOff + kWSlots, kSbOff = kSaOff + kSaSlots;
constexpr int kBufSlots = kSbOff + kSbSlots;             // 21.25 KB
constexpr int kSR = kRowsPerMath >= 32 && kMathWaves <= 4 ? 32 : 16;  // staging rows per pass
constexpr int kStageSlots = kSR * 8;                     // per consumer: kSR rows x 128 B
constexpr int kLdsSlots = kStages * kBufSlots + kMathWaves * kStageSlots;
// Tiles are taken in segments of up to kSegTiles, whose stored-block ranges
// sit in a small LDS table.
constexpr int kSegTiles = 32;
static_assert(kLdsSlots * 16 + kSegTiles * 8 <= 80 * 1024, "two workgroups per CU");

// Direct-to-LDS loads per producer and block: 4 of X, 1 of the weight, 1 of
// the row scales; producer 0 also loads the channel scales.
constexpr int kLoads = 6;

// The index arrays are read-only here: reading them through the constant
// address space lets the (uniform) reads be scalar loads, which count on the
// scalar counter instead of the vector-memory counter the producers' waits
// are built on.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ int load_index(const int32_t *p, int i) {
    return ((const_i32 *)p)[i];
}
typedef __attribute__((address_space(4))) const float const_f32;

struct Args {
    const int8_t *A;
    const float *sa;
    const int32_t *crow, *col;
    const int8_t *values;
    const float *sb;
    void *out;
    int nnzb, M, N, K, block_rows;
    Addmm am;  // used by the addmm variant only
};

// The tiles of one workgroup: lo, lo + step, ... < hi. Tile t is X slab
// t / block_rows times block row t % block_rows.
struct TileList {
    int lo, hi, step;
};

// The tiles of workgroup b: XCD x = b % 8 owns the contiguous tile range
// [x T / 8, (x + 1) T / 8), and its P / 8 workgroups take every (P / 8)-th
// tile of it. The workgroups of an XCD thus work on neighbouring tiles at the
// same time: one X slab in its L2, and output stores to adjacent 128-byte
// pieces of the same rows. The host makes P / 8 coprime with the block-row
// count, so each workgroup's tiles cycle through all block rows and the
// per-workgroup work (stored blocks) evens out.
__device__ __forceinline__ TileList tile_list(int tiles) {
    const int P = (int)gridDim.x, b = (int)blockIdx.x;
    TileList L;
    if (P >= kXcds && P % kXcds == 0) {
        const int x = b % kXcds;
        L.lo = (int)((int64_t)tiles * x / kXcds) + b / kXcds;
        L.hi = (int)((int64_t)tiles * (x + 1) / kXcds);
        L.step = P / kXcds;
    } else {
        L.lo = b;
        L.hi = tiles;
        L.step = P;
    }
    return L;
}

// ---- producers ----------------------------------------------------------

// Issue the loads of stored block j (column block colj) of the tile at rows
// m0, block row br into ring buffer `buf`. Producer p fills X rows [64 p, +64) and weight rows
// [16 p, +16): load q puts row 16 q + lane / 4 at physical slot lane % 4,
// which holds the logical chunk lane % 4 ^ bswz(row) (the same for every q).
__device__ __forceinline__ void produce_block(const Args &a, uint4 *buf, int p, int lane, int j,
                                              int colj, int m0, int br) {
    const int lrow = lane >> 2;
    const int lc = (lane & 3) ^ bswz(lrow);  // bswz(16 q + r) == bswz(r)
    const int cb = max(0, min(colj, a.K / kBS - 1));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = min(m0 + 64 * p + 16 * q + lrow, a.M - 1);
        __builtin_amdgcn_global_load_lds((global_void *)(a.A + (int64_t)row * a.K + cb * kBS + lc * 16),
                                         (lds_void *)(buf + 256 * p + 64 * q), 16, 0, 0);
    }
    __builtin_amdgcn_global_load_lds(
        (global_void *)(a.values + (int64_t)j * kBS * kBS + (16 * p + lrow) * kBS + lc * 16),
        (lds_void *)(buf + kWOff + 64 * p), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((global_void *)(a.sa + min(m0 + 64 * p + lane, a.M - 1)),
                                     (lds_void *)(buf + kSaOff + 16 * p), 4, 0, 0);
    if (p == 0)
        __builtin_amdgcn_global_load_lds((global_void *)(a.sb + br * kBS + lane),
                                         (lds_void *)(buf + kSbOff), 4, 0, 0);
}

// Wait until at most `ahead` blocks after the one to be multiplied are in
// flight from this producer, then meet the consumers.
__device__ __forceinline__ void producer_barrier(int ahead, bool p0) {
    static_assert(kStages == 3, "the waits below cover ahead in {0, 1}");
    if (ahead <= 0)
        vm_barrier<0>();
    else if (p0)
        vm_barrier<kLoads + 1>();
    else
        vm_barrier<kLoads>();
}

// Number of tiles in a workgroup's list.
__device__ __forceinline__ int list_len(const TileList &L) {
    return L.lo < L.hi ? (L.hi - L.lo + L.step - 1) / L.step : 0;
}

// The producers' share of one segment (list tiles s0 .. s0 + cnt - 1, block
// ranges in `meta`): issue the segment's stored blocks in order, STAGES - 1
// ahead of the consumers, one barrier per block. The column index of the
// next block is read (a scalar load) when the current one is issued, so its
// latency overlaps the wait at the barrier in between.
__device__ __forceinline__ void producer(const Args &a, uint4 *lds, const int2 *meta,
                                         const TileList &L, int s0, int cnt, int p, int lane) {
    // the next block to issue: block cj of segment tile ck, which has blocks
    // up to cje, column index ccol
    int ck = 0, cj = 0, cje = 0;
    auto seek = [&](int k) {  // first segment tile from k on with blocks
        for (; k < cnt; ++k) {
            const int2 r = meta[k];
            if (r.y > r.x) {
                cj = r.x;
                cje = r.y;
                break;
            }
        }
        ck = k;
    };
    seek(0);
    int ccol = ck < cnt ? load_index(a.col, cj) : 0;
    int issued = 0, consumed = 0;
    auto issue_next = [&]() {
        if (ck >= cnt) return;
        const int t = L.lo + (s0 + ck) * L.step;
        produce_block(a, lds + (issued % kStages) * kBufSlots, p, lane, cj, ccol,
                      (t / a.block_rows) * kBM, t % a.block_rows);
        ++issued;
        if (++cj == cje) seek(ck + 1);
        if (ck < cnt) ccol = load_index(a.col, cj);
    };
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue_next();
    // the consumers take the blocks in the order they were issued
    while (consumed < issued) {
        producer_barrier(issued - consumed - 1, p == 0);
        ++consumed;
        issue_next();  // into the buffer of the block multiplied before this one
    }
}

// ---- consumers ----------------------------------------------------------


template <typename OutT>
__device__ __forceinline__ void store_zero_rows(const Args &a, int m0, int br, int w, int lane) {
    // kRowsPerMath rows x 64 outputs as 16-byte pieces
    constexpr int kPieces = kBS * (int)sizeof(OutT) / 16;
    constexpr int kPer = 16 / (int)sizeof(OutT);
    for (int q = lane; q < kRowsPerMath * kPieces; q += kWave) {
        const int row = m0 + kRowsPerMath * w + q / kPieces;
        if (row < a.M)
            store16_nt(static_cast<OutT *>(a.out) + (int64_t)row * a.N + br * kBS + (q % kPieces) * kPer,
                    make_uint4(0, 0, 0, 0));
    }
}

// Tile (i, jt), element r of a lane: row 32 i + lane % 32 of this consumer's
// rows, channel 32 jt + 8 (r / 4) + 4 (lane / 32) + r % 4 (the weight is the
// first MFMA operand). The outputs go out in passes of kSR rows x 128 bytes
// (64 bf16 or 32 int32 channels), whole 128-byte lines: scale, write the pass
// into the private staging rows (16-byte chunk c of row r at slot
// c ^ oswz(r)), read it back as 16-byte pieces, 8 lanes per row, and store.
// Half-line (64-byte) pieces cost the write path about half its rate.
//
// ADDMM: out = bf16(alpha * (acc * sa * sb) + beta * bias[n]). EMPTY (addmm
// only): a block row without stored blocks, acc = 0 and no ring buffer.
template <typename OutT, bool ADDMM, bool EMPTY>
__device__ __forceinline__ void store_tile(const Args &a, const uint4 *__restrict__ buf,
                                           uint4 *__restrict__ stg, const v16i (&acc)[kTM][2],
                                           int m0, int br, int w, int lane) {
    constexpr bool kI32 = std::is_same<OutT, int32_t>::value;
    static_assert(!(kI32 && ADDMM) && (ADDMM || !EMPTY), "addmm writes bf16");
    constexpr int kCp = 128 / (int)sizeof(OutT);  // channels per 128-byte row piece
    constexpr int kPieces = kBS / kCp;            // pieces per row: 1 (bf16) or 2 (int32)
    const int frag_row = lane & 31, half = lane >> 5;
    const int srow = frag_row & (kSR - 1);        // this lane's row within a pass
    const float *sa_l = reinterpret_cast<const float *>(buf + kSaOff);
    const float *sb_l = reinterpret_cast<const float *>(buf + kSbOff);
    char *sbytes = reinterpret_cast<char *>(stg);
    // addmm: the tile's 64 bias values are uniform, read once per tile with
    // scalar loads into ub (uniform registers); each lane selects its own
    // 4 channels 32 jt + 8 g + 4 half + (0..3) where it uses them.
    // (readfirstlane keeps the compiler from turning the select of two loads
    // into one vector load, whose wait would also wait for this wavefront's
    // output stores.)
    float ub[kBS];
#pragma unroll
    for (int c = 0; c < kBS; ++c) ub[c] = 0.0f;
    if (ADDMM && a.am.bias) {
        const const_f32 *bb = (const const_f32 *)(a.am.bias + br * kBS);
#pragma unroll
        for (int c = 0; c < kBS; ++c)
            ub[c] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, bb[c])));
    }
#pragma unroll
    for (int rg = 0; rg < kRowsPerMath / kSR; ++rg) {
        const int i = rg * kSR / 32;  // MFMA row tile of this pass
        // with 16-row passes, half of the lanes hold the pass's rows
        const bool mine = kSR == 32 || (frag_row >> 4) == (rg & 1);
        // the row scale as significand and power of two (see the products below)
        const SplitScale sx =
            split_scale(kI32 || EMPTY ? 0.0f : sa_l[kRowsPerMath * w + 32 * i + frag_row]);
#pragma unroll
        for (int h = 0; h < kPieces; ++h) {
            if (mine) {
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    if ((32 * jt) / kCp != h) continue;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int c0 = 32 * jt + 8 * g + 4 * half;           // first of 4 channels
                        const int off = (c0 - kCp * h) * (int)sizeof(OutT);  // byte in the piece
                        char *dst = sbytes + srow * 128 + (((off >> 4) ^ oswz(srow)) << 4) + (off & 15);
                        if constexpr (kI32) {
                            *reinterpret_cast<v4i *>(dst) =
                                v4i{acc[i][jt][4 * g], acc[i][jt][4 * g + 1], acc[i][jt][4 * g + 2],
                                    acc[i][jt][4 * g + 3]};
                        } else {
                            const float4 s = EMPTY ? make_float4(0.0f, 0.0f, 0.0f, 0.0f)
                                                   : *reinterpret_cast<const float4 *>(sb_l + c0);
                            const int cb = 32 * jt + 8 * g;
                            const float4 bv = half ? make_float4(ub[cb + 4], ub[cb + 5], ub[cb + 6], ub[cb + 7])
                                                   : make_float4(ub[cb], ub[cb + 1], ub[cb + 2], ub[cb + 3]);
                            // acc * sa * sb as ldexp((acc * f) * sb, e) with
                            // sa = f * 2^e, f in [0.5, 1): no intermediate
                            // overflows or underflows for any row scale, nor
                            // for channel scales in [2^-125, 2^97]
                            float v[4];
                            const float sc[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                v[e] = __builtin_amdgcn_ldexpf((float)acc[i][jt][4 * g + e] * sx.f * sc[e], sx.e);
                            const uint32_t lo = pack_bf16x2(addmm<ADDMM>(v[0], a.am, bv.x),
                                                            addmm<ADDMM>(v[1], a.am, bv.y));
                            const uint32_t hi = pack_bf16x2(addmm<ADDMM>(v[2], a.am, bv.z),
                                                            addmm<ADDMM>(v[3], a.am, bv.w));
                            *reinterpret_cast<uint2 *>(dst) = make_uint2(lo, hi);
                        }
                    }
                }
            }
#pragma unroll
            for (int r8 = 0; r8 < kSR / 8; ++r8) {
                const int rr = 8 * r8 + (lane >> 3), lc = lane & 7;
                const uint4 v = stg[rr * 8 + (lc ^ oswz(rr))];
                const int row = m0 + kRowsPerMath * w + rg * kSR + rr;
                if (row < a.M)
                    store16_nt(static_cast<OutT *>(a.out) + (int64_t)row * a.N + br * kBS + kCp * h +
                                lc * (16 / (int)sizeof(OutT)),
                            v);
            }
        }
    }
}

// One stored block for a consumer: its rows of X times the weight block,
// two K=32 steps of kTM x 2 MFMA tiles; FIRST starts from zero.
template <bool FIRST>
__device__ __forceinline__ void multiply_block(const uint4 *buf, int w, int frag_row, int half,
                                               v16i (&acc)[kTM][2]) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        v4i xa[kTM], wb[2];
#pragma unroll
        for (int i = 0; i < kTM; ++i) {
            const int r = kRowsPerMath * w + 32 * i + frag_row;
            xa[i] = __builtin_bit_cast(v4i, buf[r * kRowSlots + ((kk * 2 + half) ^ bswz(r))]);
        }
#pragma unroll
        for (int jt = 0; jt < 2; ++jt) {
            const int r = 32 * jt + frag_row;
            wb[jt] = __builtin_bit_cast(v4i, buf[kWOff + r * kRowSlots + ((kk * 2 + half) ^ bswz(r))]);
        }
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
                acc[i][jt] = mfma_32x32x32(wb[jt], xa[i], FIRST && kk == 0 ? v16i{} : acc[i][jt]);
    }
}

// The consumers' share of one segment: multiply each tile's blocks as they
// land (one barrier per block), then scale and store the tile.
template <typename OutT, bool ADDMM>
__device__ __forceinline__ void consumer(const Args &a, uint4 *lds, const int2 *meta,
                                         const TileList &L, int s0, int cnt, int w, int lane) {
    const int frag_row = lane & 31, half = lane >> 5;
    uint4 *stg = lds + kStages * kBufSlots + w * kStageSlots;
    int n = 0;  // blocks of the segment multiplied so far; block n sits in buffer n % kStages
    for (int k = 0; k < cnt; ++k) {
        const int t = L.lo + (s0 + k) * L.step;
        const int br = t % a.block_rows, m0 = (t / a.block_rows) * kBM;
        const int2 r = meta[k];
        const int j0 = r.x, j1 = r.y;
        if (j0 == j1) {
            if constexpr (ADDMM) {
                v16i zero[kTM][2];
#pragma unroll
                for (int i = 0; i < kTM; ++i) zero[i][0] = zero[i][1] = v16i{};
                store_tile<OutT, true, true>(a, nullptr, stg, zero, m0, br, w, lane);
            } else {
                store_zero_rows<OutT>(a, m0, br, w, lane);
            }
            continue;
        }
        // the first block starts the accumulators from zero (an inline
        // constant operand of the MFMA, no register clearing)
        v16i acc[kTM][2];
        lds_barrier();
        const uint4 *buf = lds + (n % kStages) * kBufSlots;
        multiply_block<true>(buf, w, frag_row, half, acc);
        ++n;
        for (int j = j0 + 1; j < j1; ++j, ++n) {
            lds_barrier();
            buf = lds + (n % kStages) * kBufSlots;
            multiply_block<false>(buf, w, frag_row, half, acc);
        }
        // the buffer of the tile's last block (with its scales) is refilled
        // only after the next barrier, which this wavefront reaches after
        // its reads below
        store_tile<OutT, ADDMM, false>(a, buf, stg, acc, m0, br, w, lane);
    }
}

// Two workgroups per CU: four wavefronts per SIMD, at most 128 registers each.
template <bool OUT_I32, bool ADDMM>
__global__ __launch_bounds__(kThreads, 4) void bsr_gemm_kernel(Args a, int slabs) {
    using OutT = typename std::conditional<OUT_I32, int32_t, __bf16>::type;
    __shared__ uint4 lds[kLdsSlots];
    __shared__ int2 meta[kSegTiles];  // stored-block range of each tile of the segment
    lds_poison(lds);
    lds_poison(meta);
    lds_poison_done();
    // the wavefront index is uniform: saying so makes the role branch below a
    // scalar branch with two separate paths
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const bool math = wave < kMathWaves;
    const TileList L = tile_list(slabs * a.block_rows);
    const int nt = list_len(L);
    // The roles branch once, each with its own segment loop, so that the
    // compiler's wait analysis of the consumers never sees the producers'
    // loads. Both pass the same barriers: two per segment (the previous
    // segment is done with the ring buffers and the table; the table is
    // filled) and one per stored block.
    if (math) {
        for (int s0 = 0; s0 < nt; s0 += kSegTiles) {
            const int cnt = min(kSegTiles, nt - s0);
            lds_barrier();
            lds_barrier();
            consumer<OutT, ADDMM>(a, lds, meta, L, s0, cnt, wave, lane);
        }
    } else {
        for (int s0 = 0; s0 < nt; s0 += kSegTiles) {
            const int cnt = min(kSegTiles, nt - s0);
            vm_barrier<0>();  // the last segment's loads have all been waited for
            if (wave == kMathWaves && lane < cnt) {
                const int br = (L.lo + (s0 + lane) * L.step) % a.block_rows;
                const int j0 = max(0, min(a.crow[br], a.nnzb));
                meta[lane] = make_int2(j0, max(j0, min(a.crow[br + 1], a.nnzb)));
            }
            vm_barrier<0>();
            producer(a, lds, meta, L, s0, cnt, wave - kMathWaves, lane);
        }
        // nothing is in flight here; saying so keeps the compiler from
        // carrying the producers' loads into the consumers' path where the
        // two join
        __builtin_amdgcn_s_waitcnt(0);
    }
}

}  // namespace

hipError_t launch_bsr_gemm(const int8_t *xq, const float *xs, int M, int K, const int32_t *crow,
                           const int32_t *col, const int8_t *values, int nnzb, const float *ws,
                           int N, void *out, bool out_i32, hipStream_t stream, const Addmm *am) {
    const int slabs = (M + kBM - 1) / kBM, block_rows = N / kBS;
    const int tiles = slabs * block_rows;
    // two resident workgroups per CU, a multiple of the XCD count
    int P = 2 * device_cu_count();
    if (P > tiles) P = tiles;
    if (P >= kXcds) P -= P % kXcds;
    if (P >= kXcds) {
        // a stride coprime with the block-row count walks each workgroup
        // through all block rows
        int per = P / kXcds;
        while (per > 1 && std::gcd(per, block_rows) != 1) --per;
        P = per * kXcds;
    }
    const Args a{xq, xs, crow, col, values, ws, out, nnzb, M, N, K, block_rows,
                 am ? *am : Addmm{nullptr, 1.0f, 0.0f}};
    const dim3 grid((unsigned)P), block(kThreads);
    if (out_i32)
        bsr_gemm_kernel<true, false><<<grid, block, 0, stream>>>(a, slabs);
    else if (am)
        bsr_gemm_kernel<false, true><<<grid, block, 0, stream>>>(a, slabs);
    else
        bsr_gemm_kernel<false, false><<<grid, block, 0, stream>>>(a, slabs);
    return hipGetLastError();
}

}  // namespace w8a8
