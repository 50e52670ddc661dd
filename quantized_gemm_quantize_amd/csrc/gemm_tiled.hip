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
//  - operands travel global -> LDS with global_load_lds_dwordx4 (gfx950's
//    16-byte direct-to-LDS load), never through registers: on MI355X this
//    path moves about twice the bytes per CU per clock of loads into VGPRs,
//    which is what an int8 tile needs to keep the MFMAs fed. K advances 128
//    bytes per stage through a ring of STAGES LDS buffers, loads running
//    STAGES-1 stages ahead of the MFMAs;
//  - LDS rows are 128 bytes; chunk c of row r sits at slot
//    c ^ (r % 8) ^ ((r / 8) % 2), so 16 consecutive lanes reading the same
//    chunk of 16 consecutive rows hit 16 distinct 16-byte bank groups. A
//    direct-to-LDS load writes 64 consecutive slots, so each lane fetches the
//    global chunk that belongs in its slot;
//  - rows past M or N are read from the last valid row (their outputs are
//    never stored); chunks past K are not loaded but zeroed in LDS;
//  - the MFMA takes the weight fragment as its first operand, so each lane
//    ends with 4 consecutive output channels of one row: the epilogue scales
//    them, packs 4 bf16 into 8 bytes and stages the tile in LDS, from where
//    every store is a full 16-byte piece of a contiguous output row, written
//    as a streaming (nontemporal) store so the output does not evict the
//    operands from L2;
//  - tiles are assigned XCD-contiguously, then in groups of 4 (256x128 tiles)
//    or 8 (256x256) tile rows, so concurrently running tiles share A and B
//    rows in the same L2.
#include "common.hpp"
#include "launch.hpp"

namespace w8a8 {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// tile rows per group in the tile order (see the kernel): 4 for 256x128 tiles
// (an XCD's 32 tiles then span 1024 rows x 1024 columns: less of A and B per
// L2), 8 for 256x256
template <int BN>
constexpr int group_m() { return BN == 128 ? 4 : 8; }

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// Stages hold CPR 16-byte chunks of K per tile row (CPR = 8: 128 bytes of K,
// CPR = 4: 64 bytes). Bank-group swizzle of such an LDS row: chunk c of row r
// sits at slot c ^ swz<CPR>(r), so 8 and 16 consecutive rows reading the same
// chunk hit distinct 16-byte bank groups.
template <int CPR>
__device__ __forceinline__ int swz(int row) {
    static_assert(CPR == 8 || CPR == 4, "128- or 64-byte stage rows");
    if constexpr (CPR == 8)
        return (row & 7) ^ ((row >> 3) & 1);
    else
        return ((row >> 1) & 3) ^ ((row >> 3) & 1);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt bits
// [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier of the mainloop: this wavefront's loads up to the last
// N are in LDS and its own LDS accesses are done, then all wavefronts meet.
// No memory fence: a workgroup release fence would also wait for the
// direct-to-LDS loads still in flight for later stages. The empty asm
// statements keep the compiler from moving memory accesses across.
template <int N>
__device__ __forceinline__ void stage_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Per-lane load geometry of one tile: load l of this wavefront fills LDS slots
// [wslot + 256 l, +64) (A) or [BM*CPR + wslot + 256 l, +64) (B), i.e. tile
// rows (64/CPR) wave + (256/CPR) l + lane/CPR at physical slot lane % CPR,
// which holds the logical chunk kc = (lane % CPR) ^ swz(row) -- the same for
// every l.
template <int A_LD, int B_LD>
struct TileLoads {
    int aoff[A_LD], boff[B_LD];  // byte offsets of this lane's chunks in the tile rows
    int kc;                      // logical chunk
    int wslot;                   // 64 * wavefront
    int K, nk;
};

// Issue the direct-to-LDS loads of K stage j into `wr` (or, with KTAIL, zero
// the slots whose chunk lies past K).
template <int BM, int CPR, int A_LD, int B_LD, bool KTAIL>
__device__ __forceinline__ void load_stage(const int8_t *__restrict__ at, const int8_t *__restrict__ bt,
                                           uint4 *__restrict__ wr, const TileLoads<A_LD, B_LD> &g,
                                           int j, int lane) {
    const int k0 = j * 16 * CPR;
    const bool in = !KTAIL || g.kc * 16 + k0 < g.K;
#pragma unroll
    for (int l = 0; l < A_LD + B_LD; ++l) {
        uint4 *dst = wr + g.wslot + (l < A_LD ? 256 * l : BM * CPR + 256 * (l - A_LD));
        const int8_t *src = l < A_LD ? at + g.aoff[l] + k0 : bt + g.boff[l - A_LD] + k0;
        if (in)
            __builtin_amdgcn_global_load_lds((global_void *)src, (lds_void *)dst, 16, 0, 0);
        else
            dst[lane] = make_uint4(0, 0, 0, 0);
    }
}

// One K stage: multiply the stage held in `rd` while loading the stage
// STAGES-1 ahead into `wr`, and read the first fragments of the next stage
// from `nx`. The buffers are distinct, and the restrict qualifiers say so:
// after inlining, the fragment reads carry alias scopes that separate them
// from the loads still landing in `wr`, so the wait before the barrier covers
// only the stage that has to be complete.
//
// The barrier sits before the last K step, not at the end of the stage: by
// then every wavefront has read all of this stage's fragments, so the buffer
// may be refilled, and the next stage's first fragments are read while the
// last K step multiplies instead of after a barrier with nothing to overlap.
//
// Per K step kk: TM*TN MFMA slots. The fragment reads for the next step go
// out in two bursts, after the first and the second MFMA (reads r with
// r % 2 == slot), so they have the rest of the step's MFMAs to land; then
// one direct-to-LDS load follows each further MFMA (this step's share of the
// stage loads). The order is pinned with scheduling barriers: a wavefront
// issues in order, and a burst of loads would hold the MFMAs.
template <int BM, int CPR, int TM, int TN, int STAGES, int A_LD, int B_LD, bool KTAIL>
__device__ __forceinline__ void mainloop_stage(const int8_t *__restrict__ at,
                                               const int8_t *__restrict__ bt,
                                               const uint4 *__restrict__ rd, uint4 *__restrict__ wr,
                                               const uint4 *__restrict__ nx,
                                               const TileLoads<A_LD, B_LD> &g, int s, int lane,
                                               int a_frag, int b_frag, int half, int fswz,
                                               v16i (&acc)[TM][TN], v4i (&xa)[2][TM],
                                               v4i (&wb)[2][TN]) {
    constexpr int NLD = A_LD + B_LD;
    constexpr int NMF = TM * TN;        // MFMAs per K step
    constexpr int KS = CPR / 2;         // K steps per stage
    // With three buffers the stage being loaded is not the next one read, so
    // its loads may also follow the stage barrier: they are spread over all K
    // steps, and the barrier waits for all but the LPRE issued before it. With
    // two, every load of the next stage precedes the barrier.
    constexpr bool LATE = STAGES == 3;
    constexpr int LSTEPS = LATE ? KS : KS - 1;
    constexpr int LPK = (NLD + LSTEPS - 1) / LSTEPS;  // loads per K step
    constexpr int LPRE = LATE ? ((KS - 1) * LPK < NLD ? (KS - 1) * LPK : NLD) : 0;
    constexpr int NSLOT = NMF > 2 + LPK ? NMF : 2 + LPK;
    const int j_ahead = s + STAGES - 1;
    const bool ahead = j_ahead < g.nk;  // uniform
    const int k0 = j_ahead * 16 * CPR;
    const bool in = !KTAIL || g.kc * 16 + k0 < g.K;
    // with double buffering the next stage is the one being loaded into `wr`
    // (and `nx` is not accessed), otherwise it is `nx`
    const uint4 *next = STAGES == 2 ? wr : nx;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const int f = kk & 1;
        if (kk == KS - 1) {
            // the next stage has landed from this wavefront (only the stage
            // issued in this one may still be in flight), this wavefront's
            // reads of this stage are done; after the barrier both hold for all
            if (ahead)
                stage_barrier<LPRE>();
            else
                stage_barrier<0>();
        }
        const uint4 *src_buf = kk + 1 < KS ? rd : next;
        const int ch = (((kk + 1) % KS) * 2 + half) ^ fswz;
#pragma unroll
        for (int q = 0; q < NSLOT; ++q) {
            if (q < NMF) {
                const int i = q / TN, j = q % TN;
                acc[i][j] = mfma_32x32x32(wb[f][j], xa[f][i], acc[i][j]);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (q < 2) {
#pragma unroll
                for (int r = 0; r < TM + TN; ++r) {
                    if (r % 2 != q) continue;
                    if (r < TM)
                        xa[f ^ 1][r] = __builtin_bit_cast(v4i, src_buf[a_frag + r * 32 * CPR + ch]);
                    else
                        wb[f ^ 1][r - TM] = __builtin_bit_cast(v4i, src_buf[b_frag + (r - TM) * 32 * CPR + ch]);
                }
            }
            const int l = kk * LPK + (q - 2);
            if (kk < LSTEPS && q >= 2 && q < 2 + LPK && l < NLD && ahead) {
                uint4 *dst = wr + g.wslot + (l < A_LD ? 256 * l : BM * CPR + 256 * (l - A_LD));
                const int8_t *src = l < A_LD ? at + g.aoff[l] + k0 : bt + g.boff[l - A_LD] + k0;
                if (in)
                    __builtin_amdgcn_global_load_lds((global_void *)src, (lds_void *)dst, 16, 0, 0);
                else
                    dst[lane] = make_uint4(0, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int CPR, int OCC, bool KTAIL,
          bool OUT_I32, bool ADDMM>
__global__ __launch_bounds__(kThreads, OCC) void gemm_tiled_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ sa, const int8_t *__restrict__ B,
    const float *__restrict__ sb, void *__restrict__ out, int M, int N, int K, int tiles_m,
    int tiles_n, Addmm am) {
    static_assert(!(ADDMM && OUT_I32), "the addmm epilogue writes bf16");
    static_assert(WAVES_M * WAVES_N == kWaves, "4 wavefronts");
    static_assert(STAGES == 2 || STAGES == 3, "double or triple buffering");
    constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
    constexpr int TM = WM / 32, TN = WN / 32;
    // direct-to-LDS loads per wavefront per stage: each covers 64/CPR tile rows
    constexpr int A_LD = BM * CPR / (64 * kWaves), B_LD = BN * CPR / (64 * kWaves);
    constexpr int NLD = A_LD + B_LD;
    constexpr int STAGE = (BM + BN) * CPR;   // uint4 slots per stage
    static_assert(BM * BN * 2 <= STAGES * STAGE * 16, "bf16 tile fits in the stage buffers");
    __shared__ uint4 lds[STAGES * STAGE];
    lds_poison(lds);
    lds_poison_done();

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    // tile coordinates
    const int tiles = tiles_m * tiles_n;
    const int t = xcd_contiguous(blockIdx.x, tiles);
    constexpr int kGroupM = group_m<BN>();
    const int per_group = kGroupM * tiles_n;
    const int first_m = (t / per_group) * kGroupM;
    const int gsize = min(tiles_m - first_m, kGroupM);
    const int m0 = (first_m + (t % per_group) % gsize) * BM;
    const int n0 = ((t % per_group) / gsize) * BN;
    const int8_t *at = A + (int64_t)m0 * K;
    const int8_t *bt = B + (int64_t)n0 * K;

    TileLoads<A_LD, B_LD> g;
    {
        const int lrow = (64 / CPR) * wave + lane / CPR;
        g.kc = (lane % CPR) ^ swz<CPR>(lrow);
        const int a_last = min(BM, M - m0) - 1, b_last = min(BN, N - n0) - 1;
#pragma unroll
        for (int l = 0; l < A_LD; ++l) g.aoff[l] = min(lrow + (256 / CPR) * l, a_last) * K + g.kc * 16;
#pragma unroll
        for (int l = 0; l < B_LD; ++l) g.boff[l] = min(lrow + (256 / CPR) * l, b_last) * K + g.kc * 16;
        g.wslot = 64 * wave;
        g.K = K;
        g.nk = (K + 16 * CPR - 1) / (16 * CPR);
    }
    const int nk = g.nk;

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v16i{};

    // fragment reads: lanes 0-31 take the first 16 bytes of each 32-byte K step,
    // lanes 32-63 the second, for both operands
    const int frag_row = lane & 31, half = lane >> 5;
    const int a_frag = (wm * WM + frag_row) * CPR;
    const int b_frag = BM * CPR + (wn * WN + frag_row) * CPR;
    const int fswz = swz<CPR>(frag_row);
    v4i xa[2][TM], wb[2][TN];

    uint4 *const b0 = lds, *const b1 = lds + STAGE, *const b2 = lds + (STAGES > 2 ? 2 : 0) * STAGE;
    // prologue: stages 0 .. STAGES-2 in flight, stage 0 landed everywhere
    load_stage<BM, CPR, A_LD, B_LD, KTAIL>(at, bt, b0, g, 0, lane);
    if (STAGES == 3 && nk > 1) load_stage<BM, CPR, A_LD, B_LD, KTAIL>(at, bt, b1, g, 1, lane);
    if (STAGES == 3 && nk > 1)
        stage_barrier<NLD>();
    else
        stage_barrier<0>();
    {
        const int ch0 = half ^ fswz;
#pragma unroll
        for (int i = 0; i < TM; ++i) xa[0][i] = __builtin_bit_cast(v4i, b0[a_frag + i * 32 * CPR + ch0]);
#pragma unroll
        for (int j = 0; j < TN; ++j) wb[0][j] = __builtin_bit_cast(v4i, b0[b_frag + j * 32 * CPR + ch0]);
    }

#define W8A8_STAGE(RD, WR, NX, S_)                                                               \
    mainloop_stage<BM, CPR, TM, TN, STAGES, A_LD, B_LD, KTAIL>(at, bt, RD, WR, NX, g, S_, lane, \
                                                               a_frag, b_frag, half, fswz, acc,  \
                                                               xa, wb)
    int s = 0;
    if constexpr (STAGES == 3) {
        for (; s + 3 <= nk; s += 3) {
            W8A8_STAGE(b0, b2, b1, s);
            W8A8_STAGE(b1, b0, b2, s + 1);
            W8A8_STAGE(b2, b1, b0, s + 2);
        }
        if (s < nk) W8A8_STAGE(b0, b2, b1, s++);
        if (s < nk) W8A8_STAGE(b1, b0, b2, s++);
    } else {
        // double buffering: the buffer being filled is also the next one read
        for (; s + 2 <= nk; s += 2) {
            W8A8_STAGE(b0, b1, b1, s);
            W8A8_STAGE(b1, b0, b0, s + 1);
        }
        if (s < nk) W8A8_STAGE(b0, b1, b1, s++);
    }
#undef W8A8_STAGE
    (void)NLD;
    __syncthreads();  // all fragment reads done before the epilogue reuses LDS

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
                        __builtin_nontemporal_store(
                            v4i{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                                acc[i][j][4 * g + 3]},
                            reinterpret_cast<v4i *>(static_cast<int32_t *>(out) + (int64_t)m * N + n));
                }
        }
    } else {
        // stage the wave's WM x WN bf16 sub-tile in LDS (row-major, 16-byte
        // chunks of a row permuted by the low row bits, so that the 32 rows of
        // one store instruction spread over all banks), then store whole
        // 16-byte pieces
        constexpr int CH = WN / 8;  // 16-byte chunks per staged row
        static_assert(CH == 8 || CH == 16, "the row-chunk permutation needs 8 or 16 chunks per row");
        constexpr int PM = CH - 1;
        uint2 *st8 = reinterpret_cast<uint2 *>(lds) + wave * (WM * WN / 4);
        // per 4 channels: their scales (and bias) once, then the TM rows. The
        // plain (acc * sa) * sb when every scale of the wavefront is tame (a
        // vote per 4 channels), the split form otherwise (see tame_scale)
        float sxv[TM];
        bool rows_tame = true;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            sxv[i] = sa[min(mw0 + i * 32 + frag_row, M - 1)];
            rows_tame = rows_tame && tame_scale(sxv[i]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = min(nw0 + j * 32 + 8 * g + 4 * half, N - 4);
                const float4 w = *reinterpret_cast<const float4 *>(sb + n);
                float4 bv = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                if (ADDMM && am.bias) bv = *reinterpret_cast<const float4 *>(am.bias + n);
                const bool cheap = wave_all(rows_tame && tame_scale(w.x) && tame_scale(w.y) &&
                                            tame_scale(w.z) && tame_scale(w.w));
#pragma unroll
                for (int i = 0; i < TM; ++i) {
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
                    const uint32_t lo = pack_bf16x2(addmm<ADDMM>(v[0], am, bv.x), addmm<ADDMM>(v[1], am, bv.y));
                    const uint32_t hi = pack_bf16x2(addmm<ADDMM>(v[2], am, bv.z), addmm<ADDMM>(v[3], am, bv.w));
                    const int chunk = (j * 4 + g) ^ (ml & PM);
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
            const uint4 v = st16[ml * CH + (cc ^ (ml & PM))];
            if (m < M && n < N)
                store16_nt(static_cast<__bf16 *>(out) + (int64_t)m * N + n, v);
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int CPR, int OCC, bool KTAIL>
void launch_tail(const int8_t *xq, const float *xs, int M, const int8_t *wq, const float *ws,
                 int N, int K, void *out, bool out_i32, hipStream_t stream, const Addmm *am) {
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    const dim3 grid((unsigned)(tiles_m * tiles_n)), block(kThreads);
    const Addmm a = am ? *am : Addmm{nullptr, 1.0f, 0.0f};
    if (out_i32)
        gemm_tiled_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, CPR, OCC, KTAIL, true, false>
            <<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, tiles_m, tiles_n, a);
    else if (am)
        gemm_tiled_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, CPR, OCC, KTAIL, false, true>
            <<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, tiles_m, tiles_n, a);
    else
        gemm_tiled_kernel<BM, BN, WAVES_M, WAVES_N, STAGES, CPR, OCC, KTAIL, false, false>
            <<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, tiles_m, tiles_n, a);
}

// K not a multiple of the stage depth takes the variant that zeroes the
// chunks past K.
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES, int CPR = 8, int OCC = 1>
hipError_t launch_cfg(const int8_t *xq, const float *xs, int M, const int8_t *wq, const float *ws,
                      int N, int K, void *out, bool out_i32, hipStream_t stream, const Addmm *am) {
    if (K % (16 * CPR) == 0)
        launch_tail<BM, BN, WAVES_M, WAVES_N, STAGES, CPR, OCC, false>(xq, xs, M, wq, ws, N, K, out,
                                                                       out_i32, stream, am);
    else
        launch_tail<BM, BN, WAVES_M, WAVES_N, STAGES, CPR, OCC, true>(xq, xs, M, wq, ws, N, K, out,
                                                                      out_i32, stream, am);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_decode(const int8_t *xq, const float *xs, int M, const int8_t *wq,
                              const float *ws, int N, int K, void *out, bool out_i32,
                              hipStream_t stream, const Addmm *am);

hipError_t launch_gemm(const int8_t *xq, const float *xs, int M, const int8_t *wq, const float *ws,
                       int N, int K, void *out, bool out_i32, hipStream_t stream, const Addmm *am) {
    if (M <= 64) return launch_gemm_decode(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
    // Many tiles (enough 256x256 ones to fill 256 CUs four times over): with
    // K up to 1024, two 256x128 workgroups per CU (64-byte K stages, 72 KB of
    // LDS and at most 256 registers each), so that one tile's prologue and
    // epilogue run beside the other's MFMAs; with longer K, 256x256 tiles,
    // which halve the LDS traffic per MFMA. Otherwise 256x128 (or 128x128)
    // tiles, one workgroup per CU.
    const long t256 = (long)((M + 255) / 256) * ((N + 255) / 256);
    const long t128 = (long)((M + 255) / 256) * ((N + 127) / 128);
    if (t256 >= 4 * 256 && K <= 1024)
        return launch_cfg<256, 128, 2, 2, 3, 4, 2>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
    if (t256 >= 4 * 256) return launch_cfg<256, 256, 2, 2, 2>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
    if (t128 >= 256) return launch_cfg<256, 128, 2, 2, 3>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
    return launch_cfg<128, 128, 2, 2, 2>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
}

}  // namespace w8a8
