// Weight-streaming int8 GEMM for small M (M <= 64, decode-sized batches).
//
// At M = 16 every W byte is used for just 16 multiply-adds, so the kernel is
// bound by reading W [N,K] from HBM once (pytorch/ao PR #153 notes that fused
// dequant GEMMs aimed at compute-bound M > 16 do not serve this memory-bound
// inference case). Shape of the kernel:
//  - one workgroup per 16 output channels; its KSPLIT wavefronts (2, 4 or 8 by
//    the number of 16-row blocks) split K, so
//    every wavefront issues all of its 16-byte W loads up front and the whole
//    weight matrix is in flight at once across the chip;
//  - v_mfma_i32_16x16x64_i8: lane l holds W row (l % 16) and activation row
//    (l % 16) of each 16-row block, 16 bytes of K at offset 16 * (l / 16) of
//    every 64-byte K step, for both operands;
//  - the K-split partial int32 tiles are summed in LDS (never in HBM), then
//    scaled, rounded to bf16 and stored: the same fused epilogue as the tiled
//    kernel.
// For M <= 16 and K >= 3072 (the decode shapes) gemm_decode_lds_kernel below
// takes over: the same split and epilogue, with both operands moved global ->
// LDS in whole cache lines. The register kernel serves the rest of M <= 64.
//
// The single-launch linear (linear_decode_kernel) is the same kernel with the
// activation quantization moved into its prologue (pytorch/ao PR #821 asks for
// scaling inside the kernel), so no intermediate codes or scales leave the
// chip. Each lane loads the bf16 activations of exactly the fragment
// positions it multiplies, before its weight loads: vector loads return in
// order, so the row absmax, its reduction across the workgroup (shuffles, then
// LDS) and the quantization run while the weight bytes are still on their way
// from HBM. Every workgroup quantizes all M rows itself (the rows are L2 hits
// after the first), with the arithmetic of quant_math.hpp, so its codes and
// scales are the ones w8a8_quantize_rows writes. That redundancy is the cost:
// each CU runs about eight vector instructions for each of the M * K
// activations, which at M = 16, K = N = 4096 takes longer than the separate
// quantize launch it replaces.
#include "launch.hpp"
#include "quant_math.hpp"

namespace w8a8 {
namespace {


// kSteps: K steps (64 bytes each) whose loads a wavefront issues together.
template <int MT, int KSPLIT, bool OUT_I32, bool ADDMM, int kSteps>
__global__ __launch_bounds__(KSPLIT *kWave) void gemm_decode_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ sa, const int8_t *__restrict__ B,
    const float *__restrict__ sb, void *__restrict__ out, int M, int N, int K,
    int steps_per_wave, Addmm am) {
    __shared__ int red[KSPLIT][MT][4][kWave];
    lds_poison(red);
    lds_poison_done();

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int n0 = blockIdx.x * 16;
    const int r16 = lane & 15, kgrp = lane >> 4;
    const int8_t *brow = B + (int64_t)(n0 + r16) * K + kgrp * 16;
    const int8_t *arow[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) arow[mb] = A + (int64_t)min(mb * 16 + r16, M - 1) * K + kgrp * 16;

    v4i acc[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) acc[mb] = v4i{};

    // the epilogue's scales (and bias) for this thread's outputs, loaded
    // before the weights: they land with them instead of costing one more
    // memory round trip after the reduction
    constexpr int kThreadsWg = KSPLIT * kWave;
    constexpr int EPT = (MT * 256 + kThreadsWg - 1) / kThreadsWg;  // outputs per thread
    float esx[EPT], esw[EPT], ebias[EPT];
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = min((int)threadIdx.x + q * kThreadsWg, MT * 256 - 1);
        const int m = min((e >> 8) * 16 + ((e >> 4) & 15), M - 1), n = n0 + (e & 15);
        esx[q] = OUT_I32 ? 0.0f : sa[m];
        esw[q] = OUT_I32 ? 0.0f : sb[n];
        ebias[q] = ADDMM && am.bias ? am.bias[n] : 0.0f;
    }

    const int total_steps = (K + 63) / 64;
    const int s_begin = wave * steps_per_wave;
    const int s_end = min(s_begin + steps_per_wave, total_steps);
    const v4i zero = v4i{};
    for (int s = s_begin; s < s_end; s += kSteps) {
        v4i b[kSteps], a[MT][kSteps];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int k = (s + u) * 64;
            const bool ok = (s + u < s_end) && (k + kgrp * 16 < K);
            b[u] = ok ? __builtin_bit_cast(v4i, load16_stream(brow + k)) : zero;
#pragma unroll
            for (int mb = 0; mb < MT; ++mb) a[mb][u] = ok ? *reinterpret_cast<const v4i *>(arow[mb] + k) : zero;
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u)
#pragma unroll
            for (int mb = 0; mb < MT; ++mb) acc[mb] = mfma_16x16x64(a[mb][u], b[u], acc[mb]);
    }

#pragma unroll
    for (int mb = 0; mb < MT; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][mb][r][lane] = acc[mb][r];
    __syncthreads();

    // one output element per thread: row i, column j of 16x16 tile mb sits in
    // lane j + 16 * (i / 4), element i % 4
#pragma unroll
    for (int q = 0; q < EPT; ++q) {
        const int e = (int)threadIdx.x + q * kThreadsWg;
        if (e >= MT * 256) continue;
        const int mb = e >> 8, i = (e >> 4) & 15, j = e & 15;
        const int m = mb * 16 + i;
        if (m >= M) continue;
        const int l = j + 16 * (i >> 2), r = i & 3;
        int sum = 0;
#pragma unroll
        for (int w = 0; w < KSPLIT; ++w) sum += red[w][mb][r][l];
        const int n = n0 + j;
        if constexpr (OUT_I32) {
            static_cast<int32_t *>(out)[(int64_t)m * N + n] = sum;
        } else {
            const float v =
                addmm<ADDMM>(dequant(sum, split_scale(esx[q]), split_scale(esw[q])), am, ebias[q]);
            static_cast<__bf16 *>(out)[(int64_t)m * N + n] = (__bf16)v;
        }
    }
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// s_waitcnt on the vector-memory counter only
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Weight-streaming kernel for M <= 16 with both operands moved global -> LDS by
// 16-byte direct-to-LDS loads (the path that moves about twice the bytes per
// CU of loads into registers). One workgroup per 16 output channels; its
// WAVES wavefronts split every 4096-byte K block into slices of 4096 / WAVES
// bytes. A wavefront issues all loads of its slice at once (activations first
// within each 128-byte K pair, so they land with the weights), then waits for
// them pair by pair (vector loads complete in order) and multiplies each pair
// as soon as it is in LDS.
//
// Load geometry: one load instruction fills 64 consecutive 16-byte LDS slots
// with 8 rows x 128 bytes of K, i.e. 8 whole cache lines (the register-path
// kernel's loads touched 16 half lines; reading the 16.8 MB decode weight that
// way takes 4.57 us against 3.93 us in whole lines). Slot i of load (pair p,
// half h) holds row 8h + i/8, logical chunk (i % 8) ^ (i / 8) ^ h of the pair,
// so the
// MFMA fragment read of one K step (lane l: row l % 16, chunk 4t + l / 16)
// touches 16 distinct 16-byte bank groups per 16 lanes. Each wavefront only
// ever touches its own LDS region, so the mainloop needs no barrier.
//
// Chunks past K are read from a clamped address (every load stays in bounds
// and is always issued, so the counted waits hold) and their activation
// fragments are zeroed before the MFMA.
template <int WAVES, bool OUT_I32, bool ADDMM>
__global__ __launch_bounds__(WAVES *kWave) void gemm_decode_lds_kernel(
    const int8_t *__restrict__ A, const float *__restrict__ sa, const int8_t *__restrict__ B,
    const float *__restrict__ sb, void *__restrict__ out, int M, int N, int K, Addmm am) {
    constexpr int kBlock = 4096;                 // K bytes per block, all wavefronts
    constexpr int kSlice = kBlock / WAVES;       // K bytes per wavefront per block
    constexpr int kPairs = kSlice / 128;         // 128-byte K pairs per slice
    constexpr int kLoads = 4 * kPairs;           // X and W, two halves each
    static_assert(kPairs >= 1 && kLoads < 64, "vmcnt range");
    static_assert(kPairs <= 8, "at most 8 pairs per slice");
    // One LDS array per pair position (unused positions one slot): the
    // compiler then knows which direct-to-LDS loads a fragment read may depend
    // on and waits for those only; with a single array it waits for every
    // load in flight before the first read, so no pair could be multiplied
    // while later ones were still arriving. Pair p of wavefront w holds X
    // halves at 256 w + 64 h and W halves at 256 w + 128 + 64 h.
    constexpr int kPairSlots = WAVES * 4 * kWave;
    constexpr int kP1 = kPairs > 1 ? kPairSlots : 1, kP2 = kPairs > 2 ? kPairSlots : 1;
    constexpr int kP3 = kPairs > 3 ? kPairSlots : 1, kP4 = kPairs > 4 ? kPairSlots : 1;
    constexpr int kP5 = kPairs > 5 ? kPairSlots : 1, kP6 = kPairs > 6 ? kPairSlots : 1;
    constexpr int kP7 = kPairs > 7 ? kPairSlots : 1;
    __shared__ uint4 q0[kPairSlots], q1[kP1], q2[kP2], q3[kP3], q4[kP4], q5[kP5], q6[kP6], q7[kP7];
    __shared__ v4i red[WAVES][kWave];
    lds_poison(q0);
    lds_poison(q1);
    lds_poison(q2);
    lds_poison(q3);
    lds_poison(q4);
    lds_poison(q5);
    lds_poison(q6);
    lds_poison(q7);
    lds_poison(red);
    lds_poison_done();

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int n0 = blockIdx.x * 16;

    // the epilogue's scales (and bias), in flight with the loads
    const int e = threadIdx.x & 255;
    const int em = e >> 4, en = n0 + (e & 15);
    const float esx = OUT_I32 ? 0.0f : sa[min(em, M - 1)];
    const float esw = OUT_I32 ? 0.0f : sb[en];
    const float ebias = ADDMM && am.bias ? am.bias[en] : 0.0f;

    // this lane's rows and chunks for the two halves of every load
    const int lr = lane >> 3, lc = lane & 7;
    const int8_t *xrow[2], *wrow[2];
    int cb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 8 * h + lr;
        cb[h] = 16 * (lc ^ lr ^ h);
        xrow[h] = A + (int64_t)min(row, M - 1) * K;
        wrow[h] = B + (int64_t)(n0 + row) * K;
    }
    uint4 *const qs[8] = {q0, q1, q2, q3, q4, q5, q6, q7};
    uint4 *pr[kPairs];  // this wavefront's slots of pair p
#pragma unroll
    for (int p = 0; p < kPairs; ++p) pr[p] = qs[p] + 256 * wave;

    // fragment reads: lane l takes row l % 16, chunk 4t + l / 16 of K step t
    // of a pair
    const int fr = lane & 15, fg = lane >> 4, fh = fr >> 3, frr = fr & 7;
    v4i acc = v4i{};
    for (int k0 = 0; k0 < K; k0 += kBlock) {
        const int ks = k0 + wave * kSlice;
#pragma unroll
        for (int p = 0; p < kPairs; ++p) {
            const int kp = ks + 128 * p;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                __builtin_amdgcn_global_load_lds((global_void *)(xrow[h] + min(kp + cb[h], K - 16)),
                                                 (lds_void *)(pr[p] + 64 * h), 16, 0, 0);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                __builtin_amdgcn_global_load_lds((global_void *)(wrow[h] + min(kp + cb[h], K - 16)),
                                                 (lds_void *)(pr[p] + 128 + 64 * h), 16, 0,
                                                 kLdsLoadStream);
        }
#pragma unroll
        for (int p = 0; p < kPairs; ++p) {
            if (p == 0) wait_vm<4 * (kPairs - 1)>();
            else if (p == 1) wait_vm<(kPairs > 1 ? 4 * (kPairs - 2) : 0)>();
            else if (p == 2) wait_vm<(kPairs > 2 ? 4 * (kPairs - 3) : 0)>();
            else if (p == 3) wait_vm<(kPairs > 3 ? 4 * (kPairs - 4) : 0)>();
            else if (p == 4) wait_vm<(kPairs > 4 ? 4 * (kPairs - 5) : 0)>();
            else if (p == 5) wait_vm<(kPairs > 5 ? 4 * (kPairs - 6) : 0)>();
            else if (p == 6) wait_vm<(kPairs > 6 ? 4 * (kPairs - 7) : 0)>();
            else wait_vm<0>();
            asm volatile("" ::: "memory");
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int c = 4 * t + fg;
                const int slot = fh * kWave + 8 * frr + (c ^ frr ^ fh);
                v4i a = __builtin_bit_cast(v4i, pr[p][slot]);
                const v4i b = __builtin_bit_cast(v4i, pr[p][128 + slot]);
                if (ks + 128 * p + 16 * c >= K) a = v4i{};
                acc = mfma_16x16x64(a, b, acc);
            }
        }
        // every fragment of this block has been read (the MFMAs consumed
        // them) before the next block's loads refill the region
    }

    red[wave][lane] = acc;
    __syncthreads();
    if (threadIdx.x >= 256) return;
    // output (row i, channel j) sits in lane j + 16 * (i / 4), element i % 4
    const int i = em, j = e & 15;
    if (i >= M) return;
    const int l = j + 16 * (i >> 2), r = i & 3;
    int sum = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[w][l][r];
    if constexpr (OUT_I32) {
        static_cast<int32_t *>(out)[(int64_t)i * N + en] = sum;
    } else {
        const float v = addmm<ADDMM>(dequant(sum, split_scale(esx), split_scale(esw)), am, ebias);
        static_cast<__bf16 *>(out)[(int64_t)i * N + en] = (__bf16)v;
    }
}

constexpr int kLinSplit = 8;  // wavefronts per workgroup (K split) of the fused linear

template <int MT, int U, bool ADDMM>
__global__ __launch_bounds__(kLinSplit *kWave) void linear_decode_kernel(
    const uint16_t *__restrict__ X, const int8_t *__restrict__ B, const float *__restrict__ sb,
    __bf16 *__restrict__ out, int M, int N, int K, int steps_per_wave, Addmm am) {
    __shared__ int red[kLinSplit][MT][4][kWave];
    __shared__ uint32_t red_amax[kLinSplit][MT * 16];
    __shared__ float row_s[MT * 16];
    lds_poison(red);
    lds_poison(red_amax);
    lds_poison(row_s);
    lds_poison_done();

    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int n0 = blockIdx.x * 16;
    const int r16 = lane & 15, kgrp = lane >> 4;
    const int8_t *brow = B + (int64_t)(n0 + r16) * K;
    const uint16_t *xrow[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) xrow[mb] = X + (int64_t)min(mb * 16 + r16, M - 1) * K;

    const int total_steps = (K + 63) / 64;
    const int s_begin = wave * steps_per_wave;
    const int s_end = min(s_begin + steps_per_wave, total_steps);
    const int nchunk = s_end > s_begin ? (s_end - s_begin + U - 1) / U : 0;  // uniform

    // K step s: this lane's 16 elements start at s * 64 + 16 * kgrp; past K
    // (or past the wavefront's steps) the activations count as zeros. Loads
    // always read in bounds (offset clamped into the row) so they stay
    // unconditional 16-byte loads, issued before anything waits on them. A
    // clamped activation is an element of the same row, so it leaves the
    // absmax unchanged; the activation codes of such steps are zeroed before
    // the MFMA, which also cancels whatever weight bytes the clamped load
    // returned.
    auto k_ok = [&](int s) { return s < s_end && s * 64 + kgrp * 16 < K; };
    auto k_off = [&](int s) { return min(s * 64 + kgrp * 16, K - 16); };
    v4i xr[MT][U][2];
    v4i b[U];
    auto load_chunk = [&](int s) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int mb = 0; mb < MT; ++mb)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    xr[mb][u][h] = *reinterpret_cast<const v4i *>(xrow[mb] + k_off(s + u) + 8 * h);
        __builtin_amdgcn_sched_barrier(0);  // activations first, then weights
#pragma unroll
        for (int u = 0; u < U; ++u) b[u] = __builtin_bit_cast(v4i, load16_stream(brow + k_off(s + u)));
        __builtin_amdgcn_sched_barrier(0);  // all issued before anything waits on them
    };

    // row absmax over this lane's positions; a wavefront with more than one
    // chunk of K steps reads its later chunks here once more, absmax only
    uint32_t amax[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) amax[mb] = 0;
    if (nchunk > 0) {
        load_chunk(s_begin);
#pragma unroll
        for (int mb = 0; mb < MT; ++mb)
#pragma unroll
            for (int u = 0; u < U; ++u) {
                absmax8(__builtin_bit_cast(uint4, xr[mb][u][0]), amax[mb]);
                absmax8(__builtin_bit_cast(uint4, xr[mb][u][1]), amax[mb]);
            }
        for (int c = 1; c < nchunk; ++c) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int st = s_begin + c * U + u;
#pragma unroll
                for (int mb = 0; mb < MT; ++mb)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        absmax8(*reinterpret_cast<const uint4 *>(xrow[mb] + k_off(st) + 8 * h),
                                amax[mb]);
            }
        }
    }
    // lanes r16, r16 + 16, r16 + 32, r16 + 48 share a row; then the wavefronts
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) {
        amax[mb] = max(amax[mb], (uint32_t)__shfl_xor((int)amax[mb], 16, kWave));
        amax[mb] = max(amax[mb], (uint32_t)__shfl_xor((int)amax[mb], 32, kWave));
        if (lane < 16) red_amax[wave][mb * 16 + lane] = amax[mb];
    }
    __syncthreads();
    RowScale rs[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) {
        uint32_t a = 0;
#pragma unroll
        for (int w = 0; w < kLinSplit; ++w) a = max(a, red_amax[w][mb * 16 + r16]);
        rs[mb] = row_scale(__uint_as_float(a));
        if (wave == 0 && lane < 16) row_s[mb * 16 + lane] = rs[mb].s;
    }

    v4i acc[MT];
#pragma unroll
    for (int mb = 0; mb < MT; ++mb) acc[mb] = v4i{};
    for (int c = 0; c < nchunk; ++c) {
        if (c > 0) load_chunk(s_begin + c * U);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool ok = k_ok(s_begin + c * U + u);
#pragma unroll
            for (int mb = 0; mb < MT; ++mb) {
                float v[8];
                widen8(__builtin_bit_cast(uint4, xr[mb][u][0]), v);
                const uint2 q0 = quantize8(v, rs[mb]);
                widen8(__builtin_bit_cast(uint4, xr[mb][u][1]), v);
                const uint2 q1 = quantize8(v, rs[mb]);
                const v4i a = {(int)q0.x, (int)q0.y, (int)q1.x, (int)q1.y};
                acc[mb] = mfma_16x16x64(ok ? a : v4i{}, b[u], acc[mb]);
            }
        }
    }

#pragma unroll
    for (int mb = 0; mb < MT; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][mb][r][lane] = acc[mb][r];
    __syncthreads();

    for (int e = threadIdx.x; e < MT * 256; e += kLinSplit * kWave) {
        const int mb = e >> 8, i = (e >> 4) & 15, j = e & 15;
        const int m = mb * 16 + i;
        if (m >= M) continue;
        const int l = j + 16 * (i >> 2), r = i & 3;
        int sum = 0;
#pragma unroll
        for (int w = 0; w < kLinSplit; ++w) sum += red[w][mb][r][l];
        const int n = n0 + j;
        const float v =
            addmm<ADDMM>(dequant(sum, split_scale(row_s[m]), split_scale(sb[n])), am,
                         ADDMM && am.bias ? am.bias[n] : 0.0f);
        out[(int64_t)m * N + n] = (__bf16)v;
    }
}

template <int MT>
hipError_t launch_linear_mt(const uint16_t *x, int M, const int8_t *wq, const float *ws, int N,
                            int K, void *out, hipStream_t stream, const Addmm &am) {
    // K steps per chunk: a lane holds MT * U * 32 activation bytes while the
    // chunk's weights are in flight (64 registers), so M <= 16 covers K = 4096
    // in one chunk; more row blocks take shorter chunks (no register spills)
    constexpr int U = MT == 1 ? 8 : MT == 2 ? 4 : 2;
    const int total_steps = (K + 63) / 64;
    const int steps_per_wave = (total_steps + kLinSplit - 1) / kLinSplit;
    const dim3 grid((unsigned)(N / 16)), block(kLinSplit * kWave);
    __bf16 *o = static_cast<__bf16 *>(out);
    if (am.bias || am.alpha != 1.0f)
        linear_decode_kernel<MT, U, true>
            <<<grid, block, 0, stream>>>(x, wq, ws, o, M, N, K, steps_per_wave, am);
    else
        linear_decode_kernel<MT, U, false>
            <<<grid, block, 0, stream>>>(x, wq, ws, o, M, N, K, steps_per_wave, am);
    return hipGetLastError();
}

// Wavefronts per workgroup (the K split) and K steps per load batch, by row
// blocks. Fewer, longer wavefronts keep the same bytes in flight and are all
// dispatched sooner (M = 16, K = N = 4096: 2 x 32 runs 6.6 us, 4 x 16 6.8 us,
// 8 x 8 7.25 us; M = 17: 4 x 16 7.45 us against 7.7 us); more row blocks need
// the registers for their activations.
template <int MT> struct DecodeShape { static constexpr int split = 8, steps = 8; };
template <> struct DecodeShape<1> { static constexpr int split = 2, steps = 32; };
template <> struct DecodeShape<2> { static constexpr int split = 4, steps = 16; };

template <int MT, int KSPLIT, int STEPS>
hipError_t launch_shape(const int8_t *xq, const float *xs, int M, const int8_t *wq,
                        const float *ws, int N, int K, void *out, bool out_i32,
                        hipStream_t stream, const Addmm *am) {
    const int total_steps = (K + 63) / 64;
    const int steps_per_wave = (total_steps + KSPLIT - 1) / KSPLIT;
    const dim3 grid((unsigned)(N / 16)), block(KSPLIT * kWave);
    const Addmm a = am ? *am : Addmm{nullptr, 1.0f, 0.0f};
    if (out_i32)
        gemm_decode_kernel<MT, KSPLIT, true, false, STEPS>
            <<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, steps_per_wave, a);
    else if (am)
        gemm_decode_kernel<MT, KSPLIT, false, true, STEPS>
            <<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, steps_per_wave, a);
    else
        gemm_decode_kernel<MT, KSPLIT, false, false, STEPS>
            <<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, steps_per_wave, a);
    return hipGetLastError();
}

// The long shapes only when K fills their batches (K >= 4096): with short K
// most of a long batch would be masked steps (K = 256, M = 16: 3.75 us against
// 2.1 us for 8 x 8).
template <int MT>
hipError_t launch_mt(const int8_t *xq, const float *xs, int M, const int8_t *wq, const float *ws,
                     int N, int K, void *out, bool out_i32, hipStream_t stream, const Addmm *am) {
    constexpr int KSPLIT = DecodeShape<MT>::split, STEPS = DecodeShape<MT>::steps;
    if constexpr (KSPLIT != 8) {
        if ((K + 63) / 64 < KSPLIT * STEPS)
            return launch_shape<MT, 8, 8>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
    }
    return launch_shape<MT, KSPLIT, STEPS>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
}

}  // namespace

hipError_t launch_linear_decode(const uint16_t *x, int M, const int8_t *wq, const float *ws, int N,
                                int K, void *out, hipStream_t stream, const Addmm &am) {
    switch ((M + 15) / 16) {
        case 1: return launch_linear_mt<1>(x, M, wq, ws, N, K, out, stream, am);
        case 2: return launch_linear_mt<2>(x, M, wq, ws, N, K, out, stream, am);
        case 3: return launch_linear_mt<3>(x, M, wq, ws, N, K, out, stream, am);
        default: return launch_linear_mt<4>(x, M, wq, ws, N, K, out, stream, am);
    }
}

template <int WAVES>
hipError_t launch_lds(const int8_t *xq, const float *xs, int M, const int8_t *wq, const float *ws,
                      int N, int K, void *out, bool out_i32, hipStream_t stream, const Addmm *am) {
    const dim3 grid((unsigned)(N / 16)), block(WAVES * kWave);
    const Addmm a = am ? *am : Addmm{nullptr, 1.0f, 0.0f};
    if (out_i32)
        gemm_decode_lds_kernel<WAVES, true, false><<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, a);
    else if (am)
        gemm_decode_lds_kernel<WAVES, false, true><<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, a);
    else
        gemm_decode_lds_kernel<WAVES, false, false><<<grid, block, 0, stream>>>(xq, xs, wq, ws, out, M, N, K, a);
    return hipGetLastError();
}

// M <= 16 with K >= 3072: both operands through LDS, 4 wavefronts up to one
// 4096-byte block and 16 beyond (K = N = 4096, M = 16: 5.15 us against 6.7 us
// for the register-path kernel; M = 1: 4.6 against 5.3 us, although every
// activation row slot then repeats row 0; K = 8192: 8.7 against 11.4 us). A
// ragged last block is masked and still wins (K = 11008: 11.8 against 16.1 us,
// K = 5120: 7.35 against 9.9 us, K = 3072: 5.0 against 6.2 us); below 3072 the
// masked part of the block costs more than the LDS path saves (K = 1024: 3.9
// against 3.5 us), so short K keeps the register path.
hipError_t launch_gemm_decode(const int8_t *xq, const float *xs, int M, const int8_t *wq,
                              const float *ws, int N, int K, void *out, bool out_i32,
                              hipStream_t stream, const Addmm *am) {
    if (M <= 16 && K >= 3072) {
        if (K <= 4096) return launch_lds<4>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
        return launch_lds<16>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
    }
    switch ((M + 15) / 16) {
        case 1: return launch_mt<1>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
        case 2: return launch_mt<2>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
        case 3: return launch_mt<3>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
        default: return launch_mt<4>(xq, xs, M, wq, ws, N, K, out, out_i32, stream, am);
    }
}

}  // namespace w8a8
