/*
 * w8a8.h -- C ABI of libw8a8.so, the dynamically quantized int8 linear layer
 * (W8A8) for AMD Instinct MI355X (gfx950).
 *
 *   out[M,N] (bf16) = bf16( (sum_k xq[m,k] * wq[n,k]) * x_scale[m] * w_scale[n] )
 *   with xq, x_scale = quantize_rows(X) computed at run time.
 *
 * The layer follows the pages it was designed from:
 *  - activations are quantized dynamically, per row, with no calibration
 *    ("int8 dynamicquant", pytorch/ao PR #821; dynamic scaling in the vLLM
 *    csrc/quantization log);
 *  - a scale is the row absmax divided by 127 in binary32 (Paddle sparse_fc
 *    PR #41770, spmm_plugin.cu weight-scale hunk), values are divided by it,
 *    rounded half to even and clamped to [-127,127] before the cast (clamp
 *    commit in the vLLM log);
 *  - weights arrive already quantized, one fp32 scale per output channel, and
 *    are owned by the caller (the same Paddle PR asks for int8 weights with the
 *    model's own scale, channel-wise scale vectors, and no plugin-owned weight
 *    memory so that weights can be shared);
 *  - the product accumulates in int32 and the dequantization is fused into the
 *    GEMM so the int32 matrix never reaches memory, with bf16 output to keep
 *    small outputs (pytorch/ao PR #821: i8i8 -> bf16 change, the int32
 *    materialization and fused-dequant paragraphs, the int32/bf16 out_dtype
 *    thread);
 *  - int8 operands are K-contiguous on both sides, A row-major and B given as
 *    [N,K] (triton issue #634, layout answer and the 1.44 ms -> 0.286 ms fix);
 *  - block sparsity is passed as raw crow/col/values arrays with 64x64 blocks
 *    (pytorch/ao PR #821: custom-op paragraph, bsr_dense_addmm warning).
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing, keeps no state between calls (except the thread-local
 *    last HIP error) and is reentrant.
 *  - Work is enqueued on `stream` (a hipStream_t passed as void *, so the
 *    header needs no HIP include; NULL = the default stream) and the call
 *    returns without synchronizing. Outputs are valid once the stream reaches
 *    that point.
 *  - Arguments are validated on the host before any HIP call; a failed check
 *    returns its code and launches nothing. M == 0 is a valid empty call that
 *    launches nothing (pointers sized by M may then be NULL).
 *  - Base pointers must be 16-byte aligned (W8A8_ERR_ALIGN).
 *  - K must be a positive multiple of 16 and at most W8A8_MAX_K, so that
 *    128*128*K < 2^31 and int32 accumulation is exact for any int8 operands,
 *    -128 included (pytorch/ao PR #821, the 2**31 / 2**14 headroom remark:
 *    2^14 is the largest product of two int8 values) (W8A8_ERR_SHAPE /
 *    W8A8_ERR_K_OVERFLOW).
 *  - A launch failure returns W8A8_ERR_HIP; w8a8_last_hip_error() then gives
 *    the hipError_t.
 */
#ifndef W8A8_H
#define W8A8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W8A8_OK = 0,
    W8A8_ERR_NULL = -1,       /* a required pointer is NULL */
    W8A8_ERR_SHAPE = -2,      /* a size is out of range or not a required multiple */
    W8A8_ERR_ALIGN = -3,      /* a base pointer is not 16-byte aligned */
    W8A8_ERR_K_OVERFLOW = -4, /* K > W8A8_MAX_K: int32 accumulation could overflow */
    W8A8_ERR_BLOCKSIZE = -5,  /* BSR block size other than 64 */
    W8A8_ERR_DTYPE = -6,      /* unknown output dtype selector */
    W8A8_ERR_HIP = -7,        /* the HIP runtime reported an error at launch */
    W8A8_ERR_VALUE = -8       /* a scalar argument (alpha, beta) is not finite */
} w8a8_status;

typedef enum {
    W8A8_OUT_BF16 = 0, /* out is bf16 [M,N]: the fused dequant epilogue */
    W8A8_OUT_I32 = 1   /* out is int32 [M,N]: raw accumulators, for exactness checks */
} w8a8_out_dtype;

/* Largest K with 128*128*K < 2^31 that is a multiple of 16: the int32 sum of
 * K products of int8 values cannot overflow, whatever the caller's codes
 * (quantize_rows itself never writes -128). */
#define W8A8_MAX_K 131056

/*
 * Dynamic per-row quantization of bf16 activations: the scale is the row
 * absmax over 127 in binary32 (Paddle sparse_fc PR #41770, spmm_plugin.cu
 * weight-scale hunk), computed per token at run time with no calibration
 * (pytorch/ao PR #821, "int8 dynamicquant"), and values are clamped before
 * the cast (vLLM csrc/quantization log, FP8 clamp commit).
 *   x_bf16  [M,K] bf16, row-major (read)
 *   xq      [M,K] int8, row-major (written): clamp(rint(fl32(x / s)), -127, 127)
 *   x_scale [M]   fp32 (written): s = fl32(max_k |x[m,k]| / 127); s = 0 and
 *           xq = 0 for an all-zero row. Division is IEEE binary32, rounding
 *           half to even, subnormals kept. Non-finite inputs are outside the
 *           domain (output unspecified).
 * Errors: NULL, SHAPE (M < 0, M > 2^31 - 1, K <= 0, K % 16), K_OVERFLOW, ALIGN, HIP.
 */
w8a8_status w8a8_quantize_rows(const void *x_bf16, int64_t M, int64_t K, int8_t *xq,
                               float *x_scale, void *stream);

/*
 * The same rule on fp32 rows: per-output-channel weight preparation, W [N,K]
 * fp32 -> wq [N,K] int8 + w_scale [N] (Paddle sparse_fc PR #41770, channel-wise
 * weight scale discussion). Arguments and errors as w8a8_quantize_rows, with
 * x an fp32 [M,K] row-major array.
 */
w8a8_status w8a8_quantize_rows_f32(const float *x, int64_t M, int64_t K, int8_t *xq,
                                   float *x_scale, void *stream);

/*
 * Dense W8A8 GEMM with the fused dequant epilogue: int8 x int8 products summed
 * in int32 (pytorch/ao PR #821, "triton dot accumulator uses int32"), scaled by
 * the row and channel scales and rounded to bf16 inside the kernel so the
 * int32 matrix never reaches memory (same PR: the fused-dequant paragraph and
 * the i8i8 -> bf16 change), both operands K-contiguous (triton issue #634,
 * layout answer).
 *   xq      [M,K] int8 row-major, x_scale [M] fp32   (from w8a8_quantize_rows)
 *   wq      [N,K] int8, K-contiguous (one row per output channel)
 *   w_scale [N]   fp32 per output channel
 *   out     [M,N] row-major: bf16 = bf16_rne(acc * x_scale[m] * w_scale[n]),
 *           or int32 acc when out_dtype == W8A8_OUT_I32.
 * The int32 accumulators stay on chip. M >= 0 (any value; M <= 64 takes a
 * weight-streaming path), N a positive multiple of 16.
 * Errors: NULL, SHAPE (M < 0, N <= 0, N % 16, K <= 0, K % 16), K_OVERFLOW,
 *         ALIGN, DTYPE, HIP.
 */
w8a8_status w8a8_gemm(const int8_t *xq, const float *x_scale, int64_t M, const int8_t *wq,
                      const float *w_scale, int64_t N, int64_t K, void *out,
                      w8a8_out_dtype out_dtype, void *stream);

/*
 * Dense W8A8 GEMM with an addmm epilogue (bf16 output):
 *   out[m,n] = bf16_rne(alpha * (acc * x_scale[m] * w_scale[n]) + beta * bias[n])
 * -- the beta / alpha of bsr_dense_addmm (pytorch/ao PR #821, the warning's
 * "beta=0 alpha=1"), with bias a per-output-channel fp32 vector [N] as in a
 * linear layer. bias may be NULL when beta == 0 (no bias term). The epilogue
 * runs in fp32 in the kernel (within 1 bf16 ulp plus a few fp32 ulps of the
 * two terms of the float64 definition). Other arguments as w8a8_gemm.
 * Errors: NULL (also bias NULL with beta != 0), SHAPE, K_OVERFLOW, ALIGN
 *         (bias included), VALUE (alpha or beta not finite), HIP.
 */
w8a8_status w8a8_gemm_addmm(const int8_t *xq, const float *x_scale, int64_t M, const int8_t *wq,
                            const float *w_scale, int64_t N, int64_t K, const float *bias,
                            float alpha, float beta, void *out, void *stream);

/* Largest M taken by w8a8_fused_linear. */
#define W8A8_FUSED_MAX_M 64

/*
 * Single-launch dynamically quantized linear layer for small batches
 * (decode): quantize_rows of x_bf16 fused into the GEMM, with the addmm
 * epilogue of w8a8_gemm_addmm:
 *   out[m,n] = bf16_rne(alpha * (acc * s[m] * w_scale[n]) + beta * bias[n]),
 *   acc = sum_k q[m,k] * wq[n,k], with q and s exactly as w8a8_quantize_rows
 *   computes them (the codes and scales are not written out).
 * One launch instead of quantize + GEMM, with no intermediate buffers: the
 * quantization is the scaling work that pytorch/ao PR #821 asks to move into
 * the kernel. Every workgroup of the kernel quantizes all of x, so on MI355X
 * it is slower than w8a8_quantize_rows followed by w8a8_gemm (at M = 16,
 * K = N = 4096: about 15 us against 11 us); it serves callers that cannot
 * hold the int8 codes and scales between two calls.
 *   x_bf16  [M,K] bf16 row-major, 0 <= M <= W8A8_FUSED_MAX_M
 *   wq, w_scale, bias, alpha, beta, out as for w8a8_gemm_addmm (bias NULL,
 *   alpha 1, beta 0: the plain fused dequant epilogue).
 * Larger M: w8a8_quantize_rows, then w8a8_gemm or w8a8_gemm_addmm.
 * Errors: NULL (also bias NULL with beta != 0), SHAPE (M > W8A8_FUSED_MAX_M
 *         and as w8a8_gemm), K_OVERFLOW, ALIGN, VALUE, HIP.
 */
w8a8_status w8a8_fused_linear(const void *x_bf16, int64_t M, int64_t K, const int8_t *wq,
                              const float *w_scale, int64_t N, const float *bias, float alpha,
                              float beta, void *out, void *stream);

/*
 * Block-sparse (BSR) W8A8 GEMM with the fused dequant epilogue: only stored
 * weight blocks are read and multiplied; output channels of block rows with
 * no stored block are written as +0. The weight is given as raw crow / col /
 * values arrays of 64x64 blocks (pytorch/ao PR #821: the custom-op paragraph
 * and the bsr_dense_addmm warning for 64x64 blocks), and the output is the
 * [M,N] layer output itself, with no transposed copy (same PR, the
 * ".t().contiguous()" suggestions).
 *   xq, x_scale as for w8a8_gemm ([M,K] int8, [M] fp32)
 *   crow    [N/bs + 1] int32: block row r owns blocks crow[r] .. crow[r+1]-1,
 *           crow[0] = 0, non-decreasing, crow[N/bs] = nnzb
 *   col     [nnzb] int32: block column of each stored block (< K/bs)
 *   values  [nnzb, bs, bs] int8: values[j][i][c] = W[r*bs + i, col[j]*bs + c]
 *           (each block row K-contiguous, like the dense [N,K] weight)
 *   w_scale [N] fp32 per output channel, out [M,N] as for w8a8_gemm.
 * bs must be 64; N and K positive multiples of 64; nnzb >= 0 (col and values
 * may be NULL when nnzb == 0). The bf16 epilogue is within one bf16 ulp for
 * every row scale and for channel scales that are 0 or in [2^-125, 2^97]
 * (w8a8_quantize_rows_f32 gives such scales for weight rows whose absmax lies
 * in [2^-118, 2^104]); outside that range an output may lose that bound. Malformed index arrays (out-of-range entries,
 * decreasing crow) give unspecified output values, but the kernel clamps every
 * index so it never reads outside the given arrays.
 * Errors: NULL, SHAPE, K_OVERFLOW, BLOCKSIZE, ALIGN, DTYPE, HIP.
 */
w8a8_status w8a8_bsr_gemm(const int8_t *xq, const float *x_scale, int64_t M, int64_t K,
                          const int32_t *crow, const int32_t *col, const int8_t *values,
                          int64_t nnzb, int64_t bs, const float *w_scale, int64_t N, void *out,
                          w8a8_out_dtype out_dtype, void *stream);

/*
 * Block-sparse (BSR) W8A8 GEMM with the addmm epilogue of w8a8_gemm_addmm
 * (bf16 output) -- bsr_dense_addmm's own form (pytorch/ao PR #821, the
 * warning's "beta=0 alpha=1"), here with any finite alpha and beta and a
 * per-output-channel fp32 bias [N]:
 *   out[m,n] = bf16_rne(alpha * (acc * x_scale[m] * w_scale[n]) + beta * bias[n])
 * Block rows with no stored block have acc = 0 and write bf16(beta * bias[n])
 * (+0 or -0 without a bias). bias may be NULL when beta == 0. Other arguments
 * as w8a8_bsr_gemm.
 * Errors: NULL (also bias NULL with beta != 0), SHAPE, K_OVERFLOW, BLOCKSIZE,
 *         ALIGN (bias included), VALUE (alpha or beta not finite), HIP.
 */
w8a8_status w8a8_bsr_gemm_addmm(const int8_t *xq, const float *x_scale, int64_t M, int64_t K,
                                const int32_t *crow, const int32_t *col, const int8_t *values,
                                int64_t nnzb, int64_t bs, const float *w_scale, int64_t N,
                                const float *bias, float alpha, float beta, void *out,
                                void *stream);

/*
 * 2:4 semi-structured weights (the pages' cuSPARSELt route: Paddle sparse_fc
 * PR #41770 runs FC weights already pruned to 2:4 -- at most two nonzeros in
 * every group of 4 consecutive weights along K -- and pytorch/ao PR #821 wants
 * that path with int8 dynamic quantization and i8i8 -> bf16 output). gfx950's
 * sparse MFMA multiplies such a weight stored compressed, at half the weight
 * bytes and twice the dense MFMA rate.
 *
 * Compression of an int8 weight wq [N,K] (K a positive multiple of 128):
 *   values [K/128, N, 64] int8 and meta [K/128, N, 4] uint32 (all device,
 *   caller-owned).
 * Each group of 4 keeps the positions p0 < p1 of its two largest |w| (equal
 * magnitudes in position order), so a weight that already is 2:4 is stored
 * exactly; other weights are pruned to that pattern. Within each 64-column
 * step s the 16 groups are listed in the order 0,1,2,3, 8,9,10,11, 4,5,6,7,
 * 12,13,14,15 (list position c holds group g = 16 s + order[c]); with block
 * B = s / 2 and e = s % 2:
 *   values[B][n][32 e + 2 c + t] = wq[n][4 g + p_t]          (t = 0, 1)
 *   meta[B][n][2 e + c / 8] bits 4 (c % 8) .. +3 = p0 | p1 << 2
 * (the lane layout of the sparse MFMA operand, so every fragment is one
 * contiguous load; block-major, so a tile of rows loads whole cache lines).
 * w_scale stays the per-channel scale of wq.
 * Errors: NULL, SHAPE (N < 0, K <= 0, K % 128), ALIGN, HIP.
 */
w8a8_status w8a8_compress24(const int8_t *wq, int64_t N, int64_t K, int8_t *values,
                            uint32_t *meta, void *stream);

/*
 * W8A8 GEMM on a compressed 2:4 weight, with the fused dequant epilogue:
 *   out[m,n] = bf16_rne(acc * x_scale[m] * w_scale[n]) (or int32 acc),
 *   acc = sum_k xq[m,k] * W[n,k], W the weight values/meta hold.
 * xq, x_scale, w_scale, out and out_dtype as for w8a8_gemm; values, meta from
 * w8a8_compress24. M >= 0 (M <= 64 takes a weight-streaming path, larger M an
 * LDS-tiled one), N a positive multiple of 16, K a positive multiple of 128.
 * Errors: NULL, SHAPE, K_OVERFLOW, ALIGN, DTYPE, HIP.
 */
w8a8_status w8a8_sparse24_gemm(const int8_t *xq, const float *x_scale, int64_t M,
                               const int8_t *values, const uint32_t *meta, const float *w_scale,
                               int64_t N, int64_t K, void *out, w8a8_out_dtype out_dtype,
                               void *stream);

/*
 * W4A16: asymmetric group-wise 4-bit weights with 16-bit activations
 * (pytorch/ao PR #153, fused HQQ quantization GEMM: u4 / s4 weights upcast to
 * bfloat16 or float16, scaled and shifted group-wise by scales and zero points
 * of that type along K, then the GEMM). x, scales, zeros, w and out share one
 * 16-bit format: W4A16_BF16 or W4A16_F16 (IEEE binary16); every rounding
 * below is to that format.
 *   wq4     [N, K/2] uint8: byte j of row n holds code c[n][2j] in its low
 *           nibble and c[n][2j+1] in its high nibble; q = c with
 *           W4A16_CODES_U4 (0..15), its 4-bit two's complement with
 *           W4A16_CODES_S4 (-8..7)
 *   scales, zeros [N, K/G] 16-bit values (bit patterns), G = group_size
 *   w[n][k] = bf16(bf16(q[n][k] - zeros[n][k/G]) * scales[n][k/G])
 *           (each operation rounded to nearest-even bf16, as elementwise bf16
 *           arithmetic does)
 * N a positive multiple of 16, K a positive multiple of 128, G a positive
 * multiple of 32 dividing K; wq4, x, w and out 16-byte aligned, scales and
 * zeros 2-byte aligned. An unknown codes or dtype value is W8A8_ERR_DTYPE.
 */
typedef enum {
    W4A16_CODES_U4 = 0, /* unsigned codes, q in 0..15 */
    W4A16_CODES_S4 = 1  /* signed codes, q in -8..7 (4-bit two's complement) */
} w4a16_codes;
typedef enum {
    W4A16_BF16 = 0, /* bfloat16 */
    W4A16_F16 = 1   /* IEEE binary16 (subnormals kept) */
} w4a16_dtype;

/* Dequantized weights: w [N,K], bit-exact to the definition above (the
 * standalone dequantization the pages list next to the fused kernel). */
w8a8_status w4a16_dequant(const uint8_t *wq4, const void *scales, const void *zeros, int64_t N,
                          int64_t K, int64_t group_size, w4a16_codes codes, w4a16_dtype dtype,
                          void *w, void *stream);

/*
 * Fused dequant GEMM: out[m][n] = round(sum_k x[m][k] * w[n][k]) with x
 * [M,K] row-major, out [M,N] row-major, the products accumulated in fp32
 * (within one ulp of the format plus the fp32 summation error of the exact
 * sum).
 * The dequantized weights never leave the chip. M >= 0: M <= 64 streams the
 * weights once (dequantized in registers); larger M takes LDS tiles, each
 * tile dequantizing its weight columns once for all of its rows.
 * Errors: NULL, SHAPE, ALIGN, DTYPE (codes, dtype), HIP.
 */
w8a8_status w4a16_gemm(const void *x, int64_t M, const uint8_t *wq4, const void *scales,
                       const void *zeros, int64_t N, int64_t K, int64_t group_size,
                       w4a16_codes codes, w4a16_dtype dtype, void *out, void *stream);

/* Static, human-readable text for a status code (never NULL). */
const char *w8a8_status_string(int status);

/* hipError_t value behind the calling thread's last W8A8_ERR_HIP (0 if none). */
int w8a8_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H */
