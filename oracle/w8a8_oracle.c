/*
 * CPU oracle for the dynamically quantized int8 linear layer (W8A8).
 *
 * TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct
 * definition that the GPU path is checked against. It shares no code, header,
 * table or helper with the HIP library; only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load it. The product path never
 * calls it.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (never -ffast-math,
 * so IEEE-754 binary32 division, round-to-nearest-even and subnormals hold).
 *
 * What it computes, with the passages it follows:
 *
 *   quantize (per row of X, per output channel of W):
 *     absmax = max_k |x[k]|            -- "int8 dynamicquant", pytorch/ao PR #821;
 *                                         absmax search in the Paddle
 *                                         sparse_fc PR #41770, spmm_plugin.cu
 *                                         weight-scale hunk
 *     s      = fl32(absmax / 127)      -- same hunk: the scale is the float
 *                                         quotient of the absmax by 127
 *     q[k]   = clamp(rint(fl32(x[k] / s)), -127, 127)
 *                                      -- clamp before the integer cast, vLLM
 *                                         csrc/quantization log (FP8 clamp
 *                                         commit); half-to-even rounding
 *     absmax == 0  =>  s = 0 and q = 0 (the pages are silent; plainest reading)
 *
 *   int8 GEMM:   acc[m,n] = sum_k xq[m,k] * wq[n,k] as an exact integer,
 *                which must fit int32 -- "triton dot accumulator uses int32",
 *                pytorch/ao PR #821; the 2**31 / 2**14 headroom remark in the
 *                same thread bounds K.
 *   epilogue:    out[m,n] = bf16_rne(acc * sx[m] * sw[n]) in float64, rounded
 *                once from float64 to bf16 -- "i8i8 -> bf16 matmul to
 *                maintain accuracy", pytorch/ao PR #821, Changes list.
 *   addmm epilogue: out[m,n] = bf16_rne(alpha * (acc * sx[m] * sw[n])
 *                + beta * bias[n]) in float64, one rounding to bf16 -- the
 *                beta / alpha of bsr_dense_addmm (pytorch/ao PR #821, the
 *                warning's "beta=0 alpha=1"), with the bias a per-channel
 *                vector as in a linear layer (the pages are silent on its
 *                shape; plainest reading).
 *   BSR:         the same sum taken only over the stored 64x64 blocks
 *                (crow_indices / col_indices / values), pytorch/ao PR #821
 *                custom-op paragraph and the bsr_dense_addmm warning (Ms=64,
 *                Ks=64, beta=0, alpha=1).
 *   W4A16:       asymmetric group-wise 4-bit weights with bf16 activations
 *                (pytorch/ao PR #153, fused HQQ quantization GEMM: u4 weights
 *                upcast to bf16, then group-wise scaling and shifting by the
 *                scales and zero points, then the GEMM; quantization along K).
 *                w[n,k] = bf16(bf16(q[n,k] - z[n,g]) * s[n,g]), g = k / G --
 *                the elementwise bf16 arithmetic of that dequantization, each
 *                operation rounded once to bf16 -- and
 *                out[m,n] = bf16_rne(sum_k x[m,k] * w[n,k]), the products exact
 *                and summed in float64, rounded once.
 *   2:4 weights: in every group of 4 consecutive weights along K at most two
 *                are kept -- the pages' cuSPARSELt route (Paddle PR #41770:
 *                sparse_fc on FC weights already pruned to 2:4, the
 *                "sparse_2_4" pass; pytorch/ao PR #821: the 2:4 path and its
 *                i8i8 -> bf16 output). The product is the dense int8 GEMM of
 *                the decompressed weight; the compressed storage is the
 *                library's own (see oracle_compress24).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bf16 is the top half of a binary32: widening is exact. */
static float bf16_bits_to_float(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* One row of the absmax/127 rule, on values already widened to float. */
static void quantize_one_row(const float *x, int64_t K, int8_t *q, float *s_out) {
    float absmax = 0.0f;
    for (int64_t k = 0; k < K; ++k) {
        float a = fabsf(x[k]);
        if (a > absmax) absmax = a;
    }
    float s = absmax / 127.0f; /* one correctly rounded binary32 division */
    *s_out = s;
    for (int64_t k = 0; k < K; ++k) {
        if (s == 0.0f) {
            q[k] = 0;
            continue;
        }
        float t = x[k] / s;  /* correctly rounded binary32 quotient */
        float r = rintf(t);  /* half to even (default rounding mode) */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[k] = (int8_t)r;
    }
}

/* X bf16 [M,K] row-major (raw bit patterns) -> q int8 [M,K], s fp32 [M]. */
void oracle_quantize_rows_bf16(const uint16_t *x, int64_t M, int64_t K, int8_t *q, float *s) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        float *row = (float *)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
        for (int64_t k = 0; k < K; ++k) row[k] = bf16_bits_to_float(x[m * K + k]);
        quantize_one_row(row, K, q + m * K, s + m);
        free(row);
    }
}

/* W fp32 [N,K] row-major -> q int8 [N,K], s fp32 [N] (per output channel). */
void oracle_quantize_rows_f32(const float *x, int64_t M, int64_t K, int8_t *q, float *s) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) quantize_one_row(x + m * K, K, q + m * K, s + m);
}

/*
 * acc[m,n] = sum_k xq[m,k] * wq[n,k], summed exactly in int64.
 * Returns 0, or -1 if any sum falls outside int32 (acc then holds garbage).
 */
int oracle_gemm_i32(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                    int32_t *acc) {
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k) sum += (int64_t)xq[m * K + k] * (int64_t)wq[n * K + k];
            if (sum > INT32_MAX || sum < INT32_MIN) bad = 1;
            acc[m * N + n] = (int32_t)sum;
        }
    }
    return bad ? -1 : 0;
}

/*
 * Round a float64 to the nearest bf16 (8 significant bits, binary32 exponent
 * range, subnormals kept), ties to even; returns the bf16 bit pattern.
 * v = n * quantum with quantum a power of two, so n is exact in float64 and
 * rounding n to an integer rounds v onto the bf16 grid.
 */
uint16_t oracle_bf16_rne_from_f64(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7F80);
    int e;
    (void)frexp(a, &e);          /* a in [2^(e-1), 2^e) */
    int unbiased = e - 1;
    if (unbiased < -126) unbiased = -126; /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, unbiased - 7);
    double n = a / quantum;      /* exact: division by a power of two */
    double r = nearbyint(n);     /* half to even */
    double rounded = r * quantum;
    if (rounded >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80); /* overflow */
    float f = (float)rounded;    /* exact: rounded is on the bf16 grid */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7FFF));
}

/*
 * Round a float64 to the nearest IEEE binary16 (11 significant bits, exponents
 * -14..15, subnormals kept), ties to even; returns the bit pattern. Values
 * that round to 2^16 or beyond overflow to infinity. Same construction as the
 * bf16 rounding above.
 */
uint16_t oracle_f16_rne_from_f64(double v) {
    if (isnan(v)) return 0x7E00;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return (uint16_t)(sign | 0x7C00);
    int e;
    (void)frexp(a, &e);          /* a in [2^(e-1), 2^e) */
    int unbiased = e - 1;
    if (unbiased < -14) unbiased = -14; /* subnormal range: fixed quantum 2^-24 */
    double quantum = ldexp(1.0, unbiased - 10);
    double r = nearbyint(a / quantum); /* exact division, half to even */
    double rounded = r * quantum;
    if (rounded >= 65536.0) return (uint16_t)(sign | 0x7C00);
    if (rounded < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)r); /* subnormal: r < 1024 */
    int e2;
    (void)frexp(rounded, &e2);
    const int E = e2 - 1;        /* rounded in [2^E, 2^(E+1)) */
    const uint16_t mant = (uint16_t)((rounded / ldexp(1.0, E) - 1.0) * 1024.0); /* exact */
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | mant);
}

/* binary16 bit pattern -> float64 (exact). */
static double f16_to_f64(uint16_t h) {
    const int ex = (h >> 10) & 31, mant = h & 1023;
    const double sg = (h & 0x8000) ? -1.0 : 1.0;
    if (ex == 0) return sg * ldexp((double)mant, -24);
    if (ex == 31) return mant ? NAN : sg * INFINITY;
    return sg * ldexp((double)(1024 + mant), ex - 25);
}

/* out[m,n] = bf16_rne(acc[m,n] * sx[m] * sw[n]); sx*sw is exact in float64. */
void oracle_epilogue_bf16(const int32_t *acc, const float *sx, const float *sw, int64_t M,
                          int64_t N, uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double scale = (double)sx[m] * (double)sw[n];
            double v = (double)acc[m * N + n] * scale;
            out[m * N + n] = oracle_bf16_rne_from_f64(v);
        }
    }
}

/*
 * out[m,n] = bf16_rne(alpha * t + beta * bias[n]), t = acc[m,n] * (sx[m] * sw[n]),
 * every operation a float64 operation in this order (no contraction); bias may
 * be NULL, which means no bias term (beta is then ignored).
 */
void oracle_epilogue_addmm_bf16(const int32_t *acc, const float *sx, const float *sw,
                                const float *bias, double alpha, double beta, int64_t M,
                                int64_t N, uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double scale = (double)sx[m] * (double)sw[n];
            double t = (double)acc[m * N + n] * scale;
            double v = alpha * t;
            if (bias) v = v + beta * (double)bias[n];
            out[m * N + n] = oracle_bf16_rne_from_f64(v);
        }
    }
}

/*
 * Block-sparse weight, 'bs' x 'bs' blocks: block j covers output channels
 * [r*bs, r*bs+bs) for the block row r with crow[r] <= j < crow[r+1] and input
 * channels [col[j]*bs, col[j]*bs+bs); values[j][i][c] is W[r*bs+i, col[j]*bs+c].
 * acc[m,n] = sum over the stored blocks of block row n/bs of the int8 products;
 * channels of block rows with no stored block get 0.
 * Returns 0, or -1 if any sum falls outside int32.
 */
int oracle_bsr_gemm_i32(const int8_t *xq, int64_t M, int64_t K, const int32_t *crow,
                        const int32_t *col, const int8_t *values, int64_t bs, int64_t N,
                        int32_t *acc) {
    int64_t block_rows = N / bs;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t r = 0; r < block_rows; ++r) {
            for (int64_t i = 0; i < bs; ++i) {
                int64_t sum = 0;
                for (int64_t j = crow[r]; j < crow[r + 1]; ++j) {
                    const int8_t *blk = values + j * bs * bs;
                    int64_t k0 = (int64_t)col[j] * bs;
                    for (int64_t c = 0; c < bs; ++c)
                        sum += (int64_t)xq[m * K + k0 + c] * (int64_t)blk[i * bs + c];
                }
                if (sum > INT32_MAX || sum < INT32_MIN) bad = 1;
                acc[m * N + r * bs + i] = (int32_t)sum;
            }
        }
    }
    return bad ? -1 : 0;
}

/*
 * 2:4 compression of an int8 weight w [N,K] (K % 128 == 0).
 *
 * Group g of row n is w[n][4g .. 4g+3]. Its kept positions p0 < p1 are the two
 * largest |w| of the group, equal magnitudes taken in position order (the
 * pages take weights that are already 2:4; with at most two nonzeros in a
 * group this keeps all of them, so such a weight is stored exactly).
 *
 * Storage. Within each 64-column step s (groups 16s .. 16s+15) the groups are
 * listed in the order 0,1,2,3, 8,9,10,11, 4,5,6,7, 12,13,14,15 of the step,
 * list position c holding group 16s + order[c]. The arrays are K-block-major:
 * block B = s / 2 covers columns [128B, 128B+128), and every row's piece of a
 * block is contiguous, rows in order:
 *   values[B][n][32 (s % 2) + 2c + t] = w[n][4 (16s + order[c]) + p_t]  (t = 0, 1)
 *   meta[B][n][2 (s % 2) + c/8], bits 4 (c%8) .. 4 (c%8) + 3 = p0 | p1 << 2
 * values is int8 [K/128, N, 64], meta uint32 [K/128, N, 4].
 */
static const int kGroupOrder24[16] = {0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15};

static int abs_i8(int8_t v) { return v < 0 ? -(int)v : (int)v; }

/* The two kept positions of one group of 4, p0 < p1. */
static void kept_pair24(const int8_t *grp, int *p0, int *p1) {
    int first = 0;
    for (int p = 1; p < 4; ++p)
        if (abs_i8(grp[p]) > abs_i8(grp[first])) first = p;
    int second = -1;
    for (int p = 0; p < 4; ++p) {
        if (p == first) continue;
        if (second < 0 || abs_i8(grp[p]) > abs_i8(grp[second])) second = p;
    }
    *p0 = first < second ? first : second;
    *p1 = first < second ? second : first;
}

void oracle_compress24(const int8_t *w, int64_t N, int64_t K, int8_t *values, uint32_t *meta) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t s = 0; s < K / 64; ++s) {
            int8_t *v = values + ((s / 2) * N + n) * 64 + 32 * (s % 2);
            uint32_t *m = meta + ((s / 2) * N + n) * 4 + 2 * (s % 2);
            uint32_t words[2] = {0, 0};
            for (int c = 0; c < 16; ++c) {
                const int8_t *grp = w + n * K + 4 * (16 * s + kGroupOrder24[c]);
                int p0, p1;
                kept_pair24(grp, &p0, &p1);
                v[2 * c] = grp[p0];
                v[2 * c + 1] = grp[p1];
                words[c / 8] |= (uint32_t)(p0 | (p1 << 2)) << (4 * (c % 8));
            }
            m[0] = words[0];
            m[1] = words[1];
        }
    }
}

/* The inverse: w [N,K] with the stored values at their positions, zeros
 * elsewhere. Returns 0, or -1 if a group's two positions are not p0 < p1. */
int oracle_decompress24(const int8_t *values, const uint32_t *meta, int64_t N, int64_t K,
                        int8_t *w) {
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) w[n * K + k] = 0;
        for (int64_t s = 0; s < K / 64; ++s) {
            const int8_t *v = values + ((s / 2) * N + n) * 64 + 32 * (s % 2);
            const uint32_t *m = meta + ((s / 2) * N + n) * 4 + 2 * (s % 2);
            for (int c = 0; c < 16; ++c) {
                const uint32_t nib = (m[c / 8] >> (4 * (c % 8))) & 15u;
                const int p0 = (int)(nib & 3u), p1 = (int)(nib >> 2);
                if (!(p0 < p1)) bad = 1;
                int8_t *grp = w + n * K + 4 * (16 * s + kGroupOrder24[c]);
                grp[p0] = v[2 * c];
                grp[p1] = v[2 * c + 1];
            }
        }
    }
    return bad ? -1 : 0;
}

/* bf16 bit pattern -> float64 (exact). */
static double bf16_to_f64(uint16_t bits) { return (double)bf16_bits_to_float(bits); }

/* 16-bit floating-point formats of the W4A16 path: bf16 or IEEE binary16. */
static double h_to_f64(uint16_t bits, int half) { return half ? f16_to_f64(bits) : bf16_to_f64(bits); }
static uint16_t h_rne_from_f64(double v, int half) {
    return half ? oracle_f16_rne_from_f64(v) : oracle_bf16_rne_from_f64(v);
}

/*
 * W4A16 dequantization. wq4 [N, K/2] bytes: byte j of row n holds code
 * c[n][2j] in its low nibble and c[n][2j+1] in its high nibble; q = c (u4,
 * 0..15) or, with signed_codes, the 4-bit two's complement of c (s4, -8..7).
 * scales, zeros: bf16 [N, K/G]. w [N,K] bf16 (bit patterns):
 *   w[n][k] = bf16(bf16(q - z) * s),  s = scales[n][k/G], z = zeros[n][k/G].
 * With half, scales, zeros and w are IEEE binary16 and every bf16() above is
 * a binary16 rounding instead (the page's kernel takes float16 or bfloat16
 * scales, zeros and activations); the same exactness argument holds with 11
 * significant bits in place of 8.
 * q - z is exact in float64 unless q != 0 and |z| < 2^-41, where its float64
 * rounding moves it by far less than a bf16 ulp and never onto a bf16 tie, and
 * the product of two bf16 values is exact, so each bf16() here rounds the
 * exact value once.
 */
void oracle_w4a16_dequant(const uint8_t *wq4, const uint16_t *scales, const uint16_t *zeros,
                          int64_t N, int64_t K, int64_t G, int signed_codes, int half,
                          uint16_t *w) {
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            const uint8_t byte = wq4[n * (K / 2) + k / 2];
            const int nibble = (k % 2 == 0) ? (byte & 15) : (byte >> 4);
            /* u4: q = nibble in [0, 15]; s4: the nibble's 4-bit two's complement in [-8, 7] */
            const int q = signed_codes && nibble >= 8 ? nibble - 16 : nibble;
            const double s = h_to_f64(scales[n * (K / G) + k / G], half);
            const double z = h_to_f64(zeros[n * (K / G) + k / G], half);
            const double shifted = h_to_f64(h_rne_from_f64((double)q - z, half), half);
            w[n * K + k] = h_rne_from_f64(shifted * s, half);
        }
    }
}

/*
 * out[m][n] = bf16_rne(sum_k x[m][k] * w[n][k]) for bf16 x [M,K] and bf16 w [N,K]
 * (bit patterns). Each product of two bf16 values is exact in float64; the
 * float64 sum of K of them differs from the exact sum by far less than a bf16
 * ulp of any result that is not itself a near-cancellation.
 */
void oracle_bf16_gemm(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N, int64_t K,
                      uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) sum += bf16_to_f64(x[m * K + k]) * bf16_to_f64(w[n * K + k]);
            out[m * N + n] = oracle_bf16_rne_from_f64(sum);
        }
    }
}

/* The same product for IEEE binary16 x, w and out. Products of two binary16
 * values are exact in float64 (22 significant bits). */
void oracle_f16_gemm(const uint16_t *x, const uint16_t *w, int64_t M, int64_t N, int64_t K,
                     uint16_t *out) {
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double sum = 0.0;
            for (int64_t k = 0; k < K; ++k) sum += f16_to_f64(x[m * K + k]) * f16_to_f64(w[n * K + k]);
            out[m * N + n] = oracle_f16_rne_from_f64(sum);
        }
    }
}

/* Threads the OpenMP loops above run on (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
