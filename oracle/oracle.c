/*
 * oracle.c -- plain, slow CPU oracle for the BitNet b1.58 BitLinear path (W1.58A8).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  The GPU library never links, includes or
 * calls it, and this file includes nothing from the GPU library.
 *
 * Sources (web pages; cited by page key and the page's own section numbers):
 *   [P1] 2kiu.com, article on 1.58-bit quantization and hardware co-optimization
 *        ("从显存焦虑说起 ... 1.58-bit量化：当权重只剩下-1、0、1").
 *   [P2] nxmr.cn, tutorial "1.58 位大模型" (principles, NumPy simulation, memory estimate).
 *   [P3] chenxutan.com, "1.58-bit 大模型极限量化实战：从 BitNet 三值权重到单颗 CPU
 *        跑起 100B 模型".
 *
 * Every function is a direct, scalar transcription of the definition it cites.  There is
 * no blocking, no vectorisation and no reordering beyond the definition.  Floating point:
 *   - where the pages' code fixes fp32 (the divisions W/alpha and 127*x/beta, the
 *     +1e-8 guard on beta, the final dequant multiply), this file computes in fp32;
 *   - where the pages leave precision open (the mean of |W|, the scalar alpha*beta/127),
 *     it computes in fp64 and rounds to fp32 once.
 * Build: gcc -O2 -ffp-contract=off (no fast-math), so each C operation rounds once.
 *
 * Readings of points the pages leave open (each also listed in the design notes):
 *   R1  alpha = mean|W| is accumulated in fp64 in plain row-major order, then rounded
 *       to fp32 once.
 *   R2  round() is round-half-to-even, as the pages' code uses torch.round / np.round.
 *   R3  alpha == 0 (all-zero W): every code is 0 (the division 0/0 is not evaluated).
 *   R4  beta carries the +1e-8 guard of the pages' code, added in fp32.
 *   R5  beta is per token (per row of x); the pages' code takes one max over the
 *       tensor, which is the same thing for a single token.
 *   R6  packed code = w + 1 (00 -> -1, 01 -> 0, 10 -> +1; 11 never written), four
 *       codes per byte, weight k = 4b + i at bits 2i..2i+1 of byte b, rows of W stored
 *       one after another (row-major along K).
 *   R7  s = fp32((double)alpha * (double)beta / 127.0), y = fp32((float)acc * s), then
 *       + bias as a separate fp32 rounding.
 *   R10 the rotation before absmax [P3 §6.2] is a randomized Walsh-Hadamard transform
 *       applied to each row along K in blocks of B (a power of two dividing K): a sign
 *       flip by d[k] in {+1, -1} (the random part; an input, negative int8 = flip), then
 *       the Sylvester Hadamard matrix of order B scaled by 1/sqrt(B).  The same rotation
 *       of the rows of W keeps x . W^T unchanged in exact arithmetic (R R^T = I).
 *   R11 the rotation is evaluated in fp32 as butterflies (a, b) -> (a + b, a - b) on
 *       pairs (j, j + h), with h = 1, 2, 4, ..., B/2 in that order, then one fp32
 *       multiply of every result by fp32(1/sqrt(B)) (exact when B is a power of 4).
 *   R12 block scales [P1 §2.3, §4.2]: one alpha per 128 consecutive weights of a row,
 *       alpha[n, b] = mean |W[n, 128b .. 128b+127]| (R1 for a block), codes divided by their
 *       block's alpha; the integer sums are kept per block, acc[m, n, b], and
 *       y[m, n] = fp32(S * (beta[m] / 127)) with S = sum_b alpha[n, b] * acc[m, n, b]
 *       accumulated in fp64 in ascending b and beta/127 an fp64 division; + bias in fp32.
 *   R13 the BitMLP of [P3 §6.1] is fc2(GELU(fc1(x))) with two BitLinears; GELU is the
 *       exact (erf) GELU of torch.nn.GELU, h Phi(h) = 0.5 h (1 + erf(h / sqrt 2)), written
 *       with the complementary error function, Phi(h) = erfc(-h / sqrt 2) / 2, so that no
 *       term cancels for negative h (1 + erf(h / sqrt 2) loses every digit below h = -8.3);
 *       evaluated in fp64 as (0.5 h) erfc(-h * RN64(1/sqrt 2)) and rounded to fp32 once;
 *       fc2 quantizes the fp32 GELU output like any activation.
 *   R14 sub-2-bit packing [P2 §1.1, §6.1] (a "more compact" encoding, format not given):
 *       five codes c = W_hat + 1 per byte as the base-3 number sum_i c_i 3^i, c_i the code of
 *       weight 5b + i of the row; a row takes 16 ceil(K / 80) bytes, and trits past K hold
 *       code 1 (weight 0), so a byte with no weight left is 121.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_EBADCODE (-2)

/* [P3 §2.3] alpha = mean(|W|) over all weights of the tensor (per-tensor scale).
 * [P2 §3.1] the same formula; R1 fixes fp64 accumulation. */
float oracle_absmean(const float* w, int64_t count) {
    double s = 0.0;
    for (int64_t i = 0; i < count; ++i) s += fabs((double)w[i]);
    return (float)(s / (double)count);
}

/* [P2 §3.1, §4.2] per-output-row scale: alpha[n] = mean_k |W[n, k]|. */
int oracle_absmean_rows(const float* w, int64_t n_rows, int64_t k, float* alpha) {
    if (!w || !alpha || n_rows <= 0 || k <= 0) return ORACLE_EINVAL;
    for (int64_t n = 0; n < n_rows; ++n) alpha[n] = oracle_absmean(w + n * k, k);
    return ORACLE_OK;
}

/* [P3 §2.3, §4.1] W_hat = clip(round(W / alpha), -1, 1).
 * The quotient is an fp32 division (weight / alpha in the page's code), rounded half to
 * even (R2), clipped; -0.0 becomes code 0.  alpha == 0 gives code 0 (R3). */
static int8_t ternary_code(float w, float alpha) {
    if (alpha == 0.0f) return 0;
    float q = w / alpha;
    float r = rintf(q);
    if (r > 1.0f) r = 1.0f;
    if (r < -1.0f) r = -1.0f;
    return (int8_t)r;
}

int oracle_ternarize(const float* w, int64_t count, float alpha, int8_t* codes) {
    if (!w || !codes || count < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < count; ++i) codes[i] = ternary_code(w[i], alpha);
    return ORACLE_OK;
}

/* Per-row variant: row n uses alpha[n]. */
int oracle_ternarize_rows(const float* w, int64_t n_rows, int64_t k, const float* alpha,
                          int8_t* codes) {
    if (!w || !alpha || !codes || n_rows <= 0 || k <= 0) return ORACLE_EINVAL;
    for (int64_t n = 0; n < n_rows; ++n)
        for (int64_t j = 0; j < k; ++j) codes[n * k + j] = ternary_code(w[n * k + j], alpha[n]);
    return ORACLE_OK;
}

/* [P3 §5.3] two bits per weight, 00/01/10 for -1/0/+1; layout R6. */
int oracle_pack(const int8_t* codes, int64_t n_rows, int64_t k, uint8_t* packed) {
    if (!codes || !packed || n_rows <= 0 || k <= 0 || k % 4 != 0) return ORACLE_EINVAL;
    int64_t row_bytes = k / 4;
    for (int64_t n = 0; n < n_rows; ++n) {
        for (int64_t b = 0; b < row_bytes; ++b) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                int w = codes[n * k + 4 * b + i];
                if (w < -1 || w > 1) return ORACLE_EBADCODE;
                byte |= (unsigned)(w + 1) << (2 * i);
            }
            packed[n * row_bytes + b] = (uint8_t)byte;
        }
    }
    return ORACLE_OK;
}

/* Inverse of oracle_pack.  The pattern 11 is never written; meeting it is an error. */
int oracle_unpack(const uint8_t* packed, int64_t n_rows, int64_t k, int8_t* codes) {
    if (!codes || !packed || n_rows <= 0 || k <= 0 || k % 4 != 0) return ORACLE_EINVAL;
    int64_t row_bytes = k / 4;
    for (int64_t n = 0; n < n_rows; ++n) {
        for (int64_t b = 0; b < row_bytes; ++b) {
            unsigned byte = packed[n * row_bytes + b];
            for (int i = 0; i < 4; ++i) {
                unsigned c = (byte >> (2 * i)) & 3u;
                if (c == 3u) return ORACLE_EBADCODE;
                codes[n * k + 4 * b + i] = (int8_t)((int)c - 1);
            }
        }
    }
    return ORACLE_OK;
}

/* [P3 §2.3, §4.1, §5.3] weight quantization as one call: per-tensor alpha, codes, packing.
 * codes (nullable) receives the unpacked ternary values as well. */
int oracle_quantize_weights(const float* w, int64_t n_rows, int64_t k, int8_t* codes,
                            uint8_t* packed, float* alpha) {
    if (!w || !packed || !alpha || n_rows <= 0 || k <= 0 || k % 4 != 0) return ORACLE_EINVAL;
    float a = oracle_absmean(w, n_rows * k);
    int64_t row_bytes = k / 4;
    for (int64_t n = 0; n < n_rows; ++n) {
        for (int64_t b = 0; b < row_bytes; ++b) {
            unsigned byte = 0;
            for (int i = 0; i < 4; ++i) {
                int8_t c = ternary_code(w[n * k + 4 * b + i], a);
                if (codes) codes[n * k + 4 * b + i] = c;
                byte |= (unsigned)(c + 1) << (2 * i);
            }
            packed[n * row_bytes + b] = (uint8_t)byte;
        }
    }
    *alpha = a;
    return ORACLE_OK;
}

/* [P3 §2.4, §4.1] beta = max|x| (+1e-8, R4), x_q = clip(round(127 * x / beta), -127, 127).
 * Per token (R5): row m of x has its own beta[m].  127*x is an fp32 product and the
 * quotient an fp32 division, in the order the page's code writes them. */
int oracle_quantize_act(const float* x, int64_t m_rows, int64_t k, int8_t* xq, float* beta) {
    if (!x || !xq || !beta || m_rows <= 0 || k <= 0) return ORACLE_EINVAL;
    for (int64_t m = 0; m < m_rows; ++m) {
        const float* row = x + m * k;
        float mx = 0.0f;
        for (int64_t j = 0; j < k; ++j) {
            float a = fabsf(row[j]);
            if (a > mx) mx = a;
        }
        float b = mx + 1e-8f;
        beta[m] = b;
        for (int64_t j = 0; j < k; ++j) {
            float t = (row[j] * 127.0f) / b;
            float r = rintf(t);
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            xq[m * k + j] = (int8_t)r;
        }
    }
    return ORACLE_OK;
}

/* [P2 §3.3] Y[m][n] = sum over k with W=+1 of X[m][k] minus sum over k with W=-1 of
 * X[m][k]; zero weights are skipped.  Integer accumulation (int32 holds 127*K for any
 * K below 16.9 million).  Output rows n in [n0, n1) only, so a caller can split work. */
int oracle_ternary_matmul(const int8_t* xq, int64_t m_rows, int64_t k, const int8_t* codes,
                          int64_t n_rows, int32_t* acc, int64_t n0, int64_t n1) {
    if (!xq || !codes || !acc || m_rows <= 0 || k <= 0 || n_rows <= 0) return ORACLE_EINVAL;
    if (n0 < 0 || n1 > n_rows || n0 > n1) return ORACLE_EINVAL;
    for (int64_t m = 0; m < m_rows; ++m) {
        for (int64_t n = n0; n < n1; ++n) {
            int32_t s = 0;
            for (int64_t j = 0; j < k; ++j) {
                int8_t c = codes[n * k + j];
                if (c == 1) s += xq[m * k + j];
                else if (c == -1) s -= xq[m * k + j];
            }
            acc[m * n_rows + n] = s;
        }
    }
    return ORACLE_OK;
}

/* [P3 §2.4, §2.5, §4.2] dequantisation scale alpha*beta/127, reading R7. */
float oracle_dequant_scale(float alpha, float beta) {
    return (float)((double)alpha * (double)beta / 127.0);
}

/* [P3 §2.4, §3.2 step 4] y = acc * (alpha*beta/127) + bias.  alpha_rows (nullable)
 * selects the per-row alpha variant [P2 §3.1]: then column n uses alpha_rows[n]. */
int oracle_dequant(const int32_t* acc, const float* beta, float alpha, const float* alpha_rows,
                   int64_t m_rows, int64_t n_rows, const float* bias, float* y, int64_t n0,
                   int64_t n1) {
    if (!acc || !beta || !y || m_rows <= 0 || n_rows <= 0) return ORACLE_EINVAL;
    if (n0 < 0 || n1 > n_rows || n0 > n1) return ORACLE_EINVAL;
    for (int64_t m = 0; m < m_rows; ++m) {
        for (int64_t n = n0; n < n1; ++n) {
            float a = alpha_rows ? alpha_rows[n] : alpha;
            float s = oracle_dequant_scale(a, beta[m]);
            float v = (float)acc[m * n_rows + n] * s;
            if (bias) v = v + bias[n];
            y[m * n_rows + n] = v;
        }
    }
    return ORACLE_OK;
}

/* [P3 §6.2] randomized Hadamard rotation of each row of x [m_rows, k], readings R10, R11.
 * signs (nullable = all +1) holds d[0..k-1]; block is B.  out may equal x. */
int oracle_hadamard_rows(const float* x, int64_t m_rows, int64_t k, int64_t block, const int8_t* signs,
                         float* out) {
    if (!x || !out || m_rows <= 0 || k <= 0 || block <= 0) return ORACLE_EINVAL;
    if ((block & (block - 1)) != 0 || k % block != 0) return ORACLE_EINVAL;
    const float scale = (float)(1.0 / sqrt((double)block));
    for (int64_t m = 0; m < m_rows; ++m) {
        const float* row = x + m * k;
        float* o = out + m * k;
        for (int64_t j = 0; j < k; ++j) o[j] = (signs && signs[j] < 0) ? -row[j] : row[j];
        for (int64_t b0 = 0; b0 < k; b0 += block) {
            float* v = o + b0;
            for (int64_t h = 1; h < block; h *= 2) {
                for (int64_t i = 0; i < block; i += 2 * h) {
                    for (int64_t j = i; j < i + h; ++j) {
                        float a = v[j], b = v[j + h];
                        v[j] = a + b;
                        v[j + h] = a - b;
                    }
                }
            }
            for (int64_t j = 0; j < block; ++j) v[j] = v[j] * scale;
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- block scales (R12) */
#define ORACLE_BLOCK 128

/* [P1 §2.3, §4.2] alpha[n, b] over each block of 128 weights of row n; alpha is [N, K/128]. */
int oracle_absmean_blocks(const float* w, int64_t n_rows, int64_t k, float* alpha) {
    if (!w || !alpha || n_rows <= 0 || k <= 0 || k % ORACLE_BLOCK != 0) return ORACLE_EINVAL;
    const int64_t kb = k / ORACLE_BLOCK;
    for (int64_t n = 0; n < n_rows; ++n)
        for (int64_t b = 0; b < kb; ++b)
            alpha[n * kb + b] = oracle_absmean(w + n * k + b * ORACLE_BLOCK, ORACLE_BLOCK);
    return ORACLE_OK;
}

/* [P3 §2.3] codes with each weight divided by its own block's alpha. */
int oracle_ternarize_blocks(const float* w, int64_t n_rows, int64_t k, const float* alpha, int8_t* codes) {
    if (!w || !alpha || !codes || n_rows <= 0 || k <= 0 || k % ORACLE_BLOCK != 0) return ORACLE_EINVAL;
    const int64_t kb = k / ORACLE_BLOCK;
    for (int64_t n = 0; n < n_rows; ++n)
        for (int64_t j = 0; j < k; ++j)
            codes[n * k + j] = ternary_code(w[n * k + j], alpha[n * kb + j / ORACLE_BLOCK]);
    return ORACLE_OK;
}

/* [P2 §3.3] the add/sub sums kept per block: acc[m, n, b] over k in block b (int32). */
int oracle_ternary_matmul_blocks(const int8_t* xq, int64_t m_rows, int64_t k, const int8_t* codes,
                                 int64_t n_rows, int32_t* acc) {
    if (!xq || !codes || !acc || m_rows <= 0 || n_rows <= 0 || k <= 0 || k % ORACLE_BLOCK != 0)
        return ORACLE_EINVAL;
    const int64_t kb = k / ORACLE_BLOCK;
    for (int64_t m = 0; m < m_rows; ++m)
        for (int64_t n = 0; n < n_rows; ++n)
            for (int64_t b = 0; b < kb; ++b) {
                int32_t part = 0;
                for (int64_t j = b * ORACLE_BLOCK; j < (b + 1) * ORACLE_BLOCK; ++j) {
                    const int8_t cj = codes[n * k + j];
                    if (cj == 1) part += xq[m * k + j];
                    else if (cj == -1) part -= xq[m * k + j];
                }
                acc[(m * n_rows + n) * kb + b] = part;
            }
    return ORACLE_OK;
}

/* [P1 §2.3; P3 §2.4] y[m, n] = fp32(S * (beta[m] / 127)) (+ bias), S = sum_b alpha[n, b] *
 * acc[m, n, b] in fp64, ascending b (R12). */
int oracle_dequant_blocks(const int32_t* acc, const float* beta, const float* alpha, int64_t m_rows,
                          int64_t n_rows, int64_t kb, const float* bias, float* y) {
    if (!acc || !beta || !alpha || !y || m_rows <= 0 || n_rows <= 0 || kb <= 0) return ORACLE_EINVAL;
    for (int64_t m = 0; m < m_rows; ++m) {
        const double t = (double)beta[m] / 127.0;
        for (int64_t n = 0; n < n_rows; ++n) {
            double s = 0.0;
            for (int64_t b = 0; b < kb; ++b) s += (double)alpha[n * kb + b] * (double)acc[(m * n_rows + n) * kb + b];
            const float yv = (float)(s * t);
            y[m * n_rows + n] = bias ? yv + bias[n] : yv;
        }
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- BitMLP (R13) */
/* [P3 §6.1] the GELU between the two BitLinears of the BitMLP, elementwise:
 * GELU(h) = h Phi(h), Phi(h) = erfc(-h / sqrt 2) / 2 (R13). */
int oracle_gelu(const float* h, int64_t count, float* g) {
    if (!h || !g || count <= 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < count; ++i) {
        const double v = (double)h[i];
        g[i] = (float)(0.5 * v * erfc(-v * 0.70710678118654752440));
    }
    return ORACLE_OK;
}

/* ---------------------------------------------------------------- 5 trits per byte (R14) */
int64_t oracle_t5_row_bytes(int64_t k) { return 16 * ((k + 79) / 80); }

/* [P2 §1.1, §6.1] pack codes [n_rows, k] (values -1, 0, 1) five to a byte, reading R14. */
int oracle_pack_t5(const int8_t* codes, int64_t n_rows, int64_t k, uint8_t* packed) {
    if (!codes || !packed || n_rows <= 0 || k <= 0) return ORACLE_EINVAL;
    const int64_t rb = oracle_t5_row_bytes(k);
    for (int64_t n = 0; n < n_rows; ++n) {
        for (int64_t b = 0; b < rb; ++b) {
            unsigned v = 0, p3 = 1;
            for (int i = 0; i < 5; ++i, p3 *= 3) {
                const int64_t j = 5 * b + i;
                int c = 1;                                     /* past K: weight 0 */
                if (j < k) {
                    const int8_t w = codes[n * k + j];
                    if (w < -1 || w > 1) return ORACLE_EBADCODE;
                    c = w + 1;
                }
                v += (unsigned)c * p3;
            }
            packed[n * rb + b] = (uint8_t)v;
        }
    }
    return ORACLE_OK;
}

/* Inverse of oracle_pack_t5 for the first k weights of each row; bytes above 242 are
 * rejected. */
int oracle_unpack_t5(const uint8_t* packed, int64_t n_rows, int64_t k, int8_t* codes) {
    if (!codes || !packed || n_rows <= 0 || k <= 0) return ORACLE_EINVAL;
    const int64_t rb = oracle_t5_row_bytes(k);
    for (int64_t n = 0; n < n_rows; ++n) {
        for (int64_t j = 0; j < k; ++j) {
            unsigned v = packed[n * rb + j / 5];
            if (v > 242) return ORACLE_EBADCODE;
            for (int i = 0; i < (int)(j % 5); ++i) v /= 3;
            codes[n * k + j] = (int8_t)((int)(v % 3) - 1);
        }
    }
    return ORACLE_OK;
}
