/*
 * bitlinear.h -- C ABI of the MI355X (gfx950) BitNet b1.58 BitLinear library (W1.58A8).
 *
 * Page keys used in the citations below:
 *   [P1] 2kiu.com, article on 1.58-bit quantization and hardware co-optimization (block
 *        scales, §2.3 and §4.2).
 *   [P2] nxmr.cn tutorial "1.58 位大模型" (per-row absmean, add/sub form of the matmul, §1.1
 *        and §6.1 more compact encodings).
 *   [P3] chenxutan.com, "1.58-bit 大模型极限量化实战：从 BitNet 三值权重到单颗 CPU 跑起 100B 模型"
 *        (absmean / absmax formulas, BitLinear forward, 2-bit packing, §6.1 the BitMLP,
 *        §6.2 the rotation before absmax).
 *
 * The layer is split the way [P3 §3.2] describes BitLinear: weights are quantized once and
 * cached (bitlinear_quantize_weights); every call quantizes the activations
 * (bitlinear_quantize_act), runs the ternary x int8 integer matmul and applies the
 * alpha*beta/127 dequantization (bitlinear_forward).
 *
 * Conventions shared by every entry point
 *   - Memory: every array argument is DEVICE memory on the current HIP device, allocated and
 *     owned by the caller.  The library never allocates, frees or retains caller memory.  Its
 *     only state between calls is the per-thread code of the last HIP error (see
 *     bitlinear_last_hip_error); calls are reentrant.
 *   - Execution: every call validates its arguments on the host, enqueues its kernels on
 *     `stream` (0 = the null stream) and returns without synchronising.  Results are
 *     visible to later work on the same stream.
 *   - Errors: 0 (BITLINEAR_OK) or a negative bitlinear_status.  Argument validation happens
 *     before any HIP call, so an invalid call enqueues nothing.  BITLINEAR_ERR_HIP reports a
 *     launch error from the HIP runtime (hipGetLastError after the launch).
 *   - Layouts: row-major.  W is [N, K] (out_features x in_features, the nn.Linear
 *     convention [P3 §4.2]); x is [M, K] (M tokens); y = x W^T is [M, N].
 *   - Packed ternary weights: uint8 [N, K/4].  Weight W[n, k] is stored as the 2-bit code
 *     W_hat + 1 (00 -> -1, 01 -> 0, 10 -> +1; 11 is never written) [P3 §5.3], at bits
 *     2*(k%4) .. 2*(k%4)+1 of byte n*K/4 + k/4.  K must be a multiple of 4.
 *   - Non-finite inputs (NaN, Inf) give unspecified codes and outputs.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITLINEAR_ABI_VERSION 1

/* Largest K for which |acc| <= 127*K still fits int32. */
#define BITLINEAR_MAX_K 16909320

typedef enum bitlinear_status {
    BITLINEAR_OK = 0,
    BITLINEAR_ERR_INVALID_ARG = -1, /* null required pointer, size <= 0 */
    BITLINEAR_ERR_SHAPE = -2,       /* K % 4 != 0, K > BITLINEAR_MAX_K, size overflow */
    BITLINEAR_ERR_ALIGNMENT = -3,   /* a pointer lacks the alignment the call documents */
    BITLINEAR_ERR_WORKSPACE = -4,   /* workspace null or smaller than required */
    BITLINEAR_ERR_HIP = -5,         /* the HIP runtime reported an error at launch */
    BITLINEAR_ERR_SCRATCH = -6      /* beyond the fixed scratch of an allocation-free call */
} bitlinear_status;

/* Returns BITLINEAR_ABI_VERSION of the built library. */
int bitlinear_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* bitlinear_status_string(int status);

/* The hipError_t of the last BITLINEAR_ERR_HIP returned on the calling thread (0 if none). */
int bitlinear_last_hip_error(void);

/*
 * Bytes of device workspace bitlinear_quantize_weights needs for an [N, K] tensor:
 * N fp64 row partial sums (0 for invalid sizes).
 */
size_t bitlinear_quantize_weights_workspace_size(int64_t N, int64_t K);

/*
 * Absmean ternary weight quantization with one scale per tensor [P3 §2.3, §4.1]:
 *     alpha = mean(|W|),  W_hat = clip(round(W / alpha), -1, 1),  packed 2 bits/weight.
 * |W| is summed in fp64 (fixed order: per-row partials, then a fixed tree over rows) and
 * alpha is rounded to fp32 once; W / alpha is an IEEE fp32 division; round() is
 * round-half-to-even.  An all-zero W gives alpha = 0 and every code 0 (weight 0).
 *
 *   W          [N, K] fp32, 16-byte aligned.                                (in)
 *   W_packed   [N, K/4] uint8 in the packed layout above, 4-byte aligned.   (out)
 *   alpha      [1] fp32.                                                    (out)
 *   workspace  >= bitlinear_quantize_weights_workspace_size(N, K) bytes,
 *              8-byte aligned; scratch, contents undefined on return.
 * Errors: INVALID_ARG (null pointer, N or K <= 0), SHAPE (K % 4, K too large, N*K
 * overflow), ALIGNMENT, WORKSPACE, HIP.
 */
int bitlinear_quantize_weights(const float* W, int64_t N, int64_t K, uint8_t* W_packed,
                               float* alpha, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * bitlinear_quantize_weights without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc).  The fp64 row sums go to a fixed scratch array inside the library, one copy per
 * device, held until the process ends, of bitlinear_quantize_weights_noalloc_max_rows() rows
 * (262144, 2 MiB).  The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); the first call on a device looks up the address of that device's scratch.
 * Results are identical to bitlinear_quantize_weights.  All calls on one device share its
 * scratch, so calls that overlap on one device (different streams, or different host
 * threads) race and give undefined results; calls ordered on one stream do not.
 *   Arguments as bitlinear_quantize_weights, without the workspace.
 * Errors: as bitlinear_quantize_weights, and SCRATCH when N exceeds the scratch rows.
 */
int bitlinear_quantize_weights_noalloc(const float* W, int64_t N, int64_t K, uint8_t* W_packed,
                                       float* alpha, hipStream_t stream);

/* Rows (N) the fixed scratch of bitlinear_quantize_weights_noalloc holds. */
size_t bitlinear_quantize_weights_noalloc_max_rows(void);

/*
 * Per-output-row variant [P2 §3.1, §4.2]: alpha_rows[n] = mean_k |W[n, k]| (fp64 sum of
 * the row, one fp32 rounding); row n is ternarized with alpha_rows[n].  Needs no workspace.
 *   alpha_rows [N] fp32 (out).  Other arguments and errors as bitlinear_quantize_weights.
 */
int bitlinear_quantize_weights_rows(const float* W, int64_t N, int64_t K, uint8_t* W_packed,
                                    float* alpha_rows, hipStream_t stream);

/*
 * Per-token absmax int8 activation quantization [P3 §2.4, §4.1]:
 *     beta[m] = max_k |x[m, k]| + 1e-8 (fp32 add, as the page's code guards the division),
 *     x_q[m, k] = clip(round(fp32(127 * x[m, k]) / beta[m]), -127, 127),
 * with an IEEE fp32 division and round-half-to-even.  An all-zero token gives
 * beta = 1e-8 and x_q = 0.
 *
 *   x     [M, K] fp32.       (in)     x_q  [M, K] int8.   (out)
 *   beta  [M] fp32.          (out)
 * Any K >= 1 is accepted; K % 4 == 0 with 16-byte aligned x and 4-byte aligned x_q takes
 * the vector path.  Errors: INVALID_ARG, SHAPE (M*K overflow), HIP.
 */
int bitlinear_quantize_act(const float* x, int64_t M, int64_t K, int8_t* x_q, float* beta,
                           hipStream_t stream);

/*
 * Ternary x int8 matmul with the dequantization epilogue [P3 §2.4, §2.5, §3.2; P2 §3.3]:
 *     acc[m, n] = sum_k x_q[m, k] * W_hat[n, k]
 *               = sum_{W_hat=+1} x_q - sum_{W_hat=-1} x_q      (int32, exact)
 *     y[m, n]   = fp32(acc[m, n]) * fp32(alpha * beta[m] / 127)  (+ bias[n])
 * where alpha*beta/127 is evaluated in fp64 and rounded to fp32 once, the product is one
 * fp32 rounding and the bias a separate fp32 addition.
 *
 *   x_q       [M, K] int8 (from bitlinear_quantize_act).   (in)
 *   beta      [M] fp32.                                     (in)
 *   W_packed  [N, K/4] uint8, packed layout above.          (in)
 *   alpha     [1] fp32 (from bitlinear_quantize_weights).   (in)
 *   bias      [N] fp32 or NULL.                             (in)
 *   y         [M, N] fp32.                                  (out)
 *   acc       [M, N] int32 or NULL; when given, receives the exact integer sums.  (out)
 * The kernel is chosen by shape: one token (two on matrices of 2^26 weights or more or with
 * K >= 8192) runs a VALU GEMV (dot4 on unpacked codes); up to 64 tokens a weight-streaming int8
 * MFMA kernel; more an int8 MFMA GEMM that unpacks the ternary tiles on chip.  The fast paths
 * need K % 64 == 0 and 16-byte aligned x_q and W_packed; other inputs run a generic kernel
 * with identical results.
 * Errors: INVALID_ARG, SHAPE (K % 4, K > BITLINEAR_MAX_K, size overflow), HIP.
 */
int bitlinear_forward(const int8_t* x_q, const float* beta, int64_t M, int64_t K,
                      const uint8_t* W_packed, const float* alpha, int64_t N, const float* bias,
                      float* y, int32_t* acc, hipStream_t stream);

/*
 * bitlinear_forward with one alpha per output row [P2 §3.1]: column n of y uses
 * alpha_rows[n] ([N] fp32, from bitlinear_quantize_weights_rows).  Same contract otherwise.
 */
int bitlinear_forward_rows(const int8_t* x_q, const float* beta, int64_t M, int64_t K,
                           const uint8_t* W_packed, const float* alpha_rows, int64_t N,
                           const float* bias, float* y, int32_t* acc, hipStream_t stream);

/*
 * Activation quantization and forward in one call [P3 §3.2 steps 2-4]: y from fp32 x,
 * with results identical to bitlinear_quantize_act followed by bitlinear_forward.
 * For M <= 4, K % 64 == 0, K <= 32768 and 16-byte aligned x, W_packed (and x_q if given)
 * it is one kernel that quantizes x on chip; otherwise it makes the two calls.  For three or
 * four tokens, and for two with K > 4096, the two calls are faster, and they are made
 * whenever x_q and beta are given.
 *
 *   x      [M, K] fp32.                                               (in)
 *   x_q    [M, K] int8 or NULL; receives the quantized activations.   (out)
 *   beta   [M] fp32 or NULL; receives the per-token scales.           (out)
 *   W_packed, alpha, N, bias, y, acc: as bitlinear_forward.
 * x_q and beta may be NULL only on the one-kernel path (else INVALID_ARG).
 * Errors: as bitlinear_forward.
 */
int bitlinear_forward_fused(const float* x, int64_t M, int64_t K, const uint8_t* W_packed,
                            const float* alpha, int64_t N, const float* bias, float* y,
                            int8_t* x_q, float* beta, int32_t* acc, hipStream_t stream);

/*
 * bitlinear_forward_fused with one alpha per output row [P2 §3.1]: column n of y uses
 * alpha_rows[n] ([N] fp32).  Besides per-row quantized weights this serves grouped
 * projections: the packed rows of several projections that read the same x (the q, k and v
 * of an attention block, or gate and up of an MLP) stacked into one [N1 + N2 + ..., K/4]
 * matrix, each projection's per-tensor alpha repeated over its rows, give in one launch the
 * outputs of the separate calls, bit for bit.  Same contract as bitlinear_forward_fused.
 */
int bitlinear_forward_fused_rows(const float* x, int64_t M, int64_t K, const uint8_t* W_packed,
                                 const float* alpha_rows, int64_t N, const float* bias, float* y,
                                 int8_t* x_q, float* beta, int32_t* acc, hipStream_t stream);

/*
 * Ternary weights packed five to a byte [P2 §1.1, §6.1] (1.6 bits per weight; the pages name
 * more compact encodings than 2 bits without a format).  Byte b of a row holds the codes
 * c = W_hat + 1 of weights 5b .. 5b+4 as sum_i c_i 3^i (0..242); a row takes
 * bitlinear_t5_row_bytes(K) = 16 ceil(K / 80) bytes; trits past K hold code 1 (weight 0).
 * Quantization is that of bitlinear_quantize_weights (same alpha, same codes), packed this
 * way: W_t5 is [N, bitlinear_t5_row_bytes(K)] uint8 (out); other arguments and errors as
 * bitlinear_quantize_weights.  K % 4 == 0, K <= 65536.
 */
size_t bitlinear_t5_row_bytes(int64_t K);
int bitlinear_quantize_weights_t5(const float* W, int64_t N, int64_t K, uint8_t* W_t5, float* alpha,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The 2-bit packing of bitlinear_quantize_weights ([N, K/4]) repacked five codes per byte
 * into W_t5 ([N, bitlinear_t5_row_bytes(K)]): the same codes.  Errors: INVALID_ARG, SHAPE, HIP. */
int bitlinear_repack_t5(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W_t5, hipStream_t stream);

/*
 * bitlinear_forward on 5-trit packed weights (16-byte aligned W_t5): the same acc and y as
 * bitlinear_forward on the 2-bit packing of the same codes.  The kernel is a decode GEMV
 * (one token per grid row; more tokens re-read the weights).  No acc output.  Bytes above
 * 242 are never written by the packers; if present they give unspecified outputs.
 * Errors: INVALID_ARG, SHAPE (K > 65536, M > 65535, ...), ALIGNMENT, HIP.
 */
int bitlinear_forward_t5(const int8_t* x_q, const float* beta, int64_t M, int64_t K, const uint8_t* W_t5,
                         const float* alpha, int64_t N, const float* bias, float* y, hipStream_t stream);

/*
 * Block-scaled weights [P1 §2.3, §4.2]: one scale per block of 128 consecutive weights of a
 * row, alpha_blocks of shape [N, K/128]:
 *     alpha_blocks[n, b] = mean |W[n, 128b .. 128b+127]|   (fp64 sum, one fp32 rounding)
 *     W_hat[n, k]        = clip(round(W[n, k] / alpha_blocks[n, k/128]), -1, 1)
 * (fp32 division, round-half-to-even; an all-zero block has alpha 0 and codes 0), packed as
 * above.  W is read once.
 *   W [N, K] fp32, 16-byte aligned (in); W_packed [N, K/4] uint8 (out);
 *   alpha_blocks [N, K/128] fp32, 4-byte aligned (out).
 * Errors: INVALID_ARG, SHAPE (K % 128, sizes), ALIGNMENT, HIP.
 */
int bitlinear_quantize_weights_blocks(const float* W, int64_t N, int64_t K, uint8_t* W_packed,
                                      float* alpha_blocks, hipStream_t stream);

/*
 * Forward with block-scaled weights [P1 §2.3; P2 §3.3; P3 §2.4]:
 *     acc[m, n, b] = sum over k in block b of x_q[m, k] * W_hat[n, k]      (int32, exact)
 *     y[m, n]      = fp32(S * (beta[m] / 127))  (+ bias[n], a separate fp32 addition)
 *     S            = sum_b alpha_blocks[n, b] * acc[m, n, b]
 * with S and beta/127 in fp64.  The products alpha*acc are exact in fp64; the additions run
 * in an order fixed by the kernel, so y can differ from an fp64 sum taken in another order by
 * one fp32 rounding in rare cases (results are reproducible run to run).
 *   x_q [M, K] int8, beta [M] fp32 (from bitlinear_quantize_act); W_packed [N, K/4] uint8 and
 *   alpha_blocks [N, K/128] fp32 (from bitlinear_quantize_weights_blocks); bias [N] or NULL;
 *   y [M, N] fp32 (out).  x_q and W_packed 16-byte aligned, alpha_blocks 4-byte aligned.
 * K % 128 == 0, K <= 32768 and M <= 262140.  One or two tokens run a GEMV; 3 to 127 run an
 * int8 MFMA kernel over slices of up to 64 tokens (32 when K % 256 != 0),
 * each slice reading the codes once; 128 and more an int8 MFMA GEMM.
 * Errors: INVALID_ARG, SHAPE, ALIGNMENT, HIP.
 */
int bitlinear_forward_blocks(const int8_t* x_q, const float* beta, int64_t M, int64_t K,
                             const uint8_t* W_packed, const float* alpha_blocks, int64_t N,
                             const float* bias, float* y, hipStream_t stream);

/*
 * Randomized Hadamard rotation along K [P3 §6.2], the preprocessing that spreads an outlier
 * channel over all dimensions before the absmax.  For each row r of x and each block of B
 * consecutive columns (B = `block`, a power of two, 1 <= B <= 4096, K % B == 0):
 *     out[r, blk] = (d[blk] * x[r, blk]) . H_B / sqrt(B)
 * with d[k] = -1 where signs[k] < 0, +1 elsewhere (signs NULL: all +1), and H_B the Sylvester
 * Hadamard matrix (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]).  Evaluation, fixed so that
 * results are reproducible bit for bit: the sign flip is exact; the transform runs as fp32
 * butterflies (a, b) -> (a + b, a - b) on element pairs (j, j + h), h = 1, 2, 4, ..., B/2 in
 * that order; every result is then multiplied once by fp32(1/sqrt(B)) (exact for B a power
 * of 4).  The rotation is orthonormal (R R^T = I): rotating the rows of W with the same
 * block and signs (once, before bitlinear_quantize_weights) and every x keeps x . W^T.
 *
 *   x      [M, K] fp32, 16-byte aligned.            (in)
 *   signs  [K] int8, 4-byte aligned, or NULL.       (in; the caller draws them)
 *   out    [M, K] fp32, 16-byte aligned; may be x (in place), else must not overlap it. (out)
 * K % 4 == 0.  Errors: INVALID_ARG, SHAPE (block not a power of two in [1, 4096], K % block,
 * K % 4, size overflow), ALIGNMENT, HIP.
 */
int bitlinear_hadamard_rows(const float* x, int64_t M, int64_t K, int64_t block, const int8_t* signs,
                            float* out, hipStream_t stream);

/*
 * Rotation then activation quantization in one pass [P3 §6.2, §2.4]: x_q and beta are those
 * bitlinear_quantize_act gives for the rows rotated by bitlinear_hadamard_rows (same block
 * and signs), without writing the rotated rows.  Feed x_q and beta to bitlinear_forward with
 * weights quantized from rotated rows.
 *
 *   x      [M, K] fp32, 16-byte aligned.            (in)
 *   signs  [K] int8, 4-byte aligned, or NULL.       (in)
 *   x_q    [M, K] int8, 4-byte aligned.             (out)
 *   beta   [M] fp32.                                (out)
 * Errors as bitlinear_hadamard_rows.
 */
int bitlinear_quantize_act_hadamard(const float* x, int64_t M, int64_t K, int64_t block,
                                    const int8_t* signs, int8_t* x_q, float* beta, hipStream_t stream);

/*
 * BitMLP forward [P3 §6.1]: y = fc2(GELU(fc1(x))) with both layers BitLinear (per-tensor
 * alpha, weights from bitlinear_quantize_weights), fc1: d_model -> d_ff, fc2: d_ff -> d_model.
 * GELU is the erf form, 0.5 h (1 + erf(h / sqrt 2)), evaluated in fp64 and rounded to fp32
 * once, applied in fc1's dequantization epilogue; fc2 quantizes its fp32 input per token
 * like any activation.  Each layer runs as bitlinear_forward_fused would (one fused launch
 * for M <= 4, else quantize_act then forward), so results equal the two calls
 *     g = GELU(bitlinear_forward_fused(x, W1...)),  y = bitlinear_forward_fused(g, W2...).
 *
 *   x        [M, d_model] fp32.                                   (in)
 *   W1_packed [d_ff, d_model/4], alpha1 [1], bias1 [d_ff] or NULL. (in)
 *   W2_packed [d_model, d_ff/4], alpha2 [1], bias2 [d_model] or NULL. (in)
 *   y        [M, d_model] fp32.                                   (out)
 *   g        [M, d_ff] fp32: GELU(fc1(x)), fc2's input.            (out, required)
 *   x_q1, beta1 / x_q2, beta2: each layer's quantized input ([M, d] int8, [M] fp32), as
 *   the x_q / beta of bitlinear_forward_fused (required when M > 4 or unaligned).
 * Both layers are validated before anything is enqueued.  Errors as bitlinear_forward_fused.
 */
int bitlinear_mlp_forward(const float* x, int64_t M, int64_t d_model, int64_t d_ff,
                          const uint8_t* W1_packed, const float* alpha1, const float* bias1,
                          const uint8_t* W2_packed, const float* alpha2, const float* bias2,
                          float* y, float* g, int8_t* x_q1, float* beta1, int8_t* x_q2,
                          float* beta2, hipStream_t stream);

/*
 * Rotation, activation quantization and forward in one call [P3 §6.2, §2.4, §3.2]: y from
 * fp32 x with results identical to bitlinear_quantize_act_hadamard (same block and signs)
 * followed by bitlinear_forward on weights quantized from rotated rows.  One token with
 * K % 64 == 0, K <= 16384 and 16-byte aligned W_packed runs as a single launch (every
 * workgroup rotates and quantizes x, then streams its weight rows); other calls need x_q and
 * beta and run the two steps.  x_q / beta (may be NULL on the single-launch path) receive the
 * quantized rotated activations.  Errors as bitlinear_quantize_act_hadamard and
 * bitlinear_forward.
 */
int bitlinear_forward_fused_hadamard(const float* x, int64_t M, int64_t K, int64_t block, const int8_t* signs,
                                     const uint8_t* W_packed, const float* alpha, int64_t N, const float* bias,
                                     float* y, int8_t* x_q, float* beta, hipStream_t stream);

/* Kernel(s) bitlinear_forward_fused launches for these arguments ("gemv_fused" or
 * "quantize_act+forward"; a non-NULL x_q stands for x_q and beta given); a static string. */
const char* bitlinear_forward_fused_kernel(int64_t M, int64_t K, int64_t N, const float* x,
                                           const uint8_t* W_packed, const int8_t* x_q);

/*
 * Name of the kernel bitlinear_forward launches for these arguments ("gemv_dot4",
 * "decode_mfma_i8", "gemm_mfma_i8" or "generic"); a static string, for profiling and reports.
 */
const char* bitlinear_forward_kernel(int64_t M, int64_t K, int64_t N, const int8_t* x_q,
                                     const uint8_t* W_packed);

#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
