// api.hip -- the C ABI declared in include/bitlinear.h: host-side validation, then kernel
// selection by shape and launch on the caller's stream.  No allocation, no sync; the only
// state is the per-thread code of the last HIP error, for bitlinear_last_hip_error.
#include "bitlinear.h"

#include <limits.h>

#include "common.hpp"

using namespace bitlinear;

namespace {

thread_local int g_last_hip_error = 0;

inline int hip_status(hipError_t e) {
    if (e == hipSuccess) return BITLINEAR_OK;
    g_last_hip_error = (int)e;
    return BITLINEAR_ERR_HIP;
}

inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// a*b without overflow into a signed 64-bit result
inline bool mul_ok(int64_t a, int64_t b) { return a > 0 && b > 0 && a <= INT64_MAX / b; }

// The fast forward kernels read 16-byte rows of x_q and W_packed.
inline bool fast_forward_ok(int64_t K, const int8_t* xq, const uint8_t* wp) {
    return K % 64 == 0 && aligned(xq, 16) && aligned(wp, 16);
}

int check_forward(const int8_t* x_q, const float* beta, int64_t M, int64_t K, const uint8_t* W_packed,
                  const float* alpha, int64_t N, float* y) {
    if (!x_q || !beta || !W_packed || !alpha || !y) return BITLINEAR_ERR_INVALID_ARG;
    if (M <= 0 || K <= 0 || N <= 0) return BITLINEAR_ERR_INVALID_ARG;
    if (K % 4 != 0 || K > BITLINEAR_MAX_K) return BITLINEAR_ERR_SHAPE;
    if (!mul_ok(M, K) || !mul_ok(N, K) || !mul_ok(M, N)) return BITLINEAR_ERR_SHAPE;
    if (N > (int64_t)UINT_MAX || M > (int64_t)65535 * 128) return BITLINEAR_ERR_SHAPE;
    return BITLINEAR_OK;
}

enum class Path { Gemv, Decode, Gemm, Generic };

// One token: the VALU GEMV.  Two tokens: the GEMV for matrices of 2^26 weights or more and
// for K >= 8192, where it streams the codes faster; else the MFMA decode kernel (measured with
// weights not in cache, GEMV against decode kernel: 6.1 vs 6.7 us at K = 11008, N = 4096; 6.5
// vs 7.3 us at K = N = 8192; 14.9 vs 16.0 us at K = 8192, N = 28672; 6.9 vs 8.7 us at K = 16384,
// N = 4096).  Three to 64 tokens: the MFMA decode kernel (the GEMV only where that kernel does
// not apply), which beat the GEMV for three and four tokens on every shape measured, also on
// large matrices: M = 3, K = 8192, N = 28672: 16.1 vs 18.9 us; M = 4: 16.3 vs 21.6 us; M = 4,
// K = 16384, N = 8192: 10.7 vs 19.4 us; M = 4, K = 4096, N = 16384: 7.9 vs 10.3 us.  More than
// 64 tokens: the MFMA GEMM.  Every fast path needs K % 64 == 0 and 16-byte aligned rows; other
// calls take the generic kernel.
constexpr int64_t GEMV_BATCH_MIN_WEIGHTS = (int64_t)1 << 26;
Path choose_path(int64_t M, int64_t K, int64_t N, const int8_t* xq, const uint8_t* wp) {
    if (!fast_forward_ok(K, xq, wp)) return Path::Generic;
    if (gemv_supports(M, K) && (M == 1 || (M == 2 && (K >= 8192 || N * K >= GEMV_BATCH_MIN_WEIGHTS)) ||
                                !decode_mfma_supports(M, K)))
        return Path::Gemv;
    if (decode_mfma_supports(M, K)) return Path::Decode;
    return Path::Gemm;
}

bool fused_fast_ok(int64_t M, int64_t K, const float* x, const uint8_t* wp, const int8_t* xq_out) {
    return gemv_supports(M, K) && aligned(x, 16) && aligned(wp, 16) && (!xq_out || aligned(xq_out, 16));
}

// Several tokens: every workgroup of the one-kernel path reads all M rows of fp32 x, so for
// three or four tokens, and for two with K > 4096, quantize_act followed by the forward is the
// faster route (measured with weights not in cache: M = 4, 9.9 vs 19.1 us at K = 11008,
// N = 4096; M = 2, 12.4 vs 17.5 us at K = 16384, N = 8192; 8.9 vs 7.7 us at K = 4096,
// N = 11008).  It needs x_q and beta, so it is taken when the caller gives them; without them
// the call stays one launch.
static bool two_launch_preferred(int64_t M, int64_t K) { return M >= 3 || (M == 2 && K > 4096); }

static bool use_fused_kernel(int64_t M, int64_t K, const float* x, const uint8_t* wp, const int8_t* x_q,
                             const float* beta) {
    return fused_fast_ok(M, K, x, wp, x_q) && !(x_q && beta && two_launch_preferred(M, K));
}

int run_forward(const ForwardArgs& a, hipStream_t stream) {
    switch (choose_path(a.M, a.K, a.N, a.xq, a.wp)) {
        case Path::Gemv: return hip_status(launch_gemv_dot4(a, stream));
        case Path::Decode: return hip_status(launch_decode_mfma(a, stream));
        case Path::Gemm: return hip_status(launch_gemm_mfma(a, stream));
        default: return hip_status(launch_forward_generic(a, stream));
    }
}

}  // namespace

extern "C" {

int bitlinear_abi_version(void) { return BITLINEAR_ABI_VERSION; }

const char* bitlinear_status_string(int status) {
    switch (status) {
        case BITLINEAR_OK: return "ok";
        case BITLINEAR_ERR_INVALID_ARG: return "invalid argument (null pointer or non-positive size)";
        case BITLINEAR_ERR_SHAPE: return "unsupported shape (K % 4 != 0, K too large or size overflow)";
        case BITLINEAR_ERR_ALIGNMENT: return "pointer alignment";
        case BITLINEAR_ERR_WORKSPACE: return "workspace missing or too small";
        case BITLINEAR_ERR_HIP: return "HIP runtime error";
        case BITLINEAR_ERR_SCRATCH: return "shape exceeds the fixed scratch of the allocation-free call";
        default: return "unknown status";
    }
}

int bitlinear_last_hip_error(void) { return g_last_hip_error; }

size_t bitlinear_quantize_weights_workspace_size(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0) return 0;
    return (size_t)N * sizeof(double);
}

int bitlinear_quantize_weights(const float* W, int64_t N, int64_t K, uint8_t* W_packed, float* alpha,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!W || !W_packed || !alpha) return BITLINEAR_ERR_INVALID_ARG;
    if (N <= 0 || K <= 0) return BITLINEAR_ERR_INVALID_ARG;
    if (K % 4 != 0 || K > BITLINEAR_MAX_K || !mul_ok(N, K) || N > (int64_t)INT_MAX * 4)
        return BITLINEAR_ERR_SHAPE;
    if (!aligned(W, 16) || !aligned(W_packed, 4)) return BITLINEAR_ERR_ALIGNMENT;
    if (!workspace || workspace_bytes < bitlinear_quantize_weights_workspace_size(N, K))
        return BITLINEAR_ERR_WORKSPACE;
    if (!aligned(workspace, 8)) return BITLINEAR_ERR_ALIGNMENT;
    double* rows = static_cast<double*>(workspace);
    int st = hip_status(launch_row_abs_sums(W, N, K, rows, stream));
    if (st) return st;
    st = hip_status(launch_alpha_from_rows(rows, N, K, alpha, stream));
    if (st) return st;
    return hip_status(launch_ternary_pack(W, N, K, alpha, false, W_packed, stream));
}

size_t bitlinear_quantize_weights_noalloc_max_rows(void) { return (size_t)kQuantizeScratchRows; }

int bitlinear_quantize_weights_noalloc(const float* W, int64_t N, int64_t K, uint8_t* W_packed, float* alpha,
                                       hipStream_t stream) {
    if (!W || !W_packed || !alpha) return BITLINEAR_ERR_INVALID_ARG;
    if (N <= 0 || K <= 0) return BITLINEAR_ERR_INVALID_ARG;
    if (K % 4 != 0 || K > BITLINEAR_MAX_K || !mul_ok(N, K) || N > (int64_t)INT_MAX * 4)
        return BITLINEAR_ERR_SHAPE;
    if (N > kQuantizeScratchRows) return BITLINEAR_ERR_SCRATCH;
    if (!aligned(W, 16) || !aligned(W_packed, 4)) return BITLINEAR_ERR_ALIGNMENT;
    double* rows = nullptr;
    int st = hip_status(quantize_weights_scratch(&rows));
    if (st) return st;
    // the row sums are written, never accumulated, so the scratch needs no clearing
    st = hip_status(launch_row_abs_sums(W, N, K, rows, stream));
    if (st) return st;
    st = hip_status(launch_alpha_from_rows(rows, N, K, alpha, stream));
    if (st) return st;
    return hip_status(launch_ternary_pack(W, N, K, alpha, false, W_packed, stream));
}

int bitlinear_quantize_weights_rows(const float* W, int64_t N, int64_t K, uint8_t* W_packed,
                                    float* alpha_rows, hipStream_t stream) {
    if (!W || !W_packed || !alpha_rows) return BITLINEAR_ERR_INVALID_ARG;
    if (N <= 0 || K <= 0) return BITLINEAR_ERR_INVALID_ARG;
    if (K % 4 != 0 || K > BITLINEAR_MAX_K || !mul_ok(N, K) || N > (int64_t)INT_MAX * 4)
        return BITLINEAR_ERR_SHAPE;
    if (!aligned(W, 16) || !aligned(W_packed, 4)) return BITLINEAR_ERR_ALIGNMENT;
    int st = hip_status(launch_alpha_rows(W, N, K, alpha_rows, stream));
    if (st) return st;
    return hip_status(launch_ternary_pack(W, N, K, alpha_rows, true, W_packed, stream));
}

int bitlinear_quantize_act(const float* x, int64_t M, int64_t K, int8_t* x_q, float* beta,
                           hipStream_t stream) {
    if (!x || !x_q || !beta) return BITLINEAR_ERR_INVALID_ARG;
    if (M <= 0 || K <= 0) return BITLINEAR_ERR_INVALID_ARG;
    if (!mul_ok(M, K) || M > (int64_t)INT_MAX) return BITLINEAR_ERR_SHAPE;
    return hip_status(launch_quantize_act(x, M, K, x_q, beta, stream));
}

int bitlinear_forward(const int8_t* x_q, const float* beta, int64_t M, int64_t K, const uint8_t* W_packed,
                      const float* alpha, int64_t N, const float* bias, float* y, int32_t* acc,
                      hipStream_t stream) {
    int st = check_forward(x_q, beta, M, K, W_packed, alpha, N, y);
    if (st) return st;
    ForwardArgs a{x_q, beta, M, K, N, W_packed, alpha, false, bias, y, acc};
    return run_forward(a, stream);
}

int bitlinear_forward_rows(const int8_t* x_q, const float* beta, int64_t M, int64_t K,
                           const uint8_t* W_packed, const float* alpha_rows, int64_t N, const float* bias,
                           float* y, int32_t* acc, hipStream_t stream) {
    int st = check_forward(x_q, beta, M, K, W_packed, alpha_rows, N, y);
    if (st) return st;
    ForwardArgs a{x_q, beta, M, K, N, W_packed, alpha_rows, true, bias, y, acc};
    return run_forward(a, stream);
}

// Validation of a fused call, without launching anything.
static int check_fused(const float* x, int64_t M, int64_t K, const uint8_t* W_packed, const float* alpha, int64_t N,
                       float* y, int8_t* x_q, float* beta) {
    if (!x) return BITLINEAR_ERR_INVALID_ARG;
    int st = check_forward(reinterpret_cast<const int8_t*>(x), reinterpret_cast<const float*>(x), M, K, W_packed,
                           alpha, N, y);
    if (st) return st;
    if (fused_fast_ok(M, K, x, W_packed, x_q)) return BITLINEAR_OK;
    // other shapes: the two-call path, which needs x_q and beta as its intermediate
    if (!x_q || !beta) return BITLINEAR_ERR_INVALID_ARG;
    return BITLINEAR_OK;
}

static int forward_fused(const float* x, int64_t M, int64_t K, const uint8_t* W_packed, const float* alpha,
                         bool per_row, int64_t N, const float* bias, float* y, int8_t* x_q, float* beta, int32_t* acc,
                         int act, hipStream_t stream) {
    int st = check_fused(x, M, K, W_packed, alpha, N, y, x_q, beta);
    if (st) return st;
    ForwardArgs a{nullptr, nullptr, M, K, N, W_packed, alpha, per_row, bias, y, acc, act};
    if (use_fused_kernel(M, K, x, W_packed, x_q, beta)) return hip_status(launch_gemv_fused(a, x, x_q, beta, stream));
    st = bitlinear_quantize_act(x, M, K, x_q, beta, stream);
    if (st) return st;
    a.xq = x_q;
    a.beta = beta;
    return run_forward(a, stream);
}

int bitlinear_forward_fused(const float* x, int64_t M, int64_t K, const uint8_t* W_packed, const float* alpha,
                            int64_t N, const float* bias, float* y, int8_t* x_q, float* beta, int32_t* acc,
                            hipStream_t stream) {
    return forward_fused(x, M, K, W_packed, alpha, false, N, bias, y, x_q, beta, acc, 0, stream);
}

int bitlinear_forward_fused_rows(const float* x, int64_t M, int64_t K, const uint8_t* W_packed,
                                 const float* alpha_rows, int64_t N, const float* bias, float* y, int8_t* x_q,
                                 float* beta, int32_t* acc, hipStream_t stream) {
    return forward_fused(x, M, K, W_packed, alpha_rows, true, N, bias, y, x_q, beta, acc, 0, stream);
}

int bitlinear_mlp_forward(const float* x, int64_t M, int64_t d_model, int64_t d_ff, const uint8_t* W1_packed,
                          const float* alpha1, const float* bias1, const uint8_t* W2_packed, const float* alpha2,
                          const float* bias2, float* y, float* g, int8_t* x_q1, float* beta1, int8_t* x_q2,
                          float* beta2, hipStream_t stream) {
    // both layers are validated before either is enqueued
    int st = check_fused(x, M, d_model, W1_packed, alpha1, d_ff, g, x_q1, beta1);
    if (st) return st;
    st = check_fused(g, M, d_ff, W2_packed, alpha2, d_model, y, x_q2, beta2);
    if (st) return st;
    st = forward_fused(x, M, d_model, W1_packed, alpha1, false, d_ff, bias1, g, x_q1, beta1, nullptr, 1, stream);
    if (st) return st;
    return forward_fused(g, M, d_ff, W2_packed, alpha2, false, d_model, bias2, y, x_q2, beta2, nullptr, 0, stream);
}

size_t bitlinear_t5_row_bytes(int64_t K) { return K > 0 ? (size_t)t5_row_bytes(K) : 0; }

int bitlinear_quantize_weights_t5(const float* W, int64_t N, int64_t K, uint8_t* W_t5, float* alpha, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    if (!W || !W_t5 || !alpha) return BITLINEAR_ERR_INVALID_ARG;
    if (N <= 0 || K <= 0) return BITLINEAR_ERR_INVALID_ARG;
    if (K % 4 != 0 || !t5_supports(K) || !mul_ok(N, K) || N > (int64_t)INT_MAX * 4) return BITLINEAR_ERR_SHAPE;
    if (!aligned(W, 16)) return BITLINEAR_ERR_ALIGNMENT;
    if (!workspace || workspace_bytes < bitlinear_quantize_weights_workspace_size(N, K)) return BITLINEAR_ERR_WORKSPACE;
    if (!aligned(workspace, 8)) return BITLINEAR_ERR_ALIGNMENT;
    double* rows = static_cast<double*>(workspace);
    int st = hip_status(launch_row_abs_sums(W, N, K, rows, stream));
    if (st) return st;
    st = hip_status(launch_alpha_from_rows(rows, N, K, alpha, stream));
    if (st) return st;
    return hip_status(launch_pack_t5(W, N, K, alpha, W_t5, stream));
}

int bitlinear_repack_t5(const uint8_t* W_packed, int64_t N, int64_t K, uint8_t* W_t5, hipStream_t stream) {
    if (!W_packed || !W_t5) return BITLINEAR_ERR_INVALID_ARG;
    if (N <= 0 || K <= 0) return BITLINEAR_ERR_INVALID_ARG;
    if (K % 4 != 0 || !t5_supports(K) || !mul_ok(N, K)) return BITLINEAR_ERR_SHAPE;
    return hip_status(launch_repack_t5(W_packed, N, K, W_t5, stream));
}

int bitlinear_forward_t5(const int8_t* x_q, const float* beta, int64_t M, int64_t K, const uint8_t* W_t5,
                         const float* alpha, int64_t N, const float* bias, float* y, hipStream_t stream) {
    int st = check_forward(x_q, beta, M, K, W_t5, alpha, N, y);
    if (st) return st;
    if (!t5_supports(K) || M > 65535) return BITLINEAR_ERR_SHAPE;
    if (!aligned(W_t5, 16)) return BITLINEAR_ERR_ALIGNMENT;
    return hip_status(launch_forward_t5(x_q, beta, M, K, W_t5, alpha, N, bias, y, stream));
}

int bitlinear_quantize_weights_blocks(const float* W, int64_t N, int64_t K, uint8_t* W_packed, float* alpha_blocks,
                                      hipStream_t stream) {
    if (!W || !W_packed || !alpha_blocks) return BITLINEAR_ERR_INVALID_ARG;
    if (N <= 0 || K <= 0) return BITLINEAR_ERR_INVALID_ARG;
    if (K % 128 != 0 || K > BITLINEAR_MAX_K || !mul_ok(N, K) || N * (K / 128) > (int64_t)INT_MAX * 4)
        return BITLINEAR_ERR_SHAPE;
    if (!aligned(W, 16) || !aligned(alpha_blocks, 4)) return BITLINEAR_ERR_ALIGNMENT;
    return hip_status(launch_quantize_blocks(W, N, K, W_packed, alpha_blocks, stream));
}

int bitlinear_forward_blocks(const int8_t* x_q, const float* beta, int64_t M, int64_t K, const uint8_t* W_packed,
                             const float* alpha_blocks, int64_t N, const float* bias, float* y, hipStream_t stream) {
    int st = check_forward(x_q, beta, M, K, W_packed, alpha_blocks, N, y);
    if (st) return st;
    if (!blocks_supports(K) || M > 262140) return BITLINEAR_ERR_SHAPE;
    if (!aligned(x_q, 16) || !aligned(W_packed, 16) || !aligned(alpha_blocks, 4)) return BITLINEAR_ERR_ALIGNMENT;
    return hip_status(launch_forward_blocks(x_q, beta, M, K, W_packed, alpha_blocks, N, bias, y, stream));
}

static int check_hadamard(const float* x, int64_t M, int64_t K, int64_t block, const int8_t* signs) {
    if (!x || M <= 0 || K <= 0 || block <= 0) return BITLINEAR_ERR_INVALID_ARG;
    if ((block & (block - 1)) != 0 || block > HADAMARD_MAX_BLOCK || K % block != 0 || K % 4 != 0)
        return BITLINEAR_ERR_SHAPE;
    if (!mul_ok(M, K) || M > (int64_t)INT_MAX / ((K + 4095) / 4096)) return BITLINEAR_ERR_SHAPE;
    if (!aligned(x, 16) || (signs && !aligned(signs, 4))) return BITLINEAR_ERR_ALIGNMENT;
    return BITLINEAR_OK;
}

int bitlinear_hadamard_rows(const float* x, int64_t M, int64_t K, int64_t block, const int8_t* signs, float* out,
                            hipStream_t stream) {
    if (!out) return BITLINEAR_ERR_INVALID_ARG;
    int st = check_hadamard(x, M, K, block, signs);
    if (st) return st;
    if (!aligned(out, 16)) return BITLINEAR_ERR_ALIGNMENT;
    return hip_status(launch_hadamard_rows(x, M, K, (int)block, signs, out, stream));
}

int bitlinear_quantize_act_hadamard(const float* x, int64_t M, int64_t K, int64_t block, const int8_t* signs,
                                    int8_t* x_q, float* beta, hipStream_t stream) {
    if (!x_q || !beta) return BITLINEAR_ERR_INVALID_ARG;
    int st = check_hadamard(x, M, K, block, signs);
    if (st) return st;
    if (!aligned(x_q, 4)) return BITLINEAR_ERR_ALIGNMENT;
    return hip_status(launch_quantize_act_hadamard(x, M, K, (int)block, signs, x_q, beta, stream));
}

int bitlinear_forward_fused_hadamard(const float* x, int64_t M, int64_t K, int64_t block, const int8_t* signs,
                                     const uint8_t* W_packed, const float* alpha, int64_t N, const float* bias, float* y,
                                     int8_t* x_q, float* beta, hipStream_t stream) {
    int st = check_hadamard(x, M, K, block, signs);
    if (st) return st;
    st = check_forward(reinterpret_cast<const int8_t*>(x), x, M, K, W_packed, alpha, N, y);
    if (st) return st;
    if (gemv_hadamard_supports(M, K) && aligned(W_packed, 16) && (!x_q || aligned(x_q, 4)))
        return hip_status(launch_gemv_hadamard(x, K, (int)block, signs, W_packed, alpha, N, bias, y, x_q, beta, stream));
    // other shapes: rotation + quantization, then the forward, through x_q and beta
    if (!x_q || !beta) return BITLINEAR_ERR_INVALID_ARG;
    if (!aligned(x_q, 4)) return BITLINEAR_ERR_ALIGNMENT;
    st = hip_status(launch_quantize_act_hadamard(x, M, K, (int)block, signs, x_q, beta, stream));
    if (st) return st;
    return bitlinear_forward(x_q, beta, M, K, W_packed, alpha, N, bias, y, nullptr, stream);
}

const char* bitlinear_forward_fused_kernel(int64_t M, int64_t K, int64_t N, const float* x, const uint8_t* W_packed,
                                           const int8_t* x_q) {
    (void)N;
    // x_q given stands for x_q and beta given
    return use_fused_kernel(M, K, x, W_packed, x_q, reinterpret_cast<const float*>(x_q)) ? "gemv_fused"
                                                                                       : "quantize_act+forward";
}

const char* bitlinear_forward_kernel(int64_t M, int64_t K, int64_t N, const int8_t* x_q,
                                     const uint8_t* W_packed) {
    switch (choose_path(M, K, N, x_q, W_packed)) {
        case Path::Gemv: return "gemv_dot4";
        case Path::Decode: return "decode_mfma_i8";
        case Path::Gemm: return "gemm_mfma_i8";
        default: return "generic";
    }
}

}  // extern "C"
