// common.hpp -- shared device helpers and launch declarations for the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitlinear {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// Launch with `lds` bytes of dynamic LDS; above 64 KiB the kernel must first be allowed
// the larger allocation (gfx950 has 160 KiB of LDS per workgroup).
template <typename Kernel, typename... Args>
static inline hipError_t launch_with_lds(Kernel k, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                                         Args... args) {
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k, grid, block, lds, s, args...);
    return hipGetLastError();
}

// Wave-wide reductions.  Integer sums and float maxima are exact in any order.
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, kWave);
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v = fmaxf(v, __shfl_xor(v, s, kWave));
    return v;
}

// Butterfly sum in fp64; every lane ends with the same value, and the order of the
// additions depends only on the lane count, so the result is reproducible.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, kWave);
    return v;
}

// Dequantization scale alpha*beta/127: fp64 product and quotient, one fp32 rounding.
__device__ __forceinline__ float dequant_scale(float alpha, float beta) {
    return (float)((double)alpha * (double)beta / 127.0);
}

// y = fp32(acc) * s (+ bias) with separate roundings (the library builds with
// -ffp-contract=off, so no multiply-add is fused).
__device__ __forceinline__ float dequant(int acc, float s, const float* __restrict__ bias, int64_t n) {
    float v = (float)acc * s;
    if (bias) v = v + bias[n];
    return v;
}

// Signed 4 x int8 dot product with int32 accumulate (v_dot4_i32_i8).
__device__ __forceinline__ int dot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// 4x4 byte transpose of 16 bytes: byte j of output dword i = byte i of input dword j.
__device__ __forceinline__ u32x4 transpose4x4_bytes(u32x4 s) {
    u32x4 o;
    o.x = (s.x & 0xFFu) | ((s.y & 0xFFu) << 8) | ((s.z & 0xFFu) << 16) | ((s.w & 0xFFu) << 24);
    o.y = ((s.x >> 8) & 0xFFu) | (((s.y >> 8) & 0xFFu) << 8) | (((s.z >> 8) & 0xFFu) << 16) |
          (((s.w >> 8) & 0xFFu) << 24);
    o.z = ((s.x >> 16) & 0xFFu) | (((s.y >> 16) & 0xFFu) << 8) | (((s.z >> 16) & 0xFFu) << 16) |
          (((s.w >> 16) & 0xFFu) << 24);
    o.w = (s.x >> 24) | ((s.y >> 24) << 8) | ((s.z >> 24) << 16) | ((s.w >> 24) << 24);
    return o;
}

// 4x4 byte transpose with v_perm_b32: out[i] byte j = in[j] byte i.
__device__ __forceinline__ u32x4 transpose4x4_perm(u32x4 s) {
    const uint32_t a01l = __builtin_amdgcn_perm(s.y, s.x, 0x05010400u);   // s0b0 s1b0 s0b1 s1b1
    const uint32_t a01h = __builtin_amdgcn_perm(s.y, s.x, 0x07030602u);   // s0b2 s1b2 s0b3 s1b3
    const uint32_t a23l = __builtin_amdgcn_perm(s.w, s.z, 0x05010400u);
    const uint32_t a23h = __builtin_amdgcn_perm(s.w, s.z, 0x07030602u);
    u32x4 o;
    o.x = __builtin_amdgcn_perm(a23l, a01l, 0x05040100u);
    o.y = __builtin_amdgcn_perm(a23l, a01l, 0x07060302u);
    o.z = __builtin_amdgcn_perm(a23h, a01h, 0x05040100u);
    o.w = __builtin_amdgcn_perm(a23h, a01h, 0x07060302u);
    return o;
}

// Expansion of one packed dword (16 codes, weight 4b+i at bits 2i of byte b) into the
// 16-byte MFMA operand in weight order: byte 4b+i of the result is the code of weight 4b+i.
// Per output dword: v_perm gathers [byte b of w, byte b of w >> 2] twice, a packed 16-bit shift
// by (0, 4) brings bits 4-5 of the upper pair down, and a mask keeps bits 0-1 of every byte.
__device__ __forceinline__ i32x4 expand_codes_in_order(uint32_t w) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const uint32_t w2 = w >> 2;
    i32x4 r;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t sel = (uint32_t)b | (uint32_t)(4 + b) << 8 | (uint32_t)b << 16 | (uint32_t)(4 + b) << 24;
        u16x2 h = __builtin_bit_cast(u16x2, __builtin_amdgcn_perm(w2, w, sel));
        h = h >> (u16x2){0, 4};
        r[b] = (int)(__builtin_bit_cast(uint32_t, h) & 0x03030303u);
    }
    return r;
}

// The same with the codes mapped to signed bytes W_hat = c - 1 (v_perm with the data as its
// selector into the table {-1, 0, 1}): four instructions more per 16 codes, no sums of x_q.
__device__ __forceinline__ i32x4 expand_signed_in_order(uint32_t w) {
    const i32x4 c = expand_codes_in_order(w);
    return i32x4{(int)__builtin_amdgcn_perm(0u, 0x000100FFu, (uint32_t)c.x),
                 (int)__builtin_amdgcn_perm(0u, 0x000100FFu, (uint32_t)c.y),
                 (int)__builtin_amdgcn_perm(0u, 0x000100FFu, (uint32_t)c.z),
                 (int)__builtin_amdgcn_perm(0u, 0x000100FFu, (uint32_t)c.w)};
}

// 16 bytes per lane from global memory straight into LDS (buffer_load_dwordx4 ... lds): lane l
// writes its 16 bytes at lds + 16 l (lds the same for the whole wave), read from the buffer r at
// voff (per lane) + soff (uniform).  Offsets past the buffer's size would read zeros; every
// caller keeps them inside.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, i32x4* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
// Buffer resource over [p, p + bytes) for raw (untyped) loads: stride 0, 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

// Workgroup barrier that orders LDS accesses only: global loads in flight (a prefetch) stay
// in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sum of the four signed bytes of a dword.
__device__ __forceinline__ int byte_sum(uint32_t v) { return dot4(v, 0x01010101u, 0); }

// The add/sub sum of one 64-weight chunk: codes c = W_hat + 1 in 2-bit fields; field i of a
// code dword, masked in place, holds c * 4^i per byte (field 3 is shifted down so it stays
// below 128); each field meets its transposed activations in v_dot4_i32_i8, the four sums
// are recombined exactly, and sum (c - 1) x = sum c x - sum x.
__device__ __forceinline__ int chunk_sum(const u32x4& w, const u32x4* xs, int stride, int xsum) {
    int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
    const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const u32x4 t = xs[d * stride];
        a0 = dot4(wd[d] & 0x03030303u, t.x, a0);
        a1 = dot4(wd[d] & 0x0C0C0C0Cu, t.y, a1);
        a2 = dot4(wd[d] & 0x30303030u, t.z, a2);
        a3 = dot4((wd[d] >> 6) & 0x03030303u, t.w, a3);
    }
    return a0 + (a1 >> 2) + (a2 >> 4) + a3 - xsum;
}

// ---- launch wrappers (one per kernel family), defined in the .hip files -------------------
// Rows of the fixed scratch of the allocation-free weight quantization, and the device address
// of the current device's copy of it (looked up once per device).
constexpr int64_t kQuantizeScratchRows = 262144;
hipError_t quantize_weights_scratch(double** out);
hipError_t launch_row_abs_sums(const float* W, int64_t N, int64_t K, double* rowsum, hipStream_t s);
hipError_t launch_alpha_from_rows(const double* rowsum, int64_t N, int64_t K, float* alpha, hipStream_t s);
hipError_t launch_alpha_rows(const float* W, int64_t N, int64_t K, float* alpha_rows, hipStream_t s);
hipError_t launch_ternary_pack(const float* W, int64_t N, int64_t K, const float* alpha, bool per_row,
                               uint8_t* packed, hipStream_t s);
hipError_t launch_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq, float* beta, hipStream_t s);
// Five ternary codes per byte (base 3), rows of 16 ceil(K / 80) bytes.
int64_t t5_row_bytes(int64_t K);
bool t5_supports(int64_t K);
hipError_t launch_pack_t5(const float* W, int64_t N, int64_t K, const float* alpha, uint8_t* out, hipStream_t s);
hipError_t launch_repack_t5(const uint8_t* w2, int64_t N, int64_t K, uint8_t* out, hipStream_t s);
hipError_t launch_forward_t5(const int8_t* xq, const float* beta, int64_t M, int64_t K, const uint8_t* wp,
                             const float* alpha, int64_t N, const float* bias, float* y, hipStream_t s);
// Block scales: one alpha per 128 consecutive weights of a row, alpha [N, K / 128].
hipError_t launch_quantize_blocks(const float* W, int64_t N, int64_t K, uint8_t* packed, float* alpha, hipStream_t s);
bool blocks_supports(int64_t K);
hipError_t launch_forward_blocks(const int8_t* xq, const float* beta, int64_t M, int64_t K, const uint8_t* wp,
                                 const float* alpha, int64_t N, const float* bias, float* y, hipStream_t s);
// Randomized Hadamard rotation along K (blocks of `block`, a power of two <= HADAMARD_MAX_BLOCK
// dividing K; K % 4 == 0; x/out 16-byte aligned, signs and xq 4-byte aligned).
constexpr int64_t HADAMARD_MAX_BLOCK = 4096;
hipError_t launch_hadamard_rows(const float* x, int64_t M, int64_t K, int block, const int8_t* signs,
                                float* out, hipStream_t s);
bool gemv_hadamard_supports(int64_t M, int64_t K);
hipError_t launch_gemv_hadamard(const float* x, int64_t K, int block, const int8_t* signs, const uint8_t* wp,
                                const float* alpha, int64_t N, const float* bias, float* y, int8_t* xq_out,
                                float* beta_out, hipStream_t s);
hipError_t launch_quantize_act_hadamard(const float* x, int64_t M, int64_t K, int block, const int8_t* signs,
                                        int8_t* xq, float* beta, hipStream_t s);

struct ForwardArgs {
    const int8_t* xq;
    const float* beta;
    int64_t M, K, N;
    const uint8_t* wp;
    const float* alpha;   // [1] or [N]
    bool alpha_per_row;
    const float* bias;
    float* y;
    int32_t* acc;
    int act = 0;          // activation applied to y after the dequantization: 0 none, 1 GELU
};

// GELU (the exact, erf-based GELU of torch.nn.GELU) between the two BitLinears of the BitMLP
// [P3 §6.1]: h Phi(h) with Phi(h) = erfc(-h / sqrt 2) / 2, the complementary form, in which no
// term cancels for negative h (1 + erf(h / sqrt 2) loses every digit below h = -8.3), evaluated
// in fp64 as (0.5 h) erfc(-h * RN64(1/sqrt 2)) and rounded to fp32 once.  This is that formula
// with the library erfc; the fast path below falls back to it whenever it cannot decide the
// rounding (inlined there, so that the GELU functions make no calls and save nothing to
// scratch).
__device__ __forceinline__ float gelu_f32_erf(float h) {
    const double v = (double)h;
    return (float)(0.5 * v * erfc(-v * 0.70710678118654752440));
}

// Fast GELU in fp64 without branches: GELU(v) = v Phi(v) with Phi(v) = erfc(y) / 2 for v < 0 and
// 1 - erfc(y) / 2 otherwise, y = |v| / sqrt 2, erfc(y) = exp(-v^2 / 2) erfcx(y), and erfcx as a
// degree-16 polynomial in u = S (2 / (2 + y)) + O (Chebyshev interpolation on y in [0, 5.7], the
// variable t = 2 / (2 + y) of the classical erfc expansions; u is clamped at y = 5.7, where
// erfc < 2e-15).  Measured against long-double erfcl over v >= -4: relative error below 2e-14.
// The coefficients come from csrc/fit_gelu.py.
namespace gelu_poly {
constexpr double kS2 = 2.0 * 2.7017543859649122, kO = -1.7017543859649122;
constexpr double kC[17] = {
    0.3840490174908751, 0.4210641425092814, 0.16628657095956959, 0.031638468914700096,
    -0.0016874574521908601, -0.0015499149004059385, 0.00013185815934692365, 8.957503665028618e-05,
    -2.0876744374376674e-05, -3.47183505293702e-06, 2.4538737264270885e-06, -2.7035081443788403e-07,
    -1.586981502844185e-07, 7.209803422744851e-08, -4.939635762515718e-09, -5.870114231300212e-09,
    1.7485565120006436e-09};
}  // namespace gelu_poly

__device__ __forceinline__ double gelu_approx(double v) {
    const double y = fabs(v) * 0.70710678118654752440;
    const double d = 2.0 + y;
    double r = __builtin_amdgcn_rcp(d);                 // 1 / d, two Newton steps to full precision
    r = fma(r, fma(-d, r, 1.0), r);
    r = fma(r, fma(-d, r, 1.0), r);
    const double u = fmax(fma(r, gelu_poly::kS2, gelu_poly::kO), -1.0);
    double e = gelu_poly::kC[16];
#pragma unroll
    for (int i = 15; i >= 0; --i) e = fma(e, u, gelu_poly::kC[i]);
    const double q = exp(-0.5 * v * v) * e;            // erfc(y); -v^2 / 2 is exact for fp32 v
    return v * (v < 0.0 ? 0.5 * q : fma(-0.5, q, 1.0));
}

// The fp32 rounding of the fp64 formula, decided from the approximation c when possible (Ziv's
// rounding test): c is within 2e-14 |GELU(v)| of the exact value (measured against long-double
// erfcl), and for v >= -4 the formula evaluated in fp64 is within 3e-15 |GELU(v)| of it (the
// argument's rounding, scaled by at most 2 z^2 + 1 = 17 through erfc, erfc's own few ulps and
// the product's rounding), so tol covers both.  When c - tol and c + tol round to the same
// fp32 value, so do the exact value and the formula.  Not attempted for v < -4, where the
// polynomial's range and error bound end, nor for NaN and infinity: those take the formula.
__device__ __forceinline__ bool gelu_decided(double v, double c, float& g) {
    const double tol = fma(fabs(c), 6e-14, 2.5e-16 * fabs(v));
    g = (float)c;
    return v >= -4.0 && (float)(c - tol) == (float)(c + tol);
}

__device__ __attribute__((noinline)) float gelu_f32(float h) {
    float g;
    if (gelu_decided((double)h, gelu_approx((double)h), g)) return g;
    return gelu_f32_erf(h);
}

// Four GELUs per call: the four evaluations are independent, so their dependency chains
// interleave (the epilogue of the MFMA GEMM runs at two waves per SIMD and would otherwise
// wait on each chain in turn).
__device__ __attribute__((noinline)) float4 gelu4_f32(float4 h) {
    const float hv[4] = {h.x, h.y, h.z, h.w};
    double c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = gelu_approx((double)hv[i]);
    float g[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ok[i] = gelu_decided((double)hv[i], c[i], g[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (!ok[i]) g[i] = gelu_f32_erf(hv[i]);
    return make_float4(g[0], g[1], g[2], g[3]);
}

__device__ __forceinline__ float activate(float v, int act) { return act == 1 ? gelu_f32(v) : v; }

bool gemv_supports(int64_t M, int64_t K);
struct GemvShape {
    int waves_per_wg;         // 4 or 8
    int64_t waves_target;     // waves the grid aims at
};
GemvShape gemv_shape(int64_t M, int64_t K, int64_t N, bool fused);
hipError_t launch_gemv_dot4(const ForwardArgs& a, hipStream_t s);
hipError_t launch_gemv_fused(const ForwardArgs& a, const float* x, int8_t* xq_out, float* beta_out, hipStream_t s);
bool gemm_supports_k(int64_t K);
hipError_t launch_gemm_mfma(const ForwardArgs& a, hipStream_t s);
bool decode_mfma_supports(int64_t M, int64_t K);
hipError_t launch_decode_mfma(const ForwardArgs& a, hipStream_t s);
hipError_t launch_forward_generic(const ForwardArgs& a, hipStream_t s);

}  // namespace bitlinear
