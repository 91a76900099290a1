// quantize.hip -- weight (absmean ternary + 2-bit packing) and activation (per-token absmax
// int8) quantization kernels for gfx950.
//
// [P3] chenxutan.com, "1.58-bit 大模型极限量化实战" §2.3 (absmean), §2.4 (absmax), §4.1 (code),
//      §5.3 (2-bit packing 00/01/10 -> -1/0/+1).
// [P2] nxmr.cn, "1.58 位大模型" §3.1, §4.2 (per-row absmean).
//
// All of these are HBM-bound streaming kernels: float4 loads, one wave per row for the
// fp64 |W| partial sums, a flat grid-stride pass for codes and packing, one workgroup
// per token for the activations.
#include "common.hpp"

namespace bitlinear {

// ---------------------------------------------------------------------------------------
// |W| row sums in fp64.  One wave per row; lane l adds float4 chunks l, l+64, ... in
// ascending order (x, y, z, w inside a chunk), then a butterfly over the 64 lanes.  The
// order depends only on K, so the sums are bit-reproducible across runs and grids.
__global__ __launch_bounds__(256) void k_row_abs_sums(const float* __restrict__ W, int64_t N,
                                                      int64_t K, double* __restrict__ rowsum) {
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;
    const float4* row = reinterpret_cast<const float4*>(W + n * K);
    const int64_t nv = K >> 2;
    double acc = 0.0;
    int64_t c = lane;
    // two loads in flight per iteration; the additions stay in ascending chunk order
    for (; c + 64 < nv; c += 128) {
        float4 a = row[c];
        float4 b = row[c + 64];
        acc += fabs((double)a.x); acc += fabs((double)a.y); acc += fabs((double)a.z); acc += fabs((double)a.w);
        acc += fabs((double)b.x); acc += fabs((double)b.y); acc += fabs((double)b.z); acc += fabs((double)b.w);
    }
    if (c < nv) {
        float4 a = row[c];
        acc += fabs((double)a.x); acc += fabs((double)a.y); acc += fabs((double)a.z); acc += fabs((double)a.w);
    }
    acc = wave_sum_f64(acc);
    if (lane == 0) rowsum[n] = acc;
}

// alpha = fp32(sum_n rowsum[n] / (N*K)): one workgroup; thread t adds rows t, t+256, ...
// in ascending order, then a butterfly per wave and the four wave totals in wave order.
__global__ __launch_bounds__(256) void k_alpha_from_rows(const double* __restrict__ rowsum, int64_t N,
                                                         double count, float* __restrict__ alpha) {
    __shared__ double part[4];
    double acc = 0.0;
    for (int64_t i = threadIdx.x; i < N; i += 256) acc += rowsum[i];
    acc = wave_sum_f64(acc);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double s = ((part[0] + part[1]) + part[2]) + part[3];
        alpha[0] = (float)(s / count);
    }
}

// Per-row alpha [P2 §3.1]: alpha_rows[n] = fp32(rowsum_n / K), one wave per row.
__global__ __launch_bounds__(256) void k_alpha_rows(const float* __restrict__ W, int64_t N, int64_t K,
                                                    float* __restrict__ alpha_rows) {
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= N) return;
    const float4* row = reinterpret_cast<const float4*>(W + n * K);
    const int64_t nv = K >> 2;
    double acc = 0.0;
    for (int64_t c = lane; c < nv; c += 64) {
        float4 a = row[c];
        acc += fabs((double)a.x); acc += fabs((double)a.y); acc += fabs((double)a.z); acc += fabs((double)a.w);
    }
    acc = wave_sum_f64(acc);
    if (lane == 0) alpha_rows[n] = (float)(acc / (double)K);
}

// 2-bit code (W_hat + 1) of one weight: clip(rne(fp32(w / alpha)), -1, 1) + 1.
__device__ __forceinline__ uint32_t ternary_code(float w, float alpha) {
    if (alpha == 0.0f) return 1u;
    float r = rintf(w / alpha);
    r = fminf(fmaxf(r, -1.0f), 1.0f);
    return (uint32_t)((int)r + 1);
}

// Codes and packing over the flat tensor: because K % 4 == 0, packed byte b of the whole
// tensor holds flat weights 4b..4b+3.  Each work item turns 16 weights (four float4) into
// one dword.  `per_row` selects alpha[flat / K] instead of alpha[0].
template <bool PER_ROW>
__global__ __launch_bounds__(256) void k_ternary_pack(const float* __restrict__ W, int64_t total, int64_t K,
                                                      const float* __restrict__ alpha,
                                                      uint8_t* __restrict__ packed) {
    const int64_t groups = total >> 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    float a0 = PER_ROW ? 0.0f : alpha[0];
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
        const float4* p = reinterpret_cast<const float4*>(W) + g * 4;
        float4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = p[q];
        uint32_t word = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float a = a0;
            if (PER_ROW) a = alpha[(g * 16 + q * 4) / K];   // 4 weights of a byte share a row
            word |= ternary_code(v[q].x, a) << (8 * q + 0);
            word |= ternary_code(v[q].y, a) << (8 * q + 2);
            word |= ternary_code(v[q].z, a) << (8 * q + 4);
            word |= ternary_code(v[q].w, a) << (8 * q + 6);
        }
        reinterpret_cast<uint32_t*>(packed)[g] = word;
    }
    // tail: total % 16 weights (a multiple of 4) -> up to three single bytes
    if (blockIdx.x == 0 && threadIdx.x < ((total & 15) >> 2)) {
        int64_t b = groups * 4 + threadIdx.x;
        float a = PER_ROW ? alpha[(b * 4) / K] : a0;
        uint32_t byte = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) byte |= ternary_code(W[b * 4 + i], a) << (2 * i);
        packed[b] = (uint8_t)byte;
    }
}

// ---------------------------------------------------------------------------------------
// Per-token absmax int8 [P3 §2.4, §4.1].  One 256-thread workgroup per token.
__device__ __forceinline__ float block_max_256(float v, float* red) {
    v = wave_max_f32(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    return r;
}

// fp32(127 x) / beta rounded to nearest-even as an IEEE division would, formed from the
// reciprocal y = RN(1/beta): q = RN(a*y), r = a - q*beta (exact through the FMA),
// t = RN(q + r*y).  Markstein's theorem (reciprocal within half an ulp, first quotient within
// one ulp) makes t the correctly rounded quotient.
__device__ __forceinline__ uint32_t act_code(float x, float beta, float y) {
    const float a = x * 127.0f;
    const float q = a * y;
    const float r = __builtin_fmaf(-q, beta, a);
    const float t = __builtin_fmaf(r, y, q);
    const float c = __builtin_amdgcn_fmed3f(rintf(t), -127.0f, 127.0f);
    return (uint32_t)((int)c) & 0xFFu;
}

template <bool VEC>
__global__ __launch_bounds__(256) void k_quantize_act(const float* __restrict__ x, int64_t K,
                                                      int8_t* __restrict__ xq, float* __restrict__ beta) {
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const float* row = x + m * K;
    float mx = 0.0f;
    if (VEC) {
        const float4* r4 = reinterpret_cast<const float4*>(row);
        for (int64_t c = threadIdx.x; c < (K >> 2); c += 256) {
            float4 v = r4[c];
            mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    } else {
        for (int64_t c = threadIdx.x; c < K; c += 256) mx = fmaxf(mx, fabsf(row[c]));
    }
    mx = block_max_256(mx, red);
    const float b = mx + 1e-8f;
    const float y = 1.0f / b;
    if (threadIdx.x == 0) beta[m] = b;
    if (VEC) {
        const float4* r4 = reinterpret_cast<const float4*>(row);
        uint32_t* out = reinterpret_cast<uint32_t*>(xq + m * K);
        for (int64_t c = threadIdx.x; c < (K >> 2); c += 256) {
            float4 v = r4[c];
            out[c] = act_code(v.x, b, y) | (act_code(v.y, b, y) << 8) | (act_code(v.z, b, y) << 16) |
                     (act_code(v.w, b, y) << 24);
        }
    } else {
        for (int64_t c = threadIdx.x; c < K; c += 256) xq[m * K + c] = (int8_t)act_code(row[c], b, y);
    }
}

// ---------------------------------------------------------------------------------------
hipError_t launch_row_abs_sums(const float* W, int64_t N, int64_t K, double* rowsum, hipStream_t s) {
    hipLaunchKernelGGL(k_row_abs_sums, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, W, N, K, rowsum);
    return hipGetLastError();
}

hipError_t launch_alpha_from_rows(const double* rowsum, int64_t N, int64_t K, float* alpha, hipStream_t s) {
    hipLaunchKernelGGL(k_alpha_from_rows, dim3(1), dim3(256), 0, s, rowsum, N, (double)N * (double)K, alpha);
    return hipGetLastError();
}

hipError_t launch_alpha_rows(const float* W, int64_t N, int64_t K, float* alpha_rows, hipStream_t s) {
    hipLaunchKernelGGL(k_alpha_rows, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, W, N, K, alpha_rows);
    return hipGetLastError();
}

hipError_t launch_ternary_pack(const float* W, int64_t N, int64_t K, const float* alpha, bool per_row,
                               uint8_t* packed, hipStream_t s) {
    const int64_t total = N * K;
    int64_t groups = total >> 4;
    int64_t blocks = (groups + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    if (per_row)
        hipLaunchKernelGGL(k_ternary_pack<true>, dim3((unsigned)blocks), dim3(256), 0, s, W, total, K, alpha, packed);
    else
        hipLaunchKernelGGL(k_ternary_pack<false>, dim3((unsigned)blocks), dim3(256), 0, s, W, total, K, alpha, packed);
    return hipGetLastError();
}

hipError_t launch_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq, float* beta, hipStream_t s) {
    const bool vec = (K % 4 == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)xq % 4 == 0);
    if (vec)
        hipLaunchKernelGGL(k_quantize_act<true>, dim3((unsigned)M), dim3(256), 0, s, x, K, xq, beta);
    else
        hipLaunchKernelGGL(k_quantize_act<false>, dim3((unsigned)M), dim3(256), 0, s, x, K, xq, beta);
    return hipGetLastError();
}

}  // namespace bitlinear
