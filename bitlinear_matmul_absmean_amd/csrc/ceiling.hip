// ceiling.hip -- the two measured ceilings bench.py reports beside the published peaks: an HBM
// streaming read and an int8 MFMA issue loop, for gfx950.  Nothing here belongs to the
// BitLinear path; the library that holds these kernels is separate from libbitlinear.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitlinear_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// Each thread reads PER 16-byte units strided by the workgroup size (coalesced), all loads first.
constexpr int PER = 4;

__global__ __launch_bounds__(256) void k_read(const u32x4* __restrict__ p, int64_t n16, int* sink) {
    const int64_t base = (int64_t)blockIdx.x * 256 * PER + threadIdx.x;
    u32x4 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int64_t idx = base + (int64_t)i * 256;
        v[i] = idx < n16 ? __builtin_nontemporal_load(p + idx) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) acc ^= v[i].x ^ v[i].y ^ v[i].z ^ v[i].w;
    if (acc == 0x9E3779B9u) sink[blockIdx.x & 1023] = (int)acc;
}

// 16 independent accumulators per wave (no dependency stalls); operands from memory, rotated
// so consecutive MFMAs see different values.
__global__ __launch_bounds__(256) void k_mfma(const i32x4* __restrict__ src, int iters, int* sink) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    i32x4 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        a[j] = src[(t * 8 + j) & 16383];
        b[j] = src[(t * 8 + 4 + j) & 16383];
    }
    i32x16 c[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = i32x16{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                c[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(j + q) & 3], b[(j + 2 * q) & 3], c[q], 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += c[j][e];
    if (s == 0x7fffffff) sink[t & 1023] = s;
}

}  // namespace

extern "C" int bitlinear_ceiling_read(const void* src, size_t bytes, int* sink, hipStream_t stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0) return -1;
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t blocks = (n16 + 256 * PER - 1) / (256 * PER);
    hipLaunchKernelGGL(k_read, dim3((unsigned)blocks), dim3(256), 0, stream, (const u32x4*)src, n16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

extern "C" int bitlinear_ceiling_mfma(int blocks, int iters, const int* operands, int* sink, int64_t* ops_out,
                                      hipStream_t stream) {
    if (blocks <= 0 || iters <= 0 || !operands || !sink) return -1;
    hipLaunchKernelGGL(k_mfma, dim3((unsigned)blocks), dim3(256), 0, stream, (const i32x4*)operands, iters, sink);
    if (ops_out) *ops_out = (int64_t)blocks * 4 * iters * 16 * 2 * 32 * 32 * 32;
    return hipGetLastError() == hipSuccess ? 0 : -5;
}
