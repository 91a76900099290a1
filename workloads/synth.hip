// synth.hip -- device generator of the 70B-class weight stream's packed ternary codes.
//
// Input generation only (no step of the BitLinear method): SplitMix64 (Steele, Lea & Flood,
// "Fast splittable pseudorandom number generators", OOPSLA 2014) in counter form, output i
// = mix(state + (i + 1) * 0x9E3779B97F4A7C15).  Packed byte i of a projection takes output
// i and splits it into four 16-bit fields u_j; field j gives the 2-bit code at bits 2j:
// u < 20323 -> 01, u < 20323 + 22606 -> 00, else 10.  The NumPy implementation of the same
// definition is in workloads/__init__.py; the two share no code.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t sm64(uint64_t state, uint64_t i) {
    uint64_t z = state + (i + 1ull) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

__device__ __forceinline__ uint32_t packed_byte(uint64_t z) {
    uint32_t b = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t u = (uint32_t)(z >> (16 * j)) & 0xFFFFu;
        const uint32_t c = u < 20323u ? 1u : (u < 20323u + 22606u ? 0u : 2u);
        b |= c << (2 * j);
    }
    return b;
}

__global__ __launch_bounds__(256) void k_synth(uint8_t* __restrict__ out, int64_t nbytes, uint64_t state) {
    const int64_t groups = nbytes >> 4;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
        uint32_t w[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            uint32_t v = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) v |= packed_byte(sm64(state, (uint64_t)(g * 16 + d * 4 + b))) << (8 * b);
            w[d] = v;
        }
        reinterpret_cast<uint4*>(out)[g] = make_uint4(w[0], w[1], w[2], w[3]);
    }
    if (blockIdx.x == 0 && threadIdx.x < (nbytes & 15)) {
        const int64_t i = groups * 16 + threadIdx.x;
        out[i] = (uint8_t)packed_byte(sm64(state, (uint64_t)i));
    }
}

}  // namespace

// out: device buffer of nbytes bytes, 16-byte aligned.  Returns a hipError_t.
extern "C" int synth_ternary_packed(uint8_t* out, int64_t nbytes, uint64_t state, hipStream_t stream) {
    if (!out || nbytes <= 0 || ((uintptr_t)out & 15)) return (int)hipErrorInvalidValue;
    int64_t blocks = ((nbytes >> 4) + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(k_synth, dim3((unsigned)blocks), dim3(256), 0, stream, out, nbytes, state);
    return (int)hipGetLastError();
}
