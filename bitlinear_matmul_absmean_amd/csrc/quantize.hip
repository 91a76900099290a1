// quantize.hip -- weight (absmean ternary + 2-bit packing) and activation (per-token absmax
// int8) quantization kernels for gfx950.
//
// [P3] chenxutan.com, "1.58-bit 大模型极限量化实战" §2.3 (absmean), §2.4 (absmax), §4.1 (code),
//      §5.3 (2-bit packing 00/01/10 -> -1/0/+1).
// [P2] nxmr.cn, "1.58 位大模型" §3.1, §4.2 (per-row absmean).
// [P3] §6.2: the randomized Hadamard rotation of the activations (and, offline, of the
//      weight rows) before the absmax.
//
// All of these are HBM-bound streaming kernels: float4 loads, one wave per row for the
// fp64 |W| partial sums, a flat grid-stride pass for codes and packing, one workgroup
// per token for the activations.
#include <cmath>
#include <mutex>

#include "common.hpp"

namespace bitlinear {

// ---------------------------------------------------------------------------------------
// Fixed scratch of the allocation-free weight quantization: the fp64 |W| row sums of up to
// kQuantizeScratchRows rows (2 MiB).  Each device holds its own copy until the process ends.
// Host code never passes `scratch` itself to a kernel (in host code the name stands for a
// host-side shadow, not a device address): quantize_weights_scratch() looks up the device
// address once per device, with that device current, and every launch takes that pointer.
static __device__ __align__(256) double scratch[kQuantizeScratchRows];

hipError_t quantize_weights_scratch(double** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static double* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = static_cast<double*>(p);
    }
    *out = addr[dev];
    return hipSuccess;
}

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
// Block scales [P1 §2.3, §4.2]: alpha[n, b] = mean |W| over the 128 weights of block b of row
// n.  In row-major W the blocks are consecutive, so W is a flat array of N K / 128 blocks and
// the codes of block i are packed bytes 32 i .. 32 i + 31.  A wave takes two blocks per step
// (lanes 0-31 the first, 32-63 the second, one float4 per lane); the fp64 |w| sum runs over
// the half-wave in a fixed butterfly, then each lane packs its four codes into one byte.  W
// is read once.
__global__ __launch_bounds__(256) void k_quantize_blocks(const float* __restrict__ W, int64_t nblocks,
                                                         float* __restrict__ alpha, uint8_t* __restrict__ packed) {
    const int lane = threadIdx.x & 63, half = lane >> 5, hl = lane & 31;
    const int64_t waves = (int64_t)gridDim.x * 4;
    for (int64_t p = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6; 2 * p < nblocks; p += waves) {
        const int64_t blk = 2 * p + half;
        const bool ok = blk < nblocks;
        const float4 v = reinterpret_cast<const float4*>(W)[(ok ? blk : 2 * p) * 32 + hl];
        double s = (double)fabsf(v.x) + (double)fabsf(v.y) + (double)fabsf(v.z) + (double)fabsf(v.w);
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) s += __shfl_xor(s, o, kWave);
        const float a = (float)(s / 128.0);
        if (ok) {
            if (hl == 0) alpha[blk] = a;
            packed[blk * 32 + hl] = (uint8_t)(ternary_code(v.x, a) | (ternary_code(v.y, a) << 2) |
                                              (ternary_code(v.z, a) << 4) | (ternary_code(v.w, a) << 6));
        }
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

// Four codes, packed little-endian, of values with |x| <= beta (true for every element of the
// row beta was taken from).  The quotient t = fp32(127 x) / beta is formed as in act_code and
// satisfies |t| < 127.5, so the clip of the definition never acts; adding 1.5 * 2^23 rounds t
// half-to-even to an integer held in the low mantissa bits, whose low byte is the two's
// complement code.  v_perm gathers the four bytes.  m127 = 127 s with s a power of two
// (the unapplied rotation scale) gives the same codes: fp32(fp32(x s) 127) = fp32(x (127 s))
// whenever x s is normal, and where it is subnormal both quotients round to code 0, since
// beta >= 1e-8.
__device__ __forceinline__ uint32_t act_codes4(float x0, float x1, float x2, float x3, float beta, float y,
                                              float m127 = 127.0f) {
    auto code = [&](float x) {
        const float a = x * m127;
        const float q = a * y;
        const float r = __builtin_fmaf(-q, beta, a);
        const float t = __builtin_fmaf(r, y, q);
        return __float_as_uint(t + 12582912.0f);
    };
    const uint32_t lo = __builtin_amdgcn_perm(code(x1), code(x0), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(code(x3), code(x2), 0x04000c0cu);
    return lo | hi;
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
            out[c] = act_codes4(v.x, v.y, v.z, v.w, b, y);
        }
    } else {
        for (int64_t c = threadIdx.x; c < K; c += 256) xq[m * K + c] = (int8_t)act_code(row[c], b, y);
    }
}

// The same codes in one pass, for K <= 32768 (K % 4 == 0, x 16-byte and x_q 4-byte aligned):
// NT threads per token, each holding its V float4 of the row in registers, all loads issued
// before the first use.  (The loop above waits on each load in turn and reads x twice.)
// Indexes past the row re-read its last float4, which leaves the maximum unchanged; their
// codes are not stored.
template <int V, int NT>
__global__ __launch_bounds__(NT) void k_quantize_act_row(const float* __restrict__ x, int64_t K,
                                                         int8_t* __restrict__ xq, float* __restrict__ beta) {
    __shared__ float red[NT / 64];
    const int64_t m = blockIdx.x;
    const float4* r4 = reinterpret_cast<const float4*>(x + m * K);
    const int K4 = (int)(K >> 2);
    float4 v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] = r4[min((int)threadIdx.x + NT * j, K4 - 1)];
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < V; ++j)
        mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    mx = wave_max_f32(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < NT / 64; ++w) r = fmaxf(r, red[w]);
    const float b = r + 1e-8f;
    const float y = 1.0f / b;
    if (threadIdx.x == 0) beta[m] = b;
    uint32_t* out = reinterpret_cast<uint32_t*>(xq + m * K);
#pragma unroll
    for (int j = 0; j < V; ++j) {
        const int c = (int)threadIdx.x + NT * j;
        if (c < K4)
            out[c] = act_codes4(v[j].x, v[j].y, v[j].z, v[j].w, b, y);
    }
}

// ---------------------------------------------------------------------------------------
// Randomized Hadamard rotation [P3 §6.2] along K: sign flip by d[k] (negative int8 = flip),
// the Sylvester transform of order B on each block of B consecutive elements, then one fp32
// multiply by fp32(1/sqrt(B)).  The transform is evaluated as butterflies (a, b) -> (a + b,
// a - b) on pairs (j, j + h) with h = 1, 2, 4, ..., B/2 in that order, so every result has a
// fixed rounding sequence whatever the thread layout.
//
// A workgroup of 256 threads rotates a chunk of 4096 consecutive elements of a row (blocks
// never straddle chunks: B divides both K and 4096).  The 12 index bits of a chunk element are
// combined while they are register indices of the 16 values a thread holds, in three layouts:
//   L0  v[4q + i] = element 4t + 1024q + i      (coalesced float4 loads, code stores)
//       register strides 1, 2 -> h = 1, 2;  register strides 4, 8 -> h = 1024, 2048
//   L1  v[j] = element (t & 3) + 4j + 64((t >> 2) & 15) + 1024(t >> 6)      h = 4 .. 32
//   L2  v[j] = element (t & 63) + 64j + 1024(t >> 6)                        h = 64 .. 512
// The order is L0 (h = 1, 2), L1, L2, back to L0 (h = 1024, 2048), through LDS, skipping the
// layouts whose strides are all >= B.  A ragged last chunk holds zeros past its end; whole
// blocks are zero there, so they never mix with real data.
constexpr int HAD_CHUNK = 4096;
constexpr int HAD_LDS = HAD_CHUNK + HAD_CHUNK / 16;   // 4 words of padding per 64 elements

// LDS word of chunk element e; the padding makes every layout's access conflict-free.
__device__ __forceinline__ int had_addr(int e) { return e + ((e >> 6) << 2); }

// Butterflies between registers j and j + rs (rs = 1, 2, 4 or 8): lower + upper, lower - upper.
__device__ __forceinline__ void had_stage(float (&v)[16], int rs) {
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        if (!(j & rs)) {
            const float a = v[j], b = v[j + rs];
            v[j] = a + b;
            v[j + rs] = a - b;
        }
    }
}

// Block size known at compile time (FixedBlock<B>) or only at run time (int).  With a fixed
// block every stage test folds away, and the register renaming of the butterflies needs no
// moves at the joins of skipped stages.
template <int B>
struct FixedBlock {
    __device__ constexpr operator int() const { return B; }
};

// Register strides 1, 2, 4, 8 standing for element strides base, 2 base, 4 base, 8 base.
template <typename Blk>
__device__ __forceinline__ void had_stages16(float (&v)[16], int base, Blk block) {
    if (base < (int)block) had_stage(v, 1);
    if (2 * base < (int)block) had_stage(v, 2);
    if (4 * base < (int)block) had_stage(v, 4);
    if (8 * base < (int)block) had_stage(v, 8);
}

// SCALE = false leaves the final multiply by fp32(1/sqrt(B)) to the caller.
// t: this thread's index in the 256-thread group that rotates the chunk (every thread of the
// workgroup must call it the same number of times: it holds workgroup barriers).
template <bool SCALE = true, typename Blk>
__device__ __forceinline__ void hadamard_chunk(float (&v)[16], Blk block_, float scale, float* buf,
                                               int t = threadIdx.x) {
    const int block = (int)block_;
    if (block > 1) had_stage(v, 1);
    if (block > 2) had_stage(v, 2);
    if (block > 4) {
        lds_barrier();                                  // buf is free again
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(buf + had_addr(4 * t + 1024 * q)) =
                make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
        lds_barrier();
        // each element returns to the word it came from: one owner per word in each layout
        const int e1 = (t & 3) + 64 * ((t >> 2) & 15) + 1024 * (t >> 6);
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = buf[had_addr(e1 + 4 * j)];
        had_stages16(v, 4, block_);
#pragma unroll
        for (int j = 0; j < 16; ++j) buf[had_addr(e1 + 4 * j)] = v[j];
        lds_barrier();
        if (block > 64) {
            const int e2 = (t & 63) + 1024 * (t >> 6);
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = buf[had_addr(e2 + 64 * j)];
            had_stages16(v, 64, block_);
#pragma unroll
            for (int j = 0; j < 16; ++j) buf[had_addr(e2 + 64 * j)] = v[j];
            lds_barrier();
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 f = *reinterpret_cast<const float4*>(buf + had_addr(4 * t + 1024 * q));
            v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
        }
        if (block > 1024) had_stage(v, 4);
        if (block > 2048) had_stage(v, 8);
    }
    if constexpr (SCALE) {
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = v[j] * scale;
    }
}

// Load thread t's 16 elements of chunk [c0, c0 + len) of a row (len % 4 == 0) in layout L0,
// with the sign flips applied (an exact sign-bit toggle); zeros past the end.
__device__ __forceinline__ void load_chunk(const float* __restrict__ row, const int8_t* __restrict__ signs,
                                           int64_t c0, int len, float (&v)[16], int t = threadIdx.x) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * t + 1024 * q;
        float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
        uint32_t sg = 0;
        if (e < len) {
            f = *reinterpret_cast<const float4*>(row + c0 + e);
            if (signs) sg = *reinterpret_cast<const uint32_t*>(signs + c0 + e) & 0x80808080u;
        }
        v[4 * q + 0] = __uint_as_float(__float_as_uint(f.x) ^ (sg << 24));
        v[4 * q + 1] = __uint_as_float(__float_as_uint(f.y) ^ ((sg << 16) & 0x80000000u));
        v[4 * q + 2] = __uint_as_float(__float_as_uint(f.z) ^ ((sg << 8) & 0x80000000u));
        v[4 * q + 3] = __uint_as_float(__float_as_uint(f.w) ^ (sg & 0x80000000u));
    }
}

__device__ __forceinline__ int chunk_len(int64_t K, int64_t c0) {
    return K - c0 < HAD_CHUNK ? (int)(K - c0) : HAD_CHUNK;
}

// One workgroup per (row, chunk): out = rotated x.  Every element is read into registers
// before any is written, and a workgroup writes only its own chunk, so out may equal x.
__global__ __launch_bounds__(256) void k_hadamard_rows(const float* x, int64_t K, int64_t chunks, int block,
                                                       float scale, const int8_t* __restrict__ signs,
                                                       float* out) {
    __shared__ float buf[HAD_LDS];
    const int64_t row = blockIdx.x / chunks;
    const int64_t c0 = (blockIdx.x - row * chunks) * HAD_CHUNK;
    const int len = chunk_len(K, c0);
    float v[16];
    load_chunk(x + row * K, signs, c0, len, v);
    hadamard_chunk(v, block, scale, buf);
    float* o = out + row * K + c0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * threadIdx.x + 1024 * q;
        if (e < len) *reinterpret_cast<float4*>(o + e) = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
}

__device__ __forceinline__ void store_codes(int8_t* __restrict__ xrow, int64_t c0, int len, const float (&v)[16],
                                            float b, float y, int t = threadIdx.x) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = 4 * t + 1024 * q;
        if (e < len)
            *reinterpret_cast<uint32_t*>(xrow + c0 + e) = act_codes4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], b, y);
    }
}

// Rotation then per-token absmax int8 [P3 §6.2, §2.4]: one workgroup per token.  With
// CH > 0 the row (at most CH chunks) stays in registers between the max and the codes; with
// CH == 0 (long rows) each chunk is rotated twice, once for the max and once for the codes,
// with identical results.
template <int CH>
__global__ __launch_bounds__(256) void k_quantize_act_hadamard(const float* __restrict__ x, int64_t K, int block,
                                                               float scale, const int8_t* __restrict__ signs,
                                                               int8_t* __restrict__ xq, float* __restrict__ beta) {
    __shared__ float buf[HAD_LDS];
    __shared__ float red[4];
    const int64_t m = blockIdx.x;
    const float* row = x + m * K;
    int8_t* xrow = xq + m * K;
    float mx = 0.0f;
    if constexpr (CH > 0) {
        float v[CH][16];
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int64_t c0 = (int64_t)c * HAD_CHUNK;
            if (c0 < K) {
                load_chunk(row, signs, c0, chunk_len(K, c0), v[c]);
                hadamard_chunk(v[c], block, scale, buf);
#pragma unroll
                for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(v[c][j]));
            }
        }
        mx = block_max_256(mx, red);
        const float b = mx + 1e-8f;
        const float y = 1.0f / b;
        if (threadIdx.x == 0) beta[m] = b;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int64_t c0 = (int64_t)c * HAD_CHUNK;
            if (c0 < K) store_codes(xrow, c0, chunk_len(K, c0), v[c], b, y);
        }
    } else {
        float v[16];
        for (int64_t c0 = 0; c0 < K; c0 += HAD_CHUNK) {
            load_chunk(row, signs, c0, chunk_len(K, c0), v);
            hadamard_chunk(v, block, scale, buf);
#pragma unroll
            for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(v[j]));
        }
        mx = block_max_256(mx, red);
        const float b = mx + 1e-8f;
        const float y = 1.0f / b;
        if (threadIdx.x == 0) beta[m] = b;
        for (int64_t c0 = 0; c0 < K; c0 += HAD_CHUNK) {
            load_chunk(row, signs, c0, chunk_len(K, c0), v);
            hadamard_chunk(v, block, scale, buf);
            store_codes(xrow, c0, chunk_len(K, c0), v, b, y);
        }
    }
}

// Long rows of few tokens: four groups of 256 threads rotate four chunks at once, each in
// its own LDS buffer (dynamic, 4 x HAD_LDS floats); group g takes chunks g, g + 4, ... in
// RND rounds.  A group without a chunk in a round rotates zeros, so every thread meets the
// same barriers.  The rotated row stays in registers between the max and the codes.
template <int RND>
__global__ __launch_bounds__(1024) void k_quantize_act_hadamard_wide(const float* __restrict__ x, int64_t K,
                                                                    int block, float scale,
                                                                    const int8_t* __restrict__ signs,
                                                                    int8_t* __restrict__ xq,
                                                                    float* __restrict__ beta) {
    extern __shared__ float hbuf[];
    __shared__ float red[16];
    const int64_t m = blockIdx.x;
    const int g = threadIdx.x >> 8, t = threadIdx.x & 255;
    const float* row = x + m * K;
    int8_t* xrow = xq + m * K;
    float* buf = hbuf + g * HAD_LDS;
    float v[RND][16];
#pragma unroll
    for (int r = 0; r < RND; ++r) {
        const int64_t c0 = (int64_t)(4 * r + g) * HAD_CHUNK;
        load_chunk(row, signs, c0, c0 < K ? chunk_len(K, c0) : 0, v[r], t);
    }
    float mx = 0.0f;
#pragma unroll
    for (int r = 0; r < RND; ++r) {
        hadamard_chunk(v[r], block, scale, buf, t);
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(v[r][j]));   // zeros past K: no effect
    }
    mx = wave_max_f32(mx);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    float r16 = red[0];
#pragma unroll
    for (int w = 1; w < 16; ++w) r16 = fmaxf(r16, red[w]);
    const float b = r16 + 1e-8f;
    const float y = 1.0f / b;
    if (threadIdx.x == 0) beta[m] = b;
#pragma unroll
    for (int r = 0; r < RND; ++r) {
        const int64_t c0 = (int64_t)(4 * r + g) * HAD_CHUNK;
        if (c0 < K) store_codes(xrow, c0, chunk_len(K, c0), v[r], b, y, t);
    }
}

// Rows of K = 1024 NQ elements (NQ = 1..4), the prefill shapes: each workgroup walks rows
// m = blockIdx.x, + gridDim.x, ... and issues the loads of its next row (clamped to the last
// row) before it rotates and quantizes the current one, so HBM traffic overlaps the
// arithmetic.  The signs are loaded once.  With K a multiple of 1024 every thread owns whole
// float4 groups q < NQ, so loads and stores carry no guards and the compiler waits on the
// prefetch alone, never on the previous row's stores.
template <int NQ, bool FULL>
__global__ __launch_bounds__(256) void k_quantize_act_hadamard_pipe(const float* __restrict__ x, int64_t M,
                                                                    int block_rt, float scale,
                                                                    const int8_t* __restrict__ signs,
                                                                    int8_t* __restrict__ xq, float* __restrict__ beta) {
    constexpr int K = 1024 * NQ;
    // full-row block of 4^n elements: the scale 2^-n is exact and is applied to the max and
    // folded into the factor 127 instead of to every element (identical results)
    constexpr bool FOLD = FULL && (K == 1024 || K == 4096);
    __shared__ float buf[HAD_LDS];
    __shared__ float red[2][4];
    const int t = threadIdx.x;
    const bool wave0 = __builtin_amdgcn_readfirstlane(t >> 6) == 0;
    uint32_t sg[4] = {0u, 0u, 0u, 0u};
    if (signs) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) sg[q] = *reinterpret_cast<const uint32_t*>(signs + 4 * t + 1024 * q) & 0x80808080u;
    }
    float4 nx[NQ];
    int64_t m = blockIdx.x;
    {
        const float* row = x + (m < M ? m : M - 1) * (int64_t)K;
#pragma unroll
        for (int q = 0; q < NQ; ++q) nx[q] = *reinterpret_cast<const float4*>(row + 4 * t + 1024 * q);
    }
    // The first row is peeled so that the loop is entered, like its back edge, with the
    // prefetch followed by the previous row's stores: the wait at the loop head then leaves
    // those stores in flight.
    auto row_step = [&](int64_t m, int it) {
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 f = q < NQ ? nx[q < NQ ? q : 0] : make_float4(0.f, 0.f, 0.f, 0.f);
            v[4 * q + 0] = __uint_as_float(__float_as_uint(f.x) ^ (sg[q] << 24));
            v[4 * q + 1] = __uint_as_float(__float_as_uint(f.y) ^ ((sg[q] << 16) & 0x80000000u));
            v[4 * q + 2] = __uint_as_float(__float_as_uint(f.z) ^ ((sg[q] << 8) & 0x80000000u));
            v[4 * q + 3] = __uint_as_float(__float_as_uint(f.w) ^ (sg[q] & 0x80000000u));
        }
        {
            const int64_t mn = m + gridDim.x;
            const float* row = x + (mn < M ? mn : M - 1) * (int64_t)K;
#pragma unroll
            for (int q = 0; q < NQ; ++q) nx[q] = *reinterpret_cast<const float4*>(row + 4 * t + 1024 * q);
        }
        if constexpr (FULL) hadamard_chunk<!FOLD>(v, FixedBlock<K>{}, scale, buf);   // one block per row
        else hadamard_chunk(v, block_rt, scale, buf);
        float mx = 0.0f;
#pragma unroll
        for (int j = 0; j < 4 * NQ; ++j) mx = fmaxf(mx, fabsf(v[j]));
        mx = wave_max_f32(mx);
        float* rd = red[it & 1];                  // alternate buffers: no barrier needed before reuse
        if ((t & 63) == 0) rd[t >> 6] = mx;
        lds_barrier();
        mx = fmaxf(fmaxf(rd[0], rd[1]), fmaxf(rd[2], rd[3]));
        if constexpr (FOLD) mx = mx * scale;      // = the max of the scaled values (monotone rounding)
        const float b = mx + 1e-8f;
        const float y = 1.0f / b;
        const float m127 = FOLD ? 127.0f * scale : 127.0f;
        if (wave0) beta[m] = b;                   // every lane of wave 0 stores the same value
        int8_t* xrow = xq + m * (int64_t)K;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            *reinterpret_cast<uint32_t*>(xrow + 4 * t + 1024 * q) =
                act_codes4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], b, y, m127);
    };
    if (m >= M) return;
    row_step(m, 0);
    int it = 1;
    for (m += gridDim.x; m < M; m += gridDim.x, ++it) row_step(m, it);
}

// ---------------------------------------------------------------------------------------
// Rotation, quantization and the decode GEMV in one launch (one token, K <= 16384) [P3 §6.2,
// §2.4, §3.2].  A workgroup of HALVES x four waves loads x (branch-free, so the weight loads
// issued right after stay in flight); its 256-thread halves rotate alternate 4096-element
// chunks as quantize_act_hadamard does (two halves when K spans several chunks, so that they
// rotate in parallel; one otherwise, with no idle waves), the workgroup takes the absmax, writes the codes to LDS,
// transposes each 16-byte group 4x4 into the operand layout of the GEMV and streams its rows:
// each wave holds R rows of CPL 64-weight chunks per lane in registers, loaded before the
// rotation starts.  The results equal those of quantize_act_hadamard followed by
// bitlinear_forward, bit for bit.
struct RotGemvArgs {
    const float* x;
    int64_t K;
    int block;
    float scale;
    const int8_t* signs;
    const uint8_t* wp;
    const float* alpha;
    int64_t N;
    const float* bias;
    float* y;
    int8_t* xq_out;
    float* beta_out;
    int64_t rows_per_wave;
};

// CS chunk slots per half (chunk HALVES s + half), CPL 64-weight chunks per lane and row, R
// rows per wave.
template <int HALVES, int CS, int CPL, int R>
__global__ __launch_bounds__(256 * HALVES) void k_gemv_hadamard(RotGemvArgs a) {
    constexpr int RG_WAVES = 4 * HALVES;
    extern __shared__ u32x4 xs[];                 // [CPL][4][64] transposed groups of x_q
    __shared__ float buf[HALVES][HAD_LDS];        // each half's rotation exchange; then the x_q byte row
    __shared__ float red[RG_WAVES];
    __shared__ int redi[RG_WAVES];
    const int t = threadIdx.x, lane = t & 63, half = HALVES == 1 ? 0 : t >> 8, th = t & 255;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int64_t K = a.K, N = a.N;
    const int K64 = (int)(K >> 6);

    // x: chunk HALVES s + half, float4 group q of thread th = elements c0 + 4 th + 1024 q; clamped
    // address, masked value
    float4 xv[CS][4];
    uint32_t keep[CS][4], sg[CS][4];
#pragma unroll
    for (int c = 0; c < CS; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t e = (int64_t)(HALVES * c + half) * HAD_CHUNK + 4 * th + 1024 * q;
            const bool ok = e < K;
            const int64_t ec = ok ? e : 0;
            keep[c][q] = ok ? 0xFFFFFFFFu : 0u;
            xv[c][q] = *reinterpret_cast<const float4*>(a.x + ec);
            sg[c][q] = a.signs ? *reinterpret_cast<const uint32_t*>(a.signs + ec) & 0x80808080u : 0u;
        }
    // this wave's weight rows, every load issued now
    const int64_t r0 = ((int64_t)blockIdx.x * RG_WAVES + wave) * a.rows_per_wave;
    const int64_t r1 = r0 + a.rows_per_wave < N ? r0 + a.rows_per_wave : N;
    const u32x4* wp = reinterpret_cast<const u32x4*>(a.wp);
    u32x4 w[R][CPL];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int64_t row = r0 + r < r1 ? r0 + r : r1 - 1;
        row = row < 0 ? 0 : row;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int cc = lane + 64 * j < K64 ? lane + 64 * j : 0;
            w[r][j] = wp[row * K64 + cc];
        }
    }

    float v[CS][16];
    float mx = 0.0f;
#pragma unroll
    for (int c = 0; c < CS; ++c) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 f = xv[c][q];
            v[c][4 * q + 0] = __uint_as_float((__float_as_uint(f.x) & keep[c][q]) ^ (sg[c][q] << 24));
            v[c][4 * q + 1] = __uint_as_float((__float_as_uint(f.y) & keep[c][q]) ^ ((sg[c][q] << 16) & 0x80000000u));
            v[c][4 * q + 2] = __uint_as_float((__float_as_uint(f.z) & keep[c][q]) ^ ((sg[c][q] << 8) & 0x80000000u));
            v[c][4 * q + 3] = __uint_as_float((__float_as_uint(f.w) & keep[c][q]) ^ (sg[c][q] & 0x80000000u));
        }
        // both halves rotate in every slot (a chunk past K holds zeros), so barriers match
        hadamard_chunk(v[c], a.block, a.scale, buf[half], th);
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(v[c][j]));
    }
    mx = wave_max_f32(mx);
    if (lane == 0) red[wave] = mx;
    lds_barrier();                                // also: every rotation read of buf is done
    mx = red[0];
#pragma unroll
    for (int i = 1; i < RG_WAVES; ++i) mx = fmaxf(mx, red[i]);
    const float b = mx + 1e-8f;
    const float yi = 1.0f / b;

    // codes -> the x_q byte row in LDS (and to x_q_out from workgroup 0), sum of x_q
    uint8_t* xb = reinterpret_cast<uint8_t*>(&buf[0][0]);
    int sx = 0;
#pragma unroll
    for (int c = 0; c < CS; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t e = (int64_t)(HALVES * c + half) * HAD_CHUNK + 4 * th + 1024 * q;
            if (e < K) {
                const uint32_t code = act_codes4(v[c][4 * q], v[c][4 * q + 1], v[c][4 * q + 2], v[c][4 * q + 3], b, yi);
                *reinterpret_cast<uint32_t*>(xb + e) = code;
                sx += byte_sum(code);
                if (a.xq_out && blockIdx.x == 0) *reinterpret_cast<uint32_t*>(a.xq_out + e) = code;
            }
        }
    sx = wave_sum_i32(sx);
    if (lane == 0) redi[wave] = sx;
    if (a.beta_out && blockIdx.x == 0 && t == 0) a.beta_out[0] = b;
    lds_barrier();
    int xsum = 0;
#pragma unroll
    for (int i = 0; i < RG_WAVES; ++i) xsum += redi[i];
    // operand layout: unit (j, d, l) = 16-byte group d of 64-weight chunk l + 64 j, transposed
    for (int u = t; u < CPL * 256; u += 64 * RG_WAVES) {
        const int j = u >> 8, d = (u >> 6) & 3, l = u & 63;
        const int cidx = l + 64 * j;
        u32x4 g = {0u, 0u, 0u, 0u};
        if (cidx < K64) g = *reinterpret_cast<const u32x4*>(xb + 64 * cidx + 16 * d);
        xs[u] = transpose4x4_bytes(g);
    }
    lds_barrier();

    const float s = dequant_scale(a.alpha[0], b);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        int acc = 0;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
            if (lane + 64 * j < K64) acc += chunk_sum(w[r][j], xs + j * 256 + lane, 64, 0);
        const int total = wave_sum_i32(acc) - xsum;
        const int64_t row = r0 + r;
        if (lane == 0 && row < r1) a.y[row] = dequant(total, s, a.bias, row);
    }
}

bool gemv_hadamard_supports(int64_t M, int64_t K) { return M == 1 && K % 64 == 0 && K <= 4 * HAD_CHUNK; }

template <int HALVES, int CS, int CPL, int R>
static hipError_t launch_gemv_hadamard_r(RotGemvArgs a, hipStream_t s) {
    a.rows_per_wave = R;
    const int64_t wgs = (a.N + 4 * HALVES * R - 1) / (4 * HALVES * R);
    return launch_with_lds(k_gemv_hadamard<HALVES, CS, CPL, R>, dim3((unsigned)wgs), dim3(256 * HALVES),
                           (size_t)CPL * 256 * sizeof(u32x4), s, a);
}

// R rows per wave (at most 16 chunk loads of 16 bytes per lane), measured on the decode
// shapes: every workgroup repeats the rotation, so rows trade against workgroups.  One half:
// about 1000 workgroups of four waves, at least two rows per wave; two halves: N / 4096 rows
// per wave, at least two.
template <int HALVES, int CS, int CPL>
static hipError_t launch_gemv_hadamard_cpl(const RotGemvArgs& a, hipStream_t s) {
    constexpr int RMAX = 16 / CPL;
    int64_t want = HALVES == 1 ? (a.N + 3999) / 4000 : (a.N + 4095) / 4096;
    if (want < 2) want = 2;
    if (want <= 2 || RMAX < 4) return launch_gemv_hadamard_r<HALVES, CS, CPL, (RMAX >= 2 ? 2 : 1)>(a, s);
    if (want <= 4 || RMAX < 8) return launch_gemv_hadamard_r<HALVES, CS, CPL, (RMAX >= 4 ? 4 : 1)>(a, s);
    if (want <= 8 || RMAX < 16) return launch_gemv_hadamard_r<HALVES, CS, CPL, (RMAX >= 8 ? 8 : 1)>(a, s);
    return launch_gemv_hadamard_r<HALVES, CS, CPL, (RMAX >= 16 ? 16 : 1)>(a, s);
}

hipError_t launch_gemv_hadamard(const float* x, int64_t K, int block, const int8_t* signs, const uint8_t* wp,
                                const float* alpha, int64_t N, const float* bias, float* y, int8_t* xq_out,
                                float* beta_out, hipStream_t s) {
    const RotGemvArgs a{x, K, block, (float)(1.0 / std::sqrt((double)block)), signs, wp, alpha, N, bias, y,
                        xq_out, beta_out, 0};
    switch ((K / 64 + 63) / 64) {                 // = the number of 4096-element chunks
        case 1: return launch_gemv_hadamard_cpl<1, 1, 1>(a, s);
        case 2: return launch_gemv_hadamard_cpl<2, 1, 2>(a, s);
        case 3: return launch_gemv_hadamard_cpl<2, 2, 3>(a, s);
        case 4: return launch_gemv_hadamard_cpl<2, 2, 4>(a, s);
        default: return hipErrorInvalidValue;     // K > 16384 is refused by gemv_hadamard_supports
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

hipError_t launch_quantize_blocks(const float* W, int64_t N, int64_t K, uint8_t* packed, float* alpha, hipStream_t s) {
    const int64_t nblocks = N * (K / 128);
    int64_t wgs = ((nblocks + 1) / 2 + 3) / 4;
    if (wgs > 8192) wgs = 8192;
    hipLaunchKernelGGL(k_quantize_blocks, dim3((unsigned)wgs), dim3(256), 0, s, W, nblocks, alpha, packed);
    return hipGetLastError();
}

constexpr int64_t QA_MANY_ROWS = 256;

template <int NT>
static hipError_t launch_quantize_act_row(const float* x, int64_t M, int64_t K, int8_t* xq, float* beta, hipStream_t s) {
    const int64_t v = ((K >> 2) + NT - 1) / NT;
    const dim3 g((unsigned)M), b(NT);
    switch (v) {
        case 1: hipLaunchKernelGGL((k_quantize_act_row<1, NT>), g, b, 0, s, x, K, xq, beta); break;
        case 2: hipLaunchKernelGGL((k_quantize_act_row<2, NT>), g, b, 0, s, x, K, xq, beta); break;
        case 3: hipLaunchKernelGGL((k_quantize_act_row<3, NT>), g, b, 0, s, x, K, xq, beta); break;
        case 4: hipLaunchKernelGGL((k_quantize_act_row<4, NT>), g, b, 0, s, x, K, xq, beta); break;
        case 5: hipLaunchKernelGGL((k_quantize_act_row<5, NT>), g, b, 0, s, x, K, xq, beta); break;
        case 6: hipLaunchKernelGGL((k_quantize_act_row<6, NT>), g, b, 0, s, x, K, xq, beta); break;
        case 7: hipLaunchKernelGGL((k_quantize_act_row<7, NT>), g, b, 0, s, x, K, xq, beta); break;
        default: hipLaunchKernelGGL((k_quantize_act_row<8, NT>), g, b, 0, s, x, K, xq, beta); break;
    }
    return hipGetLastError();
}

// One pass with the row in registers for K <= 32768 (K % 4 == 0, aligned): 256 threads per
// token for many tokens and K <= 8192 (more workgroups resident to hide each one's latency),
// else 1024; the two-pass loop otherwise.  Measured with x not in cache: one token,
// K = 28672: 3.8 vs 10.7 us; 2048 tokens, K = 11008: 20.7 vs 32.5 us; K = 4096: 8.7 vs 10.7 us.
hipError_t launch_quantize_act(const float* x, int64_t M, int64_t K, int8_t* xq, float* beta, hipStream_t s) {
    const bool vec = (K % 4 == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)xq % 4 == 0);
    if (vec && M >= QA_MANY_ROWS && K <= 8192) return launch_quantize_act_row<256>(x, M, K, xq, beta, s);
    if (vec && K <= 32768) return launch_quantize_act_row<1024>(x, M, K, xq, beta, s);
    if (vec)
        hipLaunchKernelGGL(k_quantize_act<true>, dim3((unsigned)M), dim3(256), 0, s, x, K, xq, beta);
    else
        hipLaunchKernelGGL(k_quantize_act<false>, dim3((unsigned)M), dim3(256), 0, s, x, K, xq, beta);
    return hipGetLastError();
}

// Workgroups of the pipelined kernel: as many as the device holds at once (occupancy of the
// kernel times the compute units), each walking rows with a stride of the grid.
template <typename Kernel>
static int64_t resident_wgs(Kernel k) {
    int dev = 0, cus = 0, per = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k, 256, 0) != hipSuccess || cus <= 0 || per <= 0)
        return 1024;
    return (int64_t)cus * per;
}

static float hadamard_scale(int block) { return (float)(1.0 / std::sqrt((double)block)); }

hipError_t launch_hadamard_rows(const float* x, int64_t M, int64_t K, int block, const int8_t* signs, float* out,
                                hipStream_t s) {
    const int64_t chunks = (K + HAD_CHUNK - 1) / HAD_CHUNK;
    hipLaunchKernelGGL(k_hadamard_rows, dim3((unsigned)(M * chunks)), dim3(256), 0, s, x, K, chunks, block,
                       hadamard_scale(block), signs, out);
    return hipGetLastError();
}

// The full-row block (B == K) gets the compile-time stage pattern; K = 3072 has none.
template <int NQ, bool FULL>
static void launch_had_pipe_k(const float* x, int64_t M, int block, float sc, const int8_t* signs, int8_t* xq,
                              float* beta, hipStream_t s) {
    auto k = k_quantize_act_hadamard_pipe<NQ, FULL>;
    const int64_t wgs = resident_wgs(k);
    hipLaunchKernelGGL(k, dim3((unsigned)(M < wgs ? M : wgs)), dim3(256), 0, s, x, M, block, sc, signs, xq, beta);
}

template <int NQ>
static void launch_had_pipe(const float* x, int64_t M, int block, float sc, const int8_t* signs, int8_t* xq,
                            float* beta, hipStream_t s) {
    constexpr bool pow2 = (NQ & (NQ - 1)) == 0;
    if (pow2 && block == 1024 * NQ)
        launch_had_pipe_k<NQ, pow2>(x, M, block, sc, signs, xq, beta, s);
    else
        launch_had_pipe_k<NQ, false>(x, M, block, sc, signs, xq, beta, s);
}

// Fewer tokens than this with 2..12 chunks per row take the four-group kernel (one token,
// K = 28672: 8.9 vs 18.1 us); more keep one 256-thread workgroup per token, which fits more
// workgroups per CU (2048 tokens, K = 11008: 26.8 vs 29.6 us).
constexpr int64_t HAD_WIDE_ROWS = 256;

hipError_t launch_quantize_act_hadamard(const float* x, int64_t M, int64_t K, int block, const int8_t* signs,
                                        int8_t* xq, float* beta, hipStream_t s) {
    const int64_t chunks = (K + HAD_CHUNK - 1) / HAD_CHUNK;
    const float sc = hadamard_scale(block);
    const dim3 grid((unsigned)M), threads(256);
    if (K == 4096)
        launch_had_pipe<4>(x, M, block, sc, signs, xq, beta, s);
    else if (K == 3072)
        launch_had_pipe<3>(x, M, block, sc, signs, xq, beta, s);
    else if (K == 2048)
        launch_had_pipe<2>(x, M, block, sc, signs, xq, beta, s);
    else if (K == 1024)
        launch_had_pipe<1>(x, M, block, sc, signs, xq, beta, s);
    else if (chunks > 1 && chunks <= 12 && M < HAD_WIDE_ROWS) {
        const size_t lds = (size_t)4 * HAD_LDS * sizeof(float);
        const dim3 wide(1024);
        if (chunks <= 4) return launch_with_lds(k_quantize_act_hadamard_wide<1>, grid, wide, lds, s, x, K, block, sc, signs, xq, beta);
        if (chunks <= 8) return launch_with_lds(k_quantize_act_hadamard_wide<2>, grid, wide, lds, s, x, K, block, sc, signs, xq, beta);
        return launch_with_lds(k_quantize_act_hadamard_wide<3>, grid, wide, lds, s, x, K, block, sc, signs, xq, beta);
    }
    else if (chunks == 1)
        hipLaunchKernelGGL(k_quantize_act_hadamard<1>, grid, threads, 0, s, x, K, block, sc, signs, xq, beta);
    else if (chunks == 2)
        hipLaunchKernelGGL(k_quantize_act_hadamard<2>, grid, threads, 0, s, x, K, block, sc, signs, xq, beta);
    else if (chunks <= 4)
        hipLaunchKernelGGL(k_quantize_act_hadamard<4>, grid, threads, 0, s, x, K, block, sc, signs, xq, beta);
    else if (chunks <= 8)
        hipLaunchKernelGGL(k_quantize_act_hadamard<8>, grid, threads, 0, s, x, K, block, sc, signs, xq, beta);
    else
        hipLaunchKernelGGL(k_quantize_act_hadamard<0>, grid, threads, 0, s, x, K, block, sc, signs, xq, beta);
    return hipGetLastError();
}

}  // namespace bitlinear
