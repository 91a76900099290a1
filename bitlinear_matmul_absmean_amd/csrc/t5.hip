// t5.hip -- ternary weights packed five to a byte (1.6 bits per weight) for gfx950.
//
// [P2] nxmr.cn, "1.58 位大模型" §1.1 and §6.1 mention encodings more compact than 2 bits and
// table decoding on dedicated hardware, without a format.  Here: byte b of a row holds the
// codes c = W_hat + 1 of weights 5b .. 5b+4 as the base-3 number sum_i c_i 3^i (0..242); a row
// takes 16 ceil(K / 80) bytes (whole 16-byte chunks of 80 weights); trits past K hold code 1
// (weight 0), so a byte with no weight left is 121.
//
// Decode GEMV (one token per grid row y): a workgroup builds a byte -> five-codes table in
// LDS and stages the activations of every byte position p as [x(5p..5p+3) as one dword,
// x(5p+4)], stored byte-of-chunk major so that lanes reading their chunks hit distinct banks.  A lane reads one 16-byte chunk (80 weights) of a row per load; for each byte it
// looks the five codes up (4 codes in a dword for v_dot4_i32_i8, the fifth for a multiply-add),
// with the activations of its chunk held in registers across the wave's rows.  The table is
// kept in 16 copies, copy k on banks 2k and 2k+1, lane l reading copy l % 16, so a 32-lane
// pass meets at most two addresses per bank pair.  acc = sum c x - sum x as in the 2-bit
// kernels.
#include "common.hpp"

namespace bitlinear {

constexpr int T5_WAVES = 8;
constexpr int T5_COPIES = 16;

int64_t t5_row_bytes(int64_t K) { return 16 * ((K + 79) / 80); }

// Codes of one byte: thread per output byte of the whole tensor.
__global__ __launch_bounds__(256) void k_pack_t5(const float* __restrict__ W, int64_t N, int64_t K, int64_t rb,
                                                 const float* __restrict__ alpha, uint8_t* __restrict__ out) {
    const float a = alpha[0];
    const int64_t total = N * rb;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t n = i / rb, b = i - n * rb;
        uint32_t v = 0, p3 = 1;
#pragma unroll
        for (int t = 0; t < 5; ++t, p3 *= 3) {
            const int64_t k = 5 * b + t;
            uint32_t c = 1u;
            if (k < K) {
                const float w = W[n * K + k];
                if (a != 0.0f) {
                    float r = rintf(w / a);
                    r = fminf(fmaxf(r, -1.0f), 1.0f);
                    c = (uint32_t)((int)r + 1);
                }
            }
            v += c * p3;
        }
        out[i] = (uint8_t)v;
    }
}

struct T5Args {
    const int8_t* xq;
    const float* beta;
    int64_t M, K, N, rb;          // rb: bytes per row
    const uint8_t* wp;
    const float* alpha;
    const float* bias;
    float* y;
    int64_t rows_per_wave;
};

// CPL chunks of 16 bytes per lane and row, R rows per step.
template <int CPL, int R>
__global__ __launch_bounds__(64 * T5_WAVES) void k_gemv_t5(T5Args a) {
    extern __shared__ uint2 t5s[];                  // [256 * T5_COPIES] table, then [rb] activations
    __shared__ int red_i[T5_WAVES];
    uint2* lut = t5s;
    uint2* xs = t5s + 256 * T5_COPIES;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t K = a.K, N = a.N, rb = a.rb;
    const int nch = (int)(rb >> 4);
    const int64_t m = blockIdx.y;
    const int8_t* xrow = a.xq + m * K;

    const int64_t r0 = ((int64_t)blockIdx.x * T5_WAVES + wave) * a.rows_per_wave;
    const int64_t r1 = r0 + a.rows_per_wave < N ? r0 + a.rows_per_wave : N;
    const u32x4* wp = reinterpret_cast<const u32x4*>(a.wp);
    // Rows past the wave's range (or past N, for a wave with none) are clamped to the last row, so
    // the loads stay branch-free and in bounds; their sums are never stored.
    auto load_rows = [&](u32x4 (&w)[R][CPL], int64_t rbase) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = rbase + r < r1 ? rbase + r : (r1 > 0 ? r1 - 1 : 0);
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = lane + 64 * j < nch ? lane + 64 * j : 0;
                w[r][j] = wp[row * nch + c];
            }
        }
    };
    // The first rows are requested before the tables are built, so that their latency covers
    // the table and the activation staging.
    u32x4 w[R][CPL];
    load_rows(w, r0);

    // bytes 243..255 are never written; their entries only keep every lookup in bounds
    // (consecutive threads write consecutive entries: no bank conflicts)
    for (int e = tid; e < 256 * T5_COPIES; e += 64 * T5_WAVES) {
        const int v = e / T5_COPIES;
        const uint32_t c0 = v % 3, c1 = (v / 3) % 3, c2 = (v / 9) % 3, c3 = (v / 27) % 3, c4 = v / 81;
        lut[e] = make_uint2(c0 | (c1 << 8) | (c2 << 16) | (c3 << 24), c4);
    }
    int xsum = 0;
    for (int64_t p = tid; p < rb; p += 64 * T5_WAVES) {
        uint32_t lo = 0;
        int hi = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int64_t k = 5 * p + t;
            const int x = k < K ? (int)xrow[k] : 0;
            lo |= (uint32_t)(x & 0xFF) << (8 * t);
            xsum += x;
        }
        if (5 * p + 4 < K) hi = xrow[5 * p + 4];
        xsum += hi;
        xs[(p & 15) * nch + (p >> 4)] = make_uint2(lo, (uint32_t)hi);   // [byte q of a chunk][chunk]
    }
    xsum = wave_sum_i32(xsum);
    if (lane == 0) red_i[wave] = xsum;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < T5_WAVES; ++w) tot += red_i[w];
    const float s = dequant_scale(a.alpha[0], a.beta[m]);

    const uint2* myl = lut + (lane & (T5_COPIES - 1));
    for (int64_t rbase = r0; rbase < r1; rbase += R) {
        // the next rows' loads go out before this step's sums; unconditional (clamped rows), so
        // the wait for this step's rows leaves them in flight
        u32x4 wn[R][CPL];
        load_rows(wn, rbase + R);
        int acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lane + 64 * j;
            if (c < nch) {
                uint2 xv[16];
#pragma unroll
                for (int q = 0; q < 16; ++q) xv[q] = xs[q * nch + c];   // consecutive lanes, consecutive words
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t wd[4] = {w[r][j].x, w[r][j].y, w[r][j].z, w[r][j].w};
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        const uint32_t b = (wd[q >> 2] >> (8 * (q & 3))) & 0xFFu;
                        const uint2 e = myl[b * T5_COPIES];
                        acc[r] = dot4(e.x, xv[q].x, acc[r]);
                        acc[r] = dot4(e.y, xv[q].y, acc[r]);    // c4 (byte 0) times x(5p+4): one full-rate op
                    }
                }
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int total = wave_sum_i32(acc[r]) - tot;
            const int64_t row = rbase + r;
            if (lane == 0 && row < r1) a.y[m * N + row] = dequant(total, s, a.bias, row);
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < CPL; ++j) w[r][j] = wn[r][j];
    }
}

// Repack 2-bit codes (byte b: weight 4b + i at bits 2i) to five per byte: thread per output
// byte, reading the code bytes of its five weights.
__global__ __launch_bounds__(256) void k_repack_t5(const uint8_t* __restrict__ w2, int64_t N, int64_t K, int64_t rb,
                                                   uint8_t* __restrict__ out) {
    const int64_t total = N * rb, rb2 = K / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int64_t n = i / rb, b = i - n * rb;
        uint32_t v = 0, p3 = 1;
#pragma unroll
        for (int t = 0; t < 5; ++t, p3 *= 3) {
            const int64_t k = 5 * b + t;
            const uint32_t c = k < K ? (w2[n * rb2 + (k >> 2)] >> (2 * (k & 3))) & 3u : 1u;
            v += c * p3;
        }
        out[i] = (uint8_t)v;
    }
}

hipError_t launch_repack_t5(const uint8_t* w2, int64_t N, int64_t K, uint8_t* out, hipStream_t s) {
    const int64_t rb = t5_row_bytes(K);
    int64_t wgs = (N * rb + 255) / 256;
    if (wgs > 65536) wgs = 65536;
    hipLaunchKernelGGL(k_repack_t5, dim3((unsigned)wgs), dim3(256), 0, s, w2, N, K, rb, out);
    return hipGetLastError();
}

template <int CPL, int R>
static hipError_t launch_t5_r(const T5Args& a, hipStream_t s) {
    const int64_t wgs = (a.N + a.rows_per_wave * T5_WAVES - 1) / (a.rows_per_wave * T5_WAVES);
    const size_t lds = (size_t)(256 * T5_COPIES + a.rb) * sizeof(uint2);
    return launch_with_lds(k_gemv_t5<CPL, R>, dim3((unsigned)wgs, (unsigned)a.M), dim3(64 * T5_WAVES), lds, s, a);
}

// Rows over about two workgroups per CU; R rows per step with R * CPL <= 8 and R <= rows.
template <int CPL>
static hipError_t launch_t5_cpl(const T5Args& a0, hipStream_t s) {
    T5Args a = a0;
    a.rows_per_wave = (a.N + 512 * T5_WAVES - 1) / (512 * T5_WAVES);
    constexpr int RMAX = CPL >= 8 ? 1 : 8 / CPL;
    if (RMAX >= 4 && a.rows_per_wave >= 4) return launch_t5_r<CPL, (RMAX >= 4 ? 4 : 1)>(a, s);
    // three rows per wave in one step rather than two steps of two (the second half wasted on a
    // clamped row, the activations read twice)
    if (RMAX >= 3 && a.rows_per_wave == 3) return launch_t5_r<CPL, (RMAX >= 3 ? 3 : 1)>(a, s);
    if (RMAX >= 2 && a.rows_per_wave >= 2) return launch_t5_r<CPL, (RMAX >= 2 ? 2 : 1)>(a, s);
    return launch_t5_r<CPL, 1>(a, s);
}

hipError_t launch_pack_t5(const float* W, int64_t N, int64_t K, const float* alpha, uint8_t* out, hipStream_t s) {
    const int64_t rb = t5_row_bytes(K);
    int64_t wgs = (N * rb + 255) / 256;
    if (wgs > 65536) wgs = 65536;
    hipLaunchKernelGGL(k_pack_t5, dim3((unsigned)wgs), dim3(256), 0, s, W, N, K, rb, alpha, out);
    return hipGetLastError();
}

bool t5_supports(int64_t K) { return K <= 65536; }

hipError_t launch_forward_t5(const int8_t* xq, const float* beta, int64_t M, int64_t K, const uint8_t* wp,
                             const float* alpha, int64_t N, const float* bias, float* y, hipStream_t s) {
    const T5Args a{xq, beta, M, K, N, t5_row_bytes(K), wp, alpha, bias, y, 0};
    const int64_t cpl = (a.rb / 16 + 63) / 64;
    switch (cpl) {
        case 1: return launch_t5_cpl<1>(a, s);
        case 2: return launch_t5_cpl<2>(a, s);
        case 3: return launch_t5_cpl<3>(a, s);
        case 4: return launch_t5_cpl<4>(a, s);
        case 5: case 6: return launch_t5_cpl<6>(a, s);
        case 7: case 8: return launch_t5_cpl<8>(a, s);
        case 9: case 10: case 11: case 12: return launch_t5_cpl<12>(a, s);
        default: return launch_t5_cpl<16>(a, s);
    }
}

}  // namespace bitlinear
