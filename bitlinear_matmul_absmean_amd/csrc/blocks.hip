// blocks.hip -- ternary x int8 forward with block-scaled weights for gfx950.
//
// [P1] 2kiu.com, article on 1.58-bit quantization and hardware co-optimization, §2.3 and
//      §4.2: one scale shared by each block of 128 consecutive weights of a row, scales of
//      shape [C_out, C_in / 128].
// [P2] nxmr.cn, "1.58 位大模型" §3.3 (add/sub form of the matmul); [P3] chenxutan.com,
//      "1.58-bit 大模型极限量化实战" §2.4 (the beta / 127 factor).
//
// y[m, n] = fp32(S * (beta[m] / 127)) with S = sum_b alpha[n, b] * acc[m, n, b], where acc is
// the int32 add/sub sum over block b.  Each 64-weight chunk's int32 sum is multiplied by its
// block's alpha and added in fp64: the products are exact (24 x 15 bits), only the fp64
// additions round, so S matches an fp64 sum in any order to about 1e-16 of sum |alpha acc|
// and y almost always matches bit for bit after the one fp32 rounding.
//
// Decode-shaped GEMV: a workgroup stages up to four tokens of x_q in LDS (each 16-byte group
// transposed 4x4 so that a masked dword of codes meets its activations, plus the sum of x_q
// over each 64-weight chunk), then every wave streams its own rows, one 16-byte chunk of
// codes per lane and load.  More than four tokens run as a second grid dimension over groups
// of four, each group reading the codes again (mostly from L2 and the Infinity Cache).
#include "common.hpp"

namespace bitlinear {

struct BlockArgs {
    const int8_t* xq;
    const float* beta;
    int64_t M, K, N;
    const uint8_t* wp;
    const float* alpha;   // [N, K / 128]
    const float* bias;
    float* y;
    int64_t rows_per_wave;
};

constexpr int BW_WAVES = 8;

// MT tokens per workgroup (tokens past M are zero; more tokens run as a second grid
// dimension over groups of MT), CPL chunks of 64 weights per lane and row (K <= 4096 CPL),
// R rows per wave step with every load of the step issued first.
template <int MT, int CPL, int R>
__global__ __launch_bounds__(64 * BW_WAVES) void k_gemv_blocks(BlockArgs a) {
    extern __shared__ u32x4 xs[];                       // [MT][CPL][4][64] transposed groups
    int* cs = reinterpret_cast<int*>(xs + MT * CPL * 256);   // [MT][CPL * 64] chunk sums
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t K = a.K, N = a.N;
    const int K64 = (int)(K >> 6), KB = (int)(K >> 7);
    const int64_t m0 = (int64_t)blockIdx.y * MT;

    // staging: one thread per (token, chunk)
    for (int u = tid; u < MT * CPL * 64; u += 64 * BW_WAVES) {
        const int m = u / (CPL * 64), c = u - m * (CPL * 64);
        u32x4 q[4] = {};
        if (c < K64 && m0 + m < a.M) {
            const u32x4* src = reinterpret_cast<const u32x4*>(a.xq + (m0 + m) * K + 64 * c);
#pragma unroll
            for (int d = 0; d < 4; ++d) q[d] = src[d];
        }
        int sx = 0;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            sx += byte_sum(q[d].x) + byte_sum(q[d].y) + byte_sum(q[d].z) + byte_sum(q[d].w);
            xs[((m * CPL + (c >> 6)) * 4 + d) * 64 + (c & 63)] = transpose4x4_bytes(q[d]);
        }
        cs[u] = sx;
    }
    double tm[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) tm[m] = m0 + m < a.M ? (double)a.beta[m0 + m] / 127.0 : 0.0;
    __syncthreads();

    const int64_t r0 = ((int64_t)blockIdx.x * BW_WAVES + wave) * a.rows_per_wave;
    const int64_t r1 = r0 + a.rows_per_wave < N ? r0 + a.rows_per_wave : N;
    const u32x4* wp = reinterpret_cast<const u32x4*>(a.wp);
    for (int64_t rb = r0; rb < r1; rb += R) {
        u32x4 w[R][CPL];
        float al[R][CPL];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = rb + r < r1 ? rb + r : r1 - 1;      // clamped: loads stay branch-free
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = lane + 64 * j < K64 ? lane + 64 * j : 0;
                w[r][j] = wp[row * K64 + c];
                al[r][j] = a.alpha[row * KB + (c >> 1)];
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            double f[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) f[m] = 0.0;
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                if (lane + 64 * j < K64) {
#pragma unroll
                    for (int m = 0; m < MT; ++m) {
                        const int p = chunk_sum(w[r][j], xs + (m * CPL + j) * 256 + lane, 64,
                                                cs[(m * CPL + j) * 64 + lane]);
                        f[m] = __builtin_fma((double)al[r][j], (double)p, f[m]);
                    }
                }
            }
            const int64_t row = rb + r;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const double sum = wave_sum_f64(f[m]);
                if (lane == m && row < r1 && m0 + m < a.M) {
                    float v = (float)(sum * tm[m]);
                    if (a.bias) v = v + a.bias[row];
                    a.y[(m0 + m) * N + row] = v;
                }
            }
        }
    }
}

bool blocks_supports(int64_t K) { return K % 128 == 0 && K <= 32768; }

template <int MT, int CPL, int R>
static hipError_t launch_blocks_r(const BlockArgs& a, int64_t groups, hipStream_t s) {
    const int64_t wgs = (a.N + a.rows_per_wave * BW_WAVES - 1) / (a.rows_per_wave * BW_WAVES);
    const size_t lds = (size_t)MT * CPL * (256 * sizeof(u32x4) + 64 * sizeof(int));
    return launch_with_lds(k_gemv_blocks<MT, CPL, R>, dim3((unsigned)wgs, (unsigned)groups), dim3(64 * BW_WAVES), lds, s,
                           a);
}

// Rows are spread over about two workgroups per CU (512 x 8 waves); a wave's step holds up to
// 8 chunk loads per lane, so R rows of CPL chunks with R * CPL <= 8 and R <= the wave's rows.
template <int MT, int CPL>
static hipError_t launch_blocks_mt(const BlockArgs& a0, int64_t groups, hipStream_t s) {
    BlockArgs a = a0;
    constexpr int RMAX = CPL >= 8 ? 1 : 8 / CPL;
    a.rows_per_wave = (a.N + 512 * BW_WAVES - 1) / (512 * BW_WAVES);
    if (RMAX >= 8 && a.rows_per_wave >= 8) return launch_blocks_r<MT, CPL, (RMAX >= 8 ? 8 : 1)>(a, groups, s);
    if (RMAX >= 4 && a.rows_per_wave >= 4) return launch_blocks_r<MT, CPL, (RMAX >= 4 ? 4 : 1)>(a, groups, s);
    if (RMAX >= 2 && a.rows_per_wave >= 2) return launch_blocks_r<MT, CPL, (RMAX >= 2 ? 2 : 1)>(a, groups, s);
    return launch_blocks_r<MT, CPL, 1>(a, groups, s);
}

template <int MT>
static hipError_t launch_blocks_cpl(const BlockArgs& a, int64_t groups, hipStream_t s) {
    const int64_t cpl = (a.K / 64 + 63) / 64;
    switch (cpl) {
        case 1: return launch_blocks_mt<MT, 1>(a, groups, s);
        case 2: return launch_blocks_mt<MT, 2>(a, groups, s);
        case 3: return launch_blocks_mt<MT, 3>(a, groups, s);
        case 4: return launch_blocks_mt<MT, 4>(a, groups, s);
        case 5: case 6: return launch_blocks_mt<MT, 6>(a, groups, s);
        default: return launch_blocks_mt<MT, 8>(a, groups, s);
    }
}

hipError_t launch_forward_blocks(const int8_t* xq, const float* beta, int64_t M, int64_t K, const uint8_t* wp,
                                 const float* alpha, int64_t N, const float* bias, float* y, hipStream_t s) {
    const BlockArgs a{xq, beta, M, K, N, wp, alpha, bias, y, 0};
    switch (M) {
        case 1: return launch_blocks_cpl<1>(a, 1, s);
        case 2: return launch_blocks_cpl<2>(a, 1, s);
        case 3: return launch_blocks_cpl<3>(a, 1, s);
        default: return launch_blocks_cpl<4>(a, (M + 3) / 4, s);
    }
}

}  // namespace bitlinear
