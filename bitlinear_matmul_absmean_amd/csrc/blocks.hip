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
// One or two tokens, a GEMV: a workgroup stages the tokens' x_q in LDS (each 16-byte group
// transposed 4x4 so that a masked dword of codes meets its activations, plus the sum of x_q
// over each 64-weight chunk), then every wave streams its own rows, one 16-byte chunk of
// codes per lane and load.  Three to 127 tokens run on the matrix cores (below): with
// K % 256 == 0 in slices of up to 64 on the buffer-load kernel, otherwise in
// slices of 32; 128 and more on the block-scaled GEMM at the end of the file.
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

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double d) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(d), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(d), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

// Wave sum in fp64 through DPP row operations (quad swaps, then the half-row and row mirrors:
// every lane of a 16-lane row ends with the row sum) and the four row sums read from lanes
// 0, 16, 32, 48, added as (a + b) + (c + d).  The order is fixed, so results are
// reproducible; a lane shuffle per step would go through the LDS unit, about 100 cycles each.
__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
    v += dpp_f64<0xB1>(v);     // quad_perm [1,0,3,2]
    v += dpp_f64<0x4E>(v);     // quad_perm [2,3,0,1]
    v += dpp_f64<0x141>(v);    // row_half_mirror
    v += dpp_f64<0x140>(v);    // row_mirror
    auto lane_f64 = [&](int l) {
        return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                                __builtin_amdgcn_readlane(__double2loint(v), l));
    };
    return (lane_f64(0) + lane_f64(16)) + (lane_f64(32) + lane_f64(48));
}

// MT tokens per workgroup (one or two; a second grid dimension over groups of MT tokens is
// supported, tokens past M are zero), CPL chunks of 64 weights per lane and row (K <= 4096 CPL),
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
    const float* bias_src = a.bias ? a.bias : a.alpha;
    for (int64_t rb = r0; rb < r1; rb += R) {
        u32x4 w[R][CPL];
        float al[R][CPL], bi[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = rb + r < r1 ? rb + r : r1 - 1;      // clamped: loads stay branch-free
            bi[r] = bias_src[a.bias ? row : 0];                       // with the step's loads
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
                const double sum = wave_sum_f64_dpp(f[m]);
                if (lane == m && row < r1 && m0 + m < a.M) {
                    float v = (float)(sum * tm[m]);
                    if (a.bias) v = v + bi[r];
                    a.y[(m0 + m) * N + row] = v;
                }
            }
        }
    }
}

// Batched tokens (5 to 32 per launch) on 16 x 16 x 64 int8 MFMA tiles, the layout of the
// per-tensor batched-decode kernel: a workgroup of eight waves owns RB blocks of 16 weight
// rows, the waves split K into sub-steps of 256 weights, lane group g = l / 16 holds the 64
// contiguous weights k0 + 64 g of its row (block 2 s + g / 2 of sub-step s), and in MFMA q it
// takes the 16-weight group 16 q of them.  Codes go to the B operand as signed bytes c - 1
// (v_perm with the table {-1, 0, 1}), so no sum of x_q is needed.  Two MFMAs per tile and q:
// one over all four lane groups (both blocks) and one with the A operand of lane groups 0
// and 1 zeroed (the second block alone); their difference is the first block's sum, exact in
// int32.  After each sub-step both sums are scaled by their block's alpha and added into fp64
// accumulators; the eight waves' fp64 tiles are added through LDS in a fixed order and
// y = fp32(S * beta / 127) (+ bias).  16x16x64 lane layout: A/B lane l holds row/column l % 16,
// k = 16 (l / 16) + j; accumulator r of lane l is row 4 (l / 16) + r, column l % 16.
constexpr int BB_WAVES = 8;

template <int MT, int RB>
__global__ __launch_bounds__(BB_WAVES * 64) void k_bdec16_blocks(BlockArgs a) {
    // LDS: the workgroup's alpha rows (stride KB + 1: the 16 rows a load reads fall in distinct
    // banks) during the K loop, then the waves' fp64 tiles [wave][RB * MT][4][64]
    extern __shared__ double redd[];
    __shared__ double bsc[16 * MT];                // beta[m] / 127 of the slice's tokens
    float* as = reinterpret_cast<float*>(redd);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = (int)a.M;
    const int64_t K = a.K, N = a.N, rowb = K >> 2;
    const int KB = (int)(K >> 7), KBp = KB + 1;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * RB);
    const int rows = (int)(N - n0 < 16 * RB ? N - n0 : 16 * RB);
    // the epilogue's per-token beta and this thread's bias (element e = tid of the epilogue,
    // see below) are loaded before anything else: a wave's loads complete in order, so a load
    // issued later would make its use wait for every load in flight
    const float beta_ld = a.beta[tid < M ? tid : M - 1];
    const float* bias_src = a.bias ? a.bias : a.alpha;
    const int64_t nb_e = n0 + 16 * ((tid >> 6) / MT) + (tid & 15);
    const float bias_e = bias_src[a.bias && tid < RB * MT * 64 ? (nb_e < N ? nb_e : N - 1) : 0];
    const int lr = lane & 15, lg = lane >> 4;
    const int SP = (int)((K + 255) / 256);
    const int s0 = (int)((int64_t)SP * wave / BB_WAVES), s1 = (int)((int64_t)SP * (wave + 1) / BB_WAVES);
    const int8_t* xrow[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xrow[t] = a.xq + (int64_t)min(16 * t + lr, M - 1) * K;
    int64_t nrow[RB];
    int arow[RB];                                  // LDS offset of this lane's alpha row
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int lrow = min(16 * r + lr, rows - 1);
        nrow[r] = n0 + lrow;
        arow[r] = lrow * KBp;
    }
    const uint32_t hi_mask = lg >= 2 ? 0xFFFFFFFFu : 0u;  // lane groups of the sub-step's second block

    // a lane group whose 64 weights lie past K (K % 256 == 128) re-reads the row start with its
    // x_q zeroed, so its products vanish; its alpha index is clamped to the last block
    u32x4 xa[2][MT][4], wb[2][RB];
    auto load = [&](int st, int s) {
        const int64_t k0 = (int64_t)s * 256 + 64 * lg;
        const int64_t kx = k0 < K ? k0 : 0;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) xa[st][t][q] = *reinterpret_cast<const u32x4*>(xrow[t] + kx + 16 * q);
#pragma unroll
        for (int r = 0; r < RB; ++r)
            wb[st][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.wp + nrow[r] * rowb + kx / 4));
    };
    double f[RB][MT][4];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) f[r][t][i] = 0.0;

    auto compute = [&](int st, int s) {
        const bool live = (int64_t)s * 256 + 64 * lg < K;
        const int b1 = 2 * s + 1 < KB ? 2 * s + 1 : KB - 1;
        float al[RB][2];
#pragma unroll
        for (int r = 0; r < RB; ++r) {
            al[r][0] = as[arow[r] + 2 * s];
            al[r][1] = as[arow[r] + b1];
        }
        i32x4 both[RB][MT], second[RB][MT];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int t = 0; t < MT; ++t) both[r][t] = second[r][t] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            i32x4 av[MT], ah[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const u32x4 v = live ? xa[st][t][q] : u32x4{0u, 0u, 0u, 0u};
                const u32x4 tv = transpose4x4_perm(v);
                av[t] = (i32x4)tv;
                ah[t] = i32x4{(int)(tv.x & hi_mask), (int)(tv.y & hi_mask), (int)(tv.z & hi_mask), (int)(tv.w & hi_mask)};
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t w = q == 0 ? wb[st][r].x : q == 1 ? wb[st][r].y : q == 2 ? wb[st][r].z : wb[st][r].w;
                const i32x4 bv = {(int)__builtin_amdgcn_perm(0u, 0x000100FFu, w & 0x03030303u),
                                  (int)__builtin_amdgcn_perm(0u, 0x000100FFu, (w >> 2) & 0x03030303u),
                                  (int)__builtin_amdgcn_perm(0u, 0x000100FFu, (w >> 4) & 0x03030303u),
                                  (int)__builtin_amdgcn_perm(0u, 0x000100FFu, (w >> 6) & 0x03030303u)};
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    both[r][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[t], bv, both[r][t], 0, 0, 0);
                    second[r][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ah[t], bv, second[r][t], 0, 0, 0);
                }
            }
        }
        // scale each block's sums by its alpha (column l % 16 of the tile is this lane's row)
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int hi = second[r][t][i];
                    f[r][t][i] = __builtin_fma((double)al[r][0], (double)(both[r][t][i] - hi), f[r][t][i]);
                    f[r][t][i] = __builtin_fma((double)al[r][1], (double)hi, f[r][t][i]);
                }
    };
    // the workgroup's alpha rows n0 .. n0 + rows - 1 are one contiguous span of rows * KB
    // floats.  Up to 8 per thread (K <= 8192 at RB = 4) the loads are issued ahead of the weight
    // prefetches, so that the LDS stores wait for them alone; larger spans are copied first.
    // Loads and stores are branch-free: an index past the span is clamped to its last float,
    // which that thread then stores again, with the same value, where its owner stores it.
    const float* asrc = a.alpha + n0 * KB;
    const int atotal = rows * KB;
    constexpr int ABATCH = 8 * BB_WAVES * 64;
    auto alpha_load = [&](float (&v)[8], int base) {
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = asrc[min(base + j * BB_WAVES * 64 + tid, atotal - 1)];
    };
    auto alpha_store = [&](const float (&v)[8], int base) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int e = min(base + j * BB_WAVES * 64 + tid, atotal - 1);
            const int row = e / KB;
            as[row * KBp + (e - row * KB)] = v[j];
        }
    };
    float av0[8];
    const bool one_batch = atotal <= ABATCH;
    if (one_batch) {
        alpha_load(av0, 0);
    } else {
        for (int base = 0; base < atotal; base += ABATCH) {
            float v[8];
            alpha_load(v, base);
            alpha_store(v, base);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // the first two stages, issued unconditionally (s0 < SP always holds, so a wave without
    // sub-steps reads in bounds and discards them): a branch here would make the waits of the
    // alpha stores below cover these loads as well
    const int last = s1 > s0 ? s1 - 1 : s0;
    load(0, s0);
    load(1, min(s0 + 1, last));
    __builtin_amdgcn_sched_barrier(0);
    if (one_batch) alpha_store(av0, 0);
    if (tid < 16 * MT) bsc[tid] = (double)beta_ld / 127.0;
    lds_barrier();
    if (s0 < s1) {
        int s = s0;
        // one token tile: no loads past the wave's range (16 tokens at K = 4096, N = 11008:
        // 9.45 against 11.06 us); two token tiles keep the clamped loads, which hold fewer
        // registers live (the skipping form spilled at three row blocks)
        for (; s + 2 <= s1; s += 2) {
            compute(0, s);
            __builtin_amdgcn_sched_barrier(0);
            if (MT == 2 || s + 2 < s1) load(0, min(s + 2, last));
            __builtin_amdgcn_sched_barrier(0);
            compute(1, s + 1);
            __builtin_amdgcn_sched_barrier(0);
            if (MT == 2 || s + 3 < s1) load(1, min(s + 3, last));
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s < s1) compute(0, s);
    }
    __syncthreads();                               // alpha rows no longer read: the LDS is the tiles'
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) redd[(((wave * RB * MT) + r * MT + t) * 4 + i) * 64 + lane] = f[r][t][i];
    __syncthreads();
    static_assert(RB * MT * 64 <= BB_WAVES * 64, "one epilogue element per thread");
    if (tid < RB * MT * 64) {
        const int l = tid & 63, tile = tid >> 6;
        const int r = tile / MT, t = tile % MT;
        const int64_t n = n0 + 16 * r + (l & 15);
        if (n < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * t + 4 * (l >> 4) + i;
                if (m >= M) continue;
                double sum = 0.0;
#pragma unroll
                for (int w = 0; w < BB_WAVES; ++w) sum += redd[((w * RB * MT + tile) * 4 + i) * 64 + l];
                float v = (float)(sum * bsc[m]);
                if (a.bias) v = v + bias_e;
                a.y[(int64_t)m * N + n] = v;
            }
        }
    }
}

template <int MT, int RB>
static hipError_t launch_bdec16_blocks(const BlockArgs& a, hipStream_t s) {
    const int64_t wgs = (a.N + 16 * RB - 1) / (16 * RB);
    const size_t tiles = (size_t)BB_WAVES * RB * MT * 4 * 64 * sizeof(double);
    const size_t alphas = (size_t)16 * RB * (a.K / 128 + 1) * sizeof(float);
    return launch_with_lds(k_bdec16_blocks<MT, RB>, dim3((unsigned)wgs), dim3(BB_WAVES * 64),
                           tiles > alphas ? tiles : alphas, s, a);
}

// Batched tokens (3 to 64 per launch) with K % 256 == 0: the layout of the per-tensor kernel
// k_bdec16n.  Codes expanded in weight order and mapped to signed bytes W_hat = c - 1 (a v_perm
// table), so no sum of x_q is needed; x_q and the packed codes of a sub-step go from global
// memory into a wave-private LDS image through the load unit (buffer_load_dwordx4 ... lds), the
// next sub-step fetched while the current one is multiplied.  In MFMA q of a sub-step lane group
// g holds weights 64 q + 16 g .. 64 q + 16 g + 15 (packed dword g of the row's 16-byte load q,
// unit 4 q + g of the token's x_q), so MFMAs 0-1 cover the sub-step's first 128-weight block and
// 2-3 its second: each block's int32 sums come from two MFMAs started from zero, then are scaled
// by the block's alpha into fp64 accumulators.  The eight waves' fp64 tiles are added through
// LDS in a fixed order and y = fp32(S * beta / 127) (+ bias).
template <int MT, int RB>
__global__ __launch_bounds__(BB_WAVES * 64) void k_bdec16n_blocks(BlockArgs a) {
    // LDS: the waves' images [wave][(4 MT + RB) * 64 units], then the workgroup's alpha rows
    // (stride KB + 1); after the K loop, the waves' fp64 tiles [wave][RB * MT][4][64]
    extern __shared__ i32x4 img[];
    __shared__ double bsc[16 * MT];                // beta[m] / 127 of the slice's tokens
    constexpr int XI = 4 * MT, IMG = (XI + RB) * 64;
    double* redd = reinterpret_cast<double*>(img);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // a second grid dimension splits the tokens: workgroup row y takes tokens 16 MT y onwards
    if (gridDim.y > 1) {
        const int64_t m0 = (int64_t)blockIdx.y * (16 * MT);
        a.xq += m0 * a.K;
        a.beta += m0;
        a.y += m0 * a.N;
        a.M = a.M - m0 < 16 * MT ? a.M - m0 : 16 * MT;
    }
    const int M = (int)a.M;
    const int64_t K = a.K, N = a.N, rowb = K >> 2;
    const int KB = (int)(K >> 7), KBp = KB + 1;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * RB);
    const int rows = (int)(N - n0 < 16 * RB ? N - n0 : 16 * RB);
    const float beta_ld = a.beta[tid < M ? tid : M - 1];
    const float* bias_src = a.bias ? a.bias : a.alpha;
    const int64_t nb_e = n0 + 16 * ((tid >> 6) / MT) + (tid & 15);
    const float bias_e = bias_src[a.bias && tid < RB * MT * 64 ? (nb_e < N ? nb_e : N - 1) : 0];
    const int lr = lane & 15, lg = lane >> 4;
    // sub-steps interleaved over the waves (wave w takes w, w + 8, ...), as in k_bdec16n
    const int SP = (int)(K >> 8);
    i32x4* xs = img + wave * IMG;
    const uint32_t* ws32 = reinterpret_cast<const uint32_t*>(xs + XI * 64);
    float* as = reinterpret_cast<float*>(img + BB_WAVES * IMG);
    // load instruction i, lane (lr, lg): token 4i + lg (rows past M read row M - 1, never
    // written), position lr, unit lr ^ (4 (i % 4) + lg); weight load r: 16 bytes at 16 lg of
    // row n0 + 16 r + lr's 64-byte piece of the sub-step.  Offsets fit 32 bits (checked on launch).
    const uint32_t Ku = (uint32_t)K, lastx = (uint32_t)(M - 1) * Ku, lgK = (uint32_t)lg * Ku;
    uint32_t xu[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xu[j] = 16u * (uint32_t)(lr ^ (4 * j + lg));
    uint32_t xoff[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) xoff[i] = min(lgK + (uint32_t)(4 * i) * Ku, lastx) + xu[i & 3];
    uint32_t woff[RB];
    int arow[RB];                                  // LDS offset of this lane's alpha row
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        const int lrow = min(16 * r + lr, rows - 1);
        woff[r] = (uint32_t)(n0 + lrow) * (uint32_t)rowb + 16u * (uint32_t)lg;
        arow[r] = lrow * KBp;
    }
    const __amdgpu_buffer_rsrc_t xr = raw_buffer(a.xq, (uint32_t)(M * K));
    const __amdgpu_buffer_rsrc_t wr = raw_buffer(a.wp, (uint32_t)(N * rowb));
    auto fetch = [&](int s) {
#pragma unroll
        for (int i = 0; i < XI; ++i) load_lds16(xr, xoff[i], (uint32_t)s * 256u, xs + 64 * i);
#pragma unroll
        for (int r = 0; r < RB; ++r) load_lds16(wr, woff[r], (uint32_t)s * 64u, xs + 64 * (XI + r));
    };
    if (wave < SP) fetch(wave);
    // the workgroup's alpha rows n0 .. n0 + rows - 1: one contiguous span of rows * KB floats
    const float* asrc = a.alpha + n0 * KB;
    for (int e = tid; e < rows * KB; e += BB_WAVES * 64) {
        const int row = e / KB;
        as[row * KBp + (e - row * KB)] = asrc[e];
    }
    if (tid < 16 * MT) bsc[tid] = (double)beta_ld / 127.0;
    __syncthreads();
    double f[RB][MT][4];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) f[r][t][i] = 0.0;
    const i32x4 zero = {0, 0, 0, 0};
    for (int s = wave; s < SP; s += BB_WAVES) {
        // the fetch of this sub-step has landed in the image (the only loads in flight)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        i32x4 av[MT][4];
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) av[t][q] = xs[(16 * t + lr) * 16 + ((4 * q + lg) ^ lr)];
        uint32_t wd[RB][4];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) wd[r][q] = ws32[(64 * r + 16 * q + lr) * 4 + lg];
        // the next fetch rewrites the image: every read of it has to be complete first
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        if (s + BB_WAVES < SP) fetch(s + BB_WAVES);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float al[RB];
#pragma unroll
            for (int r = 0; r < RB; ++r) al[r] = as[arow[r] + 2 * s + h];
            i32x4 blk[RB][MT];
#pragma unroll
            for (int q = 2 * h; q < 2 * h + 2; ++q)
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const i32x4 bv = expand_signed_in_order(wd[r][q]);
#pragma unroll
                    for (int t = 0; t < MT; ++t)
                        blk[r][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[t][q], bv, q == 2 * h ? zero : blk[r][t], 0, 0, 0);
                }
            // column l % 16 of a tile is this lane's row: scale its block sums by the row's alpha
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        f[r][t][i] = __builtin_fma((double)al[r], (double)blk[r][t][i], f[r][t][i]);
        }
    }
    __syncthreads();                               // images and alpha rows no longer read
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) redd[(((wave * RB * MT) + r * MT + t) * 4 + i) * 64 + lane] = f[r][t][i];
    __syncthreads();
    static_assert(RB * MT * 64 <= BB_WAVES * 64, "one epilogue element per thread");
    if (tid < RB * MT * 64) {
        const int l = tid & 63, tile = tid >> 6;
        const int r = tile / MT, t = tile % MT;
        const int64_t n = n0 + 16 * r + (l & 15);
        if (n < N) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 16 * t + 4 * (l >> 4) + i;
                if (m >= M) continue;
                double sum = 0.0;
#pragma unroll
                for (int w = 0; w < BB_WAVES; ++w) sum += redd[((w * RB * MT + tile) * 4 + i) * 64 + l];
                float v = (float)(sum * bsc[m]);
                if (a.bias) v = v + bias_e;
                a.y[(int64_t)m * N + n] = v;
            }
        }
    }
}

template <int MT, int RB>
static size_t bdec16n_blocks_lds(int64_t K) {
    const size_t images = (size_t)BB_WAVES * (4 * MT + RB) * 64 * sizeof(i32x4) + (size_t)16 * RB * (K / 128 + 1) * sizeof(float);
    const size_t tiles = (size_t)BB_WAVES * RB * MT * 4 * 64 * sizeof(double);
    return images > tiles ? images : tiles;
}
// halves: the tokens in two halves of MT tiles each on a second grid dimension
template <int MT, int RB>
static hipError_t launch_bdec16n_blocks(const BlockArgs& a, hipStream_t s, bool halves = false) {
    const int64_t wgs = (a.N + 16 * RB - 1) / (16 * RB);
    const unsigned ty = halves ? (unsigned)((a.M + 16 * MT - 1) / (16 * MT)) : 1u;
    return launch_with_lds(k_bdec16n_blocks<MT, RB>, dim3((unsigned)wgs, ty), dim3(BB_WAVES * 64), bdec16n_blocks_lds<MT, RB>(a.K), s, a);
}
// Measured with weights not in cache, outputs identical to the earlier kernel (32-token slices
// of k_bdec16_blocks, in brackets): K = 4096, N = 11008: M = 8 / 16 / 32 / 64: 8.1 / 8.3 / 9.9 /
// 17.5 us (8.2 / 8.8 / 13.8 / 27.2); K = 11008, N = 4096: M = 16 / 32 / 64: 8.7 / 10.9 / 15.4 us
// (10.2 / 16.7 / 32.9); K = 8192, N = 8192, M = 64: 15.4 us (22.7 as two 32-token slices of this
// kernel).
// Sub-steps interleaved over the waves then took M = 16 to 7.7 us (8.5), M = 32 to 9.4 (10.1),
// K = 8192, N = 8192, M = 64 to 15.6 (16.7); M = 64, K = 4096, N = 11008 level.  With them it
// also beats the earlier kernel from three tokens: M = 3 / 4 / 7, K = 4096, N = 11008: 7.5 /
// 7.5 / 7.4 us (7.9 / 8.1 / 8.1); M = 4, K = 11008, N = 4096: 7.7 us (9.0).
// One slice of up to 64 tokens: MT = ceil(M / 16) token tiles and the fewest row blocks per
// workgroup that keep the grid within 256 workgroups, up to three for one or two tiles and two
// for three or four (the fp64 accumulators and the one-element-per-thread epilogue); false
// when the shape is not one this kernel takes (K % 256 != 0, more than 768 16-row blocks,
// offsets past 32 bits, images and alpha rows past the LDS).
template <int MT, int RB>
static bool bdec16n_blocks_try(const BlockArgs& a, hipStream_t s, hipError_t* e, bool halves = false) {
    if (bdec16n_blocks_lds<MT, RB>(a.K) + 16 * MT * sizeof(double) > 160 * 1024) return false;
    *e = launch_bdec16n_blocks<MT, RB>(a, s, halves);
    return true;
}
template <int MT>
static bool bdec16n_blocks_rb(const BlockArgs& a, int64_t nb16, hipStream_t s, hipError_t* e) {
    if (nb16 <= 256) return bdec16n_blocks_try<MT, 1>(a, s, e);
    if (nb16 <= 512 || MT > 2) return bdec16n_blocks_try<MT, 2>(a, s, e);
    if constexpr (MT <= 2) return bdec16n_blocks_try<MT, 3>(a, s, e);
    return false;
}
static bool bdec16n_blocks_launch(const BlockArgs& a, hipStream_t s, hipError_t* e) {
    const int64_t nb16 = (a.N + 15) / 16;
    if (a.M > 64 || a.K % 256 != 0 || nb16 > 768 || a.M * a.K >= (int64_t(1) << 31) ||
        a.N * (a.K / 4) >= (int64_t(1) << 32))
        return false;
    if (a.M <= 16) return bdec16n_blocks_rb<1>(a, nb16, s, e);
    // at most 256 16-row blocks: the tokens in two halves, each workgroup reading half of x_q
    // for twice the rows, as in the per-tensor kernel (same outputs; M = 64, K = 11008,
    // N = 4096: 13.3 against 16.1 us; K = 16384: 17.6 against 20.6 us; M = 32, K = 11008:
    // 10.0 against 10.8 us)
    if (nb16 <= 256) {
        if (a.M <= 32) return nb16 <= 128 ? bdec16n_blocks_try<1, 1>(a, s, e, true) : bdec16n_blocks_try<1, 2>(a, s, e, true);
        return nb16 <= 128 ? bdec16n_blocks_try<2, 1>(a, s, e, true) : bdec16n_blocks_try<2, 2>(a, s, e, true);
    }
    if (a.M <= 32) return bdec16n_blocks_rb<2>(a, nb16, s, e);
    if (a.M <= 48) return bdec16n_blocks_rb<3>(a, nb16, s, e);
    return bdec16n_blocks_rb<4>(a, nb16, s, e);
}

// 3 to 32 tokens: the fewest row blocks per workgroup that keep the grid within 256
// workgroups (three at N = 11008: 230 workgroups, where four left 84 CUs idle), at most 4 for
// one token block and 3 for two (beyond, the fp64 accumulators spill); larger N gets more
// workgroups.
static hipError_t launch_bdec16_blocks_m(const BlockArgs& a, hipStream_t s) {
    const int64_t rb = ((a.N + 15) / 16 + 255) / 256;
    if (a.M <= 16) {
        switch (rb) {
            case 1: return launch_bdec16_blocks<1, 1>(a, s);
            case 2: return launch_bdec16_blocks<1, 2>(a, s);
            case 3: return launch_bdec16_blocks<1, 3>(a, s);
            default: return launch_bdec16_blocks<1, 4>(a, s);
        }
    }
    switch (rb) {
        case 1: return launch_bdec16_blocks<2, 1>(a, s);
        case 2: return launch_bdec16_blocks<2, 2>(a, s);
        default: return launch_bdec16_blocks<2, 3>(a, s);
    }
}

// ---------------------------------------------------------------------------------------
// 128 tokens and more (prefill): a GEMM on 128 x 128 tiles, four waves of 64 x 64 (2 x 2 tiles
// of v_mfma_i32_32x32x32_i8), K steps of 64 through double-buffered LDS with one barrier per
// step.  x_q is transposed 4x4 on its way into LDS (as in the per-tensor GEMM); the weight
// codes go to the B operand as signed bytes W_hat = c - 1 through a v_perm table, so a
// block's int32 sums need no sums of x_q.  A block's sums start from zero (the first MFMA of
// its first step takes a zero accumulator) and after its second step are added to per-output
// fp64 accumulators as alpha[n, b] * acc: the products are exact (24 x 15 bits) and the
// blocks are added in ascending order, so S, and y after its one fp32 rounding, are those of
// the plain fp64 sum bit for bit.  Measured at M = 2048, K = 4096, N = 11008: 201 us against
// 1360 us for 64 slices of the 32-token kernel (0.92 against 0.14 POPS); N = 4096: 80 against
// 672 us.  Two workgroups per CU (253 VGPRs); one measured 276 us.
template <int WGS>
__global__ __launch_bounds__(256, WGS) void k_gemm_blocks(BlockArgs a, int tiles_m, int tiles_n) {
    constexpr int BM = 128, BN = 128, BK = 64, GK = BK / 16, APT = BM * GK / 256, ASTR = GK + 1;
    __shared__ u32x4 As[2][BM * ASTR];
    __shared__ u32x4 Bs[2][BN];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = a.M, N = a.N, K = a.K, rowb = K >> 2, KB = K >> 7;
    const int T = tiles_m * tiles_n;
    int t = blockIdx.x;
    if (T % 8 == 0) t = (t % 8) * (T / 8) + t / 8;
    const int tm = t / tiles_n, tn = t % tiles_n;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int KS = (int)(K / BK);
    const int lr = lane & 31, lg = lane >> 5;

    const int8_t* ap[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) {
        const int u = tid + 256 * i;
        ap[i] = a.xq + min(m0 + u / GK, M - 1) * K + 16 * (u % GK);
    }
    const int brow = tid & (BN - 1);                    // threads 128..255 duplicate 0..127 (not stored)
    const uint8_t* bp = a.wp + min(n0 + brow, N - 1) * rowb;
    const bool bsw = (brow >> 4) & 1;
    // this lane's two output columns, their alpha rows
    const float* alr[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) alr[j] = a.alpha + min(n0 + wn * 64 + j * 32 + lr, N - 1) * KB;

    u32x4 ra0[APT], ra1[APT], rb0, rb1;
    auto gload = [&](u32x4 (&ra)[APT], u32x4& rb, int ks) {
#pragma unroll
        for (int i = 0; i < APT; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ap[i] + (int64_t)ks * BK);
        rb = *reinterpret_cast<const u32x4*>(bp + (int64_t)ks * (BK / 4));
    };
    auto stage = [&](const u32x4 (&ra)[APT], const u32x4& rb, int buf) {
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int u = tid + 256 * i;
            As[buf][(u / GK) * ASTR + u % GK] = transpose4x4_perm(ra[i]);
        }
        if (tid < BN) Bs[buf][tid] = bsw ? u32x4{rb.z, rb.w, rb.x, rb.y} : rb;
    };
    int boff[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = wn * 64 + j * 32 + lr;
            boff[kk][j] = col * 4 + ((2 * kk + lg) ^ (((col >> 4) & 1) << 1));
        }
    // signed code bytes: c = 0, 1, 2 -> -1, 0, +1
    auto sgn = [](uint32_t f) { return (int)__builtin_amdgcn_perm(0u, 0x000100FFu, f); };

    i32x16 acc[2][2];
    double S[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            acc[i][j] = i32x16{};
#pragma unroll
            for (int r = 0; r < 16; ++r) S[i][j][r] = 0.0;
        }
    float al[2] = {0.0f, 0.0f};

    auto step = [&](int buf, int ks) {
        const uint32_t* b32 = reinterpret_cast<const uint32_t*>(&Bs[buf][0]);
        i32x4 av[2][2], bv[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int i = 0; i < 2; ++i) av[kk][i] = (i32x4)As[buf][(wm * 64 + i * 32 + lr) * ASTR + kk * 2 + lg];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const uint32_t w = b32[boff[kk][j]];
                bv[kk][j] = i32x4{sgn(w & 0x03030303u), sgn((w >> 2) & 0x03030303u), sgn((w >> 4) & 0x03030303u),
                                  sgn((w >> 6) & 0x03030303u)};
            }
        }
        const bool first = (ks & 1) == 0;
        if (first) {                                    // alpha of this block, used after its second step
#pragma unroll
            for (int j = 0; j < 2; ++j) al[j] = alr[j][ks >> 1];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[0][i], bv[0][j], first ? i32x16{} : acc[i][j], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[1][i], bv[1][j], acc[i][j], 0, 0, 0);
        if (!first) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const double aj = (double)al[j];
#pragma unroll
                    for (int r = 0; r < 16; ++r) S[i][j][r] = fma(aj, (double)acc[i][j][r], S[i][j][r]);
                }
        }
    };

    const int last = KS - 1;
    gload(ra0, rb0, 0);
    gload(ra1, rb1, KS > 1 ? 1 : 0);
    stage(ra0, rb0, 0);
    __syncthreads();
    for (int ks = 0; ks < KS; ks += 2) {           // KS is even (K % 128 == 0)
        gload(ra0, rb0, min(ks + 2, last));
        stage(ra1, rb1, 1);
        step(0, ks);
        __syncthreads();
        gload(ra1, rb1, min(ks + 3, last));
        stage(ra0, rb0, 0);
        step(1, ks + 1);
        __syncthreads();
    }
    // epilogue: y = fp32(S * (beta / 127)) (+ bias)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
            if (m >= M) continue;
            const double tb = (double)a.beta[m] / 127.0;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t n = n0 + wn * 64 + j * 32 + lr;
                if (n >= N) continue;
                float v = (float)(S[i][j][r] * tb);
                if (a.bias) v = v + a.bias[n];
                a.y[m * N + n] = v;
            }
        }
}

template <int WGS>
static hipError_t launch_gemm_blocks(const BlockArgs& a, hipStream_t s) {
    const int tm = (int)((a.M + 127) / 128), tn = (int)((a.N + 127) / 128);
    hipLaunchKernelGGL(k_gemm_blocks<WGS>, dim3((unsigned)(tm * tn)), dim3(256), 0, s, a, tm, tn);
    return hipGetLastError();
}

bool blocks_supports(int64_t K) { return K % 128 == 0 && K <= 32768; }

template <int MT, int CPL, int R>
static hipError_t launch_blocks_r(const BlockArgs& a, int64_t groups, hipStream_t s) {
    const int64_t wgs = (a.N + a.rows_per_wave * BW_WAVES - 1) / (a.rows_per_wave * BW_WAVES);
    const size_t lds = (size_t)MT * CPL * (256 * sizeof(u32x4) + 64 * sizeof(int));
    return launch_with_lds(k_gemv_blocks<MT, CPL, R>, dim3((unsigned)wgs, (unsigned)groups), dim3(64 * BW_WAVES), lds, s,
                           a);
}

// Rows are spread over 1024 workgroups of 8 waves (four per CU) for rows of up to two chunks
// per lane (K <= 8192), over 512 for longer rows, which gain from two rows per wave in the
// double-buffered walk (measured with weights not in cache, one token: 5.9 vs 7.1 us at
// K = 4096, N = 11008; 16.2 vs 16.8 us at K = 28672, N = 8192).  A wave's step holds up to 8
// chunk loads per lane, so R rows of CPL chunks with R * CPL <= 8 and R <= the wave's rows.
template <int MT, int CPL>
static hipError_t launch_blocks_mt(const BlockArgs& a0, int64_t groups, hipStream_t s) {
    BlockArgs a = a0;
    constexpr int RMAX = CPL >= 8 ? 1 : 8 / CPL;
    constexpr int64_t WGS = CPL <= 2 ? 1024 : 512;
    a.rows_per_wave = (a.N + WGS * BW_WAVES - 1) / (WGS * BW_WAVES);
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

// One or two tokens: the GEMV; 3 to 127: MFMA kernels over slices of up to 64 tokens (32 on the
// earlier kernel when K % 256 != 0; that kernel against the GEMV at three tokens, weights not in
// cache: 10.9 vs 12.8 us at K=4096, N=11008; 21.0 vs 31.7 us at K=28672, N=8192).
hipError_t launch_forward_blocks(const int8_t* xq, const float* beta, int64_t M, int64_t K, const uint8_t* wp,
                                 const float* alpha, int64_t N, const float* bias, float* y, hipStream_t s) {
    const BlockArgs a{xq, beta, M, K, N, wp, alpha, bias, y, 0};
    if (M == 1) return launch_blocks_cpl<1>(a, 1, s);
    if (M == 2) return launch_blocks_cpl<2>(a, 1, s);
    // from 128 tokens the GEMM (one 128-token tile row and more); below, 32-token slices of the
    // decode kernel (measured at M = 64, K = 4096, N = 11008, weights not in cache: two slices
    // 43.3 us, the GEMM's 86 workgroups 46.0 us)
    if (M >= 128) return launch_gemm_blocks<2>(a, s);
    for (int64_t m0 = 0; m0 < M;) {
        BlockArgs sl = a;
        sl.xq = xq + m0 * K;
        sl.beta = beta + m0;
        sl.y = y + m0 * N;
        hipError_t e = hipSuccess;
        sl.M = M - m0 < 64 ? M - m0 : 64;
        if (sl.M < 3 || !bdec16n_blocks_launch(sl, s, &e)) {
            sl.M = M - m0 < 32 ? M - m0 : 32;
            e = launch_bdec16_blocks_m(sl, s);
        }
        if (e != hipSuccess) return e;
        m0 += sl.M;
    }
    return hipSuccess;
}

}  // namespace bitlinear
