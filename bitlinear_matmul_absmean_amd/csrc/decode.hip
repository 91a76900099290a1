// decode.hip -- batched-decode ternary x int8 matmul (2 to 64 tokens) on the int8 matrix
// cores (v_mfma_i32_32x32x32_i8 and v_mfma_i32_16x16x64_i8), gfx950.
//
// What is computed ([P3] chenxutan.com "1.58-bit 大模型极限量化实战" §2.4-§2.5, §3.2;
// [P2] nxmr.cn "1.58 位大模型" §3.3): acc = x_q . W_hat^T (int32), y = fp32(acc) *
// fp32(alpha*beta[m]/127) (+ bias).
//
// With up to 64 tokens the product is bound by memory, not by the matrix cores (the ridge of
// int8 MFMA against HBM is near 78 tokens), so the layout is chosen for bytes:
//   * a workgroup of eight waves owns RB blocks of 32 weight rows, and the grid has about one
//     workgroup per CU, so every workgroup reads its weight rows once and the activations
//     x_q (M x K bytes) once;
//   * the eight waves split K: wave w walks its own range of 128-weight sub-steps, loading
//     its slice of x_q straight from global memory (cache-resident after the first
//     workgroup) into MFMA A registers, with no LDS staging and no barrier in the main loop;
//     only the eight partial 32 x 32 tiles per (row block, token block) are added through LDS
//     at the end (integer sums: exact in any order);
//   * inside a 128-weight sub-step, lane group g (lanes 32g..32g+31) takes the four 16-weight
//     groups 4g..4g+3, so each lane reads 64 contiguous bytes of x_q per token block and 16
//     contiguous bytes (64 codes) per weight row: A and B operands of one MFMA then sit at the
//     same k, and every load covers whole 64-byte runs of a row;
//   * a packed dword (16 codes, weight 4b+i at bits 2i of byte b) expands with four masks
//     (v >> 2i) & 0x03030303 into the 16-byte B operand: byte 4i+j = c of weight 4j+i, with
//     c = W + 1; the matching x_q bytes are transposed 4x4 with v_perm; acc = sum c*x_q -
//     sum x_q, the per-token sum of x_q accumulated on the way.
// MFMA 32x32x32 i8 lane layout (checked on the device): A/B lane l holds row/column l%32,
// k = 16*(l/32)+j; accumulator r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#include "common.hpp"

namespace bitlinear {

constexpr int BD_WAVES = 8;

// MT: 32-token blocks (tokens <= 32*MT); RB: 32-row blocks per workgroup.
// x_q goes through a wave-private LDS region: eight lanes read one token's 128 bytes of a
// sub-step (whole cache lines; a load instruction covers 8 tokens), transpose each 16-byte
// group 4x4 and store it; the MFMA A operands are then read back from LDS.  Reading x_q
// straight into the operand layout would touch 16 bytes of each of 32 token rows per load
// instruction, which the texture path serves one cache line at a time.
template <int MT, int RB>
__global__ __launch_bounds__(BD_WAVES * 64) void k_bdec(ForwardArgs a) {
    // first the x_q staging ([wave][MT * 32 token rows][XU units]), then the partial tiles
    extern __shared__ i32x4 red[];
    __shared__ int tsum_w[BD_WAVES][MT * 32];
    constexpr int XU = 9;                          // 16-byte units per token row (8 + 1 of padding)
    constexpr int XR = MT * 32 * XU;               // units of one wave's region
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = (int)a.M;
    const int64_t K = a.K, N = a.N, rowb = K >> 2;
    const int64_t n0 = (int64_t)blockIdx.x * (32 * RB);
    const int lr = lane & 31, lg = lane >> 5;
    i32x4* xs = red + wave * XR;

    // sub-steps of 128 weights; wave w takes [s0, s1)
    const int SP = (int)((K + 127) / 128);
    const int s0 = (int)((int64_t)SP * wave / BD_WAVES), s1 = (int)((int64_t)SP * (wave + 1) / BD_WAVES);

    // x_q loads: instruction i covers tokens 8i + lane/8, unit u = lane % 8 (16 bytes at k0 + 16u);
    // weight loads: lane (lr, lg) reads 16 bytes (64 codes at k0 + 64 lg) of row n0 + 32r + lr.
    // Rows past M or N are clamped (never written); past K (the last sub-step when
    // K % 128 == 64) the loads re-read the row start and the staged x_q is zeroed.
    const int xu = lane & 7, xt = lane >> 3;
    const int8_t* xrow[MT * 4];
#pragma unroll
    for (int i = 0; i < MT * 4; ++i) xrow[i] = a.xq + (int64_t)min(8 * i + xt, M - 1) * K + 16 * xu;
    const uint8_t* wrow[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) wrow[r] = a.wp + min(n0 + 32 * r + lr, N - 1) * rowb;

    u32x4 xa[2][MT * 4], wb[2][RB];
    auto load = [&](int st, int s) {
        const int64_t kx = (int64_t)s * 128 + 16 * xu < K ? (int64_t)s * 128 : 0;
#pragma unroll
        for (int i = 0; i < MT * 4; ++i) xa[st][i] = *reinterpret_cast<const u32x4*>(xrow[i] + kx);
        const int64_t kw = (int64_t)s * 128 + 64 * lg;
        const int64_t kwx = kw < K ? kw : 0;
#pragma unroll
        for (int r = 0; r < RB; ++r) wb[st][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[r] + kwx / 4));
    };

    i32x16 acc[RB][MT];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = i32x16{};
    int ts[MT * 4];
#pragma unroll
    for (int i = 0; i < MT * 4; ++i) ts[i] = 0;

    auto compute = [&](int st, int s) {
        // stage x_q (transposed) and expand the weights of this sub-step
        const bool xlive = (int64_t)s * 128 + 16 * xu < K;
#pragma unroll
        for (int i = 0; i < MT * 4; ++i) {
            const u32x4 v = xlive ? xa[st][i] : u32x4{0u, 0u, 0u, 0u};
            xs[(8 * i + xt) * XU + xu] = (i32x4)transpose4x4_perm(v);
            int z = ts[i];
            z = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, z, false);
            z = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, z, false);
            z = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, z, false);
            ts[i] = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, z, false);
        }
        i32x4 bv[RB][4];
#pragma unroll
        for (int r = 0; r < RB; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t w = q == 0 ? wb[st][r].x : q == 1 ? wb[st][r].y : q == 2 ? wb[st][r].z : wb[st][r].w;
                bv[r][q] = i32x4{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u),
                                 (int)((w >> 4) & 0x03030303u), (int)((w >> 6) & 0x03030303u)};
            }
        // in MFMA q, lane group g takes the 16-weight group 4g + q of the sub-step
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            i32x4 av[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) av[t] = xs[(32 * t + lr) * XU + 4 * lg + q];
#pragma unroll
            for (int r = 0; r < RB; ++r)
#pragma unroll
                for (int t = 0; t < MT; ++t)
                    acc[r][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[t], bv[r][q], acc[r][t], 0, 0, 0);
        }
    };

    // two register stages; each sub-step first consumes its stage (LDS store, weight expansion),
    // then the stage is refilled with the sub-step after next
    if (s0 < s1) {
        const int last = s1 - 1;
        load(0, s0);
        load(1, min(s0 + 1, last));
        int s = s0;
        for (; s + 2 <= s1; s += 2) {
            compute(0, s);
            __builtin_amdgcn_sched_barrier(0);
            load(0, min(s + 2, last));
            __builtin_amdgcn_sched_barrier(0);
            compute(1, s + 1);
            __builtin_amdgcn_sched_barrier(0);
            load(1, min(s + 3, last));
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s < s1) compute(0, s);
    }

    // per-token sums of x_q: the eight lanes xt of a token hold its eight 16-byte groups
#pragma unroll
    for (int i = 0; i < MT * 4; ++i) {
        int v = ts[i];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64);
        if (xu == 0) tsum_w[wave][8 * i + xt] = v;
    }
    __syncthreads();                               // every wave is done with its staging region
    // per token, once per workgroup: the x_q sum over all of K and (per-tensor alpha) the scale
    __shared__ int tsum_t[MT * 32];
    __shared__ float scale_t[MT * 32];
    if (tid < MT * 32) {
        int v = 0;
#pragma unroll
        for (int w = 0; w < BD_WAVES; ++w) v += tsum_w[w][tid];
        tsum_t[tid] = v;
        scale_t[tid] = (!a.alpha_per_row && tid < M) ? dequant_scale(a.alpha[0], a.beta[tid]) : 0.0f;
    }
    // partial tiles to LDS: tile (r, t) of wave w at red[((w * RB * MT + r * MT + t) * 4 + c) * 64 + lane]
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                red[((wave * RB * MT + r * MT + t) * 4 + c) * 64 + lane] =
                    i32x4{acc[r][t][4 * c], acc[r][t][4 * c + 1], acc[r][t][4 * c + 2], acc[r][t][4 * c + 3]};
    __syncthreads();

    // epilogue: element e = (tile, c, lane) -> accumulator regs 4c..4c+3 of that lane:
    // token 32 t + 8 c + 4 (lane / 32) + i, weight row n0 + 32 r + lane % 32
    for (int e = tid; e < RB * MT * 4 * 64; e += BD_WAVES * 64) {
        const int l = e & 63, c = (e >> 6) & 3, tile = e >> 8;
        const int r = tile / MT, t = tile % MT;
        i32x4 sum = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < BD_WAVES; ++w) sum += red[((w * RB * MT + tile) * 4 + c) * 64 + l];
        const int64_t n = n0 + 32 * r + (l & 31);
        if (n >= N) continue;
        const float al = a.alpha_per_row ? a.alpha[n] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 32 * t + 8 * c + 4 * (l >> 5) + i;
            if (m >= M) continue;
            const int total = sum[i] - tsum_t[m];
            const float sc = a.alpha_per_row ? dequant_scale(al, a.beta[m]) : scale_t[m];
            a.y[(int64_t)m * N + n] = activate(dequant(total, sc, a.bias, n), a.act);
            if (a.acc) a.acc[(int64_t)m * N + n] = total;
        }
    }
}

template <int MT, int RB>
static hipError_t launch_bdec(const ForwardArgs& a, hipStream_t s) {
    const int64_t blocks = (a.N + 32 * RB - 1) / (32 * RB);
    const size_t stage = (size_t)BD_WAVES * MT * 32 * 9 * sizeof(i32x4);
    const size_t tiles = (size_t)BD_WAVES * RB * MT * 4 * 64 * sizeof(i32x4);
    return launch_with_lds(k_bdec<MT, RB>, dim3((unsigned)blocks), dim3(BD_WAVES * 64), stage > tiles ? stage : tiles, s, a);
}

// The same scheme on 16 x 16 x 64 tiles for up to 16 tokens: four lanes share a weight row
// (lane group g = l / 16 holds 64 contiguous weights of it), so a load instruction covers 16
// rows x 64 bytes instead of 32 rows x 32 bytes, and x_q is loaded for 16 token rows instead
// of 32.  Sub-steps of 256 weights; in MFMA q of a sub-step lane group g takes the 16-weight
// group 4g + q.  16x16x64 lane layout (checked on the device): A/B lane l holds row/column
// l%16, k = 16*(l/16)+j; accumulator r of lane l is row 4*(l/16) + r, column l%16.
template <int MT, int RB>
__global__ __launch_bounds__(BD_WAVES * 64) void k_bdec16(ForwardArgs a) {
    extern __shared__ i32x4 red[];                 // [wave][RB * MT tiles][64]
    __shared__ int tsum_w[BD_WAVES][16 * MT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = (int)a.M;
    const int64_t K = a.K, N = a.N, rowb = K >> 2;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * RB);
    const int lr = lane & 15, lg = lane >> 4;
    const int SP = (int)((K + 255) / 256);
    const int s0 = (int)((int64_t)SP * wave / BD_WAVES), s1 = (int)((int64_t)SP * (wave + 1) / BD_WAVES);
    const int8_t* xrow[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) xrow[t] = a.xq + (int64_t)min(16 * t + lr, M - 1) * K;
    const uint8_t* wrow[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) wrow[r] = a.wp + min(n0 + 16 * r + lr, N - 1) * rowb;

    // a lane group whose 64 weights lie past K (K % 256 != 0) re-reads the first 64 weights of
    // its rows and its x_q is zeroed, so the products vanish
    u32x4 xa[3][MT][4], wb[3][RB];
    auto load = [&](int st, int s) {
        const int64_t k0 = (int64_t)s * 256 + 64 * lg;
        const int64_t kx = k0 < K ? k0 : 0;
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) xa[st][t][q] = *reinterpret_cast<const u32x4*>(xrow[t] + kx + 16 * q);
#pragma unroll
        for (int r = 0; r < RB; ++r) wb[st][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[r] + kx / 4));
    };
    i32x4 acc[RB][MT];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = i32x4{0, 0, 0, 0};
    int ts[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) ts[t] = 0;
    auto compute = [&](int st, int s) {
        const bool live = (int64_t)s * 256 + 64 * lg < K;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            i32x4 av[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const u32x4 v = live ? xa[st][t][q] : u32x4{0u, 0u, 0u, 0u};
                av[t] = (i32x4)transpose4x4_perm(v);
                int z = ts[t];
                z = __builtin_amdgcn_sdot4((int)v.x, 0x01010101, z, false);
                z = __builtin_amdgcn_sdot4((int)v.y, 0x01010101, z, false);
                z = __builtin_amdgcn_sdot4((int)v.z, 0x01010101, z, false);
                ts[t] = __builtin_amdgcn_sdot4((int)v.w, 0x01010101, z, false);
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t w = q == 0 ? wb[st][r].x : q == 1 ? wb[st][r].y : q == 2 ? wb[st][r].z : wb[st][r].w;
                const i32x4 bv = {(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u),
                                  (int)((w >> 4) & 0x03030303u), (int)((w >> 6) & 0x03030303u)};
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[r][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[t], bv, acc[r][t], 0, 0, 0);
            }
        }
    };
    if (s0 < s1) {
        const int last = s1 - 1;
        load(0, s0);
        load(1, min(s0 + 1, last));
        load(2, min(s0 + 2, last));
        int s = s0;
        for (; s + 3 <= s1; s += 3) {
            compute(0, s);
            __builtin_amdgcn_sched_barrier(0);
            load(0, min(s + 3, last));
            __builtin_amdgcn_sched_barrier(0);
            compute(1, s + 1);
            __builtin_amdgcn_sched_barrier(0);
            load(1, min(s + 4, last));
            __builtin_amdgcn_sched_barrier(0);
            compute(2, s + 2);
            __builtin_amdgcn_sched_barrier(0);
            load(2, min(s + 5, last));
            __builtin_amdgcn_sched_barrier(0);
        }
        if (s < s1) compute(0, s);
        if (s + 1 < s1) compute(1, s + 1);
    }
    // token sums: the four lane groups of token l%16 hold disjoint parts of its k range
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        int v = ts[t] + __shfl_xor(ts[t], 16, 64);
        v += __shfl_xor(v, 32, 64);
        if (lg == 0) tsum_w[wave][16 * t + lr] = v;
    }
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) red[(wave * RB * MT + r * MT + t) * 64 + lane] = acc[r][t];
    __syncthreads();
    // per token, once per workgroup: the x_q sum over all of K and (per-tensor alpha) the scale
    __shared__ int tsum_t[MT * 16];
    __shared__ float scale_t[MT * 16];
    if (tid < MT * 16) {
        int v = 0;
#pragma unroll
        for (int w = 0; w < BD_WAVES; ++w) v += tsum_w[w][tid];
        tsum_t[tid] = v;
        scale_t[tid] = (!a.alpha_per_row && tid < M) ? dequant_scale(a.alpha[0], a.beta[tid]) : 0.0f;
    }
    __syncthreads();
    for (int e = tid; e < RB * MT * 64; e += BD_WAVES * 64) {
        const int l = e & 63, tile = e >> 6;
        const int r = tile / MT, t = tile % MT;
        i32x4 sum = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < BD_WAVES; ++w) sum += red[(w * RB * MT + tile) * 64 + l];
        const int64_t n = n0 + 16 * r + (l & 15);
        if (n >= N) continue;
        const float al = a.alpha_per_row ? a.alpha[n] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * t + 4 * (l >> 4) + i;
            if (m >= M) continue;
            const int total = sum[i] - tsum_t[m];
            const float sc = a.alpha_per_row ? dequant_scale(al, a.beta[m]) : scale_t[m];
            a.y[(int64_t)m * N + n] = activate(dequant(total, sc, a.bias, n), a.act);
            if (a.acc) a.acc[(int64_t)m * N + n] = total;
        }
    }
}

template <int MT, int RB>
static hipError_t launch_bdec16(const ForwardArgs& a, hipStream_t s) {
    const int64_t blocks = (a.N + 16 * RB - 1) / (16 * RB);
    const size_t lds = (size_t)BD_WAVES * RB * MT * 64 * sizeof(i32x4);
    return launch_with_lds(k_bdec16<MT, RB>, dim3((unsigned)blocks), dim3(BD_WAVES * 64), lds, s, a);
}



// k_bdec16 for whole 256-weight sub-steps (K % 256 == 0, no K-tail selects) with an ST-stage
// register pipeline whose loads past the wave's range are skipped.  With two stages and as
// many 16-row blocks per workgroup as keep the grid within 256 workgroups (three at N = 11008:
// 230 workgroups, where four left 84 CUs idle), measured with weights not in cache against the
// earlier choices (k_bdec16 with 1, 2, 4 or 8 row blocks, k_bdec for 17 to 32 tokens on wide
// matrices): K = 4096, N = 11008: 4 / 8 / 16 / 24 / 32 tokens 6.37 / 6.69 / 7.17 / 8.64 / 9.34 us
// against 7.17 / 7.54 / 8.07 / 13.66 / 14.36 us; K = 8192, N = 10240: 8.8 / 9.6 / 11.4 / 14.4 /
// 15.5 against 13.4 / 14.4 / 16.6 / 19.9 / 20.9 us; K = 8192, N = 28672, 24 tokens 24.9 against
// 39.0 us; K = 11008, N = 4096 and K = 28672, N = 8192 level or up to 9% faster.  Three and four
// stages were slower on every one of these shapes except a few within 2%.
// x_q goes through a wave-private LDS image: read straight into the operand layout, a load
// instruction touched 16 bytes in each of 64 places (16 token rows x 4 lane groups); staged,
// sixteen lanes read a token's 256 bytes of the sub-step in whole lines, transpose their groups
// and store them, and the operands come back from LDS.  The token sums of x_q come from MFMAs
// against an all-ones operand.  Measured with weights not in cache, 16 / 32 tokens: K = 11008,
// N = 4096, 8.29 / 11.19 against 9.53 / 14.13 us; K = 8192, N = 10240, 9.89 / 12.39 against
// 11.37 / 15.55 us; K = 28672, N = 8192, 22.0 / 29.2 against 25.4 / 36.4 us; K = 4096,
// N = 11008, 6.90 / 8.41 against 7.16 / 9.33 us; 4 tokens level.
template <int MT, int RB, int ST>
__global__ __launch_bounds__(BD_WAVES * 64) void k_bdec16w(ForwardArgs a) {
    extern __shared__ i32x4 red[];
    __shared__ int tsum_w[BD_WAVES][16 * MT];
    __shared__ int tsum_t[MT * 16];
    __shared__ float scale_t[MT * 16];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = (int)a.M;
    const int64_t K = a.K, N = a.N, rowb = K >> 2;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * RB);
    const int lr = lane & 15, lg = lane >> 4;
    const int SP = (int)(K >> 8);
    // the wave's i-th sub-step is wave + 8 i (interleaved over the waves)
    const int s0 = 0, s1 = wave < SP ? (SP - wave + BD_WAVES - 1) / BD_WAVES : 0;
    // x_q of a sub-step (16 MT tokens x 256 bytes) is loaded in whole lines: instruction i
    // covers tokens 4i .. 4i+3, sixteen lanes per token; each lane transposes its 16-byte group
    // and stores it in a wave-private LDS image, rows padded by one unit, from which the MFMA
    // A operands are read back
    constexpr int XSTR = 17, XR = MT * 16 * XSTR;
    i32x4* xs = red + wave * XR;
    const int xg = lane & 15, xt = lane >> 4;
    const int8_t* xrow[4 * MT];
#pragma unroll
    for (int i = 0; i < 4 * MT; ++i) xrow[i] = a.xq + (int64_t)min(4 * i + xt, M - 1) * K + 16 * xg;
    const uint8_t* wrow[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) wrow[r] = a.wp + min(n0 + 16 * r + lr, N - 1) * rowb + 16 * lg;
    u32x4 xa[ST][4 * MT], wb[ST][RB];
    auto load = [&](int st, int s) {
#pragma unroll
        for (int i = 0; i < 4 * MT; ++i) xa[st][i] = *reinterpret_cast<const u32x4*>(xrow[i] + (int64_t)(wave + BD_WAVES * s) * 256);
#pragma unroll
        for (int r = 0; r < RB; ++r) wb[st][r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[r] + (int64_t)(wave + BD_WAVES * s) * 64));
    };
    i32x4 acc[RB][MT];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = i32x4{0, 0, 0, 0};
    const i32x4 ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    i32x4 tsm[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) tsm[t] = i32x4{0, 0, 0, 0};
    auto compute = [&](int st) {
#pragma unroll
        for (int i = 0; i < 4 * MT; ++i) xs[(4 * i + xt) * XSTR + xg] = (i32x4)transpose4x4_perm(xa[st][i]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            i32x4 av[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                av[t] = xs[(16 * t + lr) * XSTR + 4 * lg + q];
                tsm[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[t], ones, tsm[t], 0, 0, 0);
            }
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t w = q == 0 ? wb[st][r].x : q == 1 ? wb[st][r].y : q == 2 ? wb[st][r].z : wb[st][r].w;
                const i32x4 bv = {(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u),
                                  (int)((w >> 4) & 0x03030303u), (int)((w >> 6) & 0x03030303u)};
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[r][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[t], bv, acc[r][t], 0, 0, 0);
            }
        }
    };
    if (s0 < s1) {
        const int last = s1 - 1;
#pragma unroll
        for (int j = 0; j < ST - 1; ++j) load(j, min(s0 + j, last));
        for (int s = s0; s < s1; s += ST) {
#pragma unroll
            for (int j = 0; j < ST; ++j) {
                if (s + j < s1) {
                    __builtin_amdgcn_sched_barrier(0);
                    if (s + j + ST - 1 < s1) load((j + ST - 1) % ST, s + j + ST - 1);
                    __builtin_amdgcn_sched_barrier(0);
                    compute(j);
                }
            }
        }
    }
    // column 0 (lanes 0, 16, 32, 48) holds accumulator r of token 4 (lane / 16) + r
    if (lr == 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) tsum_w[wave][16 * t + 4 * lg + r] = tsm[t][r];
    }
    __syncthreads();                               // every wave is done with its x_q image
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) red[(wave * RB * MT + r * MT + t) * 64 + lane] = acc[r][t];
    __syncthreads();
    if (tid < MT * 16) {
        int v = 0;
#pragma unroll
        for (int w = 0; w < BD_WAVES; ++w) v += tsum_w[w][tid];
        tsum_t[tid] = v;
        scale_t[tid] = (!a.alpha_per_row && tid < M) ? dequant_scale(a.alpha[0], a.beta[tid]) : 0.0f;
    }
    __syncthreads();
    for (int e = tid; e < RB * MT * 64; e += BD_WAVES * 64) {
        const int l = e & 63, tile = e >> 6;
        const int r = tile / MT, t = tile % MT;
        i32x4 sum = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < BD_WAVES; ++w) sum += red[(w * RB * MT + tile) * 64 + l];
        const int64_t n = n0 + 16 * r + (l & 15);
        if (n >= N) continue;
        const float al = a.alpha_per_row ? a.alpha[n] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 16 * t + 4 * (l >> 4) + i;
            if (m >= M) continue;
            const int total = sum[i] - tsum_t[m];
            const float sc = a.alpha_per_row ? dequant_scale(al, a.beta[m]) : scale_t[m];
            a.y[(int64_t)m * N + n] = activate(dequant(total, sc, a.bias, n), a.act);
            if (a.acc) a.acc[(int64_t)m * N + n] = total;
        }
    }
}
template <int MT, int RB, int ST>
static hipError_t launch_bdec16w(const ForwardArgs& a, hipStream_t s) {
    const int64_t blocks = (a.N + 16 * RB - 1) / (16 * RB);
    const size_t tiles = (size_t)BD_WAVES * RB * MT * 64 * sizeof(i32x4);
    const size_t stage = (size_t)BD_WAVES * MT * 16 * 17 * sizeof(i32x4);
    const size_t lds = tiles > stage ? tiles : stage;
    return launch_with_lds(k_bdec16w<MT, RB, ST>, dim3((unsigned)blocks), dim3(BD_WAVES * 64), lds, s, a);
}


// 2 to 64 tokens, K % 256 == 0: 16 x 16 x 64 tiles with the codes expanded in weight order, so
// that x_q needs no transposition, as signed bytes W_hat = c - 1, so that no sum of x_q is
// needed.  Both operands move from global memory into LDS through the load unit itself
// (buffer_load_dwordx4 ... lds), without passing through registers: the waves take the
// 256-weight sub-steps in turn (wave w: w, w + 8, ...), and each wave keeps an LDS image of its
// sub-step (x_q of 4 XG tokens x 256 bytes, then RB x 1 KiB of packed weights).  A sub-step
// reads its image into registers, starts the fetch of the wave's next sub-step into the same
// image, and multiplies while that fetch is in flight.  No load in the loop writes a register,
// so the only waits on memory are the explicit ones below.  A second grid dimension, when
// there is one, splits the tokens into slices of 16 MT.
//   * x_q layout: token T's 16-byte unit u sits at position u ^ (T % 16) of the token's 256
//     bytes.  A load instruction covers four tokens, sixteen lanes each; a lane quad reads one
//     aligned 64-byte piece of a token's row (the XOR permutes units inside and between such
//     pieces), and the sixteen lanes of an A read (16 tokens, one unit each) hit sixteen
//     different bank groups.
//   * weights: lane (r, g) = (l % 16, l / 16) of load instruction b reads 16 bytes (64 codes at
//     k0 + 64 g) of row n0 + 16 b + r and reads them back from its own slot.
//   * in MFMA q of a sub-step, lane group g holds weights 64g + 16q .. 64g + 16q + 15: packed
//     dword q of the lane's 16 bytes, and unit 4g + q of the token's x_q.
//   * signed codes cost four VALU instructions per 16 codes; the unsigned codes with token sums
//     from MFMAs against an all-ones operand cost one MFMA per token tile and 64 weights, half
//     of all MFMAs with one row block per workgroup.
// XG: groups of four tokens whose x_q is loaded (4 MT, or fewer for a single tile of fewer than
// 16 tokens; the operand rows of tokens past them read zeros).
template <int MT, int RB, int XG = 4 * MT>
__global__ __launch_bounds__(BD_WAVES * 64) void k_bdec16n(ForwardArgs a) {
    extern __shared__ i32x4 red[];
    __shared__ __align__(16) float scale_t[MT * 16];
    constexpr int XI = XG;                         // x_q load instructions (1 KiB each) per sub-step
    constexpr int IMG = (XI + RB) * 64;            // 16-byte units of one wave's image
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // a second grid dimension splits the tokens: workgroup row y takes tokens 16 MT y onwards
    if (gridDim.y > 1) {
        const int64_t m0 = (int64_t)blockIdx.y * (16 * MT);
        a.xq += m0 * a.K;
        a.beta += m0;
        a.y += m0 * a.N;
        if (a.acc) a.acc += m0 * a.N;
        a.M = a.M - m0 < 16 * MT ? a.M - m0 : 16 * MT;
    }
    const int M = (int)a.M;
    const int64_t K = a.K, N = a.N, rowb = K >> 2;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * RB);
    const int lr = lane & 15, lg = lane >> 4;
    // sub-steps of 256 weights, interleaved over the waves (wave w takes w, w + 8, ...): at any
    // time the eight waves of a workgroup fetch 512 contiguous bytes of each of its weight rows
    const int SP = (int)(K >> 8);
    i32x4* xs = red + wave * IMG;
    i32x4* ws = xs + XI * 64;
    // instruction i, lane (lr, lg): token 4i + lg (rows past M read row M - 1, never written),
    // position lr, unit lr ^ ((4i + lg) % 16) = lr ^ (4 (i % 4) + lg).  Byte offsets from the
    // sub-step's start fit 32 bits (M K < 2^31 and N K / 4 < 2^32, checked on launch), so every
    // load is a uniform base plus one 32-bit lane offset.
    const uint32_t Ku = (uint32_t)K, lastx = (uint32_t)(M - 1) * Ku, lgK = (uint32_t)lg * Ku;
    uint32_t xu[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xu[j] = 16u * (uint32_t)(lr ^ (4 * j + lg));
    uint32_t xoff[XI];
#pragma unroll
    for (int i = 0; i < XI; ++i) xoff[i] = min(lgK + (uint32_t)(4 * i) * Ku, lastx) + xu[i & 3];
    uint32_t woff[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) woff[r] = (uint32_t)min(n0 + 16 * r + lr, N - 1) * (uint32_t)rowb + 16u * (uint32_t)lg;
    const __amdgpu_buffer_rsrc_t xr = raw_buffer(a.xq, (uint32_t)(M * K));
    const __amdgpu_buffer_rsrc_t wr = raw_buffer(a.wp, (uint32_t)(N * rowb));
    auto fetch = [&](int s) {
#pragma unroll
        for (int i = 0; i < XI; ++i) load_lds16(xr, xoff[i], (uint32_t)s * 256u, xs + 64 * i);
#pragma unroll
        for (int r = 0; r < RB; ++r) load_lds16(wr, woff[r], (uint32_t)s * 64u, ws + 64 * r);
    };
    i32x4 acc[RB][MT];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = i32x4{0, 0, 0, 0};
    if (wave < SP) fetch(wave);
    for (int s = wave; s < SP; s += BD_WAVES) {
        // the fetch of this sub-step has landed in the image (the only loads in flight)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        i32x4 av[MT][4];
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool loaded = XG == 4 * MT || 16 * t + lr < 4 * XG;
                const i32x4 v = xs[(loaded ? (16 * t + lr) * 16 : 0) + ((4 * lg + q) ^ lr)];
                av[t][q] = loaded ? v : i32x4{0, 0, 0, 0};
            }
        u32x4 wv[RB];
#pragma unroll
        for (int r = 0; r < RB; ++r) wv[r] = (u32x4)ws[64 * r + lane];
        // the next fetch rewrites the image: every read of it has to be complete first
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        if (s + BD_WAVES < SP) fetch(s + BD_WAVES);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t w = q == 0 ? wv[r].x : q == 1 ? wv[r].y : q == 2 ? wv[r].z : wv[r].w;
                const i32x4 bv = expand_signed_in_order(w);
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[r][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(av[t][q], bv, acc[r][t], 0, 0, 0);
            }
        }
    }
    __syncthreads();                               // every wave is done with its image
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) red[(wave * RB * MT + r * MT + t) * 64 + lane] = acc[r][t];
    __syncthreads();
    if (tid < MT * 16) {
        scale_t[tid] = (!a.alpha_per_row && tid < M) ? dequant_scale(a.alpha[0], a.beta[tid]) : 0.0f;
    }
    __syncthreads();
    // element e = (tile, lane): tokens 16 t + 4 (lane / 16) + i, i < 4, of weight row
    // n0 + 16 r + lane % 16; the four tokens' scales are read as one 16-byte unit
    for (int e = tid; e < RB * MT * 64; e += BD_WAVES * 64) {
        const int l = e & 63, tile = e >> 6;
        const int r = tile / MT, t = tile % MT;
        i32x4 sum = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < BD_WAVES; ++w) sum += red[(w * RB * MT + tile) * 64 + l];
        const int64_t n = n0 + 16 * r + (l & 15);
        if (n >= N) continue;
        const int m0 = 16 * t + 4 * (l >> 4);
        float sc[4];
        if (a.alpha_per_row) {
            const float al = a.alpha[n];
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = m0 + i < M ? dequant_scale(al, a.beta[m0 + i]) : 0.0f;
        } else {
            const float4 s4 = *reinterpret_cast<const float4*>(&scale_t[m0]);
            sc[0] = s4.x; sc[1] = s4.y; sc[2] = s4.z; sc[3] = s4.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (m0 + i >= M) break;
            const int total = sum[i];
            a.y[(int64_t)(m0 + i) * N + n] = activate(dequant(total, sc[i], a.bias, n), a.act);
            if (a.acc) a.acc[(int64_t)(m0 + i) * N + n] = total;
        }
    }
}

template <int MT, int RB, int XG>
static hipError_t launch_bdec16n_xg(const ForwardArgs& a, hipStream_t s) {
    const int64_t blocks = (a.N + 16 * RB - 1) / (16 * RB);
    const size_t tiles = (size_t)BD_WAVES * RB * MT * 64 * sizeof(i32x4);
    const size_t image = (size_t)BD_WAVES * (XG + RB) * 64 * sizeof(i32x4);
    return launch_with_lds(k_bdec16n<MT, RB, XG>, dim3((unsigned)blocks), dim3(BD_WAVES * 64), tiles > image ? tiles : image, s, a);
}
// One tile of fewer than 16 tokens loads only the x_q of its groups of four tokens (same outputs;
// M = 3, K = 16384, N = 4096: 8.4 against 8.8 us; M = 8, K = N = 8192: 7.3 against 7.6 us;
// M = 4, K = 11008, N = 4096: 6.8 against 7.0 us).
template <int MT, int RB>
static hipError_t launch_bdec16n(const ForwardArgs& a, hipStream_t s) {
    if constexpr (MT == 1) {
        if (a.M <= 4) return launch_bdec16n_xg<1, RB, 1>(a, s);
        if (a.M <= 8) return launch_bdec16n_xg<1, RB, 2>(a, s);
        if (a.M <= 12) return launch_bdec16n_xg<1, RB, 3>(a, s);
    }
    return launch_bdec16n_xg<MT, RB, 4 * MT>(a, s);
}
// Two halves of the tokens in one launch (a second grid dimension), MT 16-token tiles each, every
// workgroup reading its half of x_q: RB row blocks per workgroup.
template <int MT, int RB>
static hipError_t launch_bdec16n_halves(const ForwardArgs& a, hipStream_t s) {
    const int64_t blocks = (a.N + 16 * RB - 1) / (16 * RB);
    const size_t tiles = (size_t)BD_WAVES * RB * MT * 64 * sizeof(i32x4);
    const size_t image = (size_t)BD_WAVES * (4 * MT + RB) * 64 * sizeof(i32x4);
    return launch_with_lds(k_bdec16n<MT, RB>, dim3((unsigned)blocks, (unsigned)((a.M + 16 * MT - 1) / (16 * MT))),
                           dim3(BD_WAVES * 64), tiles > image ? tiles : image, s, a);
}
// (at most 256 16-row blocks: one or two per workgroup keep the grid within 256 workgroups)
template <int MT>
static hipError_t launch_bdec16n_halves_fill(const ForwardArgs& a, hipStream_t s) {
    const int64_t nb16 = (a.N + 15) / 16;
    return nb16 <= 128 ? launch_bdec16n_halves<MT, 1>(a, s) : launch_bdec16n_halves<MT, 2>(a, s);
}

// Row blocks per workgroup: the fewest (up to three, the most whose images fit the LDS beside
// four 16-token tiles) that keep the grid within 256 workgroups.
template <int MT>
static hipError_t launch_bdec16n_fill(const ForwardArgs& a, hipStream_t s) {
    const int64_t nb16 = (a.N + 15) / 16;
    if (nb16 <= 256) return launch_bdec16n<MT, 1>(a, s);
    if (nb16 <= 512) return launch_bdec16n<MT, 2>(a, s);
    return launch_bdec16n<MT, 3>(a, s);
}

// 33 to 64 tokens with K % 128 == 0: the scheme of k_bdec without its K-tail selects (every
// sub-step is whole), with plain (cached) weight loads.  A wave's 128-weight sub-steps read
// 32 bytes of each of its rows' 128-byte lines in turn; streamed past the caches, every
// sub-step fetched its line again, cached they hit in L2.  Both changes were measured with
// weights not in cache, M = 64: 12.8 against 18.5 us at K = 4096, N = 11008 (two row blocks per
// workgroup), 18.3 against 22.2 us at K = 11008, N = 4096 (one row block).  The token sums of
// x_q come from MFMAs against an all-ones operand (12.9 -> 12.6 us at K = 4096, N = 11008).
// The kernel stays bound by its VALU work (the 4x4 transposes of x_q, the weight expansion).
template <int RB>
__global__ __launch_bounds__(BD_WAVES * 64) void k_bdec64(ForwardArgs a) {
    constexpr int MT = 2;
    extern __shared__ i32x4 red[];
    __shared__ int tsum_w[BD_WAVES][MT * 32];
    __shared__ int tsum_t[MT * 32];
    __shared__ float scale_t[MT * 32];
    constexpr int XU = 9;
    constexpr int XR = MT * 32 * XU;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = (int)a.M;
    const int64_t K = a.K, N = a.N, rowb = K >> 2;
    const int64_t n0 = (int64_t)blockIdx.x * (32 * RB);
    const int lr = lane & 31, lg = lane >> 5;
    i32x4* xs = red + wave * XR;
    const int SP = (int)(K >> 7);
    // the wave's i-th sub-step is wave + 8 i (interleaved over the waves)
    const int s0 = 0, s1 = wave < SP ? (SP - wave + BD_WAVES - 1) / BD_WAVES : 0;
    // x_q: instruction i covers tokens 8i + lane/8, 16 bytes at k0 + 16 (lane % 8); weights:
    // lane (lr, lg) reads 16 bytes (64 codes at k0 + 64 lg) of row n0 + 32r + lr.  Rows past M
    // or N are clamped (never written).
    const int xu = lane & 7, xt = lane >> 3;
    const int8_t* xrow[MT * 4];
#pragma unroll
    for (int i = 0; i < MT * 4; ++i) xrow[i] = a.xq + (int64_t)min(8 * i + xt, M - 1) * K + 16 * xu;
    const uint8_t* wrow[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) wrow[r] = a.wp + min(n0 + 32 * r + lr, N - 1) * rowb + 16 * lg;
    u32x4 xa[2][MT * 4], wb[2][RB];
    auto load = [&](int st, int s) {
#pragma unroll
        for (int i = 0; i < MT * 4; ++i) xa[st][i] = *reinterpret_cast<const u32x4*>(xrow[i] + (int64_t)(wave + BD_WAVES * s) * 128);
#pragma unroll
        for (int r = 0; r < RB; ++r) wb[st][r] = *reinterpret_cast<const u32x4*>(wrow[r] + (int64_t)(wave + BD_WAVES * s) * 32);
    };
    i32x16 acc[RB][MT];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = i32x16{};
    // token sums of x_q from the matrix cores: A times an all-ones B gives, in every column,
    // each token row's sum over the sub-step's k (the matrix cores are mostly idle here; the
    // four v_dot4 per 16 bytes of x_q they replace are not)
    const i32x4 ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    i32x16 tsm[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) tsm[t] = i32x16{};
    auto compute = [&](int st) {
#pragma unroll
        for (int i = 0; i < MT * 4; ++i) {
            const u32x4 v = xa[st][i];
            xs[(8 * i + xt) * XU + xu] = (i32x4)transpose4x4_perm(v);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            i32x4 av[MT];
#pragma unroll
            for (int t = 0; t < MT; ++t) av[t] = xs[(32 * t + lr) * XU + 4 * lg + q];
#pragma unroll
            for (int t = 0; t < MT; ++t) tsm[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[t], ones, tsm[t], 0, 0, 0);
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const uint32_t w = q == 0 ? wb[st][r].x : q == 1 ? wb[st][r].y : q == 2 ? wb[st][r].z : wb[st][r].w;
                const i32x4 bv = {(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u),
                                  (int)((w >> 4) & 0x03030303u), (int)((w >> 6) & 0x03030303u)};
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[r][t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av[t], bv, acc[r][t], 0, 0, 0);
            }
        }
    };
    // two register stages; loads past the wave's range are skipped (re-reading the last
    // sub-step there measured 0.1-0.5 us slower)
    if (s0 < s1) {
        load(0, s0);
        for (int s = s0; s < s1; s += 2) {
            __builtin_amdgcn_sched_barrier(0);
            if (s + 1 < s1) load(1, s + 1);
            __builtin_amdgcn_sched_barrier(0);
            compute(0);
            if (s + 1 < s1) {
                __builtin_amdgcn_sched_barrier(0);
                if (s + 2 < s1) load(0, s + 2);
                __builtin_amdgcn_sched_barrier(0);
                compute(1);
            }
        }
    }
    // column 0 (lanes 0 and 32) holds accumulator r of token 8 (r / 4) + 4 (lane / 32) + r % 4
    if (lr == 0) {
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) tsum_w[wave][32 * t + 8 * (r / 4) + 4 * lg + r % 4] = tsm[t][r];
    }
    __syncthreads();                               // every wave is done with its staging region
    if (tid < MT * 32) {
        int v = 0;
#pragma unroll
        for (int w = 0; w < BD_WAVES; ++w) v += tsum_w[w][tid];
        tsum_t[tid] = v;
        scale_t[tid] = (!a.alpha_per_row && tid < M) ? dequant_scale(a.alpha[0], a.beta[tid]) : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                red[((wave * RB * MT + r * MT + t) * 4 + c) * 64 + lane] =
                    i32x4{acc[r][t][4 * c], acc[r][t][4 * c + 1], acc[r][t][4 * c + 2], acc[r][t][4 * c + 3]};
    __syncthreads();
    for (int e = tid; e < RB * MT * 4 * 64; e += BD_WAVES * 64) {
        const int l = e & 63, c = (e >> 6) & 3, tile = e >> 8;
        const int r = tile / MT, t = tile % MT;
        i32x4 sum = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < BD_WAVES; ++w) sum += red[((w * RB * MT + tile) * 4 + c) * 64 + l];
        const int64_t n = n0 + 32 * r + (l & 31);
        if (n >= N) continue;
        const float al = a.alpha_per_row ? a.alpha[n] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 32 * t + 8 * c + 4 * (l >> 5) + i;
            if (m >= M) continue;
            const int total = sum[i] - tsum_t[m];
            const float sc = a.alpha_per_row ? dequant_scale(al, a.beta[m]) : scale_t[m];
            a.y[(int64_t)m * N + n] = activate(dequant(total, sc, a.bias, n), a.act);
            if (a.acc) a.acc[(int64_t)m * N + n] = total;
        }
    }
}

template <int RB>
static hipError_t launch_bdec64(const ForwardArgs& a, hipStream_t s) {
    const int64_t blocks = (a.N + 32 * RB - 1) / (32 * RB);
    const size_t stage = (size_t)BD_WAVES * 2 * 32 * 9 * sizeof(i32x4);
    const size_t tiles = (size_t)BD_WAVES * RB * 2 * 4 * 64 * sizeof(i32x4);
    return launch_with_lds(k_bdec64<RB>, dim3((unsigned)blocks), dim3(BD_WAVES * 64), stage > tiles ? stage : tiles, s, a);
}

bool decode_mfma_supports(int64_t M, int64_t K) { return M >= 1 && M <= 64 && K % 64 == 0; }

// Tile shape by token count: 16 x 16 x 64 tiles up to 32 tokens (better weight loads, fewer
// token rows of x_q; with K % 256 != 0, 17 to 32 tokens on wide matrices of K <= 8192 take
// 32 x 32 x 32 tiles), 32 x 32 x 32 tiles up to 64.  Row blocks per workgroup: the fewest that
// keep the grid within about one workgroup per CU (256), so that x_q is read as few times as
// possible, within the registers (no spills) and the LDS of the final reduction.
template <int MT>
static hipError_t launch_bdec16w_fill(const ForwardArgs& a, hipStream_t s) {
    const int64_t nb16 = (a.N + 15) / 16;
    switch ((nb16 + 255) / 256) {
        case 1: return launch_bdec16w<MT, 1, 2>(a, s);
        case 2: return launch_bdec16w<MT, 2, 2>(a, s);
        case 3: return launch_bdec16w<MT, 3, 2>(a, s);
        case 4: return launch_bdec16w<MT, 4, 2>(a, s);
        case 5: return launch_bdec16w<MT, 5, 2>(a, s);
        case 6: return launch_bdec16w<MT, 6, 2>(a, s);
        case 7: return launch_bdec16w<MT, 7, 2>(a, s);
        default:
            // more than 256 workgroups from N > 32768; two 16-token tiles keep seven row blocks,
            // where eight spill registers
            if constexpr (MT == 2) return launch_bdec16w<MT, 7, 2>(a, s);
            else return launch_bdec16w<MT, 8, 2>(a, s);
    }
}


hipError_t launch_decode_mfma(const ForwardArgs& a, hipStream_t s) {
    const int64_t nb16 = (a.N + 15) / 16;
    // 2 to 16 tokens likewise, on one 16-token tile.  Against k_bdec16w, identical outputs, weights
    // not in cache: M = 16, K = 8192, N = 8192: 7.8 against 9.4 us; K = 11008, N = 4096: 7.6
    // against 8.3 us; K = 4096, N = 11008: 6.6 against 7.0 us; M = 8, K = 11008, N = 4096: 6.9
    // against 7.4 us; M = 4: 6.5 against 6.5 us at K = 4096, N = 11008, 7.1 against 7.6 us at
    // K = 11008, N = 4096.  One row block per workgroup (up to three workgroups per CU: 78 VGPRs,
    // 40 KiB of LDS) was slower on the wide matrices (M = 16, K = 4096, N = 11008: 7.3 us).
    if (a.M >= 2 && a.M <= 16 && a.K % 256 == 0 && a.N * (a.K / 4) < (int64_t(1) << 32) && nb16 <= 768)
        return launch_bdec16n_fill<1>(a, s);
    // Sub-steps interleaved over the waves rather than a contiguous range per wave, same
    // outputs, weights not in cache: M = 4, K = 4096, N = 11008: 5.9 against 6.6 us; M = 16:
    // 6.5 against 6.7 us (K = 11008, N = 4096: 7.3 against 7.7 us); M = 32: 7.7 against 8.0 us;
    // M = 64 level.  Two and three tokens then left k_bdec16w too (M = 2 / 3, K = 4096,
    // N = 11008: 5.8 / 5.9 against 6.2 / 6.3 us; M = 3, K = 11008, N = 4096: 6.9 against 7.5).
    // 17 to 64 tokens, whole 256-weight sub-steps, at most 768 16-row blocks: k_bdec16n.
    // Measured with weights not in cache, against the kernels these shapes took before
    // (k_bdec16w), identical outputs: M = 64, K = 4096, N = 11008: 10.8 against 11.7 us;
    // K = 11008, N = 4096: 14.6 against 17.3 us; K = 8192, N = 8192: 13.4 against 16.4 us;
    // K = 16384, N = 4096: 18.4 against 22.9 us; M = 48, K = 4096, N = 11008: 9.7 against
    // 10.7 us; M = 32: 8.0 against 8.4 us (K = 11008, N = 4096: 10.2 against 11.6 us); M = 17:
    // 7.5 against 7.8 us.
    if (a.M > 16 && a.M <= 64 && a.K % 256 == 0 && a.M * a.K < (int64_t(1) << 31) &&
        a.N * (a.K / 4) < (int64_t(1) << 32) && nb16 <= 768) {
        // 17 to 32 tokens on at most 256 16-row blocks likewise in two 16-token halves (M = 32,
        // K = 11008, N = 4096: 8.6 against 9.8 us; M = 24: 7.6 against 8.9 us; M = 32, K = 4096,
        // N = 4096: 5.3 against 5.8 us)
        if (a.M <= 32) return nb16 <= 256 ? launch_bdec16n_halves_fill<1>(a, s) : launch_bdec16n_fill<2>(a, s);
        // 33 to 64 tokens on at most 256 16-row blocks: two 32-token halves, each workgroup
        // reading half of x_q for twice the rows (measured with weights not in cache, same
        // outputs: M = 64, K = 11008, N = 4096: 10.9 against 14.3 us; K = 16384: 14.8 against
        // 18.8 us; K = 4096: 6.4 against 8.2 us; M = 48, K = 11008: 9.8 against 12.1 us).  Wider
        // matrices keep all tokens in a workgroup (M = 64, K = 4096, N = 11008: 10.9 against
        // 11.6 us in halves; M = 48: 9.5 against 11.1 us; K = N = 8192: M = 64 13.8 against
        // 13.1 us, M = 40 11.2 against 11.7 us).
        if (nb16 <= 256) return launch_bdec16n_halves_fill<2>(a, s);
        if (a.M <= 48) return launch_bdec16n_fill<3>(a, s);
        return launch_bdec16n_fill<4>(a, s);
    }
    // up to 32 tokens with whole 256-weight sub-steps (17 to 32 on wider matrices only): 16 x 16
    // x 64 tiles, the grid filled
    if (a.M <= 32 && a.K % 256 == 0) return a.M <= 16 ? launch_bdec16w_fill<1>(a, s) : launch_bdec16w_fill<2>(a, s);
    if (a.M <= 16) {
        if (nb16 <= 256) return launch_bdec16<1, 1>(a, s);
        if (nb16 <= 512) return launch_bdec16<1, 2>(a, s);
        if (nb16 <= 1024) return launch_bdec16<1, 4>(a, s);
        return launch_bdec16<1, 8>(a, s);
    }
    const int64_t nb = (a.N + 31) / 32;
    // K % 256 != 0: 17 to 32 tokens on wide matrices of moderate K on 32x32x32 tiles with one
    // 32-token block (measured with weights not in cache, M = 24: 19.8 vs 28.0 us at K = 8192,
    // N = 10240 for k_bdec16 with its earlier row blocks; 38.9 vs 54.5 us at K = 8192, N = 28672)
    if (a.M > 16 && a.M <= 32 && a.K <= 8192 && a.N >= 8192) {
        if (nb <= 256) return launch_bdec<1, 1>(a, s);
        if (nb <= 512) return launch_bdec<1, 2>(a, s);
        return launch_bdec<1, 4>(a, s);
    }
    if (a.M <= 32) {
        if (nb16 <= 256) return launch_bdec16<2, 1>(a, s);
        return launch_bdec16<2, 2>(a, s);
    }
    // 33 to 64 tokens, whole 128-weight sub-steps: one 32-row block per workgroup up to 256
    // workgroups (N <= 8192), two beyond (172 workgroups at N = 11008).  Measured with weights
    // not in cache, M = 64: K = 8192, N = 8192, one block 15.8 against 18.6 us for two; K = 28672,
    // N = 8192, 42.3 against 49.8 us; K = 11008, N = 4096, 18.3 against 23.9 us; K = 4096,
    // N = 11008, two blocks 12.6 against 17.0 us for one.
    if (a.K % 128 == 0) return nb <= 256 ? launch_bdec64<1>(a, s) : launch_bdec64<2>(a, s);
    if (nb <= 256) return launch_bdec<2, 1>(a, s);
    return launch_bdec<2, 2>(a, s);
}

}  // namespace bitlinear
