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


bool decode_mfma_supports(int64_t M, int64_t K) { return M >= 1 && M <= 64 && K % 64 == 0; }

// Tile shape by token count: 16 x 16 x 64 tiles up to 32 tokens (better weight loads, fewer
// token rows of x_q) except 17 to 32 tokens on wide matrices of K <= 8192, 32 x 32 x 32 tiles
// up to 64.  Row blocks per workgroup: the fewest that
// keep the grid within about one workgroup per CU (256), so that x_q is read as few times as
// possible, within the registers (no spills) and the LDS of the final reduction.
hipError_t launch_decode_mfma(const ForwardArgs& a, hipStream_t s) {
    const int64_t nb16 = (a.N + 15) / 16;
    if (a.M <= 16) {
        if (nb16 <= 256) return launch_bdec16<1, 1>(a, s);
        if (nb16 <= 512) return launch_bdec16<1, 2>(a, s);
        if (nb16 <= 1024) return launch_bdec16<1, 4>(a, s);
        return launch_bdec16<1, 8>(a, s);
    }
    const int64_t nb = (a.N + 31) / 32;
    // 17 to 32 tokens on wide matrices of moderate K: 32x32x32 tiles with one 32-token block
    // (measured with weights not in cache, M = 24: 19.8 vs 28.0 us at K = 8192, N = 10240;
    // 38.9 vs 54.5 us at K = 8192, N = 28672; level at K = 4096, N = 11008; the 16x16x64
    // tiles stay ahead at K = 11008 and 28672)
    if (a.M > 16 && a.M <= 32 && a.K <= 8192 && a.N >= 8192) {
        if (nb <= 256) return launch_bdec<1, 1>(a, s);
        if (nb <= 512) return launch_bdec<1, 2>(a, s);
        return launch_bdec<1, 4>(a, s);
    }
    if (a.M <= 32) {
        if (nb16 <= 256) return launch_bdec16<2, 1>(a, s);
        return launch_bdec16<2, 2>(a, s);
    }
    if (nb <= 256) return launch_bdec<2, 1>(a, s);
    return launch_bdec<2, 2>(a, s);
}

}  // namespace bitlinear
