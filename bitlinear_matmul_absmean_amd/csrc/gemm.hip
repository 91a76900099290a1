// gemm.hip -- prefill-regime ternary x int8 GEMM on the int8 matrix cores
// (v_mfma_i32_32x32x32_i8), gfx950; plus the generic kernel for shapes the fast paths skip.
//
// What is computed ([P3] chenxutan.com "1.58-bit 大模型极限量化实战" §2.4-§2.5, §3.2, §5.5;
// [P2] nxmr.cn "1.58 位大模型" §3.3): acc = x_q . W_hat^T in int32, y = fp32(acc) *
// fp32(alpha*beta[m]/127) (+ bias).  With many tokens (prefill) this is a dense contraction
// and the compute peak is what matters [P3 §5.5], so it runs on MFMA.
//
// Tiles: a workgroup computes 128 tokens x 256 weight rows; its four waves sit side by side in
// N (wave tile 128 x 64: four 32-row A blocks against two 32-column B blocks, 8 accumulators of
// 16 registers).  K advances in steps of 64 with double-buffered LDS, one barrier per step.
//   * A (x_q): 128 x 64 bytes per step from global, every 16-byte group transposed 4x4 with
//     v_perm so that operand byte 4i+j holds x_q[k = 4j+i], written to LDS (rows padded by one
//     16-byte unit against bank conflicts).  The same pass accumulates the per-token sum of x_q.
//   * B (weights): 256 rows x 16 bytes of packed codes per step, to LDS as they are (4x less
//     traffic than int8), dword p of column c stored at p ^ 2((c >> 4) & 1) so that columns c
//     and c + 16 fall in different banks.  The lane feeding column n reads one packed dword (16
//     codes) and expands it with four masks (v >> 2i) & 0x03030303 into its 16-byte operand:
//     byte 4i+j = c of weight 4j+i.  c = W+1, so acc = sum c*x_q - sum x_q.
// Each step first reads every operand it needs from LDS and issues the global loads of the step
// after next (two register stages), then issues its 16 MFMAs one at a time with a slice of VALU
// work (the second half's B expansion, the next step's transposes, sums and LDS stores) after
// each, fixed in place with scheduling barriers: a wave then keeps issuing VALU while its
// previous MFMA occupies the matrix core.  Without the barriers the compiler bunches the VALU
// work and the MFMAs apart.
// The 32x32x32 int8 MFMA does twice the work of the 16x16x64 one in the same issue time on
// gfx950 (measured: 4.9 vs 2.7 POPS over the chip), so the waves tile in 32x32 blocks.  Its
// lane layout (checked on the device): A/B lane l holds row/column l%32, k = 16*(l/32)+j;
// accumulator r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
// Workgroups are mapped so that each XCD (8 on the chip, workgroups dispatched round robin)
// works through a contiguous range of tiles, ordered token block by token block: one XCD's
// L2 keeps its token rows of x_q while the weights stream past.
#include "common.hpp"

namespace bitlinear {

__device__ __forceinline__ u32x4 transpose4x4_v(u32x4 s) {
    const uint32_t a01l = __builtin_amdgcn_perm(s.y, s.x, 0x05010400u);
    const uint32_t a01h = __builtin_amdgcn_perm(s.y, s.x, 0x07030602u);
    const uint32_t a23l = __builtin_amdgcn_perm(s.w, s.z, 0x05010400u);
    const uint32_t a23h = __builtin_amdgcn_perm(s.w, s.z, 0x07030602u);
    u32x4 o;
    o.x = __builtin_amdgcn_perm(a23l, a01l, 0x05040100u);
    o.y = __builtin_amdgcn_perm(a23l, a01l, 0x07060302u);
    o.z = __builtin_amdgcn_perm(a23h, a01h, 0x05040100u);
    o.w = __builtin_amdgcn_perm(a23h, a01h, 0x07060302u);
    return o;
}

__device__ __forceinline__ i32x4 unpack16(uint32_t v) {
    return i32x4{(int)(v & 0x03030303u), (int)((v >> 2) & 0x03030303u), (int)((v >> 4) & 0x03030303u),
                 (int)((v >> 6) & 0x03030303u)};
}
#define SB() __builtin_amdgcn_sched_barrier(0)
#define MF(i, j, av, bv) acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, acc[i][j], 0, 0, 0)

constexpr int GEMM_BM = 128, GEMM_BN = 256, GEMM_BK = 64;
constexpr int64_t GEMM_SMALL_GRID = 192;      // tiles of 128 x 256 up to which 64-token tiles run

// GELU: the BitMLP activation in the epilogue, fixed at compile time so that the plain
// kernel carries no call.  FM: 32-token blocks per tile, 4 (128 x 256 tiles) or 2 (64 x 256,
// for grids that 128-token tiles would leave short of the workgroup slots).
template <bool GELU, int FM>
__global__ __launch_bounds__(256, 2) void k_gemm_mfma(ForwardArgs a, int tiles_m, int tiles_n) {
    static_assert(FM == 4 || FM == 2, "128- or 64-token tiles");
    constexpr int BM = 32 * FM, BN = GEMM_BN, BK = GEMM_BK;
    constexpr int WN = BN / 4;                 // wave tile BM x 64
    constexpr int FN = 2;
    constexpr int GK = BK / 16, APT = BM * GK / 256, ASTR = GK + 1;
    __shared__ u32x4 As[2][BM * ASTR];
    __shared__ u32x4 Bs[2][BN];
    __shared__ int rsum[BM];
    __shared__ float ssc[BM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wn = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t M = a.M, N = a.N, K = a.K, rowb = K >> 2;
    const int T = tiles_m * tiles_n;
    int t = blockIdx.x;
    if (T % 8 == 0) t = (t % 8) * (T / 8) + t / 8;
    const int tm = t / tiles_n, tn = t % tiles_n;
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int KS = (int)(K / BK);
    for (int i = tid; i < BM; i += 256) {
        const int64_t m = m0 + i;
        ssc[i] = (!a.alpha_per_row && m < M) ? dequant_scale(a.alpha[0], a.beta[m]) : 0.0f;
    }

    // Staging: thread tid moves A units u = tid + 256 i (token row u / GK, 16 bytes at k = 16 (u % GK))
    // and the 16 packed bytes of weight row (column) tid.  Rows past M or N are clamped to the last
    // row, so every load is unconditional and the compiler counts outstanding loads exactly
    // (partial vmcnt waits instead of draining); the results of such rows are never written.
    const int8_t* ap[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) {
        const int u = tid + 256 * i;
        ap[i] = a.xq + min(m0 + u / GK, M - 1) * K + 16 * (u % GK);
    }
    const uint8_t* bp = a.wp + min(n0 + tid, N - 1) * rowb;
    const bool bsw = (tid >> 4) & 1;
    u32x4 ra0[APT], ra1[APT], rb0, rb1;
    int rs[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) rs[i] = 0;
    auto gload = [&](u32x4 (&ra)[APT], u32x4& rb, int ks) {
#pragma unroll
        for (int i = 0; i < APT; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ap[i] + (int64_t)ks * BK);
        rb = *reinterpret_cast<const u32x4*>(bp + (int64_t)ks * (BK / 4));
    };
    auto stage_a = [&](const u32x4& r, int i, int buf, bool count) {
        const int u = tid + 256 * i;
        As[buf][(u / GK) * ASTR + u % GK] = transpose4x4_v(r);
        int v = rs[i];
        v = __builtin_amdgcn_sdot4((int)r.x, 0x01010101, v, false);
        v = __builtin_amdgcn_sdot4((int)r.y, 0x01010101, v, false);
        v = __builtin_amdgcn_sdot4((int)r.z, 0x01010101, v, false);
        v = __builtin_amdgcn_sdot4((int)r.w, 0x01010101, v, false);
        rs[i] = count ? v : rs[i];
    };
    auto stage_b = [&](const u32x4& r, int buf) {
        Bs[buf][tid] = bsw ? u32x4{r.z, r.w, r.x, r.y} : r;
    };

    i32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = i32x16{};

    const int lr = lane & 31, lg = lane >> 5;
    int boff[2][FN];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = wn * WN + j * 32 + lr;
            boff[kk][j] = col * 4 + ((2 * kk + lg) ^ (((col >> 4) & 1) << 1));
        }

    // One K step with every piece of non-MFMA work cut into slices of about three VALU
    // instructions, one slice after each MFMA.
    auto step = [&](int buf, const u32x4 (&rc)[APT], const u32x4& rbc, u32x4 (&rn)[APT], u32x4& rbn, int ksl, bool count) {
        uint32_t bw[2][FN];
        i32x4 av[2][FM];
        const uint32_t* b32 = reinterpret_cast<const uint32_t*>(&Bs[buf][0]);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int j = 0; j < FN; ++j) bw[kk][j] = b32[boff[kk][j]];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int i = 0; i < FM; ++i) av[kk][i] = (i32x4)As[buf][(i * 32 + lr) * ASTR + kk * 2 + lg];
        SB();
        gload(rn, rbn, ksl);
        SB();
        i32x4 b0[FN], b1[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) b0[j] = unpack16(bw[0][j]);
        SB();
        const int ob = buf ^ 1;
        uint32_t q[APT][4];
        if constexpr (FM == 4) {
        // first half: B expansion of kk = 1 and the transposes of both A units
        MF(0, 0, av[0][0], b0[0]);
        b1[0].x = (int)(bw[1][0] & 0x03030303u); b1[0].y = (int)((bw[1][0] >> 2) & 0x03030303u); SB();
        MF(0, 1, av[0][0], b0[1]);
        b1[0].z = (int)((bw[1][0] >> 4) & 0x03030303u); b1[0].w = (int)((bw[1][0] >> 6) & 0x03030303u); SB();
        MF(1, 0, av[0][1], b0[0]);
        b1[1].x = (int)(bw[1][1] & 0x03030303u); b1[1].y = (int)((bw[1][1] >> 2) & 0x03030303u); SB();
        MF(1, 1, av[0][1], b0[1]);
        b1[1].z = (int)((bw[1][1] >> 4) & 0x03030303u); b1[1].w = (int)((bw[1][1] >> 6) & 0x03030303u); SB();
        MF(2, 0, av[0][2], b0[0]);
        q[0][0] = __builtin_amdgcn_perm(rc[0].y, rc[0].x, 0x05010400u); q[0][1] = __builtin_amdgcn_perm(rc[0].y, rc[0].x, 0x07030602u);
        q[0][2] = __builtin_amdgcn_perm(rc[0].w, rc[0].z, 0x05010400u); q[0][3] = __builtin_amdgcn_perm(rc[0].w, rc[0].z, 0x07030602u); SB();
        MF(2, 1, av[0][2], b0[1]);
        As[ob][(tid / GK) * ASTR + tid % GK] = u32x4{__builtin_amdgcn_perm(q[0][2], q[0][0], 0x05040100u), __builtin_amdgcn_perm(q[0][2], q[0][0], 0x07060302u),
                                                     __builtin_amdgcn_perm(q[0][3], q[0][1], 0x05040100u), __builtin_amdgcn_perm(q[0][3], q[0][1], 0x07060302u)};
        SB();
        MF(3, 0, av[0][3], b0[0]);
        q[APT - 1][0] = __builtin_amdgcn_perm(rc[APT - 1].y, rc[APT - 1].x, 0x05010400u); q[APT - 1][1] = __builtin_amdgcn_perm(rc[APT - 1].y, rc[APT - 1].x, 0x07030602u);
        q[APT - 1][2] = __builtin_amdgcn_perm(rc[APT - 1].w, rc[APT - 1].z, 0x05010400u); q[APT - 1][3] = __builtin_amdgcn_perm(rc[APT - 1].w, rc[APT - 1].z, 0x07030602u); SB();
        MF(3, 1, av[0][3], b0[1]);
        As[ob][((tid + 256) / GK) * ASTR + tid % GK] = u32x4{__builtin_amdgcn_perm(q[APT - 1][2], q[APT - 1][0], 0x05040100u), __builtin_amdgcn_perm(q[APT - 1][2], q[APT - 1][0], 0x07060302u),
                                                             __builtin_amdgcn_perm(q[APT - 1][3], q[APT - 1][1], 0x05040100u), __builtin_amdgcn_perm(q[APT - 1][3], q[APT - 1][1], 0x07060302u)};
        SB();
        // second half: sums and the B store
        int v0 = rs[0], v1 = rs[APT - 1];
        MF(0, 0, av[1][0], b1[0]);
        v0 = __builtin_amdgcn_sdot4((int)rc[0].x, 0x01010101, v0, false); v0 = __builtin_amdgcn_sdot4((int)rc[0].y, 0x01010101, v0, false); SB();
        MF(0, 1, av[1][0], b1[1]);
        v0 = __builtin_amdgcn_sdot4((int)rc[0].z, 0x01010101, v0, false); v0 = __builtin_amdgcn_sdot4((int)rc[0].w, 0x01010101, v0, false); SB();
        MF(1, 0, av[1][1], b1[0]);
        v1 = __builtin_amdgcn_sdot4((int)rc[APT - 1].x, 0x01010101, v1, false); v1 = __builtin_amdgcn_sdot4((int)rc[APT - 1].y, 0x01010101, v1, false); SB();
        MF(1, 1, av[1][1], b1[1]);
        v1 = __builtin_amdgcn_sdot4((int)rc[APT - 1].z, 0x01010101, v1, false); v1 = __builtin_amdgcn_sdot4((int)rc[APT - 1].w, 0x01010101, v1, false); SB();
        MF(2, 0, av[1][2], b1[0]);
        rs[0] = count ? v0 : rs[0]; rs[APT - 1] = count ? v1 : rs[APT - 1]; SB();
        MF(2, 1, av[1][2], b1[1]);
        stage_b(rbc, ob); SB();
        MF(3, 0, av[1][3], b1[0]); SB();
        MF(3, 1, av[1][3], b1[1]); SB();
        } else {
        // 64-token tiles, one A unit per thread: first half the B expansion of kk = 1, second
        // half the transpose, the sum and the stores
        MF(0, 0, av[0][0], b0[0]);
        b1[0].x = (int)(bw[1][0] & 0x03030303u); b1[0].y = (int)((bw[1][0] >> 2) & 0x03030303u); SB();
        MF(0, 1, av[0][0], b0[1]);
        b1[0].z = (int)((bw[1][0] >> 4) & 0x03030303u); b1[0].w = (int)((bw[1][0] >> 6) & 0x03030303u); SB();
        MF(1, 0, av[0][1], b0[0]);
        b1[1].x = (int)(bw[1][1] & 0x03030303u); b1[1].y = (int)((bw[1][1] >> 2) & 0x03030303u); SB();
        MF(1, 1, av[0][1], b0[1]);
        b1[1].z = (int)((bw[1][1] >> 4) & 0x03030303u); b1[1].w = (int)((bw[1][1] >> 6) & 0x03030303u); SB();
        int v0 = rs[0];
        MF(0, 0, av[1][0], b1[0]);
        q[0][0] = __builtin_amdgcn_perm(rc[0].y, rc[0].x, 0x05010400u); q[0][1] = __builtin_amdgcn_perm(rc[0].y, rc[0].x, 0x07030602u);
        q[0][2] = __builtin_amdgcn_perm(rc[0].w, rc[0].z, 0x05010400u); q[0][3] = __builtin_amdgcn_perm(rc[0].w, rc[0].z, 0x07030602u); SB();
        MF(0, 1, av[1][0], b1[1]);
        As[ob][(tid / GK) * ASTR + tid % GK] = u32x4{__builtin_amdgcn_perm(q[0][2], q[0][0], 0x05040100u), __builtin_amdgcn_perm(q[0][2], q[0][0], 0x07060302u),
                                                     __builtin_amdgcn_perm(q[0][3], q[0][1], 0x05040100u), __builtin_amdgcn_perm(q[0][3], q[0][1], 0x07060302u)};
        SB();
        MF(1, 0, av[1][1], b1[0]);
        v0 = __builtin_amdgcn_sdot4((int)rc[0].x, 0x01010101, v0, false); v0 = __builtin_amdgcn_sdot4((int)rc[0].y, 0x01010101, v0, false);
        v0 = __builtin_amdgcn_sdot4((int)rc[0].z, 0x01010101, v0, false); v0 = __builtin_amdgcn_sdot4((int)rc[0].w, 0x01010101, v0, false); SB();
        MF(1, 1, av[1][1], b1[1]);
        rs[0] = count ? v0 : rs[0];
        stage_b(rbc, ob); SB();
        }
    };

    // Two register stages: at the top of an iteration LDS buffer 0 holds step ks and ra1/rb1 hold
    // step ks+1.  Past the end the loads re-read the last step; `count` keeps those out of the sums.
    const int last = KS - 1;
    gload(ra0, rb0, 0);
    gload(ra1, rb1, KS > 1 ? 1 : 0);
#pragma unroll
    for (int i = 0; i < APT; ++i) stage_a(ra0[i], i, 0, true);
    stage_b(rb0, 0);
    __syncthreads();
    int ks = 0;
    for (; ks + 2 <= KS; ks += 2) {
        step(0, ra1, rb1, ra0, rb0, min(ks + 2, last), ks + 1 < KS);
        __syncthreads();
        step(1, ra0, rb0, ra1, rb1, min(ks + 3, last), ks + 2 < KS);
        __syncthreads();
    }
    if (ks < KS) step(0, ra1, rb1, ra0, rb0, last, false);

#pragma unroll
    for (int i = 0; i < APT; ++i) {
        int v = rs[i];
#pragma unroll
        for (int s = 1; s < GK; s <<= 1) v += __shfl_xor(v, s, 64);
        const int u = tid + 256 * i;
        if (u % GK == 0) rsum[u / GK] = v;
    }
    __syncthreads();
    // Output (i, r, j): token row mr, weight row n; returns false past M or N.
    auto out_at = [&](int i, int r, int j, int64_t& m, int64_t& n, int& mr) {
        mr = i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
        m = m0 + mr;
        n = n0 + wn * WN + j * 32 + lr;
        return m < M && n < N;
    };
    auto value = [&](int i, int r, int j, int64_t m, int64_t n, int mr) {
        const int total = acc[i][j][r] - rsum[mr];
        const float s = a.alpha_per_row ? dequant_scale(a.alpha[n], a.beta[m]) : ssc[mr];
        if (a.acc) a.acc[m * N + n] = total;
        return dequant(total, s, a.bias, n);
    };
    if constexpr (GELU) {
        // Two token rows x two weight rows per call of the four-wide GELU.
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float hv[4];
                int64_t mm[4], nn[4];
                bool in[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    int mr;
                    in[q] = out_at(i, r + q / 2, q % 2, mm[q], nn[q], mr);
                    hv[q] = in[q] ? value(i, r + q / 2, q % 2, mm[q], nn[q], mr) : 0.0f;
                }
                const float4 g = gelu4_f32(make_float4(hv[0], hv[1], hv[2], hv[3]));
                const float gv[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (in[q]) a.y[mm[q] * N + nn[q]] = gv[q];
            }
    } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r)
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    int64_t m, n;
                    int mr;
                    if (out_at(i, r, j, m, n, mr)) a.y[m * N + n] = value(i, r, j, m, n, mr);
                }
    }
}

bool gemm_supports_k(int64_t K) { return K % GEMM_BK == 0; }

template <int FM>
static hipError_t launch_gemm_fm(const ForwardArgs& a, hipStream_t s) {
    const int bm = 32 * FM;
    const int tm = (int)((a.M + bm - 1) / bm), tn = (int)((a.N + GEMM_BN - 1) / GEMM_BN);
    if (a.act == 1)
        hipLaunchKernelGGL((k_gemm_mfma<true, FM>), dim3((unsigned)(tm * tn)), dim3(256), 0, s, a, tm, tn);
    else
        hipLaunchKernelGGL((k_gemm_mfma<false, FM>), dim3((unsigned)(tm * tn)), dim3(256), 0, s, a, tm, tn);
    return hipGetLastError();
}

// 128 x 256 tiles, or 64 x 256 for grids of at most 128 such tiles (a quarter of the 512
// workgroup slots).  Measured: M = 1024, K = N = 4096: 34.3 vs 45.6 us; M = 512: 31.0 vs
// 44.7 us; M = 128, N = 11008: 30.0 vs 43.2 us.  With more tiles the 128-token tiles win or tie
// at long K, since a 64-token tile reads the weights twice as often (M = 2048, K = 11008,
// N = 4096: 100 vs 126 us; K = 4096: 48.9 vs 49.1 us; M = 512, N = 11008, 172 tiles: level),
// but up to 192 tiles, and up to 256 with K <= 2048, the 64-token tiles that fill the slots
// were faster (M = 1536, K = N = 4096: 42.0 vs 46.2 us; M = 2048, K = 2048, N = 4096: 28.8 vs
// 32.2 us).
hipError_t launch_gemm_mfma(const ForwardArgs& a, hipStream_t s) {
    const int64_t tiles128 = ((a.M + GEMM_BM - 1) / GEMM_BM) * ((a.N + GEMM_BN - 1) / GEMM_BN);
    const bool small = tiles128 <= GEMM_SMALL_GRID || (tiles128 <= 256 && a.K <= 2048);
    return small ? launch_gemm_fm<2>(a, s) : launch_gemm_fm<4>(a, s);
}

// ---------------------------------------------------------------------------------------
// Generic path for any K % 4 == 0 and any alignment: one wave per output row n, lanes over
// packed bytes, the add/sub of [P2 §3.3] weight by weight.  Used only for shapes the fast
// kernels do not take; its results are identical.
__global__ __launch_bounds__(256) void k_forward_generic(ForwardArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (n >= a.N) return;
    const int64_t K = a.K, rowb = K >> 2;
    for (int64_t m = 0; m < a.M; ++m) {
        int s = 0;
        for (int64_t b = lane; b < rowb; b += 64) {
            const uint32_t byte = a.wp[n * rowb + b];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t c = (byte >> (2 * i)) & 3u;
                const int x = a.xq[m * K + 4 * b + i];
                s += c == 2u ? x : (c == 0u ? -x : 0);
            }
        }
        s = wave_sum_i32(s);
        if (lane == 0) {
            const float al = a.alpha_per_row ? a.alpha[n] : a.alpha[0];
            a.y[m * a.N + n] = activate(dequant(s, dequant_scale(al, a.beta[m]), a.bias, n), a.act);
            if (a.acc) a.acc[m * a.N + n] = s;
        }
    }
}

hipError_t launch_forward_generic(const ForwardArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_forward_generic, dim3((unsigned)((a.N + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace bitlinear
