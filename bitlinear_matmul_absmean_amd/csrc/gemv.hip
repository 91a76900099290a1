// gemv.hip -- decode-regime ternary x int8 GEMV (M <= 4 tokens) on the VALU, for gfx950.
//
// What is computed ([P2] nxmr.cn "1.58 位大模型" §3.3; [P3] chenxutan.com "1.58-bit 大模型极限量化实战"
// §2.4-§2.5, §3.2): acc[m,n] = sum_{W=+1} x_q[m,k] - sum_{W=-1} x_q[m,k], then
// y = fp32(acc) * fp32(alpha*beta[m]/127) (+ bias).
//
// How: the weight stream is the only large operand, so each wave streams whole packed
// rows with 16-byte loads (one wave load = 1 KiB of one row = 4096 weights) and keeps
// several rows in flight.  A 16-byte load holds 64 codes c = W+1 in {0,1,2}; the four
// masks (v >> 2i) & 0x03030303 turn each dword into four dwords of byte codes, and
// v_dot4_i32_i8 adds c*x_q four weights at a time.  Because c - 1 = W, the per-row sum is
// acc = sum c*x_q - sum x_q: a +1 weight adds x_q once, a 0 weight adds nothing and a -1
// weight subtracts it -- the add/sub with zero skipping of the pages, four lanes of bytes
// per instruction.  sum x_q is one per-token constant computed while staging x_q.
//
// x_q is staged once per workgroup in LDS, pre-transposed so that byte j of mask dword i
// meets x_q[k] with k = 4j + i inside each 16-weight group, and laid out so that the 64
// lanes of a wave read 1 KiB of consecutive LDS per ds_read_b128 (no bank conflicts).
#include "common.hpp"

namespace bitlinear {

template <int MT, int R>
__global__ __launch_bounds__(256) void k_gemv_dot4(ForwardArgs a, int C, int CPL) {
    extern __shared__ u32x4 xs[];          // [MT][CPL][4][64] units of 16 bytes
    __shared__ int tsum[4][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t K = a.K, N = a.N, rowb = K >> 2;

    // ---- stage x_q (transposed per 16-byte group) and per-token sum of x_q ----------
    int part[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) part[t] = 0;
    const int units = MT * CPL * 256;
    for (int u = tid; u < units; u += 256) {
        const int l = u & 63, q = (u >> 6) & 3, jt = u >> 8;
        const int j = jt % CPL, t = jt / CPL;
        const int c = l + 64 * j;
        u32x4 o = {0u, 0u, 0u, 0u};
        if (c < C) {
            const u32x4 s = *reinterpret_cast<const u32x4*>(a.xq + t * K + 64 * c + 16 * q);
            o = transpose4x4_bytes(s);
            int bs = byte_sum(s.x) + byte_sum(s.y) + byte_sum(s.z) + byte_sum(s.w);
#pragma unroll
            for (int tt = 0; tt < MT; ++tt)
                if (tt == t) part[tt] += bs;
        }
        xs[u] = o;
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        int v = wave_sum_i32(part[t]);
        if (lane == 0) tsum[wave][t] = v;
    }
    __syncthreads();
    int xsum[MT];
    float sc[MT];
    const float alpha0 = a.alpha_per_row ? 0.0f : a.alpha[0];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        xsum[t] = tsum[0][t] + tsum[1][t] + tsum[2][t] + tsum[3][t];
        sc[t] = dequant_scale(alpha0, a.beta[t]);
    }

    // ---- stream rows: wave gw owns row groups gw*R, (gw + TW)*R, ... -------------------
    const int64_t TW = (int64_t)gridDim.x * 4;
    for (int64_t row0 = ((int64_t)blockIdx.x * 4 + wave) * R; row0 < N; row0 += TW * R) {
        int acc[R][MT];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[r][t] = 0;

        u32x4 cur[R], nxt[R];
        auto load = [&](u32x4 (&dst)[R], int j) {
            const int c = lane + 64 * j;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int64_t row = row0 + r;
                if (c < C && row < N)
                    dst[r] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4*>(a.wp + row * rowb + 16 * (int64_t)c));
                else
                    dst[r] = u32x4{0u, 0u, 0u, 0u};
            }
        };
        load(cur, 0);
        for (int j = 0; j < CPL; ++j) {
            if (j + 1 < CPL) load(nxt, j + 1);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4 X[MT];
#pragma unroll
                for (int t = 0; t < MT; ++t) X[t] = xs[((t * CPL + j) * 4 + q) * 64 + lane];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t v = q == 0 ? cur[r].x : q == 1 ? cur[r].y : q == 2 ? cur[r].z : cur[r].w;
                    const uint32_t d0 = v & 0x03030303u;
                    const uint32_t d1 = (v >> 2) & 0x03030303u;
                    const uint32_t d2 = (v >> 4) & 0x03030303u;
                    const uint32_t d3 = (v >> 6) & 0x03030303u;
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        int s = acc[r][t];
                        s = dot4(d0, X[t].x, s);
                        s = dot4(d1, X[t].y, s);
                        s = dot4(d2, X[t].z, s);
                        s = dot4(d3, X[t].w, s);
                        acc[r][t] = s;
                    }
                }
            }
            if (j + 1 < CPL) {
#pragma unroll
                for (int r = 0; r < R; ++r) cur[r] = nxt[r];
            }
        }

        // ---- reduce over the wave; lane r*MT + t finishes (row0 + r, token t) --------
        int mine = 0, my_xsum = 0;
        float my_sc = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                int v = wave_sum_i32(acc[r][t]);
                if (lane == r * MT + t) {
                    mine = v;
                    my_xsum = xsum[t];
                    my_sc = sc[t];
                }
            }
        if (lane < R * MT) {
            const int r = lane / MT, t = lane % MT;
            const int64_t n = row0 + r;
            if (n < N) {
                const int total = mine - my_xsum;
                const float s = a.alpha_per_row ? dequant_scale(a.alpha[n], a.beta[t]) : my_sc;
                a.y[t * N + n] = dequant(total, s, a.bias, n);
                if (a.acc) a.acc[t * N + n] = total;
            }
        }
    }
}

template <int MT>
static hipError_t launch_mt(const ForwardArgs& a, hipStream_t s) {
    const int C = (int)(a.K / 64);
    const int CPL = (C + 63) / 64;
    // rows per wave per pass: enough waves to cover the chip, at most 16 loads in flight
    int64_t want = a.N / 2048;
    int R = want >= 8 ? 8 : want >= 4 ? 4 : want >= 2 ? 2 : 1;
    while (R > 1 && R * CPL > 16) R >>= 1;
    const int64_t groups = (a.N + R - 1) / R;
    const int64_t blocks = (groups + 3) / 4;
    const size_t lds = (size_t)MT * CPL * 256 * 16;
    dim3 g((unsigned)blocks), b(256);
    switch (R) {
        case 8: return launch_with_lds(k_gemv_dot4<MT, 8>, g, b, lds, s, a, C, CPL);
        case 4: return launch_with_lds(k_gemv_dot4<MT, 4>, g, b, lds, s, a, C, CPL);
        case 2: return launch_with_lds(k_gemv_dot4<MT, 2>, g, b, lds, s, a, C, CPL);
        default: return launch_with_lds(k_gemv_dot4<MT, 1>, g, b, lds, s, a, C, CPL);
    }
}

hipError_t launch_gemv_dot4(const ForwardArgs& a, hipStream_t s) {
    switch (a.M) {
        case 1: return launch_mt<1>(a, s);
        case 2: return launch_mt<2>(a, s);
        case 3: return launch_mt<3>(a, s);
        default: return launch_mt<4>(a, s);
    }
}

}  // namespace bitlinear
