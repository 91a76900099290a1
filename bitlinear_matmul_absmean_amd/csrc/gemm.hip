// gemm.hip -- ternary x int8 GEMM on the int8 matrix cores (v_mfma_i32_16x16x64_i8), gfx950.
//
// What is computed ([P3] chenxutan.com "1.58-bit 大模型极限量化实战" §2.4-§2.5, §3.2;
// [P2] nxmr.cn "1.58 位大模型" §3.3): acc = x_q . W_hat^T in int32, y = fp32(acc) *
// fp32(alpha*beta[m]/127) (+ bias).  With many tokens the product is a real dense
// contraction, so it runs on MFMA; the weights stay 2-bit in memory and are expanded to
// byte codes on chip.
//
// Operand preparation per K-step of 64:
//   * B (weights): the packed tile [BN][16 bytes] goes to LDS as is.  A lane that feeds
//     column n of an MFMA reads one packed dword (16 codes) and expands it with four
//     masks (v >> 2i) & 0x03030303 into the 16 byte-codes c = W+1 of its operand.  Byte j
//     of mask dword i is the code of weight k = 4j + i of that 16-weight group.
//   * A (x_q): staged to LDS with each 16-byte group transposed 4x4, so that operand byte
//     4i + j holds x_q[k = 4j + i] -- the same weight order as B.  The MFMA pairs byte b of
//     A with byte b of B in every lane group, so the contraction is over true k.
//   * Since c = W + 1, sum_k x_q c = acc + sum_k x_q; the per-token sum of x_q is
//     accumulated while staging A and subtracted in the epilogue.
#include "common.hpp"

namespace bitlinear {

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(256) void k_gemm_mfma(ForwardArgs a) {
    static_assert(WGM * WGN == 4, "four waves per workgroup");
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int FM = WM / 16, FN = WN / 16;
    static_assert(FM >= 1 && FN >= 1 && BN <= 256, "tile shape");
    constexpr int AU = BM * 4;                      // 16-byte units of the A tile per K-step
    constexpr int APT = (AU + 255) / 256;           // A units per thread

    __shared__ u32x4 As[2][AU];                     // [row][group] (transposed bytes)
    __shared__ u32x4 Bs[2][BN];                     // [col] packed 64 codes
    __shared__ int rsum[BM];
    __shared__ float ssc[BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int64_t M = a.M, N = a.N, K = a.K, rowb = K >> 2;
    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int KS = (int)(K / 64);

    for (int i = tid; i < BM; i += 256) {
        rsum[i] = 0;
        const int64_t m = m0 + i;
        ssc[i] = (!a.alpha_per_row && m < M) ? dequant_scale(a.alpha[0], a.beta[m]) : 0.0f;
    }

    u32x4 ra[APT];
    u32x4 rb = {0u, 0u, 0u, 0u};
    int rs[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) rs[i] = 0;

    auto gload = [&](int ks) {
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int u = tid + 256 * i;
            ra[i] = u32x4{0u, 0u, 0u, 0u};
            if (u < AU) {
                const int64_t m = m0 + (u >> 2);
                if (m < M)
                    ra[i] = *reinterpret_cast<const u32x4*>(a.xq + m * K + (int64_t)ks * 64 + 16 * (u & 3));
            }
        }
        if (tid < BN) {
            const int64_t n = n0 + tid;
            rb = n < N ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.wp + n * rowb + (int64_t)ks * 16))
                       : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int u = tid + 256 * i;
            if (u < AU) {
                As[buf][u] = transpose4x4_bytes(ra[i]);
                rs[i] += byte_sum(ra[i].x) + byte_sum(ra[i].y) + byte_sum(ra[i].z) + byte_sum(ra[i].w);
            }
        }
        if (tid < BN) Bs[buf][tid] = rb;
    };

    i32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = i32x4{0, 0, 0, 0};

    gload(0);
    sstore(0);
    __syncthreads();

    const int lr = lane & 15, lg = lane >> 4;
    for (int ks = 0; ks < KS; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < KS) gload(ks + 1);

        i32x4 bop[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const u32x4 pk = Bs[buf][wn * WN + j * 16 + lr];
            const uint32_t v = lg == 0 ? pk.x : lg == 1 ? pk.y : lg == 2 ? pk.z : pk.w;
            bop[j] = i32x4{(int)(v & 0x03030303u), (int)((v >> 2) & 0x03030303u),
                           (int)((v >> 4) & 0x03030303u), (int)((v >> 6) & 0x03030303u)};
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const i32x4 aop = (i32x4)As[buf][(wm * WM + i * 16 + lr) * 4 + lg];
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop, bop[j], acc[i][j], 0, 0, 0);
        }
        if (ks + 1 < KS) sstore(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < APT; ++i) {
        const int u = tid + 256 * i;
        if (u < AU) atomicAdd(&rsum[u >> 2], rs[i]);
    }
    __syncthreads();

    // 16x16 MFMA result layout: lane l, element r -> row 4*(l/16) + r, column l % 16.
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int mr = wm * WM + i * 16 + 4 * lg + r;
                const int64_t m = m0 + mr, n = n0 + wn * WN + j * 16 + lr;
                if (m < M && n < N) {
                    const int total = acc[i][j][r] - rsum[mr];
                    const float s = a.alpha_per_row ? dequant_scale(a.alpha[n], a.beta[m]) : ssc[mr];
                    a.y[m * N + n] = dequant(total, s, a.bias, n);
                    if (a.acc) a.acc[m * N + n] = total;
                }
            }
}

template <int BM, int BN, int WGM, int WGN>
static hipError_t launch_tile(const ForwardArgs& a, hipStream_t s) {
    dim3 g((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    hipLaunchKernelGGL((k_gemm_mfma<BM, BN, WGM, WGN>), g, dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm_mfma(const ForwardArgs& a, hipStream_t s) {
    if (a.M <= 16) return launch_tile<16, 64, 1, 4>(a, s);
    if (a.M <= 32) return launch_tile<32, 64, 2, 2>(a, s);
    if (a.M <= 64) return launch_tile<64, 64, 2, 2>(a, s);
    return launch_tile<128, 128, 2, 2>(a, s);
}

// ---------------------------------------------------------------------------------------
// Generic path for any K % 4 == 0 and any alignment: one wave per output row n, lanes
// over packed bytes, the add/sub of [P2 §3.3] weight by weight.  Used only for shapes the
// fast kernels do not take; its results are identical.
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
            a.y[m * a.N + n] = dequant(s, dequant_scale(al, a.beta[m]), a.bias, n);
            if (a.acc) a.acc[m * a.N + n] = s;
        }
    }
}

hipError_t launch_forward_generic(const ForwardArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(k_forward_generic, dim3((unsigned)((a.N + 3) / 4)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace bitlinear
