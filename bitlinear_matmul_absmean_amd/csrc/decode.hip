// decode.hip -- batched-decode ternary x int8 matmul (a few to 64 tokens) on the int8 matrix
// cores (v_mfma_i32_16x16x64_i8), gfx950.
//
// What is computed ([P3] chenxutan.com "1.58-bit 大模型极限量化实战" §2.4-§2.5, §3.2;
// [P2] nxmr.cn "1.58 位大模型" §3.3): acc = x_q . W_hat^T (int32), y = fp32(acc) *
// fp32(alpha*beta[m]/127) (+ bias).
//
// With up to 64 tokens the product is still bound by the weight stream (the ridge of int8
// MFMA against HBM is near 78 tokens), so the weights are read exactly once, straight from
// HBM into registers, 16 bytes (64 codes) per lane: lane (n, g) of a wave holds bytes
// [16g, 16g+16) of a 64-byte block of row n, i.e. one wave load covers 16 rows x 256
// weights.  Dword d of the lane's 16 bytes (16 codes) is expanded by four masks
// (v >> 2i) & 0x03030303 into the lane's 16-byte B operand of MFMA number d, so byte 4i+j of
// the operand is the code c = W+1 of weight k = 4j + i of that 16-weight group.
//
// Work split: a workgroup owns 16*RB rows and all tokens; its waves split K in 256-weight
// chunks, round robin.  x_q is staged per K-phase into LDS with every 16-byte group
// transposed 4x4 (byte 4i+j = x_q[k = 4j+i]), which is the A operand of the MFMA, so A and B
// meet on the same k.  The per-token sum of x_q is accumulated while staging; since
// c - 1 = W, acc = sum c*x_q - sum x_q.  The waves' partial 16x16 tiles are added in LDS at
// the end (integer sums: order-free, exact).
#include "common.hpp"

namespace bitlinear {

// 4x4 byte transpose with v_perm_b32: out[i] byte j = in[j] byte i.
__device__ __forceinline__ u32x4 transpose4x4_perm(u32x4 s) {
    const uint32_t a01l = __builtin_amdgcn_perm(s.y, s.x, 0x05010400u);   // s0b0 s1b0 s0b1 s1b1
    const uint32_t a01h = __builtin_amdgcn_perm(s.y, s.x, 0x07030602u);   // s0b2 s1b2 s0b3 s1b3
    const uint32_t a23l = __builtin_amdgcn_perm(s.w, s.z, 0x05010400u);
    const uint32_t a23h = __builtin_amdgcn_perm(s.w, s.z, 0x07030602u);
    u32x4 o;
    o.x = __builtin_amdgcn_perm(a23l, a01l, 0x05040100u);
    o.y = __builtin_amdgcn_perm(a23l, a01l, 0x07060302u);
    o.z = __builtin_amdgcn_perm(a23h, a01h, 0x05040100u);
    o.w = __builtin_amdgcn_perm(a23h, a01h, 0x07060302u);
    return o;
}

// MB: 16-token column blocks (tokens <= 16*MB); RB: 16-row blocks per workgroup;
// WAVES: waves per workgroup (K split); KP: K-phase length staged in LDS (multiple of 256).
template <int MB, int RB, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void k_decode_mfma(ForwardArgs a, int KP) {
    extern __shared__ u32x4 lds[];
    __shared__ int tsum[64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = (int)a.M;
    const int64_t K = a.K, N = a.N, rowb = K >> 2;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * RB);
    const int lr = lane & 15, lg = lane >> 4;
    const int ustride = KP / 16 + 1;           // LDS units per token row (one unit of padding)

    for (int i = tid; i < 64; i += WAVES * 64) tsum[i] = 0;

    i32x4 acc[RB][MB];
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int b = 0; b < MB; ++b) acc[r][b] = i32x4{0, 0, 0, 0};

    // token row each lane feeds as A (rows past M repeat the last token; their results are dropped)
    int arow[MB];
#pragma unroll
    for (int b = 0; b < MB; ++b) arow[b] = min(16 * b + lr, M - 1) * ustride;

    for (int64_t p0 = 0; p0 < K; p0 += KP) {
        const int kp = (int)(K - p0 < KP ? K - p0 : KP);
        const int c0 = (int)(p0 / 256), c1 = (int)((p0 + kp + 255) / 256);

        // 1. this wave's weight chunks of the phase: issue every load first
        constexpr int CMAX = 8 / RB;           // chunks per wave per phase (host keeps KP small enough)
        u32x4 w[CMAX][RB];
#pragma unroll
        for (int i = 0; i < CMAX; ++i) {
            const int c = c0 + wave + WAVES * i;
            const bool cv = c < c1 && (int64_t)c * 256 + 64 * lg < K;
#pragma unroll
            for (int r = 0; r < RB; ++r) {
                const int64_t n = n0 + 16 * r + lr;
                w[i][r] = (cv && n < N)
                              ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.wp + n * rowb + 64 * (int64_t)c + 16 * lg))
                              : u32x4{0u, 0u, 0u, 0u};
            }
        }

        // 2. stage x_q[:, p0 : p0 + kp] transposed; sum x_q per token
        __syncthreads();                       // previous phase's readers are done
        const int units = M * (kp / 16);
        for (int u = tid; u < units; u += WAVES * 64) {
            const int m = u / (kp / 16), gidx = u - m * (kp / 16);
            const u32x4 s = *reinterpret_cast<const u32x4*>(a.xq + m * K + p0 + 16 * gidx);
            lds[m * ustride + gidx] = transpose4x4_perm(s);
            atomicAdd(&tsum[m], byte_sum(s.x) + byte_sum(s.y) + byte_sum(s.z) + byte_sum(s.w));
        }
        __syncthreads();

        // 3. MFMAs
#pragma unroll
        for (int i = 0; i < CMAX; ++i) {
            const int c = c0 + wave + WAVES * i;
            if (c >= c1) break;
            const int gbase = (int)((int64_t)c * 256 - p0) / 16 + 4 * lg;   // this lane group's first unit
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                i32x4 aop[MB];
#pragma unroll
                for (int b = 0; b < MB; ++b) aop[b] = (i32x4)lds[arow[b] + gbase + d];
#pragma unroll
                for (int r = 0; r < RB; ++r) {
                    const uint32_t v = d == 0 ? w[i][r].x : d == 1 ? w[i][r].y : d == 2 ? w[i][r].z : w[i][r].w;
                    const i32x4 bop = {(int)(v & 0x03030303u), (int)((v >> 2) & 0x03030303u),
                                       (int)((v >> 4) & 0x03030303u), (int)((v >> 6) & 0x03030303u)};
#pragma unroll
                    for (int b = 0; b < MB; ++b)
                        acc[r][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(aop[b], bop, acc[r][b], 0, 0, 0);
                }
            }
        }
    }

    // 4. add the waves' partial tiles (LDS reused), then the epilogue
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int b = 0; b < MB; ++b) lds[((r * MB + b) * WAVES + wave) * 64 + lane] = (u32x4)acc[r][b];
    __syncthreads();
    const float alpha0 = a.alpha_per_row ? 0.0f : a.alpha[0];
    for (int t = wave; t < RB * MB; t += WAVES) {
        const int r = t / MB, b = t % MB;
        i32x4 s = {0, 0, 0, 0};
        for (int wv = 0; wv < WAVES; ++wv) s += (i32x4)lds[(t * WAVES + wv) * 64 + lane];
        const int64_t n = n0 + 16 * r + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int m = 16 * b + 4 * lg + e;        // 16x16 result: lane l, element e -> row 4*(l/16)+e, col l%16
            if (m < M && n < N) {
                const int total = s[e] - tsum[m];
                const float al = a.alpha_per_row ? a.alpha[n] : alpha0;
                a.y[m * N + n] = dequant(total, dequant_scale(al, a.beta[m]), a.bias, n);
                if (a.acc) a.acc[m * N + n] = total;
            }
        }
    }
}

template <int MB, int RB, int WAVES>
static hipError_t launch_cfg(const ForwardArgs& a, hipStream_t s) {
    // K-phase: each wave gets at most 8/RB chunks of 256 weights per phase, and the staged
    // x_q phase must fit the LDS budget.
    int kp = WAVES * (8 / RB) * 256;
    const int64_t budget = 144 * 1024;
    while (kp > 256 && ((int64_t)a.M * (kp / 16 + 1) + 16) * 16 > budget) kp /= 2;
    const int64_t red = (int64_t)RB * MB * WAVES * 64 * 16;
    // 16 spare units: a partial last chunk's idle lane groups address up to 11 units past a row
    const int64_t stage = ((int64_t)a.M * (kp / 16 + 1) + 16) * 16;
    const size_t lds = (size_t)(stage > red ? stage : red);
    const dim3 grid((unsigned)((a.N + 16 * RB - 1) / (16 * RB))), block(WAVES * 64);
    return launch_with_lds(k_decode_mfma<MB, RB, WAVES>, grid, block, lds, s, a, kp);
}

bool decode_mfma_supports(int64_t M, int64_t K) { return M >= 1 && M <= 64 && K % 64 == 0; }

hipError_t launch_decode_mfma(const ForwardArgs& a, hipStream_t s) {
    // enough workgroups to cover the chip with 16*RB rows each
    const int64_t N = a.N;
    if (a.M <= 16) {
        if (N >= 8192) return launch_cfg<1, 2, 4>(a, s);
        return launch_cfg<1, 1, 4>(a, s);
    }
    if (a.M <= 32) {
        if (N >= 8192) return launch_cfg<2, 2, 4>(a, s);
        return launch_cfg<2, 1, 4>(a, s);
    }
    if (N >= 8192) return launch_cfg<4, 2, 8>(a, s);
    return launch_cfg<4, 1, 8>(a, s);
}

}  // namespace bitlinear
