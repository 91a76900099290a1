// gemm.hip -- prefill-regime ternary x int8 GEMM on the int8 matrix cores
// (v_mfma_i32_32x32x32_i8), gfx950; plus the generic kernel for shapes the fast paths skip.
//
// What is computed ([P3] chenxutan.com "1.58-bit 大模型极限量化实战" §2.4-§2.5, §3.2, §5.5;
// [P2] nxmr.cn "1.58 位大模型" §3.3): acc = x_q . W_hat^T in int32, y = fp32(acc) *
// fp32(alpha*beta[m]/127) (+ bias).  With many tokens (prefill) this is a dense contraction
// and the compute peak is what matters [P3 §5.5], so it runs on MFMA.
//
// Tiles: a workgroup computes BM tokens x BN weight rows, four waves in a WGM x WGN grid, K in
// steps of BK with double-buffered LDS (one barrier per step).  Per step:
//   * A (x_q): BM x BK bytes from global, every 16-byte group transposed 4x4 with v_perm so that
//     operand byte 4i+j holds x_q[k = 4j+i], written to LDS (rows padded against bank
//     conflicts).  The same pass accumulates the per-token sum of x_q.
//   * B (weights): BN rows x BK/4 bytes of packed codes, to LDS as they are (4x less traffic
//     than int8); the lane feeding column n reads one packed dword (16 codes) and expands it
//     with four masks (v >> 2i) & 0x03030303 into its 16-byte operand: byte 4i+j = c of weight
//     4j+i.  c = W+1, so acc = sum c*x_q - sum x_q.
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

template <int BM, int BN, int BK, int WGM, int WGN>
__global__ __launch_bounds__(256, 2) void k_gemm_mfma(ForwardArgs a, int tiles_m, int tiles_n) {
    static_assert(WGM * WGN == 4, "four waves per workgroup");
    constexpr int WM = BM / WGM, WN = BN / WGN;       // wave tile
    constexpr int FM = WM / 32, FN = WN / 32;         // 32x32 MFMA blocks per wave
    constexpr int GK = BK / 16;                       // 16-byte groups per row and step
    constexpr int AU = BM * GK;                       // A units per step
    constexpr int APT = AU / 256;                     // A units per thread
    constexpr int ASTR = GK + 1;                      // LDS units per A row (one of padding)
    constexpr int BPR = BK / 64;                      // 16-byte packed units per B row and step
    constexpr int BU = BN * BPR;
    constexpr int BTB = BN * BK / 4 / 256;            // bytes of the B tile each thread moves
    static_assert(AU % 256 == 0 && FM >= 1 && FN >= 1, "tile shape");
    static_assert(BTB == 8 || BTB == 16, "B staging granularity");

    __shared__ u32x4 As[2][BM * ASTR];
    __shared__ u32x4 Bs[2][BU];
    __shared__ int rsum[BM];
    __shared__ float ssc[BM];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int64_t M = a.M, N = a.N, K = a.K, rowb = K >> 2;

    // XCD-aware tile order: hardware id h runs on XCD h % 8; give XCD x the contiguous logical
    // tiles [x * T/8, (x+1) * T/8) when T % 8 == 0 (else keep the hardware order).
    const int T = tiles_m * tiles_n;
    int t = blockIdx.x;
    if (T % 8 == 0) t = (t % 8) * (T / 8) + t / 8;
    const int tm = t / tiles_n, tn = t % tiles_n;       // token block major
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int KS = (int)(K / BK);

    for (int i = tid; i < BM; i += 256) {
        const int64_t m = m0 + i;
        ssc[i] = (!a.alpha_per_row && m < M) ? dequant_scale(a.alpha[0], a.beta[m]) : 0.0f;
    }

    // Two register stages: the global loads of step ks+2 are issued while step ks computes,
    // so about two steps of MFMA work cover their L2 / Infinity Cache latency.
    // B staging words (BTB bytes per thread): dwords 0..BTB/4-1 used
    u32x4 ra0[APT], rb0[1], ra1[APT], rb1[1];
    int rs[APT];
#pragma unroll
    for (int i = 0; i < APT; ++i) rs[i] = 0;

    // Branch-free loads (rows past M or N are clamped to the last row: their results are
    // never written), so the compiler can count outstanding loads exactly.
    auto gload = [&](u32x4 (&ra)[APT], u32x4 (&rb)[1], int ks) {
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int u = tid + 256 * i;
            const int64_t m = min(m0 + u / GK, M - 1);
            ra[i] = *reinterpret_cast<const u32x4*>(a.xq + m * K + (int64_t)ks * BK + 16 * (u % GK));
        }
        {
            const int byte = tid * BTB;                   // offset inside the BN x BK/4 tile
            const int64_t n = min(n0 + byte / (BK / 4), N - 1);
            const uint8_t* src = a.wp + n * rowb + (int64_t)ks * (BK / 4) + byte % (BK / 4);
            if constexpr (BTB == 16) {
                rb[0] = *reinterpret_cast<const u32x4*>(src);
            } else {
                const uint2 v = *reinterpret_cast<const uint2*>(src);
                rb[0] = u32x4{v.x, v.y, 0u, 0u};
            }
        }
    };
    auto sstore = [&](const u32x4 (&ra)[APT], const u32x4 (&rb)[1], int buf, bool count) {
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int u = tid + 256 * i;
            As[buf][(u / GK) * ASTR + u % GK] = transpose4x4_v(ra[i]);
            const int bs = byte_sum(ra[i].x) + byte_sum(ra[i].y) + byte_sum(ra[i].z) + byte_sum(ra[i].w);
            rs[i] += count ? bs : 0;
        }
        uint8_t* bdst = reinterpret_cast<uint8_t*>(&Bs[buf][0]) + tid * BTB;
        // dword p of column c is stored at p ^ (2 * ((c >> 4) & 1)) (see the reads)
        const bool sw = ((tid * BTB / (BK / 4)) >> 4) & 1;
        if constexpr (BTB == 16) {
            *reinterpret_cast<u32x4*>(bdst) = sw ? u32x4{rb[0].z, rb[0].w, rb[0].x, rb[0].y} : rb[0];
        } else {
            // 8 bytes = dwords (2h, 2h+1) of the column: they move to (2h^2, 2h^2+1)
            const int h = (tid * BTB % (BK / 4)) / 8;
            uint8_t* col = bdst - (tid * BTB % (BK / 4));
            *reinterpret_cast<uint2*>(col + 8 * (sw ? (h ^ 1) : h)) = make_uint2(rb[0].x, rb[0].y);
        }
    };

    i32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = i32x16{};

    const int lr = lane & 31, lg = lane >> 5;
    auto compute = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < BK / 32; ++kk) {          // 32 weights per MFMA step
            i32x4 bop[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = wn * WN + j * 32 + lr;
                // packed dword 2*kk + lg of this column's BK/4-byte slice = its 16 codes
                // (stored XOR-swizzled by column so that columns c and c+16 use other banks)
                const int pos = (2 * kk + lg) ^ (((col >> 4) & 1) << 1);
                const uint32_t v = reinterpret_cast<const uint32_t*>(&Bs[buf][col * BPR])[pos];
                bop[j] = i32x4{(int)(v & 0x03030303u), (int)((v >> 2) & 0x03030303u),
                               (int)((v >> 4) & 0x03030303u), (int)((v >> 6) & 0x03030303u)};
            }
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * WM + i * 32 + lr;
                const i32x4 aop = (i32x4)As[buf][row * ASTR + kk * 2 + lg];
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop, bop[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    // Steady state: the loads are unconditional (past the end they re-read the last step,
    // whose data is then not used), so the compiler can wait for the older stage only
    // (vmcnt of the newer stage's count) instead of draining every load.
    const int last = KS - 1;
    gload(ra0, rb0, 0);
    gload(ra1, rb1, KS > 1 ? 1 : 0);
    sstore(ra0, rb0, 0, true);
    __syncthreads();
    int ks = 0;
    for (; ks + 2 <= KS; ks += 2) {
        gload(ra0, rb0, min(ks + 2, last));
        compute(0);
        sstore(ra1, rb1, 1, true);
        __syncthreads();
        gload(ra1, rb1, min(ks + 3, last));
        compute(1);
        sstore(ra0, rb0, 0, ks + 2 < KS);
        __syncthreads();
    }
    if (ks < KS) compute(0);               // odd number of steps: the last one sits in buffer 0

    // per-token sums of x_q: the GK consecutive threads that staged a row hold its parts
#pragma unroll
    for (int i = 0; i < APT; ++i) {
        int v = rs[i];
#pragma unroll
        for (int s = 1; s < GK; s <<= 1) v += __shfl_xor(v, s, 64);
        const int u = tid + 256 * i;
        if (u % GK == 0) rsum[u / GK] = v;
    }
    __syncthreads();

    // 32x32 MFMA result layout: lane l, element r -> row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int mr = wm * WM + i * 32 + 8 * (r / 4) + 4 * lg + (r % 4);
            const int64_t m = m0 + mr;
            if (m >= M) continue;
            const int xs = rsum[mr];
            const float s0 = ssc[mr];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int64_t n = n0 + wn * WN + j * 32 + lr;
                if (n < N) {
                    const int total = acc[i][j][r] - xs;
                    const float s = a.alpha_per_row ? dequant_scale(a.alpha[n], a.beta[m]) : s0;
                    a.y[m * N + n] = dequant(total, s, a.bias, n);
                    if (a.acc) a.acc[m * N + n] = total;
                }
            }
        }
}

template <int BM, int BN, int BK, int WGM, int WGN>
static hipError_t launch_tile(const ForwardArgs& a, hipStream_t s) {
    const int tm = (int)((a.M + BM - 1) / BM), tn = (int)((a.N + BN - 1) / BN);
    hipLaunchKernelGGL((k_gemm_mfma<BM, BN, BK, WGM, WGN>), dim3((unsigned)(tm * tn)), dim3(256), 0, s, a, tm, tn);
    return hipGetLastError();
}

bool gemm_supports_k(int64_t K) { return K % 64 == 0; }

hipError_t launch_gemm_mfma(const ForwardArgs& a, hipStream_t s) {
    return launch_tile<128, 256, 64, 2, 2>(a, s);
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
