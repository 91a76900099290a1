// gemv.hip -- decode-regime ternary x int8 GEMV (M <= 4 tokens) on the VALU, for gfx950.
//
// What is computed ([P2] nxmr.cn "1.58 位大模型" §3.3; [P3] chenxutan.com "1.58-bit 大模型极限量化实战"
// §2.4-§2.5, §3.2): acc[m,n] = sum_{W=+1} x_q[m,k] - sum_{W=-1} x_q[m,k], then
// y = fp32(acc) * fp32(alpha*beta[m]/127) (+ bias).  The fused variant also performs the
// per-token absmax quantization of x [P3 §2.4] inside the same launch.
//
// Decode streams every weight once, so the kernel is built around the weight stream:
//   * Each wave owns a contiguous range of rows and walks it R rows at a time with two
//     register buffers: the 16-byte loads of the next R rows are in flight while the current
//     R rows are reduced.  A wave load is 1 KiB of one packed row (4096 weights), fully
//     coalesced; row bases are wave-uniform (scalar) so a load costs one VGPR offset.
//   * Activations are staged once per workgroup into LDS; their loads are issued before the
//     weight loads, which complete in order behind them.  The fused variant reads fp32 x in
//     consecutive float4s (every wave load 1 KiB in whole lines, whatever the alignment of x)
//     and transposes each 16-weight group across the four lanes of a quad with DPP.
//   * A 16-byte load holds 64 codes c = W+1 in {0,1,2}, four per byte (weight 4b+i at bits
//     2i).  Fields i = 0,1,2 are isolated with one AND each (the byte then holds c * 4^i),
//     field 3 with a shift and an AND; v_dot4_i32_i8 multiplies each by four x_q bytes into
//     four accumulators, recombined as a0 + a1/4 + a2/16 + a3 (exact).  Because c - 1 = W,
//     acc = sum c*x_q - sum x_q: a +1 weight adds x_q, a 0 weight adds nothing, a -1 weight
//     subtracts it -- the add/sub with zero skipping, four bytes per instruction.
//   * x_q sits in LDS transposed within every 16-byte group (byte j of field dword i holds
//     x_q[k = 4j + i]) and ordered so that the 64 lanes of a wave read 1 KiB of consecutive
//     LDS per ds_read_b128.  Wave reductions use DPP inside 16-lane rows and readlane
//     across rows.
//   * One token with x quantized inside: on the shapes where it is faster the dot products run
//     on the 16x16x64 int8 MFMA instead, each lane multiplying its own codes by its own x_q
//     on the diagonal of the product (see finish_rows).
//   * The fused variant quantizes x with the quotient fp32(127x)/beta formed as q = a*y,
//     y = RN(1/beta), then q + (a - q*beta)*y with two FMAs: by Markstein's theorem (the
//     reciprocal within half an ulp, the first quotient within one ulp, the remainder exact
//     through the FMA) this is the correctly rounded IEEE quotient, bit for bit what a
//     division gives, at a third of the instructions.  The code is then rne(t) by adding
//     1.5 * 2^23 (|t| <= 127 since beta >= max |x|), its low byte gathered with v_perm.
#include "common.hpp"

namespace bitlinear {

struct GemvArgs {
    ForwardArgs f;        // f.xq / f.beta are inputs of the unfused kernel
    const float* x;       // fused: fp32 activations [M, K]
    int8_t* xq_out;       // fused: optional export of x_q [M, K]
    float* beta_out;      // fused: optional export of beta [M]
    int C;                // K / 64 (chunks of 64 weights per row)
    int64_t rows_per_wave;
};

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false); }

// Sum over each 16-lane row (every lane of the row ends with the row sum).
__device__ __forceinline__ int row16_sum(int v) {
    v += dpp_i<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_i<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_i<0x141>(v);   // row_half_mirror
    v += dpp_i<0x140>(v);   // row_mirror
    return v;
}

// Wave total, uniform (scalar) result.
__device__ __forceinline__ int wave_total(int v) {
    v = row16_sum(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ float wave_max_dpp(float f) {
    int v = __float_as_int(f);
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<0xB1>(v))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<0x4E>(v))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<0x141>(v))));
    v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp_i<0x140>(v))));
    const float a = __int_as_float(__builtin_amdgcn_readlane(v, 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(v, 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(v, 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(v, 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// int8 codes of four activations [P3 §2.4], clip(rne(fp32(127 x) / beta), -127, 127), byte i
// from component i.  The quotient is the correctly rounded one, from the reciprocal
// y = RN(1/beta) (see the file header).  beta >= max |x|, so |t| <= 127 (up to one rounding of
// fp32(127 x) above 127 beta, still far below 127.5): the clip never acts, and adding 1.5 * 2^23
// rounds t to an integer half-to-even, the sum lying in [2^23, 2^24) where floats are one
// apart.  The mantissa then holds 2^22 + rne(t), whose low byte is the two's-complement code
// (2^22 is a multiple of 256); v_perm gathers the four low bytes.
__device__ __forceinline__ uint32_t act_code_bits(float x, float beta, float y) {
    const float a = x * 127.0f;
    const float q = a * y;
    const float r = __builtin_fmaf(-q, beta, a);
    const float t = __builtin_fmaf(r, y, q);
    return __float_as_uint(t + 12582912.0f);
}

__device__ __forceinline__ uint32_t act_dword(float4 v, float beta, float y) {
    const uint32_t p01 = __builtin_amdgcn_perm(act_code_bits(v.y, beta, y), act_code_bits(v.x, beta, y), 0x0c0c0400u);
    const uint32_t p23 = __builtin_amdgcn_perm(act_code_bits(v.w, beta, y), act_code_bits(v.z, beta, y), 0x0c0c0400u);
    return __builtin_amdgcn_perm(p23, p01, 0x05040100u);
}

// MT tokens (the kernel masks tokens >= M), CPL chunks of 64 weights per lane and row,
// R rows per wave step, FUSED = quantize x inside, WAVES waves per workgroup, SINGLE = the
// wave's rows all fit one step (one register buffer, every weight load issued up front).
template <int MT, int CPL, int R, bool FUSED, int WAVES, bool SINGLE>
__global__ __launch_bounds__(64 * WAVES) void k_gemv(GemvArgs g) {
    constexpr int NT = 64 * WAVES;            // threads per workgroup
    constexpr int UNITS = MT * CPL * 256;     // 16-byte units of x_q staged per workgroup
    constexpr int UPT = (UNITS + NT - 1) / NT;
    extern __shared__ u32x4 xs[];          // [MT][CPL][4][64] units of 16 bytes
    __shared__ float red_f[MT][WAVES];
    __shared__ int red_i[MT][WAVES];
    const ForwardArgs& a = g.f;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int M = (int)a.M, C = g.C;
    const int64_t K = a.K, N = a.N, rowb = K >> 2;
    const int64_t rb = ((int64_t)blockIdx.x * WAVES + wave) * g.rows_per_wave;
    const int64_t re = rb + g.rows_per_wave < N ? rb + g.rows_per_wave : N;   // may be <= rb: no rows
    const bool tail_lane = lane + 64 * (CPL - 1) < C;   // the last chunk may be partial
    // One token, fused, MF: the dot products run on the matrix cores (see finish_rows), G rows
    // to an MFMA; lane l loads row rho of each group of G rows, 64-weight chunk slot mslot of
    // each sub-step.  Kept to where it measured faster (weights not in cache, against v_dot4):
    // four rows to an MFMA with rows of one or two chunks per lane, two with rows of two or
    // three.  K = 11008, N = 4096: 4.79 against 5.40 us; K = 8192, N = 8192: 5.38 against
    // 5.66 us; K = 8192, N = 28672: 12.41 against 13.17 us; K = 4096, N = 28672: 7.68 against
    // 8.90 us.  Slower: rows of one chunk two to an MFMA (K = 4096, N = 11008: 4.71 against
    // 4.53 us), one row to an MFMA (the trace's reduction per row), four rows of three chunks
    // (K = 11008, N = 8000: 7.92 against 7.79 us) and rows of four chunks (K = 16384, N = 8192:
    // 10.49 against 10.35 us).  Without the in-kernel quantization the weight stream hides the
    // dot products: level or up to 0.09 us slower.
    constexpr int G = R % 4 == 0 ? 4 : R % 2 == 0 ? 2 : 1;
    constexpr bool MF = MT == 1 && FUSED && ((G == 4 && CPL <= 2) || (G == 2 && CPL >= 2 && CPL <= 3));
    constexpr int LPR = 16 / G, CPI1 = 64 / G, NI = G * CPL;
    const int gl = lane >> 4, il = lane & 15;
    const int rho = il / LPR, mslot = gl * LPR + il % LPR;

    // ---- weight loads: rows r0 .. r0+R-1 into a register buffer -------------------------
    // Branch-free, so that the compiler can wait for exactly the loads it needs: rows past
    // this wave's range re-read its last row (never written back), and lanes past the last
    // 64-weight chunk of a row re-read chunk 0: the x_q staged for those lanes is zero, so
    // their products vanish.
    auto load_rows = [&](u32x4 (&w)[R][CPL], int64_t r0) {
        if constexpr (MF) {
            // sub-step s of group gr: chunk s * CPI1 + mslot of row r0 + G gr + rho (chunk 0
            // past the row end; its x_q is zero).  Issued in the order the MFMAs consume them,
            // sub-step major, so that the first sub-steps start while later loads are in flight.
            u32x4* wf = &w[0][0];
            const uint8_t* base[R / G];
#pragma unroll
            for (int gr = 0; gr < R / G; ++gr) {
                const int64_t row = r0 + gr * G + rho < re ? r0 + gr * G + rho : re - 1;
                base[gr] = a.wp + row * rowb;
            }
#pragma unroll
            for (int s = 0; s < NI; ++s) {
                const int c = s * CPI1 + mslot;
#pragma unroll
                for (int gr = 0; gr < R / G; ++gr)
                    wf[gr * NI + s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base[gr] + 16 * (c < C ? c : 0)));
            }
            return;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t row = r0 + r < re ? r0 + r : re - 1;
            const uint8_t* base = a.wp + row * rowb;     // wave-uniform
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int cj = (j < CPL - 1 || tail_lane) ? lane + 64 * j : 0;
                w[r][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + 16 * cj));
            }
        }
    };
    // ---- stage x_q.  Unit u of the LDS image holds the 16 weights' worth of x_q at
    // k = 64 c + 16 q for token t, with i = u / 256 = t * CPL + j, q = (u / 64) % 4, lane
    // l = u % 64 and c = l + 64 j: the lane that reads weight chunk c of a row finds its four
    // x_q dwords at units (i, q = 0..3, l).  Thread tid stages units tid, tid + NT, ...
    // With MF the four dwords of each chunk are stored transposed: unit (i, f, l) holds dword
    // f of units q = 0..3, so that one read gives the MFMA operand of field f (below).
    // The (small, cache-resident) activation loads are issued before the weight loads: a
    // wave's loads complete in order, so activations queued behind the weights would hold the
    // staging back until all of this wave's weights had arrived.  Out-of-range units load
    // element 0 and are masked afterwards, so the loads are unconditional.
    int part[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) part[t] = 0;
    auto unit_at = [&](int u, int& t, int& c, int& q) {
        const int i = u >> 8;
        t = i / CPL;
        c = (u & 63) + 64 * (i % CPL);
        q = (u >> 6) & 3;
        return u < UNITS && c < C && t < M;
    };
    auto add_part = [&](int t, int v) {
#pragma unroll
        for (int tt = 0; tt < MT; ++tt)
            if (tt == t) part[tt] += v;
    };
    u32x4 wa[R][CPL], wb[SINGLE ? 1 : R][SINGLE ? 1 : CPL];
    float beta_t[MT];
    // Scalars and per-row values are loaded ahead of the weights they go with: a wave's loads
    // complete in order, so a load issued after a weight prefetch makes its first use wait
    // for the whole prefetch.  The per-tensor alpha is read before anything else; a step's
    // per-row alpha and bias (for the lane that finishes row r0 + lane / MT) just before its
    // weight rows.  The loads are unconditional (element 0 when unused), so that no use of
    // them is moved up next to them.
    const float alpha0 = a.alpha[0];
    const float* bias_src = a.bias ? a.bias : a.alpha;
    struct RowAux { float al, bi; };
    auto load_aux = [&](int64_t r0) {
        const int rr = lane / MT < R ? lane / MT : R - 1;
        const int64_t row = r0 + rr < re ? r0 + rr : re - 1;
        return RowAux{a.alpha[a.alpha_per_row ? row : 0], bias_src[a.bias ? row : 0]};
    };
    RowAux auxa, auxb;
    if constexpr (FUSED) {
        // x is read in float4s, consecutive threads on consecutive float4s of the workgroup's
        // tokens (slot f = tid + NT * i is float4 f - 16 C t of token t), so every wave load
        // covers 1 KiB of x in whole cache lines whatever the alignment of x.  (Read per
        // 16-byte unit, the lanes of a wave load were 256 bytes apart; with x not at a multiple
        // of 1 KiB that cost 0.4 us per launch on the 7B shapes.)  The four lanes of a quad hold
        // the four dwords of one 16-weight group; two DPP exchanges inside the quad transpose it
        // into the LDS image.
        constexpr int SLOTS = MT * CPL * 1024;           // float4 slots, an upper bound of M * K / 4
        constexpr int FPT = (SLOTS + NT - 1) / NT;
        constexpr bool KEEP = FPT <= 16;                 // keep x in registers between the two passes
        const int k4 = (int)(K >> 2);                    // float4s per token (K % 64 == 0, K <= 32768)
        const int jj = tid & 3;                          // dword of the slot's 16-weight group
        auto slot_at = [&](int i, int& t, int& fl) {
            const int f = tid + NT * i;
            t = 0;
#pragma unroll
            for (int tt = 1; tt < MT; ++tt) t += f >= tt * k4 ? 1 : 0;
            fl = f - t * k4;
            return t < M && fl < k4;
        };
        float4 xv[KEEP ? FPT : 1];
        if constexpr (KEEP) {
#pragma unroll
            for (int i = 0; i < FPT; ++i) {
                int t, fl;
                const bool valid = slot_at(i, t, fl);
                xv[i] = reinterpret_cast<const float4*>(g.x)[valid ? t * k4 + fl : 0];
            }
        }
        auxa = load_aux(rb);
        load_rows(wa, rb);
        float mx[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) mx[t] = 0.0f;
        if constexpr (MT == 1) {
            // One token: the slots past the row re-read float4 0 of the row, which the maximum
            // already holds, so no slot is masked.  v_max3_f32 with |.| source modifiers takes two
            // activations per instruction; fmaxf made the compiler quiet every input first
            // (four instructions per float4 more).  NaN inputs give unspecified codes anyway.
#pragma unroll
            for (int i = 0; i < FPT; ++i) {
                float4 v;
                if constexpr (KEEP) v = xv[i];
                else v = reinterpret_cast<const float4*>(g.x)[tid + NT * i < k4 ? tid + NT * i : 0];
                asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(mx[0]) : "v"(v.x), "v"(v.y), "v"(mx[0]));
                asm("v_max3_f32 %0, |%1|, |%2|, %3" : "=v"(mx[0]) : "v"(v.z), "v"(v.w), "v"(mx[0]));
            }
        } else {
#pragma unroll
            for (int i = 0; i < FPT; ++i) {
                int t, fl;
                const bool valid = slot_at(i, t, fl);
                float4 v;
                if constexpr (KEEP) v = xv[i];
                else v = reinterpret_cast<const float4*>(g.x)[valid ? t * k4 + fl : 0];
                const float m = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
#pragma unroll
                for (int tt = 0; tt < MT; ++tt)
                    if (valid && tt == t) mx[tt] = fmaxf(mx[tt], m);
            }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const float m = wave_max_dpp(mx[t]);
            if (lane == 0) red_f[t][wave] = m;
        }
        __syncthreads();
        float rcp[MT];
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            float m = red_f[t][0];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) m = fmaxf(m, red_f[t][w]);
            beta_t[t] = m + 1e-8f;
            rcp[t] = 1.0f / beta_t[t];
        }
        const bool exporter = blockIdx.x == 0;
        uint32_t* xs32 = reinterpret_cast<uint32_t*>(xs);
        if constexpr (MT == 1) {
            // Slot i of thread tid is float4 f = tid + NT i: chunk c = tid / 16 + CPI i and
            // group q = (tid / 4) % 4 of it, so its LDS dword is a per-thread base plus a
            // compile-time offset.  Slots past the row (c >= C) store zero codes, which also
            // clears those chunks of the image: no separate clearing pass, no per-slot index
            // arithmetic.  With the maximum above, 12% fewer VALU instructions per wave at
            // K = 11008; measured with weights not in cache, K = 11008, N = 4096: 5.40 against
            // 5.78 us; K = 4096, N = 11008: 4.52 against 4.63 us; K = 28672, N = 8192: 14.04
            // against 15.00 us.
            constexpr int CPI = NT / 16, RPT = 64 / CPI;
            static_assert(CPI <= 64 && 64 % CPI == 0, "a slot step covers a divisor of 64 chunks");
            const int base = MF ? ((jj << 6) + (tid >> 4)) * 4 + ((tid >> 2) & 3)
                                : ((((tid >> 2) & 3) << 6) + (tid >> 4)) * 4 + jj;
            uint32_t dq[FPT];
            int sum = 0;
#pragma unroll
            for (int i = 0; i < FPT; ++i) {
                const bool valid = tid + NT * i < k4;
                float4 v;
                if constexpr (KEEP) v = xv[i];
                else v = reinterpret_cast<const float4*>(g.x)[valid ? tid + NT * i : 0];
                const uint32_t d = valid ? act_dword(v, beta_t[0], rcp[0]) : 0u;
                dq[i] = d;
                // quad transpose (a quad is valid or not as a whole: K % 64 == 0)
                const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d, 0xB1, 0xF, 0xF, true);
                const uint32_t t1 = __builtin_amdgcn_perm(p1, d, (jj & 1) ? 0x03070105u : 0x06020400u);
                const uint32_t p2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)t1, 0x4E, 0xF, 0xF, true);
                const uint32_t t2 = __builtin_amdgcn_perm(p2, t1, (jj & 2) ? 0x03020706u : 0x05040100u);
                xs32[base + (i / RPT) * 1024 + (i % RPT) * CPI * 4] = t2;
                sum += byte_sum(d);
            }
            part[0] = sum;
            if (exporter && g.xq_out) {
#pragma unroll
                for (int i = 0; i < FPT; ++i)
                    if (tid + NT * i < k4) reinterpret_cast<uint32_t*>(g.xq_out)[tid + NT * i] = dq[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < FPT; ++i) {
                int t, fl;
                const bool valid = slot_at(i, t, fl);
                float4 v;
                if constexpr (KEEP) v = xv[i];
                else v = reinterpret_cast<const float4*>(g.x)[valid ? t * k4 + fl : 0];
                float bt = beta_t[0], rt = rcp[0];
#pragma unroll
                for (int tt = 1; tt < MT; ++tt)
                    if (tt == t) { bt = beta_t[tt]; rt = rcp[tt]; }
                // x_q of weights k = 4 fl .. 4 fl + 3 (byte i = weight 4 fl + i)
                const uint32_t d = act_dword(v, bt, rt);
                // quad transpose: lane jj ends with byte j = weight 4 j + jj of the group
                const uint32_t p1 = (uint32_t)dpp_i<0xB1>((int)d);              // from lane jj ^ 1
                const uint32_t t1 = __builtin_amdgcn_perm(p1, d, (jj & 1) ? 0x03070105u : 0x06020400u);
                const uint32_t p2 = (uint32_t)dpp_i<0x4E>((int)t1);             // from lane jj ^ 2
                const uint32_t t2 = __builtin_amdgcn_perm(p2, t1, (jj & 2) ? 0x03020706u : 0x05040100u);
                if (valid) {
                    const int G = fl >> 2;                       // 16-weight group within the token
                    const int c = G >> 2, q = G & 3;
                    xs32[((((t * CPL + (c >> 6)) * 4 + q) << 6) + (c & 63)) * 4 + jj] = t2;
                    add_part(t, byte_sum(d));
                    if (exporter && g.xq_out) reinterpret_cast<uint32_t*>(g.xq_out + t * K)[fl] = d;
                }
            }
            // units of chunks past the row end (and of tokens past M) hold zeros
            for (int u = tid; u < UNITS; u += NT) {
                const int i = u >> 8;
                const int t = i / CPL, c = (u & 63) + 64 * (i % CPL);
                if (c >= C || t >= M) xs[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
        if (exporter && g.beta_out && tid < M) {
#pragma unroll
            for (int t = 0; t < MT; ++t)
                if (t == tid) g.beta_out[t] = beta_t[t];
        }
    } else {
        u32x4 xr[UPT];
#pragma unroll
        for (int k = 0; k < UPT; ++k) {
            int t, c, q;
            const bool valid = unit_at(tid + NT * k, t, c, q);
            xr[k] = *reinterpret_cast<const u32x4*>(a.xq + (valid ? t * K + 64 * c + 16 * q : 0));
        }
        auxa = load_aux(rb);
        load_rows(wa, rb);
#pragma unroll
        for (int k = 0; k < UPT; ++k) {
            const int u = tid + NT * k;
            int t, c, q;
            u32x4 o = {0u, 0u, 0u, 0u};
            if (unit_at(u, t, c, q)) {
                o = transpose4x4_bytes(xr[k]);
                add_part(t, byte_sum(xr[k].x) + byte_sum(xr[k].y) + byte_sum(xr[k].z) + byte_sum(xr[k].w));
            }
            if constexpr (MF) {
                if (u < UNITS) {
                    uint32_t* xs32 = reinterpret_cast<uint32_t*>(xs);
                    const int cc = (u & 63) + 64 * ((u >> 8) % CPL), qq = (u >> 6) & 3;
                    const int u0 = (((cc >> 6) * 4) << 6) + (cc & 63);
#pragma unroll
                    for (int f = 0; f < 4; ++f) xs32[(u0 + 64 * f) * 4 + qq] = o[f];
                }
            } else {
                if (u < UNITS) xs[u] = o;
            }
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) beta_t[t] = t < M ? a.beta[t] : 0.0f;
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int v = wave_total(part[t]);
        if (lane == 0) red_i[t][wave] = v;
    }
    __syncthreads();
    int xsum[MT];
    float sc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        xsum[t] = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) xsum[t] += red_i[t][w];
        sc[t] = a.alpha_per_row ? 0.0f : dequant_scale(alpha0, beta_t[t]);
    }

    // ---- reduce R rows held in w, finish them ------------------------------------------
    auto finish_rows = [&](const u32x4 (&w)[R][CPL], const RowAux& aux, int64_t r0) {
        if constexpr (MF) {
            // The 16x16x64 int8 MFMA pairs byte j of lane l's A operand with byte j of the same
            // lane's B operand on its diagonal: C[i][i] sums the products of lanes i, i + 16,
            // i + 32, i + 48.  So every lane puts 16 codes of its own chunk in A and the
            // matching 16 x_q in B, and the trace of C is the wave's dot product; the lanes of
            // row rho of a group feed diagonal entries rho * 16/G .. (rho + 1) * 16/G - 1.  The
            // field i codes of a chunk (c, 4c or 16c in each byte after one AND; field 3 shifted
            // down) go to four accumulators, recombined as a0 + a1/4 + a2/16 + a3 (exact).
            // Against v_dot4: 20 instead of 36 VALU instructions per 64 weights and lane.
            constexpr int RG = R / G;
            const u32x4* wf = &w[0][0];
            i32x4 acc[RG][4];
#pragma unroll
            for (int gr = 0; gr < RG; ++gr)
#pragma unroll
                for (int f = 0; f < 4; ++f) acc[gr][f] = i32x4{0, 0, 0, 0};
#pragma unroll
            for (int s = 0; s < NI; ++s) {
                // one sub-step at a time: hoisting the operands of later sub-steps ran the
                // double-buffered kernels out of registers
                __builtin_amdgcn_sched_barrier(0);
                const int c = s * CPI1 + mslot;
                const int u0 = (((c >> 6) * 4) << 6) + (c & 63);
                i32x4 B[4];
#pragma unroll
                for (int f = 0; f < 4; ++f) B[f] = (i32x4)xs[u0 + 64 * f];
#pragma unroll
                for (int gr = 0; gr < RG; ++gr) {
                    const u32x4 v = wf[gr * NI + s];
                    const i32x4 A0 = (i32x4)(v & 0x03030303u), A1 = (i32x4)(v & 0x0C0C0C0Cu);
                    const i32x4 A2 = (i32x4)(v & 0x30303030u), A3 = (i32x4)((v >> 6) & 0x03030303u);
                    acc[gr][0] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A0, B[0], acc[gr][0], 0, 0, 0);
                    acc[gr][1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A1, B[1], acc[gr][1], 0, 0, 0);
                    acc[gr][2] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A2, B[2], acc[gr][2], 0, 0, 0);
                    acc[gr][3] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A3, B[3], acc[gr][3], 0, 0, 0);
                }
            }
            // register r of lane l holds C[4 (l / 16) + r][l % 16]: C[i][i] sits in lane
            // i + 16 (i / 4), register i % 4, so lanes 0-3, 20-23, 40-43, 60-63 hold the
            // diagonal, four entries (one quad) for each quarter of the rows of C
            const int sel = il & 3;
            const bool diag = (il >> 2) == gl;
            int mine = 0;
#pragma unroll
            for (int gr = 0; gr < RG; ++gr) {
                int e[4];
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const i32x4 q = acc[gr][f];
                    e[f] = sel == 0 ? q.x : sel == 1 ? q.y : sel == 2 ? q.z : q.w;
                }
                int v = diag ? e[0] + e[3] + (e[1] >> 2) + (e[2] >> 4) : 0;
                v += dpp_i<0xB1>(v);
                v += dpp_i<0x4E>(v);
                const int q0 = __builtin_amdgcn_readlane(v, 0), q1 = __builtin_amdgcn_readlane(v, 20);
                const int q2 = __builtin_amdgcn_readlane(v, 40), q3 = __builtin_amdgcn_readlane(v, 60);
                int tr[G];
                if constexpr (G == 4) { tr[0] = q0; tr[1] = q1; tr[2] = q2; tr[3] = q3; }
                else if constexpr (G == 2) { tr[0] = q0 + q1; tr[1] = q2 + q3; }
                else tr[0] = q0 + q1 + q2 + q3;
#pragma unroll
                for (int p = 0; p < G; ++p)
                    if (lane == gr * G + p) mine = tr[p];
            }
            // lane r finishes row r0 + r
            if (lane < R) {
                const int64_t n = r0 + lane;
                if (n < re) {
                    const int total = mine - xsum[0];
                    const float sv = a.alpha_per_row ? dequant_scale(aux.al, beta_t[0]) : sc[0];
                    float yv = (float)total * sv;
                    if (a.bias) yv = yv + aux.bi;
                    a.y[n] = activate(yv, a.act);
                    if (a.acc) a.acc[n] = total;
                }
            }
            return;
        }
        int s0[R][MT], s1[R][MT], s2[R][MT], s3[R][MT];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < MT; ++t) s0[r][t] = s1[r][t] = s2[r][t] = s3[r][t] = 0;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4 X[MT];
#pragma unroll
                for (int t = 0; t < MT; ++t) X[t] = xs[((t * CPL + j) * 4 + q) * 64 + lane];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const uint32_t v = q == 0 ? w[r][j].x : q == 1 ? w[r][j].y : q == 2 ? w[r][j].z : w[r][j].w;
                    const uint32_t d0 = v & 0x03030303u;          // c
                    const uint32_t d1 = v & 0x0C0C0C0Cu;          // 4c
                    const uint32_t d2 = v & 0x30303030u;          // 16c
                    const uint32_t d3 = (v >> 6) & 0x03030303u;   // c
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        s0[r][t] = dot4(d0, X[t].x, s0[r][t]);
                        s1[r][t] = dot4(d1, X[t].y, s1[r][t]);
                        s2[r][t] = dot4(d2, X[t].z, s2[r][t]);
                        s3[r][t] = dot4(d3, X[t].w, s3[r][t]);
                    }
                }
            }
        // lane r*MT + t finishes (r0 + r, token t)
        int mine = 0, my_xsum = 0, my_t = 0, my_r = 0;
        float my_sc = 0.0f, my_beta = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const int v = wave_total(s0[r][t] + (s1[r][t] >> 2) + (s2[r][t] >> 4) + s3[r][t]);
                if (lane == r * MT + t) {
                    mine = v;
                    my_xsum = xsum[t];
                    my_sc = sc[t];
                    my_beta = beta_t[t];
                    my_t = t;
                    my_r = r;
                }
            }
        if (lane < R * MT) {
            const int64_t n = r0 + my_r;
            if (n < re && my_t < M) {
                const int total = mine - my_xsum;
                const float s = a.alpha_per_row ? dequant_scale(aux.al, my_beta) : my_sc;
                float v = (float)total * s;
                if (a.bias) v = v + aux.bi;
                a.y[my_t * N + n] = activate(v, a.act);
                if (a.acc) a.acc[my_t * N + n] = total;
            }
        }
    };

    // ---- walk the row range, two register buffers in turn -------------------------------
    if constexpr (SINGLE) {
        (void)wb;
        (void)auxb;
        if (rb < re) finish_rows(wa, auxa, rb);
    } else {
        for (int64_t r0 = rb; r0 < re; r0 += 2 * R) {
            auxb = load_aux(r0 + R);
            load_rows(wb, r0 + R);
            finish_rows(wa, auxa, r0);
            if (r0 + R >= re) break;
            auxa = load_aux(r0 + 2 * R);
            load_rows(wa, r0 + 2 * R);
            finish_rows(wb, auxb, r0 + R);
        }
    }
}

// ---------------------------------------------------------------------------------------
// Launch shape: waves per workgroup and the number of waves the grid aims at; each wave gets
// ceil(N / waves) contiguous rows: one step holding all of them when they fit the registers,
// else steps of R rows with two buffers.
// Measured on MI355X over the decode shapes (one token):
//  * forward (x_q given): with rows of one 64-weight chunk per lane (K <= 4096) many small
//    workgroups win (4 waves, 8192 waves in all, 1-2 rows each: loads of many waves overlap
//    the short compute of each); longer rows want about 2048 waves, in workgroups of 8 except
//    for three chunks per lane, where 4 win (weights not in cache: K = 8192, N = 4096, 3.84 vs
//    4.42 us with 8 and 4 waves; N = 8192, 5.30 vs 6.38 us; K = 11008, N = 4096, 5.32 vs
//    4.40 us; N = 8192, 8.01 vs 6.71 us);
//  * fused (x fp32 given): every workgroup reads all of x to find its absmax, so fewer, larger
//    workgroups win: 8 waves and 2048 in all.  16 waves and 4096 in all for rows of two to
//    four chunks per lane was 1-10% slower (weights not in cache: K = 8192, N = 4096, 5.80 vs
//    5.21 us; K = 11008, N = 4096, 7.35 vs 6.68 us; K = 16384, N = 4096, 8.65 vs 7.93 us).
// Shapes with too few rows for that many waves per CU fall back to 4-wave workgroups.
GemvShape gemv_shape(int64_t M, int64_t K, int64_t N, bool fused) {
    GemvShape sh{4, 2048};
    if (M != 1) {
        // several tokens, fused: every workgroup reads all M rows of fp32 x (twice when they do
        // not fit its registers), so half the workgroups: 1024 waves, 256 workgroups of 4
        // (several-token instances exist with 4 waves only; with 8 or 16 they spill).  Measured
        // with weights not in cache, four tokens: 19.1 vs 32.7 us at K = 11008, N = 4096; 29.6
        // vs 47.7 us at K = 16384, N = 8192; 512 waves is slower again (22.4 and 39.2 us).
        if (fused && N >= 8 * 256) sh = GemvShape{4, 1024};
        return sh;
    }
    const int64_t cpl = (K / 64 + 63) / 64;
    GemvShape want;
    if (!fused)
        want = cpl == 1 ? GemvShape{4, N >= 8192 ? 8192 : 2048} : GemvShape{cpl == 3 ? 4 : 8, 2048};
    else
        want = GemvShape{8, 2048};
    if (N >= (int64_t)want.waves_per_wg * 256) sh = want;
    return sh;
}

// single step: R from {1, 2, 3, 4, 6, 8}, the smallest not below the rows per wave, within
// 20 loads of 16 bytes per lane (4- and 8-wave workgroups have 256 VGPRs per wave)
constexpr int single_loads(int /*waves*/, int /*cpl*/) { return 20; }
constexpr int next_rows(int r) { return r == 1 ? 2 : r == 2 ? 3 : r == 3 ? 4 : r == 4 ? 6 : 8; }

template <int MT, int CPL, bool FUSED, int WAVES, int R>
static hipError_t launch_single(const GemvArgs& g, dim3 grid, dim3 block, size_t lds, int64_t rpw, hipStream_t s) {
    if constexpr (R < 8 && next_rows(R) * CPL <= single_loads(WAVES, CPL))
        if (rpw > R) return launch_single<MT, CPL, FUSED, WAVES, next_rows(R)>(g, grid, block, lds, rpw, s);
    return launch_with_lds(k_gemv<MT, CPL, R, FUSED, WAVES, true>, grid, block, lds, s, g);
}

template <int MT, int CPL, bool FUSED, int WAVES>
static hipError_t launch_shape(const GemvArgs& g0, int64_t waves_target, hipStream_t s) {
    // One token: when a wave's rows fit the registers, one step with every weight load issued
    // before the activation staging.  Otherwise (and for 2-4 tokens, whose
    // accumulators take more registers) double-buffered steps of R rows, R * CPL <= LMAX.
    constexpr int LMAX = MT == 1 ? 8 : 4;
    constexpr int R = (LMAX / CPL) < 1 ? 1 : (LMAX / CPL);
    GemvArgs g = g0;
    const int64_t N = g.f.N;
    const int64_t rpw = (N + waves_target - 1) / waves_target;
    g.rows_per_wave = rpw;
    const int64_t waves = (N + rpw - 1) / rpw;
    const int64_t blocks = (waves + WAVES - 1) / WAVES;
    const size_t lds = (size_t)MT * CPL * 256 * 16;
    const dim3 grid((unsigned)blocks), block(64 * WAVES);
    if constexpr (MT == 1) {
        int rs = 1;
        while (rs < rpw && rs < 8) rs = next_rows(rs);
        if (rs >= rpw && rs * CPL <= single_loads(WAVES, CPL))
            return launch_single<MT, CPL, FUSED, WAVES, 1>(g, grid, block, lds, rpw, s);
    }
    if constexpr (WAVES == 16 && CPL > 3) {
        return hipErrorInvalidConfiguration;   // not chosen by gemv_shape (it would spill)
    } else {
        return launch_with_lds(k_gemv<MT, CPL, R, FUSED, WAVES, false>, grid, block, lds, s, g);
    }
}

template <int MT, int CPL, bool FUSED>
static hipError_t launch_cpl(const GemvArgs& g, hipStream_t s) {
    const GemvShape sh = gemv_shape(g.f.M, g.f.K, g.f.N, FUSED);
    if constexpr (MT == 1)
        if (sh.waves_per_wg == 8) return launch_shape<MT, CPL, FUSED, 8>(g, sh.waves_target, s);
    return launch_shape<MT, CPL, FUSED, 4>(g, sh.waves_target, s);
}

template <bool FUSED>
static hipError_t launch_m1(const GemvArgs& g, hipStream_t s) {
    switch ((g.C + 63) / 64) {
        case 1: return launch_cpl<1, 1, FUSED>(g, s);
        case 2: return launch_cpl<1, 2, FUSED>(g, s);
        case 3: return launch_cpl<1, 3, FUSED>(g, s);
        case 4: return launch_cpl<1, 4, FUSED>(g, s);
        case 5: return launch_cpl<1, 5, FUSED>(g, s);
        case 6: return launch_cpl<1, 6, FUSED>(g, s);
        case 7: return launch_cpl<1, 7, FUSED>(g, s);
        default: return launch_cpl<1, 8, FUSED>(g, s);
    }
}

// Two and three tokens in their own instances: the four-token kernel would do up to twice
// the dot products.
template <int MT, bool FUSED>
static hipError_t launch_mt(const GemvArgs& g, hipStream_t s) {
    switch ((g.C + 63) / 64) {
        case 1: return launch_cpl<MT, 1, FUSED>(g, s);
        case 2: return launch_cpl<MT, 2, FUSED>(g, s);
        case 3: return launch_cpl<MT, 3, FUSED>(g, s);
        default: return launch_cpl<MT, 4, FUSED>(g, s);
    }
}

template <bool FUSED>
static hipError_t launch_m4(const GemvArgs& g, hipStream_t s) {
    switch ((g.C + 63) / 64) {
        case 1: return launch_cpl<4, 1, FUSED>(g, s);
        case 2: return launch_cpl<4, 2, FUSED>(g, s);
        case 3: return launch_cpl<4, 3, FUSED>(g, s);
        default: return launch_cpl<4, 4, FUSED>(g, s);
    }
}

// One token: up to 8 chunks of 64 weights per lane (K <= 32768); two to four tokens: up
// to 4 (K <= 16384).  Other shapes go to the MFMA kernel.
bool gemv_supports(int64_t M, int64_t K) {
    if (K % 64 != 0 || M < 1 || M > 4) return false;
    return M == 1 ? K <= 32768 : K <= 16384;
}

hipError_t launch_gemv_dot4(const ForwardArgs& a, hipStream_t s) {
    GemvArgs g{a, nullptr, nullptr, nullptr, (int)(a.K / 64), 0};
    return a.M == 1 ? launch_m1<false>(g, s) : a.M == 2 ? launch_mt<2, false>(g, s)
         : a.M == 3 ? launch_mt<3, false>(g, s) : launch_m4<false>(g, s);
}

hipError_t launch_gemv_fused(const ForwardArgs& a, const float* x, int8_t* xq_out, float* beta_out, hipStream_t s) {
    GemvArgs g{a, x, xq_out, beta_out, (int)(a.K / 64), 0};
    return a.M == 1 ? launch_m1<true>(g, s) : a.M == 2 ? launch_mt<2, true>(g, s)
         : a.M == 3 ? launch_mt<3, true>(g, s) : launch_m4<true>(g, s);
}

}  // namespace bitlinear
