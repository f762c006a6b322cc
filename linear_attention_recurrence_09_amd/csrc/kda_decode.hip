// kda_decode.hip -- decode steps of the KDA mixer (gfx950): one new token,
// or K drafted tokens, for each of B sequences.
//
// "Inside Kimi K3" (lei.chat), KDA short-convolution diagram: autoregressive
// decoding keeps the 3 previous raw inputs of every channel of the combined
// QKV; the new window is [state, x_t].  KDA one-head diagram and "Animated
// Kimi K3 architecture diagram" (github.io), local-memory panel: decay the
// key rows of S, probe with k, correct e = v - Sbar^T k, write beta k e^T,
// read S^T q.
//
// One workgroup per (sequence, head).  The state is one streaming pass: each
// of 256 threads loads its 16 (D = 128) float4 of S (non-temporal: the state
// is streamed once per call), and per token decays them, accumulates
// Sbar^T k and Sbar^T q for its 4 columns, the column sums are reduced across
// row groups, and the same registers take the rank-1 write.  The read uses
// o = Sbar^T q + beta (k . q) e, which equals S_t^T q.  HBM traffic is one read
// and at most one write of the fp32 state plus the small per-token tensors.
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kDecThreads = 256;

// The state streams through once per call: non-temporal loads and stores keep
// it from displacing cached data.
template <typename V>
__device__ __forceinline__ V stream_load(const V* p) {
    return __builtin_nontemporal_load(p);
}
template <typename V>
__device__ __forceinline__ void stream_store(V v, V* p) {
    __builtin_nontemporal_store(v, p);
}

// Several new tokens per sequence in one pass over the state: the K tokens a
// drafter proposes are checked in one call ("Kimi K3" on archdiff.com,
// component list: the MTP layer used as an EAGLE-3 drafter, and speculative
// decoding by MTP self-drafting).  Each token is the step above; the state of
// the (sequence, head) and each channel's conv window stay in registers
// across the tokens, so the state is read once and written at most once per
// call.  After token n_b of sequence b (n_b = n_tokens[b], clamped to [0, K];
// K when n_tokens is null) the state and the conv window are stored to
// state_out / cs_out (when given); outputs are written for all K tokens when
// o is given, otherwise the loop stops after n_b tokens.
//
// Two layouts of the state in registers (kStrided): thread (rg, cg) holds
// columns 4cg .. 4cg+3 of rows rg + R j (each load instruction covers R
// adjacent rows; the q, k and decay of key channel i then sit in LDS at
// position (i % R) RPT + i / R) or of rows rg RPT + j (consecutive; fewer
// registers).  Either way a thread's q, k and decays are 16-byte LDS reads.
// The strided layout streams faster; the consecutive one keeps three
// workgroups per CU, which pays once several tokens' arithmetic dominates.
// Lane sums of the token loop: DPP and permlane steps (group_sum) in the
// consecutive-row kernel, where the per-token work dominates; shuffles through
// the LDS crossbar in the strided kernel, which streams the state for one or
// two tokens and measured 1-2% faster with them.
template <bool kXbar, int width>
__device__ __forceinline__ float lane_sum(float v) {
    if constexpr (kXbar) {
#pragma unroll
        for (int m = 1; m < width; m <<= 1) v += __shfl_xor(v, m, 64);
        return v;
    } else {
        return group_sum<width>(v);
    }
}

template <typename T, int D, bool kStrided>
__global__ void __launch_bounds__(kDecThreads)
decode_multi_kernel(const T* __restrict__ x, const float* __restrict__ w, const T* cs_in,
                    T* cs_out, const T* __restrict__ g, const T* __restrict__ beta,
                    const float* state_in, float* state_out, T* __restrict__ o,
                    const int32_t* __restrict__ n_tokens, int K, int H, float l2_eps) {
    constexpr int CG = D / 4;                 // float4 column groups per row
    constexpr int R = kDecThreads / CG;       // row groups
    constexpr int RPT = D / R;                // rows per thread
    constexpr int CT = 3 * D / 2;             // conv threads (2 channels each)
    __shared__ __attribute__((aligned(16))) float su[3 * D];   // token's conv output: q | k | v
    __shared__ __attribute__((aligned(16))) float sa[D];       // per-key-channel retention
    __shared__ float sred[kDecThreads / 64][CG][8];
    __shared__ float skq;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int bh = blockIdx.x;
    const int b = bh / H;
    const int h = bh % H;
    const int P = 3 * H * D;
    int nb = K;
    if (n_tokens != nullptr) {
        nb = n_tokens[b];
        nb = nb < 0 ? 0 : (nb > K ? K : nb);
    }
    const int nt = o != nullptr ? K : nb;
    const bool snapshot = state_out != nullptr;

    // ---- state loads first: the longest-latency traffic ---------------------
    static_assert(RPT % 4 == 0, "rows per thread in fours");
    const int cg = tid % CG;
    const int rg = tid / CG;
    const int r0 = rg * RPT;   // LDS position of this thread's first row
    auto srow = [&](int j) { return kStrided ? rg + R * j : r0 + j; };   // state row
    auto pos = [](int i) { return kStrided ? (i % R) * RPT + i / R : i; };   // LDS position
    const float* Sin = state_in + (int64_t)bh * D * D;
    floatx4 sv[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j)
        sv[j] = stream_load(reinterpret_cast<const floatx4*>(Sin + srow(j) * D + 4 * cg));

    // ---- this thread's two conv channels: taps and rolling window ----------
    int part = 3;
    int64_t c = 0;
    float wt[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float w0[3] = {0.f, 0.f, 0.f}, w1[3] = {0.f, 0.f, 0.f};   // oldest first
    if (tid < CT) {
        const int cc = 2 * tid;               // channel within [q | k | v] of head h
        part = cc / D;
        c = (int64_t)part * H * D + h * D + cc % D;
        const T* sp = cs_in + ((int64_t)b * P + c) * 3;
        load2(sp, w0[0], w0[1]);
        load2(sp + 2, w0[2], w1[0]);
        load2(sp + 4, w1[1], w1[2]);
#pragma unroll
        for (int i = 0; i < 8; ++i) wt[i] = w[c * 4 + i];
    }
    auto store_states = [&]() {
        float* Sout = state_out + (int64_t)bh * D * D;
#pragma unroll
        for (int j = 0; j < RPT; ++j)
            stream_store(sv[j], reinterpret_cast<floatx4*>(Sout + srow(j) * D + 4 * cg));
        if (tid < CT) {
            T* sp = cs_out + ((int64_t)b * P + c) * 3;
            store2(sp, w0[0], w0[1]);
            store2(sp + 2, w0[2], w1[0]);
            store2(sp + 4, w1[1], w1[2]);
        }
    };
    if (snapshot && nb == 0) store_states();

    for (int t = 0; t < nt; ++t) {
        const int64_t row = (int64_t)b * K + t;   // token row of x, g, beta and o
        // the previous token's reads of su, sa, sred and skq are done
        if (t > 0) __syncthreads();

        // ---- conv window + SiLU + L2 ---------------------------------------
        float y0 = 0.f, y1 = 0.f;
        if (tid < CT) {
            float x0, x1;
            load2(x + row * P + c, x0, x1);
            const float p0 = wt[0] * w0[0] + wt[1] * w0[1] + wt[2] * w0[2] + wt[3] * x0;
            const float p1 = wt[4] * w1[0] + wt[5] * w1[1] + wt[6] * w1[2] + wt[7] * x1;
            y0 = siluf_(p0);
            y1 = siluf_(p1);
            w0[0] = w0[1]; w0[1] = w0[2]; w0[2] = x0;
            w1[0] = w1[1]; w1[1] = w1[2]; w1[2] = x1;
        }
        float ss = lane_sum<kStrided, D / 2>(y0 * y0 + y1 * y1);
        if (part < 2) {
            const float inv = rsqrt_nr(ss + l2_eps);
            y0 *= inv;
            y1 *= inv;
        }
        if (tid < CT) {
            const int cc = 2 * tid - part * D;   // channel within q, k or v
            su[part * D + (part < 2 ? pos(cc) : cc)] = y0;
            su[part * D + (part < 2 ? pos(cc + 1) : cc + 1)] = y1;
        }
        if (tid < D) sa[pos(tid)] = fast_exp2(clamp_log_decay(to_f(g[(row * H + h) * D + tid])) * kLog2e);
        const float bt = to_f(beta[row * H + h]);
        __syncthreads();

        if (wave == 0) {   // k . q
            float kq = 0.f;
            for (int i = lane; i < D; i += 64) kq += su[i] * su[D + i];
            kq = lane_sum<kStrided, 64>(kq);
            if (lane == 0) skq = kq;
        }

        // ---- decay, and the column sums Sbar^T k, Sbar^T q ------------------
        float4 ak = make_float4(0.f, 0.f, 0.f, 0.f), aq = ak;
        floatx4 kr[RPT / 4];   // k of this thread's rows, kept for the write
#pragma unroll
        for (int j4 = 0; j4 < RPT / 4; ++j4) {
            const floatx4 a4 = *reinterpret_cast<const floatx4*>(sa + r0 + 4 * j4);
            const floatx4 q4 = *reinterpret_cast<const floatx4*>(su + r0 + 4 * j4);
            kr[j4] = *reinterpret_cast<const floatx4*>(su + D + r0 + 4 * j4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * j4 + e;
                sv[j] *= a4[e];
                const float ki = kr[j4][e], qi = q4[e];
                ak.x += ki * sv[j][0]; ak.y += ki * sv[j][1]; ak.z += ki * sv[j][2]; ak.w += ki * sv[j][3];
                aq.x += qi * sv[j][0]; aq.y += qi * sv[j][1]; aq.z += qi * sv[j][2]; aq.w += qi * sv[j][3];
            }
        }
        // Sum over the row groups of the wave (lanes cg, cg + CG, ...).  The
        // 16-lane level (D = 64) keeps every sum in every lane; the 32-lane
        // level swaps two sums at once, so lanes below 32 end with those of
        // x and z and lanes from 32 on with those of y and w.
        float pr[8] = {ak.x, ak.y, ak.z, ak.w, aq.x, aq.y, aq.z, aq.w};
        if constexpr (CG == 16) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float even = pr[e], odd = pr[e];
                rows_swap16(even, odd);   // even: rows 0, 0, 2, 2   odd: rows 1, 1, 3, 3
                pr[e] = even + odd;
            }
        }
        static_assert(CG == 16 || CG == 32, "row groups of the wave");
        const int hw = lane >> 5;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            rows_swap32(pr[e], pr[e + 1]);
            pr[e] += pr[e + 1];
        }
        if ((lane & 31) < CG) {
            float* r = sred[wave][cg];
            r[hw] = pr[0]; r[2 + hw] = pr[2]; r[4 + hw] = pr[4]; r[6 + hw] = pr[6];
        }
        __syncthreads();
        float tk[4] = {0.f, 0.f, 0.f, 0.f}, tq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int wv = 0; wv < kDecThreads / 64; ++wv)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                tk[e] += sred[wv][cg][e];
                tq[e] += sred[wv][cg][4 + e];
            }
        const float kq = skq;
        float ev[4], ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ev[e] = su[2 * D + 4 * cg + e] - tk[e];
            ov[e] = tq[e] + bt * kq * ev[e];
        }
        if (o != nullptr && rg == 0) {
            T* op = o + (row * H + h) * D + 4 * cg;
#pragma unroll
            for (int e = 0; e < 4; ++e) op[e] = from_f<T>(ov[e]);
        }
        // ---- write: S = Sbar + beta k e^T -----------------------------------
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const float bk = bt * kr[j / 4][j % 4];
            sv[j][0] += bk * ev[0]; sv[j][1] += bk * ev[1]; sv[j][2] += bk * ev[2]; sv[j][3] += bk * ev[3];
        }
        if (snapshot && t == nb - 1) store_states();
    }
}

template <typename T, int D>
hipError_t launch_decode_multi_t(const void* x, const float* w, const void* cs_in, void* cs_out,
                                 const void* g, const void* beta, const float* state_in,
                                 float* state_out, void* o, const int32_t* n_tokens, int B, int K,
                                 int H, float l2_eps, hipStream_t s) {
    const int64_t blocks = (int64_t)B * H;
    if (blocks == 0) return hipSuccess;
    // up to two tokens the state streaming dominates: strided rows
    if (K <= 2)
        hipLaunchKernelGGL((decode_multi_kernel<T, D, true>), dim3((unsigned)blocks),
                           dim3(kDecThreads), 0, s, (const T*)x, w, (const T*)cs_in, (T*)cs_out,
                           (const T*)g, (const T*)beta, state_in, state_out, (T*)o, n_tokens, K,
                           H, l2_eps);
    else
        hipLaunchKernelGGL((decode_multi_kernel<T, D, false>), dim3((unsigned)blocks),
                           dim3(kDecThreads), 0, s, (const T*)x, w, (const T*)cs_in, (T*)cs_out,
                           (const T*)g, (const T*)beta, state_in, state_out, (T*)o, n_tokens, K,
                           H, l2_eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_multi(const void* x, const float* w, const void* cs_in, void* cs_out,
                               const void* g, const void* beta, const float* state_in,
                               float* state_out, void* o, const int32_t* n_tokens, int B, int K,
                               int H, int D, int dtype, float l2_eps, hipStream_t s) {
    if (dtype == 0) {
        return D == 64 ? launch_decode_multi_t<float, 64>(x, w, cs_in, cs_out, g, beta, state_in,
                                                          state_out, o, n_tokens, B, K, H, l2_eps, s)
                       : launch_decode_multi_t<float, 128>(x, w, cs_in, cs_out, g, beta, state_in,
                                                           state_out, o, n_tokens, B, K, H, l2_eps, s);
    }
    return D == 64 ? launch_decode_multi_t<__bf16, 64>(x, w, cs_in, cs_out, g, beta, state_in,
                                                       state_out, o, n_tokens, B, K, H, l2_eps, s)
                   : launch_decode_multi_t<__bf16, 128>(x, w, cs_in, cs_out, g, beta, state_in,
                                                        state_out, o, n_tokens, B, K, H, l2_eps, s);
}

// One token: the states are updated in place.
hipError_t launch_decode(const void* x, const float* w, void* conv_state, const void* g,
                         const void* beta, float* state, void* o, int B, int H, int D,
                         int dtype, float l2_eps, hipStream_t s) {
    return launch_decode_multi(x, w, conv_state, conv_state, g, beta, state, state, o, nullptr, B,
                               1, H, D, dtype, l2_eps, s);
}

}  // namespace kda
