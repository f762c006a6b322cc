// kda_chunk_pipe.hip -- KDA chunked prefill with 16-token chunks and
// producer / consumer waves (gfx950, bf16 I/O, fp32 state).
//
// Method: "Inside Kimi K3" (lei.chat), KDA one-head diagram -- per-channel
// retention alpha_t = exp(g_t) with g_t >= -5, write strength beta_t, a fixed
// dk x dv state, recurrent across chunks and parallel inside a chunk;
// "Animated Kimi K3 architecture diagram" (github.io), local-memory panel --
// decay, probe, correct e_t = v_t - Sbar_t^T k_t, write beta_t k_t e_t^T, read
// S_t^T q_t.
//
// Chunk form (exact re-association of the token recurrence).  For a chunk of
// 16 tokens with entering state S, G_r = sum_{u<=r} g_u per channel:
//   Kt = K e^G,  Qt = Q e^G,  Kh = K e^{G_15 - G},  Ki = K e^{-G}
//   A_kk = strict_lower(Kt Ki^T),  A_qk = lower(Qt Ki^T)
//   M' = (I + diag(beta) A_kk)^{-1} diag(beta)
//   U  = M' (V - Kt S)
//   O  = Qt S + A_qk U
//   S <- diag(e^{G_15}) S + Kh^T U
// A 16-token chunk spans at most e^{-80} of decay (g >= -5), so every factor
// above is a finite fp32 / bf16 number and no intra-chunk splitting is needed.
//
// Work split.  One workgroup per (sequence, head, slice of 64 value columns).
//  * Producer waves (4) build everything that does not depend on the state,
//    one whole chunk per wave: per-channel decay products with lanes on
//    channels (serial over the 16 tokens), the operand tiles Kt, Qt, Ki, Kh
//    and V in LDS, A_kk^T and A_qk^T on MFMA, and the 16 x 16 unit triangular
//    inverse by back substitution in registers (row broadcasts by DPP and the
//    gfx950 cross-row lane swaps).  Results go to a ring of LDS slots.
//  * Consumer waves (one per 16 value columns) hold their columns of the fp32
//    state in MFMA accumulators for the whole sequence; the state chain of a
//    chunk (V - Kt S, Qt S, M' Z, A_qk U, decay, Kh^T U) is wave-local, so
//    consumers never wait on each other.  S feeds the next chunk's products as
//    an in-register bf16 B operand: the contraction index is permuted to the
//    accumulator's row order, and Kt / Qt are stored in LDS in that order.
//  * Slots are handed over through LDS counters (producer: "chunk ready",
//    consumers: "slot released"), so producers run ahead of the consumers by
//    up to the ring depth.  Every wait is bounded; a wait that runs out stops
//    the workgroup and its final state is written as NaN.
#include "kda_device.hpp"
#include "kda_launch.hpp"

#ifdef KDA_PIPE_PROFILE
extern __device__ unsigned long long kda_pipe_cycles[16];
#endif

namespace kda {

namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16v4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((address_space(3))) bf16v4* lds_bf16v4_ptr;

constexpr int kNP = 4;                 // producer waves
constexpr int kRing = 6;               // LDS slots
constexpr int kSpinLimit = 1 << 17;    // polls (about 128 cycles each) before giving up

template <int DK, int DVS>
struct PipeCfg {
    static constexpr int NC = DVS / 16;                 // consumer waves
    static constexpr int THREADS = 64 * (NC + kNP);
    static constexpr int CPL = DK / 64;                 // channels per producer lane
    static constexpr int NKS = DK / 32;                 // 16x16x32 steps over the key channels
    static constexpr int NKT = DK / 16;                 // 16-row key tiles of the state
    // Row pitches (bytes).  Tiles read 16 B per lane along a row get a 16 B
    // pad (row starts 4 banks apart); tiles read by the 4-row transposed 8 B
    // read get 32 B (8 banks apart).
    static constexpr int PK = DK * 2 + 16;
    static constexpr int PH = DK * 2 + 32;
    static constexpr int PV = DVS * 2 + 32;
    static constexpr int O_KT = 0;                      // K e^G       (permuted channels)
    static constexpr int O_QT = O_KT + 16 * PK;         // Q e^G       (permuted channels)
    static constexpr int O_KI = O_QT + 16 * PK;         // K e^-G      (permuted channels)
    static constexpr int O_KH = O_KI + 16 * PK;         // K e^{G15-G} (natural order)
    static constexpr int O_V = O_KH + 16 * PH;          // V slice
    static constexpr int O_MP = O_V + 16 * PV;          // M' as 16x16x16 A operands
    static constexpr int O_AQ = O_MP + 512;             // A_qk as 16x16x16 A operands
    static constexpr int O_GM = O_AQ + 512;             // e^{G15}, consumer lane order
    static constexpr int SLOT = O_GM + 512;
    static constexpr int BYTES = kRing * SLOT;
    static_assert(DK == 64 || DK == 128, "key width");
    static_assert(DVS == 64, "value slice");
    static_assert(SLOT % 16 == 0, "slot alignment");
    static_assert(BYTES <= 160 * 1024 - 256, "LDS budget");
};

// Position of channel c inside its 32-channel group in the permuted tiles:
// lane group q of a 16x16x32 operand reads positions 8q..8q+7, which hold
// channels 4q..4q+3 and 16+4q..16+4q+3 -- the rows that lane group q holds in
// the two 16-row accumulator tiles of the state.
__device__ __forceinline__ int perm_pos(int c) {
    const int x = c & 31;
    const int p = x < 16 ? 8 * (x >> 2) + (x & 3) : 8 * ((x - 16) >> 2) + 4 + (x & 3);
    return (c & ~31) | p;
}

__device__ __forceinline__ floatx4 mfma32(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mfma16(shortx4 a, shortx4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ shortx4 pack4(float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
    return __builtin_bit_cast(shortx4, v);
}

// Transposed 8-byte LDS read (gfx950): lane j of each 16-lane group supplies
// the address of row k0 + j/4, columns n0 + 4(j%4) .. +3 of a row-major bf16
// matrix; lane n of the group receives column n0 + n, rows k0 .. k0+3.
__device__ __forceinline__ bf16v4 lds_read_tr(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16v4_ptr)(p));
}

// Lane n of every 16-lane row, broadcast to the whole row.
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x150 + N, 0xF, 0xF, false));
}
// Row G (lanes 16G .. 16G+15) copied to all four rows, lane order kept.
template <int G>
__device__ __forceinline__ float rows_from(float x) {
    const int xi = __builtin_bit_cast(int, x);
    const auto p16 = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
    const int a = (G & 1) ? (int)p16[1] : (int)p16[0];      // rows {G&1, G&1, 2+(G&1), 2+(G&1)}
    const auto p32 = __builtin_amdgcn_permlane32_swap(a, a, false, false);
    return __builtin_bit_cast(float, (G & 2) ? (int)p32[1] : (int)p32[0]);
}

// S[KT..] <- diag(e^{G_15}) S + Kh^T U for the key tiles KT .. NKT-1.  Row i
// of tile KT is channel 16 KT + 4q + i; its decay sits in lane 2 KT + i/2 of
// the lane's own row, component i % 2.
template <int KT, int NKT>
__device__ __forceinline__ void state_update(floatx4 (&S)[NKT], const bf16v4 (&kh)[NKT],
                                             shortx4 ub, floatx2 gm) {
    if constexpr (KT < NKT) {
        S[KT][0] *= row_bcast<2 * KT>(gm[0]);
        S[KT][1] *= row_bcast<2 * KT>(gm[1]);
        S[KT][2] *= row_bcast<2 * KT + 1>(gm[0]);
        S[KT][3] *= row_bcast<2 * KT + 1>(gm[1]);
        S[KT] = mfma16(__builtin_bit_cast(shortx4, kh[KT]), ub, S[KT]);
        state_update<KT + 1, NKT>(S, kh, ub, gm);
    }
}

// ---- slot hand-over ----------------------------------------------------------
__device__ __forceinline__ int flag_load(int* f) {
    return __hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Counter updates are made by lane 0 only: an atomic executed by a whole
// wave acts once per active lane.
__device__ __forceinline__ void flag_store(int* f, int v, int lane) {
    if (lane == 0) __hip_atomic_store(f, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void flag_add(int* f, int v, int lane) {
    if (lane == 0) __hip_atomic_fetch_add(f, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Wait until *f >= target.  Returns false (and raises the workgroup's stop
// flag) if the wait runs out, or if another wave has raised it.
__device__ __forceinline__ bool wait_at_least(int* f, int target, int* stop) {
    int n = 0;
    while (flag_load(f) < target) {
        if (__hip_atomic_load(stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0) return false;
        if (++n > kSpinLimit) {
            __hip_atomic_store(stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return false;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    return true;
}

template <int DK, int DVS, int THREADS = PipeCfg<DK, DVS>::THREADS>
__global__ void __launch_bounds__(THREADS)
chunk_pipe_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                  const __bf16* __restrict__ v, int64_t stride, const __bf16* __restrict__ g,
                  const __bf16* __restrict__ beta, __bf16* __restrict__ o, const float* s0,
                  float* sT, const int32_t* __restrict__ cu, int num_seqs, int T_len, int H,
                  int DV, int nsplit) {
    using Cfg = PipeCfg<DK, DVS>;
    constexpr int NC = Cfg::NC, CPL = Cfg::CPL, NKS = Cfg::NKS, NKT = Cfg::NKT;
    constexpr int PK = Cfg::PK, PH = Cfg::PH, PV = Cfg::PV, SLOT = Cfg::SLOT;

    __shared__ __attribute__((aligned(16))) char smem[Cfg::BYTES];
    __shared__ int flags[2 * kRing + 1];   // ready[kRing], released[kRing], stop
    int* ready = flags;
    int* released = flags + kRing;
    int* stop = flags + 2 * kRing;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int lr = lane & 15;
    const int lq = lane >> 4;

    // ---- workgroup -> (sequence, head, value slice); slices of one chain are
    // placed 8 ids apart so they run on the same XCD and share its L2 --------
    const int nchain = num_seqs * H;
    const int total = nchain * nsplit;
    const int bid = blockIdx.x;
    const int span = 8 * nsplit;
    const int full = (total / span) * span;
    int chain, split;
    if (bid < full) {
        const int gi = bid >> 3, xcd = bid & 7;
        chain = (gi / nsplit) * 8 + xcd;
        split = gi % nsplit;
    } else {
        const int r = bid - full;
        chain = full / nsplit + r / nsplit;
        split = r % nsplit;
    }
    const int seq = chain / H;
    const int head = chain % H;
    const int n0 = split * DVS;
    const int64_t t_begin = cu ? (int64_t)cu[seq] : (int64_t)seq * T_len;
    const int64_t t_end = cu ? (int64_t)cu[seq + 1] : t_begin + T_len;
    const int64_t n_chunks = (t_end - t_begin + 15) / 16;

    if (tid < 2 * kRing + 1) flags[tid] = 0;
    __syncthreads();

    if (wave >= NC) {
        // ===================== producer wave =================================
        const int pw = wave - NC;
        const int c0 = lane * CPL;                 // this lane's channels
        using RawC = typename RawVec<__bf16, CPL>::type;
        constexpr int VL = DVS / 32;               // 16 B pieces of V per lane
        RawC rg[16], rk[16], rq[16];
        u32x4 rv[VL];
        __bf16 rbl, rb4[4];
        const int g_row = H * DK * 2, kv_row = (int)(stride * 2), b_row = H * 2;
        auto issue_loads = [&](int64_t ci) {
            const int64_t t0 = t_begin + ci * 16;
            const int64_t rem = t_end - t0;
            const int valid = (int)(rem < 16 ? rem : 16);
            const rsrc_t r_g = make_rsrc(g + (t0 * H + head) * DK, (uint32_t)(valid * g_row));
            const rsrc_t r_k = make_rsrc(k + t0 * stride + (int64_t)head * DK, (uint32_t)(valid * kv_row));
            const rsrc_t r_q = make_rsrc(q + t0 * stride + (int64_t)head * DK, (uint32_t)(valid * kv_row));
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                rg[t] = BufLoad<__bf16, CPL>::load(r_g, t * g_row + c0 * 2);
                rk[t] = BufLoad<__bf16, CPL>::load(r_k, t * kv_row + c0 * 2);
                rq[t] = BufLoad<__bf16, CPL>::load(r_q, t * kv_row + c0 * 2);
            }
            const rsrc_t r_v = make_rsrc(v + t0 * stride + (int64_t)head * DV + n0, (uint32_t)(valid * kv_row));
#pragma unroll
            for (int j = 0; j < VL; ++j) {
                const int piece = lane * VL + j;          // 16 B pieces, DVS/8 per token
                rv[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    r_v, (piece / (DVS / 8)) * kv_row + (piece % (DVS / 8)) * 16, 0, 0));
            }
            const rsrc_t r_b = make_rsrc(beta + t0 * H + head, (uint32_t)(valid * b_row));
            rbl = BufLoad<__bf16, 1>::load(r_b, lr * b_row);
#pragma unroll
            for (int i = 0; i < 4; ++i) rb4[i] = BufLoad<__bf16, 1>::load(r_b, (4 * lq + i) * b_row);
        };
        if (pw < n_chunks) issue_loads(pw);

        for (int64_t ci = pw; ci < n_chunks; ci += kNP) {
            const int s = (int)(ci % kRing);
            const int round = (int)(ci / kRing);
            if (!wait_at_least(&released[s], NC * round, stop)) break;
            char* slot = smem + s * SLOT;

            // ---- decay products, lanes on channels, serial over tokens ------
            float a[16][CPL], F[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) F[j] = 1.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float gv[CPL], kv[CPL], qv[CPL], kt[CPL], qt[CPL];
                RawVec<__bf16, CPL>::unpack(rg[t], gv);
                RawVec<__bf16, CPL>::unpack(rk[t], kv);
                RawVec<__bf16, CPL>::unpack(rq[t], qv);
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    a[t][j] = fast_exp2(clamp_log_decay(gv[j]) * kLog2e);
                    F[j] *= a[t][j];                      // e^{G_t}
                    kt[j] = kv[j] * F[j];
                    qt[j] = qv[j] * F[j];
                }
                RawVec<__bf16, CPL>::store(reinterpret_cast<__bf16*>(slot + Cfg::O_KT + t * PK) + perm_pos(c0), kt);
                RawVec<__bf16, CPL>::store(reinterpret_cast<__bf16*>(slot + Cfg::O_QT + t * PK) + perm_pos(c0), qt);
            }
            float inv_end[CPL], R[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                inv_end[j] = fast_rcp(F[j]);              // e^{-G_15} <= e^80
                R[j] = 1.f;
            }
#pragma unroll
            for (int t = 15; t >= 0; --t) {
                float kv[CPL], kh[CPL], ki[CPL];
                RawVec<__bf16, CPL>::unpack(rk[t], kv);
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    kh[j] = kv[j] * R[j];                 // R = e^{G_15 - G_t}
                    ki[j] = kv[j] * (R[j] * inv_end[j]);  // e^{-G_t}
                    R[j] *= a[t][j];
                }
                RawVec<__bf16, CPL>::store(reinterpret_cast<__bf16*>(slot + Cfg::O_KH + t * PH) + c0, kh);
                RawVec<__bf16, CPL>::store(reinterpret_cast<__bf16*>(slot + Cfg::O_KI + t * PK) + perm_pos(c0), ki);
            }
            // e^{G_15} per channel, laid out for the consumers' row broadcasts:
            // channel 16*kt + 4*q + i -> entry [q][2*kt + i/2][i%2]
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                const int c = c0 + j;
                const int kt = c >> 4, qq = (c >> 2) & 3, i = c & 3;
                reinterpret_cast<float*>(slot + Cfg::O_GM)[(qq * 16 + 2 * kt + (i >> 1)) * 2 + (i & 1)] = F[j];
            }
#pragma unroll
            for (int j = 0; j < VL; ++j) {
                const int piece = lane * VL + j;
                *reinterpret_cast<u32x4*>(slot + Cfg::O_V + (piece / (DVS / 8)) * PV + (piece % (DVS / 8)) * 16) = rv[j];
            }
            const float bl = (float)rbl;
            float b4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) b4[i] = (float)rb4[i];

            // the next chunk of this wave streams in while this one finishes
            if (ci + kNP < n_chunks) issue_loads(ci + kNP);

            // ---- A_kk^T, A_qk^T (16x16x32 MFMA over the key channels) -------
            floatx4 akk = zero4(), aqk = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int off = lr * PK + (32 * ks + 8 * lq) * 2;
                const bf16x8 fi = *reinterpret_cast<const bf16x8*>(slot + Cfg::O_KI + off);
                const bf16x8 fk = *reinterpret_cast<const bf16x8*>(slot + Cfg::O_KT + off);
                const bf16x8 fq = *reinterpret_cast<const bf16x8*>(slot + Cfg::O_QT + off);
                akk = mfma32(fi, fk, akk);     // [s][r] = A_kk[r][s]
                aqk = mfma32(fi, fq, aqk);     // [s][r] = A_qk[r][s]
            }
            // lane (q, r) holds A[r][4q+i]: exactly the 16x16x16 A operand of row r
            *reinterpret_cast<shortx4*>(slot + Cfg::O_AQ + lane * 8) =
                pack4(4 * lq + 0 <= lr ? aqk[0] : 0.f, 4 * lq + 1 <= lr ? aqk[1] : 0.f,
                      4 * lq + 2 <= lr ? aqk[2] : 0.f, 4 * lq + 3 <= lr ? aqk[3] : 0.f);

            // ---- Y = (I + N)^{-1}, N = (diag(beta) A_kk)^T strictly upper ----
            // Column-oriented back substitution; lane (q, c) holds Y[4q+i][c].
            float nv[4], y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                nv[i] = (4 * lq + i < lr) ? bl * akk[i] : 0.f;   // N[4q+i][r] = beta_r A_kk[r][4q+i]
                y[i] = (4 * lq + i == lr) ? 1.f : 0.f;
            }
#define KDA_BACK_STEP(m)                                                   \
    {                                                                      \
        const float ym = rows_from<((m) >> 2)>(y[(m) & 3]);                  \
        _Pragma("unroll") for (int i = 0; i < 4; ++i)                      \
            y[i] = __builtin_fmaf(-row_bcast<(m)>(nv[i]), ym, y[i]);      \
    }
            KDA_BACK_STEP(15) KDA_BACK_STEP(14) KDA_BACK_STEP(13) KDA_BACK_STEP(12)
            KDA_BACK_STEP(11) KDA_BACK_STEP(10) KDA_BACK_STEP(9) KDA_BACK_STEP(8)
            KDA_BACK_STEP(7) KDA_BACK_STEP(6) KDA_BACK_STEP(5) KDA_BACK_STEP(4)
            KDA_BACK_STEP(3) KDA_BACK_STEP(2) KDA_BACK_STEP(1)
#undef KDA_BACK_STEP
            // M'[r][4q+e] = X[r][4q+e] beta[4q+e], X = Y^T: lane (q, r) holds it in y[e]
            *reinterpret_cast<shortx4*>(slot + Cfg::O_MP + lane * 8) =
                pack4(y[0] * b4[0], y[1] * b4[1], y[2] * b4[2], y[3] * b4[3]);

            flag_store(&ready[s], round + 1, lane);
        }
        return;
    }

    // ======================== consumer wave ==================================
    const int w = wave;                      // value columns n0 + 16w .. +15
    floatx4 S[NKT];
    const int64_t sbase = ((int64_t)seq * H + head) * DK * DV + n0 + 16 * w + lr;
    if (s0 != nullptr) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) S[kt][i] = s0[sbase + (int64_t)(16 * kt + 4 * lq + i) * DV];
    } else {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) S[kt] = zero4();
    }
    bool ok = true;
    for (int64_t ci = 0; ci < n_chunks; ++ci) {
        const int s = (int)(ci % kRing);
        const int round = (int)(ci / kRing);
        if (!wait_at_least(&ready[s], round + 1, stop)) { ok = false; break; }
        const char* slot = smem + s * SLOT;

        bf16x8 fk[NKS], fq[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int off = lr * PK + (32 * ks + 8 * lq) * 2;
            fk[ks] = *reinterpret_cast<const bf16x8*>(slot + Cfg::O_KT + off);
            fq[ks] = *reinterpret_cast<const bf16x8*>(slot + Cfg::O_QT + off);
        }
        const int tr_row = 4 * lq + (lr >> 2), tr_col = 4 * (lr & 3);
        const bf16v4 vv = lds_read_tr(slot + Cfg::O_V + tr_row * PV + (16 * w + tr_col) * 2);
        bf16v4 kh[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) kh[kt] = lds_read_tr(slot + Cfg::O_KH + tr_row * PH + (16 * kt + tr_col) * 2);
        const shortx4 mp = *reinterpret_cast<const shortx4*>(slot + Cfg::O_MP + lane * 8);
        const shortx4 aq = *reinterpret_cast<const shortx4*>(slot + Cfg::O_AQ + lane * 8);
        const floatx2 gm = *reinterpret_cast<const floatx2*>(slot + Cfg::O_GM + (lq * 16 + lr) * 8);

        // Z' = Kt S - V  and  O = Qt S   (S as permuted bf16 B operands)
        floatx4 z, oa = zero4();
#pragma unroll
        for (int e = 0; e < 4; ++e) z[e] = -(float)vv[e];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            bf16x8 sb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sb[e] = (__bf16)S[2 * ks][e];
                sb[4 + e] = (__bf16)S[2 * ks + 1][e];
            }
            z = mfma32(fk[ks], sb, z);
            oa = mfma32(fq[ks], sb, oa);
        }
        // U = M' (V - Kt S): the accumulator layout is the 16x16x16 B layout
        const floatx4 u = mfma16(mp, pack4(-z[0], -z[1], -z[2], -z[3]), zero4());
        const shortx4 ub = pack4(u[0], u[1], u[2], u[3]);
        oa = mfma16(aq, ub, oa);
        // S <- diag(e^{G_15}) S + Kh^T U
        state_update<0, NKT>(S, kh, ub, gm);
        flag_add(&released[s], 1, lane);

        const int64_t tok0 = t_begin + ci * 16;
        const int valid = (int)((t_end - tok0) < 16 ? (t_end - tok0) : 16);
        __bf16* op = o + (tok0 * H + head) * DV + n0 + 16 * w + lr;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (4 * lq + i < valid) op[(int64_t)(4 * lq + i) * H * DV] = (__bf16)oa[i];
    }
    if (sT != nullptr) {
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[sbase + (int64_t)(16 * kt + 4 * lq + i) * DV] = ok ? S[kt][i] : nan;
    }
}

template <int DK, int DVS>
hipError_t launch_pipe_t(const void* q, const void* k, const void* v, int64_t stride,
                         const void* g, const void* beta, void* o, const float* s0, float* sT,
                         const int32_t* cu, int num_seqs, int T_len, int H, int DV,
                         hipStream_t s) {
    const int nsplit = DV / DVS;
    const int64_t blocks = (int64_t)num_seqs * H * nsplit;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_pipe_kernel<DK, DVS>), dim3((unsigned)blocks),
                       dim3(PipeCfg<DK, DVS>::THREADS), 0, s, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, stride, (const __bf16*)g, (const __bf16*)beta, (__bf16*)o,
                       s0, sT, cu, num_seqs, T_len, H, DV, nsplit);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_pipe(const void* q, const void* k, const void* v, int64_t stride,
                             const void* g, const void* beta, void* o, const float* s0,
                             float* sT, const int32_t* cu, int num_seqs, int T, int H, int DK,
                             int DV, hipStream_t s) {
    if (DK == 128)
        return launch_pipe_t<128, 64>(q, k, v, stride, g, beta, o, s0, sT, cu, num_seqs, T, H, DV, s);
    return launch_pipe_t<64, 64>(q, k, v, stride, g, beta, o, s0, sT, cu, num_seqs, T, H, DV, s);
}

}  // namespace kda
