// kda_chunk.hip -- chunkwise gated delta rule (KDA prefill) for gfx950.
//
// Method: "Inside Kimi K3" (lei.chat), KDA one-head diagram -- per-channel
// retention alpha_t = exp(g_t) with g_t >= -5, write strength beta_t, a fixed
// dk x dv state, evaluated recurrently across chunks and in parallel within a
// chunk; "Animated Kimi K3 architecture diagram" (github.io), local-memory
// panel -- decay, probe, correct e_t = v_t - Sbar_t^T k_t, write beta_t k_t e_t^T,
// read S_t^T q_t.
//
// Chunk form used here (exact re-association of the token recurrence).  For a
// chunk of C tokens with entering state S0, G_r = sum_{i<=r} g_i per channel:
//   A_kk[r,s] = sum_c k_rc k_sc e^{G_rc - G_sc}  (s < r)
//   A_qk[r,s] = sum_c q_rc k_sc e^{G_rc - G_sc}  (s <= r)
//   M' = (I + diag(beta) A_kk)^{-1} diag(beta)
//   W = M' (K * e^G),  Utilde = M' V,  U = Utilde - W S0
//   O = (Q * e^G) S0 + A_qk U
//   S_C = diag(e^{G_C}) S0 + (K * e^{G_C - G})^T U
//
// Numerics: pairwise factors e^{G_r - G_s} are split into per-row operand
// scalings inside 16-token blocks.  With g >= -5 a block spans at most
// e^{+-80}, inside fp32/bf16 range, so every operand is finite:
//   left  rows r (block i):   k_r F_r, q_r F_r       F_r  = e^{G_r - G_{start i}} <= 1
//   right rows s, same block: k_s / F_s                     <= e^80
//   right rows s, block j<i:  k_s R_s                R_s  = e^{G_{end j} - G_s} <= 1
//   pairs with i - j >= 2 scale the left operand by the block totals between.
// Masked entries are selected away, never multiplied by zero.
//
// Work split: one 256-thread workgroup per (sequence, head, value slice of DVS
// columns); the value columns of S evolve independently, so slices only
// recompute the key-side work.  The fp32 state lives in MFMA accumulators for
// the whole sequence; a bf16 (fp32 in fp32 mode) copy of S^T in LDS feeds the
// S-dependent products.  All contractions run on MFMA (16x16x32 bf16, or
// 16x16x4 fp32 in fp32 mode); the 16x16 diagonal blocks of the unit lower
// triangular inverse are solved by forward substitution in fp32.
#include "kda_device.hpp"
#include "kda_launch.hpp"

// Optional stage timing (profiling builds define KDA_STAGE_PROFILE and the
// array; workgroup 0, thread 0 records the cycles spent in each stage).
#ifdef KDA_STAGE_PROFILE
extern __device__ unsigned long long kda_stage_cycles[8];
#define KDA_PROF_INIT()                                          \
    unsigned long long prof_t_ = __builtin_readcyclecounter();  \
    unsigned long long prof_acc_[8] = {0, 0, 0, 0, 0, 0, 0, 0}
#define KDA_PROF_MARK(i)                                                  \
    do {                                                                  \
        const unsigned long long t_ = __builtin_readcyclecounter();      \
        prof_acc_[i] += t_ - prof_t_;                                     \
        prof_t_ = t_;                                                     \
    } while (0)
#define KDA_PROF_FLUSH()                                                  \
    do {                                                                  \
        if (blockIdx.x == 0 && threadIdx.x == 0)                          \
            for (int i_ = 0; i_ < 8; ++i_) kda_stage_cycles[i_] = prof_acc_[i_]; \
    } while (0)
#else
#define KDA_PROF_INIT() do {} while (0)
#define KDA_PROF_MARK(i) do {} while (0)
#define KDA_PROF_FLUSH() do {} while (0)
#endif

namespace kda {

namespace {

constexpr int kChunkThreads = 256;
constexpr int kLdsLimit = 160 * 1024;

template <typename T, int DK, int DVS, int NB>
struct ChunkCfg {
    static constexpr int C = 16 * NB;
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LDK = DK + PAD;
    static constexpr int LDV = DVS + PAD;
    static constexpr int LDC = C + PAD;
    static constexpr int LDL = C + 4;                    // fp32 L / X rows (16-byte aligned)
    static constexpr int LDY = 20;                       // fp32 16x16 scratch tiles
    static constexpr int NX = (NB - 1) * (NB - 2) / 2;   // block pairs with i - j >= 2
    static constexpr int ES = (int)sizeof(T);
    static constexpr int al(int b) { return (b + 15) / 16 * 16; }
    // region sizes (bytes)
    static constexpr int SZ_ST = al(DVS * LDK * ES);
    static constexpr int SZ_TILE = al(C * LDK * ES);
    static constexpr int SZ_V = al(C * LDV * ES);
    static constexpr int SZ_L = al(C * LDL * 4);
    static constexpr int SZ_KI = SZ_TILE > SZ_L ? SZ_TILE : SZ_L;
    static constexpr int SZ_CC = al(C * LDC * ES);
    static constexpr int SZ_UT = al(DVS * LDC * ES);
    static constexpr int SZ_Y = al((NB > 1 ? NB - 1 : 1) * 16 * LDY * 4);
    static constexpr int SZ_GT = al(NB * DK * 4);
    static constexpr int SZ_DX = al((NX > 0 ? NX : 1) * DK * 4);
    // offsets
    static constexpr int O_ST = 0;
    static constexpr int O_KF = O_ST + SZ_ST;       // K F, then V; U^T reuses both
    static constexpr int O_V = O_KF + SZ_TILE;
    static constexpr int O_QF = O_V + SZ_V;         // Q F
    static constexpr int O_KH = O_QF + SZ_TILE;     // K e^{G_C - G}
    static constexpr int O_KI = O_KH + SZ_TILE;     // K / F, then L and X (fp32)
    static constexpr int O_AQK = O_KI + SZ_KI;
    static constexpr int O_M = O_AQK + SZ_CC;       // M', earlier the inverse's scratch
    static constexpr int O_W = O_M + SZ_CC;         // -W; earlier block log-totals
    static constexpr int O_DX = O_W + SZ_GT;        //   and the pair scales
    static constexpr int O_BETA = O_W + SZ_TILE;
    static constexpr int O_P = O_BETA + al(C * 4);
    static constexpr int O_GAM = O_P + al(NB * DK * 4);
    static constexpr int O_FT = O_GAM + al(DK * 4);
    static constexpr int BYTES = O_FT + al(NB * DK * 4);
    static_assert(SZ_UT <= SZ_TILE + SZ_V, "U^T must fit in the Kf+V region");
    static_assert(SZ_Y <= SZ_CC, "inverse scratch must fit in the M' region");
    static_assert(SZ_GT + SZ_DX <= SZ_TILE, "block totals and pair scales must fit in the W region");
    static constexpr bool fits = BYTES <= kLdsLimit;
};

// C += A B for 16 x 16 fp32 tiles read from LDS (row-major, leading dims lda,
// ldb), on one wave with the 16x16x4 fp32 MFMA.
__device__ __forceinline__ floatx4 mm16_f32(const float* A, int lda, const float* B, int ldb,
                                            floatx4 c, int lr, int lq) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(A[lr * lda + 4 * kk + lq],
                                                 B[(4 * kk + lq) * ldb + lr], c, 0, 0, 0);
    return c;
}

// index of block pair (i, j), i - j >= 2, among the scaled-left pairs
__device__ __forceinline__ constexpr int xidx(int i, int j) { return (i - 2) * (i - 1) / 2 + j; }

template <typename T, int DK, int DVS, int NB>
__global__ void __launch_bounds__(kChunkThreads)
chunk_kernel(const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
             int64_t stride, const T* __restrict__ g, const T* __restrict__ beta,
             T* __restrict__ o, const float* s0, float* sT, const int32_t* __restrict__ cu,
             int num_seqs, int T_len, int H, int DV, int nsplit) {
    using Cfg = ChunkCfg<T, DK, DVS, NB>;
    using MM = Mma<T>;
    using frag = typename MM::frag;
    constexpr int C = Cfg::C, LDK = Cfg::LDK, LDV = Cfg::LDV, LDC = Cfg::LDC, LDL = Cfg::LDL;
    constexpr int LDY = Cfg::LDY;
    constexpr int KPL = MM::KPL, KI = MM::KI;
    constexpr int NT = DVS / 16;            // value tiles
    constexpr int CTW = DK / 16 / 4;        // key tiles per wave (state update, W)
    constexpr int WPR = 4 / NB;             // waves per row block (U, O)
    constexpr int NTW = (NT + WPR - 1) / WPR;   // value tiles per wave (U, O)
    static_assert(DK % 64 == 0, "tile split");
    static_assert(C % KI == 0, "chunk must be a multiple of the MFMA depth");

    __shared__ __attribute__((aligned(16))) char smem[Cfg::BYTES];
    T* sST = reinterpret_cast<T*>(smem + Cfg::O_ST);
    T* sKf = reinterpret_cast<T*>(smem + Cfg::O_KF);
    T* sV = reinterpret_cast<T*>(smem + Cfg::O_V);
    T* sUT = reinterpret_cast<T*>(smem + Cfg::O_KF);
    T* sQf = reinterpret_cast<T*>(smem + Cfg::O_QF);
    T* sKh = reinterpret_cast<T*>(smem + Cfg::O_KH);
    T* sKi = reinterpret_cast<T*>(smem + Cfg::O_KI);
    float* sL = reinterpret_cast<float*>(smem + Cfg::O_KI);
    T* sAqk = reinterpret_cast<T*>(smem + Cfg::O_AQK);
    T* sM = reinterpret_cast<T*>(smem + Cfg::O_M);
    float* sYb = reinterpret_cast<float*>(smem + Cfg::O_M);
    T* sW = reinterpret_cast<T*>(smem + Cfg::O_W);
    float* sGt = reinterpret_cast<float*>(smem + Cfg::O_W);
    float* sBeta = reinterpret_cast<float*>(smem + Cfg::O_BETA);
    float* sP = reinterpret_cast<float*>(smem + Cfg::O_P);
    float* sGam = reinterpret_cast<float*>(smem + Cfg::O_GAM);
    float* sDx = reinterpret_cast<float*>(smem + Cfg::O_DX);
    float* sFt = reinterpret_cast<float*>(smem + Cfg::O_FT);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lr = lane & 15;        // fragment row / column
    const int lq = lane >> 4;        // fragment k-group

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
    const int64_t n_chunks = (t_end - t_begin + C - 1) / C;

    // ---- state: wave w owns key tiles [w*CTW, (w+1)*CTW) x all value tiles --
    floatx4 S[CTW][NT];
    if (s0 != nullptr) {
        const float* s0p = s0 + ((int64_t)seq * H + head) * DK * DV;
#pragma unroll
        for (int j = 0; j < CTW; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[j][nt][i] = s0p[(int64_t)((wave * CTW + j) * 16 + 4 * lq + i) * DV + n0 +
                                      nt * 16 + lr];
    } else {
#pragma unroll
        for (int j = 0; j < CTW; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) S[j][nt] = zero4();
    }
    auto write_state_lds = [&]() {
#pragma unroll
        for (int j = 0; j < CTW; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int c = (wave * CTW + j) * 16 + 4 * lq;
                const int n = nt * 16 + lr;
                T* p = sST + n * LDK + c;
#pragma unroll
                for (int i = 0; i < 4; ++i) p[i] = from_f<T>(S[j][nt][i]);
            }
    };
    write_state_lds();
    // A_qk blocks above the diagonal are never written: zero them once
    for (int e = tid; e < C * C; e += kChunkThreads) sAqk[(e / C) * LDC + (e % C)] = from_f<T>(0.f);

    // ---- stage-1 thread layout: CPT channels x 16 tokens of one block ------
    constexpr int CPT = (DK * NB >= 512) ? 2 : 1;
    constexpr int TPB = DK / CPT;
    const bool s1 = tid < NB * TPB;
    const int blk = s1 ? tid / TPB : 0;
    const int c1 = (tid % TPB) * CPT;
    using RawC = typename RawVec<T, CPT>::type;
    using Raw8 = typename RawVec<T, 8>::type;
    constexpr int VROWS = DVS / 8;                       // 8-column groups per value row
    constexpr int VPT = (C * VROWS + kChunkThreads - 1) / kChunkThreads;

    // U/O tile ownership
    const int rbw = wave / WPR;             // row block of this wave
    const int ntb = wave % WPR;             // first value tile, step WPR

    // ---- one chunk ahead: raw inputs held in registers ---------------------
    // Addresses are clamped to the last valid token so that every load is
    // issued unconditionally; rows past the sequence end are zeroed on use.
    RawC pg[16], pk[16], pq[16];
    Raw8 pv[VPT];
    T pb;
    auto issue_loads = [&](int64_t tok0n, int validn) {
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int r = blk * 16 + t;
            const int64_t tok = tok0n + (r < validn ? r : validn - 1);
            pg[t] = *reinterpret_cast<const RawC*>(g + (tok * H + head) * DK + c1);
            pk[t] = *reinterpret_cast<const RawC*>(k + tok * stride + (int64_t)head * DK + c1);
            pq[t] = *reinterpret_cast<const RawC*>(q + tok * stride + (int64_t)head * DK + c1);
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            int e = tid + u * kChunkThreads;
            e = e < C * VROWS ? e : C * VROWS - 1;
            const int r = e / VROWS;
            const int64_t tok = tok0n + (r < validn ? r : validn - 1);
            pv[u] = *reinterpret_cast<const Raw8*>(v + tok * stride + (int64_t)head * DV + n0 +
                                                  (e % VROWS) * 8);
        }
        pb = beta[(tok0n + (tid < validn ? tid : validn - 1)) * H + head];
    };
    if (n_chunks > 0) {
        const int64_t len = t_end - t_begin;
        issue_loads(t_begin, (int)(len < C ? len : C));
    }
    __syncthreads();
    KDA_PROF_INIT();

    for (int64_t ci = 0; ci < n_chunks; ++ci) {
        const int64_t tok0 = t_begin + ci * C;
        const int valid = (int)((t_end - tok0) < C ? (t_end - tok0) : C);

        // ================= stage 1: decay factors and operand tiles ==========
        // pass A: per (block, channel) log-decay totals (log2 units)
        if (s1) {
            float gs[CPT];
#pragma unroll
            for (int j = 0; j < CPT; ++j) gs[j] = 0.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const bool ok = blk * 16 + t < valid;
                float gv[CPT];
                RawVec<T, CPT>::unpack(pg[t], gv);
#pragma unroll
                for (int j = 0; j < CPT; ++j) gs[j] += ok ? clamp_log_decay(gv[j]) * kLog2e : 0.f;
            }
#pragma unroll
            for (int j = 0; j < CPT; ++j) sGt[blk * DK + c1 + j] = gs[j];
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int e = tid + u * kChunkThreads;
            if (e < C * VROWS) {
                const int r = e / VROWS;
                float vv[8];
                RawVec<T, 8>::unpack(pv[u], vv);
                if (r >= valid) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) vv[i] = 0.f;
                }
                store8(sV + r * LDV + (e % VROWS) * 8, vv);
            }
        }
        if (tid < C) sBeta[tid] = tid < valid ? to_f(pb) : 0.f;
        __syncthreads();
        KDA_PROF_MARK(0);

        // pass B: block tables, then one sweep over the block's 16 tokens with
        // G the local cumulative log-decay, F = 2^G, 1/F = 2^-G
        if (s1) {
            float Fb[CPT], Eb[CPT];
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const int c = c1 + j;
                float Ft[NB];
#pragma unroll
                for (int m = 0; m < NB; ++m) Ft[m] = fast_exp2(sGt[m * DK + c]);
                float P = 1.f, E = 1.f, F0 = 1.f;
#pragma unroll
                for (int m = 0; m < NB; ++m) {
                    if (m < blk) P *= Ft[m];
                    if (m > blk) E *= Ft[m];
                    if (m == blk) F0 = Ft[m];
                }
                Fb[j] = F0;
                Eb[j] = E;
                sP[blk * DK + c] = P;
                sFt[blk * DK + c] = F0;
                if (blk == 0) {
                    float gam = 1.f;
#pragma unroll
                    for (int m = 0; m < NB; ++m) gam *= Ft[m];
                    sGam[c] = gam;
#pragma unroll
                    for (int i2 = 2; i2 < NB; ++i2)
#pragma unroll
                        for (int j2 = 0; j2 + 2 <= i2; ++j2) {
                            float dx = 1.f;
#pragma unroll
                            for (int m = j2 + 1; m < i2; ++m) dx *= Ft[m];
                            sDx[xidx(i2, j2) * DK + c] = dx;
                        }
                }
            }
            float G[CPT];
#pragma unroll
            for (int j = 0; j < CPT; ++j) G[j] = 0.f;
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const int r = blk * 16 + t;
                const bool ok = r < valid;
                float gv[CPT], kv[CPT], qv[CPT], kf[CPT], qf[CPT], ki[CPT], kh[CPT];
                RawVec<T, CPT>::unpack(pg[t], gv);
                RawVec<T, CPT>::unpack(pk[t], kv);
                RawVec<T, CPT>::unpack(pq[t], qv);
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    G[j] += ok ? clamp_log_decay(gv[j]) * kLog2e : 0.f;
                    const float F = fast_exp2(G[j]);
                    const float Fi = fast_exp2(-G[j]);
                    const float kk = ok ? kv[j] : 0.f;
                    const float qq = ok ? qv[j] : 0.f;
                    kf[j] = kk * F;
                    qf[j] = qq * F;
                    ki[j] = kk * Fi;
                    kh[j] = (ki[j] * Fb[j]) * Eb[j];   // k e^{G_C - G_r}: both factors <= 1 in turn
                }
                RawVec<T, CPT>::store(sKf + r * LDK + c1, kf);
                RawVec<T, CPT>::store(sQf + r * LDK + c1, qf);
                RawVec<T, CPT>::store(sKi + r * LDK + c1, ki);
                RawVec<T, CPT>::store(sKh + r * LDK + c1, kh);
            }
        }
        __syncthreads();
        // the next chunk's inputs stream in while this chunk computes
        if (ci + 1 < n_chunks) {
            const int64_t rem = t_end - (tok0 + C);
            issue_loads(tok0 + C, (int)(rem < C ? rem : C));
        }
        KDA_PROF_MARK(1);

        // ================= stage 2: A_kk, A_qk tiles (MFMA) ==================
        // Wave w computes one kind (A_kk for even w, A_qk for odd w) for row
        // blocks {w/2, NB-1-w/2} (NB = 4) or {w/2} (NB = 2): five tiles each.
        // Right operand: same block -> k/F; earlier block j -> (k/F) * F_j.
        // Left operand scaled by the block totals strictly between j and i.
        constexpr int RPW = NB >= 4 ? 2 : 1;
        constexpr int KS = DK / KI;
        const int kind = wave & 1;
        const bool s2 = NB > 1 || wave < 2;
        floatx4 accA[RPW][NB];
#pragma unroll
        for (int sl = 0; sl < RPW; ++sl) {
            const int i = sl == 0 ? (wave >> 1) : NB - 1 - (wave >> 1);
            const T* left = (kind ? sQf : sKf) + (i * 16 + lr) * LDK + KPL * lq;
            frag la[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) la[ks] = MM::load(left + ks * KI);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                accA[sl][j] = zero4();
                if (!s2 || j > i) continue;
                const T* right = sKi + (j * 16 + lr) * LDK + KPL * lq;
                const float* fr = sFt + j * DK + KPL * lq;
                const float* dx = sDx + (i - j >= 2 ? xidx(i, j) : 0) * DK + KPL * lq;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    frag a = la[ks];
                    if (i - j >= 2) {
                        float av[KPL];
                        MM::unpack(a, av);
#pragma unroll
                        for (int e = 0; e < KPL; ++e) av[e] *= dx[ks * KI + e];
                        a = MM::pack(av);
                    }
                    frag b = MM::load(right + ks * KI);
                    if (j < i) {
                        float bv[KPL];
                        MM::unpack(b, bv);
#pragma unroll
                        for (int e = 0; e < KPL; ++e) bv[e] *= fr[ks * KI + e];
                        b = MM::pack(bv);
                    }
                    accA[sl][j] = MM::mma(a, b, accA[sl][j]);
                }
            }
        }
        __syncthreads();   // every read of K/F done before L overwrites it
        if (s2) {
#pragma unroll
            for (int sl = 0; sl < RPW; ++sl) {
                const int i = sl == 0 ? (wave >> 1) : NB - 1 - (wave >> 1);
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    if (j > i) continue;
#pragma unroll
                    for (int ii = 0; ii < 4; ++ii) {
                        const int rl = 4 * lq + ii, sl2 = lr;
                        const int r = i * 16 + rl, s = j * 16 + sl2;
                        if (kind == 0) {
                            const bool keep = (j < i) || (sl2 < rl);
                            sL[r * LDL + s] = keep ? sBeta[r] * accA[sl][j][ii] : 0.f;
                        } else {
                            const bool keep = (j < i) || (sl2 <= rl);
                            sAqk[r * LDC + s] = from_f<T>(keep ? accA[sl][j][ii] : 0.f);
                        }
                    }
                }
            }
        }
        __syncthreads();
        KDA_PROF_MARK(2);

        // ================= stage 3: X = (I + L)^{-1}, M' = X diag(beta) =====
        // Diagonal 16x16 blocks by forward substitution (wave b, lane = column),
        // updating the remaining rows after each solved row.
        if (wave < NB && lane < 16) {
            const int b0 = wave * 16;
            const int cc = lane;
            float acc[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = (r == cc) ? 1.f : 0.f;
#pragma unroll
            for (int m = 0; m < 16; ++m) {
                const float xm = acc[m];
#pragma unroll
                for (int r = m + 1; r < 16; ++r) acc[r] -= sL[(b0 + r) * LDL + b0 + m] * xm;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sL[(b0 + r) * LDL + b0 + cc] = acc[r];
        }
        __syncthreads();
        // Off-diagonal blocks by block rows: X_ij = -X_ii sum_{m=j}^{i-1} L_im X_mj,
        // wave j computing the (i, j) tile with fp32 MFMA.
#pragma unroll
        for (int i = 1; i < NB; ++i) {
            float* yw = sYb + wave * 16 * LDY;
            if (wave < i) {
                floatx4 y = zero4();
                for (int m = wave; m < i; ++m)
                    y = mm16_f32(sL + (16 * i) * LDL + 16 * m, LDL, sL + (16 * m) * LDL + 16 * wave,
                                 LDL, y, lr, lq);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) yw[(4 * lq + ii) * LDY + lr] = y[ii];
            }
            __syncthreads();
            if (wave < i) {
                const floatx4 x = mm16_f32(sL + (16 * i) * LDL + 16 * i, LDL, yw, LDY, zero4(), lr, lq);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) sL[(16 * i + 4 * lq + ii) * LDL + 16 * wave + lr] = -x[ii];
            }
            __syncthreads();
        }
        {
            constexpr int PER = C * C / kChunkThreads > 0 ? C * C / kChunkThreads : 1;
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                const int e = tid + u * kChunkThreads;
                if (e < C * C) {
                    const int r = e / C, s = e % C;
                    const float bs = sBeta[s];
                    float val = s < r ? sL[r * LDL + s] * bs : 0.f;
                    val = s == r ? bs : val;
                    sM[r * LDC + s] = from_f<T>(val);
                }
            }
        }
        __syncthreads();
        KDA_PROF_MARK(3);

        // ================= stage 4: -W = -M'(K e^G) and Utilde = M'V ========
        // W tiles: wave owns key tiles (CTW of them) for all row blocks
#pragma unroll
        for (int jc = 0; jc < CTW; ++jc) {
            const int ct = wave * CTW + jc;
            floatx4 accW[NB];
#pragma unroll
            for (int rb = 0; rb < NB; ++rb) accW[rb] = zero4();
#pragma unroll
            for (int ks = 0; ks < C / KI; ++ks) {
                // B[k = s][n = c] = Kf[s][c] * P[block(s)][c]  (transposed read)
                const int sb = ks * KI + KPL * lq;
                const int c = ct * 16 + lr;
                const float pf = sP[(sb / 16) * DK + c];
                float bv[KPL];
#pragma unroll
                for (int e = 0; e < KPL; ++e) bv[e] = to_f(sKf[(sb + e) * LDK + c]) * pf;
                const frag b = MM::pack(bv);
#pragma unroll
                for (int rb = 0; rb < NB; ++rb) {
                    if (ks * KI < 16 * (rb + 1)) {
                        const frag a = MM::load(sM + (rb * 16 + lr) * LDC + sb);
                        accW[rb] = MM::mma(a, b, accW[rb]);
                    }
                }
            }
#pragma unroll
            for (int rb = 0; rb < NB; ++rb)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii)
                    sW[(rb * 16 + 4 * lq + ii) * LDK + ct * 16 + lr] = from_f<T>(-accW[rb][ii]);
        }
        // Utilde tiles: row block rbw, value tiles ntb + WPR * j
        floatx4 accU[NTW], accO[NTW];
#pragma unroll
        for (int j = 0; j < NTW; ++j) { accU[j] = zero4(); accO[j] = zero4(); }
#pragma unroll
        for (int ks = 0; ks < C / KI; ++ks) {
            if (ks * KI < 16 * (rbw + 1)) {
                const int sb = ks * KI + KPL * lq;
                const frag a = MM::load(sM + (rbw * 16 + lr) * LDC + sb);
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    if (ntb + WPR * j >= NT) continue;
                    const int n = (ntb + WPR * j) * 16 + lr;
                    float bv[KPL];
#pragma unroll
                    for (int e = 0; e < KPL; ++e) bv[e] = to_f(sV[(sb + e) * LDV + n]);
                    accU[j] = MM::mma(a, MM::pack(bv), accU[j]);
                }
            }
        }
        __syncthreads();   // -W complete; Kf, V, M' no longer read
        KDA_PROF_MARK(4);

        // ================= stage 5: U += (-W) S0,  O = (Q e^G) S0 ===========
#pragma unroll
        for (int k0 = 0; k0 < DK; k0 += KI) {
            const int kk = k0 + KPL * lq;
            const frag aw = MM::load(sW + (rbw * 16 + lr) * LDK + kk);
            float qv[KPL];
            MM::unpack(MM::load(sQf + (rbw * 16 + lr) * LDK + kk), qv);
#pragma unroll
            for (int e = 0; e < KPL; ++e) qv[e] *= sP[rbw * DK + kk + e];
            const frag aq = MM::pack(qv);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                if (ntb + WPR * j >= NT) continue;
                const int n = (ntb + WPR * j) * 16 + lr;
                const frag b = MM::load(sST + n * LDK + kk);
                accU[j] = MM::mma(aw, b, accU[j]);
                accO[j] = MM::mma(aq, b, accO[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            if (ntb + WPR * j >= NT) continue;
            const int n = (ntb + WPR * j) * 16 + lr;
            T* p = sUT + n * LDC + rbw * 16 + 4 * lq;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) p[ii] = from_f<T>(accU[j][ii]);
        }
        __syncthreads();
        KDA_PROF_MARK(5);

        // ================= stage 6: O += A_qk U;  S = diag(e^{G_C}) S + K^T U
#pragma unroll
        for (int ks = 0; ks < C / KI; ++ks) {
            if (ks * KI < 16 * (rbw + 1)) {
                const int sb = ks * KI + KPL * lq;
                const frag a = MM::load(sAqk + (rbw * 16 + lr) * LDC + sb);
#pragma unroll
                for (int j = 0; j < NTW; ++j) {
                    if (ntb + WPR * j >= NT) continue;
                    const int n = (ntb + WPR * j) * 16 + lr;
                    accO[j] = MM::mma(a, MM::load(sUT + n * LDC + sb), accO[j]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            if (ntb + WPR * j >= NT) continue;
            const int n = n0 + (ntb + WPR * j) * 16 + lr;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const int r = rbw * 16 + 4 * lq + ii;
                if (r < valid) o[((tok0 + r) * H + head) * DV + n] = from_f<T>(accO[j][ii]);
            }
        }
#pragma unroll
        for (int jc = 0; jc < CTW; ++jc) {
            const int ct = wave * CTW + jc;
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
                const float gm = sGam[ct * 16 + 4 * lq + ii];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) S[jc][nt][ii] *= gm;
            }
#pragma unroll
            for (int ks = 0; ks < C / KI; ++ks) {
                // A[m = c][k = s] = Khat[s][c]  (transposed read)
                const int sb = ks * KI + KPL * lq;
                const int c = ct * 16 + lr;
                float av[KPL];
#pragma unroll
                for (int e = 0; e < KPL; ++e) av[e] = to_f(sKh[(sb + e) * LDK + c]);
                const frag a = MM::pack(av);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    S[jc][nt] = MM::mma(a, MM::load(sUT + (nt * 16 + lr) * LDC + sb), S[jc][nt]);
            }
        }
        write_state_lds();
        __syncthreads();
        KDA_PROF_MARK(6);
    }
    KDA_PROF_FLUSH();

    // ---- final state ---------------------------------------------------------
    if (sT) {
        float* sp = sT + ((int64_t)seq * H + head) * DK * DV;
#pragma unroll
        for (int j = 0; j < CTW; ++j)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = (wave * CTW + j) * 16 + 4 * lq + i;
                    const int n = n0 + nt * 16 + lr;
                    sp[(int64_t)c * DV + n] = S[j][nt][i];
                }
    }
}

template <typename T, int DK, int DVS, int NB>
hipError_t launch_chunk_t(const void* q, const void* k, const void* v, int64_t stride,
                          const void* g, const void* beta, void* o, const float* s0, float* sT,
                          const int32_t* cu, int num_seqs, int T_len, int H, int DV,
                          hipStream_t s) {
    static_assert(ChunkCfg<T, DK, DVS, NB>::fits, "LDS budget exceeded");
    const int nsplit = DV / DVS;
    const int64_t blocks = (int64_t)num_seqs * H * nsplit;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((chunk_kernel<T, DK, DVS, NB>), dim3((unsigned)blocks),
                       dim3(kChunkThreads), 0, s, (const T*)q, (const T*)k, (const T*)v, stride,
                       (const T*)g, (const T*)beta, (T*)o, s0, sT, cu, num_seqs, T_len, H, DV, nsplit);
    return hipGetLastError();
}

}  // namespace

// Variants compiled: bf16 with chunk 32/64 and value slices of 64/128 columns;
// fp32 with chunk 16/32/64 and 32-column slices (fp32 DK = 128 at chunk 64
// exceeds the LDS budget).
ChunkPlan plan_chunk(int dtype, int DK, int DV, int chunk, int64_t n_chains) {
    ChunkPlan p{0, 0, false};
    if (chunk != 16 && chunk != 32 && chunk != 64) return p;
    p.nb = chunk / 16;
    if (dtype == 1) {
        if (chunk == 16) return p;
        // fewer chains than CUs: split the value columns to fill the chip
        p.dvs = (DV == 128 && n_chains < 256) ? 64 : DV;
        p.ok = true;
    } else {
        if (DK == 128 && chunk == 64) return p;
        p.dvs = 32;
        p.ok = true;
    }
    return p;
}

#define KDA_CHUNK_CASE(T_, DK_, DVS_, NB_)                                                      \
    if (DK == DK_ && plan.dvs == DVS_ && plan.nb == NB_)                                        \
        return launch_chunk_t<T_, DK_, DVS_, NB_>(q, k, v, stride, g, beta, o, s0, sT, cu,      \
                                                  num_seqs, T, H, DV, s);

hipError_t launch_chunk(const ChunkPlan& plan, const void* q, const void* k, const void* v,
                        int64_t stride, const void* g, const void* beta, void* o,
                        const float* s0, float* sT, const int32_t* cu, int num_seqs, int T,
                        int H, int DK, int DV, int dtype, hipStream_t s) {
    if (dtype == 1) {
        KDA_CHUNK_CASE(__bf16, 128, 128, 4)
        KDA_CHUNK_CASE(__bf16, 128, 64, 4)
        KDA_CHUNK_CASE(__bf16, 64, 128, 4)
        KDA_CHUNK_CASE(__bf16, 64, 64, 4)
        KDA_CHUNK_CASE(__bf16, 128, 128, 2)
        KDA_CHUNK_CASE(__bf16, 128, 64, 2)
        KDA_CHUNK_CASE(__bf16, 64, 128, 2)
        KDA_CHUNK_CASE(__bf16, 64, 64, 2)
    } else {
        KDA_CHUNK_CASE(float, 64, 32, 4)
        KDA_CHUNK_CASE(float, 64, 32, 2)
        KDA_CHUNK_CASE(float, 64, 32, 1)
        KDA_CHUNK_CASE(float, 128, 32, 2)
        KDA_CHUNK_CASE(float, 128, 32, 1)
    }
    return hipErrorNotSupported;
}

#undef KDA_CHUNK_CASE

}  // namespace kda
