// kda_mla.hip -- one decode step of gated multi-head latent attention over
// the latent cache (gfx950).
//
// "Inside Kimi K3" (lei.chat), gated multi-head latent attention diagram: the
// KV down-projection c_t = W_c x_t keeps a 512-value latent per token (the
// cache); learned up-projections rebuild keys and values of 128 per head for
// 96 heads (no positional encoding); the new token's query takes a causal
// softmax over all cached tokens; the head output is gated by a full-rank
// sigmoid sigma(W_g x_t).
//
// The key up-projection is absorbed into the query, q'_h = W_uk[h]^T q_h
// (512 wide), so a score is q'_h . c_i and all heads read the same latent: one
// pass over the cache serves every head.  The value up-projection is applied
// after the softmax-weighted sum of latents, u_h = sum_i p_hi c_i, as
// o_h = W_uv[h] u_h.  Three kernels, all on 16x16x32 bf16 MFMA:
//  1. absorb: q' = q W_uk[h] in bf16, scaled by scale * log2(e) (the softmax
//     runs in base 2);
//  2. attention over a range of the cache, all heads at once, per
//     (sequence, split): S^T = C Q'^T and U += P C with a running (online)
//     softmax, partial m, l, U to the workspace;
//  3. combine the splits, o = u W_uv[h]^T, y = o * sigmoid(gate).
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda.h"
#include "kda_device.hpp"
#include "kda_launch.hpp"

// Device scratch of the decode entry point that allocates nothing: q' and the
// split partials of one call, at most KDA_MLA_NOALLOC_MAX_BYTES.  Each GPU
// that runs the library holds its own copy until the process ends.  In host
// code this name is only a handle: the device address comes from
// hipGetSymbolAddress (mla_scratch below).
static __device__ __align__(256) char scratch[KDA_MLA_NOALLOC_MAX_BYTES];

namespace kda {

namespace {

constexpr int kR = 512;            // latent width
constexpr int kDh = 128;           // key / value width per head
constexpr int kTL = 32;            // cached tokens per attention tile

typedef __bf16 bf16v4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((address_space(3))) bf16v4* lds_bf16v4_ptr;

__device__ __forceinline__ floatx4 mla_mfma32(bf16x8 a, bf16x8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Transposed 8-byte LDS read: lane j of each 16-lane group gives the address
// of row k0 + j/4, columns n0 + 4(j%4) .. +3; lane n receives column n0 + n,
// rows k0 .. k0+3.
__device__ __forceinline__ bf16v4 mla_read_tr(const __bf16* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16v4_ptr)(p));
}

// One row of 64 x 16 bytes from memory into LDS: lane l's 16 bytes at g land
// at lds_row + 16 l.  Issued as asm: the compiler does not count these loads,
// so it adds no wait for them before the LDS reads; the caller waits
// (vmcnt, then a barrier) before any wave reads the row.  lds_row is
// wave-uniform; M0 carries it (one wait state before the load reads it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_row_load(const char* lds_row, const void* g) {
    const uint32_t m = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)lds_row;
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(m), "v"(g)
                 : "memory", "m0");
}
#pragma clang diagnostic pop
// Wait until at most n of this wave's loads are in flight.
template <int n>
__device__ __forceinline__ void wait_loads() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(n) : "memory");
}
// ---- 1. absorb: q'[b][h][r] = s * sum_d q[b][h][d] W_uk[h][d][r] ----------
// Workgroup (head h, 32 sequences), 4 waves: a 32 x 512 x 128 product on
// 16x16x32 MFMA.  W_uk[h] (128 x 512) is staged in LDS and read as the B
// operand by transposed reads (K = d runs down its columns); q rows are the
// A operand, straight from memory.  Wave w owns latent columns 128 w .. +127.
constexpr int kGS = 32;            // sequences per absorb / combine workgroup
constexpr int kWP = kR * 2 + 16;   // LDS row pitch (bytes) of W_uk[h]: 4 banks between rows
__global__ void __launch_bounds__(256)
mla_absorb_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ w_uk,
                  __bf16* __restrict__ qp, int B, int H, float s) {
    __shared__ __attribute__((aligned(16))) char sW[kDh * kWP];
    const int h = blockIdx.x, b0 = blockIdx.y * kGS, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lq = lane >> 4;
    // all 32 loads of this thread's share of W_uk[h] in flight at once
    const __bf16* wh = w_uk + (int64_t)h * kDh * kR;
    constexpr int kWL = kDh * (kR / 8) / 256;
    bf16x8 wt[kWL];
#pragma unroll
    for (int j = 0; j < kWL; ++j) {
        const int i = tid + 256 * j, d = i / (kR / 8), c8 = i % (kR / 8);
        wt[j] = *reinterpret_cast<const bf16x8*>(wh + (int64_t)d * kR + 8 * c8);
    }
#pragma unroll
    for (int j = 0; j < kWL; ++j) {
        const int i = tid + 256 * j, d = i / (kR / 8), c8 = i % (kR / 8);
        *reinterpret_cast<bf16x8*>(sW + d * kWP + 16 * c8) = wt[j];
    }
    // A operands: rows b0 + 16 mt + lr (rows past B read row B - 1, never stored)
    bf16x8 qa[2][kDh / 32];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        int bb = b0 + 16 * mt + lr;
        bb = bb < B ? bb : B - 1;
        const __bf16* qr = q + ((int64_t)bb * H + h) * kDh + 8 * lq;
#pragma unroll
        for (int ks = 0; ks < kDh / 32; ++ks) qa[mt][ks] = *reinterpret_cast<const bf16x8*>(qr + 32 * ks);
    }
    __syncthreads();
    floatx4 acc[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDh / 32; ++ks)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            // B operand: rows d = 32 ks + 8q .. +7 of column 128 w + 16 nt + lane
            const int col = 128 * wave + 16 * nt + 4 * (lr & 3);
            const bf16v4 lo = mla_read_tr(reinterpret_cast<const __bf16*>(sW + (32 * ks + 8 * lq + (lr >> 2)) * kWP + col * 2));
            const bf16v4 hi = mla_read_tr(reinterpret_cast<const __bf16*>(sW + (32 * ks + 8 * lq + 4 + (lr >> 2)) * kWP + col * 2));
            const bf16x8 wb = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc[0][nt] = mla_mfma32(qa[0][ks], wb, acc[0][nt]);
            acc[1][nt] = mla_mfma32(qa[1][ks], wb, acc[1][nt]);
        }
    // lane (q, c): sequences b0 + 16 mt + 4q + i, latent column 128 w + 16 nt + c
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int bb = b0 + 16 * mt + 4 * lq + i;
            if (bb < B) {
                __bf16* out = qp + ((int64_t)bb * H + h) * kR + 128 * wave + lr;
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) out[16 * nt] = (__bf16)(acc[mt][nt][i] * s);
            }
        }
}

// ---- 2. attention over one range of the cache, all heads ------------------
// Workgroup (split sp, sequence b), 2 HT waves.  Wave w works for head tile
// ht = w / 2 (16 heads) and half h = w % 2: it holds the Q' rows of its heads
// for latent channels 256 h .. +255 in registers, and owns latent columns
// 256 h .. +255 of U.  Per tile of 32 cached tokens:
//  * each wave forms its half of the scores over its 256 channels; the two
//    halves are summed through LDS (x + y in one wave, y + x in the other:
//    both hold bitwise the same scores, hence the same softmax);
//  * U += P C over the wave's columns.
// Scores are formed transposed, S^T = C Q'^T (tokens x heads): lane (q, c)
// holds head c at tokens 4q .. 4q+3 of each 16-token half of the tile.  Read
// as the A operand of U += P C (rows = heads), those eight values sit at
// k = 8q .. 8q+7, so the K index of that product runs over the tokens in the
// order {4q .. 4q+3, 16+4q .. 16+4q+3}; the B operand (the tile as [token]
// [column]) is read in the same order by two transposed reads.  Softmax: a
// running max per head (base 2: q' carries log2 e); row sums stay per lane
// until the end.
// Cache tiles go straight from memory into a ring of three LDS stages (global
// loads with an LDS destination, issued by up to eight loader waves, one 1 KB
// row per instruction): while tile t is read, tile t+1 lands and tile t+2 is
// issued.  One barrier per tile.
constexpr int kCP = kR * 2 + 32;            // LDS row pitch (bytes) of a cache tile: 8 banks between rows
constexpr int kStages = 3;                  // LDS stages of cache tiles: t, t+1 and t+2 in flight
constexpr float kLazyMax = 8.f;             // growth of a head's max (base 2) before a rescale

template <int HT>
__global__ void __launch_bounds__(128 * HT)
mla_attn_kernel(const __bf16* __restrict__ qp, const __bf16* __restrict__ cache,
                const int32_t* __restrict__ lengths, float* __restrict__ part_ml,
                float* __restrict__ part_u, int Lmax, int nsplit) {
    constexpr int H = 16 * HT, NW = 2 * HT;
    constexpr int NL = NW >= 8 ? 8 : (NW >= 4 ? 4 : 2);   // loader waves
    constexpr int RPL = kTL / NL;                        // rows per loader wave and tile
    __shared__ __attribute__((aligned(16))) char sC[kStages][kTL * kCP];
    __shared__ __attribute__((aligned(16))) floatx4 sX[2][NW][2][64];   // partial scores, by tile parity
    __shared__ __attribute__((aligned(16))) float sA[NW][16];        // rescale factors

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lr = lane & 15, lq = lane >> 4;
    const int ht = wave >> 1, hf = wave & 1;
    const int sp = blockIdx.x, b = blockIdx.y;
    int L = lengths[b];
    L = L < 1 ? 1 : (L > Lmax ? Lmax : L);
    const int tiles = (L + kTL - 1) / kTL;
    const int tps = (tiles + nsplit - 1) / nsplit;
    const int t_lo = sp * tps;
    const int t_hi = t_lo + tps < tiles ? t_lo + tps : tiles;

    // Q'^T as B operands over this wave's channels (lane (q, c): head
    // ht*16 + c, k = 256 hf + 32 ks + 8q .. +7)
    const __bf16* qrow = qp + ((int64_t)b * H + ht * 16 + lr) * kR + 256 * hf + 8 * lq;
    bf16x8 qb[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
    // complete them here: otherwise the tile loop's first products wait on
    // the memory counter, which then also holds back the cache prefetch
    asm volatile("" ::"v"(qb[0]), "v"(qb[1]), "v"(qb[2]), "v"(qb[3]), "v"(qb[4]), "v"(qb[5]),
                 "v"(qb[6]), "v"(qb[7]));

    // Loader wave w (< NL) loads rows w + NL j of a tile, 16 bytes per lane;
    // rows past the length repeat the last valid row (their scores are
    // masked), so every load is in bounds.  Tiles past the range are not
    // loaded; the waits count only the tiles issued.
    const __bf16* cb = cache + (int64_t)b * Lmax * kR + 8 * lane;
    const bool loader = wave < NL;
    auto issue = [&](int t) {
        if (loader && t < t_hi) {
            const char* st = sC[(t - t_lo) % kStages];
#pragma unroll
            for (int j = 0; j < RPL; ++j) {
                const int row = wave + NL * j;
                int tok = t * kTL + row;
                tok = tok < L ? tok : L - 1;
                lds_row_load(st + row * kCP, cb + (int64_t)tok * kR);
            }
        }
    };
    float m_ref = -__builtin_inff();   // per head (lane's c), identical over q
    float l_part = 0.f;                // this lane's share of the row sum
    floatx4 U[16];                     // lane (q, c): heads 4q+i, column 256 hf + 16 j + c
#pragma unroll
    for (int j = 0; j < 16; ++j) U[j] = floatx4{0.f, 0.f, 0.f, 0.f};

    // One barrier per tile.  Before it each wave has written its partial
    // scores of tile t (double-buffered by tile parity) and waited for its
    // own rows of tile t+1; after it tile t+1 is in LDS for everyone, every
    // wave is done with tile t-1's stage, which then takes tile t+2
    // this wave's half of S^T = C Q'^T for the two 16-token halves of the
    // tile on stage st
    auto scores = [&](const char* st, floatx4& s0, floatx4& s1) {
        s0 = floatx4{0.f, 0.f, 0.f, 0.f};
        s1 = s0;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
            const int off = (256 * hf + 32 * ks + 8 * lq) * 2;
            const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(st + lr * kCP + off);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(st + (16 + lr) * kCP + off);
            s0 = mla_mfma32(a0, qb[ks], s0);
            s1 = mla_mfma32(a1, qb[ks], s1);
            if (ks % 2 == 1) __builtin_amdgcn_sched_barrier(0);   // bound the reads in flight
        }
    };
    floatx4 c0, c1;   // this wave's partial scores of the current tile
    // One barrier per tile.  Ahead of barrier t each wave has written its
    // partial scores of tile t (double-buffered by tile parity) and waited for
    // its own rows of tile t+1; after it tile t+1 is in LDS for everyone, every
    // wave is done with tile t-1's stage, which then takes tile t+2.  Tile
    // t+1's scores are formed right after the barrier, beside tile t's softmax.
    auto step = [&](int t, const char* st) {
        floatx4 s0 = c0, s1 = c1;
        if (t + 1 < t_hi) scores(sC[(t + 1 - t_lo) % kStages], c0, c1);
        s0 += sX[t & 1][wave ^ 1][0][lane];
        s1 += sX[t & 1][wave ^ 1][1][lane];
        // mask tokens past the length (only the last tile has any)
        if (t * kTL + kTL > L) {
            const int base = t * kTL + 4 * lq;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (base + i >= L) s0[i] = -__builtin_inff();
                if (base + 16 + i >= L) s1[i] = -__builtin_inff();
            }
        }
        float mt = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                         fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
        {
            float a = mt, b = mt;
            rows_swap16(a, b);
            mt = fmaxf(a, b);
            a = mt;
            b = mt;
            rows_swap32(a, b);
            mt = fmaxf(a, b);
        }
        // Lazy running max per head: a head's reference moves only when a
        // tile's max exceeds it by more than kLazyMax (base 2), so U and the
        // partial sums are rescaled on few tiles (any finite max moves the
        // -inf of the first tile, where the factor is 0).  Between moves the
        // probabilities stay below 2^kLazyMax.  Both waves of a head tile hold
        // the same scores, hence take the same decisions.
        const bool move = mt > m_ref + kLazyMax;
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
            const float m_new = move ? mt : m_ref;
            const float alpha = fast_exp2(m_ref - m_new);
            m_ref = m_new;
            l_part *= alpha;
            // U's rows are heads 4q .. 4q+3: gather their factors
            if (lq == 0) sA[wave][lr] = alpha;
            __builtin_amdgcn_wave_barrier();
            const floatx4 al = *reinterpret_cast<const floatx4*>(&sA[wave][4 * lq]);
#pragma unroll
            for (int j = 0; j < 16; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) U[j][i] *= al[i];
            __builtin_amdgcn_wave_barrier();
        }
        float p[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = fast_exp2(s0[i] - m_ref);
            p[4 + i] = fast_exp2(s1[i] - m_ref);
        }
        l_part += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        const bf16x8 pa = __builtin_convertvector(floatx8{p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]}, bf16x8);

        // U += P C over this wave's 256 latent columns
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int col = 256 * hf + 16 * j + 4 * (lr & 3);
            const bf16v4 lo = mla_read_tr(reinterpret_cast<const __bf16*>(st + (4 * lq + (lr >> 2)) * kCP + col * 2));
            const bf16v4 hi = mla_read_tr(reinterpret_cast<const __bf16*>(st + (16 + 4 * lq + (lr >> 2)) * kCP + col * 2));
            const bf16x8 cf = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            U[j] = mla_mfma32(pa, cf, U[j]);
            if (j % 4 == 3) __builtin_amdgcn_sched_barrier(0);   // bound the reads in flight
        }
        if (t + 1 < t_hi) {
            sX[(t + 1) & 1][wave][0][lane] = c0;
            sX[(t + 1) & 1][wave][1][lane] = c1;
            wait_loads<0>();   // this wave's rows of tile t+2 (the last issued)
            __syncthreads();
            issue(t + 3);
        }
    };

    issue(t_lo);
    issue(t_lo + 1);
    if (t_lo + 1 < t_hi) wait_loads<RPL>(); else wait_loads<0>();
    __syncthreads();   // tile t_lo in LDS
    if (t_lo < t_hi) {
        scores(sC[0], c0, c1);
        sX[t_lo & 1][wave][0][lane] = c0;
        sX[t_lo & 1][wave][1][lane] = c1;
        wait_loads<0>();   // tile t_lo + 1
        __syncthreads();
        issue(t_lo + 2);
    }
    for (int t = t_lo; t < t_hi; ++t) step(t, sC[(t - t_lo) % kStages]);

    // partial results of this split: m, l per head; U [H][512]
    float l_head;
    {
        float a = l_part, b = l_part;
        rows_swap16(a, b);
        l_head = a + b;
        a = l_head;
        b = l_head;
        rows_swap32(a, b);
        l_head = a + b;
    }
    const int64_t pb = ((int64_t)b * nsplit + sp) * H;
    if (hf == 0 && lq == 0) {
        part_ml[(pb + ht * 16 + lr) * 2] = m_ref;
        part_ml[(pb + ht * 16 + lr) * 2 + 1] = l_head;
    }
    if (nsplit == 1) {
        // one split: u = U / l itself, in bf16 (the combine step takes it as
        // is); U's rows are heads 4q .. 4q+3, whose sums come through sA
        if (lq == 0) sA[wave][lr] = l_head;
        __builtin_amdgcn_wave_barrier();
        const floatx4 lh = *reinterpret_cast<const floatx4*>(&sA[wave][4 * lq]);
        float inv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) inv[i] = 1.f / lh[i];
        __bf16* ub = reinterpret_cast<__bf16*>(part_u);
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ub[(pb + ht * 16 + 4 * lq + i) * kR + 256 * hf + 16 * j + lr] = (__bf16)(U[j][i] * inv[i]);
        return;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            part_u[(pb + ht * 16 + 4 * lq + i) * kR + 256 * hf + 16 * j + lr] = U[j][i];
}

// ---- 3. combine the splits, o = W_uv u, y = o * sigmoid(gate) -------------
// Workgroup (head h, 32 sequences), 4 waves.  The splits are merged into
// u = sum_s U_s 2^(m_s - M) / sum_s l_s 2^(m_s - M) (fp32, rounded to bf16 in
// LDS), then o = u W_uv[h]^T (32 x 128 x 512) on 16x16x32 MFMA: u rows are
// the A operand, rows of W_uv[h] the B operand straight from memory (K = the
// latent index runs along them).  Wave w owns output columns 32 w .. +31.
constexpr int kUP = kR * 2 + 16;   // LDS row pitch (bytes) of u
// MERGE: several splits to merge; without it (one split) the kernel only
// copies u, and leaves out the merge's registers, which would otherwise hold
// it to one wave per SIMD
template <bool MERGE>
__global__ void __launch_bounds__(256)
mla_combine_kernel(const float* __restrict__ part_ml, const float* __restrict__ part_u,
                   const __bf16* __restrict__ w_uv, const __bf16* __restrict__ gate,
                   __bf16* __restrict__ y, int B, int H, int nsplit) {
    __shared__ __attribute__((aligned(16))) char su[kGS * kUP];
    const int h = blockIdx.x, b0 = blockIdx.y * kGS, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lq = lane >> 4;
    const int nb = B - b0 < kGS ? B - b0 : kGS;
    // this wave's B operands (rows 32 w + lr and 32 w + 16 + lr of W_uv[h]),
    // all in flight while the splits are merged
    const __bf16* wr = w_uv + ((int64_t)h * kDh + 32 * wave + lr) * kR + 8 * lq;
    bf16x8 wv[kR / 32][2];
#pragma unroll
    for (int ks = 0; ks < kR / 32; ++ks) {
        wv[ks][0] = *reinterpret_cast<const bf16x8*>(wr + 32 * ks);
        wv[ks][1] = *reinterpret_cast<const bf16x8*>(wr + 16 * kR + 32 * ks);
    }
    const int j0 = 8 * wave;
    if constexpr (!MERGE) {
        // one split: the attention step stored u = U / l in bf16 already
        const __bf16* ub = reinterpret_cast<const __bf16*>(part_u);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            bf16x8 v = {};
            if (j0 + j < nb) v = *reinterpret_cast<const bf16x8*>(ub + ((int64_t)(b0 + j0 + j) * H + h) * kR + 8 * lane);
            *reinterpret_cast<bf16x8*>(su + (j0 + j) * kUP + 16 * lane) = v;
        }
    } else {
        // merge the splits: wave w takes sequences b0 + 8 w .. +7, lane l latent
        // columns 8 l .. 8 l + 7; splits outermost, so each split's loads for
        // all eight sequences are in flight together
        float M[8], den[8], num[8][8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            M[j] = -__builtin_inff();
            den[j] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) num[j][e] = 0.f;
        }
        auto row_of = [&](int j) -> int64_t {   // sequences past B reuse b0's rows (never stored)
            const int bb = b0 + j0 + j < B ? b0 + j0 + j : b0;
            return (int64_t)bb * nsplit * H + h;
        };
        for (int sp = 0; sp < nsplit; ++sp)
#pragma unroll
            for (int j = 0; j < 8; ++j) M[j] = fmaxf(M[j], part_ml[(row_of(j) + (int64_t)sp * H) * 2]);
        for (int sp = 0; sp < nsplit; ++sp) {
            floatx4 pu[8][2];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float* src = part_u + (row_of(j) + (int64_t)sp * H) * kR + 8 * lane;
                pu[j][0] = *reinterpret_cast<const floatx4*>(src);
                pu[j][1] = *reinterpret_cast<const floatx4*>(src + 4);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t ps = row_of(j) + (int64_t)sp * H;
                const float ws = fast_exp2(part_ml[ps * 2] - M[j]);   // 0 for an empty split
                den[j] += ws * part_ml[ps * 2 + 1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    num[j][e] += ws * pu[j][0][e];
                    num[j][4 + e] += ws * pu[j][1][e];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float inv = j0 + j < nb ? 1.f / den[j] : 0.f;
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = (__bf16)(num[j][e] * inv);
            *reinterpret_cast<bf16x8*>(su + (j0 + j) * kUP + 16 * lane) = v;
        }
    }
    __syncthreads();
    floatx4 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kR / 32; ++ks) {
        const bf16x8 w0 = wv[ks][0], w1 = wv[ks][1];
        const bf16x8 u0 = *reinterpret_cast<const bf16x8*>(su + lr * kUP + (32 * ks + 8 * lq) * 2);
        const bf16x8 u1 = *reinterpret_cast<const bf16x8*>(su + (16 + lr) * kUP + (32 * ks + 8 * lq) * 2);
        acc[0][0] = mla_mfma32(u0, w0, acc[0][0]);
        acc[0][1] = mla_mfma32(u0, w1, acc[0][1]);
        acc[1][0] = mla_mfma32(u1, w0, acc[1][0]);
        acc[1][1] = mla_mfma32(u1, w1, acc[1][1]);
    }
    // lane (q, c): sequences b0 + 16 mt + 4q + i, output column 32 w + 16 nt + c
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int bb = b0 + 16 * mt + 4 * lq + i;
            if (bb < B) {
#pragma unroll
                for (int nt = 0; nt < 2; ++nt) {
                    const int64_t o = ((int64_t)bb * H + h) * kDh + 32 * wave + 16 * nt + lr;
                    y[o] = (__bf16)(acc[mt][nt][i] * sigmoidf_((float)gate[o]));
                }
            }
        }
}

template <int HT>
hipError_t launch_attn_t(const void* qp, const void* cache, const int32_t* lengths, float* ml,
                         float* pu, int B, int Lmax, int nsplit, hipStream_t s) {
    hipLaunchKernelGGL((mla_attn_kernel<HT>), dim3((unsigned)nsplit, (unsigned)B),
                       dim3(128 * HT), 0, s, (const __bf16*)qp, (const __bf16*)cache, lengths,
                       ml, pu, Lmax, nsplit);
    return hipGetLastError();
}

}  // namespace

int mla_splits(int B, int Lmax) {
    const int tiles = (Lmax + kTL - 1) / kTL;
    int ns = (256 + B - 1) / (B > 0 ? B : 1);   // about one workgroup per CU
    if (ns > tiles) ns = tiles;
    return ns < 1 ? 1 : ns;
}

int64_t mla_workspace_bytes(int B, int H, int Lmax) {
    const int64_t ns = mla_splits(B, Lmax);
    return (int64_t)B * H * kR * 2                 // q' (bf16)
           + (int64_t)B * ns * H * 2 * 4           // m, l
           + (int64_t)B * ns * H * kR * 4 + 256;   // U, and alignment slack
}

void* mla_scratch(hipError_t* err) {
    // looked up once per device, with that device current
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = -1;
    *err = hipGetDevice(&dev);
    if (*err != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) {
        *err = hipErrorInvalidDevice;
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
        void* p = nullptr;
        *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (*err != hipSuccess) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

hipError_t launch_mla_decode(const void* q, const void* w_uk, const void* w_uv,
                             const void* cache, const int32_t* lengths, const void* gate, void* y,
                             void* workspace, int B, int H, int Lmax, float scale,
                             hipStream_t s) {
    if (B == 0) return hipSuccess;
    const int ns = mla_splits(B, Lmax);
    char* ws = reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(workspace) + 255) & ~uintptr_t(255));
    __bf16* qp = reinterpret_cast<__bf16*>(ws);
    float* ml = reinterpret_cast<float*>(ws + (int64_t)B * H * kR * 2);
    float* pu = ml + (int64_t)B * ns * H * 2;
    const dim3 grid_bh((unsigned)H, (unsigned)((B + kGS - 1) / kGS));
    hipLaunchKernelGGL(mla_absorb_kernel, grid_bh, dim3(256), 0, s, (const __bf16*)q,
                       (const __bf16*)w_uk, qp, B, H, scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (H / 16) {
        case 1: e = launch_attn_t<1>(qp, cache, lengths, ml, pu, B, Lmax, ns, s); break;
        case 2: e = launch_attn_t<2>(qp, cache, lengths, ml, pu, B, Lmax, ns, s); break;
        case 3: e = launch_attn_t<3>(qp, cache, lengths, ml, pu, B, Lmax, ns, s); break;
        case 4: e = launch_attn_t<4>(qp, cache, lengths, ml, pu, B, Lmax, ns, s); break;
        case 5: e = launch_attn_t<5>(qp, cache, lengths, ml, pu, B, Lmax, ns, s); break;
        default: e = launch_attn_t<6>(qp, cache, lengths, ml, pu, B, Lmax, ns, s); break;
    }
    if (e != hipSuccess) return e;
    if (ns == 1)
        hipLaunchKernelGGL(mla_combine_kernel<false>, grid_bh, dim3(256), 0, s, ml, pu,
                           (const __bf16*)w_uv, (const __bf16*)gate, (__bf16*)y, B, H, ns);
    else
        hipLaunchKernelGGL(mla_combine_kernel<true>, grid_bh, dim3(256), 0, s, ml, pu,
                           (const __bf16*)w_uv, (const __bf16*)gate, (__bf16*)y, B, H, ns);
    return hipGetLastError();
}

}  // namespace kda
