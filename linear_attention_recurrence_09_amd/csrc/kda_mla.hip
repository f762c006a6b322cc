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
// o_h = W_uv[h] u_h.  Three kernels:
//  1. absorb: q' in bf16, scaled by scale * log2(e) (the softmax runs in
//     base 2);
//  2. attention over a range of the cache, all heads at once, per
//     (sequence, split): S = Q' C^T and U += P C on 16x16x32 MFMA with a
//     running (online) softmax, partial m, l, U to the workspace;
//  3. combine the splits, o = W_uv u, y = o * sigmoid(gate).
#include <hip/hip_runtime.h>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kR = 512;            // latent width
constexpr int kDh = 128;           // key / value width per head
constexpr int kTL = 32;            // cached tokens per attention tile
constexpr int kAttnThreads = 512;  // 8 waves
constexpr int kRP = kR + 16;       // LDS row pitch (bf16) of Q' and the cache tile: 8 banks per row
constexpr int kPP = kTL + 8;       // LDS row pitch (bf16) of P
constexpr int kSP = kTL + 1;       // LDS row pitch (fp32) of S
constexpr int kSeqPerBlock = 8;    // sequences per absorb / combine workgroup

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

// ---- 1. absorb: q'[b][h][r] = s * sum_d q[b][h][d] W_uk[h][d][r] ----------
__global__ void __launch_bounds__(kR)
mla_absorb_kernel(const __bf16* __restrict__ q, const __bf16* __restrict__ w_uk,
                  __bf16* __restrict__ qp, int B, int H, float s) {
    __shared__ float sq[kSeqPerBlock][kDh];
    const int h = blockIdx.x, b0 = blockIdx.y * kSeqPerBlock, r = threadIdx.x;
    const int nb = B - b0 < kSeqPerBlock ? B - b0 : kSeqPerBlock;
    for (int i = threadIdx.x; i < kSeqPerBlock * kDh; i += kR) {
        const int j = i / kDh, d = i % kDh;
        sq[j][d] = j < nb ? (float)q[((int64_t)(b0 + j) * H + h) * kDh + d] : 0.f;
    }
    __syncthreads();
    float acc[kSeqPerBlock];
#pragma unroll
    for (int j = 0; j < kSeqPerBlock; ++j) acc[j] = 0.f;
    const __bf16* wh = w_uk + (int64_t)h * kDh * kR + r;
    for (int d = 0; d < kDh; ++d) {
        const float wv = (float)wh[(int64_t)d * kR];
#pragma unroll
        for (int j = 0; j < kSeqPerBlock; ++j) acc[j] += sq[j][d] * wv;
    }
#pragma unroll
    for (int j = 0; j < kSeqPerBlock; ++j)
        if (j < nb) qp[((int64_t)(b0 + j) * H + h) * kR + r] = (__bf16)(acc[j] * s);
}

// ---- 2. attention over one range of the cache, all heads ------------------
// Workgroup (split sp, sequence b), 8 waves.  Head tiles of 16 (HT of them);
// S tiles (head tile, 16 tokens) are dealt to the waves; U is held in
// registers, wave w owning latent columns 64 w .. 64 w + 63 of every head.
template <int HT>
__global__ void __launch_bounds__(kAttnThreads)
mla_attn_kernel(const __bf16* __restrict__ qp, const __bf16* __restrict__ cache,
                const int32_t* __restrict__ lengths, float* __restrict__ part_ml,
                float* __restrict__ part_u, int Lmax, int nsplit) {
    constexpr int H = 16 * HT;
    __shared__ __attribute__((aligned(16))) __bf16 sQ[H * kRP];
    __shared__ __attribute__((aligned(16))) __bf16 sC[kTL * kRP];
    __shared__ __attribute__((aligned(16))) float sS[H * kSP];
    __shared__ __attribute__((aligned(16))) __bf16 sP[H * kPP];
    __shared__ __attribute__((aligned(16))) float sAlpha[H];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lq = lane >> 4;
    const int sp = blockIdx.x, b = blockIdx.y;
    int L = lengths[b];
    L = L < 1 ? 1 : (L > Lmax ? Lmax : L);
    const int tiles = (L + kTL - 1) / kTL;
    const int tps = (tiles + nsplit - 1) / nsplit;
    const int t_lo = sp * tps;
    const int t_hi = t_lo + tps < tiles ? t_lo + tps : tiles;

    // Q' of this sequence into LDS (rows of 512 bf16 = 64 x 16 bytes)
    const __bf16* qb = qp + (int64_t)b * H * kR;
    for (int i = tid; i < H * (kR / 8); i += kAttnThreads) {
        const int row = i / (kR / 8), c8 = i % (kR / 8);
        *reinterpret_cast<bf16x8*>(&sQ[row * kRP + 8 * c8]) =
            *reinterpret_cast<const bf16x8*>(qb + (int64_t)row * kR + 8 * c8);
    }
    // the cache tile: 32 rows x 64 pieces of 16 bytes, 4 per thread; rows
    // past the sequence's length read as zeros (their scores are masked)
    const __bf16* cb = cache + (int64_t)b * Lmax * kR;
    bf16x8 pre[4];
    auto fetch = [&](int t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int id = tid + kAttnThreads * j, row = id / (kR / 8), c8 = id % (kR / 8);
            const int tok = t * kTL + row;
            pre[j] = tok < L ? *reinterpret_cast<const bf16x8*>(cb + (int64_t)tok * kR + 8 * c8)
                             : bf16x8{};
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int id = tid + kAttnThreads * j, row = id / (kR / 8), c8 = id % (kR / 8);
            *reinterpret_cast<bf16x8*>(&sC[row * kRP + 8 * c8]) = pre[j];
        }
    };

    // running softmax state, one thread per head (base 2: q' carries log2 e)
    float m_run = -__builtin_inff(), l_run = 0.f;
    floatx4 U[HT][4];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int j = 0; j < 4; ++j) U[ht][j] = floatx4{0.f, 0.f, 0.f, 0.f};

    if (t_lo < t_hi) fetch(t_lo);
    for (int t = t_lo; t < t_hi; ++t) {
        __syncthreads();   // the previous tile's reads of sC, sP, sAlpha are done
        stage();
        if (t + 1 < t_hi) fetch(t + 1);   // in flight while this tile computes
        __syncthreads();

        // S = Q' C^T, tiles (head tile, token tile) dealt to the waves
        for (int st = wave; st < 2 * HT; st += kAttnThreads / 64) {
            const int ht = st >> 1, tt = st & 1;
            floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < kR / 32; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sQ[(ht * 16 + lr) * kRP + 32 * ks + 8 * lq]);
                const bf16x8 c = *reinterpret_cast<const bf16x8*>(&sC[(tt * 16 + lr) * kRP + 32 * ks + 8 * lq]);
                acc = mla_mfma32(a, c, acc);
            }
            // lane (q, c): heads ht*16 + 4q + i, token tt*16 + c
#pragma unroll
            for (int i = 0; i < 4; ++i) sS[(ht * 16 + 4 * lq + i) * kSP + tt * 16 + lr] = acc[i];
        }
        __syncthreads();

        // online softmax, one thread per head
        if (tid < H) {
            const int valid = L - t * kTL < kTL ? L - t * kTL : kTL;
            float sc[kTL];
            float mt = -__builtin_inff();
#pragma unroll
            for (int j = 0; j < kTL; ++j) {
                sc[j] = j < valid ? sS[tid * kSP + j] : -__builtin_inff();
                mt = fmaxf(mt, sc[j]);
            }
            const float m_new = fmaxf(m_run, mt);
            const float alpha = fast_exp2(m_run - m_new);   // 0 on the first tile
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < kTL; j += 2) {
                const float p0 = fast_exp2(sc[j] - m_new), p1 = fast_exp2(sc[j + 1] - m_new);
                sum += p0 + p1;
                *reinterpret_cast<bf16x2*>(&sP[tid * kPP + j]) =
                    __builtin_convertvector(floatx2{p0, p1}, bf16x2);
            }
            l_run = l_run * alpha + sum;
            m_run = m_new;
            sAlpha[tid] = alpha;
        }
        __syncthreads();

        // U = diag(alpha) U + P C: wave w holds latent columns 64 w .. 64 w + 63
        bf16x8 cf[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // B operand: tokens 8q .. 8q+7 of latent column 64 w + 16 j + lr
            const int n0 = 64 * wave + 16 * j;
            const bf16v4 lo = mla_read_tr(&sC[(8 * lq + (lr >> 2)) * kRP + n0 + 4 * (lr & 3)]);
            const bf16v4 hi = mla_read_tr(&sC[(8 * lq + 4 + (lr >> 2)) * kRP + n0 + 4 * (lr & 3)]);
            cf[j] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const bf16x8 pa = *reinterpret_cast<const bf16x8*>(&sP[(ht * 16 + lr) * kPP + 8 * lq]);
            const floatx4 al = *reinterpret_cast<const floatx4*>(&sAlpha[ht * 16 + 4 * lq]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int i = 0; i < 4; ++i) U[ht][j][i] *= al[i];
                U[ht][j] = mla_mfma32(pa, cf[j], U[ht][j]);
            }
        }
    }

    // partial results of this split: m, l per head; U [H][512]
    const int64_t pb = ((int64_t)b * nsplit + sp) * H;
    if (tid < H) {
        part_ml[(pb + tid) * 2] = m_run;
        part_ml[(pb + tid) * 2 + 1] = l_run;
    }
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                part_u[(pb + ht * 16 + 4 * lq + i) * kR + 64 * wave + 16 * j + lr] = U[ht][j][i];
}

// ---- 3. combine the splits, o = W_uv u, y = o * sigmoid(gate) -------------
__global__ void __launch_bounds__(256)
mla_combine_kernel(const float* __restrict__ part_ml, const float* __restrict__ part_u,
                   const __bf16* __restrict__ w_uv, const __bf16* __restrict__ gate,
                   __bf16* __restrict__ y, int B, int H, int nsplit) {
    __shared__ float su[kSeqPerBlock][kR];
    __shared__ float so[2][kSeqPerBlock][kDh];
    const int h = blockIdx.x, b0 = blockIdx.y * kSeqPerBlock, tid = threadIdx.x;
    const int nb = B - b0 < kSeqPerBlock ? B - b0 : kSeqPerBlock;
    // u = sum_s U_s 2^(m_s - M) / sum_s l_s 2^(m_s - M)
    for (int i = tid; i < kSeqPerBlock * kR; i += 256) {
        const int j = i / kR, r = i % kR;
        float val = 0.f;
        if (j < nb) {
            const int64_t base = (int64_t)(b0 + j) * nsplit * H + h;
            float M = -__builtin_inff();
            for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_ml[(base + (int64_t)s * H) * 2]);
            float num = 0.f, den = 0.f;
            for (int s = 0; s < nsplit; ++s) {
                const int64_t ps = base + (int64_t)s * H;
                const float ws = fast_exp2(part_ml[ps * 2] - M);   // 0 for an empty split
                den += ws * part_ml[ps * 2 + 1];
                num += ws * part_u[ps * kR + r];
            }
            val = num / den;
        }
        su[j][r] = val;
    }
    __syncthreads();
    // o[j][d]: thread (d, half) sums latent columns 256 half .. +255
    const int d = tid & (kDh - 1), half = tid >> 7;
    float acc[kSeqPerBlock];
#pragma unroll
    for (int j = 0; j < kSeqPerBlock; ++j) acc[j] = 0.f;
    const __bf16* wr = w_uv + ((int64_t)h * kDh + d) * kR + 256 * half;
    for (int r8 = 0; r8 < 256; r8 += 8) {
        const bf16x8 wv = *reinterpret_cast<const bf16x8*>(wr + r8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float wf = (float)wv[e];
#pragma unroll
            for (int j = 0; j < kSeqPerBlock; ++j) acc[j] += wf * su[j][256 * half + r8 + e];
        }
    }
#pragma unroll
    for (int j = 0; j < kSeqPerBlock; ++j) so[half][j][d] = acc[j];
    __syncthreads();
    if (tid < kDh) {
        for (int j = 0; j < nb; ++j) {
            const int64_t o = ((int64_t)(b0 + j) * H + h) * kDh + tid;
            const float z = (float)gate[o];
            y[o] = (__bf16)((so[0][j][tid] + so[1][j][tid]) * sigmoidf_(z));
        }
    }
}

template <int HT>
hipError_t launch_attn_t(const void* qp, const void* cache, const int32_t* lengths, float* ml,
                         float* pu, int B, int Lmax, int nsplit, hipStream_t s) {
    hipLaunchKernelGGL((mla_attn_kernel<HT>), dim3((unsigned)nsplit, (unsigned)B),
                       dim3(kAttnThreads), 0, s, (const __bf16*)qp, (const __bf16*)cache, lengths,
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
    const dim3 grid_bh((unsigned)H, (unsigned)((B + kSeqPerBlock - 1) / kSeqPerBlock));
    hipLaunchKernelGGL(mla_absorb_kernel, grid_bh, dim3(kR), 0, s, (const __bf16*)q,
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
    hipLaunchKernelGGL(mla_combine_kernel, grid_bh, dim3(256), 0, s, ml, pu, (const __bf16*)w_uv,
                       (const __bf16*)gate, (__bf16*)y, B, H, ns);
    return hipGetLastError();
}

}  // namespace kda
