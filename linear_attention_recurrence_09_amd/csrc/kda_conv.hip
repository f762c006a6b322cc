// kda_conv.hip -- short causal depthwise convolution + SiLU over projected
// q|k|v, then L2 normalisation of q and k per (token, head) (gfx950).
//
// "Inside Kimi K3" (lei.chat), KDA short-convolution diagram: each channel is
// filtered on its own over a causal window of 4 tokens (taps w0..w3 on
// x_{t-3}..x_t), SiLU follows, the length is kept by left padding, and the
// rolling state of a sequence is its last 3 raw inputs per channel.  KDA
// one-head diagram: q and k are then L2-normalised over the 128-d head.
//
// HBM-bound stencil: read x once (plus a 3-token halo per strip) and write y
// once.  A thread owns 8 consecutive channels (one 16-byte bf16 vector) for a
// strip of tokens (128 in bf16), streamed in groups: the next group's rows are
// loaded while the current group is computed, and the 3-value window slides
// in registers across groups, so weights and halo are loaded once per strip.
// D/8 lanes of one head reduce the sum of squares with xor shuffles.  A block
// covers 2048 channels; windows restart at every sequence start.
//
// MXFP8 output (OCP microscaling: E4M3 elements, one E8M0 scale per 32
// consecutive channels): the 4 lanes of a 32-channel block exchange their
// largest magnitude (two xor shuffles, issued beside the L2 sum's, on the
// values before normalisation: scaling by the positive L2 factor and
// rounding are monotonic, so the normalised block's largest magnitude is
// that maximum times the factor, rounded), the block exponent e is the
// smallest with amax <= 448 * 2^e (read off the fp32 bits of amax), and each
// normalised value is scaled by 2^-e (exact) and rounded to E4M3 by the
// hardware's packed conversion.  Codes replace the bf16 row (8 bytes per
// lane).  A head's D/32 scale bytes are gathered into its first lane (DPP
// row shifts) and written with one 4-byte (D = 128) or 2-byte (D = 64)
// store into the q, k or v scale tensor.  With MXFP8 output a block covers
// 4096 channels (512 threads), so that its scale bytes of a token are whole
// 128-byte lines: lines shared between blocks (2048 channels write 64
// bytes of a 384-byte row) made the kernel about 50 % slower.  It streams
// 4-row groups instead of 16 (512 threads; measured faster than 8).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kConvThreads = 256;
constexpr int kConvChannels = kConvThreads * 8;
// Tokens per block (TT) and per streamed group (G).  A block walks its strip
// of TT tokens in groups of G: the next group's rows are in flight while the
// current group is computed, and the 3-token window slides across groups, so
// the weights and the halo are loaded once per strip.
template <typename T>
struct ConvTile {
    static constexpr int TT = sizeof(T) == 2 ? 128 : 8;
    static constexpr int G = sizeof(T) == 2 ? 16 : 8;
};

struct SeqRange {
    int s;
    int64_t start, end;
};

// Token range [start, end) of packed sequence s, clamped to the N tokens of
// the batch (0 <= start <= end <= N), so offsets that are not monotone or
// exceed N never move an access out of bounds.
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int s, int64_t N, int64_t& start,
                                           int64_t& end) {
    const int64_t a = cu[s], b = cu[s + 1];
    start = a < 0 ? 0 : (a > N ? N : a);
    end = b < start ? start : (b > N ? N : b);
}

// Sequence holding token t: the largest s with start(s) <= t (empty
// sequences are skipped because their successor starts at the same token).
__device__ __forceinline__ SeqRange find_seq(const int32_t* cu, int num_seqs, int T, int64_t N,
                                             int64_t t) {
    SeqRange r;
    if (cu == nullptr) {
        r.s = (int)(t / T);
        r.start = (int64_t)r.s * T;
        r.end = r.start + T;
        return r;
    }
    int lo = 0, hi = num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    r.s = lo;
    seq_bounds(cu, lo, N, r.start, r.end);
    return r;
}

// a[i] for a runtime i in [0, 3) without indexing registers dynamically
__device__ __forceinline__ float pick3(const float a[3], int i) {
    return i == 0 ? a[0] : (i == 1 ? a[1] : a[2]);
}

template <typename T>
__device__ __forceinline__ void load_state8(const T* state_in, int64_t s, int P, int c0,
                                            float st[8][3]) {
    if (state_in == nullptr) {
#pragma unroll
        for (int e = 0; e < 8; ++e) st[e][0] = st[e][1] = st[e][2] = 0.f;
        return;
    }
    // 8 channels x 3 slots = 24 contiguous values
    const T* p = state_in + (s * P + c0) * 3;
    float v[24];
    load8(p, v);
    load8(p + 8, v + 8);
    load8(p + 16, v + 16);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        st[e][0] = v[3 * e + 0];
        st[e][1] = v[3 * e + 1];
        st[e][2] = v[3 * e + 2];
    }
}

typedef short short2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// E8M0 scale byte of a block whose largest magnitude is amax (>= 0): e + 127
// with e the smallest integer such that amax <= 448 * 2^e = 1.75 * 2^(e+8),
// clamped to [-127, 127].  For amax = (1 + m/2^23) 2^(E-127) that is
// e = E - 135, plus one when the mantissa exceeds 0.75 (m > 0x600000).
__device__ __forceinline__ int mx_scale_byte(uint32_t amax_bits) {
    const int E = (int)(amax_bits >> 23);
    const int e = E - 135 + ((amax_bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    return e < -127 ? 0 : e + 127;   // the largest E (254) gives e = 120
}

// Largest magnitude of the 8 values of a lane, and over the 4 lanes of its
// 32-channel block (all 64 lanes must call it).
__device__ __forceinline__ float block_amax(const float v[8]) {
    float am = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) am = __builtin_fmaxf(am, __builtin_fabsf(v[e]));
    am = __builtin_fmaxf(am, __shfl_xor(am, 1, 64));
    return __builtin_fmaxf(am, __shfl_xor(am, 2, 64));
}

// 8 normalised values of one lane as MXFP8 codes, with their block's
// largest magnitude amax (see the header).  `scale` points at the head's
// first scale byte of the token; lanes with `head_lane` (the head's first
// lane) write the head's D/32 scale bytes.  All 64 lanes must call it.
template <int D>
__device__ __forceinline__ void store_mx8(uint8_t* codes, uint8_t* scale, bool active,
                                          bool head_lane, const float v[8], float amax) {
    static_assert(D == 64 || D == 128, "a head is 8 or 16 lanes");
    const int sb = mx_scale_byte(__builtin_bit_cast(uint32_t, amax));
    const float inv = __builtin_bit_cast(float, (uint32_t)(254 - sb) << 23);   // 2^-(sb-127)
    short2_t lo = {0, 0}, hi = {0, 0};
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, v[0] * inv, v[1] * inv, 1.0f, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, v[2] * inv, v[3] * inv, 1.0f, true);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, v[4] * inv, v[5] * inv, 1.0f, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, v[6] * inv, v[7] * inv, 1.0f, true);
    // the scale bytes of the blocks 4, 8, 12 lanes on, within the row of 16
    const uint32_t b0 = (uint32_t)sb;
    const uint32_t b1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)b0, 0x104, 0xF, 0xF, false);
    uint32_t word = b0 | (b1 << 8);
    if constexpr (D == 128) {
        const uint32_t b2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)b0, 0x108, 0xF, 0xF, false);
        const uint32_t b3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)b0, 0x10C, 0xF, 0xF, false);
        word |= (b2 << 16) | (b3 << 24);
    }
    if (active) {
        const u32x2_t w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(codes));
        if (head_lane) {
            if constexpr (D == 128) *reinterpret_cast<uint32_t*>(scale) = word;
            else *reinterpret_cast<uint16_t*>(scale) = (uint16_t)word;
        }
    }
}

template <bool MX>
constexpr int conv_threads() { return MX ? 2 * kConvThreads : kConvThreads; }

template <typename T, int D, bool MX = false>
__global__ void __launch_bounds__(conv_threads<MX>())
conv_kernel(const T* __restrict__ x, const float* __restrict__ w, void* __restrict__ yv,
            const T* __restrict__ state_in, const int32_t* __restrict__ cu, int num_seqs,
            int T_len, int64_t N, int P, int HD, float l2_eps, int tiles, int tiles_per_xcd,
            int cblocks, uint8_t* __restrict__ sq, uint8_t* __restrict__ sk,
            uint8_t* __restrict__ sv) {
    constexpr int TT = ConvTile<T>::TT;
    static_assert(!MX || sizeof(T) == 2, "MXFP8 output from bf16 inputs");
    using Raw8 = typename RawVec<T, 8>::type;
    // Block -> (token tile, channel block).  Blocks go to the 8 XCDs round
    // robin, so XCD k gets the blocks k, k+8, ...: they are given a contiguous
    // range of tiles, every channel block of a tile before the next tile.  A
    // tile's 3-token halo was then read shortly before on the same XCD and is
    // served from its L2.
    const int xcd = blockIdx.x & 7, li = blockIdx.x >> 3;
    const int tile = xcd * tiles_per_xcd + li / cblocks;
    if (tile >= tiles) return;
    const int cbase = (li % cblocks) * (conv_threads<MX>() * 8);   // the block's first channel
    const int c0 = cbase + threadIdx.x * 8;
    const bool active = c0 < P;
    const int64_t t0 = (int64_t)tile * TT;
    const int64_t t1 = t0 + TT < N ? t0 + TT : N;
    const bool is_qk = c0 < 2 * HD;   // uniform over the D/8 lanes of a head
    // output of token t: the bf16 / fp32 row, or its MXFP8 codes and scales
    uint8_t* scale_row = nullptr;
    if constexpr (MX) {
        const int part = c0 / HD;
        scale_row = (part == 0 ? sq : (part == 1 ? sk : sv)) + (c0 - part * HD) / 32;
    }
    const bool head_lane = (threadIdx.x & (D / 8 - 1)) == 0;
    // the L2 step and the store of token t: sum of squares over the head,
    // then q and k scaled by 1/sqrt(ss + eps), then the bf16 / fp32 row or
    // its MXFP8 codes and scales
    auto finish = [&](int64_t t, float (&out)[8], float ss) {
        float am = 0.f;
        if constexpr (MX) am = block_amax(out);
        ss = group_sum<D / 8>(ss);
        if (is_qk) {
            const float inv = rsqrt_nr(ss + l2_eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) out[e] *= inv;
            am *= inv;
        }
        if constexpr (MX) {
            store_mx8<D>(static_cast<uint8_t*>(yv) + t * P + c0, scale_row + t * (HD / 32),
                         active, head_lane, out, am);
        } else {
            if (active) store8_nt(static_cast<T*>(yv) + t * P + c0, out);
        }
    };

    // the thread's taps, 8 channels x 4: 128 contiguous bytes in four-float
    // loads (one float per load made as many L1-to-L2 requests as the data
    // the strip streams); channels past P read as zeros, since the resource
    // ends at channel P
    float wt[8][4];
    {
        const rsrc_t rw = make_rsrc(w + (int64_t)cbase * 4, (uint32_t)((P - cbase) * 16));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const floatx4 v = __builtin_bit_cast(
                floatx4, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)threadIdx.x * 128 + 16 * e, 0, 0));
#pragma unroll
            for (int i = 0; i < 4; ++i) wt[e][i] = v[i];
        }
    }

    SeqRange sr = find_seq(cu, num_seqs, T_len, N, t0);

    // Fast path (uniform over the block): the strip and its halo lie inside one
    // sequence, so every window reads plain inputs.
    if (sr.start <= t0 - 3 && sr.end >= t0 + TT) {
        // MXFP8 output: 4-row groups (129 VGPRs at 512 threads; measured 5 %
        // faster than 8-row groups, while bf16 output is fastest with 16)
        constexpr int G = MX ? ConvTile<T>::G / 4 : ConvTile<T>::G, NG = TT / G;
        static_assert(TT % G == 0, "whole groups per strip");
        // rows t0-3 .. of this strip from the block's first channel (a
        // wave-uniform resource; the lane's channels go in the offset).  The
        // range ends with the strip, so the prefetch past the last group and
        // lanes past the last channel read zeros.
        const int64_t rows = N - (t0 - 3) < TT + 3 ? N - (t0 - 3) : TT + 3;
        const int row_bytes = P * (int)sizeof(T);
        const rsrc_t rx = make_rsrc(x + (t0 - 3) * P + cbase,
                                    (uint32_t)(rows * row_bytes - (int64_t)cbase * (int)sizeof(T)));
        const int lane_off = (int)threadIdx.x * 8 * (int)sizeof(T);
        float win[8][3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            float v[8];
            RawVec<T, 8>::unpack(BufLoad<T, 8>::load(rx, j * row_bytes + lane_off), v);
#pragma unroll
            for (int e = 0; e < 8; ++e) win[e][j] = v[e];
        }
        auto load_group = [&](Raw8 (&r)[G], int grp) {
#pragma unroll
            for (int j = 0; j < G; ++j) r[j] = BufLoad<T, 8>::load(rx, (3 + grp * G + j) * row_bytes + lane_off);
        };
        auto run_group = [&](const Raw8 (&r)[G], int grp) {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float xv[8], out[8];
                RawVec<T, 8>::unpack(r[j], xv);
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float pre = wt[e][0] * win[e][0] + wt[e][1] * win[e][1] +
                                      wt[e][2] * win[e][2] + wt[e][3] * xv[e];
                    out[e] = siluf_(pre);
                    ss += out[e] * out[e];
                    win[e][0] = win[e][1];
                    win[e][1] = win[e][2];
                    win[e][2] = xv[e];
                }
                finish(t0 + grp * G + j, out, ss);
            }
        };
        Raw8 ra[G], rb[G];
        load_group(ra, 0);
        for (int pr = 0; pr < NG / 2; ++pr) {
            load_group(rb, 2 * pr + 1);
            run_group(ra, 2 * pr);
            load_group(ra, 2 * pr + 2);   // past the strip on the last pair: zeros
            run_group(rb, 2 * pr + 1);
        }
        if constexpr (NG % 2 == 1) run_group(ra, NG - 1);
        return;
    }

    // window: win[e][0] = x_{t-3}, win[e][1] = x_{t-2}, win[e][2] = x_{t-1}
    float win[8][3];
    if (active) {
        float st[8][3];
        load_state8(state_in, sr.s, P, c0, st);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int64_t tau = t0 - 3 + j;
            if (tau >= sr.start) {
                float xv[8];
                load8(x + tau * P + c0, xv);
#pragma unroll
                for (int e = 0; e < 8; ++e) win[e][j] = xv[e];
            } else {
                const int slot = (int)(tau - sr.start) + 3;   // in [0, 3)
#pragma unroll
                for (int e = 0; e < 8; ++e) win[e][j] = pick3(st[e], slot);
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) win[e][0] = win[e][1] = win[e][2] = 0.f;
    }

    for (int64_t t = t0; t < t1; ++t) {
        if (t >= sr.end) {               // a new sequence starts at t
            do {
                if (cu == nullptr) {
                    sr.s += 1;
                    sr.start = sr.end;
                    sr.end = sr.start + T_len;
                } else if (sr.s + 1 < num_seqs) {
                    sr.s += 1;
                    seq_bounds(cu, sr.s, N, sr.start, sr.end);
                } else {
                    sr.end = t1;         // offsets inconsistent with N: stay in bounds
                }
            } while (t >= sr.end);
            if (active) load_state8(state_in, sr.s, P, c0, win);
        }
        float xv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (active) load8(x + t * P + c0, xv);
        float out[8];
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float pre = wt[e][0] * win[e][0] + wt[e][1] * win[e][1] +
                              wt[e][2] * win[e][2] + wt[e][3] * xv[e];
            out[e] = siluf_(pre);
            ss += out[e] * out[e];
            win[e][0] = win[e][1];
            win[e][1] = win[e][2];
            win[e][2] = xv[e];
        }
        finish(t, out, ss);
    }
}

// Rolling state after each sequence: its last 3 raw inputs, taken from the
// incoming state where the sequence is shorter than 3.  Each thread reads its
// own state slots before writing them, so state_out may equal state_in.
template <typename T>
__global__ void __launch_bounds__(kConvThreads)
conv_state_kernel(const T* __restrict__ x, const T* state_in, T* state_out,
                  const int32_t* __restrict__ cu, int T_len, int64_t N, int P) {
    const int s = blockIdx.x;
    const int c0 = blockIdx.y * kConvChannels + threadIdx.x * 8;
    if (c0 >= P) return;
    int64_t start = (int64_t)s * T_len, end = start + T_len;
    if (cu) seq_bounds(cu, s, N, start, end);
    const int64_t len = end - start;
    float st[8][3];
    load_state8(state_in, s, P, c0, st);
    float v[24];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int64_t tau = len - 3 + j;
        if (tau >= 0) {
            float xv[8];
            load8(x + (start + tau) * P + c0, xv);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[3 * e + j] = xv[e];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[3 * e + j] = pick3(st[e], (int)(tau + 3));
        }
    }
    T* p = state_out + ((int64_t)s * P + c0) * 3;
    store8(p, v);
    store8(p + 8, v + 8);
    store8(p + 16, v + 16);
}

template <typename T, int D, bool MX = false>
hipError_t launch_conv_t(const void* x, const float* w, void* y, const void* state_in,
                         void* state_out, const int32_t* cu, int num_seqs, int T_len,
                         int64_t N, int H, float l2_eps, hipStream_t s, void* sq = nullptr,
                         void* sk = nullptr, void* sv = nullptr) {
    const int P = 3 * H * D;
    constexpr int threads = conv_threads<MX>();
    const unsigned cblocks = (unsigned)((P + threads * 8 - 1) / (threads * 8));
    if (N > 0) {
        constexpr int TT = ConvTile<T>::TT;
        const int64_t tiles = (N + TT - 1) / TT;
        const int64_t per_xcd = (tiles + 7) / 8;
        const int64_t blocks = 8 * per_xcd * cblocks;
        if (blocks > 0x7fffffff) return hipErrorInvalidValue;
        hipLaunchKernelGGL((conv_kernel<T, D, MX>), dim3((unsigned)blocks), dim3(threads), 0,
                           s, (const T*)x, w, y, (const T*)state_in, cu, num_seqs, T_len, N, P,
                           H * D, l2_eps, (int)tiles, (int)per_xcd, (int)cblocks, (uint8_t*)sq,
                           (uint8_t*)sk, (uint8_t*)sv);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (state_out != nullptr && num_seqs > 0) {
        const unsigned sblocks = (unsigned)((P + kConvChannels - 1) / kConvChannels);
        hipLaunchKernelGGL((conv_state_kernel<T>), dim3((unsigned)num_seqs, sblocks),
                           dim3(kConvThreads), 0, s, (const T*)x, (const T*)state_in,
                           (T*)state_out, cu, T_len, N, P);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_conv_state(const void* x, const void* state_in, void* state_out,
                             const int32_t* cu, int num_seqs, int T, int64_t N, int H, int D,
                             int dtype, hipStream_t s) {
    if (state_out == nullptr || num_seqs == 0) return hipSuccess;
    const int P = 3 * H * D;
    const unsigned sblocks = (unsigned)((P + kConvChannels - 1) / kConvChannels);
    if (dtype == 0)
        hipLaunchKernelGGL((conv_state_kernel<float>), dim3((unsigned)num_seqs, sblocks),
                           dim3(kConvThreads), 0, s, (const float*)x, (const float*)state_in,
                           (float*)state_out, cu, T, N, P);
    else
        hipLaunchKernelGGL((conv_state_kernel<__bf16>), dim3((unsigned)num_seqs, sblocks),
                           dim3(kConvThreads), 0, s, (const __bf16*)x, (const __bf16*)state_in,
                           (__bf16*)state_out, cu, T, N, P);
    return hipGetLastError();
}

hipError_t launch_conv(const void* x, const float* w, void* y, const void* state_in,
                       void* state_out, const int32_t* cu, int num_seqs, int T, int64_t N,
                       int H, int D, int dtype, float l2_eps, hipStream_t s) {
    if (dtype == 0) {
        return D == 64 ? launch_conv_t<float, 64>(x, w, y, state_in, state_out, cu, num_seqs, T,
                                                  N, H, l2_eps, s)
                       : launch_conv_t<float, 128>(x, w, y, state_in, state_out, cu, num_seqs,
                                                   T, N, H, l2_eps, s);
    }
    return D == 64 ? launch_conv_t<__bf16, 64>(x, w, y, state_in, state_out, cu, num_seqs, T, N,
                                               H, l2_eps, s)
                   : launch_conv_t<__bf16, 128>(x, w, y, state_in, state_out, cu, num_seqs, T,
                                                N, H, l2_eps, s);
}

hipError_t launch_conv_mxfp8(const void* x, const float* w, void* codes, void* q_scale,
                             void* k_scale, void* v_scale, const void* state_in, void* state_out,
                             const int32_t* cu, int num_seqs, int T, int64_t N, int H, int D,
                             float l2_eps, hipStream_t s) {
    return D == 64 ? launch_conv_t<__bf16, 64, true>(x, w, codes, state_in, state_out, cu,
                                                     num_seqs, T, N, H, l2_eps, s, q_scale,
                                                     k_scale, v_scale)
                   : launch_conv_t<__bf16, 128, true>(x, w, codes, state_in, state_out, cu,
                                                      num_seqs, T, N, H, l2_eps, s, q_scale,
                                                      k_scale, v_scale);
}

}  // namespace kda
