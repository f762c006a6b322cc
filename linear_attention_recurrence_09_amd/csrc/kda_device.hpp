// kda_device.hpp -- device helpers shared by the gfx950 KDA kernels.
//
// I/O element types: float (fp32 mode) and __bf16 (bf16 mode).  bf16 -> fp32 is
// exact; fp32 -> bf16 uses the hardware round-to-nearest-even conversion.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLogDecayMin = -5.0f;  // the pages bound the log-decay below by -5

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f(float x);
template <>
__device__ __forceinline__ float from_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return (__bf16)x; }

// ---- 8-wide vector I/O (16 B for bf16, 2 x 16 B for fp32) -------------------
__device__ __forceinline__ void load8(const float* p, float v[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const __bf16* p, float v[8]) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8(__bf16* p, const float v[8]) {
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (__bf16)v[i];
    *reinterpret_cast<bf16x8*>(p) = a;
}

// Non-temporal variants for data streamed once (no reuse through the caches).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store8_nt(float* p, const float v[8]) {
    const floatx4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<floatx4*>(p));
    __builtin_nontemporal_store(b, reinterpret_cast<floatx4*>(p + 4));
}
__device__ __forceinline__ void store8_nt(__bf16* p, const float v[8]) {
    bf16x8 a;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (__bf16)v[i];
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, a), reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void load8_nt(const float* p, float v[8]) {
    const floatx4 a = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p));
    const floatx4 b = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(p + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}
__device__ __forceinline__ void load8_nt(const __bf16* p, float v[8]) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (float)a[i];
}

// ---- 2-wide I/O --------------------------------------------------------------
__device__ __forceinline__ void load2(const float* p, float& a, float& b) {
    const float2 t = *reinterpret_cast<const float2*>(p);
    a = t.x; b = t.y;
}
__device__ __forceinline__ void load2(const __bf16* p, float& a, float& b) {
    const bf16x2 t = *reinterpret_cast<const bf16x2*>(p);
    a = (float)t[0]; b = (float)t[1];
}
__device__ __forceinline__ void store2(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
__device__ __forceinline__ void store2(__bf16* p, float a, float b) {
    bf16x2 t;
    t[0] = (__bf16)a; t[1] = (__bf16)b;
    *reinterpret_cast<bf16x2*>(p) = t;
}

// ---- raw vectors of N I/O elements, kept unconverted in registers -------------
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

template <typename T, int N>
struct RawVec;

template <int N, typename V, typename E>
struct RawVecImpl {
    typedef V type;
    static __device__ __forceinline__ void unpack(const V& r, float v[N]) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = (float)r[i];
    }
    static __device__ __forceinline__ void store(E* p, const float v[N]) {
        V r;
#pragma unroll
        for (int i = 0; i < N; ++i) r[i] = (E)v[i];
        *reinterpret_cast<V*>(p) = r;
    }
};
template <>
struct RawVec<__bf16, 1> {
    typedef __bf16 type;
    static __device__ __forceinline__ void unpack(const __bf16& r, float v[1]) { v[0] = (float)r; }
    static __device__ __forceinline__ void store(__bf16* p, const float v[1]) { *p = (__bf16)v[0]; }
};
template <>
struct RawVec<float, 1> {
    typedef float type;
    static __device__ __forceinline__ void unpack(const float& r, float v[1]) { v[0] = r; }
    static __device__ __forceinline__ void store(float* p, const float v[1]) { *p = v[0]; }
};
template <> struct RawVec<__bf16, 2> : RawVecImpl<2, bf16x2, __bf16> {};
template <> struct RawVec<__bf16, 4> : RawVecImpl<4, bf16x4, __bf16> {};
template <> struct RawVec<__bf16, 8> : RawVecImpl<8, bf16x8, __bf16> {};
template <> struct RawVec<float, 2> : RawVecImpl<2, floatx2, float> {};
template <> struct RawVec<float, 8> : RawVecImpl<8, floatx8, float> {};

// ---- raw buffer loads ---------------------------------------------------------
// A buffer resource covers [base, base + bytes); loads whose offset falls
// outside return zero, which is how rows past the end of a sequence are padded.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferWord3 = 0x00020000;   // raw (untyped) buffer, gfx9 family

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             kBufferWord3);
}

template <typename T, int N>
struct BufLoad;
template <>
struct BufLoad<__bf16, 1> {
    static __device__ __forceinline__ __bf16 load(rsrc_t r, int off) {
        return __builtin_bit_cast(__bf16, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
    }
};
template <>
struct BufLoad<__bf16, 2> {
    static __device__ __forceinline__ bf16x2 load(rsrc_t r, int off) {
        return __builtin_bit_cast(bf16x2, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
};
template <>
struct BufLoad<__bf16, 4> {
    static __device__ __forceinline__ bf16x4 load(rsrc_t r, int off) {
        return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    }
};
template <>
struct BufLoad<__bf16, 8> {
    static __device__ __forceinline__ bf16x8 load(rsrc_t r, int off) {
        return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
};
template <>
struct BufLoad<float, 1> {
    static __device__ __forceinline__ float load(rsrc_t r, int off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    }
};
template <>
struct BufLoad<float, 2> {
    static __device__ __forceinline__ floatx2 load(rsrc_t r, int off) {
        return __builtin_bit_cast(floatx2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    }
};
template <>
struct BufLoad<float, 8> {
    // Whole-vector casts only: assembling the result from per-element casts of
    // the two 128-bit loads has been seen to compile into 32-bit loads.
    static __device__ __forceinline__ floatx8 load(rsrc_t r, int off) {
        const floatx4 a = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
        const floatx4 b = __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
        return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

// ---- math --------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float sigmoidf_(float x) { return fast_rcp(1.0f + fast_exp2(-x * kLog2e)); }
__device__ __forceinline__ float siluf_(float x) { return x * sigmoidf_(x); }
__device__ __forceinline__ float clamp_log_decay(float g) {
    return __builtin_amdgcn_fmed3f(g, kLogDecayMin, 0.0f);
}
// 1/sqrt(x) with one Newton step on top of the hardware estimate.
__device__ __forceinline__ float rsqrt_nr(float x) {
    float r = __builtin_amdgcn_rsqf(x);
    return r * (1.5f - 0.5f * x * r * r);
}

// Row exchanges between two registers (gfx950 permlane swaps; both are read
// and written): swap16 trades the odd 16-lane rows of a for the even rows of
// b, swap32 rows 2, 3 of a for rows 0, 1 of b.  asm with the wait states for
// the VALU writes of the operands ahead (the compiler's builtin lost the
// second register's result when the operands differed).
__device__ __forceinline__ void rows_swap16(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void rows_swap32(float& a, float& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64), the
// same value in every lane of a group (each step adds two partial sums that
// the paired lanes hold in swapped order).  Within a 16-lane row by DPP:
// quad permutations for 2 and 4 lanes, the half-row and row mirrors for 8
// and 16 (after the quad steps a lane and its mirror hold the sums of the
// two halves); across rows by permlane swaps.  The whole wave must be
// active.  (Lane shuffles through the LDS crossbar, ds_bpermute, cost an LDS
// round trip per step.)
template <int width>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(width >= 1 && width <= 64 && (width & (width - 1)) == 0, "group width");
    if constexpr (width >= 2) v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (width >= 4) v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (width >= 8) v += dpp_f<0x141>(v);   // row_half_mirror
    if constexpr (width >= 16) v += dpp_f<0x140>(v);  // row_mirror
    if constexpr (width >= 32) {
        float a = v, b = v;
        rows_swap16(a, b);   // a: rows 0, 0, 2, 2   b: rows 1, 1, 3, 3
        v = a + b;
    }
    if constexpr (width >= 64) {
        float a = v, b = v;
        rows_swap32(a, b);   // a: rows 0, 1, 0, 1   b: rows 2, 3, 2, 3
        v = a + b;
    }
    return v;
}

// ---- MFMA fragments (16 x 16 output tiles) -----------------------------------
// A operand: lane l supplies row (l % 16) and KPL consecutive k's starting at
// KPL * (l / 16); B operand symmetric with the column index; the 4 accumulator
// values of lane l are rows 4 * (l / 16) + i, column l % 16.
template <typename OpT>
struct Mma;

template <>
struct Mma<__bf16> {
    static constexpr int KPL = 8;   // operand elements per lane
    static constexpr int KI = 32;   // reduction depth per instruction
    typedef bf16x8 frag;
    static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag load(const __bf16* p) {
        return *reinterpret_cast<const frag*>(p);
    }
    static __device__ __forceinline__ frag pack(const float v[8]) {
        frag f;
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = (__bf16)v[i];
        return f;
    }
    static __device__ __forceinline__ void unpack(frag f, float v[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)f[i];
    }
};

template <>
struct Mma<float> {
    static constexpr int KPL = 1;
    static constexpr int KI = 4;
    typedef float frag;
    static __device__ __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag load(const float* p) { return *p; }
    static __device__ __forceinline__ frag pack(const float v[1]) { return v[0]; }
    static __device__ __forceinline__ void unpack(frag f, float v[1]) { v[0] = f; }
};

__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }

}  // namespace kda
