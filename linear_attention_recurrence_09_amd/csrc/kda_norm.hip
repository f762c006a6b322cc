// kda_norm.hip -- head RMSNorm times a full-rank sigmoid gate (gfx950).
//
// "Inside Kimi K3" (lei.chat), KDA one-head diagram: the read is normalised
// per head (RMSNorm over the head's D values, weight shared by heads) and
// multiplied elementwise by sigmoid of the gate logits.
//
// HBM-bound: per element 2 reads (o, gate) and 1 write (y).  Each thread owns
// 8 consecutive elements of a row (one 16-byte bf16 vector per tensor) and
// D/8 lanes reduce a row with xor shuffles.  One row per thread: the small
// register footprint keeps more waves resident, which puts more bytes in
// flight than batching several rows per thread (measured: 1 row 0.76 ms,
// 2 rows 0.78 ms, 4 rows 0.81 ms, 8 rows 0.95 ms at 65,536 x 96 rows).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int kNormThreads = 256;
constexpr int kNormRowsPerThread = 1;

template <typename T, int D>
__global__ void __launch_bounds__(kNormThreads)
gated_norm_kernel(const T* o, const T* __restrict__ gate,
                  const float* __restrict__ w, T* y, int64_t rows, float eps) {
    constexpr int LPR = D / 8;                       // lanes per row
    constexpr int RPP = kNormThreads / LPR;          // rows per pass of the block
    const int lane_in_row = threadIdx.x % LPR;
    const int row_in_pass = threadIdx.x / LPR;
    const int64_t row0 = (int64_t)blockIdx.x * RPP * kNormRowsPerThread;
    const int d0 = lane_in_row * 8;

    float wv[8];
    load8(w + d0, wv);

    float ov[kNormRowsPerThread][8], zv[kNormRowsPerThread][8];
#pragma unroll
    for (int j = 0; j < kNormRowsPerThread; ++j) {
        const int64_t r = row0 + (int64_t)j * RPP + row_in_pass;
        if (r < rows) {
            load8_nt(o + r * D + d0, ov[j]);
            load8_nt(gate + r * D + d0, zv[j]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) { ov[j][e] = 0.f; zv[j][e] = 0.f; }
        }
    }
#pragma unroll
    for (int j = 0; j < kNormRowsPerThread; ++j) {
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += ov[j][e] * ov[j][e];
        ss = group_sum<LPR>(ss);
        const float inv = rsqrt_nr(ss * (1.0f / D) + eps);
        float out[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) out[e] = ov[j][e] * inv * wv[e] * sigmoidf_(zv[j][e]);
        const int64_t r = row0 + (int64_t)j * RPP + row_in_pass;
        if (r < rows) store8_nt(y + r * D + d0, out);
    }
}

template <typename T, int D>
hipError_t launch_norm_t(const void* o, const void* gate, const float* w, void* y, int64_t rows,
                         float eps, hipStream_t s) {
    constexpr int rows_per_block = (kNormThreads / (D / 8)) * kNormRowsPerThread;
    const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((gated_norm_kernel<T, D>), dim3((unsigned)blocks), dim3(kNormThreads), 0,
                       s, (const T*)o, (const T*)gate, w, (T*)y, rows, eps);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_norm(const void* o, const void* gate, const float* w, void* y,
                             int64_t rows, int D, float eps, int dtype, hipStream_t s) {
    if (dtype == 0) {
        return D == 64 ? launch_norm_t<float, 64>(o, gate, w, y, rows, eps, s)
                       : launch_norm_t<float, 128>(o, gate, w, y, rows, eps, s);
    }
    return D == 64 ? launch_norm_t<__bf16, 64>(o, gate, w, y, rows, eps, s)
                   : launch_norm_t<__bf16, 128>(o, gate, w, y, rows, eps, s);
}

}  // namespace kda
