// kda_launch.hpp -- host-side launchers of the gfx950 kernels (internal).
// Arguments are validated by the C ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

hipError_t launch_gated_norm(const void* o, const void* gate, const float* w, void* y,
                             int64_t rows, int D, float eps, int dtype, hipStream_t s);

hipError_t launch_conv(const void* x, const float* w, void* y, const void* state_in,
                       void* state_out, const int32_t* cu, int num_seqs, int T, int64_t N,
                       int H, int D, int dtype, float l2_eps, hipStream_t s);

// kda_conv with MXFP8 output: codes [N, 3*H*D], scales [N, H, D/32] per part.
hipError_t launch_conv_mxfp8(const void* x, const float* w, void* codes, void* q_scale,
                             void* k_scale, void* v_scale, const void* state_in, void* state_out,
                             const int32_t* cu, int num_seqs, int T, int64_t N, int H, int D,
                             float l2_eps, hipStream_t s);

hipError_t launch_decode(const void* x, const float* w, void* conv_state, const void* g,
                         const void* beta, float* state, void* o, int B, int H, int D,
                         int dtype, float l2_eps, hipStream_t s);

// K tokens per sequence from state_in / cs_in; states after n_tokens[b]
// tokens to state_out / cs_out (both null: outputs only).
hipError_t launch_decode_multi(const void* x, const float* w, const void* cs_in, void* cs_out,
                               const void* g, const void* beta, const float* state_in,
                               float* state_out, void* o, const int32_t* n_tokens, int B, int K,
                               int H, int D, int dtype, float l2_eps, hipStream_t s);

// Chunked prefill configuration chosen on the host.
struct ChunkPlan {
    int nb;       // 16-token blocks per chunk (chunk = 16 * nb)
    int dvs;      // value columns per workgroup (DV / dvs workgroups per head)
    bool ok;      // false when no compiled variant fits the request
    bool pipe;    // bf16, 16-token chunks: producer / consumer wave kernel
};
ChunkPlan plan_chunk(int dtype, int DK, int DV, int chunk, int64_t n_chains);

// bf16, 16-token chunks, 64 value columns per workgroup (kda_chunk_pipe.hip).
hipError_t launch_chunk_pipe(const void* q, const void* k, const void* v, int64_t stride,
                             const void* g, const void* beta, void* o, const float* s0,
                             float* sT, const int32_t* cu, int num_seqs, int T, int H, int DK,
                             int DV, hipStream_t s);

// MXFP8 q, k, v, g (E4M3 codes; E8M0 scales [tokens, H, 4] per tensor), bf16
// beta and o, DK = DV = 128, 16-token chunks (kda_chunk_pipe.hip).
hipError_t launch_chunk_pipe_mxfp8(const void* q, const void* qsc, const void* k,
                                   const void* ksc, const void* v, const void* vsc,
                                   int64_t stride, const void* g, const void* gsc,
                                   const void* beta, void* o, const float* s0, float* sT,
                                   const int32_t* cu, int num_seqs, int T, int H, hipStream_t s);

hipError_t launch_chunk(const ChunkPlan& plan, const void* q, const void* k, const void* v,
                        int64_t stride, const void* g, const void* beta, void* o,
                        const float* s0, float* sT, const int32_t* cu, int num_seqs, int T,
                        int H, int DK, int DV, int dtype, hipStream_t s);

// The 16-token kernel reading the projected inputs before the short conv:
// x [N, 3*H*D] bf16 (q | k | v parts), conv taps cw [3*H*D, 4] fp32, conv
// state cs_in [num_seqs, 3*H*D, 3] bf16 or null; the producers run conv,
// SiLU and L2 (kda_chunk_pipe.hip).  D = 64 or 128; o [N, H, D] bf16.
hipError_t launch_chunk_pipe_conv(const void* x, const float* cw, const void* cs_in,
                                  const void* g, const void* beta, void* o, const float* s0,
                                  float* sT, const int32_t* cu, int num_seqs, int T, int H, int D,
                                  float l2_eps, hipStream_t s);

// The rolling conv state alone (the state pass of kda_conv, kda_conv.hip).
hipError_t launch_conv_state(const void* x, const void* state_in, void* state_out,
                             const int32_t* cu, int num_seqs, int T, int64_t N, int H, int D,
                             int dtype, hipStream_t s);

// Gated latent-attention decode step (kda_mla.hip): bf16, latent 512, heads of
// 128, H a multiple of 16 up to 96.
int mla_splits(int B, int Lmax);
int64_t mla_workspace_bytes(int B, int H, int Lmax);
// The current device's address of the library's static decode scratch
// (KDA_MLA_NOALLOC_MAX_BYTES, 256-byte aligned); null with *err set on failure.
void* mla_scratch(hipError_t* err);
hipError_t launch_mla_decode(const void* q, const void* w_uk, const void* w_uv,
                             const void* cache, const int32_t* lengths, const void* gate, void* y,
                             void* workspace, int B, int H, int Lmax, float scale,
                             hipStream_t s);

}  // namespace kda
