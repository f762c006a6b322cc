/*
 * kda.h -- C ABI of the MI355X (gfx950) KDA token-mixer library, libkda.so.
 *
 * Kimi Delta Attention as drawn on "Inside Kimi K3" (lei.chat): the KDA
 * one-head diagram (projections into 96 heads of 128 dims, Swish and L2 norm of
 * q and k, channel-wise retention alpha and write strength beta with the
 * log-decay bounded below by -5, a recurrent state updated by a decay and a
 * delta-rule correction and evaluated chunkwise, the read S_t^T q_t, head
 * RMSNorm and a full-rank sigmoid gate) and the KDA short-convolution diagram
 * (a causal width-4 depthwise filter per channel, SiLU, the rolling state of the
 * 3 previous raw inputs per channel of the combined QKV).  The state update is
 * the one in the local-memory panel of "Animated Kimi K3 architecture diagram"
 * (github.io): decay S with Diag(alpha_t), probe it with k_t, correct with
 * e_t = v_t - Sbar_t^T k_t and write beta_t k_t e_t^T.
 *
 * Common rules for every entry point
 * ----------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *   allocates no device memory and keeps no state besides a thread-local error
 *   string.
 * - Every call is asynchronous on the caller's stream `s` (0 = null stream) and
 *   returns an int status; the message of the last failure on the calling
 *   thread is kda_last_error().  No C++ exception crosses the ABI.
 * - Arguments are checked on the host before anything is launched; a failed
 *   check launches nothing and returns KDA_ERR_INVALID_ARG or
 *   KDA_ERR_UNSUPPORTED.  KDA_ERR_HIP reports a launch failure.
 * - `dtype` (KDA_F32 or KDA_BF16) is the element type of every per-token
 *   tensor (x, y, q, k, v, g, beta, gate, o, conv states).  Recurrent states
 *   are always fp32; conv filter weights and RMSNorm weights are always fp32.
 *   Arithmetic is fp32 on the GPU in both modes; bf16 values are rounded to
 *   nearest-even when stored.
 * - Pointers to per-token tensors must be 16-byte aligned; token strides are
 *   in elements and must be multiples of 8.
 * - Results are deterministic: no atomics, fixed reduction orders.
 * - Packed variable-length batches: when `cu_seqlens` (device int32
 *   [num_seqs + 1], cu_seqlens[0] = 0, non-decreasing) is non-null, B must be
 *   1 and T must equal cu_seqlens[num_seqs]; sequence i occupies tokens
 *   [cu_seqlens[i], cu_seqlens[i+1]).  When it is null, there are B sequences
 *   of T tokens each (num_seqs is ignored and taken as B).  The offsets live
 *   in device memory and are not read on the host.  The kernels clamp each
 *   sequence's range to [0, T] (start first, then end to [start, T]), so
 *   offsets that break the rules give wrong results but never an access out
 *   of bounds.  Debug check: with the environment variable
 *   KDA_CHECK_CU_SEQLENS set to a value other than 0, the calls that take
 *   cu_seqlens copy it to the host (waiting for the stream) and return
 *   KDA_ERR_INVALID_ARG, launching nothing, unless it starts at 0, never
 *   decreases and ends at T.
 * - Shapes: H >= 1 heads; head sizes D, DK, DV in {64, 128}.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum kda_status {
    KDA_OK = 0,
    KDA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, forbidden alias */
    KDA_ERR_UNSUPPORTED = 2, /* valid request this build does not implement */
    KDA_ERR_HIP = 3          /* a kernel launch failed */
};

enum kda_dtype { KDA_F32 = 0, KDA_BF16 = 1 };

/* Library version, e.g. 100 for 1.0.0. */
int kda_version(void);

/* Message describing the last non-zero status returned on this thread
 * ("" if none).  The pointer stays valid until the next call on the thread. */
const char* kda_last_error(void);

/*
 * kda_conv -- short causal convolution + SiLU over projected q|k|v, then L2
 * normalisation of q and k per (token, head).
 * ("Inside Kimi K3", KDA short-convolution diagram; KDA one-head diagram.)
 *
 *   x              [B*T, 3*H*D]  projected inputs, token-major; channel index
 *                                part*H*D + h*D + d with part 0 = q, 1 = k, 2 = v
 *   w              [3*H*D, 4]    fp32 filter banks (q bank, k bank, v bank);
 *                                tap 0 multiplies x_{t-3}, tap 3 multiplies x_t
 *   y              [B*T, 3*H*D]  output: SiLU(conv) for all three parts, then
 *                                q and k divided by sqrt(sum_d u_d^2 + l2_eps)
 *   conv_state_in  [num_seqs, 3*H*D, 3] or NULL: raw inputs preceding each
 *                                sequence, oldest first (NULL = zeros)
 *   conv_state_out [num_seqs, 3*H*D, 3] or NULL: the last 3 raw inputs of each
 *                                sequence's window (from conv_state_in where a
 *                                sequence is shorter than 3); may equal
 *                                conv_state_in (updated in place)
 *   l2_eps         > 0, added under the square root (1e-6 in the tests)
 * The sequence length is preserved and channels never mix; windows never
 * cross sequence boundaries.  y must not overlap x.
 */
int kda_conv(const void* x, const float* w, void* y, const void* conv_state_in,
             void* conv_state_out, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
             int32_t T, int32_t H, int32_t D, int32_t dtype, float l2_eps, hipStream_t s);

/*
 * kda_conv_mxfp8 -- kda_conv on bf16 inputs with its output written as MXFP8
 * activations (the OCP microscaling reading of "Inside Kimi K3", model at a
 * glance; the code and scale formats are those of kda_chunk_prefill_mxfp8
 * below), ready to be read in place by kda_chunk_prefill_mxfp8.
 *
 *   x, w, conv_state_in, conv_state_out, cu_seqlens, num_seqs, B, T, H, D,
 *   l2_eps          as in kda_conv, with x and the states in bf16
 *   y_codes         [B*T, 3*H*D] E4M3 codes of kda_conv's y (q | k | v)
 *   q_scale, k_scale, v_scale
 *                   [B*T, H, D/32] E8M0 scale bytes, one per block of 32
 *                   consecutive channels of a head
 * Per block, the scale exponent e is the smallest integer with
 * max|y| <= 448 * 2^e (clamped to [-127, 127]; an all-zero block gets
 * scale byte 0), and each code is y * 2^-e rounded to the nearest E4M3
 * value, ties to even, from y in fp32.  D = 64 or 128.  x, y_codes and the
 * states must be 16-byte aligned, the scale pointers D/32-byte aligned;
 * y_codes and the scales must not overlap x or each other.
 */
int kda_conv_mxfp8(const void* x, const float* w, void* y_codes, void* q_scale, void* k_scale,
                   void* v_scale, const void* conv_state_in, void* conv_state_out,
                   const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                   int32_t D, float l2_eps, hipStream_t s);

/*
 * kda_chunk_prefill -- the gated delta rule over whole sequences, evaluated
 * chunkwise: parallel within a chunk of `chunk` tokens, recurrent across
 * chunks.  ("Inside Kimi K3", KDA one-head diagram; "Animated Kimi K3
 * architecture diagram", local-memory panel.)  Per head and token t:
 *   Sbar = Diag(exp(g_t)) S_{t-1};  e = v_t - Sbar^T k_t;
 *   S_t = Sbar + beta_t k_t e^T;    o_t = S_t^T q_t.
 *
 *   q, k           [B*T, *] rows of H*DK elements at token stride
 *                  qkv_token_stride (pass 3*H*DK to read kda_conv's y in place,
 *                  or H*DK for separate tensors); q and k L2-normalised by the
 *                  caller (kda_conv does it)
 *   v              [B*T, *] rows of H*DV elements, same token stride
 *   g              [B*T, H, DK] log-decay, precondition -5 <= g <= 0; both this
 *                  kernel and the CPU oracle clamp it to [-5, 0]
 *   beta           [B*T, H] write strength in (0, 1), already activated
 *   o              [B*T, H, DV] output
 *   initial_state  [num_seqs, H, DK, DV] fp32 or NULL (zeros)
 *   final_state    [num_seqs, H, DK, DV] fp32 or NULL (not written); may equal
 *                  initial_state (updated in place)
 *   chunk          tokens per chunk: 16, 32 or 64 (bf16; 16 is the fastest
 *                  and runs on separate producer and consumer waves); 16, 32
 *                  or 64 (fp32, where DK = 128 allows at most 32); 0 picks the
 *                  fastest (16 for bf16; 32 for fp32 with DK = 128, else 64).
 *                  The result does not depend on it beyond rounding
 * o must not overlap any input.  Unsupported (dtype, DK, DV, chunk)
 * combinations return KDA_ERR_UNSUPPORTED.
 */
int kda_chunk_prefill(const void* q, const void* k, const void* v, int64_t qkv_token_stride,
                      const void* g, const void* beta, void* o, const float* initial_state,
                      float* final_state, const int32_t* cu_seqlens, int32_t num_seqs,
                      int32_t B, int32_t T, int32_t H, int32_t DK, int32_t DV, int32_t chunk,
                      int32_t dtype, hipStream_t s);

/*
 * kda_chunk_prefill_mxfp8 -- kda_chunk_prefill (16-token chunks, fp32
 * state) with q, k, v and g given as MXFP8 activations.  ("Inside Kimi K3",
 * model at a glance: activations quantised to MXFP8; read as the OCP
 * microscaling format.)  Each tensor is a byte array of E4M3 codes (sign, 4
 * exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities,
 * S.1111.111 = NaN) and a byte array of E8M0 scales, one per 32 consecutive
 * channels: value = e4m3(code) * 2^(scale - 127), scale 255 = NaN.
 *
 *   q, k, v      [B*T, *] rows of H*128 codes at token stride
 *                qkv_token_stride bytes (a multiple of 16, >= H*128)
 *   q_scale, k_scale, v_scale, g_scale
 *                [B*T, H, 4] scale bytes, contiguous
 *   g            [B*T, H, 128] codes of the log-decay (clamped to [-5, 0]
 *                after decoding, as in kda_chunk_prefill)
 *   beta         [B*T, H] bf16; o [B*T, H, 128] bf16
 *   initial_state, final_state, cu_seqlens, num_seqs, B, T: as in
 *                kda_chunk_prefill (fp32 states, may alias)
 * DK = DV = 128 only (others: KDA_ERR_UNSUPPORTED).  Code pointers, beta,
 * o and the states must be 16-byte aligned; scale pointers need no
 * alignment.  o must not overlap any input.
 */
int kda_chunk_prefill_mxfp8(const void* q, const void* q_scale, const void* k,
                            const void* k_scale, const void* v, const void* v_scale,
                            int64_t qkv_token_stride, const void* g, const void* g_scale,
                            const void* beta, void* o, const float* initial_state,
                            float* final_state, const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t B, int32_t T, int32_t H, int32_t DK, int32_t DV,
                            hipStream_t s);

/*
 * kda_prefill_fused -- the whole prefill path with the short conv run inside
 * the chunked recurrence: the recurrence's producer waves read the projected
 * inputs before the conv and compute the conv, SiLU and the L2 norm of q and
 * k themselves, so q, k and v never go through memory; then the gated head
 * RMSNorm.  ("Inside Kimi K3", KDA short-convolution diagram and KDA one-head
 * diagram: projections -> conv + SiLU -> L2 norm of q, k -> recurrent state
 * -> head RMSNorm times a sigmoid gate.)  Same results as kda_conv ->
 * kda_chunk_prefill (16-token chunks) -> kda_gated_norm up to rounding: q
 * and k are normalised in fp32 here instead of passing through bf16 first.
 *
 *   x, conv_w, conv_state_in, conv_state_out, cu_seqlens, num_seqs, B, T, H,
 *   D, l2_eps          as in kda_conv
 *   g, beta, initial_state, final_state
 *                      as in kda_chunk_prefill (DK = DV = D)
 *   gate, norm_w, rms_eps
 *                      as kda_gated_norm's gate, weight and eps
 *   o                  [B*T, H, D] the recurrence's output S_t^T q_t (the
 *                      norm's input); may equal y
 *   y                  [B*T, H, D] the gated RMSNorm of o
 * Launches the fused recurrence kernel, the rolling-state pass (when
 * conv_state_out is given) and the gated norm, in that order on `s`.  The
 * gated norm is a separate pass: a head's 128 value columns are split over
 * two workgroups, and the norm needs all of them.  bf16 only (fp32 returns
 * KDA_ERR_UNSUPPORTED); D = 64 or 128.  final_state may equal initial_state
 * and conv_state_out may equal conv_state_in (updated in place); o and y
 * overlap no input and nothing else.
 */
int kda_prefill_fused(const void* x, const float* conv_w, const void* g, const void* beta,
                      const void* gate, const float* norm_w, void* o, void* y,
                      const void* conv_state_in, void* conv_state_out,
                      const float* initial_state, float* final_state,
                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                      int32_t H, int32_t D, int32_t dtype, float l2_eps, float rms_eps,
                      hipStream_t s);

/*
 * kda_decode_step -- one new token for each of B sequences: the conv window
 * [conv_state (3 values), x_t] per channel, SiLU, L2 of q and k, then one
 * gated-delta-rule step.  ("Inside Kimi K3", KDA short-convolution diagram,
 * autoregressive rolling state; KDA one-head diagram.)
 *
 *   x           [B, 3*H*D]     projected new token (before the conv)
 *   w           [3*H*D, 4]     fp32 filter banks, as in kda_conv
 *   conv_state  [B, 3*H*D, 3]  rolling raw inputs, oldest first; updated in
 *                              place to [x_{t-2}, x_{t-1}, x_t]
 *   g           [B, H, D]      log-decay (clamped to [-5, 0]); beta [B, H]
 *   state       [B, H, D, D]   fp32 recurrent state, updated in place
 *   o           [B, H, D]      output S_t^T q_t; must not overlap any input
 */
int kda_decode_step(const void* x, const float* w, void* conv_state, const void* g,
                    const void* beta, float* state, void* o, int32_t B, int32_t H, int32_t D,
                    int32_t dtype, float l2_eps, hipStream_t s);

/*
 * kda_decode_multi -- K new tokens for each of B sequences in one pass over
 * the states: the check of K drafted tokens in speculative decoding ("Kimi
 * K3" on archdiff.com, component list: the MTP layer used as an EAGLE-3
 * drafter, and speculative decoding by MTP self-drafting).  Token t of
 * sequence b is exactly the step of kda_decode_step applied after tokens
 * 0 .. t-1 of the same sequence.
 *
 *   x               [B, K, 3*H*D]  projected new tokens (before the conv)
 *   w               [3*H*D, 4]     fp32 filter banks, as in kda_conv
 *   conv_state_in   [B, 3*H*D, 3]  rolling raw inputs before token 0
 *   g               [B, K, H, D]   log-decay (clamped to [-5, 0])
 *   beta            [B, K, H]
 *   state_in        [B, H, D, D]   fp32 recurrent state before token 0
 *   n_tokens        [B] int32 on the device, or NULL (= K for every
 *                   sequence): how many leading tokens of sequence b the output
 *                   states take in; values are clamped to [0, K]
 *   state_out       [B, H, D, D]   fp32 state after n_tokens[b] tokens
 *   conv_state_out  [B, 3*H*D, 3]  rolling raw inputs after n_tokens[b] tokens
 *   o               [B, K, H, D]   S_t^T q_t for all K tokens, or NULL
 *
 * state_out and conv_state_out are both given or both NULL (NULL: outputs
 * only, nothing is written back).  Each output state is either exactly its
 * input (in place) or disjoint from every other tensor; o overlaps nothing.
 * With o NULL only the first n_tokens[b] tokens are processed.  Rollback after
 * a check: call once with the states NULL (outputs only), then once more with
 * o NULL, n_tokens = the accepted counts and the states in place.  The state
 * is read once per call and written at most once.  1 <= K <= 64; a larger K
 * is KDA_ERR_UNSUPPORTED.
 */
#define KDA_DECODE_MULTI_MAX_K 64
int kda_decode_multi(const void* x, const float* w, const void* conv_state_in,
                     void* conv_state_out, const void* g, const void* beta,
                     const float* state_in, float* state_out, void* o, const int32_t* n_tokens,
                     int32_t B, int32_t K, int32_t H, int32_t D, int32_t dtype, float l2_eps,
                     hipStream_t s);

/*
 * kda_gated_norm -- head RMSNorm times a full-rank sigmoid gate.
 * ("Inside Kimi K3", KDA one-head diagram: head RMSNorm and sigmoid gate.)
 *   y[t,h,d] = o[t,h,d] / sqrt(mean_d o[t,h,d]^2 + eps) * weight[d]
 *              * sigmoid(gate[t,h,d])
 *   o, gate, y  [n_tokens, H, D]; gate holds pre-sigmoid logits
 *   weight      [D] fp32, shared by all heads
 * y may equal o (in place); otherwise it must not overlap the inputs.
 */
int kda_gated_norm(const void* o, const void* gate, const float* weight, void* y,
                   int64_t n_tokens, int32_t H, int32_t D, float eps, int32_t dtype,
                   hipStream_t s);

/*
 * kda_mla_decode -- one decode step of gated multi-head latent attention over
 * the latent cache.  ("Inside Kimi K3" (lei.chat), gated multi-head latent
 * attention diagram: a 512-wide KV latent per token is cached; learned
 * up-projections rebuild keys and values of 128 per head for 96 heads, no
 * positional encoding; the new token's query takes a causal softmax over the
 * cached tokens; the head output times a full-rank sigmoid gate.)
 *
 *   y[b,h,:] = sigmoid(gate[b,h,:]) * sum_i p_i W_uv[h] c_{b,i}
 *   p = softmax_i(scale * q[b,h,:] . (W_uk[h] c_{b,i})),  i < lengths[b]
 *
 *   q        [B, H, Dk]        bf16 queries of the new token
 *   w_uk     [H, Dk, R]        bf16 key up-projection (row d of head h)
 *   w_uv     [H, Dv, R]        bf16 value up-projection
 *   cache    [B, L_max, R]     bf16 latents c_i; the new token's own latent is
 *                              already stored at position lengths[b] - 1
 *   lengths  [B] int32 on the device: cached tokens per sequence, clamped to
 *            [1, L_max]; rows at or past lengths[b] are never read
 *   gate     [B, H, Dv]        bf16 gate logits (before the sigmoid)
 *   y        [B, H, Dv]        bf16 output; overlaps no other tensor
 *   workspace  device scratch of at least kda_mla_decode_workspace_bytes(B,
 *              H, L_max) bytes, owned by the caller, disjoint from every
 *              tensor; its contents on entry do not matter
 *
 * The key up-projection is folded into the query (q' = W_uk^T q, rounded to
 * bf16) so all heads share one read of the cache; the value up-projection is
 * applied after the softmax-weighted sum of latents.  This build supports
 * dtype KDA_BF16, R = 512, Dk = Dv = 128 and H a multiple of 16 up to 96
 * (others: KDA_ERR_UNSUPPORTED); scale must be finite and > 0.  B = 0 launches
 * nothing and reads no pointer.  Calls that share a workspace must not overlap
 * in time.
 */
int64_t kda_mla_decode_workspace_bytes(int32_t B, int32_t H, int32_t L_max);
int kda_mla_decode(const void* q, const void* w_uk, const void* w_uv, const void* cache,
                   const int32_t* lengths, const void* gate, void* y, void* workspace,
                   int64_t workspace_bytes, int32_t B, int32_t H, int32_t L_max, int32_t R,
                   int32_t Dk, int32_t Dv, float scale, int32_t dtype, hipStream_t s);

/*
 * kda_mla_decode_noalloc -- kda_mla_decode for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, bitwise the same y, with the
 * workspace replaced by a static device array of the library of
 * KDA_MLA_NOALLOC_MAX_BYTES (128 MiB), which each GPU that runs the library
 * holds until the process ends.  Arguments, layouts and checks are those of
 * kda_mla_decode without `workspace` / `workspace_bytes`.
 *
 * - A call whose kda_mla_decode_workspace_bytes(B, H, L_max) exceeds
 *   KDA_MLA_NOALLOC_MAX_BYTES returns KDA_ERR_INVALID_ARG and launches
 *   nothing (B = 256, H = 96 needs about 75 MiB at any L_max; every B <= 256
 *   with H <= 96 fits).
 * - Nothing is allocated: the array's device address is looked up once per
 *   device, on the first call with that device current.
 * - Every call on a GPU shares that GPU's array, which keeps the last call's
 *   contents (no call depends on them).  Calls that overlap in time on one
 *   GPU (other streams, other threads) race on it: serialise them.
 */
#define KDA_MLA_NOALLOC_MAX_BYTES (128LL << 20)
int kda_mla_decode_noalloc(const void* q, const void* w_uk, const void* w_uv, const void* cache,
                           const int32_t* lengths, const void* gate, void* y, int32_t B,
                           int32_t H, int32_t L_max, int32_t R, int32_t Dk, int32_t Dv,
                           float scale, int32_t dtype, hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
