// kda_api.cpp -- the C ABI declared in include/kda.h: host-side argument
// checks, then one or two kernel launches on the caller's stream.
#include "kda.h"

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "kda_launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok() {
    return KDA_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(KDA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [a, a + na) and [b, b + nb) intersect (byte ranges)
bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
    if (a == nullptr || b == nullptr || na <= 0 || nb <= 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int64_t esize(int dtype) { return dtype == KDA_F32 ? 4 : 2; }

bool valid_dtype(int dtype) { return dtype == KDA_F32 || dtype == KDA_BF16; }
bool valid_head(int d) { return d == 64 || d == 128; }

// Resolve (cu_seqlens, num_seqs, B, T) into the sequence count and total tokens.
int seq_layout(const char* fn, const int32_t* cu, int32_t num_seqs, int32_t B, int32_t T,
               int* n_seqs, int64_t* n_tok) {
    if (T < 0) return fail(KDA_ERR_INVALID_ARG, "%s: T must be >= 0 (got %d)", fn, T);
    if (cu != nullptr) {
        if (B != 1) return fail(KDA_ERR_INVALID_ARG, "%s: cu_seqlens requires B == 1 (got %d)", fn, B);
        if (num_seqs < 0) return fail(KDA_ERR_INVALID_ARG, "%s: num_seqs must be >= 0", fn);
        if (num_seqs == 0 && T > 0)
            return fail(KDA_ERR_INVALID_ARG, "%s: T > 0 tokens but num_seqs == 0", fn);
        *n_seqs = num_seqs;
        *n_tok = T;
    } else {
        if (B < 0) return fail(KDA_ERR_INVALID_ARG, "%s: B must be >= 0 (got %d)", fn, B);
        *n_seqs = B;
        *n_tok = (int64_t)B * T;
    }
    return KDA_OK;
}

// Debug check of packed offsets, on when the environment sets
// KDA_CHECK_CU_SEQLENS to a value other than 0: the offsets are copied to the
// host (this waits for the stream) and must start at 0, never decrease and
// end at T.  The kernels clamp every sequence to [0, T] in any case, so bad
// offsets cannot move an access out of bounds; the check reports them.
int check_cu(const char* fn, const int32_t* cu, int num_seqs, int64_t T, hipStream_t s) {
    const char* env = std::getenv("KDA_CHECK_CU_SEQLENS");
    if (cu == nullptr || env == nullptr || env[0] == '\0' || env[0] == '0') return KDA_OK;
    std::vector<int32_t> h((size_t)num_seqs + 1);
    if (hipMemcpyAsync(h.data(), cu, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return fail(KDA_ERR_HIP, "%s: reading cu_seqlens failed", fn);
    if (h[0] != 0) return fail(KDA_ERR_INVALID_ARG, "%s: cu_seqlens[0] = %d, not 0", fn, h[0]);
    for (int i = 0; i < num_seqs; ++i)
        if (h[i + 1] < h[i])
            return fail(KDA_ERR_INVALID_ARG, "%s: cu_seqlens decreases at %d (%d > %d)", fn, i + 1,
                        h[i], h[i + 1]);
    if (h[num_seqs] != T)
        return fail(KDA_ERR_INVALID_ARG, "%s: cu_seqlens[%d] = %d, T = %lld", fn, num_seqs,
                    h[num_seqs], (long long)T);
    return KDA_OK;
}

// Argument checks shared by both latent-attention decode entry points (all
// but the scratch).
int mla_args(const char* fn, const void* q, const void* w_uk, const void* w_uv, const void* cache,
             const int32_t* lengths, const void* gate, const void* y, int32_t B, int32_t H,
             int32_t L_max, int32_t R, int32_t Dk, int32_t Dv, float scale, int32_t dtype) {
    if (!valid_dtype(dtype)) return fail(KDA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (dtype != KDA_BF16) return fail(KDA_ERR_UNSUPPORTED, "%s: only bf16 is implemented", fn);
    if (B < 0) return fail(KDA_ERR_INVALID_ARG, "%s: B must be >= 0 (got %d)", fn, B);
    if (B > 65535) return fail(KDA_ERR_UNSUPPORTED, "%s: B must be <= 65535 (got %d)", fn, B);
    if (H < 1) return fail(KDA_ERR_INVALID_ARG, "%s: H must be >= 1 (got %d)", fn, H);
    if (L_max < 1) return fail(KDA_ERR_INVALID_ARG, "%s: L_max must be >= 1 (got %d)", fn, L_max);
    if (R < 1 || Dk < 1 || Dv < 1)
        return fail(KDA_ERR_INVALID_ARG, "%s: R, Dk and Dv must be >= 1", fn);
    if (R != 512 || Dk != 128 || Dv != 128)
        return fail(KDA_ERR_UNSUPPORTED, "%s: needs R = 512, Dk = Dv = 128 (got %d, %d, %d)", fn, R,
                    Dk, Dv);
    if (H % 16 != 0 || H > 96)
        return fail(KDA_ERR_UNSUPPORTED, "%s: H must be a multiple of 16 up to 96 (got %d)", fn, H);
    if (!(scale > 0.f) || !(scale < 3.0e38f))
        return fail(KDA_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
    if (B == 0) return KDA_OK;
    if (q == nullptr || w_uk == nullptr || w_uv == nullptr || cache == nullptr ||
        lengths == nullptr || gate == nullptr || y == nullptr)
        return fail(KDA_ERR_INVALID_ARG, "%s: every pointer must be non-null", fn);
    if (!aligned16(q) || !aligned16(w_uk) || !aligned16(w_uv) || !aligned16(cache) ||
        !aligned16(gate) || !aligned16(y))
        return fail(KDA_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(lengths) & 3u) != 0)
        return fail(KDA_ERR_INVALID_ARG, "%s: lengths must be 4-byte aligned", fn);
    return KDA_OK;
}

// y apart from every tensor and the scratch; the scratch apart from the inputs.
int mla_apart(const char* fn, const void* q, const void* w_uk, const void* w_uv,
              const void* cache, const int32_t* lengths, const void* gate, const void* y,
              const void* ws, int64_t need, int32_t B, int32_t H, int32_t L_max, int32_t R,
              int32_t Dk, int32_t Dv) {
    const int64_t q_b = (int64_t)B * H * Dk * 2, wk_b = (int64_t)H * Dk * R * 2;
    const int64_t wv_b = (int64_t)H * Dv * R * 2, c_b = (int64_t)B * L_max * R * 2;
    const int64_t g_b = (int64_t)B * H * Dv * 2, y_b = g_b, l_b = (int64_t)B * 4;
    if (overlap(y, y_b, q, q_b) || overlap(y, y_b, w_uk, wk_b) || overlap(y, y_b, w_uv, wv_b) ||
        overlap(y, y_b, cache, c_b) || overlap(y, y_b, lengths, l_b) || overlap(y, y_b, gate, g_b) ||
        overlap(y, y_b, ws, need))
        return fail(KDA_ERR_INVALID_ARG, "%s: y must not overlap another tensor", fn);
    if (overlap(ws, need, q, q_b) || overlap(ws, need, w_uk, wk_b) ||
        overlap(ws, need, w_uv, wv_b) || overlap(ws, need, cache, c_b) ||
        overlap(ws, need, lengths, l_b) || overlap(ws, need, gate, g_b))
        return fail(KDA_ERR_INVALID_ARG, "%s: workspace overlaps a tensor", fn);
    return KDA_OK;
}

}  // namespace

extern "C" {

int kda_version(void) { return 100; }

const char* kda_last_error(void) { return g_last_error.c_str(); }

int kda_conv(const void* x, const float* w, void* y, const void* conv_state_in,
             void* conv_state_out, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
             int32_t T, int32_t H, int32_t D, int32_t dtype, float l2_eps, hipStream_t s) {
    const char* fn = "kda_conv";
    if (!valid_dtype(dtype)) return fail(KDA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (H < 1) return fail(KDA_ERR_INVALID_ARG, "%s: H must be >= 1 (got %d)", fn, H);
    if (!valid_head(D)) return fail(KDA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, D);
    if (!(l2_eps > 0.f)) return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps must be > 0", fn);
    if (x == nullptr || w == nullptr || y == nullptr)
        return fail(KDA_ERR_INVALID_ARG, "%s: x, w and y must be non-null", fn);
    int ns;
    int64_t N;
    if (int rc = seq_layout(fn, cu_seqlens, num_seqs, B, T, &ns, &N)) return rc;
    if (int rc = check_cu(fn, cu_seqlens, ns, N, s)) return rc;
    const int64_t P = 3LL * H * D;
    const int64_t es = esize(dtype);
    if (!aligned16(x) || !aligned16(y) || !aligned16(conv_state_in) || !aligned16(conv_state_out))
        return fail(KDA_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
    if (overlap(x, N * P * es, y, N * P * es))
        return fail(KDA_ERR_INVALID_ARG, "%s: y must not overlap x", fn);
    const int64_t sbytes = (int64_t)ns * P * 3 * es;
    if (conv_state_out != nullptr) {
        if (conv_state_out != conv_state_in && overlap(conv_state_in, sbytes, conv_state_out, sbytes))
            return fail(KDA_ERR_INVALID_ARG, "%s: conv_state_out partially overlaps conv_state_in", fn);
        if (overlap(conv_state_out, sbytes, x, N * P * es) || overlap(conv_state_out, sbytes, y, N * P * es))
            return fail(KDA_ERR_INVALID_ARG, "%s: conv_state_out overlaps x or y", fn);
    }
    if (N == 0 && (conv_state_out == nullptr || ns == 0)) return ok();
    return hip_status(kda::launch_conv(x, w, y, conv_state_in, conv_state_out, cu_seqlens, ns,
                                       T, N, H, D, dtype, l2_eps, s),
                      fn);
}

int kda_conv_mxfp8(const void* x, const float* w, void* y_codes, void* q_scale, void* k_scale,
                   void* v_scale, const void* conv_state_in, void* conv_state_out,
                   const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T, int32_t H,
                   int32_t D, float l2_eps, hipStream_t s) {
    const char* fn = "kda_conv_mxfp8";
    if (H < 1) return fail(KDA_ERR_INVALID_ARG, "%s: H must be >= 1 (got %d)", fn, H);
    if (!valid_head(D)) return fail(KDA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, D);
    if (!(l2_eps > 0.f)) return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps must be > 0", fn);
    if (x == nullptr || w == nullptr || y_codes == nullptr || q_scale == nullptr ||
        k_scale == nullptr || v_scale == nullptr)
        return fail(KDA_ERR_INVALID_ARG, "%s: x, w, y_codes and the scales must be non-null", fn);
    int ns;
    int64_t N;
    if (int rc = seq_layout(fn, cu_seqlens, num_seqs, B, T, &ns, &N)) return rc;
    if (int rc = check_cu(fn, cu_seqlens, ns, N, s)) return rc;
    const int64_t P = 3LL * H * D;
    if (!aligned16(x) || !aligned16(y_codes) || !aligned16(conv_state_in) ||
        !aligned16(conv_state_out))
        return fail(KDA_ERR_INVALID_ARG, "%s: x, y_codes and state pointers must be 16-byte aligned",
                    fn);
    const uintptr_t sal = (uintptr_t)(D / 32);   // a head's scale bytes are written together
    if ((uintptr_t)q_scale % sal || (uintptr_t)k_scale % sal || (uintptr_t)v_scale % sal)
        return fail(KDA_ERR_INVALID_ARG, "%s: scale pointers must be %d-byte aligned", fn, D / 32);
    const int64_t xb = N * P * 2, cb = N * P, sb = N * H * (D / 32);
    const void* outs[4] = {y_codes, q_scale, k_scale, v_scale};
    const int64_t lens[4] = {cb, sb, sb, sb};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], lens[i], x, xb))
            return fail(KDA_ERR_INVALID_ARG, "%s: outputs must not overlap x", fn);
        for (int j = 0; j < i; ++j)
            if (overlap(outs[i], lens[i], outs[j], lens[j]))
                return fail(KDA_ERR_INVALID_ARG, "%s: outputs must not overlap each other", fn);
    }
    const int64_t stb = (int64_t)ns * P * 3 * 2;
    if (conv_state_out != nullptr) {
        if (conv_state_out != conv_state_in && overlap(conv_state_in, stb, conv_state_out, stb))
            return fail(KDA_ERR_INVALID_ARG, "%s: conv_state_out partially overlaps conv_state_in", fn);
        if (overlap(conv_state_out, stb, x, xb))
            return fail(KDA_ERR_INVALID_ARG, "%s: conv_state_out overlaps x", fn);
        for (int i = 0; i < 4; ++i)
            if (overlap(conv_state_out, stb, outs[i], lens[i]))
                return fail(KDA_ERR_INVALID_ARG, "%s: conv_state_out overlaps an output", fn);
    }
    if (N == 0 && (conv_state_out == nullptr || ns == 0)) return ok();
    return hip_status(kda::launch_conv_mxfp8(x, w, y_codes, q_scale, k_scale, v_scale,
                                             conv_state_in, conv_state_out, cu_seqlens, ns, T, N,
                                             H, D, l2_eps, s),
                      fn);
}

int kda_chunk_prefill(const void* q, const void* k, const void* v, int64_t qkv_token_stride,
                      const void* g, const void* beta, void* o, const float* initial_state,
                      float* final_state, const int32_t* cu_seqlens, int32_t num_seqs,
                      int32_t B, int32_t T, int32_t H, int32_t DK, int32_t DV, int32_t chunk,
                      int32_t dtype, hipStream_t s) {
    const char* fn = "kda_chunk_prefill";
    if (!valid_dtype(dtype)) return fail(KDA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (H < 1) return fail(KDA_ERR_INVALID_ARG, "%s: H must be >= 1 (got %d)", fn, H);
    if (!valid_head(DK) || !valid_head(DV))
        return fail(KDA_ERR_UNSUPPORTED, "%s: DK and DV must be 64 or 128 (got %d, %d)", fn, DK, DV);
    if (q == nullptr || k == nullptr || v == nullptr || g == nullptr || beta == nullptr || o == nullptr)
        return fail(KDA_ERR_INVALID_ARG, "%s: q, k, v, g, beta and o must be non-null", fn);
    const int64_t row = (int64_t)H * (DK > DV ? DK : DV);
    if (qkv_token_stride < row || qkv_token_stride % 8 != 0)
        return fail(KDA_ERR_INVALID_ARG,
                    "%s: qkv_token_stride must be >= H*max(DK,DV) and a multiple of 8 (got %lld)",
                    fn, (long long)qkv_token_stride);
    int ns;
    int64_t N;
    if (int rc = seq_layout(fn, cu_seqlens, num_seqs, B, T, &ns, &N)) return rc;
    if (int rc = check_cu(fn, cu_seqlens, ns, N, s)) return rc;
    const kda::ChunkPlan plan = kda::plan_chunk(dtype, DK, DV, chunk, (int64_t)ns * H);
    if (!plan.ok)
        return fail(KDA_ERR_UNSUPPORTED, "%s: no variant for dtype=%d DK=%d DV=%d chunk=%d", fn,
                    dtype, DK, DV, chunk);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(o) || !aligned16(initial_state) || !aligned16(final_state))
        return fail(KDA_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
    if ((int64_t)ns * H * (DV / plan.dvs) > 0x7fffffffLL)
        return fail(KDA_ERR_INVALID_ARG, "%s: too many (sequence, head) pairs", fn);
    const int64_t es = esize(dtype);
    const int64_t qkv_bytes = N > 0 ? ((N - 1) * qkv_token_stride + row) * es : 0;
    const int64_t o_bytes = N * H * DV * es;
    if (overlap(o, o_bytes, q, qkv_bytes) || overlap(o, o_bytes, k, qkv_bytes) ||
        overlap(o, o_bytes, v, qkv_bytes) || overlap(o, o_bytes, g, N * H * DK * es) ||
        overlap(o, o_bytes, beta, N * H * es))
        return fail(KDA_ERR_INVALID_ARG, "%s: o must not overlap an input", fn);
    const int64_t st_bytes = (int64_t)ns * H * DK * DV * 4;
    if (final_state != nullptr) {
        if ((const void*)final_state != (const void*)initial_state &&
            overlap(final_state, st_bytes, initial_state, st_bytes))
            return fail(KDA_ERR_INVALID_ARG, "%s: final_state partially overlaps initial_state", fn);
        if (overlap(final_state, st_bytes, o, o_bytes))
            return fail(KDA_ERR_INVALID_ARG, "%s: final_state overlaps o", fn);
    }
    if (ns == 0) return ok();
    return hip_status(kda::launch_chunk(plan, q, k, v, qkv_token_stride, g, beta, o,
                                        initial_state, final_state, cu_seqlens, ns, T, H, DK,
                                        DV, dtype, s),
                      fn);
}

int kda_chunk_prefill_mxfp8(const void* q, const void* q_scale, const void* k,
                            const void* k_scale, const void* v, const void* v_scale,
                            int64_t qkv_token_stride, const void* g, const void* g_scale,
                            const void* beta, void* o, const float* initial_state,
                            float* final_state, const int32_t* cu_seqlens, int32_t num_seqs,
                            int32_t B, int32_t T, int32_t H, int32_t DK, int32_t DV,
                            hipStream_t s) {
    const char* fn = "kda_chunk_prefill_mxfp8";
    if (H < 1) return fail(KDA_ERR_INVALID_ARG, "%s: H must be >= 1 (got %d)", fn, H);
    if (DK != 128 || DV != 128)
        return fail(KDA_ERR_UNSUPPORTED, "%s: DK and DV must be 128 (got %d, %d)", fn, DK, DV);
    if (q == nullptr || k == nullptr || v == nullptr || g == nullptr || q_scale == nullptr ||
        k_scale == nullptr || v_scale == nullptr || g_scale == nullptr || beta == nullptr ||
        o == nullptr)
        return fail(KDA_ERR_INVALID_ARG, "%s: codes, scales, beta and o must be non-null", fn);
    const int64_t row = (int64_t)H * 128;
    if (qkv_token_stride < row || qkv_token_stride % 16 != 0)
        return fail(KDA_ERR_INVALID_ARG,
                    "%s: qkv_token_stride must be >= H*128 and a multiple of 16 (got %lld)", fn,
                    (long long)qkv_token_stride);
    int ns;
    int64_t N;
    if (int rc = seq_layout(fn, cu_seqlens, num_seqs, B, T, &ns, &N)) return rc;
    if (int rc = check_cu(fn, cu_seqlens, ns, N, s)) return rc;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(o) || !aligned16(initial_state) || !aligned16(final_state))
        return fail(KDA_ERR_INVALID_ARG,
                    "%s: code, beta, o and state pointers must be 16-byte aligned", fn);
    if ((int64_t)ns * H * 2 > 0x7fffffffLL)
        return fail(KDA_ERR_INVALID_ARG, "%s: too many (sequence, head) pairs", fn);
    const int64_t qkv_bytes = N > 0 ? (N - 1) * qkv_token_stride + row : 0;
    const int64_t sc_bytes = N * H * 4;
    const int64_t o_bytes = N * H * 128 * 2;
    if (overlap(o, o_bytes, q, qkv_bytes) || overlap(o, o_bytes, k, qkv_bytes) ||
        overlap(o, o_bytes, v, qkv_bytes) || overlap(o, o_bytes, g, N * H * 128) ||
        overlap(o, o_bytes, q_scale, sc_bytes) || overlap(o, o_bytes, k_scale, sc_bytes) ||
        overlap(o, o_bytes, v_scale, sc_bytes) || overlap(o, o_bytes, g_scale, sc_bytes) ||
        overlap(o, o_bytes, beta, N * H * 2))
        return fail(KDA_ERR_INVALID_ARG, "%s: o must not overlap an input", fn);
    const int64_t st_bytes = (int64_t)ns * H * 128 * 128 * 4;
    if (final_state != nullptr) {
        if ((const void*)final_state != (const void*)initial_state &&
            overlap(final_state, st_bytes, initial_state, st_bytes))
            return fail(KDA_ERR_INVALID_ARG, "%s: final_state partially overlaps initial_state", fn);
        if (overlap(final_state, st_bytes, o, o_bytes))
            return fail(KDA_ERR_INVALID_ARG, "%s: final_state overlaps o", fn);
    }
    if (ns == 0) return ok();
    return hip_status(kda::launch_chunk_pipe_mxfp8(q, q_scale, k, k_scale, v, v_scale,
                                                   qkv_token_stride, g, g_scale, beta, o,
                                                   initial_state, final_state, cu_seqlens, ns, T,
                                                   H, s),
                      fn);
}

int kda_prefill_fused(const void* x, const float* conv_w, const void* g, const void* beta,
                      const void* gate, const float* norm_w, void* o, void* y,
                      const void* conv_state_in, void* conv_state_out,
                      const float* initial_state, float* final_state,
                      const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int32_t T,
                      int32_t H, int32_t D, int32_t dtype, float l2_eps, float rms_eps,
                      hipStream_t s) {
    const char* fn = "kda_prefill_fused";
    if (!valid_dtype(dtype)) return fail(KDA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (dtype != KDA_BF16)
        return fail(KDA_ERR_UNSUPPORTED, "%s: bf16 only (fp32 runs kda_conv, kda_chunk_prefill and "
                    "kda_gated_norm)", fn);
    if (H < 1) return fail(KDA_ERR_INVALID_ARG, "%s: H must be >= 1 (got %d)", fn, H);
    if (!valid_head(D)) return fail(KDA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, D);
    if (!(l2_eps > 0.f) || !(rms_eps > 0.f))
        return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps and rms_eps must be > 0", fn);
    if (x == nullptr || conv_w == nullptr || g == nullptr || beta == nullptr || gate == nullptr ||
        norm_w == nullptr || o == nullptr || y == nullptr)
        return fail(KDA_ERR_INVALID_ARG, "%s: x, conv_w, g, beta, gate, norm_w, o and y must be "
                    "non-null", fn);
    int ns;
    int64_t N;
    if (int rc = seq_layout(fn, cu_seqlens, num_seqs, B, T, &ns, &N)) return rc;
    if (int rc = check_cu(fn, cu_seqlens, ns, N, s)) return rc;
    if ((int64_t)ns * H * (D / 64) > 0x7fffffffLL)
        return fail(KDA_ERR_INVALID_ARG, "%s: too many (sequence, head) pairs", fn);
    if (!aligned16(x) || !aligned16(g) || !aligned16(beta) || !aligned16(gate) ||
        !aligned16(norm_w) || !aligned16(o) || !aligned16(y) || !aligned16(conv_state_in) ||
        !aligned16(conv_state_out) || !aligned16(initial_state) || !aligned16(final_state))
        return fail(KDA_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
    const int64_t P = 3LL * H * D;
    const int64_t x_b = N * P * 2, t_b = N * H * D * 2, b_b = N * H * 2;
    const int64_t cs_b = (int64_t)ns * P * 3 * 2, st_b = (int64_t)ns * H * D * D * 4;
    const void* ins[6] = {x, g, beta, gate, conv_state_in, initial_state};
    const int64_t in_b[6] = {x_b, t_b, b_b, t_b, cs_b, st_b};
    for (int i = 0; i < 6; ++i) {
        if (overlap(o, t_b, ins[i], in_b[i]))
            return fail(KDA_ERR_INVALID_ARG, "%s: o must not overlap an input", fn);
        if (overlap(y, t_b, ins[i], in_b[i]))
            return fail(KDA_ERR_INVALID_ARG, "%s: y must not overlap an input", fn);
    }
    if (y != o && overlap(y, t_b, o, t_b))
        return fail(KDA_ERR_INVALID_ARG, "%s: y partially overlaps o", fn);
    if (final_state != nullptr) {
        if ((const void*)final_state != (const void*)initial_state &&
            overlap(final_state, st_b, initial_state, st_b))
            return fail(KDA_ERR_INVALID_ARG, "%s: final_state partially overlaps initial_state", fn);
        for (int i = 0; i < 5; ++i)
            if (overlap(final_state, st_b, ins[i], in_b[i]) || overlap(final_state, st_b, o, t_b) ||
                overlap(final_state, st_b, y, t_b))
                return fail(KDA_ERR_INVALID_ARG, "%s: final_state overlaps another tensor", fn);
    }
    if (conv_state_out != nullptr) {
        if (conv_state_out != conv_state_in && overlap(conv_state_out, cs_b, conv_state_in, cs_b))
            return fail(KDA_ERR_INVALID_ARG, "%s: conv_state_out partially overlaps conv_state_in",
                        fn);
        for (int i = 0; i < 4; ++i)
            if (overlap(conv_state_out, cs_b, ins[i], in_b[i]) ||
                overlap(conv_state_out, cs_b, o, t_b) || overlap(conv_state_out, cs_b, y, t_b) ||
                overlap(conv_state_out, cs_b, initial_state, st_b) ||
                overlap(conv_state_out, cs_b, final_state, st_b))
                return fail(KDA_ERR_INVALID_ARG, "%s: conv_state_out overlaps another tensor", fn);
    }
    if (ns == 0) return ok();
    hipError_t e = kda::launch_chunk_pipe_conv(x, conv_w, conv_state_in, g, beta, o,
                                               initial_state, final_state, cu_seqlens, ns, T, H,
                                               D, l2_eps, s);
    if (e == hipSuccess)
        e = kda::launch_conv_state(x, conv_state_in, conv_state_out, cu_seqlens, ns, T, N, H, D,
                                   dtype, s);
    if (e == hipSuccess && N > 0)
        e = kda::launch_gated_norm(o, gate, norm_w, y, N * H, D, rms_eps, dtype, s);
    return hip_status(e, fn);
}

int kda_decode_step(const void* x, const float* w, void* conv_state, const void* g,
                    const void* beta, float* state, void* o, int32_t B, int32_t H, int32_t D,
                    int32_t dtype, float l2_eps, hipStream_t s) {
    const char* fn = "kda_decode_step";
    if (!valid_dtype(dtype)) return fail(KDA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (H < 1) return fail(KDA_ERR_INVALID_ARG, "%s: H must be >= 1 (got %d)", fn, H);
    if (B < 0) return fail(KDA_ERR_INVALID_ARG, "%s: B must be >= 0 (got %d)", fn, B);
    if (!valid_head(D)) return fail(KDA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, D);
    if (!(l2_eps > 0.f)) return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps must be > 0", fn);
    if (x == nullptr || w == nullptr || conv_state == nullptr || g == nullptr || beta == nullptr ||
        state == nullptr || o == nullptr)
        return fail(KDA_ERR_INVALID_ARG, "%s: every pointer must be non-null", fn);
    if (!aligned16(x) || !aligned16(conv_state) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(state) || !aligned16(o))
        return fail(KDA_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
    if ((int64_t)B * H > 0x7fffffffLL)
        return fail(KDA_ERR_INVALID_ARG, "%s: too many (sequence, head) pairs", fn);
    const int64_t es = esize(dtype);
    const int64_t P = 3LL * H * D;
    const int64_t o_bytes = (int64_t)B * H * D * es;
    if (overlap(o, o_bytes, x, B * P * es) || overlap(o, o_bytes, conv_state, B * P * 3 * es) ||
        overlap(o, o_bytes, g, (int64_t)B * H * D * es) || overlap(o, o_bytes, beta, (int64_t)B * H * es) ||
        overlap(o, o_bytes, state, (int64_t)B * H * D * D * 4))
        return fail(KDA_ERR_INVALID_ARG, "%s: o must not overlap an input", fn);
    if (overlap(state, (int64_t)B * H * D * D * 4, conv_state, B * P * 3 * es))
        return fail(KDA_ERR_INVALID_ARG, "%s: state overlaps conv_state", fn);
    if (B == 0) return ok();
    return hip_status(kda::launch_decode(x, w, conv_state, g, beta, state, o, B, H, D, dtype,
                                         l2_eps, s),
                      fn);
}

int kda_decode_multi(const void* x, const float* w, const void* conv_state_in,
                     void* conv_state_out, const void* g, const void* beta,
                     const float* state_in, float* state_out, void* o, const int32_t* n_tokens,
                     int32_t B, int32_t K, int32_t H, int32_t D, int32_t dtype, float l2_eps,
                     hipStream_t s) {
    const char* fn = "kda_decode_multi";
    if (!valid_dtype(dtype)) return fail(KDA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (H < 1) return fail(KDA_ERR_INVALID_ARG, "%s: H must be >= 1 (got %d)", fn, H);
    if (B < 0) return fail(KDA_ERR_INVALID_ARG, "%s: B must be >= 0 (got %d)", fn, B);
    if (K < 1) return fail(KDA_ERR_INVALID_ARG, "%s: K must be >= 1 (got %d)", fn, K);
    if (K > KDA_DECODE_MULTI_MAX_K)
        return fail(KDA_ERR_UNSUPPORTED, "%s: K must be <= %d (got %d)", fn, KDA_DECODE_MULTI_MAX_K, K);
    if (!valid_head(D)) return fail(KDA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, D);
    if (!(l2_eps > 0.f)) return fail(KDA_ERR_INVALID_ARG, "%s: l2_eps must be > 0", fn);
    if (x == nullptr || w == nullptr || conv_state_in == nullptr || g == nullptr ||
        beta == nullptr || state_in == nullptr)
        return fail(KDA_ERR_INVALID_ARG, "%s: x, w, conv_state_in, g, beta and state_in must be non-null", fn);
    if ((state_out == nullptr) != (conv_state_out == nullptr))
        return fail(KDA_ERR_INVALID_ARG, "%s: state_out and conv_state_out are given together or not at all", fn);
    if (o == nullptr && state_out == nullptr)
        return fail(KDA_ERR_INVALID_ARG, "%s: neither o nor the output states are given", fn);
    if (!aligned16(x) || !aligned16(conv_state_in) || !aligned16(g) || !aligned16(beta) ||
        !aligned16(state_in) || !aligned16(conv_state_out) || !aligned16(state_out) || !aligned16(o))
        return fail(KDA_ERR_INVALID_ARG, "%s: tensor pointers must be 16-byte aligned", fn);
    if ((reinterpret_cast<uintptr_t>(n_tokens) & 3u) != 0)
        return fail(KDA_ERR_INVALID_ARG, "%s: n_tokens must be 4-byte aligned", fn);
    if ((int64_t)B * H > 0x7fffffffLL)
        return fail(KDA_ERR_INVALID_ARG, "%s: too many (sequence, head) pairs", fn);
    const int64_t es = esize(dtype);
    const int64_t P = 3LL * H * D;
    const int64_t x_b = (int64_t)B * K * P * es, g_b = (int64_t)B * K * H * D * es;
    const int64_t beta_b = (int64_t)B * K * H * es, o_b = (int64_t)B * K * H * D * es;
    const int64_t st_b = (int64_t)B * H * D * D * 4, cs_b = (int64_t)B * P * 3 * es;
    const int64_t nt_b = (int64_t)B * 4;
    // o overlaps nothing; each output state is its input (in place) or apart
    // from every other tensor
    if (overlap(o, o_b, x, x_b) || overlap(o, o_b, conv_state_in, cs_b) || overlap(o, o_b, g, g_b) ||
        overlap(o, o_b, beta, beta_b) || overlap(o, o_b, state_in, st_b) ||
        overlap(o, o_b, state_out, st_b) || overlap(o, o_b, conv_state_out, cs_b) ||
        overlap(o, o_b, n_tokens, nt_b))
        return fail(KDA_ERR_INVALID_ARG, "%s: o must not overlap another tensor", fn);
    if (state_out != nullptr) {
        if (state_out != state_in && overlap(state_out, st_b, state_in, st_b))
            return fail(KDA_ERR_INVALID_ARG, "%s: state_out partly overlaps state_in", fn);
        if (conv_state_out != conv_state_in && overlap(conv_state_out, cs_b, conv_state_in, cs_b))
            return fail(KDA_ERR_INVALID_ARG, "%s: conv_state_out partly overlaps conv_state_in", fn);
        if (overlap(state_out, st_b, x, x_b) || overlap(state_out, st_b, g, g_b) ||
            overlap(state_out, st_b, beta, beta_b) || overlap(state_out, st_b, conv_state_in, cs_b) ||
            overlap(state_out, st_b, conv_state_out, cs_b) || overlap(state_out, st_b, n_tokens, nt_b))
            return fail(KDA_ERR_INVALID_ARG, "%s: state_out overlaps another tensor", fn);
        if (overlap(conv_state_out, cs_b, x, x_b) || overlap(conv_state_out, cs_b, g, g_b) ||
            overlap(conv_state_out, cs_b, beta, beta_b) || overlap(conv_state_out, cs_b, state_in, st_b) ||
            overlap(conv_state_out, cs_b, n_tokens, nt_b))
            return fail(KDA_ERR_INVALID_ARG, "%s: conv_state_out overlaps another tensor", fn);
    }
    if (B == 0) return ok();
    return hip_status(kda::launch_decode_multi(x, w, conv_state_in, conv_state_out, g, beta,
                                               state_in, state_out, o, n_tokens, B, K, H, D,
                                               dtype, l2_eps, s),
                      fn);
}

int kda_gated_norm(const void* o, const void* gate, const float* weight, void* y,
                   int64_t n_tokens, int32_t H, int32_t D, float eps, int32_t dtype,
                   hipStream_t s) {
    const char* fn = "kda_gated_norm";
    if (!valid_dtype(dtype)) return fail(KDA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
    if (H < 1) return fail(KDA_ERR_INVALID_ARG, "%s: H must be >= 1 (got %d)", fn, H);
    if (n_tokens < 0) return fail(KDA_ERR_INVALID_ARG, "%s: n_tokens must be >= 0", fn);
    if (!valid_head(D)) return fail(KDA_ERR_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", fn, D);
    if (!(eps > 0.f)) return fail(KDA_ERR_INVALID_ARG, "%s: eps must be > 0", fn);
    if (o == nullptr || gate == nullptr || weight == nullptr || y == nullptr)
        return fail(KDA_ERR_INVALID_ARG, "%s: o, gate, weight and y must be non-null", fn);
    if (!aligned16(o) || !aligned16(gate) || !aligned16(weight) || !aligned16(y))
        return fail(KDA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned", fn);
    const int64_t rows = n_tokens * H;
    const int64_t bytes = rows * D * esize(dtype);
    if (y != o && overlap(y, bytes, o, bytes))
        return fail(KDA_ERR_INVALID_ARG, "%s: y partially overlaps o", fn);
    if (overlap(y, bytes, gate, bytes))
        return fail(KDA_ERR_INVALID_ARG, "%s: y overlaps gate", fn);
    if (rows == 0) return ok();
    return hip_status(kda::launch_gated_norm(o, gate, weight, y, rows, D, eps, dtype, s), fn);
}

int64_t kda_mla_decode_workspace_bytes(int32_t B, int32_t H, int32_t L_max) {
    const char* fn = "kda_mla_decode_workspace_bytes";
    if (B < 0 || H < 1 || L_max < 1) {
        fail(KDA_ERR_INVALID_ARG, "%s: need B >= 0, H >= 1, L_max >= 1 (got %d, %d, %d)", fn, B, H,
             L_max);
        return -1;
    }
    return B == 0 ? 0 : kda::mla_workspace_bytes(B, H, L_max);
}

int kda_mla_decode(const void* q, const void* w_uk, const void* w_uv, const void* cache,
                   const int32_t* lengths, const void* gate, void* y, void* workspace,
                   int64_t workspace_bytes, int32_t B, int32_t H, int32_t L_max, int32_t R,
                   int32_t Dk, int32_t Dv, float scale, int32_t dtype, hipStream_t s) {
    const char* fn = "kda_mla_decode";
    if (int rc = mla_args(fn, q, w_uk, w_uv, cache, lengths, gate, y, B, H, L_max, R, Dk, Dv,
                          scale, dtype))
        return rc;
    if (B == 0) return ok();   // nothing to read or write
    if (workspace == nullptr) return fail(KDA_ERR_INVALID_ARG, "%s: workspace must be non-null", fn);
    const int64_t need = kda::mla_workspace_bytes(B, H, L_max);
    if (workspace_bytes < need)
        return fail(KDA_ERR_INVALID_ARG, "%s: workspace of %lld bytes, %lld needed", fn,
                    (long long)workspace_bytes, (long long)need);
    if (int rc = mla_apart(fn, q, w_uk, w_uv, cache, lengths, gate, y, workspace, need, B, H,
                           L_max, R, Dk, Dv))
        return rc;
    return hip_status(kda::launch_mla_decode(q, w_uk, w_uv, cache, lengths, gate, y, workspace, B,
                                             H, L_max, scale, s),
                      fn);
}

int kda_mla_decode_noalloc(const void* q, const void* w_uk, const void* w_uv, const void* cache,
                           const int32_t* lengths, const void* gate, void* y, int32_t B,
                           int32_t H, int32_t L_max, int32_t R, int32_t Dk, int32_t Dv,
                           float scale, int32_t dtype, hipStream_t s) {
    const char* fn = "kda_mla_decode_noalloc";
    if (int rc = mla_args(fn, q, w_uk, w_uv, cache, lengths, gate, y, B, H, L_max, R, Dk, Dv,
                          scale, dtype))
        return rc;
    if (B == 0) return ok();
    const int64_t need = kda::mla_workspace_bytes(B, H, L_max);
    if (need > KDA_MLA_NOALLOC_MAX_BYTES)
        return fail(KDA_ERR_INVALID_ARG,
                    "%s: B=%d, H=%d, L_max=%d need %lld bytes of scratch; the library's static "
                    "scratch holds %lld (use kda_mla_decode with a workspace)",
                    fn, B, H, L_max, (long long)need, (long long)KDA_MLA_NOALLOC_MAX_BYTES);
    // the tensors apart from each other first (no HIP call yet), then from
    // the scratch
    if (int rc = mla_apart(fn, q, w_uk, w_uv, cache, lengths, gate, y, nullptr, 0, B, H, L_max,
                           R, Dk, Dv))
        return rc;
    hipError_t e = hipSuccess;
    void* scratch = kda::mla_scratch(&e);
    if (scratch == nullptr)
        return fail(KDA_ERR_HIP, "%s: no device address for the static scratch: %s", fn,
                    hipGetErrorString(e));
    if (int rc = mla_apart(fn, q, w_uk, w_uv, cache, lengths, gate, y, scratch, need, B, H,
                           L_max, R, Dk, Dv))
        return rc;
    return hip_status(kda::launch_mla_decode(q, w_uk, w_uv, cache, lengths, gate, y, scratch, B,
                                             H, L_max, scale, s),
                      fn);
}

}  // extern "C"
