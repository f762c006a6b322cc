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
//   Kt = K e^G,  Qt = Q e^G,  Ki = K e^{-G}
//   A_kk = strict_lower(Kt Ki^T),  A_qk = lower(Qt Ki^T)
//   M' = (I + diag(beta) A_kk)^{-1} diag(beta)
//   U  = M' (V - Kt S)
//   O  = Qt S + A_qk U
//   S <- diag(e^{G_15}) (S + Ki^T U)
// A 16-token chunk spans at most e^{-80} of decay (g >= -5), so every factor
// above is a finite fp32 / bf16 number and no intra-chunk splitting is needed.
//
// Work split.  One workgroup per (sequence, head, slice of 64 value columns).
//  * Producer waves (8, two per SIMD) build everything that does not depend
//    on the state, one whole chunk per wave: per-channel decay products with
//    each lane holding all 16 tokens of its channels, the operand tiles -Kt,
//    Qt, Ki and the V slice in LDS, A_kk^T and A_qk^T on MFMA.  Each chunk's
//    16 x 16 unit triangular system is solved by its own producer, by
//    forward substitution in registers (a lane holds one row; the finished
//    row is broadcast within a 16-lane row by DPP), so a chunk never waits
//    for another producer.  Results go to a ring of LDS slots.
//  * Consumer waves (one per 16 value columns) hold their columns of the fp32
//    state in MFMA accumulators for the whole sequence; the state chain of a
//    chunk (V - Kt S, Qt S, M' R, A_qk U, Ki^T U, decay) is wave-local, so
//    consumers never wait on each other.  S feeds the next chunk's products as
//    an in-register bf16 B operand: the contraction index is permuted to the
//    accumulator's row order, and -Kt / Qt are stored in LDS in that order.
//    A consumer reads the next chunk's leading operands while it updates the
//    state, and issues no global loads (V comes through the slot).
//  * Output rows.  For one sequence of bf16 inputs the consumers write their
//    pieces of the chunk's output rows to an LDS staging area beside the
//    slot, and the producer that refills the slot stores each row whole
//    (128 bytes of one line); otherwise each consumer stores its 8-byte
//    pieces itself.
//  * Slots are handed over through LDS counters (producer: "chunk ready",
//    each consumer: "slot released"), so producers run ahead of the consumers
//    by up to the ring depth.  Every wait is bounded; a wait that runs out
//    stops the workgroup and its final state is written as NaN.
//
// MXFP8 inputs ("Inside Kimi K3", model at a glance: MXFP8 activations, read
// as OCP microscaling).  A second instantiation takes q, k, v and g as E4M3
// code bytes with one E8M0 scale byte per 32 channels.  Only the producers'
// loads and unpacking differ: a lane loads one 16-bit code word per token and
// tensor, and one scale byte per tensor and chunk (lane (block b, token t) of
// row b); token t's scale is broadcast across the row by DPP and is the scale
// operand of the scaled fp8 -> fp32 conversion, which yields the exact
// values; V codes are decoded the same way and stored to the slot as bf16
// (exact).  Everything after that is the bf16 kernel's code, so on the
// decoded values both give bitwise equal results.
//
// Conv inputs ("Inside Kimi K3", KDA short-convolution diagram and one-head
// diagram).  A third instantiation reads the projected inputs before the
// short convolution.  Each producer runs the 4-tap causal conv and SiLU on its
// lane's two channels of q and k over the chunk's 16 tokens (the 3 rows
// before the chunk come from the input, or on a sequence's first chunk from
// the incoming rolling state) and on a 2-column x 8-token patch of the
// workgroup's V slice.  The squares of a token's q (k) values are summed
// across the wave by a transposing butterfly that leaves lane l holding the
// sum of one (token, part) pair; its inverse square root is broadcast by
// readlane where q and k are scaled.  From the decay products on it is the
// bf16 kernel's code.
#include <type_traits>

#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16v4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __attribute__((address_space(3))) bf16v4* lds_bf16v4_ptr;

constexpr int kNP = 8;                 // producer waves (two per SIMD)
constexpr int kRing = 8;               // LDS slots
constexpr int kSpinLimit = 1 << 17;    // polls (about 128 cycles each) before giving up
constexpr int kOob = 0x40000000;       // a buffer offset past every range here (reads give 0)
constexpr int kSleep = 2;              // s_sleep argument between polls (64 cycles each)

template <int DK, int DVS>
struct PipeCfg {
    static constexpr int NC = DVS / 16;                 // consumer waves
    static constexpr int THREADS = 64 * (NC + kNP);
    static constexpr int CPT = DK / 16;                 // channels per producer lane (4 tokens each)
    static constexpr int NKS = DK / 32;                 // 16x16x32 steps over the key channels
    static constexpr int NKT = DK / 16;                 // 16-row key tiles of the state
    // Row pitches (bytes).  Tiles read 16 B per lane along a row get a 16 B
    // pad (row starts 4 banks apart); tiles read by the 4-row transposed 8 B
    // read get 32 B (8 banks apart).
    static constexpr int PK = DK * 2 + 16;
    static constexpr int PH = DK * 2 + 32;
    static constexpr int PV = DVS * 2 + 32;
    // one ring slot (a chunk handed to the consumers)
    static constexpr int O_KT = 0;                      // K e^G   (permuted channels)
    static constexpr int O_QT = O_KT + 16 * PK;         // Q e^G   (permuted channels)
    static constexpr int O_KI = O_QT + 16 * PK;         // K e^{-G} (natural order)
    static constexpr int O_V = O_KI + 16 * PH;          // V, this workgroup's columns
    static constexpr int O_MP = O_V + 16 * PV;          // M' as 16x16x16 A operands
    static constexpr int O_AQ = O_MP + 512;             // A_qk as 16x16x16 A operands
    static constexpr int O_GM = O_AQ + 512;             // e^{G15}, consumer lane order
    static constexpr int SLOT = O_GM + 512;
    static constexpr int RING = kRing * SLOT;
    // behind the ring, one of two per-slot areas:
    //  * the triangular solve's scratch: the 16 rows of -N in fp32, 80 bytes
    //    apart (a lane's 16-byte reads of rows 0..15 then use all 64 banks
    //    once);
    //  * (with output staging) the chunk's output rows, 16 tokens x this
    //    workgroup's value columns in bf16, gathered from the consumers and
    //    stored to memory whole.  It doubles as the solve's scratch: the
    //    slot's producer stores the previous rows before its solve, and the
    //    consumers write the next ones after its publication.
    static constexpr int PN = 80;
    static constexpr int O_NB = RING;
    static constexpr int SCRATCH = kRing * 16 * PN;
    static constexpr int PO = DVS * 2 + 16;             // output row pitch: rows 36 words apart
    static constexpr int O_OS = RING;
    static constexpr int STAGE = kRing * 16 * PO;
    static_assert(16 * PN <= 16 * PO, "solve scratch inside a slot's staging rows");
    static_assert(DK == 64 || DK == 128, "key width");
    static_assert(DVS == 64, "value slice");
    static_assert(SLOT % 16 == 0, "slot alignment");
    // the ring sizes that are built and tested: a divisor of the producer
    // count (output staging needs exactly one slot per producer, below)
    static_assert(kNP % kRing == 0, "ring size divides the producer count");
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
    // two paired conversions (one v_cvt_pk_bf16_f32 each)
    const bf16x2 lo = __builtin_convertvector(floatx2{a, b}, bf16x2);
    const bf16x2 hi = __builtin_convertvector(floatx2{c, d}, bf16x2);
    return __builtin_bit_cast(shortx4, u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)});
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
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                              0x150 + N, 0xF, 0xF, true));
}
// Forward substitution for X = (I + N)^{-1} diag(beta), N strictly lower
// triangular, one chunk per wave.  Lane (q, r) holds row r of -N in nn[] and
// X[r][4q .. 4q+3] in x[] (started at diag(beta)).  Row M of X is final once
// the steps before it are done; step M adds -N[r][M] X[M][.] to every row r,
// the finished row coming from lane M of the lane's own 16-lane row by a DPP
// broadcast folded into the multiply-add (rows r <= M add a masked zero).
// 60 multiply-adds, written as asm: the compiler does not fold a broadcast
// whose source is the accumulator itself (it adds a DPP move and a wait).
// The four of a step are independent and keep their order (volatile asm), so
// each broadcast read lies three instructions after the write of its
// operand; forward_rows puts the wait states ahead of the first step.  Step
// 15 would change no row and is left out.
template <int M>
__device__ __forceinline__ void forward_step(float (&x)[4], float n) {
    if constexpr (M < 15) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            asm volatile("v_fmac_f32_dpp %0, %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf"
                         : "+v"(x[k])
                         : "v"(n), "i"(M));
    }
}
// Steps 4J .. 4J+3 with entries 4J .. 4J+3 of the row of -N.
template <int J>
__device__ __forceinline__ void forward_group(float (&x)[4], floatx4 n) {
    forward_step<4 * J + 0>(x, n[0]);
    forward_step<4 * J + 1>(x, n[1]);
    forward_step<4 * J + 2>(x, n[2]);
    forward_step<4 * J + 3>(x, n[3]);
}
// The whole solve from the lane's row of -N in LDS (16 floats at row).
__device__ __forceinline__ void forward_rows(float (&x)[4], const char* row) {
    const floatx4* r = reinterpret_cast<const floatx4*>(row);
    const floatx4 a = r[0], b = r[1], c = r[2], d = r[3];
    // the wait states before the first broadcast read of x (its VALU writes
    // may be the instructions just before)
    asm volatile("s_nop 1" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
    forward_group<0>(x, a);
    forward_group<1>(x, b);
    forward_group<2>(x, c);
    forward_group<3>(x, d);
}

// Rows of the state tiles KT .. NKT-1 times their decay e^{G_15}: row i of
// tile KT is channel 16 KT + 4q + i; its decay sits in lane 2 KT + i/2 of the
// lane's own 16-lane row, component i % 2.
template <int KT, int NKT>
__device__ __forceinline__ void decay_rows(floatx4 (&S)[NKT], floatx2 gm) {
    if constexpr (KT < NKT) {
        S[KT][0] *= row_bcast<2 * KT>(gm[0]);
        S[KT][1] *= row_bcast<2 * KT>(gm[1]);
        S[KT][2] *= row_bcast<2 * KT + 1>(gm[0]);
        S[KT][3] *= row_bcast<2 * KT + 1>(gm[1]);
        decay_rows<KT + 1, NKT>(S, gm);
    }
}

// ---- slot hand-over ----------------------------------------------------------
// (every lane reads the same counter: the value is made wave-uniform, so the
// polling loops branch on scalars)
__device__ __forceinline__ int flag_load(int* f) {
    return __builtin_amdgcn_readfirstlane(
        __hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
}
// Counter updates are made by lane 0 only: an atomic executed by a whole
// wave acts once per active lane.
__device__ __forceinline__ void flag_store(int* f, int v, int lane) {
    if (lane == 0) __hip_atomic_store(f, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Wait until all N counters f[0..N-1] are >= target (N = 4).  Returns false
// (and raises the workgroup's stop flag) if the wait runs out, or if another
// wave has raised it.  The polls are relaxed (four loads in flight at once);
// the acquire fence after the poll that succeeds pairs with the consumers'
// releases, so the slot writes that follow stay behind it.
template <int N>
__device__ __forceinline__ bool wait_all_at_least(int* f, int target, int* stop) {
    static_assert(N == 4, "four consumer counters");
    int n = 0;
    for (;;) {
        // (LDS atomic loads: a volatile vector read through a generic pointer
        // becomes a flat load, which waits for every global load in flight)
        const int v0 = __hip_atomic_load(f + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int v1 = __hip_atomic_load(f + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int v2 = __hip_atomic_load(f + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int v3 = __hip_atomic_load(f + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const int m = __builtin_amdgcn_readfirstlane(min(min(v0, v1), min(v2, v3)));
        if (m >= target) break;
        if (__builtin_amdgcn_readfirstlane(
                __hip_atomic_load(stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != 0)
            return false;
        if (++n > kSpinLimit) {
            __hip_atomic_store(stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return false;
        }
        __builtin_amdgcn_s_sleep(kSleep);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    return true;
}

// Wait until *f >= target.  Returns false (and raises the workgroup's stop
// flag) if the wait runs out, or if another wave has raised it.
__device__ __forceinline__ bool wait_at_least(int* f, int target, int* stop) {
    int n = 0;
    while (flag_load(f) < target) {
        if (__builtin_amdgcn_readfirstlane(
                __hip_atomic_load(stop, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) != 0)
            return false;
        if (++n > kSpinLimit) {
            __hip_atomic_store(stop, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return false;
        }
        __builtin_amdgcn_s_sleep(kSleep);
    }
    return true;
}

// What the producers read for q, k and v:
//  kInBf16  q, k (L2-normalised) and v in bf16, e.g. kda_conv's output;
//  kInMx    the same as MXFP8 (E4M3 codes with one E8M0 scale byte per 32
//           consecutive channels in separate [tokens, H, D/32] tensors);
//  kInConv  the projected inputs before the short convolution: the producers
//           run the conv, SiLU and (for q, k) the L2 norm themselves.
// g is bf16 (kInBf16, kInConv) or MXFP8 (kInMx).
constexpr int kInBf16 = 0, kInMx = 1, kInConv = 2;
template <int IN> struct PipeIn { using type = __bf16; };
template <> struct PipeIn<kInMx> { using type = uint8_t; };

// lane n of the lane's 16-lane row, for a token index known after unrolling
__device__ __forceinline__ float row_bcast_t(float x, int t) {
    switch (t) {
        case 0: return row_bcast<0>(x);   case 1: return row_bcast<1>(x);
        case 2: return row_bcast<2>(x);   case 3: return row_bcast<3>(x);
        case 4: return row_bcast<4>(x);   case 5: return row_bcast<5>(x);
        case 6: return row_bcast<6>(x);   case 7: return row_bcast<7>(x);
        case 8: return row_bcast<8>(x);   case 9: return row_bcast<9>(x);
        case 10: return row_bcast<10>(x); case 11: return row_bcast<11>(x);
        case 12: return row_bcast<12>(x); case 13: return row_bcast<13>(x);
        case 14: return row_bcast<14>(x); default: return row_bcast<15>(x);
    }
}

// E8M0 scale byte to its value 2^(s - 127) (code 0: 2^-127, code 255: NaN)
__device__ __forceinline__ float e8m0_scale(uint32_t s) {
    const uint32_t bits = s == 0 ? 0x00400000u : (s == 255 ? 0x7FC00000u : s << 23);
    return __builtin_bit_cast(float, bits);
}

template <int DK, int DVS, int IN, bool SO, int THREADS = PipeCfg<DK, DVS>::THREADS>
__global__ void __launch_bounds__(THREADS)
chunk_pipe_kernel(const typename PipeIn<IN>::type* __restrict__ q,
                  const typename PipeIn<IN>::type* __restrict__ k,
                  const typename PipeIn<IN>::type* __restrict__ v, int64_t stride,
                  const typename PipeIn<IN>::type* __restrict__ g,
                  const __bf16* __restrict__ beta, __bf16* __restrict__ o, const float* s0,
                  float* sT, const int32_t* __restrict__ cu, int num_seqs, int T_len, int H,
                  int DV, int nsplit, const uint8_t* __restrict__ qsc,
                  const uint8_t* __restrict__ ksc, const uint8_t* __restrict__ vsc,
                  const uint8_t* __restrict__ gsc, const float* __restrict__ cw,
                  const __bf16* __restrict__ cs_in, float l2_eps, int blocked) {
    constexpr bool MX = IN == kInMx, CV = IN == kInConv;
    static_assert(!MX || DK == 128, "MXFP8 inputs: two channels per producer lane");
    static_assert(!CV || DVS == 64, "conv inputs: a value slice of 64 columns");
    constexpr int ES = MX ? 1 : 2;   // bytes per q, k, v, g element
    using Cfg = PipeCfg<DK, DVS>;
    constexpr int NC = Cfg::NC, NKS = Cfg::NKS, NKT = Cfg::NKT;
    constexpr int PK = Cfg::PK, PH = Cfg::PH, SLOT = Cfg::SLOT;
    // conv inputs: the workgroup's conv taps (q and k channels of the head,
    // then its value columns), 4 floats each, behind the ring
    // Output rows staged in LDS and stored whole by the producers (SO), or
    // stored by the consumers in 32-byte pieces.  Staged for one sequence of
    // bf16 inputs, where four consumers writing 32-byte pieces of one 128-byte
    // line made the workgroups of some heads 7 % slower (per-workgroup
    // timing; the same rows written whole removed it); direct for packed
    // batches and MXFP8 inputs (measured faster there) and for conv inputs
    // (no room for the staging area beside the scratch and the taps)
    constexpr bool kStageO = SO;
    static_assert(!SO || !CV, "no output staging with conv inputs");
    // A slot's staged rows are stored by the producer that refills it, and
    // the last rows of every slot by the producer of that slot's last chunk
    // (at its end): right only with one slot per producer, so that the last
    // kNP chunks are the producers' last chunks and sit in distinct slots.
    static_assert(!SO || kRing == kNP, "output staging needs one slot per producer");
    constexpr int O_W = Cfg::RING + (kStageO ? Cfg::STAGE : Cfg::SCRATCH);
    constexpr int WBYTES = CV ? (2 * DK + DVS) * 16 : 0;
    static_assert(O_W + WBYTES <= 160 * 1024 - 256, "LDS budget");

    __shared__ __attribute__((aligned(16))) char smem[O_W + WBYTES];
    // ready[kRing], released[kRing][NC] (one counter per consumer), stop
    constexpr int NFLAGS = kRing + kRing * NC + 1;
    __shared__ __attribute__((aligned(16))) int flags[NFLAGS];
    int* ready = flags;
    int* released = flags + kRing;
    int* stop = flags + kRing + kRing * NC;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int lr = lane & 15;
    const int lq = lane >> 4;

    // ---- workgroup -> (sequence, head, value slice).  Workgroups are dealt to
    // the 8 XCDs in turn (ids x, x+8, ... run on XCD x), and the value slices
    // of a chain sit 8 ids apart, on one XCD.  With blocked heads (and heads
    // that split evenly) XCD x takes heads [x H/8, (x+1) H/8) of every
    // sequence, the sequences in order, so a token's block-scale and beta
    // bytes for an XCD's heads are one short run of its row, fetched into that
    // XCD's L2 alone (chosen for MXFP8 inputs and for several sequences, where
    // it measured faster); otherwise consecutive chains go to consecutive
    // XCDs (faster for one sequence of bf16 inputs) -------------------------
    const int nchain = num_seqs * H;
    const int total = nchain * nsplit;
    const int bid = blockIdx.x;
    int seq, head, split;
    if (blocked && H % 8 == 0) {
        const int hpx = H / 8, j = bid >> 3, idx = j / nsplit;
        split = j % nsplit;
        seq = idx / hpx;
        head = (bid & 7) * hpx + idx % hpx;
    } else {
        const int span = 8 * nsplit;
        const int full = (total / span) * span;
        int chain;
        if (bid < full) {
            const int gi = bid >> 3;
            chain = (gi / nsplit) * 8 + (bid & 7);
            split = gi % nsplit;
        } else {
            const int r = bid - full;
            chain = full / nsplit + r / nsplit;
            split = r % nsplit;
        }
        seq = chain / H;
        head = chain % H;
    }
    const int n0 = split * DVS;
    // packed offsets are clamped to the T_len tokens of the batch, so offsets
    // that are not monotone or exceed it never move an access out of bounds
    int64_t t_begin = (int64_t)seq * T_len, t_end = t_begin + T_len;
    if (cu) {
        const int64_t a = cu[seq], b = cu[seq + 1];
        t_begin = a < 0 ? 0 : (a > T_len ? T_len : a);
        t_end = b < t_begin ? t_begin : (b > T_len ? T_len : b);
    }
    const int64_t n_chunks = (t_end - t_begin + 15) / 16;
    const int nch = (int)n_chunks;

    if (tid < NFLAGS) flags[tid] = 0;
    if constexpr (CV) {
        // conv taps of this workgroup: the head's DK q channels, its DK k
        // channels, then its DVS value columns (the k and v parts of the
        // filter banks start H*DK and 2*H*DK channels in)
        float* wl = reinterpret_cast<float*>(smem + O_W);
        for (int i = tid; i < (2 * DK + DVS) * 4; i += THREADS) {
            const int r = i >> 2;
            const int64_t ch = r < DK ? (int64_t)head * DK + r
                                      : (r < 2 * DK ? (int64_t)H * DK + head * DK + (r - DK)
                                                    : 2LL * H * DK + (int64_t)head * DV + n0 +
                                                          (r - 2 * DK));
            wl[i] = cw[ch * 4 + (i & 3)];
        }
    }
    __syncthreads();

    if (wave >= NC) {
        // ===================== producer wave =================================
        // Stage-1 lane layout: lane l holds channels CPL*l .. CPL*l+CPL-1 of
        // all 16 tokens (one 4- or 2-byte load per token and tensor), so the
        // decay products over the chunk run serially inside the lane.
        const int pw = wave - NC;
        constexpr int CPL = DK / 64;
        const int c0 = CPL * lane;
        uint32_t rg[16], rk[16], rq[16];   // CPL bf16 channels per word
        // V slice of the chunk: lane holds token lane/4, columns 16 (lane%4) .. +15
        bf16x8 rv[2];
        // MXFP8: the V codes (16 per lane) and their scale byte; the scale
        // bytes of g, k, q for the chunk's 16 tokens x 4 channel blocks, lane
        // (block b, token t) holding (t, b) -- row b of lanes serves block b
        u32x4 rvm;
        uint32_t rvs, rsg, rsk, rsq;
        // conv inputs: the raw x words of the lane's q and k channels for the
        // chunk's tokens t0-3 .. t0+15 (row j = token t0-3+j), the conv state
        // words of those channels (first chunk of a sequence only), and for V
        // the raw x words of columns n0+2cp, +1 (cp = lane % 32) for the tokens
        // t0+8h-3 .. t0+8h+7 (h = lane / 32) with their state words
        uint32_t rxq[CV ? 19 : 1], rxk[CV ? 19 : 1], rcq[3], rck[3];
        uint32_t rxv[CV ? 11 : 1], rsv[3];
        const int cp = lane & 31, hv = lane >> 5;
        // beta of token lr as a zero-extended 32-bit word (16-bit values would
        // be packed in pairs right after the loads, which makes the wave wait)
        uint32_t rbl;
        const int g_row = H * DK * ES, kv_row = (int)(stride * ES), b_row = H * 2;
        const int sc_row = H * (DK / 32);   // scale bytes per token
        const int vt = lane >> 2, vc = 16 * (lane & 3);
        auto load_word = [](rsrc_t r, int off) -> uint32_t {
            if constexpr (MX) return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
            else if constexpr (CPL == 2) return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
            else return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
        };
        // Loads of chunk ci (g, k, q, beta; V separately).  Past the last chunk
        // the resources cover no bytes and the loads return zeros; they are
        // issued anyway, so that every iteration issues the same memory
        // operations and no register copy has to wait for loads in flight.
        auto chunk_rows = [&](int64_t ci, int64_t& t0) -> int {
            t0 = t_begin + ci * 16;
            const int64_t rem = t_end - t0;
            return (int)(rem < 16 ? (rem > 0 ? rem : 0) : 16);
        };
        // conv inputs: the chunk's rows come through one resource, the 3 rows
        // before it through another, which is empty on a sequence's first
        // chunk (whose halo is the conv state, through a resource that is
        // empty on every other chunk); the per-lane offsets do not depend on
        // the chunk
        auto halo_rsrc = [&](const __bf16* base, int64_t ci, int64_t t0, int valid) -> rsrc_t {
            const bool on = ci > 0 && valid > 0;
            return make_rsrc(base + (on ? t0 - 3 : t0) * stride, on ? (uint32_t)(3 * kv_row) : 0u);
        };
        auto issue_gkq = [&](int64_t ci) {
            int64_t t0;
            const int valid = chunk_rows(ci, t0);
            const rsrc_t r_g = make_rsrc(g + (t0 * H + head) * DK, (uint32_t)(valid * g_row));
            if constexpr (CV) {
                const __bf16* bq = q + (int64_t)head * DK;
                const __bf16* bk = k + (int64_t)head * DK;
                const rsrc_t r_q = make_rsrc(bq + t0 * stride, (uint32_t)(valid * kv_row));
                const rsrc_t r_k = make_rsrc(bk + t0 * stride, (uint32_t)(valid * kv_row));
                const rsrc_t h_q = halo_rsrc(bq, ci, t0, valid);
                const rsrc_t h_k = halo_rsrc(bk, ci, t0, valid);
#pragma unroll
                for (int j = 0; j < 19; ++j) {
                    rxq[j] = load_word(j < 3 ? h_q : r_q, (j < 3 ? j : j - 3) * kv_row + c0 * 2);
                    rxk[j] = load_word(j < 3 ? h_k : r_k, (j < 3 ? j : j - 3) * kv_row + c0 * 2);
                }
                const bool st = ci == 0 && cs_in != nullptr;
                const int64_t sb = ((int64_t)seq * stride + (int64_t)head * DK) * 3;
                const uint32_t sbytes = st ? (uint32_t)(DK * 3 * 2) : 0u;
                const rsrc_t s_q = make_rsrc(st ? cs_in + sb : q, sbytes);
                const rsrc_t s_k = make_rsrc(st ? cs_in + sb + (int64_t)H * DK * 3 : q, sbytes);
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    rcq[j] = load_word(s_q, c0 * 6 + j * 2 * CPL);
                    rck[j] = load_word(s_k, c0 * 6 + j * 2 * CPL);
                }
            }
            if constexpr (CV) {
#pragma unroll
                for (int t = 0; t < 16; ++t) rg[t] = load_word(r_g, t * g_row + c0 * ES);
            } else {
                const rsrc_t r_k = make_rsrc(k + t0 * stride + (int64_t)head * DK, (uint32_t)(valid * kv_row));
                const rsrc_t r_q = make_rsrc(q + t0 * stride + (int64_t)head * DK, (uint32_t)(valid * kv_row));
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    rg[t] = load_word(r_g, t * g_row + c0 * ES);
                    rk[t] = load_word(r_k, t * kv_row + c0 * ES);
                    rq[t] = load_word(r_q, t * kv_row + c0 * ES);
                }
            }
            if constexpr (MX) {
                const int64_t sb = (t0 * H + head) * (DK / 32);
                const uint32_t sbytes = (uint32_t)(valid * sc_row);
                const int soff = lr * sc_row + lq;
                rsg = (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(make_rsrc(gsc + sb, sbytes), soff, 0, 0);
                rsk = (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(make_rsrc(ksc + sb, sbytes), soff, 0, 0);
                rsq = (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(make_rsrc(qsc + sb, sbytes), soff, 0, 0);
            }
            const rsrc_t r_b = make_rsrc(beta + t0 * H + head, (uint32_t)(valid * b_row));
            rbl = (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(r_b, lr * b_row, 0, 0);
        };
        auto issue_v = [&](int64_t ci) {
            int64_t t0;
            const int valid = chunk_rows(ci, t0);
            if constexpr (CV) {
                // row r of this lane is token t0 + 8 hv - 3 + r: rows before t0
                // (first half, r < 3) come from the halo resource and get an
                // out-of-range offset (kOob, past any range) in the main one,
                // and the other way round
                const __bf16* bv = v + (int64_t)head * DV + n0;
                const rsrc_t r_v = make_rsrc(bv + t0 * stride, (uint32_t)(valid * kv_row));
                const rsrc_t h_v = halo_rsrc(bv, ci, t0, valid);
#pragma unroll
                for (int r = 0; r < 11; ++r) {
                    const int off = r < 3 && hv == 0 ? kOob : (8 * hv - 3 + r) * kv_row + cp * 4;
                    rxv[r] = __builtin_amdgcn_raw_buffer_load_b32(r_v, off, 0, 0);
                    if (r < 3)
                        rxv[r] |= __builtin_amdgcn_raw_buffer_load_b32(h_v, hv ? kOob : r * kv_row + cp * 4, 0, 0);
                }
                // the state of columns n0+2cp, +1 (lanes of the first half only)
                const bool st = ci == 0 && cs_in != nullptr;
                const int64_t sb = ((int64_t)seq * stride + 2LL * H * DK + (int64_t)head * DV + n0) * 3;
                const rsrc_t s_v = make_rsrc(st ? cs_in + sb : v, st ? (uint32_t)(DVS * 3 * 2) : 0u);
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    rsv[j] = __builtin_amdgcn_raw_buffer_load_b32(s_v, hv ? kOob : cp * 12 + 4 * j, 0, 0);
                return;
            }
            const rsrc_t r_v = make_rsrc(v + t0 * stride + (int64_t)head * DV + n0, (uint32_t)(valid * kv_row));
            if constexpr (MX) {
                rvm = __builtin_amdgcn_raw_buffer_load_b128(r_v, vt * kv_row + vc, 0, 0);
                const int vrow = H * (DV / 32);
                rvs = (uint32_t)(uint8_t)__builtin_amdgcn_raw_buffer_load_b8(
                    make_rsrc(vsc + (t0 * H + head) * (DV / 32), (uint32_t)(valid * vrow)),
                    vt * vrow + (n0 + vc) / 32, 0, 0);
            } else {
                rv[0] = BufLoad<__bf16, 8>::load(r_v, vt * kv_row + vc * 2);
                rv[1] = BufLoad<__bf16, 8>::load(r_v, vt * kv_row + vc * 2 + 16);
            }
        };
        // channel j of a word as fp32 (bf16 is the top half of an fp32)
        auto chan = [](uint32_t w, int j) -> float {
            return __builtin_bit_cast(float, j == 0 ? w << 16 : w & 0xffff0000u);
        };
        // CPL fp32 values as CPL packed bf16 (the low half first), and their
        // one-word / half-word LDS store
        auto pack = [](const float (&x)[CPL]) -> uint32_t {
            if constexpr (CPL == 2)
                return __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{x[0], x[1]}, bf16x2));
            else
                return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x[0]);
        };
        auto put = [](char* p, uint32_t w) {
            if constexpr (CPL == 2) *reinterpret_cast<uint32_t*>(p) = w;
            else *reinterpret_cast<uint16_t*>(p) = (uint16_t)w;
        };
        // Where a chunk's loads are issued: bf16 and conv inputs one chunk
        // ahead (bf16 as soon as this chunk's words are consumed, conv inputs
        // after the publication), MXFP8 at the top of the chunk's own
        // iteration.  The MXFP8 loads stall the top of the iteration either
        // way (they follow the publication), and carried across the loop's
        // latch their 48 code words were copied between registers every
        // iteration (measured 5 % faster without the copies; conv inputs
        // measured no better).
        constexpr bool kTopLoad = MX;
        if constexpr (!kTopLoad) {
            issue_gkq(pw);
            issue_v(pw);
        }

        // The loop has no early exit: an exit path would merge with the
        // prefetch registers at the loop's latch and make every iteration wait
        // for its loads.  A wait that runs out (the stop flag is then raised)
        // lets the body run once more on whatever the slot holds, publishes
        // nothing, and ends the loop.
        const int pos = perm_pos(c0);   // this lane's channels in the permuted tiles
        // The output rows of chunk c, gathered in the slot's staging area by
        // the four consumers before they released the slot: lane l stores 32
        // bytes of row l / 4, so each row of the workgroup's value columns is
        // written whole; rows past the sequence end fall outside the resource.
        auto store_o = [&](int64_t c, int s_c) {
            int64_t t0;
            const int valid = chunk_rows(c, t0);
            const int o_row = H * DV * 2;
            const char* st = smem + Cfg::O_OS + s_c * 16 * Cfg::PO + (lane >> 2) * Cfg::PO + (lane & 3) * 32;
            const u32x4 a = *reinterpret_cast<const u32x4*>(st);
            const u32x4 b = *reinterpret_cast<const u32x4*>(st + 16);
            const rsrc_t r_o = make_rsrc(o + (t0 * H + head) * DV + n0, (uint32_t)(valid * o_row));
            const int off = (lane >> 2) * o_row + (lane & 3) * 32;
            __builtin_amdgcn_raw_buffer_store_b128(a, r_o, off, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b128(b, r_o, off + 16, 0, 0);
        };
        int64_t last = -1;               // the last chunk this wave published
        for (int64_t ci = pw; ci < n_chunks;) {
            const int s = (int)(ci % kRing);
            const int round = (int)(ci / kRing);
            // The slot is waited for before the chunk's work, except with MXFP8
            // or conv inputs: there the decoding (or the convolution) and the
            // decay products are worked up in registers first and only the
            // slot writes wait, which takes that work off the hand-over's
            // critical path (measured faster for both; the bf16 instantiation
            // measured no faster with the wait last)
            constexpr bool kLateWait = MX || CV;
            if constexpr (kTopLoad) {
                issue_gkq(ci);
                issue_v(ci);
            }
            bool go = kLateWait ? true : wait_all_at_least<NC>(&released[s * NC], round, stop);
            char* slot = smem + s * SLOT;
            // every consumer has released the slot's previous chunk, so its
            // output rows are complete in the staging area
            if constexpr (kStageO && !kLateWait) {
                if (go && ci >= kRing) store_o(ci - kRing, s);
            }

            // ---- conv inputs: short conv, SiLU, L2 of q and k ------------------
            // ("Inside Kimi K3", KDA short-convolution diagram: 4 taps per
            // channel over x_{t-3} .. x_t, then SiLU; KDA one-head diagram: L2
            // norm of q and k.)  V stays in vw as bf16 words until the slot is
            // free; q and k stay in rq / rk as bf16 words before the norm, and
            // inv_l holds the inverse norm of (token, part) = (l/2 % 16, l/32)
            // for lane l
            float inv_l = 1.f;
            uint32_t vw[CV ? 8 : 1];
            if constexpr (CV) {
                const float* wl = reinterpret_cast<const float*>(smem + O_W);
                // on the first chunk the 3 rows before it come from the state
                // words: per channel pair the three words hold
                // [s0 c | s1 c], [s2 c | s0 c'], [s1 c' | s2 c'] (CPL = 2)
                auto halo = [](uint32_t (&x)[3], const uint32_t (&st)[3]) {
                    if constexpr (CPL == 2) {
                        x[0] |= __builtin_amdgcn_perm(st[1], st[0], 0x07060100u);
                        x[1] |= __builtin_amdgcn_perm(st[2], st[0], 0x05040302u);
                        x[2] |= __builtin_amdgcn_perm(st[2], st[1], 0x07060100u);
                    } else {
                        x[0] |= st[0];
                        x[1] |= st[1];
                        x[2] |= st[2];
                    }
                };
                // V: columns n0 + 2cp, +1 of tokens 8hv .. 8hv + 7
                {
                    uint32_t hx[3] = {rxv[0], rxv[1], rxv[2]};
                    uint32_t hs[3] = {rsv[0], rsv[1], rsv[2]};
                    // (a column pair's state: [s0 c | s1 c], [s2 c | s0 c'], [s1 c' | s2 c'])
                    hx[0] |= __builtin_amdgcn_perm(hs[1], hs[0], 0x07060100u);
                    hx[1] |= __builtin_amdgcn_perm(hs[2], hs[0], 0x05040302u);
                    hx[2] |= __builtin_amdgcn_perm(hs[2], hs[1], 0x07060100u);
                    const floatx4 w[2] = {*reinterpret_cast<const floatx4*>(wl + (2 * DK + 2 * cp) * 4),
                                          *reinterpret_cast<const floatx4*>(wl + (2 * DK + 2 * cp + 1) * 4)};
                    auto xv = [&](int r, int j) { return chan(r < 3 ? hx[r] : rxv[r], j); };
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        float y[2];
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            y[j] = siluf_(w[j][0] * xv(t, j) + w[j][1] * xv(t + 1, j) +
                                          w[j][2] * xv(t + 2, j) + w[j][3] * xv(t + 3, j));
                        vw[t] = __builtin_bit_cast(uint32_t, __builtin_convertvector(floatx2{y[0], y[1]}, bf16x2));
                    }
                }
                // q and k: conv + SiLU per channel, squares summed per token
                float ss[32];   // [part][token]
                auto conv_part = [&](const uint32_t (&rx)[19], const uint32_t (&rs)[3], int part,
                                     uint32_t (&out)[16]) {
                    uint32_t hx[3] = {rx[0], rx[1], rx[2]};
                    halo(hx, rs);
                    floatx4 w[CPL];
#pragma unroll
                    for (int j = 0; j < CPL; ++j) w[j] = *reinterpret_cast<const floatx4*>(wl + (part * DK + c0 + j) * 4);
                    auto xv = [&](int r, int j) { return chan(r < 3 ? hx[r] : rx[r], j); };
#pragma unroll
                    for (int t = 0; t < 16; ++t) {
                        float sq = 0.f, y[CPL];
#pragma unroll
                        for (int j = 0; j < CPL; ++j) {
                            y[j] = siluf_(w[j][0] * xv(t, j) + w[j][1] * xv(t + 1, j) +
                                          w[j][2] * xv(t + 2, j) + w[j][3] * xv(t + 3, j));
                            sq += y[j] * y[j];
                        }
                        ss[16 * part + t] = sq;
                        out[t] = pack(y);
                    }
                };
                conv_part(rxq, rcq, 0, rq);
                conv_part(rxk, rck, 1, rk);
                // sums over the 64 lanes: at each step a lane keeps half of
                // its values (the upper half when its lane bit is set) and adds
                // the partner's copy of them; lane l ends with value l/2
                auto step = [&](auto n_c, int m, auto xchg) {
                    constexpr int n = decltype(n_c)::value;
                    const bool up = (lane & m) != 0;
#pragma unroll
                    for (int i = 0; i < n / 2; ++i) {
                        const float send = up ? ss[i] : ss[i + n / 2];
                        const float keep = up ? ss[i + n / 2] : ss[i];
                        ss[i] = keep + xchg(send);
                    }
                };
                auto dpp = [](float x, auto ctrl_c) {
                    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                                              decltype(ctrl_c)::value, 0xF, 0xF, true));
                };
                using I8 = std::integral_constant<int, 8>;
                using I4 = std::integral_constant<int, 4>;
                using I2 = std::integral_constant<int, 2>;
                // the 32- and 16-lane steps are one permlane swap per pair: after
                // swapping, each lane holds its own kept value and the partner's
                // copy of it
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    rows_swap32(ss[i], ss[i + 16]);
                    ss[i] += ss[i + 16];
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    rows_swap16(ss[i], ss[i + 8]);
                    ss[i] += ss[i + 8];
                }
                step(I8{}, 8, [&](float x) { return dpp(x, std::integral_constant<int, 0x128>{}); });   // row_ror:8
                step(I4{}, 4, [&](float x) { return dpp(x, std::integral_constant<int, 0x141>{}); });   // row_half_mirror
                step(I2{}, 2, [&](float x) { return dpp(x, std::integral_constant<int, 0x4E>{}); });    // quad_perm 2,3,0,1
                const float tot = ss[0] + dpp(ss[0], std::integral_constant<int, 0xB1>{});            // quad_perm 1,0,3,2
                inv_l = rsqrt_nr(tot + l2_eps);
            }

            // ---- decay products, in registers -------------------------------
            // a_t = e^{g_t}; F_t = e^{G_t} = a_0 .. a_t (forward), then
            // E_t = e^{-G_t} = e^{-G_15} a_{t+1} .. a_15 (backward)
            float a[CPL][16], F[CPL];
            uint32_t wkt[16], wqt[16], wki[16];   // packed bf16 tile words per token
            // MXFP8: the block scales of g, k, q (one per lane: token lr of
            // block lq); value j of token t is then one scaled conversion of
            // the two codes with the scale broadcast from lane t of the row
            float fsg = 0.f, fsk = 0.f, fsq = 0.f;
            if constexpr (MX) {
                fsg = e8m0_scale(rsg);
                fsk = e8m0_scale(rsk);
                fsq = e8m0_scale(rsq);
            }
            auto val = [&](uint32_t w, float fs, int t, int j) -> float {
                if constexpr (MX) return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, row_bcast_t(fs, t), false)[j];
                else return chan(w, j);
            };
            // conv inputs: q and k of token t times their inverse norms
            auto inv_q = [&](int t) -> float {
                if constexpr (CV) return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv_l), 2 * t));
                else return 1.f;
            };
            auto inv_k = [&](int t) -> float {
                if constexpr (CV) return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, inv_l), 32 + 2 * t));
                else return 1.f;
            };
            float kv[CPL][16];   // k (normalised) in fp32, for both passes
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                float kt[CPL], qt[CPL];
                const float iq = inv_q(t), ik = inv_k(t);
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    a[j][t] = fast_exp2(clamp_log_decay(val(rg[t], fsg, t, j)) * kLog2e);
                    F[j] = t == 0 ? a[j][0] : F[j] * a[j][t];
                    kv[j][t] = CV ? val(rk[t], fsk, t, j) * ik : val(rk[t], fsk, t, j);
                    kt[j] = -(kv[j][t] * F[j]);   // stored negated: -K e^G
                    qt[j] = (CV ? val(rq[t], fsq, t, j) * iq : val(rq[t], fsq, t, j)) * F[j];
                }
                wkt[t] = pack(kt);
                wqt[t] = pack(qt);
            }
            float E[CPL];
#pragma unroll
            for (int j = 0; j < CPL; ++j) E[j] = fast_rcp(F[j]);   // e^{-G_15} <= e^80
#pragma unroll
            for (int t = 15; t >= 0; --t) {
                float ki[CPL];
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    if (t < 15) E[j] *= a[j][t + 1];
                    ki[j] = kv[j][t] * E[j];
                }
                wki[t] = pack(ki);
            }
            // beta to fp32 before the next chunk's loads reuse its registers
            // (a conversion sunk below them would keep both copies live and
            // add a register move that waits for the loads)
            float bl = __builtin_bit_cast(float, rbl << 16);   // bf16 -> fp32
            asm volatile("" : "+v"(bl));
            if constexpr (kLateWait) {
                // (the empty asm keeps the work above on this side of the
                // wait: the compiler would otherwise sink it to its uses)
#pragma unroll
                for (int t = 0; t < 16; ++t) asm volatile("" : "+v"(wkt[t]), "+v"(wqt[t]), "+v"(wki[t]));
#pragma unroll
                for (int j = 0; j < CPL; ++j) asm volatile("" : "+v"(F[j]));
                if constexpr (CV) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) asm volatile("" : "+v"(vw[t]));
                }
                go = wait_all_at_least<NC>(&released[s * NC], round, stop);
                if constexpr (kStageO) {
                    if (go && ci >= kRing) store_o(ci - kRing, s);
                }
            }
            // ---- into the slot -----------------------------------------------
            {
#pragma unroll
                for (int t = 0; t < 16; ++t) {
                    put(slot + Cfg::O_KT + t * PK + pos * 2, wkt[t]);
                    put(slot + Cfg::O_QT + t * PK + pos * 2, wqt[t]);
                    put(slot + Cfg::O_KI + t * PH + c0 * 2, wki[t]);
                }
            }
            // e^{G_15} per channel, laid out for the consumers' row
            // broadcasts: channel 16*kt + 4*q + i -> entry [q][2*kt + i/2][i%2]
            {
                const int kt = c0 >> 4, qq = (c0 >> 2) & 3, i = c0 & 3;
                float* gp = reinterpret_cast<float*>(slot + Cfg::O_GM) + ((qq * 16 + 2 * kt + (i >> 1)) * 2 + (i & 1));
                if constexpr (CPL == 2) *reinterpret_cast<floatx2*>(gp) = floatx2{F[0], F[1]};
                else *gp = F[0];
            }
            if constexpr (MX) {
                // the 16 V codes of this lane to bf16 (exact: E4M3 times a
                // power of two fits bf16)
                const float fv = e8m0_scale(rvs);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const floatx2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(rvm[2 * h], fv, false);
                    const floatx2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(rvm[2 * h], fv, true);
                    const floatx2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(rvm[2 * h + 1], fv, false);
                    const floatx2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(rvm[2 * h + 1], fv, true);
                    const bf16x2 b0 = __builtin_convertvector(p0, bf16x2), b1 = __builtin_convertvector(p1, bf16x2);
                    const bf16x2 b2 = __builtin_convertvector(p2, bf16x2), b3 = __builtin_convertvector(p3, bf16x2);
                    rv[h] = bf16x8{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
                }
            }
            if constexpr (!CV) {
                *reinterpret_cast<bf16x8*>(slot + Cfg::O_V + vt * Cfg::PV + vc * 2) = rv[0];
                *reinterpret_cast<bf16x8*>(slot + Cfg::O_V + vt * Cfg::PV + vc * 2 + 16) = rv[1];
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    *reinterpret_cast<uint32_t*>(slot + Cfg::O_V + (8 * hv + t) * Cfg::PV + cp * 4) = vw[t];
            }
            // the next chunk of this wave streams in from here on (with the
            // slot wait last: conv inputs from the end of this chunk, MXFP8 at
            // the top of its own iteration; the loads then stay off the path
            // from the slot's release to its publication)
            if constexpr (!kLateWait) {
                issue_gkq(ci + kNP);
                issue_v(ci + kNP);
            }

            // ---- A_kk^T, A_qk^T (16x16x32 MFMA over the key channels) -------
            floatx4 akk = zero4(), aqk = zero4();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int off = lr * PK + (32 * ks + 8 * lq) * 2;
                // Ki is in natural channel order: the channels of permuted
                // positions 8q .. 8q+7 are 4q .. 4q+3 and 16+4q .. 16+4q+3
                const char* kir = slot + Cfg::O_KI + lr * PH + (32 * ks + 4 * lq) * 2;
                const bf16x4 i0 = *reinterpret_cast<const bf16x4*>(kir);
                const bf16x4 i1 = *reinterpret_cast<const bf16x4*>(kir + 32);
                const bf16x8 fi = {i0[0], i0[1], i0[2], i0[3], i1[0], i1[1], i1[2], i1[3]};
                const bf16x8 fk = *reinterpret_cast<const bf16x8*>(slot + Cfg::O_KT + off);
                const bf16x8 fq = *reinterpret_cast<const bf16x8*>(slot + Cfg::O_QT + off);
                akk = mfma32(fi, fk, akk);     // [s][r] = -A_kk[r][s] (the tile holds -Kt)
                aqk = mfma32(fi, fq, aqk);     // [s][r] = A_qk[r][s]
            }
            // lane (q, r) holds A[r][4q+i]: exactly the 16x16x16 A operand of row r
            *reinterpret_cast<shortx4*>(slot + Cfg::O_AQ + lane * 8) =
                pack4(4 * lq + 0 <= lr ? aqk[0] : 0.f, 4 * lq + 1 <= lr ? aqk[1] : 0.f,
                      4 * lq + 2 <= lr ? aqk[2] : 0.f, 4 * lq + 3 <= lr ? aqk[3] : 0.f);

            // ---- M' = (I + N)^{-1} diag(beta), N = diag(beta) A_kk -----------
            // Lane (q, c) holds -A_kk[c][4q+i] (the tile holds -Kt); masked to
            // the strict lower triangle and scaled by beta_c (this lane's
            // beta, token c), entries 4q .. 4q+3 of row c of -N.  Through the
            // slot's scratch every lane then reads a whole row r = lr of -N
            // and solves (I + N) X = diag(beta) for X[r][4q .. 4q+3], which is
            // M' in the 16x16x16 A-operand layout (lane (q, r): row r,
            // columns 4q .. 4q+3).
            const floatx4 nq = {4 * lq + 0 < lr ? bl * akk[0] : 0.f, 4 * lq + 1 < lr ? bl * akk[1] : 0.f,
                                4 * lq + 2 < lr ? bl * akk[2] : 0.f, 4 * lq + 3 < lr ? bl * akk[3] : 0.f};
            if (go) {
                char* scr = smem + (kStageO ? Cfg::O_OS + s * 16 * Cfg::PO : Cfg::O_NB + s * 16 * Cfg::PN) +
                            lr * Cfg::PN;
                *reinterpret_cast<floatx4*>(scr + 16 * lq) = nq;
                float x[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) x[k] = lr == 4 * lq + k ? bl : 0.f;
                forward_rows(x, scr);
                *reinterpret_cast<shortx4*>(slot + Cfg::O_MP + lane * 8) = pack4(x[0], x[1], x[2], x[3]);
                // publish the chunk after every lane's M' writes (the LDS
                // performs this wave's operations in order; the release keeps
                // the compiler from sinking the writes below it)
                if (lane == 0)
                    __hip_atomic_store(&ready[s], round + 1, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            }
            if constexpr (kLateWait && !kTopLoad) {
                issue_gkq(ci + kNP);
                issue_v(ci + kNP);
            }
            if (go) last = ci;
            ci = go ? ci + kNP : n_chunks;
        }
        // the output rows of this wave's last chunk, once every consumer has
        // released it (a wait that runs out leaves them unwritten; the final
        // state then reads NaN)
        if constexpr (kStageO) {
            if (last >= 0) {
                const int s = (int)(last % kRing);
                if (wait_all_at_least<NC>(&released[s * NC], (int)(last / kRing) + 1, stop)) store_o(last, s);
            }
        }
        return;
    }

    // ======================== consumer wave ==================================
    const int w = wave;                      // value columns n0 + 16w .. +15
    // The consumers' chain paces the kernel while the producers wait for
    // releases about half the time, so a consumer wins the SIMD's issue
    // arbitration (same-box timing: bf16 and MXFP8 1.3-1.5 % faster).  Not
    // with conv inputs, whose producers are the slower side (1.7 % slower).
    if constexpr (!CV) __builtin_amdgcn_s_setprio(1);
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
    // Software pipeline over the chunks.  The operands of a chunk's products
    // with S (Kt, Qt) and V, M' are read while the previous chunk updates the
    // state; Ki, A_qk and the decays at the start of the chunk, behind the
    // Kt S products.  The loop has no early exit (an exit path would merge
    // with the carried operand registers at the loop's latch and add a wait
    // for them): a wait that runs out raises the stop flag and ends the loop
    // through its condition.
    const int tr_row = 4 * lq + (lr >> 2), tr_col = 4 * (lr & 3);
    bf16x8 fk[NKS], fq[NKS];
    bf16v4 vv;
    shortx4 mp;
    auto read_head = [&](const char* slot) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const int off = lr * PK + (32 * ks + 8 * lq) * 2;
            fk[ks] = *reinterpret_cast<const bf16x8*>(slot + Cfg::O_KT + off);
            fq[ks] = *reinterpret_cast<const bf16x8*>(slot + Cfg::O_QT + off);
        }
        // V in accumulator layout: tokens 4q .. 4q+3 of column 16w + c
        // (transposed read: lane (q, c) receives rows 4q .. 4q+3 of column c)
        vv = lds_read_tr(slot + Cfg::O_V + tr_row * Cfg::PV + (16 * w + tr_col) * 2);
        mp = *reinterpret_cast<const shortx4*>(slot + Cfg::O_MP + lane * 8);
    };
    bool ok = nch == 0 || wait_at_least(&ready[0], 1, stop);
    // the slot is read only after its counter was seen (the compiler keeps
    // the reads below this point; the LDS serves a wave's operations in order)
    asm volatile("" ::"s"((int)ok) : "memory");
    read_head(smem);
    // output: a pointer that advances one chunk of rows per step and the
    // rows left in the sequence
    const int o_row = H * DV * 2;   // bytes between tokens
    const __bf16* o_chunk = o + (t_begin * H + head) * DV + n0 + 16 * w;
    int rows_left = (int)(t_end - t_begin);
    for (unsigned ci = ok ? 0u : (unsigned)nch; ci < (unsigned)nch;) {
        const char* slot = smem + (ci % kRing) * SLOT;
        // the rest of this chunk's operands
        bf16v4 ki[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) ki[kt] = lds_read_tr(slot + Cfg::O_KI + tr_row * PH + (16 * kt + tr_col) * 2);
        const shortx4 aq = *reinterpret_cast<const shortx4*>(slot + Cfg::O_AQ + lane * 8);
        const floatx2 gm = *reinterpret_cast<const floatx2*>(slot + Cfg::O_GM + (lq * 16 + lr) * 8);
        // Release point.  Packed batches of bf16 inputs (no output staging)
        // are done with the slot once these reads are issued (the LDS serves
        // them before the release): released here, 1.9 % faster than at the
        // end of the iteration.  With staging the output rows go into the
        // slot's staging area first; MXFP8 and conv inputs measured no
        // better (conv inputs 2.9 % slower) and keep the late release.
        constexpr bool kEarlyRelease = !kStageO && !MX && !CV;
        if constexpr (kEarlyRelease) flag_store(&released[(ci % kRing) * NC + w], (int)(ci / kRing) + 1, lane);
        // the next chunk's counter, read early (a value already at the target
        // saves the polling round trip later); the acquire that pairs with the
        // producer's release is the fence below, once the value is used, so
        // the products need not wait for this chunk's operand reads
        const unsigned cn = ci + 1;
        int* rdy = &ready[cn % kRing];
        const int target = cn < (unsigned)nch ? (int)(cn / kRing) + 1 : 0;
        const int peek = __hip_atomic_load(rdy, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);

        // S as permuted bf16 operands: the same registers are the B operand of
        // S and the A operand of S^T
        bf16x8 sb[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sb[ks][e] = (__bf16)S[2 * ks][e];
                sb[ks][4 + e] = (__bf16)S[2 * ks + 1][e];
            }
        // R = V - Kt S (the state chain) first, then O^T = S^T Qt^T, which
        // fills the wait for R.  V is the chain's initial accumulator (its
        // transposed read is the accumulator layout; bf16 to fp32 is exact)
        // and the Kt tile holds -Kt.  (V no longer enters through a 16x16x16
        // identity product: a 16x16x16 result read as the accumulator of a
        // 16x16x32 product with no wait states between them came out wrong
        // on gfx950, and the compiler puts none there.)
        floatx4 z = {(float)vv[0], (float)vv[1], (float)vv[2], (float)vv[3]};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) z = mfma32(fk[ks], sb[ks], z);
        __builtin_amdgcn_sched_barrier(0);
        floatx4 oa = zero4();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) oa = mfma32(sb[ks], fq[ks], oa);
        __builtin_amdgcn_sched_barrier(0);
        // U = M' (V - Kt S): the accumulator layout is the 16x16x16 B layout
        const floatx4 u = mfma16(mp, pack4(z[0], z[1], z[2], z[3]), zero4());
        const shortx4 ub = pack4(u[0], u[1], u[2], u[3]);
        // S + Ki^T U, tile by tile (the decay follows below)
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) S[kt] = mfma16(__builtin_bit_cast(shortx4, ki[kt]), ub, S[kt]);
        // O^T += U^T A_qk^T: U's accumulator is the A operand of U^T, and the
        // A_qk operand registers are the B operand of A_qk^T.  This 16x16x16
        // product takes the 16x16x32 chain's O^T as its accumulator; the
        // scheduling barriers keep the U product, the wait for its result and
        // its packing between them (21 or more wait states in every
        // instantiation).
        oa = mfma16(ub, aq, oa);
        // lane (q, t) holds O[t][16w + 4q .. +3]: 8 bytes of the chunk's output
        // rows, staged for the producer that refills this slot
        if constexpr (kStageO)
            *reinterpret_cast<u32x2*>(smem + Cfg::O_OS + (ci % kRing) * 16 * Cfg::PO + lr * Cfg::PO +
                                      (16 * w + 4 * lq) * 2) =
                __builtin_bit_cast(u32x2, pack4(oa[0], oa[1], oa[2], oa[3]));
        // every read of this slot (and the staging write) has been issued; the
        // release waits for them
        if constexpr (!kEarlyRelease) flag_store(&released[(ci % kRing) * NC + w], (int)(ci / kRing) + 1, lane);
        // the next chunk's leading operands, read while the state updates
        ok = __builtin_amdgcn_readfirstlane(peek) >= target || wait_at_least(rdy, target, stop);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        asm volatile("" ::"s"((int)ok) : "memory");
        read_head(smem + (cn % kRing) * SLOT);
        // S <- diag(e^{G_15}) (S + Ki^T U): row i of tile kt is channel
        // 16 kt + 4q + i; its decay sits in lane 2 kt + i/2 of the lane's own
        // row, component i % 2
        decay_rows<0, NKT>(S, gm);

        // unstaged (packed batches, MXFP8 and conv inputs): lane (q, t) stores
        // O[t][16w + 4q .. +3] itself, 8 bytes; the resource covers the
        // chunk's rows inside the sequence, so rows past its end are dropped
        // without a branch
        if constexpr (!kStageO) {
            const rsrc_t r_o = make_rsrc(o_chunk, (uint32_t)((rows_left < 16 ? rows_left : 16) * o_row));
            __builtin_amdgcn_raw_buffer_store_b64(
                __builtin_bit_cast(u32x2, pack4(oa[0], oa[1], oa[2], oa[3])), r_o,
                lr * o_row + 8 * lq, 0, 0);
            o_chunk += 16 * H * DV;
            rows_left -= 16;
        }
        ci = ok ? cn : (unsigned)nch;
    }
    if (sT != nullptr) {
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sT[sbase + (int64_t)(16 * kt + 4 * lq + i) * DV] = ok ? S[kt][i] : nan;
    }
}

template <int DK, int DVS, int IN>
hipError_t launch_pipe_t(const void* q, const void* k, const void* v, int64_t stride,
                         const void* g, const void* beta, void* o, const float* s0, float* sT,
                         const int32_t* cu, int num_seqs, int T_len, int H, int DV,
                         const void* qsc, const void* ksc, const void* vsc, const void* gsc,
                         const float* cw, const void* cs_in, float l2_eps, hipStream_t s) {
    using TIn = typename PipeIn<IN>::type;
    const int nsplit = DV / DVS;
    const int64_t blocks = (int64_t)num_seqs * H * nsplit;
    if (blocks == 0) return hipSuccess;
    const int blocked = (IN == kInMx || num_seqs > 1) ? 1 : 0;
    auto go = [&](auto so) {
        hipLaunchKernelGGL((chunk_pipe_kernel<DK, DVS, IN, decltype(so)::value>), dim3((unsigned)blocks),
                           dim3(PipeCfg<DK, DVS>::THREADS), 0, s, (const TIn*)q, (const TIn*)k,
                           (const TIn*)v, stride, (const TIn*)g, (const __bf16*)beta, (__bf16*)o,
                           s0, sT, cu, num_seqs, T_len, H, DV, nsplit, (const uint8_t*)qsc,
                           (const uint8_t*)ksc, (const uint8_t*)vsc, (const uint8_t*)gsc, cw,
                           (const __bf16*)cs_in, l2_eps, blocked);
    };
    if (IN == kInBf16 && !blocked)
        go(std::integral_constant<bool, IN == kInBf16>{});
    else
        go(std::false_type{});
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_pipe(const void* q, const void* k, const void* v, int64_t stride,
                             const void* g, const void* beta, void* o, const float* s0,
                             float* sT, const int32_t* cu, int num_seqs, int T, int H, int DK,
                             int DV, hipStream_t s) {
    if (DK == 128)
        return launch_pipe_t<128, 64, kInBf16>(q, k, v, stride, g, beta, o, s0, sT, cu, num_seqs,
                                               T, H, DV, nullptr, nullptr, nullptr, nullptr,
                                               nullptr, nullptr, 0.f, s);
    return launch_pipe_t<64, 64, kInBf16>(q, k, v, stride, g, beta, o, s0, sT, cu, num_seqs, T, H,
                                          DV, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                          0.f, s);
}

hipError_t launch_chunk_pipe_mxfp8(const void* q, const void* qsc, const void* k,
                                   const void* ksc, const void* v, const void* vsc,
                                   int64_t stride, const void* g, const void* gsc,
                                   const void* beta, void* o, const float* s0, float* sT,
                                   const int32_t* cu, int num_seqs, int T, int H, hipStream_t s) {
    return launch_pipe_t<128, 64, kInMx>(q, k, v, stride, g, beta, o, s0, sT, cu, num_seqs, T, H,
                                         128, qsc, ksc, vsc, gsc, nullptr, nullptr, 0.f, s);
}

hipError_t launch_chunk_pipe_conv(const void* x, const float* cw, const void* cs_in,
                                  const void* g, const void* beta, void* o, const float* s0,
                                  float* sT, const int32_t* cu, int num_seqs, int T, int H, int D,
                                  float l2_eps, hipStream_t s) {
    const int64_t HD = (int64_t)H * D;
    const __bf16* xb = static_cast<const __bf16*>(x);
    if (D == 128)
        return launch_pipe_t<128, 64, kInConv>(xb, xb + HD, xb + 2 * HD, 3 * HD, g, beta, o, s0,
                                               sT, cu, num_seqs, T, H, D, nullptr, nullptr,
                                               nullptr, nullptr, cw, cs_in, l2_eps, s);
    return launch_pipe_t<64, 64, kInConv>(xb, xb + HD, xb + 2 * HD, 3 * HD, g, beta, o, s0, sT,
                                          cu, num_seqs, T, H, D, nullptr, nullptr, nullptr,
                                          nullptr, cw, cs_in, l2_eps, s);
}

}  // namespace kda
