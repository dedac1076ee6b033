// Sparse latent attention with a per-head sink for gfx950 (MI355X).
//
// Operation: DeepSeek-V4.1 pages, "Output projection" page, Attention.forward
// excerpt (o = sparse_attn(q, kv, attn_sink, topk_idxs, softmax_scale)); the
// semantics and layouts are stated in include/sparse_attn.h.
//
// Kernels (the host picks one attention kernel per call from the dims)
//   attn_fwd_kernel     deep gather: one workgroup per (query, 64 or 32 heads,
//                       split).  Index decode + compaction of the query's list
//                       into LDS, a per-split slice of the valid entries, then
//                       chunks of 32 rows: LDS-DMA gather into a 4-chunk ring,
//                       S^T = K Q^T on 16x16x32 bf16 MFMAs (a pair of waves per
//                       16 heads, one per half of d), the online sink softmax in
//                       float32, O^T += V^T P^T with V through LDS transpose
//                       loads.  Epilogue: bf16 output, or a split's fp16
//                       partial (a power of two per row), staged through LDS
//                       into whole-row stores.
//   attn_fwd_mq_kernel  many queries (prefill): the same steps with two
//                       workgroups of four waves per compute unit, each wave
//                       over the whole of d for its 16 heads.
//   attn_fwd_hs_kernel  head split (short lists, unsplit): one workgroup per
//                       (query, 16 heads) over the whole list; rows staged
//                       through registers, no partials.
//   combine_kernel      log-sum-exp merge of split partials plus the sink.
//   topk_reg_kernel /   the lists' compressed segment: radix select of the k
//   topk_long_kernel    best scores per row, in index order.
//   check_idxs_kernel   counts entries >= N (checked mode).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "sparse_attn.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int KC = 32;                // rows (list entries) per chunk
constexpr int DMA_LAG = 6;            // QK^T steps before a group of row DMAs goes out

// The QK^T step that issues group q of ng groups of row DMAs spread evenly
// over nsteps steps.
constexpr int dma_step(int q, int ng, int nsteps) {
    return q * nsteps / ng + DMA_LAG < nsteps ? q * nsteps / ng + DMA_LAG : nsteps - 1;
}
constexpr int LIST_CAP = 2048;        // longest index list a workgroup compacts
constexpr int LDS_BYTES = 160 * 1024; // LDS per compute unit (gfx950)

// Static LDS of attn_fwd_kernel<D, NHQ, HT> (its ring, partial scores,
// published weights and factors, per-wave counts); the compacted list comes on
// top as dynamic LDS, 4 bytes per entry.
constexpr size_t fwd_ring_slots(int NHQ) {
    return 2 + (63 / (32 / (2 * NHQ)) >= 2 ? 2 : 63 / (32 / (2 * NHQ)));
}
constexpr size_t fwd_static_lds(int D, int NHQ, int HT) {
    return fwd_ring_slots(NHQ) * 32 * (2 * D + 32) + (size_t)(2 * NHQ) * (2 * HT) * 64 * 16 +
           (size_t)NHQ * HT * 1024 + (size_t)NHQ * HT * 64 + (size_t)(2 * NHQ) * 4;
}
size_t list_lds_bytes(int K) { return ((size_t)(K > 0 ? K : 1) * 4 + 15) / 16 * 16; }
// Static LDS of attn_fwd_hs_kernel<D>: three round buffers of 48 padded rows,
// two sets of published weights (3 blocks x 64 lanes x 8 bytes) with their
// references and sums, per-wave counts.
constexpr size_t hs_static_lds(int D) {
    return 3 * 48 * (size_t)(2 * D + 32) + 2 * 3 * 64 * 8 + 2 * 2 * 3 * 16 * 4 + 8 * 4;
}
constexpr int MAX_SPLITS = 64;
constexpr float LOG2E = 1.4426950408889634f;
// The running max is only raised when a chunk beats it by more than this many
// log2 units; until then weights stay <= 2^8 relative to the kept max, which
// float32 sums and bf16 weights hold without loss, and the output (numerator
// and denominator share the reference) is unchanged.
constexpr float MAX_SLACK = 8.0f;

// Division by a launch-constant d >= 1 of dividends 0 <= n < 2^31 as a
// multiply and a shift: n / d == (n * m) >> k with l = ceil(log2 d),
// k = 31 + l and m = ceil(2^k / d) < 2^32 (Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994, Theorem 4.2
// with N = 31 bits: 2^k <= m d <= 2^k + 2^l).  The host computes (m, k); on
// the device it is three scalar instructions instead of a reciprocal
// sequence, ahead of the kernels' first memory requests.
struct Div32 {
    uint32_t m, k;
};
__host__ __device__ inline int udiv(int n, Div32 d) {
    return (int)(((uint64_t)(uint32_t)n * d.m) >> d.k);
}

struct FwdParams {
    const uint16_t *q;
    // Rows: index j < W is row j of the first source (rows_a rows per
    // sequence), j >= W is row j - W of the second (rows_b per sequence).
    // One tensor is the case W = N.
    const uint16_t *kv;     // first source  [B, rows_a, D]
    const uint16_t *kv2;    // second source [B, rows_b, D]
    int64_t W, rows_a, rows_b;
    int32_t rec2;           // 0: the second source holds bf16 rows; else it holds FP4
                            // records of rec2 bytes (see expand_fp4_own)
    const float *sink;
    const int32_t *idxs;
    uint16_t *out;     // non-split path
    uint16_t *ws_o;    // split path: [Q, S, H, D] fp16, each split normalised by its ws_l
                       // and divided by the power of two ws_x of its row
    float *ws_m;       // [Q, S, H] running max, log2 units
    float *ws_l;       // [Q, S, H] denominator relative to ws_m
    float *ws_x;       // [Q, S, H] power-of-two scale of each row of ws_o
    int32_t *ws_plan;  // [Q] splits each query's list was cut into (written by split 0)
    int64_t N;
    int32_t T, H, K;
    int32_t S, HG, units, per_xcd, bs;  // see unit_of
    Div32 dv_bs, dv_S, dv_HG, dv_T;      // division by bs, S, HG and T
    float qk_scale_log2;  // scale * log2(e)
    // f3: the output's last rd dims rotated back, pair i of query (b, t) by
    // rope[t, i] = (cos, sin) (rd = 0: none)
    const float *rope;
    int32_t rd;
};

// f3: inverse rotary step on two pairs (x0, y0), (x1, y1) of an output row
// (DeepSeek-V4.1 pages, "Output projection" page, Attention.forward excerpt:
// apply_rotary_emb on o[..., -rd:] with inverse=True).  A pair is the complex
// number x + iy, multiplied by the conjugate of freqs_cis = cs.x + i cs.y
// (and cs.z + i cs.w for the second pair).
__device__ __forceinline__ void rotate_back2(float &x0, float &y0, float &x1, float &y1, float4 cs) {
    const float a0 = x0 * cs.x + y0 * cs.y, b0 = y0 * cs.x - x0 * cs.y;
    const float a1 = x1 * cs.z + y1 * cs.w, b1 = y1 * cs.z - x1 * cs.w;
    x0 = a0, y0 = b0, x1 = a1, y1 = b1;
}

// Swizzle of the epilogue's output staging rows (16-bit rows of 256 B to
// 1 KB in LDS): 8-byte piece k of row r lives at piece position k ^ (r & 15).
// A staging write stores one 8-byte piece per lane, the 16 lanes of a lane
// group on 16 rows at the same piece; gfx950's LDS takes such a b64 write 16
// lanes (128 bytes, 32 four-byte banks) per cycle, so the 16 pieces must land
// on 16 distinct 8-byte bank pairs ((byte address / 8) mod 16), which the
// row-dependent XOR gives (every row starts on pair 0).  Measured with
// SQ_LDS_BANK_CONFLICT: 12 conflict cycles per write instruction with a
// 16-byte-granular swizzle of 2r, 4 with r, none with this one.  Reading a
// 16-byte slot back gives one 16-byte chunk of the row, its two halves
// swapped when r is odd (see store_outputs).
__device__ __forceinline__ int stage_swz(int r) { return r & 15; }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// a10: the split plan of one query, from its own count of valid entries.
// A launch provides S split slots per query (S chosen on the host from the
// list capacity K); a query with n valid entries uses the first
// Sq = ceil(n S / K) of them (1 <= Sq <= S), each taking a contiguous range
// of about n / Sq valid entries.  No range is longer than with the capacity
// plan, short lists leave their spare slots idle, and the combine merges only
// Sq partials.  Computed on the device by every workgroup of the query after
// compaction; split 0 records Sq for the combine.
__device__ __forceinline__ int query_splits(int n, int K, int S) {
    if (S <= 1 || K <= 0) return 1;
    const int sq = (n * S + K - 1) / K;  // n <= K <= LIST_CAP, S <= MAX_SPLITS: 32 bits suffice
    return sq < 1 ? 1 : (sq > S ? S : sq);
}

// Workgroup -> unit (one (query, head group, split) each), or -1 for a spare
// workgroup.  Workgroups go to the eight XCDs round-robin by blockIdx; XCD x
// runs blocks x, x+8, x+16, ... of bs consecutive units, so the splits and
// head groups of a query (bs is a multiple of their count) and neighbouring
// queries share an XCD's L2, while every XCD gets a share of every part of
// the batch.  Units run in reverse order: in causal prefill the late queries
// have the longest lists, and starting them first shortens the tail.
__device__ __forceinline__ int unit_of(int bid, int units, int bs, Div32 dv_bs) {
    const int x = bid & 7, j = bid >> 3;
    const int jb = udiv(j, dv_bs);
    const int u = (jb * 8 + x) * bs + (j - jb * bs);
    return u < units ? units - 1 - u : -1;
}

// Sum and max of x over the lanes l mod 16 + 16k, k = 0..3 (the four 16-lane
// rows of a wave), returned in every lane: two lane swaps on the VALU
// (gfx950's v_permlane16_swap and v_permlane32_swap) in place of two LDS
// permutes.  Swapping x with itself returns, in its two results, x of the
// lane and x of the lane one row (then one half-wave) away, in the same order
// in every lane, so all lanes agree bit for bit, as with xor shuffles.  Every
// lane of the wave must be active.
__device__ __forceinline__ float sum_rows4(float x) {
    const u32x2_t p = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false));
    const float y = __uint_as_float(p[0]) + __uint_as_float(p[1]);
    const u32x2_t q = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false));
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float max_rows4(float x) {
    const u32x2_t p = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false));
    const float y = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
    const u32x2_t q = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false));
    return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// Max or sum of x over each aligned group of G lanes (G = 16, 32 or 64),
// returned in every lane of the group, on the VALU: within a 16-lane row by
// DPP (quad permutes, then the half-row and row mirrors, each pairing every
// lane with one from the other half of its group), across rows by the lane
// swaps above.  (Cross-lane shuffles through LDS would take one LDS round
// trip per step.)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int G, bool MAX>
__device__ __forceinline__ float group_reduce(float x) {
    static_assert(G == 16 || G == 32 || G == 64, "rows of 16 lanes");
    auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
    x = op(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
    x = op(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
    x = op(x, dpp_f<0x141>(x));  // row_half_mirror
    x = op(x, dpp_f<0x140>(x));  // row_mirror
    if constexpr (G >= 32) {
        const u32x2_t p = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false));
        x = op(__uint_as_float(p[0]), __uint_as_float(p[1]));
    }
    if constexpr (G == 64) {
        const u32x2_t q = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false));
        x = op(__uint_as_float(q[0]), __uint_as_float(q[1]));
    }
    return x;
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Two floats to two bf16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// lo + hi of a packed pair of bf16 values, plus acc, in one v_dot2_f32_bf16
// (dot product with (1, 1); the products are exact).
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float acc) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), one, acc, false);
}

// Two floats to two fp16 (round to nearest even), low half first.
__device__ __forceinline__ uint32_t pack2_f16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}

__device__ __forceinline__ f32x2_t unpack2_f16(uint32_t w) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
}

// a1: index decode + compaction of a list already staged in LDS.  Wave w
// takes a contiguous segment of the list (a multiple of 64 entries); a ballot
// per 64 entries ranks its valid entries, one barrier publishes the per-wave
// counts, and each wave writes its entries after those of the waves before
// it, so the order is kept.  All reads of `lst` happen before the first
// barrier and all writes after it, so `list` may be `lst` (compaction in
// place).  cnt holds NT/64 ints.  Returns the number of valid entries
// (0 <= idx < N); `list` is complete for every wave on return.
template <int NT>
__device__ int compact_list(const LDS_AS int32_t *lst, int K, int64_t N, int32_t *list,
                            int32_t *cnt) {
    constexpr int NWV = NT / 64;
    constexpr int MAXR = (LIST_CAP + NT - 1) / NT;  // rounds of 64 per wave, at most
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int seg = ((K + NWV - 1) / NWV + 63) / 64 * 64;
    const int k0 = wid * seg;
    int v[MAXR];
    uint64_t mask[MAXR];
    int total = 0;
    // 0 <= v < N as one unsigned 32-bit compare (entries are int32)
    const uint32_t Nu = (uint32_t)(N < 0x80000000LL ? N : 0x80000000LL);
    // every read is issued before any is used (indices clamped into the
    // list, the entries beyond it discarded after)
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
        const int k = k0 + r * 64 + lane;
        v[r] = lst[k < K ? k : (K > 0 ? K - 1 : 0)];
    }
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
        const int k = k0 + r * 64 + lane;
        if (!(r * 64 < seg && k < K)) v[r] = -1;
        mask[r] = __ballot((uint32_t)v[r] < Nu);
        total += __popcll(mask[r]);
    }
    if (lane == 0) cnt[wid] = total;
    __syncthreads();
    int base = 0, n = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
        const int c = cnt[w];
        base += w < wid ? c : 0;
        n += c;
    }
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
        if ((mask[r] >> lane) & 1ull) list[base + __popcll(mask[r] & ((1ull << lane) - 1ull))] = v[r];
        base += __popcll(mask[r]);
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(n);
}

// One LDS-DMA wave instruction: every lane fetches 16 bytes from its own
// global address; they land at lds_base + 16 * lane.  Issued through asm so
// the compiler does not order later LDS reads behind it (it would otherwise
// wait for every DMA in flight before any LDS read); the ring below waits for
// exactly the chunk it needs with wait_vm_ahead.
__device__ __forceinline__ void lds_dma16(const void *gptr, const LDS_AS void *lds_base) {
    // the LDS base is wave-uniform; readfirstlane puts it in an SGPR for M0
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gptr), "s"(m0)
                 : "memory", "m0");
}

// Same, non-temporal: for rows that one workgroup reads once (the deep-gather
// kernel's decode-shaped launches), so they do not take cache lines from data
// that is reused (q, partials on their way to the combine).
__device__ __forceinline__ void lds_dma16_nt(const void *gptr, const LDS_AS void *lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                 :
                 : "v"(gptr), "s"(m0)
                 : "memory", "m0");
}

// Same with a wave-uniform row base in SGPRs and a per-lane byte offset
// (saddr form: no 64-bit per-lane address arithmetic).
__device__ __forceinline__ void lds_dma16_s(const void *sbase, uint32_t voff,
                                            const LDS_AS void *lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0)
                 : "memory", "m0");
}

// Four rows with one M0 write.  The instruction offset is added to both the
// global and the LDS address, so row j (0..3) lands at lds_base + j*RS +
// 16*lane when its global address is passed less j*RS.  Writing M0 once per
// four rows instead of once per row roughly doubles the rate at which a
// compute unit issues these DMAs (a 640-row-per-workgroup gather over 64
// workgroups takes 17 us instead of 33).  The addresses less j*RS are never
// accessed themselves; they are formed as integers (they may lie before the
// allocation).
__device__ __forceinline__ uint64_t addr_less(const uint8_t *p, int bytes) {
    return (uint64_t)(uintptr_t)p - (uint64_t)bytes;
}
template <int RS>
__device__ __forceinline__ void lds_dma16x4_nt(const uint8_t *g0, const uint8_t *g1, const uint8_t *g2,
                                               const uint8_t *g3, const LDS_AS void *lds_base) {
    static_assert(3 * RS < 4096, "row offsets fit the instruction's offset field");
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %4\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, off nt\n\t"
                 "global_load_lds_dwordx4 %1, off offset:%5 nt\n\t"
                 "global_load_lds_dwordx4 %2, off offset:%6 nt\n\t"
                 "global_load_lds_dwordx4 %3, off offset:%7 nt"
                 :
                 : "v"(g0), "v"(addr_less(g1, RS)), "v"(addr_less(g2, 2 * RS)), "v"(addr_less(g3, 3 * RS)),
                   "s"(m0), "n"(RS), "n"(2 * RS), "n"(3 * RS)
                 : "memory", "m0");
}

// Same in the saddr form: wave-uniform row bases in SGPRs, one per-lane byte
// offset shared by the four rows.
template <int RS>
__device__ __forceinline__ void lds_dma16x4_s(const uint8_t *s0, const uint8_t *s1, const uint8_t *s2,
                                              const uint8_t *s3, uint32_t voff, const LDS_AS void *lds_base) {
    static_assert(3 * RS < 4096, "row offsets fit the instruction's offset field");
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %5\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %1\n\t"
                 "global_load_lds_dwordx4 %0, %2 offset:%6\n\t"
                 "global_load_lds_dwordx4 %0, %3 offset:%7\n\t"
                 "global_load_lds_dwordx4 %0, %4 offset:%8"
                 :
                 : "v"(voff), "s"(s0), "s"(addr_less(s1, RS)), "s"(addr_less(s2, 2 * RS)),
                   "s"(addr_less(s3, 3 * RS)), "s"(m0), "n"(RS), "n"(2 * RS), "n"(3 * RS)
                 : "memory", "m0");
}

// The saddr forms with the non-temporal hint (rows read once).
__device__ __forceinline__ void lds_dma16_s_nt(const void *sbase, uint32_t voff,
                                               const LDS_AS void *lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(voff), "s"(sbase), "s"(m0)
                 : "memory", "m0");
}
template <int RS>
__device__ __forceinline__ void lds_dma16x4_s_nt(const uint8_t *s0, const uint8_t *s1, const uint8_t *s2,
                                                 const uint8_t *s3, uint32_t voff, const LDS_AS void *lds_base) {
    static_assert(3 * RS < 4096, "row offsets fit the instruction's offset field");
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %5\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %0, %1 nt\n\t"
                 "global_load_lds_dwordx4 %0, %2 offset:%6 nt\n\t"
                 "global_load_lds_dwordx4 %0, %3 offset:%7 nt\n\t"
                 "global_load_lds_dwordx4 %0, %4 offset:%8 nt"
                 :
                 : "v"(voff), "s"(s0), "s"(addr_less(s1, RS)), "s"(addr_less(s2, 2 * RS)),
                   "s"(addr_less(s3, 3 * RS)), "s"(m0), "n"(RS), "n"(2 * RS), "n"(3 * RS)
                 : "memory", "m0");
}

// Same with 4 bytes per lane (landing at lds_base + 4 * lane).
__device__ __forceinline__ void lds_dma4(const void *gptr, const LDS_AS void *lds_base) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_base);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :
                 : "v"(gptr), "s"(m0)
                 : "memory", "m0");
}

// s_waitcnt with a vmcnt chosen at run time among the few values the ring can
// need (the immediate must be a constant).  Waits until at most `n` vector
// memory operations of this wave are still outstanding.
template <int STEP, int MAXA>
__device__ __forceinline__ void wait_vm_ahead(int ahead) {
    static_assert(STEP > 0 && MAXA >= 0 && MAXA <= 2 && MAXA * STEP <= 63, "vmcnt is 6 bits");
    if (MAXA >= 2 && ahead >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * STEP) : "memory");
    else if (MAXA >= 1 && ahead >= 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(STEP) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// s_waitcnt until at most n (0 <= n <= MAXN <= 16) vector memory operations
// of this wave are outstanding, n known only at run time (the immediate must
// be a constant): one branch per possible value.
template <int MAXN>
__device__ __forceinline__ void wait_vm_upto(int n) {
    static_assert(MAXN >= 0 && MAXN <= 16, "a few cases");
#define SA_WAIT_CASE(k) \
    if (MAXN >= k && n == k) { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(k) : "memory"); return; }
    SA_WAIT_CASE(16) SA_WAIT_CASE(15) SA_WAIT_CASE(14) SA_WAIT_CASE(13) SA_WAIT_CASE(12)
    SA_WAIT_CASE(11) SA_WAIT_CASE(10) SA_WAIT_CASE(9) SA_WAIT_CASE(8) SA_WAIT_CASE(7)
    SA_WAIT_CASE(6) SA_WAIT_CASE(5) SA_WAIT_CASE(4) SA_WAIT_CASE(3) SA_WAIT_CASE(2) SA_WAIT_CASE(1)
#undef SA_WAIT_CASE
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// a7 / a8: epilogue shared by the attention kernels.  The workgroup holds
// HWG = 16*NTL heads; wave w of NW holds the output columns
// w*DW .. w*DW + DW - 1 (DW = D/NW) of every head: lane (li, g) holds
// O^T[w*DW + 16u + 4g + i, 16t + li] in o[t][u][i].  mh / lh give each head's
// running max (log2 units) and total denominator; red is scratch for NW*HWG
// floats.  Every output (final, or a split's partial) is normalised by its own
// denominator, then staged through LDS (HWG rows of 2D bytes at `stage_out`,
// which the caller has freed with a barrier) so that each wave instruction
// stores whole rows: the final output as bf16, a split's partial as fp16
// divided by a power of two per row.  In LDS, 8-byte piece k (columns 4k ..
// 4k + 3) of head row hl sits at piece position k ^ stage_swz(hl), which keeps
// the 16 rows written by one store instruction on distinct banks.
template <int D, int NW, int NTL>
__device__ __forceinline__ void store_outputs(const FwdParams &p, const f32x4_t (&o)[NTL][D / NW / 16],
                                              const LDS_AS float *mh, const LDS_AS float *lh,
                                              LDS_AS float *red, int qi, int s, int hg,
                                              LDS_AS uint8_t *stage_out) {
    constexpr int NT = NW * 64;
    constexpr int HWG = 16 * NTL;
    constexpr int DW = D / NW;
    constexpr int NU = DW / 16;
    constexpr int C16 = D / 8;  // 16-byte chunks per 16-bit row
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int hbase = hg * HWG;
    // the sink of every head tile requested before any is used (in a branch
    // each, they would go out one memory round trip at a time)
    const bool with_sink = p.S == 1 && p.sink != nullptr;
    float zsv[NTL];
    if (with_sink) {
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            const int h = hbase + 16 * t + li;
            zsv[t] = p.sink[h < p.H ? h : 0];
        }
    }
    float inv[NTL];
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
        const int hl = 16 * t + li;
        const int h = hbase + hl;
        const float ltot = lh[hl], mm = mh[hl];
        inv[t] = ltot > 0.f ? 1.f / ltot : 0.f;
        if (with_sink && h < p.H) {
            // the sink joins the softmax: M = max(m, sink), L = l 2^(m-M) + 2^(sink-M);
            // nothing to attend to (m and the sink both -inf) gives 0
            const float zs = zsv[t] * LOG2E;
            const float M = fmaxf(mm, zs);
            const float alpha = mm == -INFINITY ? 0.f : exp2_fast(mm - M);
            inv[t] = M == -INFINITY ? 0.f : alpha / (ltot * alpha + exp2_fast(zs - M));
        }
    }
    if (p.S == 1) {
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            const int hl = 16 * t + li;
            LDS_AS uint8_t *Rrow = stage_out + hl * (D * 2);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int col = wid * DW + 16 * u + 4 * g;  // first of 4 columns (piece col / 4)
                const int pk = (col >> 2) ^ stage_swz(hl);
                float v0 = o[t][u][0] * inv[t], v1 = o[t][u][1] * inv[t];
                float v2 = o[t][u][2] * inv[t], v3 = o[t][u][3] * inv[t];
                if (col >= D - p.rd) {  // rotary dims: pairs (col, col+1), (col+2, col+3)
                    const int64_t pr = (int64_t)(qi % p.T) * (p.rd / 2) + (col - (D - p.rd)) / 2;
                    rotate_back2(v0, v1, v2, v3, *(const float4 *)(p.rope + 2 * pr));
                }
                const u32x2_t w = {pack2_bf16(v0, v1), pack2_bf16(v2, v3)};
                *(LDS_AS u32x2_t *)(Rrow + pk * 8) = w;
            }
        }
    } else {
        // A split's partial: fp16 rows (11 significant bits) divided by a power
        // of two 2^e per (head, split), chosen from the row's largest magnitude
        // so that it lands in [2^14, 2^15): no overflow for large rows, no
        // subnormals for small ones.  inv >= 0 and rounding is monotonic, so
        // max |o| * inv is exactly max |o * inv|.
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            float amax = 0.f;
#pragma unroll
            for (int u = 0; u < NU; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(o[t][u][i]));
            amax = max_rows4(amax);
            if (g == 0) red[wid * HWG + 16 * t + li] = amax;
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            const int hl = 16 * t + li;
            const int h = hbase + hl;
            float amax = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) amax = fmaxf(amax, red[w * HWG + hl]);
            amax *= inv[t];
            int ex = 15;  // amax = f 2^ex, f in [0.5, 1); zero or non-finite rows: e = 0
            if (amax > 0.f && amax < INFINITY) (void)frexpf(amax, &ex);
            const int e = ex - 15 > -100 ? ex - 15 : -100;
            const float down = ldexpf(inv[t], -e);
            LDS_AS uint8_t *Rrow = stage_out + hl * (D * 2);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int col = wid * DW + 16 * u + 4 * g;
                const int pk = (col >> 2) ^ stage_swz(hl);
                const u32x2_t w = {pack2_f16(o[t][u][0] * down, o[t][u][1] * down),
                                   pack2_f16(o[t][u][2] * down, o[t][u][3] * down)};
                *(LDS_AS u32x2_t *)(Rrow + pk * 8) = w;
            }
            if (wid == 0 && g == 0 && h < p.H) {
                const int64_t slot = ((int64_t)qi * p.S + s) * p.H + h;
                p.ws_x[slot] = ldexpf(1.f, e);
                p.ws_m[slot] = mh[hl];
                p.ws_l[slot] = lh[hl];
            }
        }
    }
    __syncthreads();
    // every LDS read first, then every store (one LDS round trip in all).
    // The stores are non-temporal: outputs and split partials are written
    // once and read once, by a later kernel, so they bypass the caches'
    // allocation (partials: ~9% off the decode main kernel).
    uint16_t *dst = p.S == 1 ? p.out + (int64_t)qi * p.H * D
                             : p.ws_o + ((int64_t)qi * p.S + s) * p.H * D;
    constexpr int NIT = HWG * C16 / NT;
    static_assert(HWG * C16 % NT == 0, "whole rows per pass");
    u32x4_t v[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i = it * NT + tid;
        v[it] = *(const LDS_AS u32x4_t *)(stage_out + (i / C16) * (D * 2) + (i % C16) * 16);
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
        const int i = it * NT + tid;
        const int r = i / C16, pos = i % C16;
        // slot pos holds pieces 2 pos and 2 pos + 1, i.e. pieces (2 pos) ^ z and
        // (2 pos + 1) ^ z of the row (z = stage_swz(r)): chunk pos ^ (z >> 1),
        // its halves swapped when z is odd
        const int z = stage_swz(r);
        const u32x4_t val = (z & 1) ? u32x4_t{v[it][2], v[it][3], v[it][0], v[it][1]} : v[it];
        if (hbase + r < p.H)
            __builtin_nontemporal_store(val, (u32x4_t *)(dst + (int64_t)(hbase + r) * D + ((pos ^ (z >> 1)) << 3)));
    }
}

// OCP E4M3 (the scale format of the pages' compressed cache): sign, 4-bit
// exponent with bias 7, 3-bit mantissa; exponent 0 is subnormal (m * 2^-9);
// the all-ones code is NaN.  Exact in float32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * (1.f / 512.f);
    if (e == 15u && m == 7u) mag = __uint_as_float(0x7FC00000u);
    return (b & 0x80u) ? -mag : mag;
}

// f2: rows of the second source packed as the pages' cache quantises them
// (DeepSeek-V4.1 pages, "blocks, re-index groups" page, compressor excerpt:
// groups of 16 elements, E2M1 codes with one E4M3 scale per group).  A record
// holds D/2 bytes of codes (byte k: element 2k in the low nibble, 2k + 1 in
// the high one) and then D/16 scale bytes, padded to `rec` bytes.  Each
// record lands by LDS-DMA in its padded ring row (RS bytes): in the last `rec`
// bytes of an even row, in the first `rec` bytes of an odd one, so that the
// records of rows 2i and 2i + 1 are adjacent and one DMA instruction fetches
// both.  Each wave rewrites the ring rows it requested itself (rows
// wid*IPW .. wid*IPW + IPW - 1 of the chunk) in place as bf16 once its own
// requests have landed (element i = E2M1(code i) * E4M3(scale i/16), exact in
// bf16: 2 and 4 significant bits): no other wave writes those rows, so the
// wave reads every record of its rows into registers before it writes any
// bf16 row (a bf16 row covers its record), and the chunk's barrier publishes
// them; the expansion needs no barrier of its own.  Rows whose list entry is
// below W hold bf16 already.
template <int D, int IPW>
__device__ __forceinline__ void expand_fp4_own(LDS_AS uint8_t *T, int RS, int rec, const int32_t *list,
                                               int e0, int hi, int64_t W) {
    constexpr int G = D / 16;  // groups (and scale bytes) per row
    constexpr int ITEMS = IPW * G;
    constexpr int PER = (ITEMS + 63) / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    u32x2_t codes[PER];
    uint32_t sc[PER];
    bool on[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int i = k * 64 + lane;
        const int r = wid * IPW + i / G, g = i % G;
        const int e = e0 + r;
        on[k] = i < ITEMS && list[e < hi ? e : e0] >= W;
        codes[k] = u32x2_t{0u, 0u};
        sc[k] = 0u;
        if (on[k]) {
            const LDS_AS uint8_t *src = T + r * RS + ((r & 1) ? 0 : RS - rec);
            codes[k] = *(const LDS_AS u32x2_t *)(src + 8 * g);
            sc[k] = src[D / 2 + g];
        }
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        if (on[k]) {
            const int i = k * 64 + lane;
            const int r = wid * IPW + i / G, g = i % G;
            const float s = e4m3_to_f32(sc[k]);
            const uint32_t c0 = codes[k][0], c1 = codes[k][1];
            const f32x2_t f[8] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, 1.0f, 0),
                                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, 1.0f, 1),
                                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, 1.0f, 2),
                                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c0, 1.0f, 3),
                                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, 1.0f, 0),
                                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, 1.0f, 1),
                                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, 1.0f, 2),
                                  __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c1, 1.0f, 3)};
            uint32_t w[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = pack2_bf16(f[j][0] * s, f[j][1] * s);
            LDS_AS uint8_t *dst = T + r * RS + 32 * g;
            *(LDS_AS u32x4_t *)dst = u32x4_t{w[0], w[1], w[2], w[3]};
            *(LDS_AS u32x4_t *)(dst + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
        }
    }
}

// Work split: a workgroup holds NHQ groups of 16*HT heads; each group is
// served by a pair of waves, one per half of the head dimension.  For QK^T a
// wave sums over its half of d and the pair adds the two partial scores
// through LDS, so both waves of the pair hold the same scores and run the same
// softmax; one of them publishes the bf16 weights (and the rescale factor of
// the running max) in LDS.  For PV every wave takes D/NW output columns of all
// the workgroup's heads, so each V operand read from LDS (a transpose read,
// the slowest LDS access) feeds one MFMA per head tile of the workgroup and
// every row of V is read from LDS once per chunk.  The PV of chunk c runs
// after the barrier that opens chunk c + 1, so publishing the weights needs no
// barrier of its own.  A pair holds HT tiles of 16 heads for QK^T: every K
// operand it reads feeds HT MFMAs.
template <int D, int NHQ, int HT, bool FP4>
__global__ __launch_bounds__(NHQ * 128) void attn_fwd_kernel(FwdParams p) {
    constexpr int NW = 2 * NHQ;            // waves per workgroup
    constexpr int NT = NW * 64;
    constexpr int HW = 16 * HT;            // heads per wave pair (QK^T, softmax)
    constexpr int HWG = NHQ * HW;          // heads per workgroup
    constexpr int NTL = HWG / 16;          // head tiles per workgroup (PV)
    constexpr int ROWB = D * 2;            // bytes per row
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    // Ring rows are padded to RS bytes: with RS = 2D + 32 the 16-byte slot of
    // row r, chunk c is (r (D/8 + 2) + c) mod 32, and 2(D/8 + 2) mod 32 keeps
    // rows apart, so the QK^T operand loads (16 rows x two chunk parities per
    // half-wave) and the PV transpose loads (16 rows x 4 eight-byte words per
    // wave) are free of bank conflicts with affine addresses (immediate
    // offsets, no per-load address arithmetic).
    constexpr int RS = ROWB + 32;          // LDS bytes per ring row
    constexpr int IPW = KC / NW;           // DMA wave instructions (one row each) per wave
    constexpr int DSH = D / 64;            // MFMA k-steps over one half of d
    constexpr int DW = D / NW;             // output columns per wave (PV)
    constexpr int NU = DW / 16;            // 16-wide output tiles per wave
    // LDS ring depth (chunks): up to 4, as long as the DMA instructions of the
    // chunks in flight fit the 6-bit vmcnt
    constexpr int NBUF = 2 + (63 / IPW >= 2 ? 2 : 63 / IPW);
    static_assert(CPR >= 16 && 64 % CPR == 0, "row swizzle needs D in {128, 256, 512}");
    static_assert(KC % NW == 0, "DMA instructions must split evenly over the waves");
    static_assert(HT == 1 || HT == 2, "one or two head tiles per wave");
    static_assert(NU >= 1 && DW % 16 == 0, "whole 16-column tiles per wave");

    __shared__ __attribute__((aligned(16))) uint8_t tile[NBUF][KC * RS];
    __shared__ __attribute__((aligned(16))) f32x4_t xbuf[NW][2 * HT][64];  // partial scores
    // bf16 weights per head tile and row tile (each wave writes 8 contiguous
    // bytes per lane: free of bank conflicts)
    __shared__ __attribute__((aligned(16))) u32x2_t pbuf[NTL][2][64];
    __shared__ float abuf[NTL][16];                                        // rescale factors
    __shared__ int32_t cnt[NW];
    extern __shared__ int32_t list[];  // the compacted list (K entries, dynamic)
    static_assert(sizeof(xbuf) >= (2 + NW) * HWG * sizeof(float), "epilogue state fits in xbuf");
    static_assert(NBUF == fwd_ring_slots(NHQ) &&
                  sizeof(tile) + sizeof(xbuf) + sizeof(pbuf) + sizeof(abuf) + sizeof(cnt) ==
                      fwd_static_lds(D, NHQ, HT),
                  "the host's LDS figure matches the declarations");

    const int bid = blockIdx.x;
    const int unit = unit_of(bid, p.units, p.bs, p.dv_bs);
    if (unit < 0) return;
    // workgroup- and wave-uniform values, in scalar registers
    const int us = udiv(unit, p.dv_S);
    const int s = unit - us * p.S;
    const int qi = udiv(us, p.dv_HG);
    const int hg = us - qi * p.HG;
    const int b = udiv(qi, p.dv_T);

    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hq = wid >> 1;      // head group of this wave
    const int dh = wid & 1;       // half of d this wave covers
    const int g = lane >> 4;      // 16-lane block of the wave
    const int li = lane & 15;

    // head of this lane in head tile t: hw0 + 16 t + li
    const int hw0 = hg * HWG + hq * HW;
    // row j of this sequence lives at (j < W ? kva : kvb2) + j * D, or is the
    // FP4 record at recb + j * rec2
    const uint16_t *kva = p.kv + (int64_t)b * p.rows_a * D;
    const uint16_t *kvb2 = p.kv2 + ((int64_t)b * p.rows_b - p.W) * D;
    const uint8_t *recb = (const uint8_t *)p.kv2 + ((int64_t)b * p.rows_b - p.W) * p.rec2;
    static_assert(NBUF == 4, "the prologue stages the list in slot 3");

    // Prologue.  Per wave, in issue order: its share of the raw list (LDS-DMA,
    // 4 bytes per lane, into slot 3), its q (ordinary loads straight into the
    // MFMA B operands: a compute unit issues LDS-DMA at a limited rate, and q
    // would queue 64 KB ahead of the first rows), then chunk 0 as soon as the
    // list has landed.
    LDS_AS int32_t *raw = (LDS_AS int32_t *)&tile[3][0];
    {
        const int32_t *lst = p.idxs + (int64_t)qi * p.K;
        const int NI = (p.K + 63) / 64;
        for (int i = wid; i < NI; i += NW) {
            const int k = i * 64 + lane;
            if (k < p.K) lds_dma4(lst + k, raw + i * 64);
        }
    }
    // a3: qf[t][k] = q[hw0 + 16t + li, dh*D/2 + 32k + 8g .. +7]; heads beyond
    // H read head 0 (in bounds) and are zeroed once q has landed
    bf16x8_t qf[HT][DSH];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
        const int h = hw0 + 16 * t + li;
        const uint16_t *qrow = p.q + ((int64_t)qi * p.H + (h < p.H ? h : 0)) * D + dh * (D / 2) + 8 * g;
#pragma unroll
        for (int k = 0; k < DSH; ++k) qf[t][k] = *(const bf16x8_t *)(qrow + 32 * k);
    }
    // the raw list of this wave has landed once only its q loads are pending
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(HT * DSH) : "memory");
    __syncthreads();

    // a2: the wave's k-th row of chunk c into ring slot c % NBUF with LDS-DMA.
    // A wave takes IPW consecutive entries of the chunk (its k-th is entry
    // wid*IPW + k, at that position of the slot), so that four of its rows
    // sit within reach of one instruction's offset.  Each wave instruction
    // moves one bf16 row: lane l < D/8 fetches its 16 bytes and lands at byte
    // 16*l of the row's padded slot.  FP4 build, rows >= W: an FP4 record
    // (rec2/16 lanes) lands at the tail of an even row and at the head of an
    // odd one, so a pair of records shares one instruction (see expand_fp4_own).
    // The lambdas return the number of DMA instructions they issued.
    static_assert(IPW % 4 == 0, "rows are requested four at a time");
    // Row numbers and W are below 2^31 (a row holds at least 256 bytes), so
    // the source test is a 32-bit scalar compare and a row's address a scalar
    // base plus the lane's 16-byte offset (saddr form).
    const int Wc = (int)(p.W < 0x7FFFFFFF ? p.W : 0x7FFFFFFF);
    auto row_base = [&](int rw) {
        return (const uint8_t *)((rw < Wc ? kva : kvb2) + (int64_t)rw * D);
    };
    auto dma_row = [&](int c, int k, int rw) {
        LDS_AS uint8_t *dst = (LDS_AS uint8_t *)&tile[c % NBUF][0] + (wid * IPW + k) * RS;
        if (!FP4 || rw < p.W) {
            if (CPR == 64 || lane < CPR) lds_dma16_s_nt(row_base(rw), lane * 16, (LDS_AS void *)dst);
        } else if (lane * 16 < p.rec2) {
            lds_dma16_nt(recb + (int64_t)rw * p.rec2 + lane * 16,
                         (LDS_AS void *)(dst + ((k & 1) ? 0 : RS - p.rec2)));
        }
        return 1;
    };
    // FP4 build: rows k (even) and k + 1; two records in one instruction
    auto dma_pair = [&](int c, int k, int r0, int r1) {
        if (r0 >= p.W && r1 >= p.W) {
            const int nl = p.rec2 / 16;  // lanes per record
            LDS_AS uint8_t *dst = (LDS_AS uint8_t *)&tile[c % NBUF][0] + (wid * IPW + k) * RS + RS - p.rec2;
            const uint8_t *src = lane < nl ? recb + (int64_t)r0 * p.rec2 + lane * 16
                                           : recb + (int64_t)r1 * p.rec2 + (lane - nl) * 16;
            if (lane < 2 * nl) lds_dma16_nt(src, (LDS_AS void *)dst);
            return 1;
        }
        return dma_row(c, k, r0) + dma_row(c, k + 1, r1);
    };
    // the wave's rows k0 .. k0+3 of chunk c (bf16 rows: one M0 write)
    auto dma_quad = [&](int c, int k0, int r0, int r1, int r2, int r3) {
        if constexpr (FP4) {
            return dma_pair(c, k0, r0, r1) + dma_pair(c, k0 + 2, r2, r3);
        } else {
            LDS_AS uint8_t *dst = (LDS_AS uint8_t *)&tile[c % NBUF][0] + (wid * IPW + k0) * RS;
            if (CPR == 64 || lane < CPR)
                lds_dma16x4_s_nt<RS>(row_base(r0), row_base(r1), row_base(r2), row_base(r3), lane * 16, dst);
            return 4;
        }
    };

    // Chunk 0 ahead of the compaction: the rows it holds when every entry is
    // valid (this split's slice K*s/S .. K*(s+1)/S of the raw list) are
    // requested now; once the list is compacted each wave requests again only
    // the rows whose number differs.  A later DMA into the same LDS row lands
    // after the earlier one, and every later wait only lets younger loads
    // remain, so the extra requests need no wait of their own.  Raw entries
    // that are not rows (< 0 or >= N) are never fetched.
    int spec[IPW];
    {
        const int slo = udiv(p.K * s, p.dv_S), shi = udiv(p.K * (s + 1), p.dv_S);  // K <= LIST_CAP
#pragma unroll
        for (int k = 0; k < IPW; ++k) {
            const int e = slo + wid * IPW + k;
            const int v = slo < shi ? raw[e < shi ? e : slo] : -1;
            const int rw = __builtin_amdgcn_readfirstlane(v);
            spec[k] = (uint32_t)rw < (uint32_t)(p.N < 0x80000000LL ? p.N : 0x80000000LL) ? rw : -1;
        }
#pragma unroll
        for (int k = 0; k < IPW; k += 4) {
            if ((spec[k] | spec[k + 1] | spec[k + 2] | spec[k + 3]) >= 0) {
                dma_quad(0, k, spec[k], spec[k + 1], spec[k + 2], spec[k + 3]);
            } else {
#pragma unroll
                for (int j = k; j < k + 4; ++j)
                    if (spec[j] >= 0) dma_row(0, j, spec[j]);
            }
        }
    }

    // a1: decode and compact the list, then take this split's slice.
    const int n = compact_list<NT>(raw, p.K, p.N, list, cnt);
    const int Sq = query_splits(n, p.K, p.S);  // a10
    if (p.S > 1 && s == 0 && hg == 0 && tid == 0) p.ws_plan[qi] = Sq;
    if (s >= Sq) {  // a spare split slot: nothing to do once the early rows have landed
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }
    // n <= LIST_CAP and s < MAX_SPLITS: no overflow; a query with every entry
    // valid uses all S slots, and the host's divisor by S serves
    const int lo = Sq == p.S ? udiv(n * s, p.dv_S) : (n * s) / Sq;
    const int hi = Sq == p.S ? udiv(n * (s + 1), p.dv_S) : (n * (s + 1)) / Sq;
    const int nchunks = (hi - lo + KC - 1) / KC;

    // Tail slots repeat the chunk's first row; their scores are masked to
    // -inf below.  All row numbers are read from the list before the first
    // DMA is issued: the DMA asm orders memory, so interleaving them would put
    // one LDS round trip in front of every DMA.
    auto chunk_rows = [&](int c, int (&row)[IPW]) {
        const int e0 = lo + c * KC;
#pragma unroll
        for (int k = 0; k < IPW; ++k) {
            const int e = e0 + wid * IPW + k;
            // the row number is wave-uniform: scalar branches, one DMA per row
            row[k] = __builtin_amdgcn_readfirstlane(list[e < hi ? e : e0]);
        }
    };
    if (nchunks > 0) {
        int row[IPW];
        chunk_rows(0, row);
#pragma unroll
        for (int k = 0; k < IPW; ++k)
            if (row[k] != spec[k]) dma_row(0, k, row[k]);
    }

    // Chunk 0 and q (and any early request) have landed once nothing is
    // pending; the wait goes through the builtin so that the compiler knows
    // q is in its registers.  Chunks 1 and 2 are requested inside the first
    // QK^T (below).
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
    for (int t = 0; t < HT; ++t) {
        if (hw0 + 16 * t + li >= p.H) {
#pragma unroll
            for (int k = 0; k < DSH; ++k) qf[t][k] = bf16x8_t{};
        }
    }

    // Softmax state of head hw0 + 16t + li (log2 units), identical in both
    // waves of the pair.  The sink is folded in by the epilogue.
    float m[HT], lsum[HT];
#pragma unroll
    for (int t = 0; t < HT; ++t) {
        m[t] = -INFINITY;
        lsum[t] = 0.f;
    }
    // O^T over this wave's output columns for every head tile of the workgroup
    f32x4_t o[NTL][NU];
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int u = 0; u < NU; ++u) o[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // a6: O^T[d, h] += V^T[d, j] P^T[j, h] for this wave's columns, chunk cc,
    // with the weights and rescale factors the pairs published.  A operand
    // through transpose loads: lane i of block g addresses row 4g + i/4 (and
    // +16), columns 16u + 4(i%4) .. +3; the load hands lane i column 16u + i of
    // rows 4g..4g+3, matching the weight slots j = 4g + e and 16 + 4g + e.
    // Each V operand feeds NTL MFMAs (pipelined by hand: transpose pair u + PVP
    // is requested right after the MFMAs of pair u).
    auto pv_chunk = [&](int cc) {
        const LDS_AS uint8_t *T = (const LDS_AS uint8_t *)&tile[cc % NBUF][0];
        // every tile's weights and factor and the first V operands are
        // requested before any is used (one LDS round trip, not one per tile)
        bf16x8_t pb[NTL];
        float al[NTL];
#pragma unroll
        for (int t = 0; t < NTL; ++t) {
            const u32x2_t w0 = pbuf[t][0][lane], w1 = pbuf[t][1][lane];
            pb[t] = __builtin_bit_cast(bf16x8_t, u32x4_t{w0[0], w0[1], w1[0], w1[1]});
            al[t] = abuf[t][li];
        }
        constexpr int PVP = NU < 4 ? NU : 4;
        const int r0 = 4 * g + (li >> 2);
        const LDS_AS uint8_t *R0 = T + r0 * RS + (li & 3) * 8;
        const LDS_AS uint8_t *R1 = R0 + 16 * RS;
        auto vload = [&](int u) {
            const int pos = (wid * NU + u) * 32;
            const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t *)(R0 + pos));
            const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t *)(R1 + pos));
            return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8_t va[PVP];
#pragma unroll
        for (int u = 0; u < PVP; ++u) va[u] = vload(u);
        bool scaled = false;
#pragma unroll
        for (int t = 0; t < NTL; ++t) scaled |= al[t] != 1.f;
        if (__ballot(scaled)) {  // a running max moved (rare): rescale
#pragma unroll
            for (int t = 0; t < NTL; ++t)
#pragma unroll
                for (int u = 0; u < NU; ++u) o[t][u] *= al[t];
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int t = 0; t < NTL; ++t)
                o[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[u % PVP], pb[t], o[t][u], 0, 0, 0);
            if (u + PVP < NU) va[u % PVP] = vload(u + PVP);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    LDS_AS f32x4_t *xmine = (LDS_AS f32x4_t *)&xbuf[wid][0][lane];
    const LDS_AS f32x4_t *xpeer = (const LDS_AS f32x4_t *)&xbuf[wid ^ 1][0][lane];

    // The loop requests chunk c + 2 during chunk c's QK^T (chunks 1 and 2
    // during chunk 0's), a group of four rows between MFMAs: a compute unit
    // issues LDS-DMA at a limited rate, so more chunks in flight only queue
    // up, and a burst of requests would hold the issuing waves back before
    // their MFMAs.  Row numbers are read a chunk ahead (lane k holds the
    // wave's k-th), so requesting one only moves it to an SGPR.
    auto rows_of = [&](int c) {
        const int e0 = lo + c * KC;
        const int e = e0 + wid * IPW + lane % IPW;
        return list[e < hi ? e : e0];
    };
    // the wave's rows 4q .. 4q+3 of chunk cc, from the lanes of `rows`
    auto quad_from = [&](int cc, int q, int rows) {
        return dma_quad(cc, 4 * q, __builtin_amdgcn_readlane(rows, 4 * q),
                        __builtin_amdgcn_readlane(rows, 4 * q + 1),
                        __builtin_amdgcn_readlane(rows, 4 * q + 2),
                        __builtin_amdgcn_readlane(rows, 4 * q + 3));
    };
    int next_rows = 1 < nchunks ? rows_of(1) : 0;   // the chunk requested next
    int next2_rows = 2 < nchunks ? rows_of(2) : 0;  // chunk 2, during chunk 0
    // DMA instructions this wave issued for the chunk after the current one
    // (FP4 build: pairs of records share one, so the count varies)
    int issued_ahead = 0;
    for (int c = 0; c < nchunks; ++c) {
        // chunk c has landed once at most the chunk after it is pending
        if constexpr (FP4) {
            wait_vm_upto<IPW>(c + 1 < nchunks ? issued_ahead : 0);
            // this wave's FP4 records of chunk c have landed: expand them
            expand_fp4_own<D, IPW>((LDS_AS uint8_t *)&tile[c % NBUF][0], RS, p.rec2, list,
                                   lo + c * KC, hi, p.W);
        } else {
            wait_vm_ahead<IPW, 1>(min(1, nchunks - 1 - c));
        }
        __syncthreads();
        // PV of chunk c - 1 (its weights were published before this barrier)
        if (c > 0) pv_chunk(c - 1);
        // chunk c + 2 goes into slot (c + 2) % NBUF, last read by the PV of
        // chunk c - 2, which every wave finished before the barrier above
        const int rq = c == 0 ? 1 : c + 2;  // first chunk requested in this QK^T
        const bool do_stage = rq < nchunks;
        const bool two = c == 0 && 2 < nchunks;  // chunk 2 as well

        const LDS_AS uint8_t *T = (const LDS_AS uint8_t *)&tile[c % NBUF][0];
        const int cnt_c = min(KC, hi - (lo + c * KC));

        // a4: partial S^T[j, h] over this wave's half of d (two 16-row tiles
        // x HT head tiles; each K operand feeds HT MFMAs).  Software-pipelined
        // by hand: operand i + QKP is requested right after the MFMAs of
        // operand i, and the scheduling barriers keep that order (left alone,
        // the scheduler requests each operand next to its MFMA and the LDS
        // latency is exposed on every one).
        int issued_now = 0;  // DMA instructions of the last chunk requested below
        f32x4_t sacc[2][HT];
#pragma unroll
        for (int jt = 0; jt < 2; ++jt)
#pragma unroll
            for (int t = 0; t < HT; ++t) sacc[jt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        {
            constexpr int QKP = 4, NQK = 2 * DSH;
            auto kload = [&](int i) {  // operand i: k-step i/2, row tile i%2
                const int r = (i & 1) * 16 + li;
                const int pos = 4 * (dh * DSH + (i >> 1)) + g;
                return __builtin_bit_cast(bf16x8_t, *(const LDS_AS u32x4_t *)(T + r * RS + pos * 16));
            };
            bf16x8_t ka[QKP];
#pragma unroll
            for (int i = 0; i < QKP; ++i) ka[i] = kload(i);
#pragma unroll
            for (int i = 0; i < NQK; ++i) {
#pragma unroll
                for (int t = 0; t < HT; ++t)
                    sacc[i & 1][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i % QKP], qf[t][i >> 1],
                                                                             sacc[i & 1][t], 0, 0, 0);
                if (i + QKP < NQK) ka[i % QKP] = kload(i + QKP);
                // groups of four rows, spread evenly (dma_step)
                if (two) {  // chunk 1's groups, then chunk 2's
                    constexpr int NG = 2 * IPW / 4;
#pragma unroll
                    for (int q = 0; q < NG; ++q)
                        if (i == dma_step(q, NG, NQK)) {
                            if (q < NG / 2) quad_from(1, q, next_rows);
                            else issued_now += quad_from(2, q - NG / 2, next2_rows);
                        }
                } else if (do_stage) {
                    constexpr int NG = IPW / 4;
#pragma unroll
                    for (int q = 0; q < NG; ++q)
                        if (i == dma_step(q, NG, NQK)) issued_now += quad_from(rq, q, next_rows);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (two || do_stage) issued_ahead = issued_now;
        if (c + 3 < nchunks) next_rows = rows_of(c + 3);
        // the pair adds its two halves (a + b == b + a, so both waves agree)
#pragma unroll
        for (int t = 0; t < HT; ++t) {
            xmine[(2 * t) * 64] = sacc[0][t];
            xmine[(2 * t + 1) * 64] = sacc[1][t];
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < HT; ++t) {
            sacc[0][t] += xpeer[(2 * t) * 64];
            sacc[1][t] += xpeer[(2 * t + 1) * 64];
        }

        // a5: mask + online softmax.  Lane (li, g) holds rows j = 16 jt + 4 g + i
        // of head tile t.  The kept max m only moves when a score beats it by
        // more than MAX_SLACK; a per-lane check and one ballot decide that, and
        // the exact chunk max (two cross-lane reductions) is only taken then.
        // Both waves of the pair hold the same scores and take the same max
        // decision; each then forms the bf16 weights of one row tile (wave dh:
        // rows 16 dh + 4 g + i) and publishes them as that row tile's
        // weights, so lsum holds the wave's row tile only (the epilogue adds
        // the pair's two).  Wave dh == 0 publishes the factor that
        // rescales the accumulators (1 when the max stayed).
#pragma unroll
        for (int t = 0; t < HT; ++t) {
            // (scaled in place and masked in place in the list's last chunk,
            // so that both cases share registers; the max is only formed when
            // some score beats the kept one by more than MAX_SLACK)
            float sv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) sv[e] = sacc[e >> 2][t][e & 3] * p.qk_scale_log2;
            if (cnt_c != KC) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (16 * (e >> 2) + 4 * g + (e & 3) >= cnt_c) sv[e] = -INFINITY;
            }
            const float th = m[t] + MAX_SLACK;
            bool over = false;
#pragma unroll
            for (int e = 0; e < 8; ++e) over |= sv[e] > th;
            float alpha = 1.f;
            if (__ballot(over)) {
                const float lmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                                         fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
                const float cmax = max_rows4(lmax);
                const bool raise = cmax > th;
                const float mnew = raise ? cmax : m[t];
                alpha = exp2_fast(m[t] - mnew);
                lsum[t] *= alpha;
                m[t] = mnew;
            }
            // The weights enter the value product as bf16; the denominator sums
            // the same rounded weights, so numerator and denominator agree.
            float own[4];  // this wave's row tile (separate copies: a select, not an index)
            if (dh) {
                own[0] = sv[4], own[1] = sv[5], own[2] = sv[6], own[3] = sv[7];
            } else {
                own[0] = sv[0], own[1] = sv[1], own[2] = sv[2], own[3] = sv[3];
            }
            float pv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) pv[e] = exp2_fast(own[e] - m[t]);
            const u32x2_t pw = {pack2_bf16(pv[0], pv[1]), pack2_bf16(pv[2], pv[3])};
            lsum[t] = add_bf16_pair(pw[1], add_bf16_pair(pw[0], lsum[t]));
            pbuf[hq * HT + t][dh][lane] = pw;
            if (dh == 0 && g == 0) abuf[hq * HT + t][li] = alpha;
        }
    }

    // a7 / a8: epilogue.  The last chunk's PV, then each pair publishes the
    // running max and total denominator of its heads for every wave (the
    // second wave's half of the denominator passes through red, free until
    // store_outputs).
    static_assert(HWG * D * 2 <= NBUF * KC * RS, "output staging fits in the ring");
    __syncthreads();
    if (nchunks > 0) pv_chunk(nchunks - 1);
    LDS_AS float *mh = (LDS_AS float *)&xbuf[0][0][0];
    LDS_AS float *lh = mh + HWG;
    LDS_AS float *red = lh + HWG;
#pragma unroll
    for (int t = 0; t < HT; ++t) {
        const float ltot = sum_rows4(lsum[t]);
        if (g == 0) {
            if (dh == 0) {
                mh[hq * HW + 16 * t + li] = m[t];
                lh[hq * HW + 16 * t + li] = ltot;
            } else {
                red[hq * HW + 16 * t + li] = ltot;
            }
        }
    }
    __syncthreads();  // every wave is done with the ring; reuse it for staging
    if (tid < HWG) lh[tid] += red[tid];
    __syncthreads();
    store_outputs<D, NW, NTL>(p, o, mh, lh, red, qi, s, hg, (LDS_AS uint8_t *)&tile[0][0]);
}

// Many-query variant, for launches with at least two workgroups per compute
// unit (prefill), where MFMA throughput rather than gather depth decides.
// Same steps and results as attn_fwd_kernel; the work is split differently:
//   * for QK^T and the softmax each wave takes one tile of 16 heads over the
//     whole of d (no partial scores to add up); the waves then publish their
//     bf16 weights (and rescale factors) in LDS, and for PV each wave takes
//     D/NW output columns of every head of the workgroup, so every V operand
//     read from LDS (a transpose read, the slowest LDS access) feeds one MFMA
//     per head tile and each row of V is read from LDS once per chunk;
//   * a 2-chunk ring of 32 padded rows, the weight exchange and the list
//     (compacted in place, sized by K in dynamic LDS) take about 75 KB of
//     LDS, so two workgroups share a compute unit and one's softmax,
//     barriers, prologue and epilogue overlap the other's MFMAs.
template <int D, int NHQ, bool FP4>
__global__ __launch_bounds__(NHQ * 128, 2) void attn_fwd_mq_kernel(FwdParams p) {
    constexpr int HT = 2;                  // head tiles per pair
    constexpr int NW = 2 * NHQ;            // waves per workgroup
    constexpr int NT = NW * 64;
    constexpr int HP = 16 * HT;            // heads per pair
    constexpr int ROWB = D * 2;
    constexpr int RS = ROWB + 32;          // padded ring row (see attn_fwd_kernel)
    constexpr int CPR = D / 8;
    constexpr int NB = 2;                  // ring chunks
    constexpr int IPW = KC / NW;           // DMA instructions (one row each) per wave per chunk
    constexpr int DS = D / 32;             // MFMA k-steps over d
    constexpr int NTL = NW;                // head tiles per workgroup (wave w owns tile w)
    constexpr int HWG = 16 * NTL;
    constexpr int DW = D / NW;             // output columns per wave (PV)
    constexpr int NU = DW / 16;            // 16-wide output tiles per wave
    static_assert(KC % NW == 0 && IPW <= 63, "ring shape");
    static_assert(NHQ * HP * D * 2 <= NB * KC * RS, "output staging fits in the ring");

    __shared__ __attribute__((aligned(16))) uint8_t tile[NB][KC * RS];
    __shared__ __attribute__((aligned(16))) u32x4_t xp[NW][64];  // bf16 weights of the tiles
    __shared__ float xa[NW][16];                                  // rescale factors
    __shared__ int32_t cnt[NW];
    extern __shared__ int32_t list[];  // K entries: raw, then compacted in place

    const int bid = blockIdx.x;
    const int unit = unit_of(bid, p.units, p.bs, p.dv_bs);
    if (unit < 0) return;
    // workgroup-uniform values in scalar registers, so the row and record
    // base addresses below are scalar too
    const int us = udiv(unit, p.dv_S);
    const int s = unit - us * p.S;
    const int qi = udiv(us, p.dv_HG);
    const int hg = us - qi * p.HG;
    const int b = udiv(qi, p.dv_T);

    // the wave number is uniform: in a scalar register, so are the offsets it sets
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hq = wid >> 1;      // pair
    const int w = wid & 1;        // own head tile (QK^T, softmax) and half of d (PV)
    const int g = lane >> 4, li = lane & 15;
    const int hown = hg * (NHQ * HP) + hq * HP + 16 * w + li;  // head of this lane's scores
    const uint16_t *kva = p.kv + (int64_t)b * p.rows_a * D;          // rows j < W
    const uint16_t *kvb2 = p.kv2 + ((int64_t)b * p.rows_b - p.W) * D;  // rows j >= W
    const uint8_t *recb = (const uint8_t *)p.kv2 + ((int64_t)b * p.rows_b - p.W) * p.rec2;

    // Prologue: the raw list into `list` by LDS-DMA.
    {
        const int32_t *lst = p.idxs + (int64_t)qi * p.K;
        const int NI = (p.K + 63) / 64;
        for (int i = wid; i < NI; i += NW) {
            const int k = i * 64 + lane;
            if (k < p.K) lds_dma4(lst + k, (LDS_AS int32_t *)list + i * 64);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    // a1: decode and compact the list (in place), then take this split's slice.
    const int n = compact_list<NT>((const LDS_AS int32_t *)list, p.K, p.N, list, cnt);
    const int Sq = query_splits(n, p.K, p.S);  // a10
    if (p.S > 1 && s == 0 && hg == 0 && tid == 0) p.ws_plan[qi] = Sq;
    if (s >= Sq) return;  // a spare split slot
    // n <= LIST_CAP and s < MAX_SPLITS: no overflow; a query with every entry
    // valid uses all S slots, and the host's divisor by S serves
    const int lo = Sq == p.S ? udiv(n * s, p.dv_S) : (n * s) / Sq;
    const int hi = Sq == p.S ? udiv(n * (s + 1), p.dv_S) : (n * (s + 1)) / Sq;
    const int nchunks = (hi - lo + KC - 1) / KC;

    // a2: chunk c (KC rows) into ring slot c % NB, one row per DMA
    // instruction; the wave's k-th is entry wid*IPW + k, at that position of
    // the slot, so four of its rows sit within reach of one instruction's
    // offset.  Tail slots repeat the chunk's first row (masked below).
    // rows_of reads the chunk's row numbers one chunk ahead (lane k holds the
    // k-th), so a stage only moves them to SGPRs and issues the DMAs.
    static_assert(IPW % 4 == 0, "rows are requested four at a time");
    auto rows_of = [&](int c) {
        const int e0 = lo + c * KC;
        int ln = lane;  // formed here, not held across the loop (see stage_pair)
        asm volatile("" : "+v"(ln));
        const int e = e0 + wid * IPW + ln % IPW;
        return list[e < hi ? e : e0];
    };
    // Row numbers and W are below 2^31 (a row holds at least 256 bytes), so
    // the source test is a 32-bit scalar compare.
    const int Wc = (int)(p.W < 0x7FFFFFFF ? p.W : 0x7FFFFFFF);
    // this wave's k-th row of chunk c: a bf16 row, or (FP4 build, rows >= W)
    // a record landing at the tail of the row's slot
    auto stage_one = [&](int c, int rows, int k) {
        const int row = __builtin_amdgcn_readlane(rows, k);
        LDS_AS uint8_t *dst = (LDS_AS uint8_t *)&tile[c % NB][0] + (wid * IPW + k) * RS;
        if (!FP4 || row < Wc) {
            const uint16_t *src = (row < Wc ? kva : kvb2) + (int64_t)row * D;
            if (CPR == 64 || lane < CPR) lds_dma16_s(src, lane * 16, dst);
        } else if (lane * 16 < p.rec2) {
            // an FP4 record: at the tail of an even row, the head of an odd one
            lds_dma16_s(recb + (int64_t)row * p.rec2, lane * 16, dst + ((k & 1) ? 0 : RS - p.rec2));
        }
    };
    // FP4 build: rows k (even) and k + 1; two records share one instruction,
    // addressed from the lower record (a scalar base) plus a 32-bit lane
    // offset, so that no per-lane 64-bit address stays live across the loop
    auto stage_pair = [&](int c, int rows, int k) {
        const int r0 = __builtin_amdgcn_readlane(rows, k), r1 = __builtin_amdgcn_readlane(rows, k + 1);
        const int rlo = r0 < r1 ? r0 : r1;
        const int64_t span = (int64_t)(r0 < r1 ? r1 - r0 : r0 - r1) * p.rec2;
        if (r0 >= Wc && r1 >= Wc && span < 0x7FFFFFFF - 1024) {
            const int nl = p.rec2 / 16;  // lanes per record
            LDS_AS uint8_t *dst = (LDS_AS uint8_t *)&tile[c % NB][0] + (wid * IPW + k) * RS + RS - p.rec2;
            // the lane's offset is formed here, not hoisted out of the chunk
            // loop (a register held across the loop spilled, and each reload
            // waited for every row request in flight)
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const uint32_t voff = ln < nl ? (uint32_t)((r0 - rlo) * p.rec2 + ln * 16)
                                          : (uint32_t)((r1 - rlo) * p.rec2 + (ln - nl) * 16);
            if (ln < 2 * nl) lds_dma16_s(recb + (int64_t)rlo * p.rec2, voff, (LDS_AS void *)dst);
        } else {
            stage_one(c, rows, k);
            stage_one(c, rows, k + 1);
        }
    };
    // rows 4q .. 4q+3 (bf16 rows: one M0 write)
    auto stage_quad = [&](int c, int rows, int q) {
        if constexpr (FP4) {
            stage_pair(c, rows, 4 * q);
            stage_pair(c, rows, 4 * q + 2);
        } else {
            auto src = [&](int k) {
                const int row = __builtin_amdgcn_readlane(rows, k);
                return (const uint8_t *)((row < Wc ? kva : kvb2) + (int64_t)row * D);
            };
            LDS_AS uint8_t *dst = (LDS_AS uint8_t *)&tile[c % NB][0] + (wid * IPW + 4 * q) * RS;
            if (CPR == 64 || lane < CPR)
                lds_dma16x4_s<RS>(src(4 * q), src(4 * q + 1), src(4 * q + 2), src(4 * q + 3), lane * 16, dst);
        }
    };
    auto stage = [&](int c, int rows) {
#pragma unroll
        for (int q = 0; q < IPW / 4; ++q) stage_quad(c, rows, q);
    };
    int next_rows = 0;
    if (nchunks > 0) stage(0, rows_of(0));
    if (nchunks > 1) next_rows = rows_of(1);

    // a3: qf[k] = q[hown, 32k + 8g .. +7], the B operands over the whole of
    // d, loaded straight into registers while chunk 0 is in flight.  Heads
    // beyond H read head 0: their scores, weights and accumulators only feed
    // their own output rows, which are never stored.  The first wait of the
    // loop (for chunk 0) covers these loads too.
    bf16x8_t qf[DS];
    {
        const uint16_t *qrow = p.q + ((int64_t)qi * p.H + (hown < p.H ? hown : 0)) * D + 8 * g;
#pragma unroll
        for (int k = 0; k < DS; ++k) qf[k] = *(const bf16x8_t *)(qrow + 32 * k);
    }

    float m = -INFINITY, lsum = 0.f;  // softmax state of head hown (log2 units)
    f32x4_t o[NTL][NU];               // O^T of every head tile over this wave's columns
#pragma unroll
    for (int t = 0; t < NTL; ++t)
#pragma unroll
        for (int u = 0; u < NU; ++u) o[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int c = 0; c < nchunks; ++c) {
        // chunk c has landed once at most the chunk after it is pending
        // Chunk c (and, before the first chunk, q) is the only load in flight.
        // The wait goes through the builtin so the compiler knows q has
        // landed; otherwise it would wait for q's loads inside the MFMA
        // sequence, which also drains the next chunk's DMAs issued there.
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        // FP4 build: this wave's records of chunk c have landed; expand them
        if (FP4) expand_fp4_own<D, IPW>((LDS_AS uint8_t *)&tile[c % NB][0], RS, p.rec2, list, lo + c * KC,
                                        hi, p.W);
        __syncthreads();
        // chunk c + 1 goes into the slot chunk c - 1 left; its DMAs are spread
        // through the QK^T MFMAs below, so that a wave never waits for a burst
        // of them to be accepted
        const bool do_stage = c + 1 < nchunks;

        const LDS_AS uint8_t *T = (const LDS_AS uint8_t *)&tile[c % NB][0];
        const int cnt_c = min(KC, hi - (lo + c * KC));

        // a4: S^T[j, hown] over the whole of d, rows j = 16 jt + 4 g + i.
        // Software-pipelined by hand: operand load i + QKP is issued right
        // after MFMA i, and the scheduling barriers keep that order (left
        // alone, the scheduler issues each load next to its MFMA and the LDS
        // latency is exposed on every one).
        f32x4_t sacc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
        {
            constexpr int QKP = 4, NQK = 2 * DS;
            auto kload = [&](int i) {  // operand i: k-step i/2, row tile i%2
                return __builtin_bit_cast(bf16x8_t, *(const LDS_AS u32x4_t *)(
                    T + ((i & 1) * 16 + li) * RS + (4 * (i >> 1) + g) * 16));
            };
            bf16x8_t ka[QKP];
#pragma unroll
            for (int i = 0; i < QKP; ++i) ka[i] = kload(i);
#pragma unroll
            for (int i = 0; i < NQK; ++i) {
                sacc[i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i % QKP], qf[i >> 1],
                                                                      sacc[i & 1], 0, 0, 0);
                if (i + QKP < NQK) ka[i % QKP] = kload(i + QKP);
                if (do_stage) {  // groups of four rows, spread evenly (dma_step)
                    constexpr int NG = IPW / 4;
#pragma unroll
                    for (int q = 0; q < NG; ++q)
                        if (i == dma_step(q, NG, NQK)) stage_quad(c + 1, next_rows, q);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if (do_stage && c + 2 < nchunks) next_rows = rows_of(c + 2);

        // a5: online softmax of the own tile (lazy max, as in attn_fwd_kernel:
        // scaled and tail-masked in place, the max formed only when needed)
        float sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = sacc[e >> 2][e & 3] * p.qk_scale_log2;
        if (cnt_c != KC) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (16 * (e >> 2) + 4 * g + (e & 3) >= cnt_c) sv[e] = -INFINITY;
        }
        const float th = m + MAX_SLACK;
        bool over = false;
#pragma unroll
        for (int e = 0; e < 8; ++e) over |= sv[e] > th;
        float alpha = 1.f;
        if (__ballot(over)) {
            const float lmax = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
            const float cmax = max_rows4(lmax);
            const float mnew = cmax > th ? cmax : m;
            alpha = exp2_fast(m - mnew);
            lsum *= alpha;
            m = mnew;
        }
        const u32x4_t pw = {pack2_bf16(exp2_fast(sv[0] - m), exp2_fast(sv[1] - m)),
                            pack2_bf16(exp2_fast(sv[2] - m), exp2_fast(sv[3] - m)),
                            pack2_bf16(exp2_fast(sv[4] - m), exp2_fast(sv[5] - m)),
                            pack2_bf16(exp2_fast(sv[6] - m), exp2_fast(sv[7] - m))};
#pragma unroll
        for (int e = 0; e < 4; ++e) lsum = add_bf16_pair(pw[e], lsum);

        // every wave publishes its tile's weights and rescale factor
        xp[wid][lane] = pw;
        if (g == 0) xa[wid][li] = alpha;
        __syncthreads();

        // a6: O^T[d, h] += V^T[d, j] P^T[j, h] over this wave's columns; the
        // transpose loads hand lane (li, g) column 16u + li of rows 4g..4g+3
        // and 16+4g..16+4g+3, the k-slots of its weights
        // (pipelined by hand like QK^T: transpose pair u + PVP is loaded right
        // after the MFMAs of pair u).  Every tile's weights and factor and the
        // first V operands are requested before any is used, so the LDS
        // latency is paid once (a branch on each factor as it arrives would
        // serialise the round trips).
        {
            constexpr int PVP = NU < 3 ? NU : 3;
            bf16x8_t pb[NTL];
            float al[NTL];
#pragma unroll
            for (int t = 0; t < NTL; ++t) {
                pb[t] = __builtin_bit_cast(bf16x8_t, xp[t][lane]);
                al[t] = xa[t][li];
            }
            const LDS_AS uint8_t *R0 = T + (4 * g + (li >> 2)) * RS + (li & 3) * 8;
            const LDS_AS uint8_t *R1 = R0 + 16 * RS;
            auto vload = [&](int u) {
                const int off = (wid * NU + u) * 32;
                const bf16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t *)(R0 + off));
                const bf16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LDS_AS bf16x4_t *)(R1 + off));
                return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            };
            bf16x8_t va[PVP];
#pragma unroll
            for (int u = 0; u < PVP; ++u) va[u] = vload(u);
            bool scaled = false;
#pragma unroll
            for (int t = 0; t < NTL; ++t) scaled |= al[t] != 1.f;
            if (__ballot(scaled)) {  // a running max moved (rare): rescale
#pragma unroll
                for (int t = 0; t < NTL; ++t)
#pragma unroll
                    for (int u = 0; u < NU; ++u) o[t][u] *= al[t];
            }
#pragma unroll
            for (int u = 0; u < NU; ++u) {
#pragma unroll
                for (int t = 0; t < NTL; ++t)
                    o[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[u % PVP], pb[t], o[t][u], 0, 0, 0);
                if (u + PVP < NU) va[u % PVP] = vload(u + PVP);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // a7 / a8: epilogue.  Every wave publishes the running max and total
    // denominator of its tile's heads for the others.
    __syncthreads();  // every wave is done with the ring and the exchange buffers
    LDS_AS float *mh = (LDS_AS float *)&xp[0][0];
    LDS_AS float *lh = mh + HWG;
    LDS_AS float *red = lh + HWG;
    static_assert(sizeof(xp) >= (2 + NW) * HWG * sizeof(float), "epilogue state fits in xp");
    const float ltot = sum_rows4(lsum);
    if (g == 0) {
        mh[16 * wid + li] = m;
        lh[16 * wid + li] = ltot;
    }
    __syncthreads();
    store_outputs<D, NW, NTL>(p, o, mh, lh, red, qi, s, hg, (LDS_AS uint8_t *)&tile[0][0]);
}

// Head-split variant, for unsplit launches whose (query, 16 heads) units all
// fit the compute units at once and whose lists are short (decode steps with
// few valid entries, window-only lists).  Same steps and results as
// attn_fwd_kernel up to the rounding of the softmax reference; the work is
// split the other way round: a workgroup serves 16 heads of one query over the
// query's whole list, so no partials leave the workgroup and no combine runs,
// at the price of every row being read by each of the query's head groups
// (they share an XCD, so the repeats come from L2).
//
// FP4 build (f2): a row of the second source is its record (rec2 bytes, one
// load, the first rec2/16 lanes' bytes kept), written into its padded LDS row where
// expand_fp4_own expects it and expanded there in place by the wave that wrote
// it, before the round's barrier; the bf16 rows the kernel then reads are the
// ones the bf16 build reads, so both builds agree bit for bit.
//
// The list is consumed in rounds of RR = 48 entries.  Rows travel through
// registers: each of the 8 waves requests RPW = 6 rows of round i + 2
// (ordinary 16-byte loads, the compiler tracks them) while round i is
// computed, and writes round i into one of three LDS round buffers, so no LDS
// holds rows in flight.  (The compiler's waits before those writes cover every
// load in flight, round i + 1's too.  Issuing every round's loads
// unconditionally, past the list the last round's rows again, lets it wait for
// round i alone, but measured slower on MI355X: 10.7 against 9.7 us for 64
// window-only lists, and slower at every list length up to 512: the extra
// rounds of loads and the extra barrier at the end cost more.)
// Iteration i: round i's rows go to LDS, one barrier, then
//   - waves 0..2 (the scorers) each take one 16-row block of round i: S^T over
//     all of d (q of the 16 heads in registers), the block's softmax weights
//     as bf16, published with the block's reference max and weight sum;
//   - every wave adds round i - 1's blocks to O^T for its D/8 output columns of
//     all 16 heads (the published weights are the MFMA operands as written).
// Three round buffers and two weight buffers keep each iteration's writers off
// what the previous iteration's readers use, so one barrier per round does.
//
// a5 with per-block references: a scorer takes the running reference R (log2
// units, identical in every wave) and raises its block's reference to the
// block's max only when that beats R by more than MAX_SLACK, as the
// deep-gather kernel does per chunk.  The column owners then move R to the
// largest reference of the round (rescaling O and the denominator once) and
// add each block with factor 2^(m_b - R), which is 1 unless a block raised
// its reference; only then do the blocks go through a scaled path.
template <int D, bool FP4>
__global__ __launch_bounds__(512) void attn_fwd_hs_kernel(FwdParams p) {
    constexpr int NW = 8, NT = NW * 64;
    constexpr int RR = 48;               // list entries per round
    constexpr int RPW = RR / NW;         // rows each wave loads per round
    constexpr int NB = RR / 16;          // 16-row blocks per round, one scorer wave each
    constexpr int NBUF = 3;              // LDS round buffers
    constexpr int RS = 2 * D + 32;       // padded LDS row (see attn_fwd_kernel)
    constexpr int KS = D / 32;           // QK^T k-steps
    constexpr int CW = D / NW;           // output columns per wave
    constexpr int NTL = CW / 16;         // 16-column output tiles per wave
    static_assert(D == 512, "one row per wave load instruction (64 lanes x 16 bytes)");
    static_assert(RPW * NW == RR && NB * 16 == RR, "rounds split evenly");
    __shared__ __attribute__((aligned(16))) uint8_t rbuf[NBUF][RR * RS];
    __shared__ __attribute__((aligned(16))) u32x2_t pub[2][NB][64];  // bf16 weights per block
    __shared__ float mbs[2][NB][16], lbs[2][NB][16];                 // reference and sum per head
    __shared__ int32_t cnt[NW];
    extern __shared__ int32_t list[];  // the compacted list (K entries, dynamic)
    static_assert(sizeof(rbuf) + sizeof(pub) + sizeof(mbs) + sizeof(lbs) + sizeof(cnt) == hs_static_lds(D),
                  "the host's LDS figure matches the declarations");

    const int unit = unit_of(blockIdx.x, p.units, p.bs, p.dv_bs);
    if (unit < 0) return;
    // workgroup- and wave-uniform values, in scalar registers
    const int qi = udiv(unit, p.dv_HG);
    const int hg = unit - qi * p.HG;
    const int b = udiv(qi, p.dv_T);
    const int tid = threadIdx.x, lane = tid & 63, wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, li = lane & 15;
    const int h = hg * 16 + li;  // head of this lane (QK^T columns, softmax, outputs)
    const bool scorer = wid < NB;
    const uint16_t *kva = p.kv + (int64_t)b * p.rows_a * D;
    const uint16_t *kvb2 = p.kv2 + ((int64_t)b * p.rows_b - p.W) * D;
    const uint8_t *recb = (const uint8_t *)p.kv2 + ((int64_t)b * p.rows_b - p.W) * p.rec2;
    // a2: where this lane's 16 bytes of row j are (one wave instruction per
    // row); FP4 build, j >= W: of its record, lanes past the record reading
    // its last 16 bytes again (unused).  Every lane loads, so no load sits in a
    // lane-dependent branch and the compiler can count them.
    // (row numbers and W are below 2^31: the source test is a 32-bit scalar compare)
    const int Wc = (int)(p.W < 0x7FFFFFFF ? p.W : 0x7FFFFFFF);
    auto row_src = [&](int j) {
        if (FP4 && j >= Wc)
            return (const u32x4_t *)(recb + (int64_t)j * p.rec2 + (lane * 16 < p.rec2 ? lane * 16 : p.rec2 - 16));
        return (const u32x4_t *)((j < Wc ? kva : kvb2) + (int64_t)j * D) + lane;
    };
    auto load_row = [&](int j, u32x4_t &dst) { dst = *row_src(j); };
    // row j into position r of a round buffer (a record where expand_fp4_own reads it)
    auto write_row = [&](LDS_AS uint8_t *Lb, int r, int j, const u32x4_t &v) {
        if (!FP4 || j < Wc)
            *(LDS_AS u32x4_t *)(Lb + r * RS + lane * 16) = v;
        else if (lane * 16 < p.rec2)
            *(LDS_AS u32x4_t *)(Lb + r * RS + ((r & 1) ? 0 : RS - p.rec2) + lane * 16) = v;
    };

    // Prologue: the raw list and the 16 heads' q (into the last round buffer,
    // untouched until round 2) by LDS-DMA; the scorers then take q into
    // registers as the B operands of QK^T.
    LDS_AS uint8_t *qlds = (LDS_AS uint8_t *)&rbuf[NBUF - 1][0];
    {
        const int32_t *lst = p.idxs + (int64_t)qi * p.K;
        const int NI = (p.K + 63) / 64;
        for (int i = wid; i < NI; i += NW) {
            const int k = i * 64 + lane;
            if (k < p.K) lds_dma4(lst + k, (LDS_AS int32_t *)&list[i * 64]);
        }
#pragma unroll
        for (int j = wid; j < 16; j += NW) {
            const int hh = hg * 16 + j < p.H ? hg * 16 + j : 0;  // heads beyond H: zeroed below
            lds_dma16(p.q + ((int64_t)qi * p.H + hh) * D + lane * 8, (LDS_AS void *)(qlds + j * RS));
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // a3: qf[k] = q[h, 32k + 8g .. +7]
    bf16x8_t qf[KS];
    if (scorer) {
        const LDS_AS uint8_t *Q = qlds + li * RS + g * 16;
#pragma unroll
        for (int k = 0; k < KS; ++k) qf[k] = __builtin_bit_cast(bf16x8_t, *(const LDS_AS u32x4_t *)(Q + 64 * k));
        if (h >= p.H) {
#pragma unroll
            for (int k = 0; k < KS; ++k) qf[k] = bf16x8_t{};
        }
    }

    // a1, then rounds 0 and 1, every load unconditional (a round past the
    // list reads q's first 1 KB, in bounds, and is never used), so that the
    // compiler's count lets the first round's write wait for round 0 alone.
    // Requesting them from the raw list before the compaction held every wave
    // in row-request issue (~3300 cycles for 12 rows each) ahead of the
    // compaction's barriers, and the conditional re-requests after it made
    // the first write wait for both rounds.
    const int n = compact_list<NT>((const LDS_AS int32_t *)&list[0], p.K, p.N, list, cnt);
    const int nr = (n + RR - 1) / RR;
    // the wave's rows of round r (lane k < RPW holds its k-th); positions
    // past n repeat the round's first row, whose scores are masked
    auto round_rows = [&](int r) {
        const int e = RR * r + RPW * wid + (lane % RPW);
        return list[e < n ? e : RR * r];
    };
    u32x4_t rg[2][RPW];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int rows = r < nr ? round_rows(r) : 0;
#pragma unroll
        for (int k = 0; k < RPW; ++k) {
            const int rw = __builtin_amdgcn_readlane(rows, k);
            rg[r][k] = *(r < nr ? row_src(rw) : (const u32x4_t *)p.q + lane);
        }
    }

    // Running reference and denominator of head h (the same in every wave),
    // and O^T over this wave's columns: o[t][i] = O^T[CW wid + 16t + 4g + i, h].
    float Rs = -INFINITY, lsum = 0.f;
    f32x4_t o[NTL];
#pragma unroll
    for (int t = 0; t < NTL; ++t) o[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // a4 / a5 (scorer wid): block wid of round r (in buffer Lb), published into pub[pbi]
    auto score = [&](int r, const LDS_AS uint8_t *Lb, int pbi) {
        const int cntb = n - RR * r - 16 * wid;  // valid rows of the block
        f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
        const LDS_AS uint8_t *T = Lb + (16 * wid + li) * RS + g * 16;
        constexpr int QKP = 4;  // K operands requested ahead
        bf16x8_t ka[QKP];
#pragma unroll
        for (int k = 0; k < QKP; ++k) ka[k] = __builtin_bit_cast(bf16x8_t, *(const LDS_AS u32x4_t *)(T + 64 * k));
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[k % QKP], qf[k], sacc, 0, 0, 0);
            if (k + QKP < KS) ka[k % QKP] = __builtin_bit_cast(bf16x8_t, *(const LDS_AS u32x4_t *)(T + 64 * (k + QKP)));
            __builtin_amdgcn_sched_barrier(0);
        }
        // lane (li, g) holds rows 4g + i of head h
        float sv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[i] = 4 * g + i < cntb ? sacc[i] * p.qk_scale_log2 : -INFINITY;
        const float lmax = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        float mb = Rs;
        if (__ballot(lmax > Rs + MAX_SLACK)) {
            const float cmax = max_rows4(lmax);
            mb = cmax > Rs + MAX_SLACK ? cmax : Rs;
        }
        // the weights enter the value product as bf16; the sum counts the same rounded weights
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pv[i] = sv[i] == -INFINITY ? 0.f : exp2_fast(sv[i] - mb);
        const u32x2_t pw = {pack2_bf16(pv[0], pv[1]), pack2_bf16(pv[2], pv[3])};
        const float ps = sum_rows4(add_bf16_pair(pw[1], add_bf16_pair(pw[0], 0.f)));
        pub[pbi][wid][lane] = pw;
        if (g == 0) {
            mbs[pbi][wid][li] = mb;
            lbs[pbi][wid][li] = ps;
        }
    };
    // a6 (every wave): O^T[d, h] += V^T[d, j] P^T[j, h] over the round's blocks
    // for d in this wave's columns.  A transpose load hands lane (li, g)
    // column 16t + li of rows 4g .. 4g+3 of a block, the k-slice of the
    // 16x16x16 MFMA whose B operand is the scorer's packed weights of those
    // rows.  Every LDS read of the round is requested before any is used.
    auto pv_round = [&](const LDS_AS uint8_t *Lb, int pbi) {
        float mv[NB], lv[NB];
        s16x4_t pbv[NB];
        s16x4_t va[NB][NTL];
        const LDS_AS uint8_t *V0 = Lb + (4 * g + (li >> 2)) * RS + (CW * wid + 4 * (li & 3)) * 2;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            mv[bb] = mbs[pbi][bb][li];
            lv[bb] = lbs[pbi][bb][li];
            pbv[bb] = __builtin_bit_cast(s16x4_t, pub[pbi][bb][lane]);
#pragma unroll
            for (int t = 0; t < NTL; ++t)
                va[bb][t] = __builtin_bit_cast(s16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                                            (LDS_AS bf16x4_t *)(V0 + 16 * bb * RS + 32 * t)));
        }
        float Rn = Rs;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) Rn = fmaxf(Rn, mv[bb]);
        float c[NB];  // factor of each block against the new reference
        bool scaled = false;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            c[bb] = lv[bb] == 0.f || mv[bb] == Rn ? 1.f : exp2_fast(mv[bb] - Rn);
            scaled |= c[bb] != 1.f;
        }
        if (__ballot(Rn > Rs)) {  // a reference moved up (rare after the first round)
            const float a = Rn > Rs ? (Rs == -INFINITY ? 0.f : exp2_fast(Rs - Rn)) : 1.f;
            lsum *= a;
#pragma unroll
            for (int t = 0; t < NTL; ++t) o[t] *= a;
            Rs = Rn;
        }
        if (__ballot(scaled)) {
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
                for (int t = 0; t < NTL; ++t) {
                    const f32x4_t z = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[bb][t], pbv[bb],
                                                                               f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    o[t] += z * c[bb];
                }
                lsum += lv[bb] * c[bb];
            }
        } else {
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
#pragma unroll
                for (int t = 0; t < NTL; ++t)
                    o[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[bb][t], pbv[bb], o[t], 0, 0, 0);
                lsum += lv[bb];
            }
        }
    };
    // Iteration i: round i's rows into LDS buffer i % 3 and round i + 2's
    // requested into the registers they leave; one barrier; the value
    // product of round i - 1; the scoring of round i.  Buffer i % 3 was last
    // read by iteration i - 2, and weight buffer i % 2 by iteration i - 1,
    // both before the barrier of iteration i - 1 that every wave has passed.
    auto iter = [&](int i, u32x4_t (&buf)[RPW], int pbi) {
        LDS_AS uint8_t *Lw = (LDS_AS uint8_t *)&rbuf[i % NBUF][0];
        if (i < nr) {
            const int now = FP4 ? round_rows(i) : 0;
#pragma unroll
            for (int k = 0; k < RPW; ++k)
                write_row(Lw, RPW * wid + k, FP4 ? __builtin_amdgcn_readlane(now, k) : 0, buf[k]);
            if (i + 2 < nr) {
                const int rows = round_rows(i + 2);
#pragma unroll
                for (int k = 0; k < RPW; ++k) load_row(__builtin_amdgcn_readlane(rows, k), buf[k]);
            }
            if constexpr (FP4) expand_fp4_own<D, RPW>(Lw, RS, p.rec2, list, RR * i, n, p.W);
        }
        __syncthreads();
        if (i > 0) pv_round((const LDS_AS uint8_t *)&rbuf[(i - 1) % NBUF][0], pbi ^ 1);
        if (i < nr && scorer) score(i, Lw, pbi);
    };
    // unrolled by two so that each round's register buffer is a fixed one
    for (int i = 0; i <= nr; i += 2) {
        iter(i, rg[0], 0);
        if (i + 1 <= nr) iter(i + 1, rg[1], 1);
    }

    // a7 / a8: the sink joins the denominator (as in store_outputs); the
    // outputs go straight to memory, 8 bytes per lane
    float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    if (p.sink != nullptr && h < p.H) {
        const float zs = p.sink[h] * LOG2E;
        const float Mx = fmaxf(Rs, zs);
        const float alpha = Rs == -INFINITY ? 0.f : exp2_fast(Rs - Mx);
        inv = Mx == -INFINITY ? 0.f : alpha / (lsum * alpha + exp2_fast(zs - Mx));
    }
    uint16_t *dst = p.out + ((int64_t)qi * p.H + h) * D;
#pragma unroll
    for (int t = 0; t < NTL; ++t) {
        const int col = CW * wid + 16 * t + 4 * g;
        float v0 = o[t][0] * inv, v1 = o[t][1] * inv, v2 = o[t][2] * inv, v3 = o[t][3] * inv;
        if (col >= D - p.rd) {  // f3: rotary dims, pairs (col, col+1), (col+2, col+3)
            const int64_t pr = (int64_t)(qi % p.T) * (p.rd / 2) + (col - (D - p.rd)) / 2;
            rotate_back2(v0, v1, v2, v3, *(const float4 *)(p.rope + 2 * pr));
        }
        if (h < p.H) *(u32x2_t *)(dst + col) = u32x2_t{pack2_bf16(v0, v1), pack2_bf16(v2, v3)};
    }
}

// a9: log-sum-exp merge of the splits.  Split s holds p_s (its output
// normalised by its own denominator l_s; fp16 times the power of two x_s of
// the row), its max m_s and l_s (log2 units).  With
// M = max(sink, max_s m_s) and L = 2^(sink - M) + sum_s 2^(m_s - M) l_s,
// out = sum_s (2^(m_s - M) l_s / L) p_s.
//
// LPR = D/8 lanes own one output row (8 columns each), so a wave merges
// 64/LPR rows and a workgroup 4x that.  The first SB splits of the rows and
// every (m, l, x) of the lane's row are requested before anything is waited
// for, so the merge costs about one memory round trip.  The max and the
// denominator are reduced over the row's lanes on the VALU; each split's
// factor is then read from the lane that holds it (a row per wave, D = 512)
// or through a small LDS table (D < 512).  Workgroups are laid out so that the rows
// of a query are merged on the XCD whose workgroups wrote its partials (the
// same blockIdx-to-XCD order as attn_fwd), where they may still sit in L2.
template <int D, int SB>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t *__restrict__ ws_o,
                                                      const float *__restrict__ ws_m,
                                                      const float *__restrict__ ws_l,
                                                      const float *__restrict__ ws_x,
                                                      const int32_t *__restrict__ ws_plan,
                                                      const float *__restrict__ sink,
                                                      uint16_t *__restrict__ out, int QH,
                                                      int H, int S, int per_xcd,
                                                      const float *__restrict__ rope, int rd,
                                                      int T, Div32 dvH, Div32 dvT) {
    constexpr int LPR = D / 8;       // lanes per row
    constexpr int RPW = 64 / LPR;    // rows per wave
    constexpr int RWG = 4 * RPW;     // rows per workgroup
    // SB: splits per batch of row loads (4 for launches with up to 4 splits, else 8)
    constexpr int SPL = MAX_SPLITS / LPR > 0 ? MAX_SPLITS / LPR : 1;  // scalar slots per lane
    __shared__ float coef[RWG][MAX_SPLITS];

    const int bid = blockIdx.x;
    // reversed blocks per XCD, like the attention kernels' unit order (the
    // partials of a query were written on the XCD that merges them)
    // output rows are numbered in 32 bits (the host keeps B*T*H below 2^31),
    // so the divisions below are 32-bit ones; the workgroup's numbers are
    // scalar
    const int wg = __builtin_amdgcn_readfirstlane(8 * per_xcd - 1 - ((bid & 7) * per_xcd + (bid >> 3)));
    const int lane = threadIdx.x & 63, wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rw = wid * RPW + lane / LPR;   // row within the workgroup
    const int sl = lane % LPR;               // lane within the row
    const int qh = wg * RWG + rw;
    const bool ok = qh < QH;                  // (no early exit: the row's lanes shuffle)
    const int qi = ok ? udiv(qh, dvH) : 0;
    const int h = ok ? qh - qi * H : 0;
    const int c8 = sl * 8;
    const int64_t slot0 = (int64_t)qi * S * H + h;  // slot of split j: slot0 + j * H
    // a10: the splits this query's list was cut into (the first Sq slots).
    // The first batch of partials and every scalar are requested before Sq
    // arrives (all S slots lie inside the workspace; a slot the plan leaves
    // out may hold stale bits and is masked once Sq is known), so the merge
    // costs one memory round trip, not two.
    // Lanes past the last row (!ok) read row 0's slots, which exist, and
    // store nothing: every load below is unconditional in the lane, so none
    // sits in a branch of its own and the compiler issues them all before
    // waiting for any.
    int Sq = ws_plan[qi];

    // The partials are read once: non-temporal loads with up to four splits
    // (measured faster there; with eight, ordinary loads were faster).
    auto part = [&](int j) {
        const u32x4_t *ptr = (const u32x4_t *)(ws_o + (slot0 + (int64_t)j * H) * D + c8);
        return S <= 4 ? __builtin_nontemporal_load(ptr) : *ptr;
    };
    // the first batch: slots past S read slot S - 1 again (no branch per
    // load) and are zeroed below with the ones past Sq
    u32x4_t v[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) v[j] = part(j < S ? j : S - 1);
    // rotary dims: the (cos, sin) of the lane's four pairs (other lanes read
    // the first pair's and keep the identity)
    const bool rot = c8 >= D - rd;
    float4 cs0 = {1.f, 0.f, 1.f, 0.f}, cs1 = cs0;
    if (rd > 0) {
        const float *f = rope + 2 * ((int64_t)(qi - udiv(qi, dvT) * T) * (rd / 2) + (rot ? (c8 - (D - rd)) / 2 : 0));
        const float4 r0 = *(const float4 *)f, r1 = *(const float4 *)(f + 4);
        if (rot) cs0 = r0, cs1 = r1;
    }
    // lane sl holds the scalars of splits sl, sl + LPR, ... (lanes past S
    // read split 0's and drop them)
    float mj[SPL], lj[SPL], xj[SPL];
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
        const int j = sl + k * LPR;
        const int64_t slot = slot0 + (int64_t)(j < S ? j : 0) * H;
        mj[k] = ws_m[slot];
        lj[k] = ws_l[slot];
        xj[k] = ws_x[slot];
    }
    const float zs = sink != nullptr ? sink[h] : 0.f;
    Sq = Sq < 1 ? 1 : (Sq > S ? S : Sq);
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
        if (!ok || sl + k * LPR >= Sq) {
            mj[k] = -INFINITY;
            lj[k] = 0.f;
            xj[k] = 0.f;
        }
    }
#pragma unroll
    for (int j = 0; j < SB; ++j)
        if (!ok || j >= Sq) v[j] = u32x4_t{0, 0, 0, 0};
    const float mz = ok && sink != nullptr ? zs * LOG2E : -INFINITY;
    float mx = mz;
#pragma unroll
    for (int k = 0; k < SPL; ++k) mx = fmaxf(mx, mj[k]);
    mx = group_reduce<LPR, true>(mx);
    float L = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
        for (int k = 0; k < SPL; ++k) L += exp2_fast(mj[k] - mx) * lj[k];
    }
    L = group_reduce<LPR, false>(L);
    if (mx != -INFINITY && sink != nullptr) L += exp2_fast(mz - mx);
    const float invL = L > 0.f ? 1.f / L : 0.f;
    // split j's factor: with a row per wave (LPR = 64, one slot per lane) lane
    // j holds it and the others read it with a lane read; else through LDS
    float cj[SPL];
#pragma unroll
    for (int k = 0; k < SPL; ++k) {
        const int j = sl + k * LPR;
        const float c = mx != -INFINITY ? exp2_fast(mj[k] - mx) * lj[k] * invL : 0.f;
        cj[k] = c * xj[k];
        if (LPR < 64 && j < S) coef[rw][j] = cj[k];
    }
    if constexpr (LPR < 64) __syncthreads();
    auto coef_of = [&](int j) {
        if constexpr (LPR == 64) return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cj[0]), j));
        else return coef[rw][j];
    };

    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < S; j0 += SB) {
        if (j0 > 0) {
#pragma unroll
            for (int j = 0; j < SB; ++j)
                v[j] = ok && j0 + j < Sq ? part(j0 + j) : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int j = 0; j < SB; ++j) {
            if (j0 + j < S) {
                const float c = coef_of(j0 + j);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const f32x2_t f = unpack2_f16(v[j][e]);
                    acc[2 * e] += c * f[0];
                    acc[2 * e + 1] += c * f[1];
                }
            }
        }
    }
    if (rot) {
        rotate_back2(acc[0], acc[1], acc[2], acc[3], cs0);
        rotate_back2(acc[4], acc[5], acc[6], acc[7], cs1);
    }
    if (ok) {
        const u32x4_t w = {pack2_bf16(acc[0], acc[1]), pack2_bf16(acc[2], acc[3]),
                           pack2_bf16(acc[4], acc[5]), pack2_bf16(acc[6], acc[7])};
        *(u32x4_t *)(out + (int64_t)qh * D + c8) = w;
    }
}

// f4: top-k selection of compressed positions (DeepSeek-V4.1 pages, "blocks,
// re-index groups" page, the _compress_topk_idxs excerpt: index_topk positions
// per query, int32 lists offset by the window length, -1 where fewer are
// visible).  Scores are ranked by value as an unsigned key: NaN lowest, -0 and
// +0 equal; equal keys are taken in ascending index order.
__device__ __forceinline__ uint32_t score_key(float f) {
    if (f != f) return 0u;        // NaN below everything
    if (f == 0.f) f = 0.f;        // -0 -> +0
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave: row shifts by 1, 2, 4
// and 8 lanes (DPP, within each row of 16) scan the rows, then the totals of
// the lower rows are added from lanes 15, 31 and 47.
__device__ __forceinline__ int wave_inclusive_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
    const int lane = threadIdx.x & 63;
    const int r15 = __builtin_amdgcn_readlane(x, 15);
    const int r31 = __builtin_amdgcn_readlane(x, 31);
    const int r47 = __builtin_amdgcn_readlane(x, 47);
    return x + (lane >= 16 ? r15 : 0) + (lane >= 32 ? r31 : 0) + (lane >= 48 ? r47 : 0);
}

// Exclusive prefix sum over the NT threads of a workgroup; returns the sum of
// the lower threads' values, and the total in *total.  ws holds NT/64 ints.
template <int NT>
__device__ int block_exclusive_scan(int v, int *ws, int *total) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int incl = wave_inclusive_scan(v);
    if (lane == 63) ws[wid] = incl;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int c = ws[w];
        before += w < wid ? c : 0;
        all += c;
    }
    __syncthreads();  // ws may be reused
    *total = all;
    return before + incl - v;
}

// Radix digits of the select, most significant first: 11, 11 and 10 bits
// (2048 bins), so that one pass usually leaves a single key per bin near the
// k-th and two passes suffice.
constexpr int TOPK_BINS = 2048;
__device__ __forceinline__ int digit_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ uint32_t digit_mask(int pass) { return pass == 2 ? 1023u : 2047u; }

// The digit of the current pass where the count of keys from the top reaches
// `need`.  Thread t owns the BPT bins just below 2048 - t*BPT (so lower
// threads hold higher digits); a workgroup scan of the chunk sums gives the
// count above each chunk, and the thread whose chunk holds the crossing walks
// its bins.  Leaves the digit, what is still needed within it and its bin
// count in sh[0..2].  Every thread calls it; it ends with a barrier.
template <int NT>
__device__ void find_digit(const int *hist, int need, int *ws, int *sh) {
    constexpr int BPT = TOPK_BINS / NT, NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int lo = TOPK_BINS - (tid + 1) * BPT;
    int h[BPT], sum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        h[j] = hist[lo + j];
        sum += h[j];
    }
    const int incl = wave_inclusive_scan(sum);
    if (lane == 63) ws[wid] = incl;
    __syncthreads();
    int above = incl - sum;
#pragma unroll
    for (int w = 0; w < NW; ++w) above += w < wid ? ws[w] : 0;
    if (above < need && above + sum >= need) {
#pragma unroll
        for (int j = BPT - 1; j >= 0; --j) {
            if (above < need && above + h[j] >= need) {
                sh[0] = lo + j;
                sh[1] = need - above;
                sh[2] = h[j];
            }
            above += h[j];
        }
    }
    __syncthreads();
}

// Histogram slot of digit b in the register kernel: the 16-byte groups of
// each 32-bin block are permuted by the block number, so that the one wave
// that reads the whole histogram (lane l one block, a 16-byte group per
// instruction) spreads every instruction's 64 lanes over all 32 banks.
__device__ __forceinline__ int bin_slot(int b) { return b ^ (((b >> 5) & 7) << 2); }

// find_digit for a swizzled histogram, done by wave 0 alone: lane l sums the
// 32 bins of block 63 - l (so lower lanes hold higher digits), one scan over
// the wave gives the count above each block, and the block where the count
// reaches `need` is scanned again bin by bin, one bin per lane.  Leaves the
// digit, what is still needed within it and its bin count in sh[0..2].  Every
// thread calls it; it ends with a barrier.
__device__ void find_digit_wave(const int *hist, int need, int *sh) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x, blk = 63 - lane;
        int sum = 0;
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            const int4 v = *(const int4 *)&hist[32 * blk + 4 * (g ^ (blk & 7))];
            sum += v.x + v.y + v.z + v.w;
        }
        const int above = wave_inclusive_scan(sum) - sum;
        // exactly one block holds the crossing (1 <= need <= the total)
        const uint64_t cross = __ballot(above < need && above + sum >= need);
        if (cross != 0) {
            const int cl = __ffsll((unsigned long long)cross) - 1;
            const int cabove = __builtin_amdgcn_readlane(above, cl);
            const int bin = 32 * (63 - cl) + 31 - (lane & 31);  // descending within the block
            const int hv = lane < 32 ? hist[bin_slot(bin)] : 0;
            const int upto = cabove + wave_inclusive_scan(hv);
            if (lane < 32 && upto - hv < need && upto >= need) {
                sh[0] = bin;
                sh[1] = need - (upto - hv);
                sh[2] = hv;
            }
        }
    }
    __syncthreads();
}

// One workgroup per query, KPT keys per thread in registers (thread t holds
// positions t*KPT .. t*KPT+KPT-1, so the workgroup covers NT*KPT positions).
// A radix select over the keys narrows the key of the k-th best down to a
// prefix; it stops early once every key that matches the prefix is taken.
// Then one scan of the packed counts (keys above the prefix, keys equal to it)
// gives each thread its output position, and each thread stores its picks
// there in index order.  The chain is short on purpose (it bounds the kernel
// at one row per workgroup): both histograms are cleared while the keys load,
// one wave finds each digit, and the scan takes one barrier.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void topk_reg_kernel(const float *__restrict__ scores,
                                                      const int32_t *__restrict__ lens, int32_t C,
                                                      int32_t k, int32_t offset, int32_t *out,
                                                      int64_t out_stride) {
    static_assert(NT >= 64 && TOPK_BINS % NT == 0 && KPT % 4 == 0, "bins per thread, float4 loads");
    static_assert(TOPK_BINS == 64 * 32, "one wave reads the histogram, 32 bins per lane");
    // two histograms used by alternate passes
    __shared__ __attribute__((aligned(16))) int hist[2][TOPK_BINS];
    __shared__ int ws[NT / 64];
    __shared__ int sh[3];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int64_t q = blockIdx.x;
    const float *s = scores + q * C;
    int L = lens != nullptr ? lens[q] : C;
    L = L < 0 ? 0 : (L > C ? C : L);
    const int kk = k < L ? k : L;
    int32_t *o = out + q * out_stride;
    for (int j = kk + tid; j < k; j += NT) o[j] = -1;
    if (kk == L) {  // everything visible is taken
        for (int j = tid; j < L; j += NT) o[j] = j + offset;
        return;
    }
#pragma unroll
    for (int j = 0; j < TOPK_BINS / NT; ++j) hist[0][tid + j * NT] = 0, hist[1][tid + j * NT] = 0;
    const int base = tid * KPT;
    const int nv = L - base < 0 ? 0 : (L - base > KPT ? KPT : L - base);
    const bool vec = ((C & 3) == 0) && ((reinterpret_cast<uintptr_t>(scores) & 15) == 0);
    uint32_t key[KPT];
    if (vec && nv == KPT) {
#pragma unroll
        for (int g = 0; g < KPT / 4; ++g) {
            const float4 f = *reinterpret_cast<const float4 *>(s + base + 4 * g);
            key[4 * g] = score_key(f.x), key[4 * g + 1] = score_key(f.y);
            key[4 * g + 2] = score_key(f.z), key[4 * g + 3] = score_key(f.w);
        }
    } else {  // slots past the visible length get key 0, taken off bin 0 below
        // every load unconditional (past nv: the first visible score again,
        // L > 0 here), so the thread's loads go out together and it waits once
        const float *src = s + (nv > 0 ? base : 0);
        float f[KPT];
#pragma unroll
        for (int j = 0; j < KPT; ++j) f[j] = src[j < nv ? j : 0];
#pragma unroll
        for (int j = 0; j < KPT; ++j) key[j] = j < nv ? score_key(f[j]) : 0u;
    }
    __syncthreads();

    // pass 0: every key counts, by its top digit
#pragma unroll
    for (int j = 0; j < KPT; ++j) atomicAdd(&hist[0][bin_slot(key[j] >> 21)], 1);
    if (tid == 0 && NT * KPT > L) atomicAdd(&hist[0][bin_slot(0)], L - NT * KPT);
    __syncthreads();
    find_digit_wave(hist[0], kk, sh);
    uint32_t prefix = (uint32_t)sh[0] << 21, mask = 2047u << 21;
    int need = sh[1];  // still to take among the keys that match the prefix
#pragma unroll 1
    for (int pass = 1; pass < 3 && sh[2] != need; ++pass) {
        const int shift = digit_shift(pass);
        const uint32_t dm = digit_mask(pass);
        int *hc = hist[pass & 1];
        // only keys that match the prefix count (a few percent of them after
        // pass 0): an LDS atomic costs per active lane, so the rest sit out
#pragma unroll
        for (int j = 0; j < KPT; ++j) {
            if (j < nv && (key[j] & mask) == prefix) atomicAdd(&hc[bin_slot((int)((key[j] >> shift) & dm))], 1);
        }
        // pass 2 counts into histogram 0, last read before the previous barrier
        if (pass < 2) {
#pragma unroll
            for (int j = 0; j < TOPK_BINS / NT; ++j) hist[0][tid + j * NT] = 0;
        }
        __syncthreads();
        find_digit_wave(hc, need, sh);
        prefix |= (uint32_t)sh[0] << shift;
        mask |= dm << shift;
        need = sh[1];
    }
    // (the loop ends once every key that matches the prefix is taken)
    // take every key whose masked value is above the prefix and the first
    // `need` (by index) equal to it; counts < 2^16 pack into one scan
    int gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const uint32_t m = key[j] & mask;
        gt += j < nv && m > prefix;
        eq += j < nv && m == prefix;
    }
    const int v = (eq << 16) | gt;
    const int incl = wave_inclusive_scan(v);
    if (lane == 63) ws[wid] = incl;
    __syncthreads();
    int before = incl - v;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) before += w < wid ? ws[w] : 0;
    const int eq_before = before >> 16, gt_before = before & 0xFFFF;
    int take_eq = need - eq_before;
    take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
    int pos = gt_before + (eq_before < need ? eq_before : need);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
        const uint32_t m = key[j] & mask;
        const bool tie = j < nv && m == prefix && take_eq > 0;
        const bool pick = (j < nv && m > prefix) || tie;
        if (pick && pos < kk) o[pos] = base + j + offset;
        pos += pick;
        take_eq -= tie;
    }
}

// Rows longer than the register kernels hold: the same selection with the
// scores re-read from memory on every pass.  Thread t owns a contiguous
// segment of positions for the final, order-keeping write.
template <int NT>
__global__ __launch_bounds__(NT) void topk_long_kernel(const float *__restrict__ scores,
                                                       const int32_t *__restrict__ lens,
                                                       int32_t C, int32_t k, int32_t offset,
                                                       int32_t *out, int64_t out_stride) {
    static_assert(TOPK_BINS % NT == 0, "bins per thread");
    __shared__ __attribute__((aligned(16))) int hist[TOPK_BINS];
    __shared__ int ws[NT / 64];
    __shared__ int sh[3];
    const int tid = threadIdx.x;
    const int64_t q = blockIdx.x;
    const float *s = scores + q * C;
    int L = lens != nullptr ? lens[q] : C;
    L = L < 0 ? 0 : (L > C ? C : L);
    const int kk = k < L ? k : L;
    int32_t *o = out + q * out_stride;
    for (int j = kk + tid; j < k; j += NT) o[j] = -1;
    if (kk == L) {
        for (int j = tid; j < L; j += NT) o[j] = j + offset;
        return;
    }
    uint32_t prefix = 0u, mask = 0u;
    int need = kk;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = digit_shift(pass);
        const uint32_t dm = digit_mask(pass);
        for (int j = tid; j < TOPK_BINS; j += NT) hist[j] = 0;
        __syncthreads();
        for (int i = tid; i < L; i += NT) {
            const uint32_t u = score_key(s[i]);
            if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & dm], 1);
        }
        __syncthreads();
        find_digit<NT>(hist, need, ws, sh);
        prefix |= (uint32_t)sh[0] << shift;
        mask |= dm << shift;
        need = sh[1];
        if (sh[2] == need) break;
    }
    const int seg = (L + NT - 1) / NT;
    const int i0 = tid * seg, i1 = i0 + seg < L ? i0 + seg : L;
    int gt = 0, eq = 0;
    for (int i = i0; i < i1; ++i) {
        const uint32_t m = score_key(s[i]) & mask;
        gt += m > prefix;
        eq += m == prefix;
    }
    int tot;
    const int eq_before = block_exclusive_scan<NT>(eq, ws, &tot);
    int take_eq = need - eq_before;
    take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
    int pos = block_exclusive_scan<NT>(gt + take_eq, ws, &tot);
    for (int i = i0; i < i1; ++i) {
        const uint32_t m = score_key(s[i]) & mask;
        if (m > prefix || (m == prefix && take_eq > 0)) {
            if (m == prefix) --take_eq;
            if (pos < kk) o[pos] = i + offset;
            ++pos;
        }
    }
}

__global__ __launch_bounds__(256) void check_idxs_kernel(const int32_t *__restrict__ idxs,
                                                         int64_t total, int64_t N,
                                                         int32_t *bad) {
    int cnt = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256)
        cnt += (int64_t)idxs[i] >= N ? 1 : 0;
    // wave reduction, then one vector atomic per wave
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    if ((threadIdx.x & 63) == 0 && cnt) atomicAdd(bad, cnt);
}

// ------------------------------------------------------------------ host side

int device_cu_count() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
    std::lock_guard<std::mutex> lock(mu);
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            return -1;
        cache[dev] = n;
    }
    return cache[dev];
}

// Workgroup shape for H heads: NHQ wave pairs of HT tiles of 16 heads.
// 64 heads: four pairs of 16-head waves (two waves per SIMD, so one wave's
// LDS reads overlap the other's MFMAs); 32 heads: one pair of 32-head waves;
// up to 16: one pair of 16-head waves.
struct WgShape {
    int nhq, ht;
    int heads() const { return 16 * nhq * ht; }
};
WgShape shape_for(int H) { return H > 32 ? WgShape{4, 1} : H > 16 ? WgShape{1, 2} : WgShape{1, 1}; }
int head_groups(int H) { return (H + shape_for(H).heads() - 1) / shape_for(H).heads(); }

int check_dims(const sa_dims *d) {
    if (d == nullptr) return SA_ERR_NULL;
    if (d->B < 0 || d->T < 0 || d->H < 1 || d->D < 1 || d->N < 0 || d->K < 0) return SA_ERR_SHAPE;
    if (d->D != 128 && d->D != 256 && d->D != 512) return SA_ERR_UNSUPPORTED;
    if (d->K > LIST_CAP) return SA_ERR_UNSUPPORTED;
    // output rows (query, head) are numbered in 32 bits on the device
    if ((int64_t)d->B * d->T * d->H > 0x7FFFFFFF) return SA_ERR_SHAPE;
    return SA_OK;
}

bool aligned(const void *ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

int64_t queries(const sa_dims *d) { return (int64_t)d->B * d->T; }

// The shape a call with S splits launches.  Above 32 heads a deep-gather
// workgroup serves 64 heads; when the workgroups of 32 heads (two wave pairs)
// would still fit the compute units in one round, it serves 32 instead:
// twice the workgroups on a launch that would leave half of the compute units
// idle, each row read by two of them (the second read mostly from L2: both
// sit on one XCD).  Measured at H=64, 640 entries: 32 queries at S=4 take
// 18.4 us per step instead of 20.1, 64 window-only lists at S=1 12.6 instead
// of 13.3; where 64-head workgroups already fill the device (64 queries at
// S=4, 256 queries at S=1) they stay (24.8 and 65 us otherwise, against 23.4
// and 41).  The split count is planned with the 64-head shape.
WgShape shape_for(const sa_dims *d, int S) {
    const WgShape base = shape_for(d->H);
    if (base.nhq != 4) return base;
    // the 64-head workgroup's LDS leaves room for lists of up to ~1970 entries
    if (fwd_static_lds(d->D, 4, 1) + list_lds_bytes(d->K) > (size_t)LDS_BYTES) return WgShape{2, 1};
    const int cus = device_cu_count();
    const int64_t narrow_units = queries(d) * ((d->H + 31) / 32) * S;
    return cus > 0 && narrow_units <= cus ? WgShape{2, 1} : base;
}
int head_groups(const sa_dims *d, int S) {
    const int h = shape_for(d, S).heads();
    return (d->H + h - 1) / h;
}

struct WsLayout {
    size_t o_off, m_off, l_off, x_off, plan_off, bytes;
};

WsLayout ws_layout(const sa_dims *d, int S) {
    WsLayout w{0, 0, 0, 0, 0, 0};
    if (S <= 1) return w;
    const size_t slots = (size_t)queries(d) * S * d->H;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    w.o_off = 0;
    w.m_off = up(slots * d->D * sizeof(uint16_t));
    w.l_off = w.m_off + up(slots * sizeof(float));
    w.x_off = w.l_off + up(slots * sizeof(float));
    w.plan_off = w.x_off + up(slots * sizeof(float));
    w.bytes = w.plan_off + up((size_t)queries(d) * sizeof(int32_t));
    return w;
}

// Unsplit launches at D = 512 whose (query, 16 heads) units all
// fit the compute units at once, with lists of up to HS_MAX_K entries, run
// the head-split kernel.  Measured on MI355X at 64 queries x 64 heads, all
// entries valid, against the deep-gather kernel's best of 2 to 4 splits:
// 11.4 / 13.0 / 15.8 / 17.3 / 18.9 / 21.8 / 23.3 us against 15.9 / 17.3 / 18.5
// / 20.0 / 21.2 / 22.3 / 23.4 us for lists of 128 / 192 / 256 / 320 / 384 /
// 448 / 512 entries, behind at 640 (27.9 against 24.7 us), where every row
// read by four head groups costs more than the split partials save.
constexpr int HS_MAX_K = 512;
bool hs_fits(const sa_dims *d) {
    if (d->D != 512 || d->K > HS_MAX_K) return false;
    if (hs_static_lds(512) + list_lds_bytes(d->K) > (size_t)LDS_BYTES) return false;
    const int cus = device_cu_count();
    return cus > 0 && queries(d) * ((d->H + 15) / 16) <= cus;
}

// Split count for launches with fewer units than compute units.  A split
// shortens every workgroup's share of the list, but its partials cost a
// combine kernel worth about four 32-row chunks of the attention kernel plus
// one per split (fitted on MI355X at 64 heads and 640 entries: ~1.2 us per
// chunk, ~5.5 us per combine, and the step at 32 and 64 queries over S = 2
// to 16).  S minimises rounds(S) * K/(32 S) + (S > 1 ? 4 + S : 0), where
// rounds(S) is the number of waves of workgroups over the compute units,
// among S up to ceil(CUs / units) and K/64.
int plan_splits(const sa_dims *d) {
    const int cus = device_cu_count();
    if (cus < 0) return -SA_ERR_HIP;
    if (hs_fits(d)) return 1;  // the head-split kernel needs no partials
    const int64_t units = queries(d) * head_groups(d->H);
    if (units <= 0 || units >= cus) return 1;
    int64_t smax = (cus + units - 1) / units;
    const int64_t max_by_len = d->K / 64 > 1 ? d->K / 64 : 1;
    if (smax > max_by_len) smax = max_by_len;
    if (smax > MAX_SPLITS) smax = MAX_SPLITS;
    int best = 1;
    double best_cost = d->K / 32.0;
    for (int64_t S = 2; S <= smax; ++S) {
        const int64_t rounds = (units * S + cus - 1) / cus;
        const double cost = (double)rounds * d->K / (32.0 * S) + 4.0 + (double)S;
        if (cost < best_cost) {
            best_cost = cost;
            best = (int)S;
        }
    }
    return best;
}

template <int D, int NHQ, int HT>
hipError_t launch_fwd(const FwdParams &p, hipStream_t stream) {
    const int grid = 8 * p.per_xcd;
    // bf16 rows only, or FP4 records in the second source (a separate build of
    // the kernel, so the bf16 one carries none of the expansion code)
    const size_t lb = list_lds_bytes(p.K);
    if (p.rec2 > 0)
        hipLaunchKernelGGL((attn_fwd_kernel<D, NHQ, HT, true>), dim3(grid), dim3(NHQ * 128), lb, stream, p);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<D, NHQ, HT, false>), dim3(grid), dim3(NHQ * 128), lb, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(WgShape w, const FwdParams &p, hipStream_t stream) {
    if (w.ht == 1) {
        if (w.nhq == 4) return launch_fwd<D, 4, 1>(p, stream);
        if (w.nhq == 2) return launch_fwd<D, 2, 1>(p, stream);
        return launch_fwd<D, 1, 1>(p, stream);
    }
    return launch_fwd<D, 1, 2>(p, stream);
}

// (m, k) of Div32 for a divisor 1 <= d < 2^31
Div32 div32(int64_t d) {
    uint32_t l = 0;
    while (((int64_t)1 << l) < d) ++l;
    const uint32_t k = 31 + l;
    const uint64_t pw = (uint64_t)1 << k;
    return Div32{(uint32_t)(pw / (uint64_t)d + (pw % (uint64_t)d != 0)), k};
}
hipError_t launch_combine(const sa_dims *d, int S, const float *sink, void *out,
                          const void *ws, const WsLayout &L, hipStream_t stream,
                          const float *rope = nullptr, int rd = 0) {
    const int64_t QH = queries(d) * d->H;
    const Div32 dvH = div32(d->H), dvT = div32(d->T > 0 ? d->T : 1);
    const int rwg = 4 * (64 / (d->D / 8));  // rows per workgroup
    const int64_t wgs = (QH + rwg - 1) / rwg;
    const int per_xcd = (int)((wgs + 7) / 8);
    const unsigned grid = (unsigned)(8 * per_xcd);
    const uint16_t *wo = (const uint16_t *)((const uint8_t *)ws + L.o_off);
    const float *wm = (const float *)((const uint8_t *)ws + L.m_off);
    const float *wl = (const float *)((const uint8_t *)ws + L.l_off);
    const float *wx = (const float *)((const uint8_t *)ws + L.x_off);
    const int32_t *wp = (const int32_t *)((const uint8_t *)ws + L.plan_off);
    uint16_t *o = (uint16_t *)out;
#define SA_COMBINE(DD, SB) \
    hipLaunchKernelGGL((combine_kernel<DD, SB>), dim3(grid), dim3(256), 0, stream, wo, wm, wl, wx, wp, sink, o, (int)QH, d->H, S, per_xcd, rope, rd, d->T, dvH, dvT)
    const bool small = S <= 4;  // one batch of four holds every split
    switch (d->D) {
        case 128: if (small) SA_COMBINE(128, 4); else SA_COMBINE(128, 8); break;
        case 256: if (small) SA_COMBINE(256, 4); else SA_COMBINE(256, 8); break;
        default: if (small) SA_COMBINE(512, 4); else SA_COMBINE(512, 8); break;
    }
#undef SA_COMBINE
    return hipGetLastError();
}

// Argument checks shared by the entry points; resolves the split count.
int check_common(const void *q, const void *kv, const int32_t *idxs, const sa_dims *d,
                 int32_t num_splits, void *ws, size_t ws_bytes, bool need_ws, int *S_out) {
    int rc = check_dims(d);
    if (rc != SA_OK) return rc;
    if (num_splits < 0 || num_splits > MAX_SPLITS) return SA_ERR_SPLITS;
    if (queries(d) == 0) {
        *S_out = num_splits > 0 ? num_splits : 1;
        return SA_OK;
    }
    if (q == nullptr || kv == nullptr || (idxs == nullptr && d->K > 0)) return SA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(idxs, 4)) return SA_ERR_ALIGN;
    int S = num_splits;
    if (S == 0) {
        if (ws == nullptr && !need_ws) {
            S = 1;
        } else {
            S = plan_splits(d);
            if (S < 0) return -S;
        }
    }
    if (need_ws && S < 2) return SA_ERR_SPLITS;
    if (S > 1) {
        if (ws == nullptr) return SA_ERR_WORKSPACE;
        if (!aligned(ws, 256)) return SA_ERR_ALIGN;
        if (ws_bytes < ws_layout(d, S).bytes) return SA_ERR_WORKSPACE;
    }
    *S_out = S;
    return SA_OK;
}

void set_divisors(FwdParams &p) {
    p.dv_bs = div32(p.bs > 0 ? p.bs : 1);
    p.dv_S = div32(p.S > 0 ? p.S : 1);
    p.dv_HG = div32(p.HG > 0 ? p.HG : 1);
    p.dv_T = div32(p.T > 0 ? p.T : 1);
}

FwdParams make_params(const void *q, const void *kv, const float *sink, const int32_t *idxs,
                      float scale, void *out, const sa_dims *d, int S, void *ws) {
    FwdParams p{};
    p.q = (const uint16_t *)q;
    p.kv = (const uint16_t *)kv;
    p.kv2 = (const uint16_t *)kv;
    p.W = d->N;
    p.rows_a = d->N;
    p.rows_b = 0;
    p.sink = sink;
    p.idxs = idxs;
    p.out = (uint16_t *)out;
    const WsLayout L = ws_layout(d, S);
    if (S > 1) {
        p.ws_o = (uint16_t *)((uint8_t *)ws + L.o_off);
        p.ws_m = (float *)((uint8_t *)ws + L.m_off);
        p.ws_l = (float *)((uint8_t *)ws + L.l_off);
        p.ws_x = (float *)((uint8_t *)ws + L.x_off);
        p.ws_plan = (int32_t *)((uint8_t *)ws + L.plan_off);
    }
    p.N = d->N;
    p.T = d->T;
    p.H = d->H;
    p.K = d->K;
    p.S = S;
    p.HG = head_groups(d, S);
    const int64_t units = queries(d) * p.HG * S;
    p.units = (int32_t)units;
    // blocks of up to 64 queries' units per XCD turn (see unit_of)
    const int64_t per_q = (int64_t)p.HG * S;
    const int64_t even = (units + 7) / 8;
    const int64_t bs = even < 64 * per_q ? even : 64 * per_q;
    p.bs = (int32_t)bs;
    p.per_xcd = (int32_t)(((even + bs - 1) / bs) * bs);
    p.qk_scale_log2 = scale * LOG2E;
    set_divisors(p);
    return p;
}

template <int D, int NHQ>
hipError_t launch_mq(const FwdParams &p, hipStream_t stream) {
    const int grid = 8 * p.per_xcd;
    const size_t list_bytes = ((size_t)(p.K > 0 ? p.K : 1) * 4 + 15) / 16 * 16;
    if (p.rec2 > 0)
        hipLaunchKernelGGL((attn_fwd_mq_kernel<D, NHQ, true>), dim3(grid), dim3(NHQ * 128),
                           list_bytes, stream, p);
    else
        hipLaunchKernelGGL((attn_fwd_mq_kernel<D, NHQ, false>), dim3(grid), dim3(NHQ * 128),
                           list_bytes, stream, p);
    return hipGetLastError();
}

// The many-query kernel pays off once two of its workgroups can share every
// compute unit; below that the deep-ring kernel keeps more rows in flight.
bool use_mq(const FwdParams &p, int H) {
    const int cus = device_cu_count();
    return H > 16 && cus > 0 && (int64_t)p.units >= 2 * (int64_t)cus;
}

// One workgroup per (query, 16 heads); a query's head groups are consecutive
// units, so they share an XCD (unit_of with bs a multiple of them).
hipError_t launch_hs(FwdParams p, const sa_dims *d, hipStream_t stream) {
    const size_t lb = list_lds_bytes(p.K);
    p.HG = (d->H + 15) / 16;
    const int64_t units = queries(d) * p.HG;
    p.units = (int32_t)units;
    const int64_t even = (units + 7) / 8;
    const int64_t bs = ((even + p.HG - 1) / p.HG) * p.HG;
    p.bs = (int32_t)bs;
    p.per_xcd = (int32_t)bs;
    set_divisors(p);
    if (p.rec2 > 0)
        hipLaunchKernelGGL((attn_fwd_hs_kernel<512, true>), dim3(8 * p.per_xcd), dim3(512), lb, stream, p);
    else
        hipLaunchKernelGGL((attn_fwd_hs_kernel<512, false>), dim3(8 * p.per_xcd), dim3(512), lb, stream, p);
    return hipGetLastError();
}

hipError_t run_fwd(const FwdParams &p, const sa_dims *d, hipStream_t stream) {
    const int D = d->D, H = d->H;
    if (p.S == 1 && hs_fits(d)) return launch_hs(p, d, stream);
    if (use_mq(p, H)) {
        const bool two = H > 32;
        switch (D) {
            case 128: return two ? launch_mq<128, 2>(p, stream) : launch_mq<128, 1>(p, stream);
            case 256: return two ? launch_mq<256, 2>(p, stream) : launch_mq<256, 1>(p, stream);
            default: return two ? launch_mq<512, 2>(p, stream) : launch_mq<512, 1>(p, stream);
        }
    }
    const WgShape w = shape_for(d, p.S);
    switch (D) {
        case 128: return launch_fwd_d<128>(w, p, stream);
        case 256: return launch_fwd_d<256>(w, p, stream);
        default: return launch_fwd_d<512>(w, p, stream);
    }
}

// unit and workgroup numbers (including the spare workgroups of the last
// XCD turn, at most 8 blocks of 64 queries' units) stay below 2^31
bool units_fit(const sa_dims *d, int S) {
    const int64_t per_q = (int64_t)head_groups(d, S) * S;
    return queries(d) * per_q + 512 * per_q <= (int64_t)0x7FFFFFF0;
}

}  // namespace

extern "C" {

int32_t sparse_attn_plan_splits(const sa_dims *d) {
    const int rc = check_dims(d);
    if (rc != SA_OK) return -rc;
    return plan_splits(d);
}

size_t sparse_attn_workspace_bytes_splits(const sa_dims *d, int32_t num_splits) {
    if (check_dims(d) != SA_OK || num_splits < 0 || num_splits > MAX_SPLITS) return 0;
    int S = num_splits;
    if (S == 0) {
        S = plan_splits(d);
        if (S < 0) return 0;
    }
    return ws_layout(d, S).bytes;
}

size_t sparse_attn_workspace_bytes(const sa_dims *d) {
    return sparse_attn_workspace_bytes_splits(d, 0);
}

int sparse_attn_fwd_splits(const void *q, const void *kv, const float *sink, const int32_t *idxs,
                           float scale, void *out, const sa_dims *d, int32_t num_splits,
                           void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return sparse_attn_fwd_rope(q, kv, sink, idxs, scale, nullptr, 0, out, d, num_splits,
                                workspace, workspace_bytes, stream);
}

int sparse_attn_fwd(const void *q, const void *kv, const float *sink, const int32_t *idxs,
                    float scale, void *out, const sa_dims *d, void *workspace,
                    size_t workspace_bytes, hipStream_t stream) {
    return sparse_attn_fwd_rope(q, kv, sink, idxs, scale, nullptr, 0, out, d, 0, workspace,
                                workspace_bytes, stream);
}

int sparse_attn_fwd_rope(const void *q, const void *kv, const float *sink, const int32_t *idxs,
                         float scale, const float *freqs, int32_t rd, void *out, const sa_dims *d,
                         int32_t num_splits, void *workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    int S = 1;
    int rc = check_common(q, kv, idxs, d, num_splits, workspace, workspace_bytes, false, &S);
    if (rc != SA_OK) return rc;
    if (rd < 0 || rd % 8 != 0 || rd > d->D) return SA_ERR_SHAPE;
    if (queries(d) == 0) return SA_OK;
    if (out == nullptr || (rd > 0 && freqs == nullptr)) return SA_ERR_NULL;
    if (!aligned(out, 16) || !aligned(sink, 4) || !aligned(freqs, 16)) return SA_ERR_ALIGN;
    if (!units_fit(d, S)) return SA_ERR_SHAPE;
    FwdParams p = make_params(q, kv, sink, idxs, scale, out, d, S, workspace);
    p.rope = rd > 0 ? freqs : nullptr;
    p.rd = rd;
    if (run_fwd(p, d, stream) != hipSuccess) return SA_ERR_HIP;
    if (S > 1 && launch_combine(d, S, sink, out, workspace, ws_layout(d, S), stream, p.rope,
                                rd) != hipSuccess)
        return SA_ERR_HIP;
    return SA_OK;
}

}  // extern "C"

namespace {

// shared by the two-source entry points; rec = 0 for bf16 compressed rows
int fwd_two_source(const void *q, const void *kv_win, int32_t win_rows, const void *kv_cmp,
                   int32_t cmp_rows, int32_t W, int32_t rec, const float *sink,
                   const int32_t *idxs, float scale, void *out, const sa_dims *d,
                   int32_t num_splits, void *workspace, size_t workspace_bytes,
                   hipStream_t stream) {
    int rc = check_dims(d);
    if (rc != SA_OK) return rc;
    if (W < 0 || W > d->N || win_rows < W || cmp_rows < d->N - W) return SA_ERR_SHAPE;
    if (queries(d) == 0) return num_splits < 0 || num_splits > MAX_SPLITS ? SA_ERR_SPLITS : SA_OK;
    if ((W > 0 && kv_win == nullptr) || (d->N > W && kv_cmp == nullptr)) return SA_ERR_NULL;
    if (!aligned(kv_win, 16) || !aligned(kv_cmp, 16)) return SA_ERR_ALIGN;
    // the common checks see one non-null source; both were checked above
    const void *any = W > 0 ? kv_win : (d->N > W ? kv_cmp : q);
    int S = 1;
    rc = check_common(q, any, idxs, d, num_splits, workspace, workspace_bytes, false, &S);
    if (rc != SA_OK) return rc;
    if (out == nullptr) return SA_ERR_NULL;
    if (!aligned(out, 16) || !aligned(sink, 4)) return SA_ERR_ALIGN;
    if (!units_fit(d, S)) return SA_ERR_SHAPE;
    FwdParams p = make_params(q, any, sink, idxs, scale, out, d, S, workspace);
    p.kv = (const uint16_t *)(kv_win != nullptr ? kv_win : any);
    p.kv2 = (const uint16_t *)(kv_cmp != nullptr ? kv_cmp : any);
    p.W = W;
    p.rows_a = win_rows;
    p.rows_b = cmp_rows;
    p.rec2 = rec;
    if (run_fwd(p, d, stream) != hipSuccess) return SA_ERR_HIP;
    if (S > 1 && launch_combine(d, S, sink, out, workspace, ws_layout(d, S), stream) != hipSuccess)
        return SA_ERR_HIP;
    return SA_OK;
}

// bytes of one FP4 record: D/2 code bytes + D/16 scale bytes, padded to 16
int32_t fp4_record_bytes(int32_t D) { return (9 * D / 16 + 15) / 16 * 16; }

// Workspace of sparse_attn_fwd_noalloc: a static device array (one copy on
// every device the library runs on, held until the process ends).  33 MiB
// covers every planned split count: a split is only planned when the
// workgroups of one split do not fill the device, and then S workgroups per
// query stay below twice the compute units, i.e. under 2 * 256 * 64 partial
// rows of 1 KB at D = 512 plus their scalars and plan.
constexpr size_t SCRATCH_BYTES = (size_t)33 << 20;
__device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

// Device address of the current device's copy of `scratch`, looked up once per
// device (hipGetSymbolAddress with that device current) and kept: in host code
// the array's name is not a device address.  nullptr if the lookup fails.
void *scratch_device_ptr() {
    static std::mutex mu;
    static void *ptr[64] = {nullptr};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

}  // namespace

extern "C" {

int sparse_attn_fwd_2src(const void *q, const void *kv_win, int32_t win_rows, const void *kv_cmp,
                         int32_t cmp_rows, int32_t W, const float *sink, const int32_t *idxs,
                         float scale, void *out, const sa_dims *d, int32_t num_splits,
                         void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return fwd_two_source(q, kv_win, win_rows, kv_cmp, cmp_rows, W, 0, sink, idxs, scale, out, d,
                          num_splits, workspace, workspace_bytes, stream);
}

int32_t sparse_attn_fp4_record_bytes(int32_t D) {
    return D == 128 || D == 256 || D == 512 ? fp4_record_bytes(D) : 0;
}

int sparse_attn_fwd_2src_fp4(const void *q, const void *kv_win, int32_t win_rows,
                             const void *cmp_records, int32_t cmp_rows, int32_t W,
                             const float *sink, const int32_t *idxs, float scale, void *out,
                             const sa_dims *d, int32_t num_splits, void *workspace,
                             size_t workspace_bytes, hipStream_t stream) {
    if (d == nullptr) return SA_ERR_NULL;
    return fwd_two_source(q, kv_win, win_rows, cmp_records, cmp_rows, W,
                          sparse_attn_fp4_record_bytes(d->D), sink, idxs, scale, out, d,
                          num_splits, workspace, workspace_bytes, stream);
}

int sparse_attn_fwd_noalloc(const void *q, const void *kv, const float *sink, const int32_t *idxs,
                            float scale, void *out, const sa_dims *d, int32_t num_splits,
                            hipStream_t stream) {
    int rc = check_dims(d);
    if (rc != SA_OK) return rc;
    if (num_splits < 0 || num_splits > MAX_SPLITS) return SA_ERR_SPLITS;
    if (queries(d) == 0) return SA_OK;
    int S = num_splits;
    if (S == 0) {
        S = plan_splits(d);
        if (S < 0) return -S;
    }
    if (ws_layout(d, S).bytes > SCRATCH_BYTES) return SA_ERR_WORKSPACE;
    void *ws = nullptr;
    if (S > 1) {
        ws = scratch_device_ptr();
        if (ws == nullptr) return SA_ERR_HIP;
    }
    return sparse_attn_fwd_rope(q, kv, sink, idxs, scale, nullptr, 0, out, d, S, ws,
                                S > 1 ? SCRATCH_BYTES : 0, stream);
}

size_t sparse_attn_noalloc_max_bytes(void) { return SCRATCH_BYTES; }

int sparse_attn_fwd_partial(const void *q, const void *kv, const int32_t *idxs, float scale,
                            const sa_dims *d, int32_t num_splits, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
    int S = 1;
    int rc = check_common(q, kv, idxs, d, num_splits, workspace, workspace_bytes, true, &S);
    if (rc != SA_OK) return rc;
    if (queries(d) == 0) return SA_OK;
    if (!units_fit(d, S)) return SA_ERR_SHAPE;
    const FwdParams p = make_params(q, kv, nullptr, idxs, scale, nullptr, d, S, workspace);
    return run_fwd(p, d, stream) == hipSuccess ? SA_OK : SA_ERR_HIP;
}

int sparse_attn_fwd_combine(const float *sink, void *out, const sa_dims *d, int32_t num_splits,
                            const void *workspace, size_t workspace_bytes, hipStream_t stream) {
    int rc = check_dims(d);
    if (rc != SA_OK) return rc;
    if (num_splits < 2 || num_splits > MAX_SPLITS) return SA_ERR_SPLITS;
    if (queries(d) == 0) return SA_OK;
    if (out == nullptr) return SA_ERR_NULL;
    if (workspace == nullptr) return SA_ERR_WORKSPACE;
    if (!aligned(out, 16) || !aligned(sink, 4) || !aligned(workspace, 256)) return SA_ERR_ALIGN;
    const WsLayout L = ws_layout(d, num_splits);
    if (workspace_bytes < L.bytes) return SA_ERR_WORKSPACE;
    return launch_combine(d, num_splits, sink, out, workspace, L, stream) == hipSuccess
               ? SA_OK
               : SA_ERR_HIP;
}

int sparse_attn_check_idxs(const int32_t *idxs, const sa_dims *d, int32_t *d_bad_count,
                           hipStream_t stream) {
    if (d == nullptr) return SA_ERR_NULL;
    if (d->B < 0 || d->T < 0 || d->N < 0 || d->K < 0) return SA_ERR_SHAPE;
    const int64_t total = queries(d) * d->K;
    if (total == 0) return SA_OK;
    if (idxs == nullptr || d_bad_count == nullptr) return SA_ERR_NULL;
    if (!aligned(idxs, 4) || !aligned(d_bad_count, 4)) return SA_ERR_ALIGN;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(check_idxs_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, idxs, total,
                       (int64_t)d->N, d_bad_count);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

const char *sparse_attn_plan_kernel(const sa_dims *d, int32_t num_splits) {
    if (check_dims(d) != SA_OK || num_splits < 0 || num_splits > MAX_SPLITS) return nullptr;
    int S = num_splits;
    if (S == 0) {
        S = plan_splits(d);
        if (S < 0) return nullptr;
    }
    if (S == 1 && hs_fits(d)) return "attn_fwd_hs_kernel<512,false>";
    FwdParams p{};
    p.units = (int32_t)(queries(d) * head_groups(d, S) * S);
    if (use_mq(p, d->H)) {
        const bool two = d->H > 32;
        switch (d->D) {
            case 128: return two ? "attn_fwd_mq_kernel<128,2,false>" : "attn_fwd_mq_kernel<128,1,false>";
            case 256: return two ? "attn_fwd_mq_kernel<256,2,false>" : "attn_fwd_mq_kernel<256,1,false>";
            default: return two ? "attn_fwd_mq_kernel<512,2,false>" : "attn_fwd_mq_kernel<512,1,false>";
        }
    }
    const WgShape w = shape_for(d, S);
    static const char *names[3][4] = {
        {"attn_fwd_kernel<128,4,1,false>", "attn_fwd_kernel<128,1,2,false>", "attn_fwd_kernel<128,1,1,false>",
         "attn_fwd_kernel<128,2,1,false>"},
        {"attn_fwd_kernel<256,4,1,false>", "attn_fwd_kernel<256,1,2,false>", "attn_fwd_kernel<256,1,1,false>",
         "attn_fwd_kernel<256,2,1,false>"},
        {"attn_fwd_kernel<512,4,1,false>", "attn_fwd_kernel<512,1,2,false>", "attn_fwd_kernel<512,1,1,false>",
         "attn_fwd_kernel<512,2,1,false>"}};
    const int di = d->D == 128 ? 0 : d->D == 256 ? 1 : 2;
    const int wi = w.ht == 1 ? (w.nhq == 4 ? 0 : w.nhq == 2 ? 3 : 2) : 1;
    return names[di][wi];
}

int sparse_attn_topk(const float *scores, const int32_t *lens, int32_t Q, int32_t C, int32_t k,
                     int32_t offset, int32_t *out, int64_t out_stride, hipStream_t stream) {
    if (Q < 0 || C < 0 || k < 0 || out_stride < k) return SA_ERR_SHAPE;
    if (Q == 0 || k == 0) return SA_OK;
    if (out == nullptr || (scores == nullptr && C > 0)) return SA_ERR_NULL;
    if (!aligned(out, 4) || !aligned(scores, 4) || !aligned(lens, 4)) return SA_ERR_ALIGN;
    if ((int64_t)offset + C > 0x7FFFFFFF) return SA_ERR_SHAPE;
    // keys held in registers up to 16384 candidates, else re-read from memory;
    // up to 8192 candidates 1024 threads of 8 keys beat 512 of 16 (7.9 against
    // 8.1 us for 64 queries) and 256 of 32 (10.5 us)
    const dim3 grid((unsigned)Q);
    if (C <= 2048)
        hipLaunchKernelGGL((topk_reg_kernel<256, 8>), grid, dim3(256), 0, stream, scores, lens, C, k,
                           offset, out, out_stride);
    else if (C <= 4096)
        hipLaunchKernelGGL((topk_reg_kernel<256, 16>), grid, dim3(256), 0, stream, scores, lens, C, k,
                           offset, out, out_stride);
    else if (C <= 8192)
        hipLaunchKernelGGL((topk_reg_kernel<1024, 8>), grid, dim3(1024), 0, stream, scores, lens, C, k,
                           offset, out, out_stride);
    else if (C <= 16384)
        hipLaunchKernelGGL((topk_reg_kernel<1024, 16>), grid, dim3(1024), 0, stream, scores, lens, C,
                           k, offset, out, out_stride);
    else
        hipLaunchKernelGGL(topk_long_kernel<256>, grid, dim3(256), 0, stream, scores, lens, C, k,
                           offset, out, out_stride);
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

const char *sparse_attn_status_str(int status) {
    switch (status) {
        case SA_OK: return "ok";
        case SA_ERR_NULL: return "a required pointer is NULL";
        case SA_ERR_SHAPE: return "a dimension is out of range";
        case SA_ERR_UNSUPPORTED: return "unsupported size (D must be 128, 256 or 512; K <= 2048)";
        case SA_ERR_ALIGN: return "misaligned pointer (q/kv/out 16 B, idxs/sink 4 B, workspace 256 B)";
        case SA_ERR_WORKSPACE: return "workspace missing or too small";
        case SA_ERR_INDEX_RANGE: return "an index list holds an entry >= N (checked mode)";
        case SA_ERR_HIP: return "HIP error";
        case SA_ERR_SPLITS: return "num_splits out of range";
        default: return "unknown status";
    }
}

}  // extern "C"
