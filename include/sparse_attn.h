/*
 * sparse_attn -- sparse latent attention with a per-head attention sink, for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (DeepSeek-V4.1 pages, "Output projection" page, Attention.forward
 * excerpt: o = sparse_attn(q, kv, attn_sink, topk_idxs, softmax_scale)):
 *
 *   for every query (b, t) and head h, with J = the entries of idxs[b, t, :]
 *   that are >= 0 and < N (each occurrence counts, as a gather does):
 *     s_j = scale * <q[b,t,h,:], kv[b,j,:]>                 for j in J
 *     o[b,t,h,:] = sum_j exp(s_j) kv[b,j,:] / (exp(sink[h]) + sum_j exp(s_j))
 *
 * One latent row kv[b, j, :] is both the key and the value of position j for
 * every head (the same excerpt joins the window rows and the compressed rows
 * into one kv tensor and one index list).  The sink is one float32 logit per
 * head (Attention.__init__ excerpt: attn_sink) that enlarges the denominator
 * and carries no value; it is not multiplied by scale.  The caller passes
 * scale (head_dim ** -0.5 in that excerpt).  With no valid entry the output is
 * zero.  Outputs are bfloat16, rounded to nearest even from float32; scores,
 * the running max, the denominator and the accumulators are float32, and the
 * softmax weights enter the value product as bfloat16.
 *
 * Layouts (all row-major and contiguous, element strides implied by sa_dims):
 *   q     bf16  [B, T, H, D]      (the query after unflatten to heads)
 *   kv    bf16  [B, N, D]         (window rows first, then compressed rows)
 *   sink  f32   [H] or NULL       (NULL = no sink)
 *   idxs  int32 [B, T, K]         (negative = unused slot; K may be 0)
 *   out   bf16  [B, T, H, D]      (must not overlap any input)
 * q, kv and out must be 16-byte aligned; idxs and sink 4-byte aligned;
 * workspace 256-byte aligned.  Supported: D in {128, 256, 512}, any H >= 1,
 * K <= 2048.  Entries >= N are skipped by the kernels (never read); they break
 * the caller's contract and sparse_attn_check_idxs counts them.
 *
 * Ownership and behaviour: the caller owns every buffer; the library never
 * allocates or frees device memory and keeps no state beyond a once-only cache
 * of each device's compute-unit count.  Every entry point only enqueues work
 * on `stream` (it never synchronises or reads device memory from the host),
 * so calls can be captured in a HIP graph.  Inputs must stay alive until the
 * stream reaches the work.  Argument errors are reported synchronously, before
 * any HIP call; launch failures return SA_ERR_HIP.  Nothing throws across the
 * boundary.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

/* Sizes of one call.  B, T >= 0 (zero queries is a no-op); H, D >= 1; N >= 0; K >= 0;
 * B*T*H < 2^31 (output rows are numbered in 32 bits; else SA_ERR_SHAPE). */
typedef struct sa_dims {
    int32_t B, T, H, D, N, K;
} sa_dims;

enum sa_status {
    SA_OK = 0,
    SA_ERR_NULL = 1,        /* a required pointer is NULL */
    SA_ERR_SHAPE = 2,       /* a dimension is out of range */
    SA_ERR_UNSUPPORTED = 3, /* D or K outside what the kernels are built for */
    SA_ERR_ALIGN = 4,       /* a pointer is not aligned as required */
    SA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than sparse_attn_workspace_bytes */
    SA_ERR_INDEX_RANGE = 6, /* checked mode: a list holds an entry >= N.  The enqueue-only entry
                               points never return it (they cannot read device data);
                               sparse_attn_check_idxs counts such entries on the device, and a
                               caller that reads the count reports this code */
    SA_ERR_HIP = 7,         /* a HIP call failed (device query or kernel launch) */
    SA_ERR_SPLITS = 8       /* num_splits outside [0, 64] (the *_splits entry points) */
};

/* Number of index-range splits the library picks when num_splits is 0: one
 * split when the queries alone fill the device or when the head-split kernel
 * serves the launch (see sparse_attn_fwd), else enough splits (each at least 64
 * list entries) to give every compute unit work.  Returns >= 1, or a negative
 * sa_status on bad dims or a failed device query. */
int32_t sparse_attn_plan_splits(const sa_dims *d);

/* Bytes of workspace sparse_attn_fwd needs for the split count the library
 * plans for these dims (sparse_attn_plan_splits): 0 when one split is planned.
 * Returns 0 on bad dims. */
size_t sparse_attn_workspace_bytes(const sa_dims *d);

/* Bytes of workspace for `num_splits` splits (0 = the planned count): 0 for one
 * split, else each split's output normalised by its own denominator as fp16
 * [B*T, S, H, D] (each row divided by a power of two chosen from its largest
 * magnitude, so that no value overflows or sinks into fp16 subnormals), its
 * running max (log2 units), its denominator and the row's scale, float32
 * [B*T, S, H] each, and the per-query split plan, int32 [B*T]; every part
 * padded to 256 bytes.  Returns 0 on bad dims or num_splits outside [0, 64]. */
size_t sparse_attn_workspace_bytes_splits(const sa_dims *d, int32_t num_splits);

/* The whole step: out = sparse_attn(q, kv, sink, idxs, scale), the call of the
 * pages' Attention.forward excerpt with the dims and a workspace made explicit.
 * An unsplit launch at D = 512 with K <= 512 whose B*T*ceil(H/16) units all fit
 * the device's compute units at once runs the head-split kernel: one workgroup
 * per query and 16 heads over the whole list, no workspace; the planner then
 * picks one split.  Its softmax weights are rounded to bf16 against a
 * reference per block of 16 entries instead of per 32-entry chunk, so its
 * results agree with the deep-gather kernel's to within that rounding.
 * workspace NULL: one split (always correct, no workspace).  Otherwise the
 * planned split count (sparse_attn_plan_splits), which needs
 * workspace_bytes >= sparse_attn_workspace_bytes(d), else SA_ERR_WORKSPACE.
 * With more than one split the index list of each query is cut into
 * contiguous ranges of its valid entries, each range is reduced by its own
 * workgroup into a partial (output, max, denominator) in `workspace`, and a
 * second kernel merges the partials with the sink (log-sum-exp combine).  How
 * many ranges a query uses follows its own count of valid entries (a query
 * with n of K entries valid uses ceil(n S / K) of the S split slots), decided on
 * the device.  The partials hold the output in fp16 (11 significant bits,
 * scaled per row), so split counts agree to about 2^-11 of each row's largest
 * value before the final bf16 rounding. */
int sparse_attn_fwd(const void *q, const void *kv, const float *sink, const int32_t *idxs,
                    float scale, void *out, const sa_dims *d, void *workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* sparse_attn_fwd with an explicit split count: num_splits 0 = planned (one
 * split when workspace is NULL), else 1..64 (SA_ERR_SPLITS outside [0, 64]);
 * with more than one split the workspace must hold
 * sparse_attn_workspace_bytes_splits(d, num_splits) bytes. */
int sparse_attn_fwd_splits(const void *q, const void *kv, const float *sink, const int32_t *idxs,
                           float scale, void *out, const sa_dims *d, int32_t num_splits,
                           void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The step followed by the inverse rotary step on the output (DeepSeek-V4.1
 * pages, "Output projection" page, Attention.forward excerpt:
 * apply_rotary_emb(o[..., -rd:], freqs_cis, True) right after sparse_attn),
 * fused into the output's last rounding.
 *   freqs  fp32 [T, rd/2, 2], 16-byte aligned: (cos, sin) of pair i at query
 *          position t (freqs_cis[t, i] as real and imaginary parts; row t serves
 *          query (b, t) of every sequence b, as the excerpt's slice does)
 *   rd     0 (no rotation; freqs may be NULL) or a multiple of 8, <= D
 * Pair i of head h of query (b, t) is the complex number
 * x + iy = o[b,t,h,D-rd+2i] + i o[b,t,h,D-rd+2i+1]; it becomes
 * (x + iy) * conj(cos + i sin), computed in float32 on the normalised output
 * before the one bf16 rounding (the unfused pair of calls rounds twice).  The
 * first D - rd dims equal sparse_attn_fwd's bit for bit.  SA_ERR_SHAPE for a
 * bad rd, SA_ERR_NULL for freqs NULL with rd > 0, SA_ERR_ALIGN for freqs not
 * 16-byte aligned; other arguments as sparse_attn_fwd_splits. */
int sparse_attn_fwd_rope(const void *q, const void *kv, const float *sink, const int32_t *idxs,
                         float scale, const float *freqs, int32_t rd, void *out, const sa_dims *d,
                         int32_t num_splits, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* The same step with the rows in two buffers instead of one concatenated kv
 * (DeepSeek-V4.1 pages, "Output projection" page, Attention.forward excerpt:
 * kv = cat([window_kv, compress_kv], dim=1), with compressed indices offset by
 * the window length).  Entry j of a list (0 <= j < N = d->N) addresses
 *   j <  W : kv_win[b, j, :]        kv_win bf16 [B, win_rows, D], W <= win_rows
 *   j >= W : kv_cmp[b, j - W, :]    kv_cmp bf16 [B, cmp_rows, D], N - W <= cmp_rows
 * so a window ring and a compressed cache (with spare rows beyond the filled
 * length) are read in place, without the copy the concatenation makes.  The
 * result equals sparse_attn_fwd on the concatenated rows, bit for bit.
 * kv_win may be NULL when W == 0 and kv_cmp when W == N; both 16-byte aligned.
 * SA_ERR_SHAPE when W is outside [0, N] or a buffer has too few rows.  Other
 * arguments, checks and behaviour as sparse_attn_fwd_splits. */
int sparse_attn_fwd_2src(const void *q, const void *kv_win, int32_t win_rows, const void *kv_cmp,
                         int32_t cmp_rows, int32_t W, const float *sink, const int32_t *idxs,
                         float scale, void *out, const sa_dims *d, int32_t num_splits,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of one packed FP4 row record for head dimension D (D/2 code bytes +
 * D/16 scale bytes, rounded up to 16): 288 at D = 512.  0 for an unsupported D. */
int32_t sparse_attn_fp4_record_bytes(int32_t D);

/* sparse_attn_fwd_2src with the compressed rows packed as the pages' cache
 * quantises them (DeepSeek-V4.1 pages, "blocks, re-index groups" page,
 * compressor excerpt: groups of 16 elements, FP4 values with E4M3 scales).
 * cmp_records holds one record of R = sparse_attn_fp4_record_bytes(D) bytes per
 * row, [B, cmp_rows, R], 16-byte aligned: bytes 0 .. D/2-1 are OCP E2M1 codes
 * (byte k: element 2k in the low nibble, element 2k+1 in the high nibble),
 * bytes D/2 .. D/2 + D/16 - 1 are OCP E4M3 scales (scale g for elements
 * 16g .. 16g+15), the rest is padding.  Element i of the row is
 * E2M1(code i) x E4M3(scale i/16); the product is exact in bf16, and the result
 * equals sparse_attn_fwd_2src on those bf16 rows, bit for bit (the same kernel
 * runs for both).  The window rows stay bf16.  A NaN scale code makes its
 * group NaN.  On the head-split kernel (see sparse_attn_fwd) each record is
 * expanded in LDS before the round's barrier, which costs more than in the
 * deep-gather kernel: measured at 64 queries x 64 heads with 128 window + 256
 * compressed entries, 26.8 us against 23.0 us with num_splits = 3 (the
 * deep-gather kernel; bf16 rows 16.9 and 20.6 us). */
int sparse_attn_fwd_2src_fp4(const void *q, const void *kv_win, int32_t win_rows,
                             const void *cmp_records, int32_t cmp_rows, int32_t W,
                             const float *sink, const int32_t *idxs, float scale, void *out,
                             const sa_dims *d, int32_t num_splits, void *workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * sparse_attn_fwd_splits with the split workspace taken from a static device
 * array of the library instead of a caller's buffer.  The array holds
 * sparse_attn_noalloc_max_bytes() bytes (33 MiB, enough for every planned split
 * count) on each device the library runs on, from when the library is loaded
 * until the process ends; its address is looked up once per device on the
 * first call there.  num_splits 0 = planned, else 1..64; a split count whose
 * workspace (sparse_attn_workspace_bytes_splits) exceeds the array returns
 * SA_ERR_WORKSPACE.  The call allocates nothing (no hipMalloc, no library
 * allocation) and only enqueues on `stream`.  Every call on one device shares
 * that device's array, which keeps the last call's partials: calls that can
 * overlap on one device (other streams, other threads) race and must be
 * serialised by the caller.  Other arguments, checks and results as
 * sparse_attn_fwd_splits. */
int sparse_attn_fwd_noalloc(const void *q, const void *kv, const float *sink, const int32_t *idxs,
                            float scale, void *out, const sa_dims *d, int32_t num_splits,
                            hipStream_t stream);

/* Bytes of the static array sparse_attn_fwd_noalloc uses. */
size_t sparse_attn_noalloc_max_bytes(void);

/* First half of the split path (num_splits >= 2): writes the partials of every
 * split into `workspace` and nothing into out.  Same arguments and checks as
 * sparse_attn_fwd_splits, without out. */
int sparse_attn_fwd_partial(const void *q, const void *kv, const int32_t *idxs, float scale,
                            const sa_dims *d, int32_t num_splits, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Second half of the split path: merges the partials written by
 * sparse_attn_fwd_partial for the same dims and num_splits with the sink and
 * writes out. */
int sparse_attn_fwd_combine(const float *sink, void *out, const sa_dims *d, int32_t num_splits,
                            const void *workspace, size_t workspace_bytes, hipStream_t stream);

/* The index lists' compressed segment from indexer scores (DeepSeek-V4.1 pages,
 * "blocks, re-index groups" page, _compress_topk_idxs excerpt: index_topk = 512
 * compressed positions per query, int32, offset by the window length, -1 where
 * fewer are visible).
 *   scores  fp32 [Q, C]: the score of compressed position c for query q
 *   lens    int32 [Q] or NULL: query q sees positions 0 .. lens[q]-1 (clamped
 *           to [0, C]); NULL = all C
 *   out     int32, row q at out + q * out_stride (out_stride >= k, so a call can
 *           write the compressed segment of [B, T, K] lists in place): the
 *           indices + offset of the min(k, visible) best scores, in ascending
 *           index order, then -1 up to k.
 * Ranking: by value, NaN below every number, -0 equal to +0; equal scores are
 * taken in ascending index order, so the result is unique.  One workgroup per
 * query; C <= 16384 keeps the scores in registers, longer rows are re-read from
 * memory on each radix pass.
 * Errors: SA_ERR_SHAPE (negative sizes, out_stride < k, offset + C beyond
 * int32), SA_ERR_NULL, SA_ERR_ALIGN (4 bytes), SA_ERR_HIP.  Only enqueues. */
int sparse_attn_topk(const float *scores, const int32_t *lens, int32_t Q, int32_t C, int32_t k,
                     int32_t offset, int32_t *out, int64_t out_stride, hipStream_t stream);

/* Checked mode: adds to *d_bad_count (a device int32, zeroed by the caller)
 * the number of entries of idxs that are >= N.  Such entries break the
 * contract of sparse_attn_fwd (the fast path skips them). */
int sparse_attn_check_idxs(const int32_t *idxs, const sa_dims *d, int32_t *d_bad_count,
                           hipStream_t stream);

/* Name of the attention kernel a call with these dims and num_splits (0 =
 * planned) launches on the current device, as profilers list it (static
 * text), or NULL on bad arguments or a failed device query.  Unsplit launches
 * the head-split kernel serves (see sparse_attn_fwd) take it; other launches
 * of at least two workgroups per compute unit take the many-query kernel (two
 * workgroups share a unit); smaller ones the deep-gather kernel.  The name is
 * that of the bf16-rows build (sparse_attn_fwd_2src_fp4 runs the same kernel
 * built with FP4 records, <..., true>).  For profiling and reports; no call
 * needs it. */
const char *sparse_attn_plan_kernel(const sa_dims *d, int32_t num_splits);

/* Static text for a status code (never NULL). */
const char *sparse_attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
