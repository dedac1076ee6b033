/*
 * ORACLE -- test infrastructure only.
 *
 * A plain, slow, double-precision CPU definition of sparse latent attention
 * with a per-head attention sink.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the product path never does.  It
 * shares no code, header, table or helper with the GPU library.
 *
 * What it follows:
 *  - DeepSeek-V4.1 page "Output projection" (Attention.forward excerpt): the
 *    call sparse_attn(q, kv, attn_sink, topk_idxs, softmax_scale) where q is the
 *    query unflattened to [batch, positions, local heads, head_dim], kv is the
 *    window rows joined with the compressed rows along the position axis (one
 *    latent row of width head_dim per position, used as key and as value), and
 *    topk_idxs is the index list joined along its last axis.
 *  - Same page, Attention.__init__ excerpt: attn_sink is one float32 parameter
 *    per local head; softmax_scale is head_dim ** -0.5 (handed in by the caller).
 *  - DeepSeek-V4.1 page "blocks, re-index groups", _compress_topk_idxs excerpt:
 *    index lists are int32 and may be empty (last axis of length 0).
 *  - GLM-5 page "Sparse latent attention, keys", eager_attention_forward and the
 *    DSA index-mask excerpt: scores are query-key products times the scaling,
 *    unselected positions are removed from the softmax, the softmax is taken in
 *    float32 or wider, and the weights multiply the value rows.
 *
 * Readings where the pages are silent (each one is also listed in the design
 * notes of the repository):
 *  - any negative index means "unused slot" and contributes nothing;
 *  - the sink is a logit in the already-scaled score domain: it adds exp(sink)
 *    to the softmax denominator and has a zero value row.  No page prints a
 *    value that fixes whether the sink is multiplied by the softmax scale, so
 *    the other reading (exp(scale * sink)) is selectable (flag ORACLE_SINK_SCALED)
 *    and each reading is pinned against its own brute force;
 *  - a repeated index counts once per occurrence, as a gather does.  The GLM
 *    index mask (a scatter of the selection into a boolean mask) would count it
 *    once; that reading is selectable too (flag ORACLE_DEDUP: an entry whose
 *    index already appeared earlier in the same list is skipped);
 *  - with no valid index and no sink the output is zero, never NaN;
 *  - an index >= N breaks the contract: the oracle returns an error.
 *
 * Method (three passes per query and head, all in double precision):
 *   pass 1: s_j = scale * <q_h, kv_j> for every valid entry j, and the maximum
 *           m over those scores and the sink logit;
 *   pass 2: w_j = exp(s_j - m), w_sink = exp(sink - m), L = w_sink + sum_j w_j;
 *   pass 3: o_h = (sum_j w_j kv_j) / L.
 * bf16 inputs are widened exactly; scale (a float32) is widened to double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Exact widening of a bfloat16 bit pattern: it is the top half of a float32. */
static double widen_bf16(uint16_t bits)
{
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * flags : 0 for the default readings, or ORACLE_SINK_SCALED | ORACLE_DEDUP
 * q     : bf16 bits [B, T, H, D]
 * kv    : bf16 bits [B, N, D]
 * sink  : float32 [H], or NULL for "no sink"
 * idxs  : int32 [B, T, K]; negative = unused
 * out   : double [B, T, H, D]
 * w     : optional double [B, T, H, K] -- softmax weight of each list entry
 *         (0 for unused entries); NULL to skip
 * wsink : optional double [B, T, H] -- weight that went to the sink; NULL to skip
 * Returns 0, or 1 when some index is >= N (outputs are then unspecified),
 * or 2 on a bad dimension.
 */
#define ORACLE_SINK_SCALED 1
#define ORACLE_DEDUP 2

int oracle_sparse_attn_f64_flags(const uint16_t *q, const uint16_t *kv, const float *sink,
                                 const int32_t *idxs, float scale, int64_t B, int64_t T,
                                 int64_t H, int64_t D, int64_t N, int64_t K, int flags,
                                 double *out, double *w, double *wsink)
{
    if (B < 0 || T < 0 || H <= 0 || D <= 0 || N < 0 || K < 0)
        return 2;
    int bad = 0;
    const double sc = (double)scale;
    const int64_t nq = B * T;

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t qi = 0; qi < nq; ++qi) {
        const int64_t b = qi / T;
        const int32_t *list = idxs + qi * K;
        const uint16_t *kvb = kv + b * N * D;
        double *s = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        double *acc = (double *)malloc(sizeof(double) * (size_t)D);
        char *use = (char *)malloc((size_t)(K > 0 ? K : 1));

        for (int64_t k = 0; k < K; ++k)
            if (list[k] >= N)
                bad = 1;
        /* which entries take part: the valid ones, and with ORACLE_DEDUP only
         * the first occurrence of each index */
        for (int64_t k = 0; k < K; ++k) {
            use[k] = list[k] >= 0;
            if (use[k] && (flags & ORACLE_DEDUP))
                for (int64_t e = 0; e < k; ++e)
                    if (list[e] == list[k])
                        use[k] = 0;
        }

        for (int64_t h = 0; h < H && !bad; ++h) {
            const uint16_t *qh = q + (qi * H + h) * D;
            double *oh = out + (qi * H + h) * D;

            /* pass 1: scores of the valid entries and their maximum, sink included */
            const double zraw = sink ? (double)sink[h] : -INFINITY;
            const double z = (flags & ORACLE_SINK_SCALED) ? sc * zraw : zraw;
            double m = z;
            for (int64_t k = 0; k < K; ++k) {
                const int32_t j = list[k];
                if (!use[k])
                    continue;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d)
                    dot += widen_bf16(qh[d]) * widen_bf16(kvb[(int64_t)j * D + d]);
                s[k] = sc * dot;
                if (s[k] > m)
                    m = s[k];
            }

            if (m == -INFINITY) { /* no sink and no valid entry */
                for (int64_t d = 0; d < D; ++d)
                    oh[d] = 0.0;
                if (w)
                    for (int64_t k = 0; k < K; ++k)
                        w[(qi * H + h) * K + k] = 0.0;
                if (wsink)
                    wsink[qi * H + h] = 0.0;
                continue;
            }

            /* pass 2: unnormalised weights and the denominator */
            const double wz = sink ? exp(z - m) : 0.0;
            double L = wz;
            for (int64_t k = 0; k < K; ++k) {
                if (!use[k])
                    continue;
                s[k] = exp(s[k] - m);
                L += s[k];
            }

            /* pass 3: weighted sum of the value rows, divided by the denominator */
            for (int64_t d = 0; d < D; ++d)
                acc[d] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const int32_t j = list[k];
                if (!use[k])
                    continue;
                for (int64_t d = 0; d < D; ++d)
                    acc[d] += s[k] * widen_bf16(kvb[(int64_t)j * D + d]);
            }
            for (int64_t d = 0; d < D; ++d)
                oh[d] = acc[d] / L;

            if (w)
                for (int64_t k = 0; k < K; ++k)
                    w[(qi * H + h) * K + k] = use[k] ? s[k] / L : 0.0;
            if (wsink)
                wsink[qi * H + h] = wz / L;
        }
        free(s);
        free(acc);
        free(use);
    }
    return bad ? 1 : 0;
}

/* The default readings (sink not scaled, every occurrence counts). */
int oracle_sparse_attn_f64(const uint16_t *q, const uint16_t *kv, const float *sink,
                           const int32_t *idxs, float scale, int64_t B, int64_t T,
                           int64_t H, int64_t D, int64_t N, int64_t K, double *out,
                           double *w, double *wsink)
{
    return oracle_sparse_attn_f64_flags(q, kv, sink, idxs, scale, B, T, H, D, N, K, 0, out, w,
                                        wsink);
}
