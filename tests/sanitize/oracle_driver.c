/* Runs the oracle's C entry point under AddressSanitizer / UBSan on edge
 * cases (empty lists, all unused, out-of-range entries, repeated indices,
 * no sink, weight outputs) and prints a checksum per case.  Test
 * infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_sparse_attn_f64_flags(const uint16_t *q, const uint16_t *kv, const float *sink,
                                 const int32_t *idxs, float scale, int64_t B, int64_t T,
                                 int64_t H, int64_t D, int64_t N, int64_t K, int flags,
                                 double *out, double *w, double *wsink);

static uint16_t bits_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

static int run(int64_t B, int64_t T, int64_t H, int64_t D, int64_t N, int64_t K, int flags,
               int with_sink, int with_weights, const int32_t *idxs, double *sum)
{
    uint16_t *q = malloc(sizeof(uint16_t) * (size_t)(B * T * H * D));
    uint16_t *kv = malloc(sizeof(uint16_t) * (size_t)(B * N * D + 1));
    float *sink = malloc(sizeof(float) * (size_t)H);
    double *out = malloc(sizeof(double) * (size_t)(B * T * H * D));
    double *w = with_weights ? malloc(sizeof(double) * (size_t)(B * T * H * (K > 0 ? K : 1))) : NULL;
    double *ws = with_weights ? malloc(sizeof(double) * (size_t)(B * T * H)) : NULL;
    for (int64_t i = 0; i < B * T * H * D; ++i) q[i] = bits_of((float)((i * 37 % 19) - 9) / 7.0f);
    for (int64_t i = 0; i < B * N * D; ++i) kv[i] = bits_of((float)((i * 23 % 17) - 8) / 5.0f);
    for (int64_t h = 0; h < H; ++h) sink[h] = (float)h / 3.0f - 1.0f;
    int rc = oracle_sparse_attn_f64_flags(q, kv, with_sink ? sink : NULL, idxs, 0.125f, B, T, H, D,
                                          N, K, flags, out, w, ws);
    double s = 0.0;
    if (rc == 0) {
        for (int64_t i = 0; i < B * T * H * D; ++i) s += out[i] * (double)((i % 7) + 1);
        if (w)
            for (int64_t i = 0; i < B * T * H * K; ++i) s += w[i];
    }
    *sum = s;
    free(q); free(kv); free(sink); free(out); free(w); free(ws);
    return rc;
}

int main(void)
{
    double s;
    int32_t full[2 * 3 * 5] = {0, 1, 2, 3, 4,  -1, 5, 6, -1, 2,  7, 7, 7, -1, -1,
                               3, 1, 4, 1, 5,  -1, -1, -1, -1, -1,  0, 9, 2, 8, 6};
    int32_t bad[2 * 3 * 5];
    memcpy(bad, full, sizeof bad);
    bad[7] = 10; /* N = 10: out of range */
    for (int flags = 0; flags < 4; ++flags)
        for (int sk = 0; sk < 2; ++sk)
            for (int wt = 0; wt < 2; ++wt) {
                int rc = run(2, 3, 4, 16, 10, 5, flags, sk, wt, full, &s);
                printf("full flags=%d sink=%d weights=%d rc=%d sum=%.17g\n", flags, sk, wt, rc, s);
            }
    printf("bad rc=%d\n", run(2, 3, 4, 16, 10, 5, 0, 1, 1, bad, &s));
    printf("empty rc=%d sum=%.17g\n", run(2, 3, 4, 16, 10, 0, 0, 1, 1, NULL, &s), s);
    printf("dims rc=%d\n", run(2, 3, 0, 16, 10, 5, 0, 1, 0, full, &s));
    return 0;
}
