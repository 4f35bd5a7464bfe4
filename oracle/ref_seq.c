/*
 * fp64 CPU oracle for the Mamba-2 SSD scan, plain C + OpenMP.
 * Test infrastructure only: it is the timed CPU baseline and the parity
 * checker for large shapes.  The HIP library never links or calls it.
 *
 * Follows the per-head recurrence of "Mamba-2架构与LaCT并行计算技术解析"
 * (jsqmd.com), §1.1:
 *     d_t  = softplus(d_raw_t + d_init)
 *     H_t  = exp(-d_t) * H_{t-1} + d_t * B_t^T X_t      (N x P, outer product)
 *     y_t  = C_t H_t
 * heads independent (§1.2), the time-flipped pass of §3.1 when reverse != 0
 * (y written back at each token's own position), and one sequence per
 * cu_seqlens segment ("长序列 Mamba 多卡训练，算力和显存怎么同时省", §三),
 * each starting from its own initial state.
 *
 * Inputs are float32 arrays holding exactly the values the GPU reads
 * (bf16 values widen to float32 exactly); all arithmetic is double.
 * Layouts (row-major): x [b,L,H,P], d_raw [b,L,H], B/C [b,L,G,N],
 * init [S,H,N,P] (may be NULL = zeros), y [b,L,H,P] double,
 * final [S,H,N,P] double (may be NULL).  S = b, or nseq when cu != NULL
 * (then b must be 1).  Head h uses group h*G/H.
 *
 * Parity unpinned: no -- tests/test_oracle_pins.py checks it against the
 * numpy oracle, which is itself pinned to closed forms and brute force.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double softplus_d(double z) {
    return (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z)));
}

int ssd_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Returns 0 on success, -1 on a bad argument, -2 when out of memory. */
int ssd_oracle_seq(const float* x, const float* d_raw, float d_init,
                   const float* B, const float* C, const float* init,
                   const int32_t* cu, int32_t nseq,
                   int32_t batch, int64_t L, int32_t H, int32_t P, int32_t N,
                   int32_t G, int32_t reverse, double* y, double* final_state)
{
    if (!x || !d_raw || !B || !C || !y || batch < 1 || L < 0 || H < 1 ||
        P < 1 || N < 1 || G < 1 || H % G != 0)
        return -1;
    if (cu && batch != 1) return -1;
    const int64_t S = cu ? nseq : batch;
    const int64_t units = S * H;
    const double dinit = (double)d_init;
    int err = 0;

    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t u = 0; u < units; ++u) {
        const int64_t i = u / H;
        const int32_t h = (int32_t)(u % H);
        const int32_t g = (int32_t)(((int64_t)h * G) / H);
        int64_t row = cu ? 0 : i;
        int64_t start = cu ? cu[i] : 0;
        int64_t len = cu ? (int64_t)cu[i + 1] - cu[i] : L;
        double* st = (double*)malloc(sizeof(double) * (size_t)N * P);
        if (!st) {
            #pragma omp atomic write
            err = -2;
            continue;
        }
        if (init) {
            const float* h0 = init + ((i * H + h) * (int64_t)N) * P;
            for (int64_t k = 0; k < (int64_t)N * P; ++k) st[k] = (double)h0[k];
        } else {
            memset(st, 0, sizeof(double) * (size_t)N * P);
        }
        for (int64_t j = 0; j < len; ++j) {
            const int64_t t = start + (reverse ? (len - 1 - j) : j);
            const int64_t tok = row * L + t;
            const double d = softplus_d((double)d_raw[tok * H + h] + dinit);
            const double decay = exp(-d);
            const float* xt = x + (tok * H + h) * (int64_t)P;
            const float* bt = B + (tok * G + g) * (int64_t)N;
            const float* ct = C + (tok * G + g) * (int64_t)N;
            double* yt = y + (tok * H + h) * (int64_t)P;
            for (int32_t p = 0; p < P; ++p) yt[p] = 0.0;
            for (int32_t n = 0; n < N; ++n) {
                const double wb = d * (double)bt[n];
                const double cn = (double)ct[n];
                double* srow = st + (int64_t)n * P;
                for (int32_t p = 0; p < P; ++p) {
                    srow[p] = decay * srow[p] + wb * (double)xt[p];
                    yt[p] += cn * srow[p];
                }
            }
        }
        if (final_state) {
            double* f = final_state + ((i * H + h) * (int64_t)N) * P;
            memcpy(f, st, sizeof(double) * (size_t)N * P);
        }
        free(st);
    }
    return err;
}
