/*
 * fp64 CPU oracle for the backward pass of the Mamba-2 SSD scan, plain C +
 * OpenMP.  Test infrastructure only: it checks the HIP library's gradients
 * at sizes the numpy adjoint oracle (ssd_oracle_bwd.py) cannot reach.  The
 * HIP library never links or calls it.
 *
 * It computes the same thing as ssd_oracle_bwd.scan_core_bwd: the adjoint
 * of the recurrence of "Mamba-2架构与LaCT并行计算技术解析" (jsqmd.com), §1.1,
 *     d_t = softplus(d_raw_t + d_init),  H_t = e^{-d_t} H_{t-1} + d_t B_t^T x_t,
 *     y_t = C_t H_t,
 * for the loss L = sum_t <dy_t, y_t> + <d_final, H_last> per sequence and
 * head, walked from the last processed token back to the first, with
 * G_t = dL/dH_t:
 *     G_t   = C_t^T dy_t + e^{-d_{t+1}} G_{t+1}      (G_last adds d_final)
 *     dx_t  = d_t B_t G_t
 *     dB_t  = d_t G_t x_t^T                          (summed over heads)
 *     dC_t  = H_t dy_t                               (summed over heads)
 *     dd_t  = < G_t, -e^{-d_t} H_{t-1} + B_t^T x_t >
 *     d d_raw = dd * sigmoid(d_raw + d_init),  d d_init = sum of d d_raw,
 *     dinit = e^{-d_first} G_first.
 * The pages name this pass (the Mamba context-parallel backward of
 * "揭秘MindSpeed-LLM多潜在注意力（MLA）与Mamba上下文并行实现原理", §三.2)
 * without writing it out; it is the derivative of the map above.
 *
 * Work split.  A state column (fixed headdim index p) evolves on its own:
 * H_t[:, p] and G_t[:, p] depend only on column p of x, dy, init and
 * d_final.  So the units are (sequence, head, block of columns), run in
 * parallel; the sums over columns (dd) and over heads (dB, dC) are
 * per-unit partials added afterwards in a fixed order (heads, then column
 * blocks, ascending), so the result does not depend on the thread count.
 * A unit walks its sequence forward once storing the state every Q tokens
 * (Q about sqrt(length)), then walks the segments from last to first,
 * recomputing each segment's states from its checkpoint before stepping
 * back through it.  All arithmetic is double; inputs are float32 arrays
 * (bf16 values widen exactly).
 *
 * Layouts (row-major): x, dy [b,L,H,P]; d_raw [b,L,H]; B, C [b,L,G,N];
 * init, d_final [S,H,N,P] (NULL = zeros); outputs dx [b,L,H,P], dd_raw
 * [b,L,H], dB, dC [b,L,G,N], dinit [S,H,N,P], dd_init one double; any
 * output may be NULL to skip it (dd_init needs dd_raw's partials, computed
 * whenever either is asked for).  Outputs at tokens outside every segment
 * are left as they are.  S = b, or nseq when cu != NULL (then b == 1).
 *
 * Parity unpinned: no -- tests/test_oracle_bwd_pins.py checks it against
 * the numpy adjoint oracle, which is pinned by central finite differences
 * of the forward oracle.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double softplus_b(double z) { return (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z))); }

static double sigmoid_b(double z) {
    const double e = exp(-fabs(z));
    return z >= 0.0 ? 1.0 / (1.0 + e) : e / (1.0 + e);
}

typedef struct {
    double* dd;  /* [len] sum over the unit's columns of dd_t      */
    double* dB;  /* [len][N] sum over the unit's columns of dB_t   */
    double* dC;  /* [len][N]                                        */
    int err;
} Partial;

/* One unit: sequence segment (row, start, len), head h, columns [p0, p1). */
static void unit_bwd(const float* x, const double* dseq, const float* B, const float* C,
                     const float* init, const float* dy, const float* dfin, int64_t row,
                     int64_t start, int64_t len, int64_t iseq, int32_t h, int32_t p0, int32_t p1,
                     int64_t L, int32_t H, int32_t P, int32_t N, int32_t G, int32_t reverse,
                     double* dx, double* dinit, Partial* out) {
    /* (an empty segment walks nothing: its initial-state gradient is d_final) */
    const int32_t np = p1 - p0;
    const int32_t g = (int32_t)(((int64_t)h * G) / H);
    const int64_t SZ = (int64_t)N * np;
    int64_t Q = (int64_t)ceil(sqrt((double)(len > 0 ? len : 1)));
    if (Q < 16) Q = 16;
    const int64_t nseg = (len + Q - 1) / Q;
    double* ck = (double*)malloc(sizeof(double) * (size_t)((nseg > 0 ? nseg : 1) * SZ));
    double* seg = (double*)malloc(sizeof(double) * (size_t)(Q * SZ));
    double* S = (double*)malloc(sizeof(double) * (size_t)SZ);
    double* Gs = (double*)malloc(sizeof(double) * (size_t)SZ);
    if (!ck || !seg || !S || !Gs) {
        out->err = -2;
        free(ck); free(seg); free(S); free(Gs);
        return;
    }
    /* token index (b*L + t) of the j-th processed token */
#define TOK(j) (row * L + start + (reverse ? (len - 1 - (j)) : (j)))
    const double* dstep = dseq; /* d_t of the j-th processed token: dstep[j] */
    /* one step H <- e^{-d} H + d B^T x over the unit's columns */
#define STEP(Sp, j)                                                         \
    do {                                                                    \
        const int64_t tk_ = TOK(j);                                         \
        const double d_ = dstep[j], e_ = exp(-d_);                          \
        const float* xt_ = x + (tk_ * H + h) * (int64_t)P + p0;            \
        const float* bt_ = B + (tk_ * G + g) * (int64_t)N;                 \
        for (int32_t n_ = 0; n_ < N; ++n_) {                                \
            const double wb_ = d_ * (double)bt_[n_];                        \
            double* r_ = (Sp) + (int64_t)n_ * np;                           \
            for (int32_t q_ = 0; q_ < np; ++q_) r_[q_] = e_ * r_[q_] + wb_ * (double)xt_[q_]; \
        }                                                                   \
    } while (0)

    /* forward walk, checkpoint before every segment */
    for (int32_t n = 0; n < N; ++n)
        for (int32_t q = 0; q < np; ++q)
            S[(int64_t)n * np + q] =
                init ? (double)init[((iseq * H + h) * (int64_t)N + n) * P + p0 + q] : 0.0;
    for (int64_t j = 0; j < len; ++j) {
        if (j % Q == 0) memcpy(ck + (j / Q) * SZ, S, sizeof(double) * (size_t)SZ);
        STEP(S, j);
    }
    /* the gradient of the state after the last token */
    for (int32_t n = 0; n < N; ++n)
        for (int32_t q = 0; q < np; ++q)
            Gs[(int64_t)n * np + q] =
                dfin ? (double)dfin[((iseq * H + h) * (int64_t)N + n) * P + p0 + q] : 0.0;
    for (int64_t k = nseg - 1; k >= 0; --k) {
        const int64_t j0 = k * Q, j1 = (j0 + Q < len) ? j0 + Q : len;
        memcpy(S, ck + k * SZ, sizeof(double) * (size_t)SZ);
        for (int64_t j = j0; j < j1; ++j) {
            STEP(S, j);
            memcpy(seg + (j - j0) * SZ, S, sizeof(double) * (size_t)SZ);
        }
        for (int64_t j = j1 - 1; j >= j0; --j) {
            const int64_t tk = TOK(j);
            const double d = dstep[j], e = exp(-d);
            const float* xt = x + (tk * H + h) * (int64_t)P + p0;
            const float* dyt = dy + (tk * H + h) * (int64_t)P + p0;
            const float* bt = B + (tk * G + g) * (int64_t)N;
            const float* ct = C + (tk * G + g) * (int64_t)N;
            const double* Hj = seg + (j - j0) * SZ;                     /* H_t     */
            const double* Hp = j > j0 ? seg + (j - j0 - 1) * SZ : ck + k * SZ; /* H_{t-1} */
            /* G_t = C_t^T dy_t + (e^{-d_{t+1}} G_{t+1}, already in Gs) */
            for (int32_t n = 0; n < N; ++n) {
                const double cn = (double)ct[n];
                double* r = Gs + (int64_t)n * np;
                for (int32_t q = 0; q < np; ++q) r[q] += cn * (double)dyt[q];
            }
            if (dx) {
                double* dxt = dx + (tk * H + h) * (int64_t)P + p0;
                for (int32_t q = 0; q < np; ++q) {
                    double acc = 0.0;
                    for (int32_t n = 0; n < N; ++n) acc += (double)bt[n] * Gs[(int64_t)n * np + q];
                    dxt[q] = d * acc;
                }
            }
            if (out->dB) {
                double* o = out->dB + j * (int64_t)N;
                for (int32_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int32_t q = 0; q < np; ++q) acc += Gs[(int64_t)n * np + q] * (double)xt[q];
                    o[n] = d * acc;
                }
            }
            if (out->dC) {
                double* o = out->dC + j * (int64_t)N;
                for (int32_t n = 0; n < N; ++n) {
                    double acc = 0.0;
                    for (int32_t q = 0; q < np; ++q) acc += Hj[(int64_t)n * np + q] * (double)dyt[q];
                    o[n] = acc;
                }
            }
            if (out->dd) {
                double acc = 0.0;
                for (int32_t n = 0; n < N; ++n) {
                    const double bn = (double)bt[n];
                    for (int32_t q = 0; q < np; ++q) {
                        const int64_t o = (int64_t)n * np + q;
                        acc += Gs[o] * (-e * Hp[o] + bn * (double)xt[q]);
                    }
                }
                out->dd[j] = acc;
            }
            /* on to G_{t-1}'s carried part */
            for (int64_t o = 0; o < SZ; ++o) Gs[o] *= e;
        }
    }
    if (dinit) {
        for (int32_t n = 0; n < N; ++n)
            for (int32_t q = 0; q < np; ++q)
                dinit[((iseq * H + h) * (int64_t)N + n) * P + p0 + q] = Gs[(int64_t)n * np + q];
    }
#undef STEP
#undef TOK
    free(ck); free(seg); free(S); free(Gs);
}

/* Returns 0 on success, -1 on a bad argument, -2 when out of memory. */
int ssd_oracle_bwd(const float* x, const float* d_raw, float d_init, const float* B,
                   const float* C, const float* init, const float* dy, const float* d_final,
                   const int32_t* cu, int32_t nseq, int32_t batch, int64_t L, int32_t H,
                   int32_t P, int32_t N, int32_t G, int32_t reverse, int32_t pblk, double* dx,
                   double* dd_raw, double* dB, double* dC, double* dinit, double* dd_init) {
    if (!x || !d_raw || !B || !C || !dy || batch < 1 || L < 0 || H < 1 || P < 1 || N < 1 ||
        G < 1 || H % G != 0 || pblk < 1)
        return -1;
    if (cu && batch != 1) return -1;
    const int64_t S = cu ? nseq : batch;
    const double dinit_d = (double)d_init;
    const int32_t nblk = (P + pblk - 1) / pblk;
    const int want_dd = dd_raw || dd_init;
    double ddsum = 0.0;
    int err = 0;
    for (int64_t i = 0; i < S && !err; ++i) {
        const int64_t row = cu ? 0 : i;
        const int64_t start = cu ? cu[i] : 0;
        const int64_t len = cu ? (int64_t)cu[i + 1] - cu[i] : L;
        if (len < 0 || start < 0 || start + len > L) return -1;
        /* d_t per head in processing order */
        double* dseq = (double*)malloc(sizeof(double) * (size_t)((len > 0 ? len : 1) * H));
        const int64_t units = (int64_t)H * nblk;
        Partial* part = (Partial*)calloc((size_t)units, sizeof(Partial));
        if (!dseq || !part) {
            free(dseq); free(part);
            return -2;
        }
        for (int32_t h = 0; h < H; ++h)
            for (int64_t j = 0; j < len; ++j) {
                const int64_t tk = row * L + start + (reverse ? (len - 1 - j) : j);
                dseq[(int64_t)h * len + j] = softplus_b((double)d_raw[tk * H + h] + dinit_d);
            }
        #pragma omp parallel for schedule(dynamic, 1)
        for (int64_t u = 0; u < units; ++u) {
            const int32_t h = (int32_t)(u / nblk), bk = (int32_t)(u % nblk);
            const int32_t p0 = bk * pblk, p1 = (p0 + pblk < P) ? p0 + pblk : P;
            Partial* pt = &part[u];
            const size_t n1 = (size_t)(len > 0 ? len : 1);
            if (want_dd) pt->dd = (double*)calloc(n1, sizeof(double));
            if (dB) pt->dB = (double*)calloc(n1 * (size_t)N, sizeof(double));
            if (dC) pt->dC = (double*)calloc(n1 * (size_t)N, sizeof(double));
            if ((want_dd && !pt->dd) || (dB && !pt->dB) || (dC && !pt->dC)) {
                pt->err = -2;
                continue;
            }
            unit_bwd(x, dseq + (int64_t)h * len, B, C, init, dy, d_final, row, start, len, i, h,
                     p0, p1, L, H, P, N, G, reverse, dx, dinit, pt);
        }
        for (int64_t u = 0; u < units; ++u)
            if (part[u].err) err = part[u].err;
        if (!err) {
            /* fixed-order sums: heads ascending, then column blocks */
            for (int64_t j = 0; j < len; ++j) {
                const int64_t tk = row * L + start + (reverse ? (len - 1 - j) : j);
                for (int32_t h = 0; h < H; ++h) {
                    if (!want_dd) break;
                    double acc = 0.0;
                    for (int32_t bk = 0; bk < nblk; ++bk) acc += part[(int64_t)h * nblk + bk].dd[j];
                    const double v = acc * sigmoid_b((double)d_raw[tk * H + h] + dinit_d);
                    if (dd_raw) dd_raw[tk * H + h] = v;
                    ddsum += v;
                }
                for (int32_t gg = 0; gg < G; ++gg) {
                    for (int32_t n = 0; n < N; ++n) {
                        double ab = 0.0, ac = 0.0;
                        for (int32_t h = 0; h < H; ++h) {
                            if ((int32_t)(((int64_t)h * G) / H) != gg) continue;
                            for (int32_t bk = 0; bk < nblk; ++bk) {
                                const Partial* pt = &part[(int64_t)h * nblk + bk];
                                if (dB) ab += pt->dB[j * (int64_t)N + n];
                                if (dC) ac += pt->dC[j * (int64_t)N + n];
                            }
                        }
                        if (dB) dB[(tk * G + gg) * (int64_t)N + n] = ab;
                        if (dC) dC[(tk * G + gg) * (int64_t)N + n] = ac;
                    }
                }
            }
        }
        for (int64_t u = 0; u < units; ++u) {
            free(part[u].dd); free(part[u].dB); free(part[u].dC);
        }
        free(part);
        free(dseq);
    }
    if (!err && dd_init) *dd_init = ddsum;
    return err;
}
