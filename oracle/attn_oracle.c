/*
 * Attention forward oracle: plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call this code;
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * load it. It shares no code, header, table or helper with the HIP library.
 *
 * What it computes, per output row (b, h, i), is the plain definition of the
 * attention forward pass as the pages describe it:
 *   - "CS149 L11: Programming Specialized Hardware" (quidproquo.cc), section 5,
 *     slide 54: FlashAttention is the chain Q·Kᵀ -> mask -> softmax -> (dropout)
 *     -> ×V; section 6 lists the decoder's attention as Q·Kᵀ, scale, mask,
 *     softmax, ×V.
 *   - same page, section 5 "Programming with parallel patterns", slide 48:
 *     softmax is Map(exp) -> Reduce(+) -> Zip(/).
 *   - "Distilling a 4.5 hour CUDA talk" (levidiamode.com), section 7: the
 *     kernel keeps a running max and normalizer; that online form is an exact
 *     reordering of the same softmax, so the oracle uses the two-pass form.
 *
 * Steps, for row (b, h, i), kv head g = h / (H_q / H_kv):
 *   1. s_j = scale * sum_c Q[b,h,i,c] * K[b,g,j,c]   for every key j that is
 *      not masked (causal: j <= i, top-left aligned; dropout probability 0);
 *   2. m   = max_j s_j (a shift that cancels in the ratio; it only keeps
 *      exp() in range);
 *   3. e_j = exp(s_j - m)                 (Map(exp))
 *   4. l   = sum_j e_j                    (Reduce(+))
 *   5. p_j = e_j / l                      (Zip(/))
 *   6. O[b,h,i,:] = sum_j p_j * V[b,g,j,:]
 *   7. lse[b,h,i] = m + ln(l)  (natural log of sum_j exp(s_j); the pages only
 *      name "running max and normalizer", this is the reading used).
 *
 * Inputs are fp32 arrays (bf16 values widen to fp32 exactly), contiguous in
 * [B, H, N, d] order. All arithmetic is fp64. Rows are spread over POSIX
 * threads; nothing else is tuned.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <unistd.h>

typedef struct {
    const float *Q, *K, *V;
    int64_t B, Hq, Hkv, Nq, Nkv, dqk, dv;
    int causal;
    double scale;
    const int64_t *rows; /* n_rows x 3 (b, h, i) or NULL for every row */
    int64_t n_rows;
    double *O, *lse;
    int64_t next; /* shared row counter */
    pthread_mutex_t lock;
} oracle_job;

static void one_row(const oracle_job *J, int64_t b, int64_t h, int64_t i,
                    double *s, double *out_o, double *out_lse) {
    const int64_t group = J->Hq / J->Hkv;
    const int64_t g = h / group;
    const float *q = J->Q + ((b * J->Hq + h) * J->Nq + i) * J->dqk;
    const float *kbase = J->K + (b * J->Hkv + g) * J->Nkv * J->dqk;
    const float *vbase = J->V + (b * J->Hkv + g) * J->Nkv * J->dv;
    const int64_t n_keys = J->causal ? (i + 1 < J->Nkv ? i + 1 : J->Nkv) : J->Nkv;

    /* step 1 (scores) and step 2 (max) */
    double m = -INFINITY;
    for (int64_t j = 0; j < n_keys; ++j) {
        const float *k = kbase + j * J->dqk;
        double dot = 0.0;
        for (int64_t c = 0; c < J->dqk; ++c) dot += (double)q[c] * (double)k[c];
        s[j] = J->scale * dot;
        if (s[j] > m) m = s[j];
    }
    /* steps 3-4: Map(exp), Reduce(+) */
    double l = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        s[j] = exp(s[j] - m);
        l += s[j];
    }
    /* steps 5-6: Zip(/), then the weighted sum of value rows */
    for (int64_t c = 0; c < J->dv; ++c) out_o[c] = 0.0;
    for (int64_t j = 0; j < n_keys; ++j) {
        const double p = s[j] / l;
        const float *v = vbase + j * J->dv;
        for (int64_t c = 0; c < J->dv; ++c) out_o[c] += p * (double)v[c];
    }
    /* step 7 */
    *out_lse = m + log(l);
}

static void *worker(void *arg) {
    oracle_job *J = (oracle_job *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)J->Nkv);
    if (!s) return (void *)1;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        const int64_t r = J->next;
        J->next += 1;
        pthread_mutex_unlock(&J->lock);
        if (r >= J->n_rows) break;
        int64_t b, h, i;
        if (J->rows) {
            b = J->rows[3 * r + 0];
            h = J->rows[3 * r + 1];
            i = J->rows[3 * r + 2];
        } else {
            i = r % J->Nq;
            h = (r / J->Nq) % J->Hq;
            b = r / (J->Nq * J->Hq);
        }
        one_row(J, b, h, i, s, J->O + r * J->dv, J->lse + r);
    }
    free(s);
    return NULL;
}

/*
 * Returns the number of threads used (> 0) on success, or a negative value:
 *   -1 invalid sizes, -2 a requested row outside the tensors, -3 out of memory.
 * O receives n_rows x dv doubles and lse n_rows doubles, in the order of
 * `rows` (or, with rows == NULL, every (b, h, i) in row-major order, so that
 * n_rows must be B*H_q*N_q).
 */
int attn_oracle_fp64(const float *Q, const float *K, const float *V,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv,
                     int64_t dqk, int64_t dv, int causal, float scale,
                     const int64_t *rows, int64_t n_rows,
                     double *O, double *lse, int n_threads) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nkv < 1 || dqk < 1 || dv < 1) return -1;
    if (Hq % Hkv != 0) return -1;
    if (causal && Nq != Nkv) return -1;
    if (!rows && n_rows != B * Hq * Nq) return -1;
    if (rows) {
        for (int64_t r = 0; r < n_rows; ++r) {
            const int64_t b = rows[3 * r], h = rows[3 * r + 1], i = rows[3 * r + 2];
            if (b < 0 || b >= B || h < 0 || h >= Hq || i < 0 || i >= Nq) return -2;
        }
    }
    oracle_job J;
    J.Q = Q; J.K = K; J.V = V;
    J.B = B; J.Hq = Hq; J.Hkv = Hkv; J.Nq = Nq; J.Nkv = Nkv; J.dqk = dqk; J.dv = dv;
    J.causal = causal;
    J.scale = (double)scale;
    J.rows = rows; J.n_rows = n_rows;
    J.O = O; J.lse = lse;
    J.next = 0;
    pthread_mutex_init(&J.lock, NULL);

    if (n_threads <= 0) n_threads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (n_threads < 1) n_threads = 1;
    if ((int64_t)n_threads > n_rows) n_threads = (int)(n_rows > 0 ? n_rows : 1);
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)n_threads);
    if (!tid) return -3;
    int started = 0, failed = 0;
    for (int t = 0; t < n_threads; ++t) {
        if (pthread_create(&tid[t], NULL, worker, &J) != 0) break;
        ++started;
    }
    if (started == 0) { /* run inline */
        if (worker(&J) != NULL) failed = 1;
        started = 1;
    } else {
        for (int t = 0; t < started; ++t) {
            void *rv = NULL;
            pthread_join(tid[t], &rv);
            if (rv != NULL) failed = 1;
        }
    }
    free(tid);
    pthread_mutex_destroy(&J.lock);
    return failed ? -3 : started;
}
