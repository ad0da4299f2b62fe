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
 * Dropout (attn_oracle_dropout_fp64; slide 54 puts it between softmax and
 * ×V): p_j is replaced by p_j * keep_j / (1 - q), where q = thr / 256 is the
 * drop probability and keep_j = [byte(b, h, i, j) >= thr]. lse stays that of
 * the softmax before dropout. byte() is one byte of the counter-based
 * generator Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), written here from that definition:
 *   key  = (seed mod 2^32, seed / 2^32)
 *   ctr  = (i, 2 * (j / 32) + (j / 4) mod 2, b * H_q + h, 0)
 *   byte = bits 8t .. 8t+7 of output word w, w = (j / 8) mod 4, t = j mod 4.
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
    int dropout;           /* apply dropout with threshold drop_thr */
    uint32_t drop_thr;     /* 1 .. 255: drop when the element's byte < drop_thr */
    uint64_t seed;
    int64_t next; /* shared row counter */
    pthread_mutex_t lock;
} oracle_job;

/* One Philox4x32 round: two 32x32 -> 64-bit products, the high halves xored
 * with the other two words and the key, then the words permuted. */
static void philox_round(uint32_t c[4], const uint32_t k[2]) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k[0];
    const uint32_t n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k[1];
    const uint32_t n3 = (uint32_t)p0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
}

/* Philox4x32-10: ten rounds, the key advanced by the Weyl constants between
 * rounds. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
    uint32_t k[2] = {key[0], key[1]};
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k[0] += 0x9E3779B9u;
            k[1] += 0xBB67AE85u;
        }
        philox_round(c, k);
    }
    for (int w = 0; w < 4; ++w) out[w] = c[w];
}

/* keep_j / (1 - q) for element (b, h, i, j) */
static double keep_factor(const oracle_job *J, int64_t b, int64_t h, int64_t i, int64_t j) {
    const uint32_t key[2] = {(uint32_t)J->seed, (uint32_t)(J->seed >> 32)};
    const uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(2 * (j / 32) + (j / 4) % 2),
                             (uint32_t)(b * J->Hq + h), 0u};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    const uint32_t byte = (out[(j / 8) % 4] >> (8 * (j % 4))) & 0xFFu;
    if (byte < J->drop_thr) return 0.0;
    return 256.0 / (256.0 - (double)J->drop_thr);
}

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
        const double pd = J->dropout ? p * keep_factor(J, b, h, i, j) : p;
        const float *v = vbase + j * J->dv;
        for (int64_t c = 0; c < J->dv; ++c) out_o[c] += pd * (double)v[c];
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
static int run_oracle(const float *Q, const float *K, const float *V,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv,
                      int64_t dqk, int64_t dv, int causal, float scale,
                      const int64_t *rows, int64_t n_rows,
                      double *O, double *lse, int n_threads,
                      int dropout, uint32_t drop_thr, uint64_t seed) {
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
    J.dropout = dropout;
    J.drop_thr = drop_thr;
    J.seed = seed;
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

int attn_oracle_fp64(const float *Q, const float *K, const float *V,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv,
                     int64_t dqk, int64_t dv, int causal, float scale,
                     const int64_t *rows, int64_t n_rows,
                     double *O, double *lse, int n_threads) {
    return run_oracle(Q, K, V, B, Hq, Hkv, Nq, Nkv, dqk, dv, causal, scale, rows, n_rows, O,
                      lse, n_threads, 0, 0u, 0u);
}

/* As attn_oracle_fp64, with dropout at probability drop_thr / 256
 * (1 <= drop_thr <= 255); -1 for a threshold outside that range. */
int attn_oracle_dropout_fp64(const float *Q, const float *K, const float *V,
                             int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nkv,
                             int64_t dqk, int64_t dv, int causal, float scale,
                             const int64_t *rows, int64_t n_rows,
                             double *O, double *lse, int n_threads,
                             uint32_t drop_thr, uint64_t seed) {
    if (drop_thr < 1u || drop_thr > 255u) return -1;
    return run_oracle(Q, K, V, B, Hq, Hkv, Nq, Nkv, dqk, dv, causal, scale, rows, n_rows, O,
                      lse, n_threads, 1, drop_thr, seed);
}
