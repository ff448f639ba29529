/*
 * kda_oracle.c -- CPU fp64 reference for the Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that GPU results are checked
 * against.  Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it; the product library never links or calls it.  It shares no code,
 * header, table or constant with the HIP path.
 *
 * What it computes (one independent recurrence per (sequence n, head h)):
 *   state S in R^{dk x dv}, rows = key channels, S <- S0 (or zeros).
 *   for each token t of the sequence, in order:
 *     1. a_c = exp(max(lambda_{t,c}, floor))            per key channel c
 *     2. S   <- Diag(a) S                              each row decays at its own rate
 *     3. w   =  S^T k_t                                 (reads the decayed state)
 *     4. S   <- S + beta_t k_t (v_t - w)^T             = (I - beta k k^T) S + beta k v^T:
 *                                                      row along k keeps (1-beta) of the
 *                                                      old value and takes beta of v
 *     5. o_t =  g_t (elementwise) (S^T (scale q_t))   readout of the updated state
 *
 * Sources (page title, section/figure):
 *   - "Kimi-K3 为什么这么强？" (xiaored5.github.io), §① KDA, part ② and the
 *     "一次 KDA 更新" figure caption: per-row forgetting, then the current key's row
 *     is weakened by beta (keeps 1-beta, not cleared), then the new value is written
 *     so the row becomes an interpolation of old and new; fixed-size table updated in
 *     place.  Per-channel Diag(alpha) instead of a scalar gate.
 *   - "Kimi K3 深度拆解" (idataagent.com), 突破一 KDA: per-channel diagonal decay on a
 *     Diagonal-Plus-Low-Rank transition, i.e. (I - beta k k^T) Diag(alpha).
 *   - Digest of "Kimi K3: Open Frontier Intelligence" (fupanwang.com), section
 *     "KDA：百万上下文先要过「数值 算子」这一关": lower-bounded per-step log-decay
 *     (the constant is lost in the page text; it is a parameter here), and the output
 *     gate as an input-dependent channel-wise switch on the recurrence output (the
 *     gate values g are inputs; the projection producing them is outside the op).
 *   - Readout after the write (o_t = S_t^T q_t) is the plainest reading; the pages do
 *     not fix the order of readout and write.
 *
 * Inputs are float32 (bf16 values widen to float32 exactly); all arithmetic is double.
 * Layout: packed tokens, q/k/log_alpha [T_total, H, dk], v/g/out [T_total, H, dv],
 * beta [T_total, H], states [N, H, dk, dv] row-major.  Sequence n owns tokens
 * cu_seqlens[n] .. cu_seqlens[n+1]-1.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

typedef struct {
    int64_t num_seqs;
    const int64_t* cu_seqlens;
    int64_t H, dk, dv;
    const float *q, *k, *v, *log_alpha, *beta, *gate;
    const float* S0;   /* may be NULL: zero initial state */
    double floor_, scale;
    double* out;       /* may be NULL: outputs not wanted */
    double* S_final;   /* may be NULL */
    const int64_t* pairs; /* optional list of (n*H + h) to run; NULL = all */
    int64_t num_pairs;
    int64_t next;      /* work counter, guarded by mu */
    pthread_mutex_t mu;
} job_t;

/* One (sequence, head) recurrence, token by token. */
static void run_pair(const job_t* J, int64_t n, int64_t h, double* S, double* a, double* w,
                     double* u) {
    const int64_t H = J->H, dk = J->dk, dv = J->dv;
    const int64_t t0 = J->cu_seqlens[n], t1 = J->cu_seqlens[n + 1];
    const float* S0 = J->S0 ? J->S0 + (n * H + h) * dk * dv : NULL;
    for (int64_t i = 0; i < dk * dv; ++i) S[i] = S0 ? (double)S0[i] : 0.0;

    for (int64_t t = t0; t < t1; ++t) {
        const float* q = J->q + (t * H + h) * dk;
        const float* k = J->k + (t * H + h) * dk;
        const float* la = J->log_alpha + (t * H + h) * dk;
        const float* v = J->v + (t * H + h) * dv;
        const float* g = J->gate + (t * H + h) * dv;
        const double beta = (double)J->beta[t * H + h];

        /* 1-2. per-channel decay of each row */
        for (int64_t c = 0; c < dk; ++c) {
            double l = (double)la[c];
            if (l < J->floor_) l = J->floor_;
            a[c] = exp(l);
        }
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < dv; ++j) S[c * dv + j] *= a[c];

        /* 3. what the decayed state currently returns for key k */
        for (int64_t j = 0; j < dv; ++j) w[j] = 0.0;
        for (int64_t c = 0; c < dk; ++c) {
            const double kc = (double)k[c];
            for (int64_t j = 0; j < dv; ++j) w[j] += S[c * dv + j] * kc;
        }

        /* 4. delta-rule erase/write along k */
        for (int64_t j = 0; j < dv; ++j) u[j] = beta * ((double)v[j] - w[j]);
        for (int64_t c = 0; c < dk; ++c) {
            const double kc = (double)k[c];
            for (int64_t j = 0; j < dv; ++j) S[c * dv + j] += kc * u[j];
        }

        /* 5. gated readout of the updated state */
        if (J->out) {
            double* o = J->out + (t * H + h) * dv;
            for (int64_t j = 0; j < dv; ++j) w[j] = 0.0;
            for (int64_t c = 0; c < dk; ++c) {
                const double qc = J->scale * (double)q[c];
                for (int64_t j = 0; j < dv; ++j) w[j] += S[c * dv + j] * qc;
            }
            for (int64_t j = 0; j < dv; ++j) o[j] = (double)g[j] * w[j];
        }
    }
    if (J->S_final) {
        double* Sf = J->S_final + (n * H + h) * dk * dv;
        memcpy(Sf, S, sizeof(double) * dk * dv);
    }
}

static void* worker(void* arg) {
    job_t* J = (job_t*)arg;
    double* S = (double*)malloc(sizeof(double) * J->dk * J->dv);
    double* a = (double*)malloc(sizeof(double) * J->dk);
    double* w = (double*)malloc(sizeof(double) * J->dv);
    double* u = (double*)malloc(sizeof(double) * J->dv);
    const int64_t total = J->pairs ? J->num_pairs : J->num_seqs * J->H;
    for (;;) {
        pthread_mutex_lock(&J->mu);
        const int64_t i = J->next++;
        pthread_mutex_unlock(&J->mu);
        if (i >= total) break;
        const int64_t p = J->pairs ? J->pairs[i] : i;
        run_pair(J, p / J->H, p % J->H, S, a, w, u);
    }
    free(S); free(a); free(w); free(u);
    return NULL;
}

/*
 * Run the recurrence for every (sequence, head) pair, or for the listed pairs only
 * (pairs[i] = n*H + h).  nthreads <= 0 uses every online CPU.  Returns the number of
 * threads used, or -1 on bad arguments.
 */
int kda_oracle_run(int64_t num_seqs, const int64_t* cu_seqlens, int64_t H, int64_t dk,
                   int64_t dv, const float* q, const float* k, const float* v,
                   const float* log_alpha, const float* beta, const float* gate,
                   const float* S0, double floor_, double scale, double* out,
                   double* S_final, const int64_t* pairs, int64_t num_pairs, int nthreads) {
    if (num_seqs < 0 || H < 1 || dk < 1 || dv < 1 || !cu_seqlens) return -1;
    if (!q || !k || !v || !log_alpha || !beta || !gate) return -1;
    job_t J;
    J.num_seqs = num_seqs; J.cu_seqlens = cu_seqlens; J.H = H; J.dk = dk; J.dv = dv;
    J.q = q; J.k = k; J.v = v; J.log_alpha = log_alpha; J.beta = beta; J.gate = gate;
    J.S0 = S0; J.floor_ = floor_; J.scale = scale; J.out = out; J.S_final = S_final;
    J.pairs = pairs; J.num_pairs = num_pairs; J.next = 0;
    pthread_mutex_init(&J.mu, NULL);
    if (nthreads <= 0) nthreads = (int)sysconf(_SC_NPROCESSORS_ONLN);
    if (nthreads < 1) nthreads = 1;
    const int64_t total = pairs ? num_pairs : num_seqs * H;
    if (nthreads > total) nthreads = total > 0 ? (int)total : 1;
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nthreads);
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, worker, &J);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
    free(th);
    pthread_mutex_destroy(&J.mu);
    return nthreads;
}
