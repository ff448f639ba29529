/* Runs the fp64 oracle (oracle/kda_oracle.c, linked in) on a small packed batch with an
 * empty and a one-token sequence, several threads and a pair subset, for the
 * AddressSanitizer / UndefinedBehaviorSanitizer build.  Exits non-zero if a call fails or a
 * result is not finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int kda_oracle_run(int64_t num_seqs, const int64_t* cu_seqlens, int64_t H, int64_t dk,
                   int64_t dv, const float* q, const float* k, const float* v,
                   const float* log_alpha, const float* beta, const float* gate,
                   const float* S0, double floor_, double scale, double* out,
                   double* S_final, const int64_t* pairs, int64_t num_pairs, int nthreads);

static float urand(unsigned* s) {
    *s = *s * 1664525u + 1013904223u;
    return (float)((*s >> 8) & 0xffff) / 65536.0f;
}

int main(void) {
    const int64_t cu[] = {0, 37, 37, 38, 100};
    const int64_t N = 4, H = 2, dk = 16, dv = 8, T = 100;
    unsigned seed = 7;
    float* q = malloc(sizeof(float) * T * H * dk);
    float* k = malloc(sizeof(float) * T * H * dk);
    float* la = malloc(sizeof(float) * T * H * dk);
    float* v = malloc(sizeof(float) * T * H * dv);
    float* g = malloc(sizeof(float) * T * H * dv);
    float* b = malloc(sizeof(float) * T * H);
    float* S0 = malloc(sizeof(float) * N * H * dk * dv);
    double* out = malloc(sizeof(double) * T * H * dv);
    double* Sf = malloc(sizeof(double) * N * H * dk * dv);
    for (int64_t i = 0; i < T * H * dk; ++i) {
        q[i] = urand(&seed) - 0.5f; k[i] = urand(&seed) - 0.5f; la[i] = -urand(&seed);
    }
    for (int64_t i = 0; i < T * H * dv; ++i) { v[i] = urand(&seed) - 0.5f; g[i] = urand(&seed); }
    for (int64_t i = 0; i < T * H; ++i) b[i] = urand(&seed);
    for (int64_t i = 0; i < N * H * dk * dv; ++i) S0[i] = 0.1f * (urand(&seed) - 0.5f);
    int bad = 0;
    if (kda_oracle_run(N, cu, H, dk, dv, q, k, v, la, b, g, S0, -0.3, 0.9, out, Sf, NULL, 0, 3) <= 0) ++bad;
    for (int64_t i = 0; i < T * H * dv; ++i) bad += !isfinite(out[i]);
    for (int64_t i = 0; i < N * H * dk * dv; ++i) bad += !isfinite(Sf[i]);
    const int64_t pairs[] = {1, 6};
    if (kda_oracle_run(N, cu, H, dk, dv, q, k, v, la, b, g, NULL, -0.5, 1.0, out, Sf, pairs, 2, 2) <= 0) ++bad;
    if (kda_oracle_run(-1, cu, H, dk, dv, q, k, v, la, b, g, NULL, -0.5, 1.0, out, Sf, NULL, 0, 1) != -1) ++bad;
    free(q); free(k); free(la); free(v); free(g); free(b); free(S0); free(out); free(Sf);
    printf("oracle driver: %d problems\n", bad);
    return bad ? 1 : 0;
}
