/*
 * Plain fp64 per-token KDA recurrence (CPU).
 *
 * TEST INFRASTRUCTURE. Only tests/, __graft_entry__.smoke() and the cpu_baseline leg of
 * bench.py may load this library. It shares no code with the GPU library.
 *
 * Definition ("Noyaux KDA et FlashKDA", sections "Le conflit fondamental" and "Le rôle de la
 * décroissance bornée"; update order is a reading, see kda_oracle.py): per token t,
 *     S'  = diag(exp(max(g_t, g_min))) S
 *     S   = S' + beta_t k_t (v_t - S'^T k_t)^T
 *     o_t = scale * S^T q_t
 * Value columns of S never mix, so independent work units are (sequence, head, block of
 * value columns); OpenMP runs over them. Inputs are float32 (exact copies of the device
 * bits: bf16 and fp32 both upcast exactly); every operation is in double precision.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int kda_oracle_recurrence(const float* q, const float* k, const float* v, const float* g,
                          const float* beta, const float* h0, const int64_t* cu_seqlens,
                          int64_t n_seqs, int64_t total_tokens, int64_t H, int64_t dk,
                          int64_t dv, double scale, double g_min, int64_t col_block,
                          double* o, double* ht, int n_threads) {
  if (!q || !k || !v || !g || !beta || !cu_seqlens || !o || !ht) return -1;
  if (n_seqs < 0 || H <= 0 || dk <= 0 || dv <= 0 || col_block <= 0) return -1;
  if (cu_seqlens[0] != 0 || cu_seqlens[n_seqs] != total_tokens) return -1;
  for (int64_t n = 0; n < n_seqs; ++n)
    if (cu_seqlens[n + 1] < cu_seqlens[n]) return -1;

  const int64_t n_cb = (dv + col_block - 1) / col_block;
  const int64_t n_units = n_seqs * H * n_cb;
  int failed = 0;
#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif

#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)(dk * col_block));
    double* a = (double*)malloc(sizeof(double) * (size_t)dk);
    double* e = (double*)malloc(sizeof(double) * (size_t)col_block);
    if (!S || !a || !e) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t u = 0; u < n_units; ++u) {
      if (!S || !a || !e) continue;
      const int64_t cb = u % n_cb;
      const int64_t h = (u / n_cb) % H;
      const int64_t n = u / (n_cb * H);
      const int64_t c0 = cb * col_block;
      const int64_t nc = (c0 + col_block <= dv) ? col_block : dv - c0;

      /* entering state: rows = key channels, columns c0 .. c0 + nc - 1 */
      for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < nc; ++j)
          S[i * nc + j] = h0 ? (double)h0[((n * H + h) * dk + i) * dv + c0 + j] : 0.0;

      for (int64_t t = cu_seqlens[n]; t < cu_seqlens[n + 1]; ++t) {
        const float* kt = k + (t * H + h) * dk;
        const float* qt = q + (t * H + h) * dk;
        const float* gt = g + (t * H + h) * dk;
        const float* vt = v + (t * H + h) * dv + c0;
        const double bt = (double)beta[t * H + h];
        for (int64_t i = 0; i < dk; ++i) {
          double gi = (double)gt[i];
          a[i] = exp(gi > g_min ? gi : g_min);
        }
        /* decay the key rows, then the delta error e = v - S'^T k */
        for (int64_t j = 0; j < nc; ++j) e[j] = (double)vt[j];
        for (int64_t i = 0; i < dk; ++i) {
          const double ki = (double)kt[i];
          for (int64_t j = 0; j < nc; ++j) {
            S[i * nc + j] *= a[i];
            e[j] -= S[i * nc + j] * ki;
          }
        }
        /* beta-weighted correction, then the read-out */
        double* ot = o + (t * H + h) * dv + c0;
        for (int64_t j = 0; j < nc; ++j) ot[j] = 0.0;
        for (int64_t i = 0; i < dk; ++i) {
          const double bki = bt * (double)kt[i];
          const double qi = (double)qt[i];
          for (int64_t j = 0; j < nc; ++j) {
            S[i * nc + j] += bki * e[j];
            ot[j] += S[i * nc + j] * qi;
          }
        }
        for (int64_t j = 0; j < nc; ++j) ot[j] *= scale;
      }
      for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < nc; ++j)
          ht[((n * H + h) * dk + i) * dv + c0 + j] = S[i * nc + j];
    }
    free(S);
    free(a);
    free(e);
  }
  return failed ? -2 : 0;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int kda_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
