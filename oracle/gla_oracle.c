/*
 * CPU oracle: the key-only gated linear attention recurrence, token by token,
 * in double precision. TEST INFRASTRUCTURE ONLY: this code checks the GPU
 * path and is never part of it.
 *
 * What it computes (GTR project page, "How GTR Works": key-only gated linear
 * attention along one scan order; ai.info summary of GTR, "Methodology in
 * Plain English": a running summary state in which only the key-side
 * dimensions decay, with the value-side decay fixed at one, and a zero
 * initial state for the deployed operator). The pages print no equation; the
 * recurrence is the gated linear attention form of the GLA paper they cite
 * ("Gated Linear Attention Transformers with Hardware-Efficient Training",
 * mlsanity reference list), restricted to a key-side gate:
 *
 *     S_0 = 0                                     S_t in R^{dk x dv}
 *     S_t = diag(exp(g_t)) S_{t-1} + k_t^T v_t    (decay, then add token t)
 *     o_t = q_t S_t                               (output includes token t)
 *
 * Inputs are already in scan order. Layout of every array: [B][T][H][D]
 * contiguous, D = dk for q, k, g and D = dv for v, o.
 *
 * Carried state (ai.info summary of GTR, "Future Directions": carrying the
 * state across frames as the natural extension of the zero-state operator):
 * gla_oracle_recurrence_state starts from a given S_0 instead of zero and can
 * hand back the state after the last token, S_T. Both are [B][H][dk][dv];
 * a NULL s0 means S_0 = 0 and a NULL s_final skips the hand-back.
 *
 * Each value column e of S evolves on its own:
 *     S[:, e] <- exp(g_t) * S[:, e] + k_t * v_t[e],   o_t[e] = q_t . S[:, e]
 * so the loop runs one independent recurrence per (b, h, e). OpenMP spreads
 * those columns over threads; nothing else is reordered.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int gla_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Returns 0 on success, -1 on a bad argument. */
int gla_oracle_recurrence_state(const double* q, const double* k, const double* v,
                                const double* g, const double* s0, double* o,
                                double* s_final, int64_t B, int64_t T, int64_t H,
                                int64_t dk, int64_t dv) {
  if (!q || !k || !v || !g || !o || B < 0 || T < 0 || H < 0 || dk <= 0 ||
      dv <= 0)
    return -1;
  const int64_t ncol = B * H * dv;
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)dk);
#pragma omp for schedule(static)
    for (int64_t c = 0; c < ncol; ++c) {
      const int64_t e = c % dv;
      const int64_t h = (c / dv) % H;
      const int64_t b = c / (dv * H);
      const int64_t st = (b * H + h) * dk * dv; /* state [b][h][.][.] */
      for (int64_t d = 0; d < dk; ++d) S[d] = s0 ? s0[st + d * dv + e] : 0.0;
      for (int64_t t = 0; t < T; ++t) {
        const int64_t rk = ((b * T + t) * H + h) * dk; /* q, k, g row */
        const int64_t rv = ((b * T + t) * H + h) * dv; /* v, o row */
        const double ve = v[rv + e];
        double acc = 0.0;
        for (int64_t d = 0; d < dk; ++d) {
          S[d] = exp(g[rk + d]) * S[d] + k[rk + d] * ve;
          acc += q[rk + d] * S[d];
        }
        o[rv + e] = acc;
      }
      if (s_final)
        for (int64_t d = 0; d < dk; ++d) s_final[st + d * dv + e] = S[d];
    }
    free(S);
  }
  return 0;
}

/* The zero-initial-state forward of the deployed operator. */
int gla_oracle_recurrence(const double* q, const double* k, const double* v,
                          const double* g, double* o, int64_t B, int64_t T,
                          int64_t H, int64_t dk, int64_t dv) {
  return gla_oracle_recurrence_state(q, k, v, g, NULL, o, NULL, B, T, H, dk, dv);
}
