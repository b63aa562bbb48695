/*
 * CPU baseline driver (TEST INFRASTRUCTURE, like the rest of oracle/): the
 * oracle's layer, unchanged, run over tokens on all host cores with an
 * OpenMP parallel for.  Each token is an independent orc_layer call of one
 * token (the layer's output rows do not interact), so the result equals one
 * orc_layer call over all tokens.  Only the benchmark's CPU-baseline leg
 * loads it; it is built into its own library next to the oracle's.
 */
#include <omp.h>
#include <stdint.h>

int64_t orc_layer(const uint8_t *pg, const float *sg, const uint8_t *pu,
                  const float *su, const uint8_t *pd, const float *sd,
                  int64_t experts, int64_t hidden, int64_t inter, int64_t gs,
                  const double *x, int64_t tokens, const int32_t *ids,
                  const float *w, int64_t k, double *out);

/* Threads the OpenMP runtime uses (omp_get_max_threads). */
int orc_omp_threads(void) { return omp_get_max_threads(); }

int64_t orc_layer_omp(const uint8_t *pg, const float *sg, const uint8_t *pu,
                      const float *su, const uint8_t *pd, const float *sd,
                      int64_t experts, int64_t hidden, int64_t inter, int64_t gs,
                      const double *x, int64_t tokens, const int32_t *ids,
                      const float *w, int64_t k, double *out) {
    int64_t bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(+ : bad)
    for (int64_t t = 0; t < tokens; t++)
        bad += orc_layer(pg, sg, pu, su, pd, sd, experts, hidden, inter, gs,
                         x + t * hidden, 1, ids + t * k, w + t * k, k, out + t * hidden);
    return bad;
}
