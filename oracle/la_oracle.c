/*
 * la_oracle.c -- CPU oracle for the Lightning Attention forward (prefill) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain, obviously-correct definition the GPU path is
 * checked against. Only the test suite, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes. Sources: the page "[LA] Lightning Attention MTP decode + KVBuffer parallel verify /
 * commit", Description, the closed form used by verify; and the page "[Lightning Attention] Add Hopper SM90
 * CuTe DSL prefill", Reviewer notes (public state is FP32 in [V, K] orientation) and the accuracy section
 * (lambda = exp(-slope), exponent offset 1):
 *
 *     S_t = lambda * S_{t-1} + v_t k_t^T          (S is DV x D, row index = value dim, column = key dim)
 *     o_t = scale * S_t q_t
 *
 * evaluated token by token in double precision, starting from S_{-1} = S0 (or zero). Unrolled, this is
 * o_t = scale * (lambda^{t+1} S0 q_t + sum_{i<=t} lambda^{t-i} (q_t . k_i) v_i), the verify page's closed form;
 * the state decays before token t is added, so token t itself carries weight lambda^0 = 1 and S0 carries
 * lambda^{t+1} (the prefill page's "exponent offset 1").
 *
 * Inputs are bf16 bit patterns (uint16), widened exactly to double. Nothing is rounded on the way out:
 * outputs and final states are returned in double.
 *
 * Parallelism: OpenMP over independent (sequence, value head) units; each unit is a sequential loop.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_bits_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * One call evaluates `nunits` independent units. Unit u is the sequence whose tokens occupy rows
 * [row0[u], row0[u] + len[u]) of the token-major inputs, paired with value head hv[u]. Its q/k head is
 * hv[u] / (HV / H): value heads hv = G*h ... G*h + G - 1 share q/k head h (grouped value attention).
 *
 *   q, k : bf16 bits, [rows, H, D] (D fastest); q may be NULL when o is NULL (state only)
 *   v    : bf16 bits, [rows, HV, DV] (DV fastest)
 *   slope: float [HV]; lambda = exp(-slope[hv]) evaluated in double
 *   s0   : double [nunits, DV, D] initial states, or NULL for zero initial state
 *   o    : double, unit u writes len[u] rows of DV values starting at o + o_off[u] * DV (may be NULL)
 *   s_fin: double [nunits, DV, D] final states (may be NULL)
 *
 * Returns 0, or -1 on an argument that makes the definition meaningless (non-positive dims, HV % H != 0).
 */
int la_oracle_fwd(const uint16_t *q, const uint16_t *k, const uint16_t *v, int32_t H, int32_t HV, int32_t D,
                  int32_t DV, double scale, const float *slope, int32_t nunits, const int64_t *row0,
                  const int64_t *len, const int32_t *hv_of_unit, const double *s0, double *o,
                  const int64_t *o_off, double *s_fin)
{
    if (H <= 0 || HV <= 0 || D <= 0 || DV <= 0 || HV % H != 0 || nunits < 0 || (o && !q))
        return -1;
    const int32_t G = HV / H;

#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t u = 0; u < nunits; ++u) {
        const int32_t hv = hv_of_unit[u];
        const int32_t h = hv / G;
        const double lambda = exp(-(double)slope[hv]);
        double *S = (double *)malloc(sizeof(double) * (size_t)DV * (size_t)D);
        double *kt = (double *)malloc(sizeof(double) * (size_t)D);
        double *qt = (double *)malloc(sizeof(double) * (size_t)D);
        double *vt = (double *)malloc(sizeof(double) * (size_t)DV);
        if (s0)
            memcpy(S, s0 + (size_t)u * DV * D, sizeof(double) * (size_t)DV * D);
        else
            memset(S, 0, sizeof(double) * (size_t)DV * D);

        for (int64_t t = 0; t < len[u]; ++t) {
            const int64_t r = row0[u] + t;
            for (int32_t d = 0; d < D; ++d) {
                kt[d] = bf16_bits_to_double(k[((size_t)r * H + h) * D + d]);
                qt[d] = q ? bf16_bits_to_double(q[((size_t)r * H + h) * D + d]) : 0.0;
            }
            for (int32_t e = 0; e < DV; ++e)
                vt[e] = bf16_bits_to_double(v[((size_t)r * HV + hv) * DV + e]);

            /* S <- lambda * S + v k^T, then o = scale * S q */
            for (int32_t e = 0; e < DV; ++e) {
                double *row = S + (size_t)e * D;
                double acc = 0.0;
                for (int32_t d = 0; d < D; ++d) {
                    row[d] = lambda * row[d] + vt[e] * kt[d];
                    acc += row[d] * qt[d];
                }
                if (o)
                    o[(size_t)(o_off[u] + t) * DV + e] = scale * acc;
            }
        }
        if (s_fin)
            memcpy(s_fin + (size_t)u * DV * D, S, sizeof(double) * (size_t)DV * D);
        free(S);
        free(kt);
        free(qt);
        free(vt);
    }
    return 0;
}

/* Number of threads an OpenMP parallel region of this library uses. */
int la_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
