/*
 * CPU ORACLE -- TEST INFRASTRUCTURE ONLY (see cfc_oracle_body.h for the
 * definitions and their sources).  Built with plain gcc, no fast-math and no
 * floating-point contraction, so every +, -, * rounds on its own.
 *
 * Exported symbols (all sizes are int64, all arrays row-major, host memory):
 *   oracle_fwd_step_{f64,f32}, oracle_bwd_step_{f64,f32},
 *   oracle_sum_axis0_{f64,f32}, oracle_cfc_forward_{f64,f32},
 *   oracle_cfc_train_{f64,f32}, oracle_input_projection_{f64,f32},
 *   oracle_reduce_axis0_f64, oracle_set_threads, oracle_threads.
 *
 * Host threads (OpenMP): the loops over samples (forward and backward steps)
 * and the reduction's loop over columns may run on several threads.  Sums
 * across samples (the batch-axis sums) stay serial in increasing b, so every
 * result is bitwise the same for any thread count.
 */
#include <math.h>
#include <omp.h>
#include <stdlib.h>

#define REAL double
#define SUF f64
#define EXP exp
#define TANH tanh
#include "cfc_oracle_body.h"
#undef REAL
#undef SUF
#undef EXP
#undef TANH

#define REAL float
#define SUF f32
#define EXP expf
#define TANH tanhf
#include "cfc_oracle_body.h"
#undef REAL
#undef SUF
#undef EXP
#undef TANH

/* The reference for the batch-axis reduction of fp32 data: each column summed
 * in double, in increasing b, then stored as double (no final rounding), per
 * "K-loop Parallelization -- Block-per-Batch Kernel Refactor", section
 * Architecture Choice, reduce_axis0 ([B, N] -> [N], sum over the batch axis,
 * output overwritten) and section Risks + Mitigations (sum in batch-index
 * order).  B == 0 gives zeros.  Columns are independent, so they may be
 * split over host threads; each column's sum is the same whatever the split. */
void oracle_reduce_axis0_f64(const float* x, long B, long N, double* out)
{
#pragma omp parallel for schedule(static)
    for (long n = 0; n < N; ++n) {
        double acc = 0.0;
        for (long b = 0; b < B; ++b) acc += (double)x[b * N + n];
        out[n] = acc;
    }
}

/* Threads the oracle's parallel loops use from now on (n >= 1). */
void oracle_set_threads(int n)
{
    if (n >= 1) omp_set_num_threads(n);
}

/* Threads a parallel loop of the oracle would use now. */
int oracle_threads(void) { return omp_get_max_threads(); }
