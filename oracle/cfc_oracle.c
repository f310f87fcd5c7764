/*
 * CPU ORACLE -- TEST INFRASTRUCTURE ONLY (see cfc_oracle_body.h for the
 * definitions and their sources).  Built with plain gcc, no fast-math and no
 * floating-point contraction, so every +, -, * rounds on its own.
 *
 * Exported symbols (all sizes are int64, all arrays row-major, host memory):
 *   oracle_fwd_step_{f64,f32}, oracle_bwd_step_{f64,f32},
 *   oracle_sum_axis0_{f64,f32}, oracle_cfc_forward_{f64,f32},
 *   oracle_cfc_train_{f64,f32}, oracle_input_projection_{f64,f32},
 *   oracle_reduce_axis0_f64.
 */
#include <math.h>
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
 * order).  B == 0 gives zeros. */
void oracle_reduce_axis0_f64(const float* x, long B, long N, double* out)
{
    for (long n = 0; n < N; ++n) {
        double acc = 0.0;
        for (long b = 0; b < B; ++b) acc += (double)x[b * N + n];
        out[n] = acc;
    }
}
