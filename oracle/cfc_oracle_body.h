/*
 * CPU ORACLE -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously-correct loops for the closed-form continuous-time
 * (CfC) recurrent cell trained by full backpropagation through time, with
 * per-sample weight-gradient scratch and a batch-axis column sum.  Only the
 * test-suite, the smoke entry point and the CPU-baseline leg of the benchmark
 * may load this code.  The GPU library shares nothing with it.
 *
 * This header is the single body of the oracle.  cfc_oracle.c includes it
 * twice, once with REAL = double (suffix f64) and once with REAL = float
 * (suffix f32), so both precisions run the same statements.
 *
 * The cell.  The pages ("K-loop Parallelization -- Block-per-Batch Kernel
 * Refactor", section Problem and the Per-Kernel Breakdown table) name the
 * CfC step kernels but never write their equations.  This library fixes them
 * as follows, with dt = 1:
 *     z      = [u_t ; h_{t-1}]                    (length n_in = n_x + C)
 *     a_q    = W_q z + b_q       for heads q = f, g, h (in that order)
 *     gate   = sigmoid(-a_f * dt) = 1 / (1 + exp(a_f))
 *     g      = tanh(a_g),  hh = tanh(a_h)
 *     h_t    = gate * g + (1 - gate) * hh
 *     L      = 0.5 * sum_{b, t=1..K, c} (h_t[b,c] - y_t[b,c])^2
 * Layouts (row-major): W [3, C, n_in] (head-major), bias [3, C],
 * u [K, B, n_x], y [K, B, C], h_hist [K+1, B, C], act [K, 3, B, C] holding
 * (gate, g, hh); scratch S [B, 3, C, n_in], Sb [B, 3, C].
 *
 * Per-sample scratch and the reduction follow the same page, section
 * Architecture Choice ("Param-grad writes": each (sample, channel) is the
 * sole writer of its scratch row; "reduce_axis0": the final gradient is the
 * sum over the batch axis and OVERWRITES its output) and the subsections
 * "Per-K-iteration accumulation invariant" (scratch zeroed once at step start,
 * every K-iteration adds into it, one reduction after the K-loop).
 */

#define CAT_(a, b) a##_##b
#define CAT(a, b) CAT_(a, b)
#define FN(name) CAT(name, SUF)

/* One forward step for every sample: h_t and the saved activations.
 * Loop order b -> c -> q -> k; the dot product runs k = 0 .. n_in-1.
 * Samples are independent (each writes only its own rows), so the b loop
 * may run on several host threads; every value is computed by the same
 * statements in the same order whatever the thread count. */
void FN(oracle_fwd_step)(const REAL* u_t, const REAL* h_prev, const REAL* W,
                         const REAL* bias, long B, long C, long n_x,
                         REAL* h_t, REAL* act_t)
{
    const long n_in = n_x + C;
#pragma omp parallel for schedule(static)
    for (long b = 0; b < B; ++b) {
        REAL* z = (REAL*)malloc(sizeof(REAL) * (size_t)(n_in > 0 ? n_in : 1));
        /* z = [u_t[b] ; h_prev[b]] */
        for (long k = 0; k < n_x; ++k) z[k] = u_t[b * n_x + k];
        for (long k = 0; k < C; ++k) z[n_x + k] = h_prev[b * C + k];
        for (long c = 0; c < C; ++c) {
            REAL a[3];
            for (int q = 0; q < 3; ++q) {
                const REAL* row = W + ((long)q * C + c) * n_in;
                REAL acc = 0;
                for (long k = 0; k < n_in; ++k) acc += row[k] * z[k];
                a[q] = acc + bias[(long)q * C + c];
            }
            const REAL gate = (REAL)1 / ((REAL)1 + EXP(a[0]));
            const REAL g = TANH(a[1]);
            const REAL hh = TANH(a[2]);
            h_t[b * C + c] = gate * g + ((REAL)1 - gate) * hh;
            act_t[(0 * B + b) * C + c] = gate;
            act_t[(1 * B + b) * C + c] = g;
            act_t[(2 * B + b) * C + c] = hh;
        }
        free(z);
    }
}

/* The input part of the pre-activations for M rows of inputs at once:
 *   X[m, q C + c] = b_q[c] + sum_{k < n_x} W_q[c, k] u[m, k]
 * i.e. a_q of oracle_fwd_step restricted to the input columns of z.  The sum
 * runs k = 0 .. n_x-1, then the bias is added. */
void FN(oracle_input_projection)(const REAL* u, const REAL* W, const REAL* bias, long M, long C,
                                 long n_x, REAL* X)
{
    const long n_in = n_x + C;
    for (long m = 0; m < M; ++m)
        for (long r = 0; r < 3 * C; ++r) {
            const REAL* row = W + r * n_in;
            REAL acc = 0;
            for (long k = 0; k < n_x; ++k) acc += row[k] * u[m * n_x + k];
            X[m * 3 * C + r] = acc + bias[r];
        }
}

/* One backward step for every sample (the b loop may run on several host
 * threads, as in oracle_fwd_step: sample b writes only its own rows).
 *   dh    = (h_t - y_t) + dh_in                       (loss residual + carry)
 *   dp_f  = dh * (g - hh) * (-gate * (1 - gate))       (d/da_f; dgate/da_f = -gate(1-gate))
 *   dp_g  = dh * gate * (1 - g^2)
 *   dp_h  = dh * (1 - gate) * (1 - hh^2)
 *   S [b,q,c,k] += dp_q[c] * z[k];  Sb[b,q,c] += dp_q[c]
 *   dz[k] = sum_{q=f,g,h} sum_{c=0..C-1} W_q[c,k] * dp_q[c]
 *   dh_out = dz[n_x:]  (carry to step t-1),  du_t = dz[:n_x] (if du_t != NULL)
 * dh_out is overwritten; S and Sb accumulate.  dp_out (nullable, [3,B,C])
 * receives the pre-activation gradients dp_q of this step. */
void FN(oracle_bwd_step)(const REAL* u_t, const REAL* h_prev, const REAL* h_t,
                         const REAL* y_t, const REAL* W, const REAL* act_t,
                         const REAL* dh_in, REAL* dh_out, REAL* du_t,
                         REAL* S, REAL* Sb, long B, long C, long n_x,
                         REAL* dp_out)
{
    const long n_in = n_x + C;
#pragma omp parallel for schedule(static)
    for (long b = 0; b < B; ++b) {
        REAL* z = (REAL*)malloc(sizeof(REAL) * (size_t)(n_in > 0 ? n_in : 1));
        REAL* dp = (REAL*)malloc(sizeof(REAL) * (size_t)(3 * C > 0 ? 3 * C : 1));
        for (long k = 0; k < n_x; ++k) z[k] = u_t[b * n_x + k];
        for (long k = 0; k < C; ++k) z[n_x + k] = h_prev[b * C + k];
        for (long c = 0; c < C; ++c) {
            const REAL gate = act_t[(0 * B + b) * C + c];
            const REAL g = act_t[(1 * B + b) * C + c];
            const REAL hh = act_t[(2 * B + b) * C + c];
            const REAL dh = (h_t[b * C + c] - y_t[b * C + c]) + dh_in[b * C + c];
            dp[0 * C + c] = dh * (g - hh) * (-gate * ((REAL)1 - gate));
            dp[1 * C + c] = dh * gate * ((REAL)1 - g * g);
            dp[2 * C + c] = dh * ((REAL)1 - gate) * ((REAL)1 - hh * hh);
            if (dp_out)
                for (int q = 0; q < 3; ++q) dp_out[((long)q * B + b) * C + c] = dp[(long)q * C + c];
            for (int q = 0; q < 3; ++q) {
                REAL* srow = S + (((long)b * 3 + q) * C + c) * n_in;
                for (long k = 0; k < n_in; ++k) srow[k] += dp[(long)q * C + c] * z[k];
                Sb[((long)b * 3 + q) * C + c] += dp[(long)q * C + c];
            }
        }
        for (long k = 0; k < n_in; ++k) {
            REAL acc = 0;
            for (int q = 0; q < 3; ++q)
                for (long c = 0; c < C; ++c)
                    acc += W[((long)q * C + c) * n_in + k] * dp[(long)q * C + c];
            if (k >= n_x)
                dh_out[b * C + (k - n_x)] = acc;
            else if (du_t)
                du_t[b * n_x + k] = acc;
        }
        free(dp);
        free(z);
    }
}

/* Column sum over the batch axis, in increasing b, in REAL:
 * out[n] = sum_{b=0..B-1} x[b, n].  OVERWRITES out (B == 0 gives zeros). */
void FN(oracle_sum_axis0)(const REAL* x, long B, long N, REAL* out)
{
    for (long n = 0; n < N; ++n) {
        REAL acc = 0;
        for (long b = 0; b < B; ++b) acc += x[b * N + n];
        out[n] = acc;
    }
}

/* Forward over all K steps; returns the loss.  h_hist[0] = h0. */
REAL FN(oracle_cfc_forward)(const REAL* u, const REAL* y, const REAL* h0,
                            const REAL* W, const REAL* bias, long B, long C,
                            long n_x, long K, REAL* h_hist, REAL* act)
{
    for (long i = 0; i < B * C; ++i) h_hist[i] = h0[i];
    for (long t = 1; t <= K; ++t)
        FN(oracle_fwd_step)(u + (t - 1) * B * n_x, h_hist + (t - 1) * B * C, W, bias,
                            B, C, n_x, h_hist + t * B * C, act + (t - 1) * 3 * B * C);
    REAL loss = 0;
    for (long t = 1; t <= K; ++t)
        for (long i = 0; i < B * C; ++i) {
            const REAL r = h_hist[t * B * C + i] - y[(t - 1) * B * C + i];
            loss += (REAL)0.5 * r * r;
        }
    return loss;
}

/* One whole training step of the K-loop: forward t = 1..K, then the scratch
 * is zeroed once, the backward runs t = K..1 adding into it (carry_K = 0),
 * and the batch-axis sum overwrites the final gradients gW, gb.
 * dh0 receives the gradient of L with respect to h0; du (nullable, [K,B,n_x])
 * the one with respect to u; dp (nullable, [K,3,B,C]) the pre-activation
 * gradients of every step.  Returns the loss. */
REAL FN(oracle_cfc_train)(const REAL* u, const REAL* y, const REAL* h0,
                          const REAL* W, const REAL* bias, long B, long C,
                          long n_x, long K, REAL* h_hist, REAL* act, REAL* S,
                          REAL* Sb, REAL* gW, REAL* gb, REAL* dh0, REAL* du,
                          REAL* dp)
{
    const long n_in = n_x + C;
    const REAL loss = FN(oracle_cfc_forward)(u, y, h0, W, bias, B, C, n_x, K, h_hist, act);

    for (long i = 0; i < B * 3 * C * n_in; ++i) S[i] = 0;
    for (long i = 0; i < B * 3 * C; ++i) Sb[i] = 0;

    REAL* carry = (REAL*)malloc(sizeof(REAL) * (size_t)(B * C > 0 ? B * C : 1));
    REAL* carry_next = (REAL*)malloc(sizeof(REAL) * (size_t)(B * C > 0 ? B * C : 1));
    for (long i = 0; i < B * C; ++i) carry[i] = 0;
    for (long t = K; t >= 1; --t) {
        FN(oracle_bwd_step)(u + (t - 1) * B * n_x, h_hist + (t - 1) * B * C,
                            h_hist + t * B * C, y + (t - 1) * B * C, W,
                            act + (t - 1) * 3 * B * C, carry, carry_next,
                            du ? du + (t - 1) * B * n_x : (REAL*)0, S, Sb, B, C, n_x,
                            dp ? dp + (t - 1) * 3 * B * C : (REAL*)0);
        REAL* tmp = carry;
        carry = carry_next;
        carry_next = tmp;
    }
    for (long i = 0; i < B * C; ++i) dh0[i] = carry[i];
    free(carry);
    free(carry_next);

    FN(oracle_sum_axis0)(S, B, 3 * C * n_in, gW);
    FN(oracle_sum_axis0)(Sb, B, 3 * C, gb);
    return loss;
}

#undef FN
#undef CAT
#undef CAT_
