/*
 * cfc.h -- C ABI of libcfc.so: a closed-form continuous-time (CfC) recurrent
 * cell trained over a K-step loop (forward, then full backpropagation through
 * time) on AMD Instinct MI355X (gfx950).
 *
 * Sources.  "K-loop Parallelization -- Block-per-Batch Kernel Refactor"
 * (design spec of the foxhunt project):
 *   - section Problem: the CfC forward and backward step kernels run once per
 *     K-iteration (64 calls each per training step) and are parallel across
 *     the batch;
 *   - section Architecture Choice, "Param-grad writes": every (sample,
 *     channel) pair is the sole writer of its row of a per-sample weight
 *     gradient scratch [B, C, n_in], accumulated with +=;
 *   - same section, "reduce_axis0": one parameterised reducer [B, N] -> [N]
 *     that OVERWRITES its output, sums over the batch axis without atomics;
 *   - subsection "Per-K-iteration accumulation invariant": scratch is zeroed
 *     once at step start, every K-iteration adds into it, the reducer runs
 *     once after the K-loop;
 *   - subsection "AdamW-after-reducer invariant": the final gradient buffers
 *     hold this step's values only after the reducer has run;
 *   - section Trainer Wiring: the whole step, reducers included, is one
 *     captured graph.
 * The pages do not write the cell equations.  This library fixes them, with
 * dt = 1, heads ordered f, g, h:
 *     z    = [u_t ; h_{t-1}]            n_in = n_x + C
 *     a_q  = W_q z + b_q
 *     gate = 1 / (1 + exp(a_f))          (= sigmoid(-a_f * dt))
 *     g    = tanh(a_g),  hh = tanh(a_h)
 *     h_t  = gate * g + (1 - gate) * hh
 *     L    = 0.5 * sum over b, t = 1..K, c of (h_t - y_t)^2
 *
 * Conventions for every entry point.
 *   - All float* are DEVICE pointers to contiguous row-major fp32 arrays,
 *     owned by the caller.  The library never allocates, frees or keeps them,
 *     except that cfc_train_kloop remembers pointer VALUES as a graph-cache key.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls only enqueue work on it and never synchronise the host; device
 *     faults surface at the caller's next synchronisation.
 *   - Return value: CFC_OK (0) or a negative cfc_status.  Nothing throws
 *     across the ABI.  cfc_last_error() describes the last failure on the
 *     calling thread.
 *   - Sizes: B >= 0, C >= 1, n_x >= 0, K >= 0; C <= CFC_MAX_C and
 *     n_in <= CFC_MAX_N_IN.  Index arithmetic is 64-bit.
 *   - Outputs must not overlap the inputs of the same call (CFC_EINVAL).
 *   - Results are deterministic: no atomics; every sum has an order fixed by
 *     the sizes, so repeated calls give identical bits, and row b of a batched
 *     call equals a B = 1 call on sample b bit for bit.
 */
#ifndef CFC_H
#define CFC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum cfc_status {
    CFC_OK = 0,
    CFC_EINVAL = -1, /* null pointer, size out of range, forbidden overlap */
    CFC_EHIP = -2    /* a HIP runtime call failed (launch, capture, instantiate) */
};

#define CFC_MAX_C 2048
#define CFC_MAX_N_IN 8192

/* One forward step for all B samples ("K-loop Parallelization", section
 * Problem: the forward step kernel; the equations in the header comment).
 *   u_t    [B, n_x]      input at step t
 *   h_prev [B, C]        h_{t-1}
 *   W      [3, C, n_in]  weights, heads f, g, h; column k < n_x multiplies
 *                        u_t, column n_x + j multiplies h_{t-1}[j]
 *   bias   [3, C]
 *   h_t    [B, C]        out, overwritten; must not overlap any input
 *   act_t  [3, B, C]     out, overwritten: (gate, g, hh) saved for backward
 */
int cfc_fwd_step(const float* u_t, const float* h_prev, const float* W,
                 const float* bias, float* h_t, float* act_t,
                 int B, int C, int n_x, void* stream);

/* One backward (BPTT) step for all B samples ("K-loop Parallelization",
 * section Architecture Choice, "Param-grad writes"):
 *   dh    = (h_t - y_t) + dh_in
 *   dp_f  = dh * (g - hh) * (-gate * (1 - gate))
 *   dp_g  = dh * gate * (1 - g^2),   dp_h = dh * (1 - gate) * (1 - hh^2)
 *   gW_scratch[b, q, c, :] += dp_q[b, c] * z_b     (sole writer per (b, c))
 *   gb_scratch[b, q, c]    += dp_q[b, c]
 *   dz_b = sum_q W_q^T dp_q[b, :];  dh_out = dz[n_x:],  du_t = dz[:n_x]
 * Arguments:
 *   u_t, h_prev, h_t, y_t, act_t  as in the forward step ([B,n_x], [B,C],
 *                        [B,C], [B,C] targets, [3,B,C])
 *   dh_in  [B, C]        carry from step t+1, or NULL for a zero carry (t = K)
 *   dh_out [B, C]        out, overwritten: carry to step t-1; != dh_in
 *   du_t   [B, n_x]      out, overwritten, or NULL to skip
 *   gW_scratch [B, 3, C, n_in], gb_scratch [B, 3, C]   accumulated (+=)
 */
int cfc_bwd_step(const float* u_t, const float* h_prev, const float* h_t,
                 const float* y_t, const float* W, const float* act_t,
                 const float* dh_in, float* dh_out, float* du_t,
                 float* gW_scratch, float* gb_scratch,
                 int B, int C, int n_x, void* stream);

/* Batch-axis reduction ("K-loop Parallelization", section Architecture
 * Choice, reduce_axis0; section Risks + Mitigations: deterministic order).
 *   out[n] = sum_{b < n_batch} per_batch[b, n]      for n < n_tail
 * per_batch [n_batch, n_tail] fp32, out [n_tail] fp32, OVERWRITTEN.
 * Sums are carried in fp64 in an order fixed by n_batch alone and rounded to
 * fp32 once.  n_batch == 0 writes zeros; n_tail == 0 is a no-op; n_batch == 1
 * is an exact copy.  out must not overlap per_batch.  Negative sizes: EINVAL.
 */
int reduce_axis0(const float* per_batch, int64_t n_batch, int64_t n_tail,
                 float* out, void* stream);

/* One whole training step of the K-loop, replayed as one HIP graph
 * ("K-loop Parallelization", sections Trainer Wiring and Architecture
 * Choice): forward t = 1..K, backward t = K..1, the per-sample scratch
 * (overwritten: it holds this step's sums only, as if zeroed at step start
 * and added to by every K-iteration), then reduce_axis0 over the batch
 * overwrites gW and gb.
 *   u [K, B, n_x], y [K, B, C], h0 [B, C], W [3, C, n_in], bias [3, C]
 *   h_hist [K+1, B, C]   out: h_hist[0] = h0, h_hist[t] = h_t
 *   act    [K, 3, B, C]  out: saved (gate, g, hh) of every step
 *   ws, ws_bytes         workspace of at least
 *                        cfc_train_kloop_workspace_bytes(B, C, n_x, K) bytes
 *                        (the pre-activation gradients of every step, the
 *                        input projection of every step, the BPTT carry,
 *                        the step kernels' re-laid copy of W and the step
 *                        flags of the resident and persistent launches);
 *                        contents are undefined afterwards
 *   gW_scratch [B, 3, C, n_in], gb_scratch [B, 3, C]   out: per-sample sums
 *                        S[b,q,c,:] = sum_t dp_q[t,b,c] z_t[b,:] (t = K..1)
 *   gW [3, C, n_in], gb [3, C]   out, OVERWRITTEN; valid only once this
 *                        call's work on `stream` has completed
 * The paths give the same bits:
 *  - persistent (C <= 128): one workgroup per sample running every K step
 *    with the recurrent W in registers, after the input projection of all
 *    steps, then the scratch fill and the reduction, enqueued directly on
 *    `stream`.  With B <= 128 the projection is formed by extra workgroups
 *    of the same launch, which the sample workgroups wait for -- three
 *    launches.  When, besides, every array is 16-byte aligned, C and n_x are
 *    multiples of 4, n_in <= 256 and the launch's workgroups fit the device's
 *    CUs one each, those workgroups then also form the scratch, following
 *    the backward one chunk of 16 steps at a time (a flag per sample and
 *    chunk in ws) -- two launches.  The waits are bounded: only other work
 *    holding the device's CUs for about a second makes one give up, which
 *    marks an error word in ws and leaves the results undefined.
 *    Otherwise, and on a stream under capture, the projection is a launch of
 *    its own -- four launches;
 *  - resident MFMA (B >= 64, C > 128, shapes of the MFMA step kernels whose
 *    grid fits the device at once): a W re-layout, one cooperative launch
 *    running all 2K steps, the fill and the reduction, enqueued directly (a
 *    cooperative launch is not captured into graphs: on a stream under
 *    capture the call takes the MFMA step kernels instead);
 *  - step kernels (any C): 2K step launches, the fill and the reduction,
 *    captured once as a HIP graph per (device, pointers, sizes) and replayed
 *    on later calls with the same key.  Calls sharing a key must be issued
 *    on one stream at a time.  At most 64 graphs are cached; the least
 *    recently used one is evicted and destroyed by a later call once its
 *    last replay has completed (the call never waits for it).
 * cfc_set_kloop_mode() can force a path for the calling thread.  K == 0 or B == 0 writes
 * h_hist[0] = h0 and zeros to the scratch and gradients.
 */
int cfc_train_kloop(const float* u, const float* y, const float* h0,
                    const float* W, const float* bias,
                    float* h_hist, float* act, float* ws, size_t ws_bytes,
                    float* gW_scratch, float* gb_scratch,
                    float* gW, float* gb,
                    int B, int C, int n_x, int K, void* stream);

/* The two phases of cfc_train_kloop before its reduction, callable on their
 * own (same kernels, same bits):
 * cfc_kloop_fwd_bwd -- forward t = 1..K and backward t = K..1 for every
 *   sample (the persistent kernel or 2K step launches, per the kloop mode).
 *   Writes h_hist [K+1,B,C] and act [K,3,B,C] as cfc_train_kloop does, and
 *   the pre-activation gradients dp_t into the first K*B*3C floats of ws as
 *   [K, B, 3C] (row r = q C + c), which cfc_scratch_fill consumes.
 * cfc_scratch_fill -- per-sample scratch from saved dp ("K-loop
 *   Parallelization", section Architecture Choice, "Per-K-iteration
 *   accumulation invariant": the sum over the K-iterations of each
 *   sample's terms, computed once rather than in K read-modify-writes):
 *     gW_scratch[b,q,c,k] = fma chain over t = K..1 of dp[t,b,q,c] z_t[b,k]
 *     gb_scratch[b,q,c]   = sum over t = K..1 of dp[t,b,q,c]
 *   with z_t = [u[t-1,b,:] ; h_hist[t-1,b,:]].  Both outputs are overwritten
 *   (zeros when K == 0).  dp [K,B,3C], u [K,B,n_x], h_hist [K(+1),B,C].
 */
int cfc_kloop_fwd_bwd(const float* u, const float* y, const float* h0,
                      const float* W, const float* bias,
                      float* h_hist, float* act, float* ws, size_t ws_bytes,
                      int B, int C, int n_x, int K, void* stream);

/* cfc_train_kloop up to its reduction ("K-loop Parallelization", section
 * Architecture Choice: the K-loop's per-sample scratch, before the
 * reducer): the same launches and bits as cfc_train_kloop without the
 * reduction, writing h_hist, act, the dp block of ws, gW_scratch and
 * gb_scratch as it does (same arguments, layouts and errors; gW and gb are
 * not touched).  On the persistent path with B <= 128 this is one launch
 * whenever cfc_train_kloop's is (see there); otherwise cfc_kloop_fwd_bwd's
 * launches followed by cfc_scratch_fill's.  K == 0 or B == 0 writes
 * h_hist[0] = h0 and zero scratch. */
int cfc_kloop_fwd_bwd_fill(const float* u, const float* y, const float* h0,
                           const float* W, const float* bias,
                           float* h_hist, float* act, float* ws, size_t ws_bytes,
                           float* gW_scratch, float* gb_scratch,
                           int B, int C, int n_x, int K, void* stream);

/* AdamW after the reducer ("K-loop Parallelization", section Trainer Wiring:
 * the optimizer consumes the final gradient buffers and runs strictly after
 * every reducer -- on the same stream after cfc_train_kloop, stream order
 * guarantees it).  One launch updates up to 4 tensors (a flat fused update,
 * as in "H100 Epoch Optimization Phase 2", the single-flat-kernel tasks):
 * for segment i, arrays params[i], grads[i], m[i], v[i] of n[i] floats each
 * (device pointers, host arrays of nseg entries), with decoupled weight
 * decay:
 *   p <- p (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2;
 *   p <- p - (lr / (1 - b1^step)) m / (sqrt(v) / sqrt(1 - b2^step) + eps)
 * params, m and v are updated in place; grads are read only.  step is the
 * 1-based step count.  nseg in [0, 4]; step >= 1; lr, wd >= 0; b1, b2 in
 * [0, 1); eps > 0; arrays that overlap give CFC_EINVAL. */
int cfc_adamw_step(float* const* params, const float* const* grads, float* const* m, float* const* v,
                   const int64_t* n, int nseg, float lr, float beta1, float beta2, float eps,
                   float weight_decay, int step, void* stream);

/* GEMM-form weight gradient, an alternative to the per-sample scratch and
 * its reducer ("K-loop Parallelization", section Architecture Choice, "Why
 * scratch+reducer", weighs the per-sample scratch against other ways of
 * summing over the batch; "H100 Epoch Optimization Phase 2", Task 2, forms
 * a weight gradient as dY^T X over the batch).  It writes no scratch:
 *   gW[q, c, k] = sum over t = 1..K, b of dp_t[b, q C + c] z_t[b, k],
 *   gb[q, c]    = sum over t, b of dp_t[b, q C + c],
 * with z_t = [u_t ; h_{t-1}], as ONE contraction over the K*B (t, b) rows on
 * the matrix cores, cut into fixed row splits whose fp32 partials are added
 * in fp64 by the batch-axis reducer.  Same values as cfc_train_kloop's gW,
 * gb to rounding (a different, equally fixed summation order: not the same
 * bits).
 *   dp     [K, B, 3C]  pre-activation gradients (cfc_kloop_fwd_bwd leaves
 *                      them at the start of its workspace)
 *   u      [K, B, n_x], h_hist [K+1, B, C] (rows 0 .. K-1 are read)
 *   gW     [3, C, n_in], gb [3, C]   OVERWRITTEN
 *   ws     cfc_weight_grad_gemm_workspace_bytes() bytes of device memory.
 * K*B up to 2^30 rows (and K*B*3C below 2^31); K*B == 0 writes zeros. */
int cfc_weight_grad_gemm(const float* dp, const float* u, const float* h_hist, float* gW, float* gb, int B, int C,
                         int n_x, int K, void* ws, size_t ws_bytes, void* stream);
size_t cfc_weight_grad_gemm_workspace_bytes(int B, int C, int n_x, int K);

/* The K-loop training step with the GEMM-form weight gradient in place of
 * the scratch and its reducer: cfc_kloop_fwd_bwd, then
 * cfc_weight_grad_gemm on the dp it leaves in the workspace.  Arguments as
 * cfc_train_kloop without the scratch; ws holds
 * cfc_train_kloop_gemm_workspace_bytes() bytes. */
int cfc_train_kloop_gemm(const float* u, const float* y, const float* h0, const float* W, const float* bias,
                         float* h_hist, float* act, float* gW, float* gb, void* ws, size_t ws_bytes, int B, int C,
                         int n_x, int K, void* stream);
size_t cfc_train_kloop_gemm_workspace_bytes(int B, int C, int n_x, int K);

/* The two launches of cfc_kloop_fwd_bwd's persistent path, callable on
 * their own (same kernels, same bits):
 * cfc_input_projection -- the input part of every step's pre-activations,
 *   for M rows at once (in the K-loop the rows are (t, b), M = K B):
 *     X[m, q C + c] = bias[q, c] + sum_{k < n_x} W[q, c, k] u[m, k]
 *   in the library's canonical order (four fma chains over the input
 *   columns k = j mod 4, then bias + ((x0 + x1) + (x2 + x3))).
 *   u [M, n_x], W [3, C, n_in] (only columns < n_x are read), bias [3, C],
 *   X [M, 3C] out, OVERWRITTEN; X must not overlap the inputs.
 * cfc_kloop_recurrence -- forward t = 1..K and backward t = K..1 of every
 *   sample given X [K, B, 3C] from cfc_input_projection (the cell of
 *   cfc_fwd_step with a_q = X_q + the recurrent part, BPTT of
 *   cfc_bwd_step), one workgroup per sample ("K-loop Parallelization",
 *   section Architecture Choice).  Writes h_hist [K+1,B,C], act [K,3,B,C]
 *   and dp [K,B,3C] (row r = q C + c) as cfc_kloop_fwd_bwd does.  Only for
 *   C <= 128 (CFC_EINVAL otherwise).  K == 0 or B == 0 writes h_hist[0] = h0.
 */
int cfc_input_projection(const float* u, const float* W, const float* bias,
                         float* X, int64_t M, int C, int n_x, void* stream);

int cfc_kloop_recurrence(const float* X, const float* y, const float* h0,
                         const float* W, float* h_hist, float* act, float* dp,
                         int B, int C, int n_x, int K, void* stream);

int cfc_scratch_fill(const float* dp, const float* u, const float* h_hist,
                     float* gW_scratch, float* gb_scratch,
                     int B, int C, int n_x, int K, void* stream);

/* Bytes of workspace cfc_train_kloop needs: 4 * (round_up(6 K B C + 2 B C, 64)
 *   + 3 C ldf + 1024 C + 32 ceil(B / 16) (round_up(C, 32) + 1024)
 *   + round_up(32 (ceil(B / 16) ceil(C / 16) + 1), 64)),
 *   ldf = round_up(n_x, 16) + round_up(C, 32).
 * Returns 0 for invalid sizes. */
size_t cfc_train_kloop_workspace_bytes(int B, int C, int n_x, int K);

/* Path selection of cfc_train_kloop, cfc_kloop_fwd_bwd and cfc_kloop_path
 * for the CALLING THREAD (each thread starts in CFC_KLOOP_AUTO; a setting
 * never affects the calls of another thread).
 * CFC_KLOOP_AUTO (default): the persistent kernel when C <= 128; otherwise,
 *   when B >= 64 and the shape fits the MFMA step kernels (C <= 320 and
 *   n_x <= 128, both multiples of 4; 16-byte aligned arrays), the resident
 *   MFMA kernel if its ceil(B / 16) ceil(C / 16) workgroups can all be
 *   resident on the device at once, else the MFMA step kernels; otherwise
 *   the step kernels on VALU;
 * CFC_KLOOP_STEPS: the step kernels, MFMA or VALU as in AUTO;
 * CFC_KLOOP_PERSISTENT: the persistent kernel;
 * CFC_KLOOP_STEPS_VALU / CFC_KLOOP_STEPS_MFMA: the step kernels on VALU / on
 *   MFMA;
 * CFC_KLOOP_RESIDENT: the resident MFMA kernel (the MFMA step kernels' steps,
 *   all 2K of them in one cooperative launch, each workgroup holding its W
 *   operands in registers and the workgroups of a sample tile handing one
 *   another h_t and dp_t through memory, every wait bounded).
 * A mode that forces a path the sizes cannot take makes cfc_train_kloop and
 * cfc_kloop_fwd_bwd return CFC_EINVAL.  All paths give the same bits. */
enum cfc_kloop_mode {
    CFC_KLOOP_AUTO = 0,
    CFC_KLOOP_STEPS = 1,
    CFC_KLOOP_PERSISTENT = 2,
    CFC_KLOOP_STEPS_VALU = 3,
    CFC_KLOOP_STEPS_MFMA = 4,
    CFC_KLOOP_RESIDENT = 5
};
int cfc_set_kloop_mode(int mode);

/* The path cfc_train_kloop takes for these sizes under the calling thread's
 * mode:
 * CFC_KLOOP_PERSISTENT, CFC_KLOOP_STEPS_VALU, CFC_KLOOP_STEPS_MFMA or
 * CFC_KLOOP_RESIDENT (the workspace is assumed 16-byte aligned; the
 * resident kernel's fit is that of the current device); -1 for invalid
 * sizes or a forced path the sizes cannot take. */
int cfc_kloop_path(int B, int C, int n_x, int K);

/* Whether the bounded waits of the last K-loop call on `ws` ended normally.
 * The resident launch's workgroups, and the persistent launch's sample
 * workgroups (B <= 128, outside graph capture), wait for other workgroups
 * of the same launch; a wait gives up only after about a second (other work
 * holding the device's CUs), marks an error word in ws and lets the kernel
 * finish, with undefined results.  Call once that call's work on `stream`
 * has completed, with its sizes, on the thread that made it (the path is
 * the one cfc_kloop_path reports there).  Reads at most two words of ws
 * with a copy on `stream` and waits for it: unlike the compute calls, this
 * one synchronises the host with the stream.  Returns CFC_EHIP if a wait
 * gave up, CFC_OK otherwise (also for paths without waits and for K == 0 or
 * B == 0), CFC_EINVAL for bad sizes, a null or short ws, or a kloop mode
 * that forces a path these sizes cannot take.
 */
int cfc_kloop_status(const float* ws, size_t ws_bytes, int B, int C, int n_x,
                     int K, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * K-loop training step of cfc_train_kloop, same arguments without ws and
 * ws_bytes, same kernels and the same bits, with its workspace in a fixed
 * array that the library holds on each device until the process ends
 * (CFC_NOALLOC_MAX_WS_BYTES; sizes whose cfc_train_kloop_workspace_bytes
 * exceed it give CFC_EINVAL before anything is enqueued).  The call
 * allocates and frees nothing, builds no graph (every launch is enqueued
 * directly on `stream`, on every path, honouring the calling thread's
 * cfc_set_kloop_mode) and never waits on the device.  Every call on one
 * device shares that device's array: calls whose work overlaps on one device
 * (several streams or threads at once) race and give undefined results;
 * calls issued one after another on a stream are safe.  Each call writes
 * every part of the array it reads, so no state carries over between calls.
 */
#define CFC_NOALLOC_MAX_WS_BYTES (32u << 20)
int cfc_train_kloop_noalloc(const float* u, const float* y, const float* h0,
                            const float* W, const float* bias,
                            float* h_hist, float* act,
                            float* gW_scratch, float* gb_scratch,
                            float* gW, float* gb,
                            int B, int C, int n_x, int K, void* stream);

/* Text of the last error raised on the calling thread ("" if none). */
const char* cfc_last_error(void);

/* Drop every cached graph (waits for their last replay to finish). */
int cfc_clear_graph_cache(void);

#ifdef __cplusplus
}
#endif

#endif /* CFC_H */
