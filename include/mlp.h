/*
 * mlp.h -- C ABI of the batched MLP training step in libcfc.so (gfx950).
 *
 * Source.  "H100 Epoch Optimization Phase 2: Kernel Occupancy & cuBLAS",
 * section Implementation Tasks:
 *   - Task 1: each layer's forward over the whole batch is one matrix product
 *     [B, in] x [in, out], then the bias and a ReLU;
 *   - Task 2: the backward forms the weight gradient as dW = dY^T X (an outer
 *     product summed over the batch, no atomics) and the upstream gradient
 *     as dX = dY W;
 *   - Task 3: parameters live in ONE flat buffer.
 * Conventions this library fixes where the page is silent:
 *   - n_layers layers, layer l maps dims[l] -> dims[l+1]: W_l [dims[l+1],
 *     dims[l]] row-major, b_l [dims[l+1]], a_l = x_{l-1} W_l^T + b_l;
 *     ReLU after every layer but the last; ReLU'(0) = 0;
 *   - loss = mean over B * dims[n_layers] outputs of (y - t)^2, so the
 *     output gradient is 2 (y - t) / (B * dims[n_layers]);
 *   - no gradient is formed for the input X.
 *
 * Flat parameter layout (mlp_param_offsets): W_0, b_0, W_1, b_1, ... in that
 * order, each tensor starting at a multiple of 4 floats (16 bytes), the gaps
 * zero in every gradient the library writes.  The gradient buffer has the
 * same layout as the parameters.
 *
 * Conventions shared with cfc.h: float* are DEVICE pointers to fp32 arrays
 * owned by the caller; `stream` is a hipStream_t (NULL = null stream); calls
 * only enqueue; return CFC_OK or a negative cfc_status with cfc_last_error()
 * set; outputs must not overlap inputs (CFC_EINVAL).  Every sum has an order
 * fixed by the sizes (no atomics), so repeated calls give identical bits.
 * Arithmetic is fp32 on the matrix cores (v_mfma_f32_16x16x4f32); the batch
 * reductions (weight and bias gradients, loss) add fixed splits in fp64.
 */
#ifndef MLP_H
#define MLP_H

#include <stddef.h>
#include <stdint.h>

#include "cfc.h"

#ifdef __cplusplus
extern "C" {
#endif

#define MLP_MAX_LAYERS 8
#define MLP_MAX_DIM 4096
#define MLP_MAX_B (1 << 24)

/* Offsets (in floats) of W_l and b_l in the flat layout; returns the total
 * number of floats of the flat buffer (padding included), or -1 for bad
 * dims (n_layers in [1, MLP_MAX_LAYERS], dims[i] in [1, MLP_MAX_DIM]).
 * w_off and b_off (nullable) receive n_layers entries each.  Host only. */
int64_t mlp_param_offsets(const int* dims, int n_layers, int64_t* w_off, int64_t* b_off);

/* One layer's forward (Task 1): Y = X W^T + b, then ReLU when relu != 0.
 *   X [M, n_in], W [n_out, n_in], b [n_out] (nullable: no bias), Y [M, n_out].
 * M in [0, MLP_MAX_B]; n_in, n_out in [1, MLP_MAX_DIM]. */
int mlp_linear_fwd(const float* X, const float* W, const float* b, float* Y, int M, int n_in, int n_out, int relu,
                   void* stream);

/* One layer's upstream gradient (Task 2): dX = dY W, then, when mask is not
 * NULL, dX is zeroed where mask <= 0 (mask = the layer's input after the
 * previous ReLU: the previous layer's ReLU'(a) = [a > 0] = [x > 0]).
 *   dY [M, n_out], W [n_out, n_in], mask [M, n_in] (nullable), dX [M, n_in]. */
int mlp_linear_bwd_data(const float* dY, const float* W, const float* mask, float* dX, int M, int n_in, int n_out,
                        void* stream);

/* One layer's parameter gradients (Task 2): gW = dY^T X [n_out, n_in] and
 * gb = column sums of dY [n_out], both summed over the M rows and
 * OVERWRITTEN.  The M rows are cut into mlp_weight_grad_splits(M) fixed
 * splits; each split is one fp32 matrix-core chain, and the splits are added
 * in fp64 in a fixed order (the batch-axis reducer of cfc.h).
 *   dY [M, n_out], X [M, n_in], gW [n_out, n_in], gb [n_out] (nullable);
 *   ws: device workspace of mlp_linear_bwd_weight_workspace_bytes() bytes. */
int mlp_linear_bwd_weight(const float* dY, const float* X, float* gW, float* gb, int M, int n_in, int n_out,
                          void* ws, size_t ws_bytes, void* stream);
size_t mlp_linear_bwd_weight_workspace_bytes(int M, int n_in, int n_out);
int mlp_weight_grad_splits(int M);

/* Mean squared error and its gradient: dY = 2 (Y - T) / (M N) and
 * loss = mean of (Y - T)^2 (one float, OVERWRITTEN).  The per-split partial
 * sums are fp64, added in a fixed order.
 *   Y, T, dY [M, N]; loss [1]; ws: mlp_mse_workspace_bytes(M) bytes. */
int mlp_mse_loss_grad(const float* Y, const float* T, float* dY, float* loss, int M, int N, void* ws,
                      size_t ws_bytes, void* stream);
size_t mlp_mse_workspace_bytes(int M);

/* One whole training step over the batch: the forward of every layer, the
 * loss, the backward, and the gradients of every parameter.
 *   X [B, dims[0]], T [B, dims[n_layers]];
 *   params, grads: flat buffers of mlp_param_offsets() floats (grads
 *     OVERWRITTEN; its layout gaps written as 0);
 *   act: n_layers pointers, act[l] [B, dims[l+1]] receives layer l's output
 *     (after its ReLU; act[n_layers-1] is the network output);
 *   loss [1] OVERWRITTEN;
 *   ws: mlp_train_step_workspace_bytes() bytes of device memory.
 * B in [1, MLP_MAX_B].  Launches: one per layer forward, one for the loss,
 * one per layer > 0 for dX, one for the weight and bias gradient splits of
 * every group of layers whose widths allow the same operand loads (one or
 * two groups), ONE fixed-order reduction of all splits and of the loss. */
int mlp_train_step(const float* X, const float* T, int B, const int* dims, int n_layers, const float* params,
                   float* grads, float* const* act, float* loss, void* ws, size_t ws_bytes, void* stream);
size_t mlp_train_step_workspace_bytes(int B, const int* dims, int n_layers);

#ifdef __cplusplus
}
#endif

#endif /* MLP_H */
