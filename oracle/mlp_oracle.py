"""CPU oracle for the batched MLP training step -- TEST INFRASTRUCTURE ONLY.

Plain fp64 numpy, written from the definitions (page "H100 Epoch
Optimization Phase 2: Kernel Occupancy & cuBLAS", Implementation Tasks:
Task 1 batches each layer's forward as one [B, in] x [in, out] product
followed by bias and ReLU; Task 2 forms the weight gradient as dW = dY^T X
summed over the batch and the upstream gradient as dX = dY W).  Conventions
where the page is silent (this library's reading):
  - layer l maps dims[l] -> dims[l+1] with W_l [dims[l+1], dims[l]] and
    b_l [dims[l+1]]: a_l = x_{l-1} W_l^T + b_l;
  - ReLU after every layer but the last; ReLU'(0) = 0 (a unit passes the
    gradient only where its pre-activation is > 0);
  - loss = mean over all B * dims[-1] outputs of (y - t)^2, so
    dL/dy = 2 (y - t) / (B * dims[-1]);
  - no gradient is formed for the input X.
A matrix product (numpy matmul in fp64) is the one library step; nothing is
blocked, fused or reordered beyond the definitions above.
"""
import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def mlp_forward(X, Ws, bs):
    """Pre-activations a_l and outputs x_l of every layer (fp64 lists)."""
    x = _f64(X)
    pre, post = [], []
    L = len(Ws)
    for l in range(L):
        a = x @ _f64(Ws[l]).T + _f64(bs[l])
        x = np.maximum(a, 0.0) if l < L - 1 else a
        pre.append(a)
        post.append(x)
    return pre, post


def mlp_train_step(X, T, Ws, bs):
    """One training step's loss and gradients in fp64.

    Returns dict(loss, gW (list), gb (list), pre (list), post (list),
    dA (list: dL/da_l of every layer))."""
    X = _f64(X)
    T = _f64(T)
    pre, post = mlp_forward(X, Ws, bs)
    L = len(Ws)
    y = post[-1]
    n = y.size
    loss = float(np.sum((y - T) ** 2) / n)
    g = 2.0 * (y - T) / n                       # dL/dy = dL/da of the last (linear) layer
    gW = [None] * L
    gb = [None] * L
    dA = [None] * L
    for l in range(L - 1, -1, -1):
        dA[l] = g
        x_in = X if l == 0 else post[l - 1]
        gW[l] = g.T @ x_in                       # dW = dY^T X, summed over the batch
        gb[l] = g.sum(axis=0)
        if l > 0:
            dx = g @ _f64(Ws[l])                 # dX = dY W
            g = dx * (pre[l - 1] > 0.0)          # through the previous layer's ReLU
    return dict(loss=loss, gW=gW, gb=gb, pre=pre, post=post, dA=dA)


def linear_fwd(X, W, b, relu):
    """One layer's forward (Task 1): X W^T + b, then ReLU when relu."""
    a = _f64(X) @ _f64(W).T
    if b is not None:
        a = a + _f64(b)
    return np.maximum(a, 0.0) if relu else a


def linear_bwd_data(dY, W, mask):
    """One layer's upstream gradient (Task 2): dY W, zeroed where mask <= 0."""
    dx = _f64(dY) @ _f64(W)
    return dx if mask is None else dx * (_f64(mask) > 0.0)


def linear_bwd_weight(dY, X):
    """One layer's parameter gradients (Task 2): dY^T X and the column sums of dY."""
    return _f64(dY).T @ _f64(X), _f64(dY).sum(axis=0)


def mse_loss_grad(Y, T):
    """Mean of (Y - T)^2 and its gradient 2 (Y - T) / Y.size."""
    d = _f64(Y) - _f64(T)
    return float(np.sum(d * d) / d.size), 2.0 * d / d.size
