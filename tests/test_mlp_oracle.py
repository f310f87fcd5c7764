"""Pins of the MLP oracle (CPU only): a library autograd in fp64, central
finite differences, the least-squares optimum, and the ReLU'(0) = 0
convention."""
import numpy as np
import pytest
import torch

from oracle.mlp_oracle import mlp_forward, mlp_train_step
from recurrent_cell_amd.inputs import MLP_DIMS, MlpInputs


def _torch_step(x):
    X = torch.tensor(x.X, dtype=torch.float64)
    T = torch.tensor(x.T, dtype=torch.float64)
    Ws = [torch.tensor(w, dtype=torch.float64, requires_grad=True) for w in x.W]
    bs = [torch.tensor(b, dtype=torch.float64, requires_grad=True) for b in x.b]
    h = X
    for l in range(len(Ws)):
        h = torch.nn.functional.linear(h, Ws[l], bs[l])
        if l < len(Ws) - 1:
            h = torch.relu(h)
    loss = torch.nn.functional.mse_loss(h, T)
    loss.backward()
    return loss.item(), [w.grad.numpy() for w in Ws], [b.grad.numpy() for b in bs], h.detach().numpy()


@pytest.mark.parametrize("B,dims,bias", [(64, MLP_DIMS, 0.0), (37, (5, 9, 3), 0.3), (8, (48, 51), 0.1)])
def test_mlp_oracle_matches_torch_autograd(B, dims, bias):
    x = MlpInputs(B, dims, seed=3, bias_scale=bias)
    r = mlp_train_step(x.X, x.T, x.W, x.b)
    loss, gW, gb, y = _torch_step(x)
    assert abs(r["loss"] - loss) <= 1e-13 * abs(loss)
    np.testing.assert_allclose(r["post"][-1], y, rtol=1e-13, atol=1e-14)
    for l in range(len(dims) - 1):
        np.testing.assert_allclose(r["gW"][l], gW[l], rtol=1e-11, atol=1e-16)
        np.testing.assert_allclose(r["gb"][l], gb[l], rtol=1e-11, atol=1e-16)


def test_mlp_oracle_central_differences():
    x = MlpInputs(6, (3, 5, 4, 2), seed=4, bias_scale=0.5)
    W = [w.astype(np.float64) for w in x.W]
    b = [v.astype(np.float64) for v in x.b]
    r = mlp_train_step(x.X, x.T, W, b)
    h = 1e-6

    def loss_at(Wp, bp):
        return mlp_train_step(x.X, x.T, Wp, bp)["loss"]
    for l in range(3):
        for idx in np.ndindex(W[l].shape):
            Wp = [w.copy() for w in W]
            Wm = [w.copy() for w in W]
            Wp[l][idx] += h
            Wm[l][idx] -= h
            fd = (loss_at(Wp, b) - loss_at(Wm, b)) / (2 * h)
            assert abs(fd - r["gW"][l][idx]) <= 1e-7, (l, idx)
        for j in range(b[l].size):
            bp = [v.copy() for v in b]
            bm = [v.copy() for v in b]
            bp[l][j] += h
            bm[l][j] -= h
            fd = (loss_at(W, bp) - loss_at(W, bm)) / (2 * h)
            assert abs(fd - r["gb"][l][j]) <= 1e-7, (l, j)


def test_mlp_oracle_gradient_vanishes_at_the_least_squares_optimum():
    """One linear layer: at the least-squares solution (a library solver) the
    gradient of the mean squared error is zero."""
    rng = np.random.default_rng(5)
    X = rng.standard_normal((200, 7))
    T = rng.standard_normal((200, 3))
    A = np.hstack([X, np.ones((200, 1))])
    sol = np.linalg.lstsq(A, T, rcond=None)[0]      # [8, 3]
    W, b = sol[:7].T, sol[7]
    r = mlp_train_step(X, T, [W], [b])
    assert np.abs(r["gW"][0]).max() < 1e-14 and np.abs(r["gb"][0]).max() < 1e-14
    # and away from it the gradient is the residual's projection, not zero
    r2 = mlp_train_step(X, T, [W + 0.1], [b])
    assert np.abs(r2["gW"][0]).max() > 1e-3


def test_mlp_oracle_relu_derivative_at_zero():
    """A hidden unit whose pre-activation is exactly 0 passes no gradient."""
    X = np.array([[3.0, 3.0], [1.0, 1.0]])
    T = np.array([[1.0], [2.0]])
    W = [np.array([[1.0, -1.0]]), np.array([[2.0]])]
    b = [np.zeros(1), np.array([0.5])]
    r = mlp_train_step(X, T, W, b)
    assert (r["pre"][0] == 0.0).all()
    assert not r["gW"][0].any() and not r["gb"][0].any()
    assert r["gb"][1][0] != 0.0
    pre, post = mlp_forward(X, W, b)
    assert (post[-1] == 0.5).all()


def test_single_layer_helpers_match_torch():
    from oracle.mlp_oracle import linear_bwd_data, linear_bwd_weight, linear_fwd, mse_loss_grad
    rng = np.random.default_rng(6)
    X = rng.standard_normal((33, 7))
    W = rng.standard_normal((5, 7))
    b = rng.standard_normal(5)
    tX, tW, tb = (torch.tensor(a, requires_grad=True) for a in (X, W, b))
    a = torch.nn.functional.linear(tX, tW, tb)
    np.testing.assert_allclose(linear_fwd(X, W, b, False), a.detach().numpy(), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(linear_fwd(X, W, b, True), torch.relu(a).detach().numpy(), rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(linear_fwd(X, W, None, False), (tX @ tW.T).detach().numpy(), rtol=1e-14, atol=1e-14)
    dY = rng.standard_normal((33, 5))
    a.backward(torch.tensor(dY))
    np.testing.assert_allclose(linear_bwd_data(dY, W, None), tX.grad.numpy(), rtol=1e-13, atol=1e-14)
    gW, gb = linear_bwd_weight(dY, X)
    np.testing.assert_allclose(gW, tW.grad.numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(gb, tb.grad.numpy(), rtol=1e-13, atol=1e-14)
    mask = rng.standard_normal((33, 7))
    np.testing.assert_array_equal(linear_bwd_data(dY, W, mask)[mask <= 0], 0.0)
    Y = rng.standard_normal((9, 4))
    T = rng.standard_normal((9, 4))
    tY = torch.tensor(Y, requires_grad=True)
    l = torch.nn.functional.mse_loss(tY, torch.tensor(T))
    l.backward()
    loss, g = mse_loss_grad(Y, T)
    assert abs(loss - l.item()) <= 1e-14 * l.item()
    np.testing.assert_allclose(g, tY.grad.numpy(), rtol=1e-13, atol=1e-15)
