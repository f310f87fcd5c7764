"""GPU parity of the batched MLP training step: the HIP library, called
through its C ABI, against the fp64 oracle (oracle/mlp_oracle.py) with the
bounds of tests/tolerances.py (mlp_bounds), plus exact structural checks."""
import sys

import numpy as np
import pytest
import torch

from recurrent_cell_amd.inputs import MLP_B, MLP_DIMS, MlpInputs, normal
from tests.tolerances import assert_ok, check_bound, mlp_bounds

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": (37, (5, 9, 3), 0.3),                     # one tile, ragged everything
    "ragged": (300, (48, 70, 33, 51), 0.3),           # widths not multiples of 4 or 16
    "splits": (3000, (48, 256, 128, 51), 0.1),        # several weight-gradient splits, 2 column tiles
    "deep_narrow": (130, (1, 7, 1, 7, 1, 5, 1, 3, 2), 0.5),   # eight layers, width-1 layers
    "headline": (MLP_B, MLP_DIMS, 0.0),               # the 48-256-256-128-51 net at B = 16384
    "max_width": (65, (4096, 33, 4096), 0.1),         # MLP_MAX_DIM-wide input and output layers
}


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def M():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from recurrent_cell_amd import mlp
    mlp.lib()
    return mlp


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def run_step(M, x):
    dims = x.dims
    params = M.pack_params([dev(w) for w in x.W], [dev(b) for b in x.b], dims)
    out = M.mlp_train_step(dev(x.X), dev(x.T), dims, params)
    return out, params


@pytest.mark.parametrize("case", list(CASES))
def test_mlp_train_step_matches_oracle(M, case):
    from oracle.mlp_oracle import mlp_train_step
    B, dims, bias = CASES[case]
    say("mlp train step parity", case, B, dims)
    x = MlpInputs(B, dims, seed=11, bias_scale=bias)
    out, _ = run_step(M, x)
    ref = mlp_train_step(x.X, x.T, x.W, x.b)
    S = M.mlp_weight_grad_splits(B)
    ks = -(-B // S)
    bd = mlp_bounds(x.X, x.W, x.b, ref, ks + 31)
    L = len(dims) - 1
    for l in range(L):
        assert_ok(check_bound("act%d" % l, host(out.act[l]), ref["post"][l], bd["act"][l]))
    loss = float(host(out.loss)[0])
    assert abs(loss - ref["loss"]) <= bd["loss_fn"](x.T), (loss, ref["loss"])
    grads = host(out.grads)
    w_off, b_off, total = M.mlp_param_offsets(dims)
    used = np.zeros(total, bool)
    for l in range(L):
        n_out, n_in = dims[l + 1], dims[l]
        gW = grads[w_off[l]:w_off[l] + n_out * n_in].reshape(n_out, n_in)
        gb = grads[b_off[l]:b_off[l] + n_out]
        used[w_off[l]:w_off[l] + n_out * n_in] = True
        used[b_off[l]:b_off[l] + n_out] = True
        assert_ok(check_bound("gW%d" % l, gW, ref["gW"][l], bd["gW"][l]))
        assert_ok(check_bound("gb%d" % l, gb, ref["gb"][l], bd["gb"][l]))
    assert not grads[~used].any(), "layout gaps of the gradient must be zero"


def test_mlp_train_step_is_deterministic_and_overwrites(M):
    B, dims, bias = CASES["splits"]
    say("mlp determinism", B, dims)
    x = MlpInputs(B, dims, seed=12, bias_scale=bias)
    dimsl = list(dims)
    params = M.pack_params([dev(w) for w in x.W], [dev(b) for b in x.b], dimsl)
    out = M.MlpBuffers.allocate(B, dimsl, "cuda")
    out.grads.fill_(float("nan"))
    out.loss.fill_(float("nan"))
    Xd, Td = dev(x.X), dev(x.T)
    M.mlp_train_step(Xd, Td, dimsl, params, out=out)
    g1, l1 = host(out.grads).copy(), host(out.loss).copy()
    assert np.isfinite(g1).all() and np.isfinite(l1).all()
    for _ in range(2):
        out.grads.fill_(1e30)
        M.mlp_train_step(Xd, Td, dimsl, params, out=out)
        np.testing.assert_array_equal(host(out.grads).view(np.uint32), g1.view(np.uint32))
        np.testing.assert_array_equal(host(out.loss).view(np.uint32), l1.view(np.uint32))


def test_mlp_step_equals_its_layer_calls(M):
    """The fused step and the single-layer ABI calls (forward, loss, upstream
    gradient, weight gradient) run the same kernels on the same splits: the
    same bits."""
    B, dims, bias = CASES["ragged"]
    say("mlp step == layer calls", B, dims)
    x = MlpInputs(B, dims, seed=13, bias_scale=bias)
    out, params = run_step(M, x)
    L = len(dims) - 1
    Ws = [dev(w) for w in x.W]
    bs = [dev(b) for b in x.b]
    h = dev(x.X)
    acts = []
    for l in range(L):
        h = M.mlp_linear_fwd(h, Ws[l], bs[l], relu=l < L - 1)
        acts.append(h)
    dY, loss = M.mlp_mse_loss_grad(acts[-1], dev(x.T))
    grads = {}
    g = dY
    for l in range(L - 1, -1, -1):
        xin = dev(x.X) if l == 0 else acts[l - 1]
        grads[l] = M.mlp_linear_bwd_weight(g, xin)
        if l > 0:
            g = M.mlp_linear_bwd_data(g, Ws[l], mask=acts[l - 1])
    for l in range(L):
        np.testing.assert_array_equal(host(acts[l]), host(out.act[l]))
    np.testing.assert_array_equal(host(loss), host(out.loss))
    per = M.unpack(out.grads, list(dims))
    for l in range(L):
        np.testing.assert_array_equal(host(grads[l][0]), host(per[l][0]), err_msg="gW%d" % l)
        np.testing.assert_array_equal(host(grads[l][1]), host(per[l][1]), err_msg="gb%d" % l)


@pytest.mark.parametrize("M_,n_in,n_out,relu,bias", [(1, 1, 1, True, True), (129, 48, 256, True, True),
                                                     (1000, 256, 51, False, True), (77, 13, 300, True, False),
                                                     (4096, 256, 256, True, True)])
def test_mlp_linear_fwd_matches_oracle(M, M_, n_in, n_out, relu, bias):
    from oracle.mlp_oracle import linear_fwd
    say("mlp linear fwd", M_, n_in, n_out, relu, bias)
    X = normal((M_, n_in), 21, 0)
    W = normal((n_out, n_in), 21, 1) / np.float32(np.sqrt(n_in))
    b = normal((n_out,), 21, 2) if bias else None
    Y = host(M.mlp_linear_fwd(dev(X), dev(W), dev(b) if bias else None, relu=relu))
    ref = linear_fwd(X, W, b, relu)
    mass = np.abs(X.astype(np.float64)) @ np.abs(W.astype(np.float64)).T + (np.abs(b) if bias else 0.0)
    assert_ok(check_bound("Y", Y, ref, 4.0 * np.sqrt(n_in + 1) * 2.0 ** -24 * mass))


@pytest.mark.parametrize("M_,n_in,n_out,mask", [(129, 48, 256, True), (1000, 128, 51, True), (37, 300, 5, False),
                                                (4096, 256, 256, True)])
def test_mlp_linear_bwd_data_matches_oracle(M, M_, n_in, n_out, mask):
    from oracle.mlp_oracle import linear_bwd_data
    say("mlp linear bwd data", M_, n_in, n_out, mask)
    dY = normal((M_, n_out), 22, 0)
    W = normal((n_out, n_in), 22, 1)
    Xm = normal((M_, n_in), 22, 2) if mask else None
    dX = host(M.mlp_linear_bwd_data(dev(dY), dev(W), mask=dev(Xm) if mask else None))
    ref = linear_bwd_data(dY, W, Xm)
    mass = np.abs(dY.astype(np.float64)) @ np.abs(W.astype(np.float64))
    assert_ok(check_bound("dX", dX, ref, 4.0 * np.sqrt(n_out) * 2.0 ** -24 * mass))
    if mask:
        assert not dX[Xm <= 0].any()


@pytest.mark.parametrize("M_,n_in,n_out,with_bias", [(1, 3, 2, True), (37, 5, 9, True), (3000, 48, 256, True),
                                                     (16384, 128, 51, True), (2000, 33, 7, False)])
def test_mlp_linear_bwd_weight_matches_oracle(M, M_, n_in, n_out, with_bias):
    from oracle.mlp_oracle import linear_bwd_weight
    say("mlp linear bwd weight", M_, n_in, n_out, with_bias)
    dY = normal((M_, n_out), 23, 0)
    X = normal((M_, n_in), 23, 1)
    gW, gb = M.mlp_linear_bwd_weight(dev(dY), dev(X), with_bias=with_bias)
    rW, rb = linear_bwd_weight(dY, X)
    ks = -(-M_ // M.mlp_weight_grad_splits(M_)) + 31
    massW = np.abs(dY.astype(np.float64)).T @ np.abs(X.astype(np.float64))
    assert_ok(check_bound("gW", host(gW), rW, 4.0 * np.sqrt(ks + 1) * 2.0 ** -24 * massW + 2.0 ** -24 * np.abs(rW)))
    if with_bias:
        massb = np.abs(dY.astype(np.float64)).sum(axis=0)
        assert_ok(check_bound("gb", host(gb), rb, 4.0 * np.sqrt(ks + 1) * 2.0 ** -24 * massb + 2.0 ** -24 * np.abs(rb)))
    else:
        assert gb is None


def test_mlp_mse_matches_oracle(M):
    from oracle.mlp_oracle import mse_loss_grad
    say("mlp mse")
    Y = normal((1001, 51), 24, 0)
    T = normal((1001, 51), 24, 1)
    dY, loss = M.mlp_mse_loss_grad(dev(Y), dev(T))
    rl, rg = mse_loss_grad(Y, T)
    assert abs(float(host(loss)[0]) - rl) <= 4 * 2.0 ** -24 * rl
    assert_ok(check_bound("dY", host(dY), rg, 3 * 2.0 ** -24 * np.abs(rg)))


def test_mlp_integer_data_is_exact(M):
    """Small integers: every product and partial sum is an exact fp32
    integer, so the forward and the weight gradient are exact."""
    say("mlp exact integers")
    rng = np.random.default_rng(25)
    X = rng.integers(-3, 4, (2000, 40)).astype(np.float32)
    W = rng.integers(-3, 4, (24, 40)).astype(np.float32)
    b = rng.integers(-3, 4, 24).astype(np.float32)
    Y = host(M.mlp_linear_fwd(dev(X), dev(W), dev(b), relu=True))
    np.testing.assert_array_equal(Y, np.maximum(X.astype(np.int64) @ W.T.astype(np.int64) + b, 0))
    dY = rng.integers(-3, 4, (2000, 24)).astype(np.float32)
    gW, gb = M.mlp_linear_bwd_weight(dev(dY), dev(X))
    np.testing.assert_array_equal(host(gW), dY.T.astype(np.int64) @ X.astype(np.int64))
    np.testing.assert_array_equal(host(gb), dY.astype(np.int64).sum(axis=0))
