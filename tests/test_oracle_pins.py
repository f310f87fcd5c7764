"""Pins of the CPU oracle to things other than itself (CPU only, no GPU).

The pages print no worked numeric example of the cell, so the oracle is pinned by:
  * central finite differences of its own loss (backward vs forward: every
    weight, bias, h0 entry and a sample of u entries);
  * a library routine: with W_f = 0 and W_g = W_h the cell is an Elman tanh
    RNN, which torch.nn.RNN computes (forward, and autograd gradients);
    with the gate driven to 0 or 1 by a large f-bias the cell follows one
    head alone, which pins the gate's sign and the head order;
  * the closed form of a single step (K = 1: no carry; the gradients are
    outer products of the written-out dp with z), computed here with numpy;
  * exact special cases (gate = 0.5 exactly when a_f = 0; gW_f = 0 exactly
    when the g and h heads coincide), invariants (gate in (0,1), |h_t| <= 1),
    descent of the loss along -grad, linearity over the batch;
  * the fp32 instantiation against the fp64 one within the fp32 bounds.
A plausible slip -- a dropped term, a flipped sign, swapped heads, a transposed
W, u and h swapped in z, a missing BPTT carry -- fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

from recurrent_cell_amd.inputs import CONFIGS, cfc_inputs
from tests.tolerances import assert_ok, check_act, check_grad, grad_mass


def _loss(oracle_mod, u, y, h0, W, bias):
    return oracle_mod.forward(u, y, h0, W, bias, "f64")[0]


def test_finite_differences_tiny(oracle_mod):
    """Central differences on the tiny configuration (B=4, C=16, n_x=8, K=4),
    with non-zero biases, all 3*16*24 weights, 48 biases and 64 h0 entries."""
    x = cfc_inputs(**CONFIGS["tiny"], seed=3, bias_scale=0.5)
    u, y, h0 = (a.astype(np.float64) for a in (x.u, x.y, x.h0))
    W, bias = x.W.astype(np.float64), x.bias.astype(np.float64)
    r = oracle_mod.train(u, y, h0, W, bias, "f64", want_du=True)
    eps = 1e-6

    def fd(arr, idx):
        old = arr[idx]
        arr[idx] = old + eps
        lp = _loss(oracle_mod, u, y, h0, W, bias)
        arr[idx] = old - eps
        lm = _loss(oracle_mod, u, y, h0, W, bias)
        arr[idx] = old
        return (lp - lm) / (2 * eps)

    for arr, grad in ((W, r["gW"]), (bias, r["gb"]), (h0, r["dh0"])):
        num = np.array([fd(arr, idx) for idx in np.ndindex(arr.shape)]).reshape(arr.shape)
        err = np.abs(num - grad)
        assert np.all(err <= 1e-6 * np.maximum(1.0, np.abs(grad))), err.max()
    rng = np.random.default_rng(0)
    for _ in range(40):
        idx = tuple(int(rng.integers(0, s)) for s in u.shape)
        assert abs(fd(u, idx) - r["du"][idx]) <= 1e-6 * max(1.0, abs(r["du"][idx]))


def _rnn(Wq, bq, n_x, u, h0, y):
    """torch.nn.RNN (tanh) with W_ih = Wq[:, :n_x], W_hh = Wq[:, n_x:], b_ih = bq,
    b_hh = 0; loss 0.5 * sum (h_t - y_t)^2.  Returns outputs and gradients."""
    C = Wq.shape[0]
    rnn = torch.nn.RNN(n_x, C, nonlinearity="tanh", bias=True, dtype=torch.float64)
    with torch.no_grad():
        rnn.weight_ih_l0.copy_(torch.from_numpy(Wq[:, :n_x]))
        rnn.weight_hh_l0.copy_(torch.from_numpy(Wq[:, n_x:]))
        rnn.bias_ih_l0.copy_(torch.from_numpy(bq))
        rnn.bias_hh_l0.zero_()
    h0t = torch.from_numpy(h0.copy())[None].requires_grad_(True)
    out, _ = rnn(torch.from_numpy(u), h0t)
    loss = 0.5 * ((out - torch.from_numpy(y)) ** 2).sum()
    loss.backward()
    gw = torch.cat([rnn.weight_ih_l0.grad, rnn.weight_hh_l0.grad], dim=1).numpy()
    return dict(h=out.detach().numpy(), loss=loss.item(), gW=gw,
                gb=rnn.bias_ih_l0.grad.numpy(), dh0=h0t.grad[0].numpy())


@pytest.mark.parametrize("cfg", ["tiny", "pages"])
def test_tied_heads_reduce_to_torch_rnn(oracle_mod, cfg):
    """W_f = 0, W_g = W_h, b_g = b_h: h_t = tanh(W_g z + b_g) whatever the gate,
    so the cell is torch.nn.RNN; the gradient of the tied weight is gW_g + gW_h
    and gW_f, gb_f are exactly zero."""
    d = dict(CONFIGS[cfg])
    if cfg == "pages":
        d.update(B=4, K=8)
    x = cfc_inputs(**d, seed=5, bias_scale=0.3)
    n_x = d["n_x"]
    W = x.W.astype(np.float64)
    bias = x.bias.astype(np.float64)
    W[0] = 0.0
    W[2] = W[1]
    bias[2] = bias[1]
    u, y, h0 = (a.astype(np.float64) for a in (x.u, x.y, x.h0))
    r = oracle_mod.train(u, y, h0, W, bias, "f64")
    t = _rnn(W[1], bias[1], n_x, u, h0, y)
    np.testing.assert_allclose(r["h_hist"][1:], t["h"], rtol=0, atol=1e-13)
    assert abs(r["loss"] - t["loss"]) <= 1e-11 * abs(t["loss"])
    np.testing.assert_allclose(r["gW"][1] + r["gW"][2], t["gW"], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(r["gb"][1] + r["gb"][2], t["gb"], rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(r["dh0"], t["dh0"], rtol=1e-11, atol=1e-11)
    assert np.all(r["gW"][0] == 0.0) and np.all(r["gb"][0] == 0.0)


@pytest.mark.parametrize("beta,head", [(40.0, 2), (-40.0, 1)])
def test_gate_limits_follow_one_head(oracle_mod, beta, head):
    """b_f = +40 drives gate = 1/(1+e^40) ~ 4e-18, so h_t = hh (head h);
    b_f = -40 drives gate to 1 (exactly, in fp64), so h_t = g (head g).
    With W_g != W_h this pins the sign of the gate and the head order."""
    d = CONFIGS["tiny"]
    x = cfc_inputs(**d, seed=7, bias_scale=0.3)
    W = x.W.astype(np.float64)
    bias = x.bias.astype(np.float64)
    W[0] = 0.0
    bias[0] = beta
    u, y, h0 = (a.astype(np.float64) for a in (x.u, x.y, x.h0))
    r = oracle_mod.train(u, y, h0, W, bias, "f64")
    t = _rnn(W[head], bias[head], d["n_x"], u, h0, y)
    np.testing.assert_allclose(r["h_hist"][1:], t["h"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["gW"][head], t["gW"], rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(r["gb"][head], t["gb"], rtol=1e-9, atol=1e-12)
    other = 1 if head == 2 else 2
    assert np.abs(r["gW"][other]).max() < 1e-12


def test_gate_is_exactly_half_when_f_preactivation_is_zero(oracle_mod):
    x = cfc_inputs(**CONFIGS["tiny"], seed=2)
    W = x.W.astype(np.float64)
    W[0] = 0.0
    _, h_hist, act = oracle_mod.forward(x.u, x.y, x.h0, W, x.bias, "f64")
    assert np.all(act[:, 0] == 0.5)
    np.testing.assert_array_equal(h_hist[1:], 0.5 * act[:, 1] + 0.5 * act[:, 2])


@pytest.mark.parametrize("cfg", ["tiny", "pages"])
def test_invariants_gate_open_interval_and_convex_h(oracle_mod, cfg):
    x = cfc_inputs(**CONFIGS[cfg], seed=0)
    for prec in ("f64", "f32"):
        _, h_hist, act = oracle_mod.forward(x.u, x.y, x.h0, x.W, x.bias, prec)
        gate = act[:, 0]
        assert np.all(gate > 0) and np.all(gate < 1)
        assert np.all(np.abs(h_hist[1:]) <= 1.0)
        assert np.all(np.abs(act[:, 1:]) <= 1.0)
        # h_t lies between g and hh (a convex combination)
        lo = np.minimum(act[:, 1], act[:, 2])
        hi = np.maximum(act[:, 1], act[:, 2])
        tol = 4 * np.finfo(h_hist.dtype).eps
        assert np.all(h_hist[1:] >= lo - tol) and np.all(h_hist[1:] <= hi + tol)


def test_descent_along_negative_gradient(oracle_mod):
    x = cfc_inputs(**CONFIGS["tiny"], seed=11, bias_scale=0.2)
    W, bias = x.W.astype(np.float64), x.bias.astype(np.float64)
    r = oracle_mod.train(x.u, x.y, x.h0, W, bias, "f64")
    gnorm = math.sqrt((r["gW"] ** 2).sum() + (r["gb"] ** 2).sum())
    for scale in (1e-3, 1e-2):
        eta = scale / gnorm
        l1 = _loss(oracle_mod, x.u, x.y, x.h0, W - eta * r["gW"], bias - eta * r["gb"])
        assert l1 < r["loss"]
        # first-order prediction of the decrease holds to second order
        pred = eta * gnorm ** 2
        assert abs((r["loss"] - l1) - pred) <= 0.05 * pred


def test_single_step_gradients_match_the_closed_form(oracle_mod):
    """At K = 1 there is no carry.  With z = [u_1; h_0], a_q = W_q z + b_q,
    gate = 1 / (1 + e^{a_f}), g = tanh a_g, hh = tanh a_h, h = gate g + (1 - gate) hh
    and r = h - y, the per-sample pre-activation gradients are
      dp_f = r (g - hh) (-gate (1 - gate)),  dp_g = r gate (1 - g^2),
      dp_h = r (1 - gate) (1 - hh^2),
    the weight gradients their outer products with z summed over the batch,
    gb_q the sums of dp_q, dh0 the recurrent columns of sum_q W_q^T dp_q and
    the loss 0.5 sum r^2 -- written out here with numpy, not the oracle's code."""
    B, C, n_x = 5, 7, 3
    x = cfc_inputs(B=B, C=C, n_x=n_x, K=1, seed=21, bias_scale=0.3)
    u, y, h0, W, bias = (a.astype(np.float64) for a in (x.u, x.y, x.h0, x.W, x.bias))
    z = np.concatenate([u[0], h0], axis=1)                         # [B, n_in]
    a = np.einsum("qck,bk->qbc", W, z) + bias[:, None, :]          # [3, B, C]
    gate, g, hh = 1.0 / (1.0 + np.exp(a[0])), np.tanh(a[1]), np.tanh(a[2])
    h = gate * g + (1.0 - gate) * hh
    r = h - y[0]
    dp = np.stack([r * (g - hh) * (-gate * (1.0 - gate)),
                   r * gate * (1.0 - g ** 2),
                   r * (1.0 - gate) * (1.0 - hh ** 2)])            # [3, B, C]
    gW = np.einsum("qbc,bk->qck", dp, z)
    gb = dp.sum(axis=1)
    dh0 = np.einsum("qck,qbc->bk", W, dp)[:, n_x:]
    out = oracle_mod.train(x.u, x.y, x.h0, x.W, x.bias, "f64")
    np.testing.assert_allclose(out["h_hist"][1], h, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(out["act"][0], np.stack([gate, g, hh]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(out["gW"], gW, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["gb"], gb, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["dh0"], dh0, rtol=1e-12, atol=1e-14)
    assert abs(out["loss"] - 0.5 * (r ** 2).sum()) <= 1e-12 * (r ** 2).sum()


def test_batch_linearity_and_per_sample_scratch(oracle_mod):
    """S[b] depends on sample b only (bitwise), and gW = sum_b gW(sample b alone)."""
    x = cfc_inputs(**CONFIGS["tiny"], seed=4, bias_scale=0.1)
    full = oracle_mod.train(x.u, x.y, x.h0, x.W, x.bias, "f64")
    acc_W = np.zeros_like(full["gW"])
    acc_b = np.zeros_like(full["gb"])
    for b in range(x.h0.shape[0]):
        one = oracle_mod.train(x.u[:, b:b + 1], x.y[:, b:b + 1], x.h0[b:b + 1], x.W, x.bias, "f64")
        np.testing.assert_array_equal(one["S"][0], full["S"][b])
        np.testing.assert_array_equal(one["Sb"][0], full["Sb"][b])
        np.testing.assert_array_equal(one["h_hist"][:, 0], full["h_hist"][:, b])
        np.testing.assert_array_equal(one["gW"], one["S"][0])
        acc_W += one["gW"]
        acc_b += one["gb"]
    np.testing.assert_allclose(acc_W, full["gW"], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(acc_b, full["gb"], rtol=1e-13, atol=1e-13)


def test_steps_compose_to_train(oracle_mod):
    """The per-step functions chained by hand give the train function's results."""
    x = cfc_inputs(**CONFIGS["tiny"], seed=9, bias_scale=0.2)
    K, B, n_x = x.u.shape
    C = x.h0.shape[1]
    full = oracle_mod.train(x.u, x.y, x.h0, x.W, x.bias, "f64", want_du=True)
    hs = [x.h0.astype(np.float64)]
    acts = []
    for t in range(K):
        h, a = oracle_mod.fwd_step(x.u[t], hs[-1], x.W, x.bias, "f64")
        hs.append(h)
        acts.append(a)
    np.testing.assert_array_equal(np.stack(hs), full["h_hist"])
    S = np.zeros((B, 3, C, n_x + C))
    Sb = np.zeros((B, 3, C))
    carry = np.zeros((B, C))
    for t in range(K, 0, -1):
        carry, du, S, Sb, _ = oracle_mod.bwd_step(x.u[t - 1], hs[t - 1], hs[t], x.y[t - 1], x.W,
                                                  acts[t - 1], carry, S, Sb, "f64")
        np.testing.assert_array_equal(du, full["du"][t - 1])
    np.testing.assert_array_equal(S, full["S"])
    np.testing.assert_array_equal(carry, full["dh0"])
    np.testing.assert_array_equal(oracle_mod.sum_axis0(S.reshape(B, -1), "f64").reshape(3, C, -1), full["gW"])


@pytest.mark.parametrize("cfg", ["tiny", "pages"])
def test_fp32_instantiation_within_fp32_bounds(oracle_mod, cfg):
    x = cfc_inputs(**CONFIGS[cfg], seed=1)
    r64 = oracle_mod.train(x.u, x.y, x.h0, x.W, x.bias, "f64", want_dp=True)
    r32 = oracle_mod.train(x.u, x.y, x.h0, x.W, x.bias, "f32")
    m = grad_mass(x.u, r64["h_hist"], r64["dp"])
    assert_ok(check_act("h_hist", r32["h_hist"], r64["h_hist"]))
    assert_ok(check_act("act", r32["act"], r64["act"]))
    for k in ("S", "Sb", "gW", "gb"):
        assert_ok(check_grad(k, r32[k], r64[k], m[k]))


# ---------------------------------------------------------------- input projection

def test_input_projection_is_the_zero_state_preactivation(oracle_mod):
    """With h_{t-1} = 0 the recurrent columns of z contribute nothing, so the
    forward step's gate, g and hh are the cell functions of X = W_x u + b."""
    x = cfc_inputs(B=5, C=12, n_x=7, K=1, seed=11, bias_scale=0.4)
    X = oracle_mod.input_projection(x.u[0], x.W, x.bias, "f64")          # [B, 3C]
    _, act = oracle_mod.fwd_step(x.u[0], np.zeros_like(x.h0), x.W, x.bias, "f64")
    C = 12
    a_f, a_g, a_h = X[:, :C], X[:, C:2 * C], X[:, 2 * C:]
    np.testing.assert_allclose(act[0], 1.0 / (1.0 + np.exp(a_f)), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(act[1], np.tanh(a_g), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(act[2], np.tanh(a_h), rtol=1e-14, atol=1e-15)


def test_input_projection_special_cases(oracle_mod):
    x = cfc_inputs(B=4, C=6, n_x=5, K=3, seed=12, bias_scale=0.5)
    C, n_x = 6, 5
    b = x.bias.reshape(-1).astype(np.float64)
    # no inputs: X is the bias on every row
    X0 = oracle_mod.input_projection(np.zeros((3, 4, 0), np.float32), x.W[:, :, n_x:], x.bias, "f64")
    np.testing.assert_array_equal(X0, np.broadcast_to(b, X0.shape))
    # one-hot input j: column j of W_x plus the bias, exactly
    for j in range(n_x):
        u = np.zeros((1, n_x), np.float32)
        u[0, j] = 1.0
        Xj = oracle_mod.input_projection(u, x.W, x.bias, "f64")[0]
        np.testing.assert_array_equal(Xj, x.W[:, :, j].reshape(-1).astype(np.float64) + b)
    # rows are independent and the map is affine in u
    Xa = oracle_mod.input_projection(x.u, x.W, x.bias, "f64")
    for t in range(3):
        np.testing.assert_array_equal(Xa[t], oracle_mod.input_projection(x.u[t], x.W, x.bias, "f64"))
    u2 = x.u[0] * 2.0
    lin = oracle_mod.input_projection(u2, x.W, x.bias, "f64") - b
    np.testing.assert_allclose(lin, 2.0 * (Xa[0] - b), rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------- AdamW

def test_adamw_oracle_matches_torch_adamw(oracle_mod):
    """The fp64 oracle against the library routine torch.optim.AdamW (CPU,
    fp64) over three steps with fresh gradients each step."""
    rng = np.random.default_rng(21)
    p0 = rng.standard_normal(257)
    hp = dict(lr=3e-3, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.05)
    tp = torch.tensor(p0.copy(), dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                            weight_decay=hp["weight_decay"])
    p, m, v = p0.copy(), np.zeros_like(p0), np.zeros_like(p0)
    for step in range(1, 4):
        g = rng.standard_normal(257)
        tp.grad = torch.tensor(g, dtype=torch.float64)
        opt.step()
        p, m, v = oracle_mod.adamw_step(p, g, m, v, step=step, **hp)
        np.testing.assert_allclose(p, tp.detach().numpy(), rtol=1e-13, atol=1e-15)
        st = opt.state[tp]
        np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-13, atol=1e-15)


def test_adamw_oracle_special_cases(oracle_mod):
    rng = np.random.default_rng(22)
    p0 = rng.standard_normal(33)
    # zero gradient and zero moments: only the decay acts
    p, m, v = oracle_mod.adamw_step(p0, np.zeros(33), np.zeros(33), np.zeros(33), lr=1e-2, beta1=0.9,
                                    beta2=0.999, eps=1e-8, weight_decay=0.1, step=1)
    np.testing.assert_array_equal(p, p0 * (1.0 - 1e-3))
    assert not m.any() and not v.any()
    # first step, no decay, eps -> 0: the update is lr * sign(g)
    g = rng.standard_normal(33)
    p, _, _ = oracle_mod.adamw_step(p0, g, np.zeros(33), np.zeros(33), lr=1e-2, beta1=0.9, beta2=0.999,
                                    eps=1e-30, weight_decay=0.0, step=1)
    np.testing.assert_allclose(p, p0 - 1e-2 * np.sign(g), rtol=0, atol=1e-15)


@pytest.mark.parametrize("precision", ["f64", "f32"])
def test_thread_count_does_not_change_the_oracle(oracle_mod, precision):
    """The oracle's per-sample loops on several host threads give the bits of
    one thread: samples write disjoint rows and the batch-axis sums stay serial
    in increasing b (this is what makes the all-core CPU baseline the same
    computation as the single-thread one)."""
    x = cfc_inputs(B=9, C=24, n_x=7, K=5, seed=3, bias_scale=0.2)
    u, y, h0, W, bias = (a if precision == "f32" else a.astype(np.float64) for a in (x.u, x.y, x.h0, x.W, x.bias))
    before = oracle_mod.threads()
    try:
        oracle_mod.set_threads(1)
        one = oracle_mod.train(u, y, h0, W, bias, precision, want_du=True, want_dp=True)
        r1 = oracle_mod.reduce_axis0_f64(x.u.reshape(-1, 7 * 9)[:, :50].copy())
        oracle_mod.set_threads(4)
        assert oracle_mod.threads() == 4
        many = oracle_mod.train(u, y, h0, W, bias, precision, want_du=True, want_dp=True)
        r4 = oracle_mod.reduce_axis0_f64(x.u.reshape(-1, 7 * 9)[:, :50].copy())
    finally:
        oracle_mod.set_threads(before)
    for k in one:
        a, b = np.asarray(one[k]), np.asarray(many[k])
        assert a.tobytes() == b.tobytes(), k
    assert r1.tobytes() == r4.tobytes()
