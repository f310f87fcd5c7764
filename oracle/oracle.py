"""ctypes front end of the CPU oracle -- TEST INFRASTRUCTURE ONLY.

Argument marshalling only: every number of the cell, the BPTT and the
reductions is computed by the C oracle in cfc_oracle_body.h; adamw_step is
the optimizer's definition written out in fp64 numpy.  Inputs are numpy arrays; for precision "f64" they are
upcast exactly (fp32 -> fp64 is exact), for "f32" they must already be fp32.

Shapes (row-major): u [K,B,n_x], y [K,B,C], h0 [B,C], W [3,C,n_in],
bias [3,C], act [K,3,B,C] (gate, g, hh), scratch S [B,3,C,n_in], Sb [B,3,C].
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_I64 = ctypes.c_long
_P = ctypes.c_void_p


def lib_path() -> str:
    return _build.LIB


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not os.path.exists(path):
            _build.build()
        lib = ctypes.CDLL(path)
        for suf in ("f64", "f32"):
            real = ctypes.c_double if suf == "f64" else ctypes.c_float
            f = getattr(lib, "oracle_fwd_step_" + suf)
            f.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _P, _P]
            f.restype = None
            f = getattr(lib, "oracle_bwd_step_" + suf)
            f.argtypes = [_P] * 11 + [_I64, _I64, _I64, _P]
            f.restype = None
            f = getattr(lib, "oracle_sum_axis0_" + suf)
            f.argtypes = [_P, _I64, _I64, _P]
            f.restype = None
            f = getattr(lib, "oracle_cfc_forward_" + suf)
            f.argtypes = [_P] * 5 + [_I64] * 4 + [_P, _P]
            f.restype = real
            f = getattr(lib, "oracle_cfc_train_" + suf)
            f.argtypes = [_P] * 5 + [_I64] * 4 + [_P] * 9
            f.restype = real
            f = getattr(lib, "oracle_input_projection_" + suf)
            f.argtypes = [_P] * 3 + [_I64] * 3 + [_P]
            f.restype = None
        lib.oracle_reduce_axis0_f64.argtypes = [_P, _I64, _I64, _P]
        lib.oracle_reduce_axis0_f64.restype = None
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_threads.restype = None
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        _LIB = lib
    return _LIB


def set_threads(n):
    """Host threads of the oracle's per-sample and per-column loops (n >= 1).
    Results are bitwise the same for any count."""
    _lib().oracle_set_threads(int(n))


def threads():
    """Threads the oracle's parallel loops use now."""
    return int(_lib().oracle_threads())


def _dt(precision):
    if precision == "f64":
        return np.float64
    if precision == "f32":
        return np.float32
    raise ValueError("precision must be 'f64' or 'f32'")


def _in(a, precision):
    dt = _dt(precision)
    a = np.asarray(a)
    if precision == "f32" and a.dtype != np.float32:
        raise TypeError("f32 oracle takes fp32 arrays")
    return np.ascontiguousarray(a, dtype=dt)


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def fwd_step(u_t, h_prev, W, bias, precision="f64"):
    """One forward step: returns (h_t [B,C], act_t [3,B,C])."""
    u_t, h_prev, W, bias = (_in(a, precision) for a in (u_t, h_prev, W, bias))
    B, n_x = u_t.shape
    C = h_prev.shape[1]
    assert W.shape == (3, C, n_x + C) and bias.shape == (3, C) and h_prev.shape == (B, C)
    h_t = np.zeros((B, C), _dt(precision))
    act_t = np.zeros((3, B, C), _dt(precision))
    getattr(_lib(), "oracle_fwd_step_" + precision)(
        _p(u_t), _p(h_prev), _p(W), _p(bias), B, C, n_x, _p(h_t), _p(act_t))
    return h_t, act_t


def input_projection(u, W, bias, precision="f64"):
    """X [.., 3C] = bias + W[:, :, :n_x] u for every row of u [.., n_x]."""
    dt = _dt(precision)
    u = _in(u, precision)
    W = _in(W, precision)
    bias = _in(bias, precision)
    C = W.shape[1]
    n_x = u.shape[-1]
    M = int(np.prod(u.shape[:-1]))
    X = np.zeros(tuple(u.shape[:-1]) + (3 * C,), dtype=dt)
    getattr(_lib(), "oracle_input_projection_" + precision)(_p(u), _p(W), _p(bias), M, C, n_x, _p(X))
    return X


def bwd_step(u_t, h_prev, h_t, y_t, W, act_t, dh_in, S, Sb, precision="f64", want_du=True):
    """One backward step.  Returns (dh_out [B,C], du_t [B,n_x] or None, S, Sb, dp)
    where S [B,3,C,n_in] and Sb [B,3,C] are the inputs plus this step's terms
    and dp [3,B,C] the step's pre-activation gradients."""
    u_t, h_prev, h_t, y_t, W, act_t, dh_in = (
        _in(a, precision) for a in (u_t, h_prev, h_t, y_t, W, act_t, dh_in))
    B, n_x = u_t.shape
    C = h_prev.shape[1]
    S = np.array(_in(S, precision), copy=True)
    Sb = np.array(_in(Sb, precision), copy=True)
    assert S.shape == (B, 3, C, n_x + C) and Sb.shape == (B, 3, C)
    dh_out = np.zeros((B, C), _dt(precision))
    du_t = np.zeros((B, n_x), _dt(precision)) if want_du else None
    dp = np.zeros((3, B, C), _dt(precision))
    getattr(_lib(), "oracle_bwd_step_" + precision)(
        _p(u_t), _p(h_prev), _p(h_t), _p(y_t), _p(W), _p(act_t), _p(dh_in),
        _p(dh_out), _p(du_t), _p(S), _p(Sb), B, C, n_x, _p(dp))
    return dh_out, du_t, S, Sb, dp


def _dims(u, y, h0, W, bias):
    K, B, n_x = u.shape
    C = h0.shape[1]
    assert y.shape == (K, B, C) and h0.shape == (B, C)
    assert W.shape == (3, C, n_x + C) and bias.shape == (3, C)
    return K, B, C, n_x


def forward(u, y, h0, W, bias, precision="f64"):
    """Forward over all K steps: returns (loss, h_hist [K+1,B,C], act [K,3,B,C])."""
    u, y, h0, W, bias = (_in(a, precision) for a in (u, y, h0, W, bias))
    K, B, C, n_x = _dims(u, y, h0, W, bias)
    dt = _dt(precision)
    h_hist = np.zeros((K + 1, B, C), dt)
    act = np.zeros((K, 3, B, C), dt)
    loss = getattr(_lib(), "oracle_cfc_forward_" + precision)(
        _p(u), _p(y), _p(h0), _p(W), _p(bias), B, C, n_x, K, _p(h_hist), _p(act))
    return float(loss), h_hist, act


def train(u, y, h0, W, bias, precision="f64", want_du=False, want_dp=False):
    """One K-loop training step.  Returns a dict with loss, h_hist, act,
    S, Sb (per-sample scratch), gW [3,C,n_in], gb [3,C], dh0 [B,C], du
    [K,B,n_x] (if want_du) and dp [K,3,B,C] (if want_dp)."""
    u, y, h0, W, bias = (_in(a, precision) for a in (u, y, h0, W, bias))
    K, B, C, n_x = _dims(u, y, h0, W, bias)
    n_in = n_x + C
    dt = _dt(precision)
    out = dict(
        h_hist=np.zeros((K + 1, B, C), dt), act=np.zeros((K, 3, B, C), dt),
        S=np.zeros((B, 3, C, n_in), dt), Sb=np.zeros((B, 3, C), dt),
        gW=np.zeros((3, C, n_in), dt), gb=np.zeros((3, C), dt),
        dh0=np.zeros((B, C), dt),
        du=np.zeros((K, B, n_x), dt) if want_du else None,
        dp=np.zeros((K, 3, B, C), dt) if want_dp else None)
    loss = getattr(_lib(), "oracle_cfc_train_" + precision)(
        _p(u), _p(y), _p(h0), _p(W), _p(bias), B, C, n_x, K,
        _p(out["h_hist"]), _p(out["act"]), _p(out["S"]), _p(out["Sb"]),
        _p(out["gW"]), _p(out["gb"]), _p(out["dh0"]), _p(out["du"]), _p(out["dp"]))
    out["loss"] = float(loss)
    return out


def sum_axis0(x, precision="f64"):
    """Column sum over axis 0 of a [B,N] array in the given precision, increasing b."""
    x = _in(x, precision)
    B, N = x.shape
    out = np.zeros(N, _dt(precision))
    getattr(_lib(), "oracle_sum_axis0_" + precision)(_p(x), B, N, _p(out))
    return out


def reduce_axis0_f64(x):
    """The batch-axis reduction reference: fp32 [B,N] summed in double over
    increasing b; returns float64 [N] (not rounded to fp32)."""
    x = np.ascontiguousarray(x)
    if x.dtype != np.float32 or x.ndim != 2:
        raise TypeError("reduce_axis0 reference takes a 2-D fp32 array")
    B, N = x.shape
    out = np.zeros(N, np.float64)
    _lib().oracle_reduce_axis0_f64(_p(x), B, N, _p(out))
    return out


def adamw_step(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step):
    """One AdamW step in fp64 (decoupled weight decay), from its definition:
    p <- p (1 - lr wd); m <- b1 m + (1 - b1) g; v <- b2 v + (1 - b2) g^2;
    p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).
    Returns new (p, m, v); the inputs are not modified."""
    p = np.asarray(p, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** step)
    v_hat = v / (1.0 - beta2 ** step)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v
