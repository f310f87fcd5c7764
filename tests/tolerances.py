"""Pass/fail criteria shared by the tests (numpy only).

Activations (h_hist, act): |x - ref| <= 1e-5 |ref| + 1e-6 against the fp64
oracle -- the stated relative tolerance with an absolute floor for entries
near zero.

Gradients (gW, gb, per-sample scratch S, Sb):
    |x - ref| <= 1e-6 + 1e-4 |ref| + KAPPA * u * mass
with u = 2^-24 and mass = sum over the (b, t) terms of |dp| * |z| (for the
bias sums, of |dp|): the absolute size of what the gradient adds up.  The
stated rel 1e-4 / abs 1e-6 alone cannot be met by any fp32 evaluation on
entries where the terms cancel: the oracle's own fp32 instantiation misses it
on about 0.1% of the headline-shape weight gradients, by up to 4x.  The mass
term is the first-order forward-error bound of a sum of rounded terms;
KAPPA = 16 leaves at least 2x margin over the worst error of the plain fp32
oracle measured on the tiny, pages-shaped and wide configurations.

AdamW (one step from fp32 state; the oracle evaluates the definition in
fp64 on the same fp32 inputs and fp32-rounded hyperparameters):
    m: |x - ref| <= 4 u (|beta1 m0| + |(1 - beta1) g|)
    v: |x - ref| <= 4 u v_ref                      (terms of one sign)
    p: |x - ref| <= 16 u (|p0| + step_size (|beta1 m0| + |(1 - beta1) g|) / den)
with den = sqrt(v_ref / (1 - beta2^t)) + eps and step_size = lr / (1 - beta1^t):
each of m, v takes at most three roundings of terms bounded by that mass
(1 - beta for beta in [0.5, 1) is exact in fp32), and the update's quotient,
square root, bias-correction constants, decay and final subtraction add a
handful more relative roundings of |p0| and of the update; 16 covers them
with margin.

Batch-axis reduction: |x - ref| <= 1e-6 |ref| + 2^-24 * |ref| + eps64, where
the reference is the fp64 column sum; the library rounds an fp64 sum once,
so the only error besides that rounding is the fp64 reordering term
eps64 = B * 2^-53 * sum_b |x_b|.
"""
import numpy as np

U32 = 2.0 ** -24
U64 = 2.0 ** -53
KAPPA = 16.0


def _report(name, x, ref, bound):
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(x - ref)
    ratio = err / bound
    bad = ~(err <= bound)  # NaN fails
    norm = np.linalg.norm(ref)
    return dict(name=name, n=int(x.size), fails=int(bad.sum()),
                worst_ratio=float(np.nanmax(ratio)) if x.size else 0.0,
                max_err=float(err.max()) if x.size else 0.0,
                normwise=float(np.linalg.norm(x - ref) / norm) if norm > 0 else float(np.linalg.norm(x - ref)),
                first_bad=np.argwhere(bad)[:5].tolist())


def check_act(name, x, ref, rtol=1e-5, atol=1e-6):
    ref = np.asarray(ref, np.float64)
    return _report(name, x, ref, atol + rtol * np.abs(ref))


def check_grad(name, x, ref, mass, rtol=1e-4, atol=1e-6, kappa=KAPPA):
    ref = np.asarray(ref, np.float64)
    return _report(name, x, ref, atol + rtol * np.abs(ref) + kappa * U32 * np.asarray(mass))


def check_reduce(name, x, ref, absmass, B, rtol=1e-6):
    ref = np.asarray(ref, np.float64)
    bound = rtol * np.abs(ref) + U32 * np.abs(ref) + B * U64 * np.asarray(absmass)
    bound = np.maximum(bound, np.finfo(np.float32).tiny)
    return _report(name, x, ref, bound)


def grad_mass(u, h_hist, dp):
    """mass for S [B,3,C,n_in], Sb [B,3,C], gW [3,C,n_in], gb [3,C] from the
    fp64 oracle's h_hist [K+1,B,C] and dp [K,3,B,C] and the inputs u [K,B,n_x]:
    mass_S[b,q,c,k] = sum_t |dp[t,q,b,c]| |z_t[b,k]|."""
    z = np.concatenate([np.asarray(u, np.float64), np.asarray(h_hist, np.float64)[:-1]], axis=2)
    adp = np.abs(np.asarray(dp, np.float64))
    A = np.ascontiguousarray(adp.transpose(2, 1, 3, 0))          # [B,3,C,K]
    Z = np.ascontiguousarray(np.abs(z).transpose(1, 0, 2))[:, None]  # [B,1,K,n_in]
    mS = np.matmul(A, Z)
    mSb = adp.sum(axis=0).transpose(1, 0, 2)
    return dict(S=mS, Sb=mSb, gW=mS.sum(axis=0), gb=mSb.sum(axis=0))


def assert_ok(rep):
    assert rep["fails"] == 0, rep


def check_adamw(p, m, v, ref, p0, m0, g, lr, beta1, beta2, eps, step):
    """Reports for (p, m, v) against ref = oracle (p, m, v); see the module
    docstring for the bounds."""
    p0, m0, g = (np.asarray(a, np.float64) for a in (p0, m0, g))
    rp, rm, rv = (np.asarray(a, np.float64) for a in ref)
    mass_m = np.abs(beta1 * m0) + np.abs((1.0 - beta1) * g)
    den = np.sqrt(rv / (1.0 - beta2 ** step)) + eps
    step_size = lr / (1.0 - beta1 ** step)
    return [_report("p", p, rp, 16 * U32 * (np.abs(p0) + step_size * mass_m / den)),
            _report("m", m, rm, 4 * U32 * mass_m),
            _report("v", v, rv, np.maximum(4 * U32 * rv, np.finfo(np.float32).tiny))]
