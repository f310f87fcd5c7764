"""Python binding of libcfc.so (include/cfc.h), same names as the C ABI.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libcfc.so.  PyTorch provides device memory (CUDA/HIP tensors) and
the current stream.  There is no fallback: if the library is missing or a
call fails, an exception is raised.
"""
import ctypes
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcfc.so")

CFC_OK = 0
CFC_EINVAL = -1
CFC_EHIP = -2
KLOOP_AUTO = 0
KLOOP_STEPS = 1
KLOOP_PERSISTENT = 2
KLOOP_STEPS_VALU = 3
KLOOP_STEPS_MFMA = 4
KLOOP_RESIDENT = 5

_LIB = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64


class CfcError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__("%s failed (%d): %s" % (fn, code, msg))
        self.code = code


def lib():
    """The loaded libcfc.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libcfc.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        L.cfc_fwd_step.argtypes = [_P] * 6 + [_I, _I, _I, _P]
        L.cfc_bwd_step.argtypes = [_P] * 11 + [_I, _I, _I, _P]
        L.reduce_axis0.argtypes = [_P, _I64, _I64, _P, _P]
        L.cfc_train_kloop.argtypes = [_P] * 8 + [ctypes.c_size_t] + [_P] * 4 + [_I, _I, _I, _I, _P]
        L.cfc_kloop_fwd_bwd.argtypes = [_P] * 8 + [ctypes.c_size_t, _I, _I, _I, _I, _P]
        L.cfc_kloop_fwd_bwd_fill.argtypes = [_P] * 8 + [ctypes.c_size_t, _P, _P, _I, _I, _I, _I, _P]
        L.cfc_train_kloop_noalloc.argtypes = [_P] * 11 + [_I, _I, _I, _I, _P]
        L.cfc_scratch_fill.argtypes = [_P] * 5 + [_I, _I, _I, _I, _P]
        L.cfc_input_projection.argtypes = [_P] * 4 + [_I64, _I, _I, _P]
        L.cfc_kloop_recurrence.argtypes = [_P] * 7 + [_I, _I, _I, _I, _P]
        _F = ctypes.c_float
        L.cfc_adamw_step.argtypes = [_P] * 5 + [_I, _F, _F, _F, _F, _F, _I, _P]
        L.cfc_weight_grad_gemm.argtypes = [_P] * 5 + [_I, _I, _I, _I, _P, ctypes.c_size_t, _P]
        L.cfc_weight_grad_gemm_workspace_bytes.argtypes = [_I, _I, _I, _I]
        L.cfc_weight_grad_gemm_workspace_bytes.restype = ctypes.c_size_t
        L.cfc_train_kloop_gemm.argtypes = [_P] * 9 + [_P, ctypes.c_size_t, _I, _I, _I, _I, _P]
        L.cfc_train_kloop_gemm_workspace_bytes.argtypes = [_I, _I, _I, _I]
        L.cfc_train_kloop_gemm_workspace_bytes.restype = ctypes.c_size_t
        L.cfc_train_kloop_workspace_bytes.argtypes = [_I, _I, _I, _I]
        L.cfc_train_kloop_workspace_bytes.restype = ctypes.c_size_t
        L.cfc_set_kloop_mode.argtypes = [_I]
        L.cfc_kloop_path.argtypes = [_I, _I, _I, _I]
        L.cfc_kloop_path.restype = _I
        L.cfc_kloop_status.argtypes = [_P, ctypes.c_size_t, _I, _I, _I, _I, _P]
        L.cfc_kloop_status.restype = _I
        L.cfc_last_error.argtypes = []
        L.cfc_last_error.restype = ctypes.c_char_p
        L.cfc_clear_graph_cache.argtypes = []
        L.cfc_probe_fma.argtypes = [_I, _I, _I, _I, _P, _P]
        for f in (L.cfc_fwd_step, L.cfc_bwd_step, L.reduce_axis0, L.cfc_train_kloop,
                  L.cfc_kloop_fwd_bwd, L.cfc_scratch_fill, L.cfc_clear_graph_cache,
                  L.cfc_set_kloop_mode, L.cfc_input_projection, L.cfc_kloop_recurrence, L.cfc_adamw_step,
                  L.cfc_weight_grad_gemm, L.cfc_train_kloop_gemm, L.cfc_probe_fma, L.cfc_train_kloop_noalloc):
            f.restype = _I
        _LIB = L
    return _LIB


def last_error() -> str:
    return lib().cfc_last_error().decode()


def _check(fn, rc):
    if rc != CFC_OK:
        raise CfcError(fn, rc, last_error())


def _dev(t, name, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise TypeError("%s must be contiguous float32" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    return t.data_ptr()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def cfc_fwd_step(u_t, h_prev, W, bias, h_t=None, act_t=None):
    """One forward step; returns (h_t [B,C], act_t [3,B,C])."""
    B, n_x = u_t.shape
    C = h_prev.shape[1]
    if h_t is None:
        h_t = torch.empty((B, C), dtype=torch.float32, device=h_prev.device)
    if act_t is None:
        act_t = torch.empty((3, B, C), dtype=torch.float32, device=h_prev.device)
    args = (_dev(u_t, "u_t", (B, n_x)), _dev(h_prev, "h_prev", (B, C)),
            _dev(W, "W", (3, C, n_x + C)), _dev(bias, "bias", (3, C)),
            _dev(h_t, "h_t", (B, C)), _dev(act_t, "act_t", (3, B, C)))
    _check("cfc_fwd_step", lib().cfc_fwd_step(*args, B, C, n_x, _stream(h_prev)))
    return h_t, act_t


def cfc_bwd_step(u_t, h_prev, h_t, y_t, W, act_t, dh_in, gW_scratch, gb_scratch,
                 dh_out=None, du_t=None, want_du=False):
    """One backward step.  dh_in may be None (zero carry).  gW_scratch and
    gb_scratch are accumulated in place.  Returns (dh_out, du_t or None)."""
    B, n_x = u_t.shape
    C = h_prev.shape[1]
    n_in = n_x + C
    dev = h_prev.device
    if dh_out is None:
        dh_out = torch.empty((B, C), dtype=torch.float32, device=dev)
    if want_du and du_t is None:
        du_t = torch.empty((B, n_x), dtype=torch.float32, device=dev)
    args = (_dev(u_t, "u_t", (B, n_x)), _dev(h_prev, "h_prev", (B, C)), _dev(h_t, "h_t", (B, C)),
            _dev(y_t, "y_t", (B, C)), _dev(W, "W", (3, C, n_in)), _dev(act_t, "act_t", (3, B, C)),
            _dev(dh_in, "dh_in", (B, C)), _dev(dh_out, "dh_out", (B, C)),
            _dev(du_t, "du_t", (B, n_x)), _dev(gW_scratch, "gW_scratch", (B, 3, C, n_in)),
            _dev(gb_scratch, "gb_scratch", (B, 3, C)))
    _check("cfc_bwd_step", lib().cfc_bwd_step(*args, B, C, n_x, _stream(h_prev)))
    return dh_out, du_t


def reduce_axis0(per_batch, out=None):
    """out[n] = sum_b per_batch[b, n] (overwrites out); per_batch is [B, N]."""
    B, N = per_batch.shape
    if out is None:
        out = torch.empty((N,), dtype=torch.float32, device=per_batch.device)
    p_in = _dev(per_batch, "per_batch", (B, N))
    p_out = _dev(out, "out", (N,))
    _check("reduce_axis0", lib().reduce_axis0(p_in, B, N, p_out, _stream(out)))
    return out


def cfc_train_kloop_workspace_bytes(B, C, n_x, K):
    return int(lib().cfc_train_kloop_workspace_bytes(B, C, n_x, K))


@dataclass
class KloopBuffers:
    """Outputs and workspace of cfc_train_kloop.  Reuse one instance across
    steps: the library caches its graph per set of pointers."""
    h_hist: torch.Tensor      # [K+1, B, C]
    act: torch.Tensor         # [K, 3, B, C]
    ws: torch.Tensor          # workspace, cfc_train_kloop_workspace_bytes / 4 floats
    gW_scratch: torch.Tensor  # [B, 3, C, n_in]
    gb_scratch: torch.Tensor  # [B, 3, C]
    gW: torch.Tensor          # [3, C, n_in]
    gb: torch.Tensor          # [3, C]

    @staticmethod
    def allocate(B, C, n_x, K, device):
        n_in = n_x + C
        e = lambda *s: torch.empty(s, dtype=torch.float32, device=device)  # noqa: E731
        ws_floats = cfc_train_kloop_workspace_bytes(B, C, n_x, K) // 4
        return KloopBuffers(h_hist=e(K + 1, B, C), act=e(K, 3, B, C), ws=e(max(ws_floats, 1)),
                            gW_scratch=e(B, 3, C, n_in), gb_scratch=e(B, 3, C),
                            gW=e(3, C, n_in), gb=e(3, C))


def cfc_train_kloop(u, y, h0, W, bias, out=None):
    """One training step of the K-loop (forward, BPTT, scratch, reduce):
    two to four direct launches on the persistent path (include/cfc.h
    says which), one graph replay on the step path.  Returns the KloopBuffers holding h_hist, act, the per-sample
    scratch, gW and gb."""
    K, B, n_x = u.shape
    C = h0.shape[1]
    n_in = n_x + C
    if out is None:
        out = KloopBuffers.allocate(B, C, n_x, K, h0.device)
    if out.ws.dim() != 1 or not out.ws.is_contiguous():
        raise ValueError("ws must be a contiguous 1-D tensor")
    args = (_dev(u, "u", (K, B, n_x)), _dev(y, "y", (K, B, C)), _dev(h0, "h0", (B, C)),
            _dev(W, "W", (3, C, n_in)), _dev(bias, "bias", (3, C)),
            _dev(out.h_hist, "h_hist", (K + 1, B, C)), _dev(out.act, "act", (K, 3, B, C)),
            _dev(out.ws, "ws"), out.ws.numel() * 4,
            _dev(out.gW_scratch, "gW_scratch", (B, 3, C, n_in)),
            _dev(out.gb_scratch, "gb_scratch", (B, 3, C)), _dev(out.gW, "gW", (3, C, n_in)),
            _dev(out.gb, "gb", (3, C)))
    _check("cfc_train_kloop", lib().cfc_train_kloop(*args, B, C, n_x, K, _stream(h0)))
    return out


def cfc_train_kloop_noalloc(u, y, h0, W, bias, out):
    """cfc_train_kloop with the library's fixed workspace (no allocation in
    the call, no graph; see include/cfc.h): out supplies h_hist, act, the
    scratch, gW and gb (its ws is not used).  Returns out."""
    K, B, n_x = u.shape
    C = h0.shape[1]
    n_in = n_x + C
    args = (_dev(u, "u", (K, B, n_x)), _dev(y, "y", (K, B, C)), _dev(h0, "h0", (B, C)),
            _dev(W, "W", (3, C, n_in)), _dev(bias, "bias", (3, C)),
            _dev(out.h_hist, "h_hist", (K + 1, B, C)), _dev(out.act, "act", (K, 3, B, C)),
            _dev(out.gW_scratch, "gW_scratch", (B, 3, C, n_in)),
            _dev(out.gb_scratch, "gb_scratch", (B, 3, C)), _dev(out.gW, "gW", (3, C, n_in)),
            _dev(out.gb, "gb", (3, C)))
    _check("cfc_train_kloop_noalloc", lib().cfc_train_kloop_noalloc(*args, B, C, n_x, K, _stream(h0)))
    return out


def cfc_kloop_fwd_bwd(u, y, h0, W, bias, out):
    """Forward and backward of the K-loop into out.h_hist, out.act and the
    dp_t block of out.ws (see include/cfc.h); no scratch, no reduction."""
    K, B, n_x = u.shape
    C = h0.shape[1]
    args = (_dev(u, "u", (K, B, n_x)), _dev(y, "y", (K, B, C)), _dev(h0, "h0", (B, C)),
            _dev(W, "W", (3, C, n_x + C)), _dev(bias, "bias", (3, C)),
            _dev(out.h_hist, "h_hist", (K + 1, B, C)), _dev(out.act, "act", (K, 3, B, C)),
            _dev(out.ws, "ws"), out.ws.numel() * 4)
    _check("cfc_kloop_fwd_bwd", lib().cfc_kloop_fwd_bwd(*args, B, C, n_x, K, _stream(h0)))
    return out


def cfc_input_projection(u, W, bias, X=None):
    """X [.., 3C] = bias + W[:, :, :n_x] u for every row of u [.., n_x]
    (the canonical input part of the pre-activations; see include/cfc.h)."""
    n_x = u.shape[-1]
    C = W.shape[1]
    M = 1
    for d in u.shape[:-1]:
        M *= int(d)
    if X is None:
        X = torch.empty(tuple(u.shape[:-1]) + (3 * C,), device=W.device, dtype=torch.float32)
    args = (_dev(u, "u"), _dev(W, "W", (3, C, n_x + C)), _dev(bias, "bias", (3, C)), _dev(X, "X"))
    if X.numel() != M * 3 * C:
        raise ValueError("X must hold %d rows of 3C floats" % M)
    _check("cfc_input_projection", lib().cfc_input_projection(*args, M, C, n_x, _stream(W)))
    return X


def cfc_kloop_recurrence(X, y, h0, W, out):
    """Forward and backward of the K-loop given X [K,B,3C] from
    cfc_input_projection, into out.h_hist, out.act and the dp_t block of
    out.ws (persistent kernel, C <= 128)."""
    K, B, C = y.shape
    n_x = W.shape[2] - C
    dp = out.ws[:K * B * 3 * C]
    args = (_dev(X, "X", (K, B, 3 * C)), _dev(y, "y", (K, B, C)), _dev(h0, "h0", (B, C)),
            _dev(W, "W", (3, C, n_x + C)), _dev(out.h_hist, "h_hist", (K + 1, B, C)),
            _dev(out.act, "act", (K, 3, B, C)), _dev(dp, "dp"))
    _check("cfc_kloop_recurrence", lib().cfc_kloop_recurrence(*args, B, C, n_x, K, _stream(h0)))
    return out


def cfc_adamw_step(params, grads, ms, vs, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1):
    """One AdamW step over the tensors of `params` (lists of up to 4 same-shaped
    parameter / gradient / moment tensors), one launch, in place."""
    n = len(params)
    if not (len(grads) == len(ms) == len(vs) == n):
        raise ValueError("params, grads, ms and vs must have the same length")
    arr = lambda xs, name: (ctypes.c_void_p * max(n, 1))(*[_dev(x, name) for x in xs])  # noqa: E731
    for p, g, m, v in zip(params, grads, ms, vs):
        if not (p.shape == g.shape == m.shape == v.shape):
            raise ValueError("a segment's tensors must have one shape")
    counts = (ctypes.c_int64 * max(n, 1))(*[p.numel() for p in params])
    stream = _stream(params[0]) if n else None
    _check("cfc_adamw_step", lib().cfc_adamw_step(arr(params, "param"), arr(grads, "grad"), arr(ms, "m"),
                                                  arr(vs, "v"), counts, n, lr, beta1, beta2, eps,
                                                  weight_decay, int(step), stream))
    return params


def cfc_probe_fma(out, blocks, threads, iters, one_per_cu=True):
    """FMA-rate probe (include/probe.h): 2 * 64 * iters * blocks * threads
    flops of non-packed fp32 FMA; out [blocks * threads] receives each lane's
    chain sum."""
    if out.numel() < blocks * threads:
        raise ValueError("out holds fewer than blocks * threads floats")
    _check("cfc_probe_fma", lib().cfc_probe_fma(int(blocks), int(threads), int(bool(one_per_cu)), int(iters),
                                                _dev(out, "out"), _stream(out)))
    return out


def cfc_weight_grad_gemm(dp, u, h_hist, gW=None, gb=None, ws=None):
    """GEMM-form weight gradient from the saved dp [K, B, 3C] (no scratch)."""
    K, B, n_x = u.shape
    C = h_hist.shape[2]
    n_in = n_x + C
    dev = dp.device
    e = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)  # noqa: E731
    gW = e(3, C, n_in) if gW is None else gW
    gb = e(3, C) if gb is None else gb
    if ws is None:
        ws = e(max(lib().cfc_weight_grad_gemm_workspace_bytes(B, C, n_x, K) // 4, 1))
    args = (_dev(dp, "dp", (K, B, 3 * C)), _dev(u, "u", (K, B, n_x)), _dev(h_hist, "h_hist", (K + 1, B, C)),
            _dev(gW, "gW", (3, C, n_in)), _dev(gb, "gb", (3, C)))
    _check("cfc_weight_grad_gemm", lib().cfc_weight_grad_gemm(*args, B, C, n_x, K, _dev(ws, "ws"), ws.numel() * 4,
                                                              _stream(dp)))
    return gW, gb


@dataclass
class KloopGemmBuffers:
    """Outputs and workspace of cfc_train_kloop_gemm (no scratch)."""
    h_hist: torch.Tensor
    act: torch.Tensor
    ws: torch.Tensor
    gW: torch.Tensor
    gb: torch.Tensor

    @staticmethod
    def allocate(B, C, n_x, K, device):
        e = lambda *s: torch.empty(s, dtype=torch.float32, device=device)  # noqa: E731
        ws_floats = lib().cfc_train_kloop_gemm_workspace_bytes(B, C, n_x, K) // 4
        return KloopGemmBuffers(h_hist=e(K + 1, B, C), act=e(K, 3, B, C), ws=e(max(ws_floats, 1)),
                                gW=e(3, C, n_x + C), gb=e(3, C))


def cfc_kloop_fwd_bwd_fill(u, y, h0, W, bias, out):
    """cfc_train_kloop up to its reduction: h_hist, act, dp in out.ws and the
    per-sample scratch (out.gW_scratch, out.gb_scratch); gW and gb untouched."""
    K, B, n_x = u.shape
    C = h0.shape[1]
    n_in = n_x + C
    args = (_dev(u, "u", (K, B, n_x)), _dev(y, "y", (K, B, C)), _dev(h0, "h0", (B, C)),
            _dev(W, "W", (3, C, n_in)), _dev(bias, "bias", (3, C)),
            _dev(out.h_hist, "h_hist", (K + 1, B, C)), _dev(out.act, "act", (K, 3, B, C)),
            _dev(out.ws, "ws"), out.ws.numel() * 4,
            _dev(out.gW_scratch, "gW_scratch", (B, 3, C, n_in)), _dev(out.gb_scratch, "gb_scratch", (B, 3, C)))
    _check("cfc_kloop_fwd_bwd_fill", lib().cfc_kloop_fwd_bwd_fill(*args, B, C, n_x, K, _stream(h0)))
    return out


def cfc_train_kloop_gemm(u, y, h0, W, bias, out=None):
    """The K-loop step with the GEMM-form weight gradient (no scratch)."""
    K, B, n_x = u.shape
    C = h0.shape[1]
    n_in = n_x + C
    if out is None:
        out = KloopGemmBuffers.allocate(B, C, n_x, K, h0.device)
    args = (_dev(u, "u", (K, B, n_x)), _dev(y, "y", (K, B, C)), _dev(h0, "h0", (B, C)),
            _dev(W, "W", (3, C, n_in)), _dev(bias, "bias", (3, C)),
            _dev(out.h_hist, "h_hist", (K + 1, B, C)), _dev(out.act, "act", (K, 3, B, C)),
            _dev(out.gW, "gW", (3, C, n_in)), _dev(out.gb, "gb", (3, C)))
    _check("cfc_train_kloop_gemm", lib().cfc_train_kloop_gemm(*args, _dev(out.ws, "ws"), out.ws.numel() * 4,
                                                              B, C, n_x, K, _stream(u)))
    return out


def cfc_scratch_fill(dp, u, h_hist, gW_scratch, gb_scratch):
    """Per-sample scratch from saved dp [K,B,3C] (overwrites both outputs)."""
    K, B, n_x = u.shape
    C = h_hist.shape[2]
    args = (_dev(dp, "dp", (K, B, 3 * C)), _dev(u, "u", (K, B, n_x)), _dev(h_hist, "h_hist"),
            _dev(gW_scratch, "gW_scratch", (B, 3, C, n_x + C)), _dev(gb_scratch, "gb_scratch", (B, 3, C)))
    if h_hist.shape[0] < K or tuple(h_hist.shape[1:]) != (B, C):
        raise ValueError("h_hist must be [>=K, B, C]")
    _check("cfc_scratch_fill", lib().cfc_scratch_fill(*args, B, C, n_x, K, _stream(u)))
    return gW_scratch, gb_scratch


def cfc_set_kloop_mode(mode):
    """KLOOP_AUTO, KLOOP_STEPS, KLOOP_PERSISTENT, KLOOP_STEPS_VALU,
    KLOOP_STEPS_MFMA or KLOOP_RESIDENT for the calling thread (other threads
    keep their own)."""
    _check("cfc_set_kloop_mode", lib().cfc_set_kloop_mode(int(mode)))


def cfc_kloop_path(B, C, n_x, K):
    """KLOOP_PERSISTENT, KLOOP_STEPS_VALU, KLOOP_STEPS_MFMA or KLOOP_RESIDENT:
    the path cfc_train_kloop takes now on this thread (-1 if its mode cannot
    take these sizes)."""
    return int(lib().cfc_kloop_path(B, C, n_x, K))


def cfc_kloop_status(out, B, C, n_x, K):
    """Raises CfcError (code CFC_EHIP) if a bounded wait of the last K-loop
    call on out.ws gave up (that call's results are then undefined).  Waits
    for the current stream.  Call on the thread that made the call."""
    if out.ws.dim() != 1 or not out.ws.is_contiguous():
        raise ValueError("ws must be a contiguous 1-D tensor")
    _check("cfc_kloop_status", lib().cfc_kloop_status(_dev(out.ws, "ws"), out.ws.numel() * 4, B, C, n_x, K,
                                                      _stream(out.ws)))


def clear_graph_cache():
    _check("cfc_clear_graph_cache", lib().cfc_clear_graph_cache())
