"""Python binding of the batched MLP training step in libcfc.so
(include/mlp.h), same names as the C ABI.

Argument marshalling only: every step runs in the HIP kernels of libcfc.so;
torch tensors provide device memory and the current stream.  There is no
fallback: a missing library or a failed call raises.
"""
import ctypes
from dataclasses import dataclass

import torch

from . import cfc as _cfc

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_READY = False


def lib():
    """libcfc.so with the MLP entry points' signatures declared."""
    global _READY
    L = _cfc.lib()
    if not _READY:
        L.mlp_param_offsets.argtypes = [_P, _I, _P, _P]
        L.mlp_param_offsets.restype = _I64
        L.mlp_linear_fwd.argtypes = [_P] * 4 + [_I, _I, _I, _I, _P]
        L.mlp_linear_bwd_data.argtypes = [_P] * 4 + [_I, _I, _I, _P]
        L.mlp_linear_bwd_weight.argtypes = [_P] * 4 + [_I, _I, _I, _P, _SZ, _P]
        L.mlp_linear_bwd_weight_workspace_bytes.argtypes = [_I, _I, _I]
        L.mlp_linear_bwd_weight_workspace_bytes.restype = _SZ
        L.mlp_weight_grad_splits.argtypes = [_I]
        L.mlp_weight_grad_splits.restype = _I
        L.mlp_mse_loss_grad.argtypes = [_P] * 4 + [_I, _I, _P, _SZ, _P]
        L.mlp_mse_workspace_bytes.argtypes = [_I]
        L.mlp_mse_workspace_bytes.restype = _SZ
        L.mlp_train_step.argtypes = [_P, _P, _I, _P, _I, _P, _P, _P, _P, _P, _SZ, _P]
        L.mlp_train_step_workspace_bytes.argtypes = [_I, _P, _I]
        L.mlp_train_step_workspace_bytes.restype = _SZ
        for f in (L.mlp_linear_fwd, L.mlp_linear_bwd_data, L.mlp_linear_bwd_weight, L.mlp_mse_loss_grad,
                  L.mlp_train_step):
            f.restype = _I
        _READY = True
    return L


def _dims(dims):
    return (ctypes.c_int * len(dims))(*[int(d) for d in dims])


def mlp_param_offsets(dims):
    """(w_off, b_off, total) of the flat parameter layout."""
    L = len(dims) - 1
    w = (ctypes.c_int64 * max(L, 1))()
    b = (ctypes.c_int64 * max(L, 1))()
    total = lib().mlp_param_offsets(_dims(dims), L, w, b)
    if total < 0:
        raise _cfc.CfcError("mlp_param_offsets", -1, _cfc.last_error())
    return list(w)[:L], list(b)[:L], int(total)


def mlp_linear_fwd(X, W, b, Y=None, relu=True):
    M, n_in = X.shape
    n_out = W.shape[0]
    if Y is None:
        Y = torch.empty((M, n_out), dtype=torch.float32, device=X.device)
    args = (_cfc._dev(X, "X", (M, n_in)), _cfc._dev(W, "W", (n_out, n_in)),
            _cfc._dev(b, "b", (n_out,)) if b is not None else None, _cfc._dev(Y, "Y", (M, n_out)))
    _cfc._check("mlp_linear_fwd", lib().mlp_linear_fwd(*args, M, n_in, n_out, 1 if relu else 0, _cfc._stream(X)))
    return Y


def mlp_linear_bwd_data(dY, W, mask=None, dX=None):
    M, n_out = dY.shape
    n_in = W.shape[1]
    if dX is None:
        dX = torch.empty((M, n_in), dtype=torch.float32, device=dY.device)
    args = (_cfc._dev(dY, "dY", (M, n_out)), _cfc._dev(W, "W", (n_out, n_in)),
            _cfc._dev(mask, "mask", (M, n_in)) if mask is not None else None, _cfc._dev(dX, "dX", (M, n_in)))
    _cfc._check("mlp_linear_bwd_data", lib().mlp_linear_bwd_data(*args, M, n_in, n_out, _cfc._stream(dY)))
    return dX


def mlp_linear_bwd_weight(dY, X, gW=None, gb=None, ws=None, with_bias=True):
    M, n_out = dY.shape
    n_in = X.shape[1]
    dev = dY.device
    if gW is None:
        gW = torch.empty((n_out, n_in), dtype=torch.float32, device=dev)
    if gb is None and with_bias:
        gb = torch.empty((n_out,), dtype=torch.float32, device=dev)
    need = lib().mlp_linear_bwd_weight_workspace_bytes(M, n_in, n_out)
    if ws is None:
        ws = torch.empty((max(need // 4, 1),), dtype=torch.float32, device=dev)
    args = (_cfc._dev(dY, "dY", (M, n_out)), _cfc._dev(X, "X", (M, n_in)), _cfc._dev(gW, "gW", (n_out, n_in)),
            _cfc._dev(gb, "gb", (n_out,)) if gb is not None else None)
    _cfc._check("mlp_linear_bwd_weight", lib().mlp_linear_bwd_weight(*args, M, n_in, n_out, _cfc._dev(ws, "ws"),
                                                                      ws.numel() * 4, _cfc._stream(dY)))
    return gW, gb


def mlp_weight_grad_splits(M):
    return lib().mlp_weight_grad_splits(M)


def mlp_mse_loss_grad(Y, T, dY=None, loss=None, ws=None):
    M, N = Y.shape
    dev = Y.device
    if dY is None:
        dY = torch.empty((M, N), dtype=torch.float32, device=dev)
    if loss is None:
        loss = torch.empty((1,), dtype=torch.float32, device=dev)
    if ws is None:
        ws = torch.empty((max(lib().mlp_mse_workspace_bytes(M) // 4, 1),), dtype=torch.float32, device=dev)
    args = (_cfc._dev(Y, "Y", (M, N)), _cfc._dev(T, "T", (M, N)), _cfc._dev(dY, "dY", (M, N)),
            _cfc._dev(loss, "loss", (1,)))
    _cfc._check("mlp_mse_loss_grad", lib().mlp_mse_loss_grad(*args, M, N, _cfc._dev(ws, "ws"), ws.numel() * 4,
                                                              _cfc._stream(Y)))
    return dY, loss


def mlp_train_step_workspace_bytes(B, dims):
    return lib().mlp_train_step_workspace_bytes(B, _dims(dims), len(dims) - 1)


@dataclass
class MlpBuffers:
    """Outputs and workspace of mlp_train_step."""
    grads: torch.Tensor   # flat, mlp_param_offsets layout
    act: list             # act[l] [B, dims[l+1]]
    loss: torch.Tensor    # [1]
    ws: torch.Tensor

    @staticmethod
    def allocate(B, dims, device):
        e = lambda *s: torch.empty(s, dtype=torch.float32, device=device)  # noqa: E731
        total = mlp_param_offsets(dims)[2]
        return MlpBuffers(grads=e(total), act=[e(B, d) for d in dims[1:]], loss=e(1),
                          ws=e(max(mlp_train_step_workspace_bytes(B, dims) // 4, 1)))


def mlp_train_step(X, T, dims, params, out=None):
    """One training step: forward, loss, backward, every parameter's gradient
    (flat, same layout as params).  Returns the MlpBuffers."""
    B = X.shape[0]
    L = len(dims) - 1
    if out is None:
        out = MlpBuffers.allocate(B, dims, X.device)
    total = mlp_param_offsets(dims)[2]
    acts = (ctypes.c_void_p * L)(*[_cfc._dev(a, "act", (B, dims[l + 1])) for l, a in enumerate(out.act)])
    rc = lib().mlp_train_step(_cfc._dev(X, "X", (B, dims[0])), _cfc._dev(T, "T", (B, dims[-1])), B, _dims(dims), L,
                              _cfc._dev(params, "params", (total,)), _cfc._dev(out.grads, "grads", (total,)), acts,
                              _cfc._dev(out.loss, "loss", (1,)), _cfc._dev(out.ws, "ws"), out.ws.numel() * 4,
                              _cfc._stream(X))
    _cfc._check("mlp_train_step", rc)
    return out


def pack_params(Ws, bs, dims):
    """Flat parameter tensor (mlp_param_offsets layout, gaps zero) from lists
    of per-layer tensors on one device."""
    w_off, b_off, total = mlp_param_offsets(dims)
    flat = torch.zeros(total, dtype=torch.float32, device=Ws[0].device)
    for l, (W, b) in enumerate(zip(Ws, bs)):
        flat[w_off[l]:w_off[l] + W.numel()] = W.reshape(-1)
        flat[b_off[l]:b_off[l] + b.numel()] = b.reshape(-1)
    return flat


def unpack(flat, dims):
    """Per-layer (W, b) views of a flat buffer."""
    w_off, b_off, _ = mlp_param_offsets(dims)
    out = []
    for l in range(len(dims) - 1):
        n_out, n_in = dims[l + 1], dims[l]
        out.append((flat[w_off[l]:w_off[l] + n_out * n_in].view(n_out, n_in), flat[b_off[l]:b_off[l] + n_out]))
    return out
