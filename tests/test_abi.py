"""Host-side checks of the C ABI (CPU only: no call here reaches a kernel).

* libcfc.so loads and exports every function include/cfc.h declares;
* argument validation rejects bad sizes, null pointers and overlapping
  buffers before anything is enqueued (fake addresses are safe here because
  every call below is refused by the checks that run first);
* the kernel sources contain no atomics, and the product package never
  touches the oracle.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("cfc.h", "mlp.h", "probe.h")]


def _declared():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:int|int64_t|size_t|const char\*)\s+(\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    from recurrent_cell_amd import build as hbuild
    hbuild.build(force=False)
    from recurrent_cell_amd import cfc
    return cfc.lib()


def test_header_declares_the_four_entry_points():
    names = _declared()
    for n in ("cfc_fwd_step", "cfc_bwd_step", "reduce_axis0", "cfc_train_kloop", "cfc_adamw_step",
              "mlp_linear_fwd", "mlp_linear_bwd_data", "mlp_linear_bwd_weight", "mlp_mse_loss_grad",
              "mlp_train_step", "mlp_param_offsets"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name
        assert isinstance(getattr(L, name), ctypes._CFuncPtr)


FAKE = 1 << 40  # never dereferenced: every call below fails validation first


def test_reduce_axis0_argument_errors(L):
    assert L.reduce_axis0(FAKE, -1, 4, FAKE + 4096, None) == -1
    assert L.reduce_axis0(FAKE, 4, -1, FAKE + 4096, None) == -1
    assert L.reduce_axis0(FAKE, 4, 8, None, None) == -1
    assert L.reduce_axis0(None, 4, 8, FAKE, None) == -1
    # out inside per_batch
    assert L.reduce_axis0(FAKE, 4, 8, FAKE + 16, None) == -1
    assert b"overlap" in L.cfc_last_error()
    # n_tail == 0 is a no-op that succeeds without touching memory
    assert L.reduce_axis0(None, 4, 0, None, None) == 0


def test_step_argument_errors(L):
    B, C, n_x = 4, 16, 8
    n_in = n_x + C
    u, h, W, b = FAKE, FAKE + (1 << 20), FAKE + (2 << 20), FAKE + (3 << 20)
    ht, act = FAKE + (4 << 20), FAKE + (5 << 20)
    assert L.cfc_fwd_step(u, h, W, b, ht, act, -1, C, n_x, None) == -1
    assert L.cfc_fwd_step(u, h, W, b, ht, act, B, 0, n_x, None) == -1
    assert L.cfc_fwd_step(u, h, W, b, ht, act, B, 4097, n_x, None) == -1
    assert L.cfc_fwd_step(u, h, W, b, ht, act, B, C, -1, None) == -1
    assert L.cfc_fwd_step(u, h, W, b, ht, act, B, 2048, 8000, None) == -1
    assert L.cfc_fwd_step(u, None, W, b, ht, act, B, C, n_x, None) == -1
    # h_t aliasing h_prev is a race: refused
    assert L.cfc_fwd_step(u, h, W, b, h, act, B, C, n_x, None) == -1
    assert b"overlap" in L.cfc_last_error()
    # act_t overlapping W
    assert L.cfc_fwd_step(u, h, W, b, ht, W + 4 * 3 * C * n_in - 8, B, C, n_x, None) == -1
    # backward: dh_out == dh_in, scratch overlapping W, missing scratch
    y, dhi, dho = FAKE + (6 << 20), FAKE + (7 << 20), FAKE + (8 << 20)
    S, Sb = FAKE + (9 << 20), FAKE + (10 << 20)
    assert L.cfc_bwd_step(u, h, ht, y, W, act, dhi, dhi, None, S, Sb, B, C, n_x, None) == -1
    assert L.cfc_bwd_step(u, h, ht, y, W, act, dhi, dho, None, W, Sb, B, C, n_x, None) == -1
    assert L.cfc_bwd_step(u, h, ht, y, W, act, dhi, dho, None, None, Sb, B, C, n_x, None) == -1
    assert L.cfc_bwd_step(u, h, ht, y, W, act, dhi, dho, None, S, Sb, B, C, n_x + 9000, None) == -1


def _kloop_args(B, C, n_x, K):
    """Twelve fake, non-overlapping addresses and a large enough workspace size."""
    a = [FAKE + (i << 28) for i in range(12)]
    return a[:8] + [ws_bytes(B, C, n_x, K)] + a[8:]


def test_kloop_argument_errors(L):
    B, C, n_x, K = 4, 16, 8, 3
    a = _kloop_args(B, C, n_x, K)
    assert L.cfc_train_kloop(*a, B, C, n_x, -1, None) == -1
    assert L.cfc_train_kloop(*a, -2, C, n_x, K, None) == -1
    bad = list(a)
    bad[5] = None  # h_hist
    assert L.cfc_train_kloop(*bad, B, C, n_x, K, None) == -1
    bad = list(a)
    bad[11] = bad[10]  # gW == gb_scratch
    assert L.cfc_train_kloop(*bad, B, C, n_x, K, None) == -1
    assert b"overlap" in L.cfc_last_error()
    bad = list(a)
    bad[6] = a[0]  # act over u
    assert L.cfc_train_kloop(*bad, B, C, n_x, K, None) == -1
    bad = list(a)
    bad[8] = a[8] - 4  # workspace one float short
    assert L.cfc_train_kloop(*bad, B, C, n_x, K, None) == -1
    assert b"workspace" in L.cfc_last_error()


def test_kloop_fwd_bwd_fill_argument_errors(L):
    B, C, n_x, K = 4, 16, 8, 3
    a = _kloop_args(B, C, n_x, K)[:11]   # through gb_scratch: no gW, gb
    assert L.cfc_kloop_fwd_bwd_fill(*a, B, C, n_x, -1, None) == -1
    bad = list(a)
    bad[9] = None  # gW_scratch
    assert L.cfc_kloop_fwd_bwd_fill(*bad, B, C, n_x, K, None) == -1
    assert b"null" in L.cfc_last_error()
    bad = list(a)
    bad[10] = a[0]  # gb_scratch over u
    assert L.cfc_kloop_fwd_bwd_fill(*bad, B, C, n_x, K, None) == -1
    assert b"overlap" in L.cfc_last_error()
    bad = list(a)
    bad[8] = a[8] - 4  # workspace one float short
    assert L.cfc_kloop_fwd_bwd_fill(*bad, B, C, n_x, K, None) == -1
    assert b"workspace" in L.cfc_last_error()


def test_kloop_status_argument_errors(L):
    """cfc_kloop_status refuses bad sizes and a null or short workspace before
    any HIP call; with K == 0 or B == 0 nothing was launched: CFC_OK."""
    B, C, n_x, K = 4, 16, 8, 3
    need = ws_bytes(B, C, n_x, K)
    assert L.cfc_kloop_status(None, need, B, C, n_x, K, None) == -1
    assert L.cfc_kloop_status(FAKE, need - 4, B, C, n_x, K, None) == -1
    assert b"workspace" in L.cfc_last_error()
    assert L.cfc_kloop_status(FAKE, need, B, 0, n_x, K, None) == -1
    assert L.cfc_kloop_status(FAKE, need, B, C, n_x, -1, None) == -1
    assert L.cfc_kloop_status(FAKE, ws_bytes(B, C, n_x, 0), B, C, n_x, 0, None) == 0
    assert L.cfc_kloop_status(FAKE, ws_bytes(0, C, n_x, K), 0, C, n_x, K, None) == 0


def test_projection_and_recurrence_argument_errors(L):
    # input projection: bad sizes, null pointers, output overlapping an input
    assert L.cfc_input_projection(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), -1, 8, 4, None) == -1
    assert L.cfc_input_projection(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), 16, 0, 4, None) == -1
    assert L.cfc_input_projection(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), None, 16, 8, 4, None) == -1
    assert L.cfc_input_projection(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + 64, 16, 8, 4, None) == -1
    assert b"overlap" in L.cfc_last_error()
    assert L.cfc_input_projection(None, None, None, None, 0, 8, 4, None) == 0   # M == 0: nothing to do
    # recurrence: C above what the persistent kernel holds, nulls, overlaps
    a = [FAKE + i * (1 << 30) for i in range(7)]
    assert L.cfc_kloop_recurrence(*a, 4, 129, 8, 4, None) == -1
    assert b"C <= 128" in L.cfc_last_error()
    assert L.cfc_kloop_recurrence(*(a[:6] + [None]), 4, 16, 8, 4, None) == -1
    assert L.cfc_kloop_recurrence(*(a[:4] + [a[0]] + a[5:]), 4, 16, 8, 4, None) == -1   # h_hist == X
    assert b"overlap" in L.cfc_last_error()
    assert L.cfc_kloop_recurrence(*a, 4, 16, 8, -1, None) == -1


def ws_bytes(B, C, n_x, K):
    ldf = (n_x + 15) // 16 * 16 + (C + 31) // 32 * 32
    nbt = (B + 15) // 16
    flags = (32 * (nbt * ((C + 15) // 16) + 1) + 63) // 64 * 64
    xch = 32 * nbt * ((C + 31) // 32 * 32 + 1024)
    # flags of the persistent launch that also forms X: one per workgroup
    # (one 64 x 64 tile of X each), then the error word
    proj = ((K * B + 63) // 64 * ((3 * C + 63) // 64) + 1 + B * ((K + 15) // 16) + 63) // 64 * 64
    return 4 * (((6 * K * B * C + 2 * B * C + 63) // 64) * 64 + 3 * C * ldf + 1024 * C + xch + flags + proj)


def test_workspace_size_and_path_queries(L):
    assert L.cfc_train_kloop_workspace_bytes(32, 128, 64, 64) == ws_bytes(32, 128, 64, 64)
    assert L.cfc_train_kloop_workspace_bytes(3, 37, 5, 7) == ws_bytes(3, 37, 5, 7)
    assert L.cfc_train_kloop_workspace_bytes(-1, 128, 64, 64) == 0
    # persistent kernel for C <= 128 (any n_x: X is precomputed); step kernels otherwise,
    # on MFMA from B = 64 where the shape fits them (C <= 320, n_x + C up to ~540).  The
    # resident MFMA kernel needs a device that holds its whole grid at once: without a
    # GPU (here) it fits nowhere, so its shapes take the MFMA step kernels and forcing it
    # is refused
    P, VALU, MFMA, RES = 2, 3, 4, 5
    assert L.cfc_kloop_path(32, 128, 64, 64) == P
    assert L.cfc_kloop_path(256, 256, 128, 64) == MFMA
    assert L.cfc_kloop_path(32, 256, 128, 64) == VALU      # B below the MFMA threshold
    assert L.cfc_kloop_path(256, 512, 0, 64) == VALU       # 8 channels per dz group: no MFMA layout
    assert L.cfc_kloop_path(256, 256, 400, 64) == VALU     # rows too long for the MFMA LDS tile
    assert L.cfc_kloop_path(4, 16, 8, 4) == P
    assert L.cfc_kloop_path(4, 64, 100, 4) == P
    assert L.cfc_kloop_path(4, 48, 300, 4) == P
    assert L.cfc_kloop_path(4, 100, 20, 4) == P              # 2 channels per dz group
    assert L.cfc_kloop_path(4, 128, 4000, 4) == P
    assert L.cfc_kloop_path(4, 129, 0, 4) == VALU
    assert L.cfc_set_kloop_mode(7) == -1
    assert L.cfc_set_kloop_mode(6) == -1
    assert L.cfc_set_kloop_mode(RES) == 0
    assert L.cfc_kloop_path(256, 256, 128, 64) == -1
    assert L.cfc_set_kloop_mode(0) == 0
    assert L.cfc_set_kloop_mode(1) == 0                      # steps: MFMA or VALU by shape
    assert L.cfc_kloop_path(32, 128, 64, 64) == VALU
    assert L.cfc_kloop_path(64, 128, 64, 64) == MFMA
    assert L.cfc_set_kloop_mode(4) == 0                      # MFMA forced
    assert L.cfc_kloop_path(4, 16, 8, 4) == MFMA
    assert L.cfc_kloop_path(256, 512, 0, 64) == -1
    assert L.cfc_set_kloop_mode(3) == 0                      # VALU forced
    assert L.cfc_kloop_path(256, 256, 128, 64) == VALU
    assert L.cfc_set_kloop_mode(2) == 0                      # persistent forced
    assert L.cfc_kloop_path(4, 129, 0, 4) == -1
    assert L.cfc_set_kloop_mode(0) == 0
    assert L.cfc_kloop_path(32, 128, 64, 64) == P


def test_path_mode_is_per_thread(L):
    """A mode set on one thread leaves every other thread's path alone: each
    thread starts in the automatic mode, and the setting of one thread is not
    seen by calls made on another (no process-wide path state)."""
    import threading
    P, VALU = 2, 3
    seen = {}
    go = threading.Event()
    done = threading.Event()

    def other():
        seen["before"] = L.cfc_kloop_path(32, 128, 64, 64)
        go.wait(10)
        seen["after"] = L.cfc_kloop_path(32, 128, 64, 64)
        assert L.cfc_set_kloop_mode(2) == 0          # forces persistent on this thread only
        seen["own"] = L.cfc_kloop_path(4, 129, 0, 4)
        done.set()

    th = threading.Thread(target=other)
    th.start()
    try:
        assert L.cfc_set_kloop_mode(3) == 0              # VALU forced on the main thread
        assert L.cfc_kloop_path(32, 128, 64, 64) == VALU
        go.set()
        assert done.wait(10)
        th.join(10)
        assert seen == {"before": P, "after": P, "own": -1}
        assert L.cfc_kloop_path(4, 129, 0, 4) == VALU     # the other thread's setting is not seen here
    finally:
        assert L.cfc_set_kloop_mode(0) == 0


def test_graph_cache_never_waits_on_the_device():
    """The K-loop's graph cache evicts without blocking: destruction of an
    evicted graph is deferred until its completion event reports done, so no
    call path of cfc_train_kloop reaches a host synchronisation."""
    text = open(os.path.join(ROOT, "recurrent_cell_amd", "csrc", "cfc_api.hip")).read()
    body = text[text.index("int cfc_train_kloop("):]
    body = body[:body.index("\n}\n")]
    assert "Synchronize" not in body and "destroy_entry" not in body
    reap = text[text.index("void reap_retired()"):]
    reap = reap[:reap.index("\n}\n")]
    assert "hipEventQuery" in reap and "Synchronize" not in reap
    # the one blocking destruction is reachable only from cfc_clear_graph_cache
    callers = [m.start() for m in re.finditer(r"destroy_entry\(", text)]
    clear = text.index("int cfc_clear_graph_cache(")
    assert all(c > clear for c in callers[1:]), "destroy_entry called outside cfc_clear_graph_cache"


def test_no_atomics_in_kernel_sources():
    """Device code (kernels and the shared device math) uses no read-modify-write
    atomics.  The only atomic builtins allowed are plain loads and stores with an
    agent coherence scope (__hip_atomic_load / __hip_atomic_store), by which the
    resident kernel's workgroups read one another's step counters and outputs."""
    csrc = os.path.join(ROOT, "recurrent_cell_amd", "csrc")
    for fn in ("cfc_kernels.hip", "cfc_math.h", "cfc_kernels.h", "gemm_kernels.hip", "gemm_kernels.h"):
        text = open(os.path.join(csrc, fn)).read()
        assert not re.search(r"\batomic\w*\s*\(|__atomic_|std::atomic", text), fn
        for m in re.finditer(r"__hip_atomic_\w+", text):
            assert m.group(0) in ("__hip_atomic_load", "__hip_atomic_store"), (fn, m.group(0))


def test_product_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "recurrent_cell_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, flags=re.M), fn
                assert "liboracle" not in text, fn


def _ptrs(*xs):
    return (ctypes.c_void_p * len(xs))(*xs)


def test_adamw_argument_errors(L):
    P = [FAKE + i * (1 << 30) for i in range(4)]
    n = (ctypes.c_int64 * 1)(1000)
    hp = (1e-3, 0.9, 0.999, 1e-8, 0.01)
    args = lambda nseg, hp=hp, step=1: (_ptrs(P[0]), _ptrs(P[1]), _ptrs(P[2]), _ptrs(P[3]), n, nseg,  # noqa: E731
                                        *hp, step, None)
    assert L.cfc_adamw_step(*args(5)) == -1
    assert L.cfc_adamw_step(*args(-1)) == -1
    assert L.cfc_adamw_step(*args(1, step=0)) == -1
    for bad in ((-1e-3, 0.9, 0.999, 1e-8, 0.01), (1e-3, 1.0, 0.999, 1e-8, 0.01), (1e-3, 0.9, 1.0, 1e-8, 0.01),
                (1e-3, 0.9, 0.999, 0.0, 0.01), (1e-3, 0.9, 0.999, 1e-8, -0.1),
                (float("nan"), 0.9, 0.999, 1e-8, 0.01)):
        assert L.cfc_adamw_step(*args(1, hp=bad)) == -1
        assert b"hyperparameters" in L.cfc_last_error()
    assert L.cfc_adamw_step(None, None, None, None, None, 1, *hp, 1, None) == -1
    assert L.cfc_adamw_step(_ptrs(P[0]), _ptrs(None), _ptrs(P[2]), _ptrs(P[3]), n, 1, *hp, 1, None) == -1
    neg = (ctypes.c_int64 * 1)(-4)
    assert L.cfc_adamw_step(_ptrs(P[0]), _ptrs(P[1]), _ptrs(P[2]), _ptrs(P[3]), neg, 1, *hp, 1, None) == -1
    # a parameter aliasing its own gradient, and two segments sharing a moment buffer
    assert L.cfc_adamw_step(_ptrs(P[0]), _ptrs(P[0] + 64), _ptrs(P[2]), _ptrs(P[3]), n, 1, *hp, 1, None) == -1
    assert b"overlap" in L.cfc_last_error()
    n2 = (ctypes.c_int64 * 2)(1000, 1000)
    Q = [p + (1 << 28) for p in P]
    assert L.cfc_adamw_step(_ptrs(P[0], Q[0]), _ptrs(P[1], Q[1]), _ptrs(P[2], P[2] + 256), _ptrs(P[3], Q[3]),
                            n2, 2, *hp, 1, None) == -1
    assert b"overlap" in L.cfc_last_error()
    # nothing to update: no launch
    assert L.cfc_adamw_step(None, None, None, None, None, 0, *hp, 1, None) == 0
    n0 = (ctypes.c_int64 * 1)(0)
    assert L.cfc_adamw_step(_ptrs(None), _ptrs(None), _ptrs(None), _ptrs(None), n0, 1, *hp, 1, None) == 0


# ---------------------------------------------------------------- MLP

@pytest.fixture(scope="module")
def ML(L):
    from recurrent_cell_amd import mlp
    return mlp.lib()


def _dims(*d):
    return (ctypes.c_int * len(d))(*d)


def test_mlp_param_layout(ML):
    """W_0, b_0, W_1, .. each starting at a multiple of 4 floats."""
    dims = (48, 256, 256, 128, 51)
    w = (ctypes.c_int64 * 4)()
    b = (ctypes.c_int64 * 4)()
    total = ML.mlp_param_offsets(_dims(*dims), 4, w, b)
    expect_w, expect_b, off = [], [], 0
    for l in range(4):
        expect_w.append(off)
        off += dims[l + 1] * dims[l]
        off = -(-off // 4) * 4
        expect_b.append(off)
        off += dims[l + 1]
        off = -(-off // 4) * 4
    assert list(w) == expect_w and list(b) == expect_b and total == off == 117812
    assert sum(dims[l + 1] * (dims[l] + 1) for l in range(4)) == 117811   # the parameters themselves
    assert ML.mlp_param_offsets(_dims(3, 5), 1, None, None) == 16 + 8
    assert ML.mlp_param_offsets(_dims(3, 0), 1, None, None) == -1
    assert ML.mlp_param_offsets(_dims(3, 5), 0, None, None) == -1
    assert ML.mlp_param_offsets(_dims(*([4] * 10)), 9, None, None) == -1
    assert ML.mlp_param_offsets(_dims(4097, 5), 1, None, None) == -1


def test_mlp_splits_and_workspace(ML):
    assert ML.mlp_weight_grad_splits(16384) == 32
    assert ML.mlp_weight_grad_splits(1) == 1
    assert ML.mlp_weight_grad_splits(1000) == 1
    assert ML.mlp_weight_grad_splits(1100) == 2
    # splits of at most 2^24 rows still 32
    assert ML.mlp_weight_grad_splits(1 << 24) == 32
    S = 32
    assert ML.mlp_linear_bwd_weight_workspace_bytes(16384, 256, 256) == 4 * (S * 65536 + S * 256)
    assert ML.mlp_linear_bwd_weight_workspace_bytes(16384, 128, 51) == 4 * (S * 51 * 128 + (-(-S * 51 // 4)) * 4)
    assert ML.mlp_linear_bwd_weight_workspace_bytes(-1, 4, 4) == 0
    assert ML.mlp_mse_workspace_bytes(16384) == 4 * 256
    dims = _dims(48, 256, 256, 128, 51)
    ldy = [256, 256, 128, 52]
    expect = 16384 * sum(ldy) + S * 117812 + 256
    assert ML.mlp_train_step_workspace_bytes(16384, dims, 4) == 4 * expect
    assert ML.mlp_train_step_workspace_bytes(0, dims, 4) == 0


def test_mlp_argument_errors(ML):
    F = FAKE
    a = [F + i * (1 << 32) for i in range(8)]
    assert ML.mlp_linear_fwd(a[0], a[1], a[2], a[3], -1, 4, 4, 1, None) == -1
    assert ML.mlp_linear_fwd(a[0], a[1], a[2], a[3], 16, 0, 4, 1, None) == -1
    assert ML.mlp_linear_fwd(a[0], a[1], a[2], a[3], 16, 4, 4097, 1, None) == -1
    assert ML.mlp_linear_fwd(None, a[1], a[2], a[3], 16, 4, 4, 1, None) == -1
    assert ML.mlp_linear_fwd(a[0], a[1], a[2], a[0] + 32, 16, 4, 4, 1, None) == -1   # Y overlaps X
    assert b"overlap" in ML.cfc_last_error()
    assert ML.mlp_linear_fwd(None, None, None, None, 0, 4, 4, 1, None) == 0           # M == 0: nothing to do
    assert ML.mlp_linear_bwd_data(a[0], a[1], a[2], a[2] + 16, 16, 4, 4, None) == -1  # dX overlaps the mask
    assert ML.mlp_linear_bwd_data(a[0], None, None, a[3], 16, 4, 4, None) == -1
    ws_need = ML.mlp_linear_bwd_weight_workspace_bytes(16, 4, 4)
    assert ML.mlp_linear_bwd_weight(a[0], a[1], a[2], a[3], 16, 4, 4, a[4], ws_need - 4, None) == -1
    assert b"workspace" in ML.cfc_last_error()
    assert ML.mlp_linear_bwd_weight(a[0], a[1], a[2], a[2] + 8, 16, 4, 4, a[4], ws_need, None) == -1
    assert ML.mlp_linear_bwd_weight(a[0], a[1], None, a[3], 16, 4, 4, a[4], ws_need, None) == -1
    assert ML.mlp_mse_loss_grad(a[0], a[1], a[2], a[3], 0, 4, a[4], 4096, None) == -1
    assert ML.mlp_mse_loss_grad(a[0], a[1], a[0], a[3], 16, 4, a[4], 4096, None) == -1
    assert ML.mlp_mse_loss_grad(a[0], a[1], a[2], a[3], 16, 4, a[4], 0, None) == -1
    dims = _dims(8, 16, 4)
    acts = (ctypes.c_void_p * 2)(a[5], a[6])
    need = ML.mlp_train_step_workspace_bytes(32, dims, 2)
    ok = (a[0], a[1], 32, dims, 2, a[2], a[3], acts, a[4], a[7], need, None)
    bad = list(ok)
    bad[10] = need - 4
    assert ML.mlp_train_step(*bad) == -1 and b"workspace" in ML.cfc_last_error()
    bad = list(ok)
    bad[2] = 0
    assert ML.mlp_train_step(*bad) == -1
    bad = list(ok)
    bad[4] = 0
    assert ML.mlp_train_step(*bad) == -1
    bad = list(ok)
    bad[7] = (ctypes.c_void_p * 2)(a[5], None)
    assert ML.mlp_train_step(*bad) == -1
    bad = list(ok)
    bad[7] = (ctypes.c_void_p * 2)(a[5], a[5] + 64)                                      # two outputs overlap
    assert ML.mlp_train_step(*bad) == -1 and b"overlap" in ML.cfc_last_error()
    bad = list(ok)
    bad[3] = (ctypes.c_int * 3)(8, 0, 4)
    assert ML.mlp_train_step(*bad) == -1


def test_weight_grad_gemm_argument_errors(L):
    a = [FAKE + i * (1 << 32) for i in range(10)]
    need = L.cfc_weight_grad_gemm_workspace_bytes(32, 128, 64, 64)
    assert need > 0 and need % 16 == 0
    assert L.cfc_weight_grad_gemm_workspace_bytes(32, 0, 64, 64) == 0
    ok = (a[0], a[1], a[2], a[3], a[4], 32, 128, 64, 64, a[5], need, None)
    bad = list(ok)
    bad[10] = need - 4
    assert L.cfc_weight_grad_gemm(*bad) == -1 and b"workspace" in L.cfc_last_error()
    bad = list(ok)
    bad[4] = a[3] + 64                      # gb inside gW
    assert L.cfc_weight_grad_gemm(*bad) == -1 and b"overlap" in L.cfc_last_error()
    bad = list(ok)
    bad[0] = None
    assert L.cfc_weight_grad_gemm(*bad) == -1
    bad = list(ok)
    bad[8] = -1
    assert L.cfc_weight_grad_gemm(*bad) == -1
    kneed = L.cfc_train_kloop_gemm_workspace_bytes(32, 128, 64, 64)
    assert kneed == L.cfc_train_kloop_workspace_bytes(32, 128, 64, 64) + need
    kok = (a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7], a[8], a[9], kneed, 32, 128, 64, 64, None)
    bad = list(kok)
    bad[10] = kneed - 4
    assert L.cfc_train_kloop_gemm(*bad) == -1
    bad = list(kok)
    bad[7] = a[5]                            # gW on h_hist
    assert L.cfc_train_kloop_gemm(*bad) == -1 and b"overlap" in L.cfc_last_error()


# ---------------------------------------------------------------- FMA-rate probe

def test_probe_fma_argument_errors(L):
    L.cfc_probe_fma.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    L.cfc_probe_fma.restype = ctypes.c_int
    for blocks, threads, iters in ((0, 512, 1), (65537, 512, 1), (1, 0, 1), (1, 96, 1), (1, 1088, 1),
                                   (1, 512, 0), (1, 512, (1 << 20) + 1)):
        assert L.cfc_probe_fma(blocks, threads, 1, iters, FAKE, None) == -1
    assert L.cfc_probe_fma(1, 512, 1, 1, None, None) == -1
    assert b"NULL" in L.cfc_last_error()


def test_noalloc_size_check_comes_first(L):
    """cfc_train_kloop_noalloc refuses sizes whose workspace exceeds its fixed
    array before any HIP call (so this runs without a GPU)."""
    a = [FAKE + i * (1 << 32) for i in range(11)]
    limit = 32 << 20
    assert L.cfc_train_kloop_workspace_bytes(256, 256, 128, 64) > limit
    assert L.cfc_train_kloop_noalloc(*a, 256, 256, 128, 64, None) == -1
    assert b"fixed workspace" in L.cfc_last_error()
    assert L.cfc_train_kloop_noalloc(*a, 4, 0, 8, 4, None) == -1          # C = 0
    assert L.cfc_train_kloop_noalloc(*a, 4, 16, 8, -1, None) == -1        # K < 0
