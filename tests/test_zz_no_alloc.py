"""The K-loop step without a caller workspace (cfc_train_kloop_noalloc),
called through the C ABI, against cfc_train_kloop on the same inputs: the
same kernels on the same arrays, so every output must have the same bits.
Two calls in a row on each path, the second with smaller sizes, so that the
second runs on the fixed workspace the first one left behind."""
import sys

import numpy as np
import pytest
import torch

from recurrent_cell_amd.inputs import cfc_inputs

pytestmark = pytest.mark.gpu

OUTPUTS = ("h_hist", "act", "gW_scratch", "gb_scratch", "gW", "gb")


def say(*a):
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def cfc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from recurrent_cell_amd import cfc as mod
    mod.lib()
    return mod


def run_both(cfc, d, seed):
    x = cfc_inputs(**d, seed=seed, bias_scale=0.2)
    t = [torch.from_numpy(a).cuda() for a in (x.u, x.y, x.h0, x.W, x.bias)]
    ref = cfc.cfc_train_kloop(*t)
    out = cfc.KloopBuffers.allocate(d["B"], d["C"], d["n_x"], d["K"], "cuda")
    for k in OUTPUTS:
        getattr(out, k).fill_(float("nan"))
    cfc.cfc_train_kloop_noalloc(*t, out=out)
    torch.cuda.synchronize()
    for k in OUTPUTS:
        a = getattr(out, k).view(torch.int32).cpu().numpy()
        b = getattr(ref, k).view(torch.int32).cpu().numpy()
        np.testing.assert_array_equal(a, b, err_msg=k)


@pytest.mark.parametrize("mode,first,second", [
    ("auto", dict(B=32, C=128, n_x=64, K=64), dict(B=4, C=16, n_x=8, K=4)),           # persistent kernel
    ("steps", dict(B=64, C=132, n_x=4, K=5), dict(B=3, C=129, n_x=0, K=2)),           # MFMA, then VALU steps
    ("steps_valu", dict(B=33, C=40, n_x=12, K=6), dict(B=2, C=20, n_x=5, K=3)),       # VALU steps, ragged
    ("resident", dict(B=64, C=132, n_x=4, K=5), dict(B=32, C=128, n_x=64, K=8)),      # resident MFMA kernel
])
def test_noalloc_equals_train_kloop_on_two_calls(cfc, mode, first, second):
    m = {"auto": cfc.KLOOP_AUTO, "steps": cfc.KLOOP_STEPS, "steps_valu": cfc.KLOOP_STEPS_VALU,
         "resident": cfc.KLOOP_RESIDENT}[mode]
    cfc.cfc_set_kloop_mode(m)
    try:
        for i, d in enumerate((first, second)):
            if cfc.cfc_kloop_path(d["B"], d["C"], d["n_x"], d["K"]) < 0:
                pytest.skip("the forced path cannot take this shape on this device")
            say("no-alloc K-loop", mode, "call", i + 1, d, "path", cfc.cfc_kloop_path(d["B"], d["C"], d["n_x"],
                                                                                    d["K"]))
            run_both(cfc, d, seed=31 + i)
    finally:
        cfc.cfc_set_kloop_mode(cfc.KLOOP_AUTO)


def test_noalloc_refuses_sizes_beyond_its_workspace(cfc):
    """The wide configuration needs about 100 MB of workspace: refused before
    anything is enqueued."""
    d = dict(B=256, C=256, n_x=128, K=64)
    say("no-alloc refusal", d)
    assert cfc.cfc_train_kloop_workspace_bytes(**d) > (32 << 20)
    out = cfc.KloopBuffers.allocate(1, 1, 0, 1, "cuda")
    L = cfc.lib()
    p = out.gW.data_ptr()
    rc = L.cfc_train_kloop_noalloc(p, p, p, p, p, p, p, p, p, p, p, d["B"], d["C"], d["n_x"], d["K"], None)
    assert rc == cfc.CFC_EINVAL
    assert "fixed workspace" in cfc.last_error()
