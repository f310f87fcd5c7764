"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Every case prints its name before touching the GPU.  Floating-point criteria
are in tests/tolerances.py; structural properties (determinism, K-loop
(graph replay or direct launches) == eager single-step calls, batched row ==
single-sample run, scratch cleared between steps,
overwrite semantics, exact special cases) are checked bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

from recurrent_cell_amd.inputs import CONFIGS, adamw_inputs, cfc_inputs, normal, reduce_rows, small_int_rows
from tests.tolerances import (assert_ok, check_act, check_adamw, check_grad, check_reduce, check_vs_fp32,
                              describe, grad_mass)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": CONFIGS["tiny"],
    "pages": CONFIGS["pages"],
    "wide": CONFIGS["wide"],
    "ragged_scalar": dict(B=3, C=20, n_x=5, K=3),     # n_in = 25: scalar path, partial tile
    "three_tiles": dict(B=5, C=40, n_x=12, K=5),       # 3 channel tiles, last one partial
    "sample_tiles": dict(B=130, C=24, n_x=8, K=3),     # 4 samples per workgroup, ragged last
    "no_input": dict(B=2, C=16, n_x=0, K=3),           # n_x = 0: autonomous recurrence
    "long_input64": dict(B=3, C=64, n_x=100, K=6),     # n_x > C; one channel per dz group, 2 column blocks
    "long_input48": dict(B=2, C=48, n_x=200, K=5),     # n_in = 248; ragged second column block
    "two_channel_groups": dict(B=3, C=100, n_x=20, K=7),  # 2 channels per dz group, last groups partial
    "three_blocks": dict(B=3, C=72, n_x=36, K=5),      # 3 recurrent column blocks of 32, 2 channels per group
    "odd_channels": dict(B=2, C=37, n_x=3, K=4),       # C and n_x not multiples of 4: scalar moves
    "mfma_max": dict(B=64, C=320, n_x=128, K=3),       # the largest shape the MFMA step kernels take
    "long_ragged_k": dict(B=3, C=64, n_x=12, K=37),    # whole chunks, then a ragged one, in both directions
    "single_step": dict(B=1, C=16, n_x=8, K=1),        # K = 1, one sample
    "single_step_max_c": dict(B=3, C=128, n_x=64, K=1),  # K = 1 at the persistent kernel's largest C
    "one_channel": dict(B=2, C=1, n_x=3, K=2),         # C = 1
    "valu_c129": dict(B=65, C=129, n_x=4, K=2),        # one channel past the persistent kernel: VALU steps
    "mfma_long_k": dict(B=64, C=132, n_x=4, K=17),     # MFMA step kernels over more steps than a chunk
    "whole_chunks": dict(B=3, C=100, n_x=20, K=32),    # K a multiple of the chunk: backward's first chunk from LDS
    "whole_chunks_odd": dict(B=2, C=37, n_x=3, K=16),  # the same with scalar moves (C % 4 != 0)
}
MAX_SIZE = dict(B=1, C=2048, n_x=6144, K=2)            # CFC_MAX_C channels, n_in = CFC_MAX_N_IN


def need_path(cfc, d):
    """Skip when the forced K-loop path cannot take this shape."""
    if cfc.cfc_kloop_path(d["B"], d["C"], d["n_x"], d["K"]) < 0:
        pytest.skip("the forced path cannot take this shape")


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


@pytest.fixture
def path(cfc, request):
    """Force a K-loop path for one test ("auto" keeps the default), then restore it."""
    mode = {"auto": cfc.KLOOP_AUTO, "steps": cfc.KLOOP_STEPS, "persistent": cfc.KLOOP_PERSISTENT,
            "steps_valu": cfc.KLOOP_STEPS_VALU, "steps_mfma": cfc.KLOOP_STEPS_MFMA,
            "resident": cfc.KLOOP_RESIDENT}[request.param]
    cfc.cfc_set_kloop_mode(mode)
    yield request.param
    cfc.cfc_set_kloop_mode(cfc.KLOOP_AUTO)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def kloop_dev(cfc, x, out=None):
    t = [dev(a) for a in (x.u, x.y, x.h0, x.W, x.bias)]
    return cfc.cfc_train_kloop(*t, out=out), t


def bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


# ---------------------------------------------------------------- K-loop parity

PATH_NAMES = {2: "persistent", 3: "steps_valu", 4: "steps_mfma", 5: "resident"}


# the seeds of the parity cases: three at the configured pages and wide shapes,
# one elsewhere
KLOOP_CASES = [(c, s) for c in CASES for s in ((0, 1, 2) if c in ("pages", "wide") else (1,))]


def kloop_parity(cfc, oracle_mod, x, label, vs_fp32=False):
    """Every K-loop path that takes these sizes (the automatic one when it is
    the persistent kernel, then the VALU and the MFMA step kernels) against
    one fp64 oracle run at the activation and gradient tolerances -- or, with
    vs_fp32, no worse than 4x the oracle's own fp32 evaluation in units of
    those tolerances (for inputs where no fp32 evaluation meets them); returns
    the paths checked and the GPU outputs of the first."""
    K, B, n_x = x.u.shape
    C = x.h0.shape[1]
    r = oracle_mod.train(x.u, x.y, x.h0, x.W, x.bias, "f64", want_dp=True)
    r32 = oracle_mod.train(x.u, x.y, x.h0, x.W, x.bias, "f32") if vs_fp32 else None
    m = grad_mass(x.u, r["h_hist"], r["dp"])
    names = (("h_hist", "h_hist"), ("act", "act"), ("S", "gW_scratch"), ("Sb", "gb_scratch"), ("gW", "gW"),
             ("gb", "gb"))
    checked, first = [], None
    for mode in (cfc.KLOOP_AUTO, cfc.KLOOP_STEPS_VALU, cfc.KLOOP_STEPS_MFMA, cfc.KLOOP_RESIDENT):
        cfc.cfc_set_kloop_mode(mode)
        try:
            taken = cfc.cfc_kloop_path(B, C, n_x, K)
            if taken < 0 or (mode == cfc.KLOOP_AUTO and taken != cfc.KLOOP_PERSISTENT):
                continue
            say("kloop parity", label, "path", PATH_NAMES[taken])
            out, _ = kloop_dev(cfc, x)
            g = {k: host(getattr(out, a)) for k, a in names}
        finally:
            cfc.cfc_set_kloop_mode(cfc.KLOOP_AUTO)
        if vs_fp32:
            bound = {k: 1e-6 + 1e-5 * np.abs(r[k]) for k in ("h_hist", "act")}
            bound.update({k: 1e-6 + 1e-4 * np.abs(r[k]) + 16 * 2.0 ** -24 * m[k] for k in ("S", "Sb", "gW", "gb")})
            reps = [check_vs_fp32(k, g[k], r[k], r32[k], bound[k]) for k, _ in names]
            for rep in reps:
                say("  ", rep["name"], "worst", "%.3g" % rep["worst_ratio"], "fp32 oracle",
                    "%.3g" % rep["worst_fp32"], "normwise", "%.3g" % rep["normwise"], "fp32",
                    "%.3g" % rep["normwise_fp32"])
        else:
            reps = [check_act(k, g[k], r[k]) for k in ("h_hist", "act")]
            reps += [check_grad(k, g[k], r[k], m[k]) for k in ("S", "Sb", "gW", "gb")]
            for rep in reps:
                say("  ", describe(rep))
        for rep in reps:
            assert_ok(rep)
        checked.append(PATH_NAMES[taken])
        if first is None:
            first = g
    return checked, first


@pytest.mark.parametrize("case,seed", KLOOP_CASES, ids=["%s-seed%d" % cs for cs in KLOOP_CASES])
def test_kloop_matches_oracle(cfc, oracle_mod, case, seed):
    d = CASES[case]
    x = cfc_inputs(**d, seed=seed, bias_scale=0.2)
    checked, _ = kloop_parity(cfc, oracle_mod, x, "%s seed %d %s" % (case, seed, d))
    assert checked


SAT_SHAPE = dict(B=8, C=64, n_x=16, K=8)


def test_kloop_saturated_cell_matches_oracle(cfc, oracle_mod):
    """The cell at its saturated edges, on every path (the resident kernel
    too where the device holds its grid), through the biases:
    channel c mod 4 = 0, 1 has b_f = +100, -100 (exp(a_f) overflows or
    underflows in fp32: gate exactly 0 or 1), c mod 4 = 2 has b_f = +40,
    b_g = +30, b_h = -30, and c mod 4 = 3 has b_f = -40, b_g = -60, b_h = +60
    (exp(2a) overflows or underflows: tanh exactly +-1).  Outputs stay finite,
    gate in [0, 1] and |h| <= 1, within the stated tolerances of the oracle
    (the recurrence stays well conditioned: saturated heads pass no error)."""
    d = SAT_SHAPE
    x = cfc_inputs(**d, seed=21, bias_scale=0.2)
    pat = np.arange(d["C"]) % 4
    x.bias[0] = np.choose(pat, [100.0, -100.0, 40.0, -40.0]).astype(np.float32)
    x.bias[1] = np.where(pat == 2, 30.0, np.where(pat == 3, -60.0, x.bias[1])).astype(np.float32)
    x.bias[2] = np.where(pat == 2, -30.0, np.where(pat == 3, 60.0, x.bias[2])).astype(np.float32)
    checked, g = kloop_parity(cfc, oracle_mod, x, "saturated by the biases %s" % d)
    assert {"persistent", "steps_valu", "steps_mfma"} <= set(checked), checked
    for k, v in g.items():
        assert np.isfinite(v).all(), k
    gate = g["act"][:, 0]
    assert np.all(gate >= 0) and np.all(gate <= 1)
    assert np.all(gate[:, :, pat == 0] == 0) and np.all(gate[:, :, pat == 1] == 1)
    tanh = g["act"][:, 1:]
    assert np.all(np.abs(tanh[:, :, :, pat >= 2]) == 1.0)
    assert np.all(np.abs(g["h_hist"][1:]) <= 1.0)


def test_kloop_large_weights_no_worse_than_fp32(cfc, oracle_mod):
    """Saturation through large weights: the g and hh heads' weights scaled
    40x drive |a| far past 10 (tanh rounds to +-1 on most entries) and f-head
    biases of +-40 and +-100 saturate the gate.  Where a head is not saturated
    the recurrence then amplifies every rounding error about 40x per step, so
    no fp32 evaluation meets the stated tolerances (the oracle's own fp32 run
    misses them by hundreds of times); every path must be no worse than 4x
    that fp32 evaluation."""
    d = SAT_SHAPE
    x = cfc_inputs(**d, seed=21, bias_scale=0.2)
    x.bias[0] = np.resize(np.array([40.0, -40.0, 100.0, -100.0], np.float32), d["C"])
    x.W[1] *= 40.0
    x.W[2] *= 40.0
    a_g = np.einsum("ck,bk->bc", x.W[1].astype(np.float64),
                    np.concatenate([x.u[0], x.h0], axis=1).astype(np.float64))
    assert np.mean(np.abs(a_g) > 10) > 0.5
    checked, g = kloop_parity(cfc, oracle_mod, x, "large weights %s" % d, vs_fp32=True)
    assert {"persistent", "steps_valu", "steps_mfma"} <= set(checked), checked
    for k, v in g.items():
        assert np.isfinite(v).all(), k
    gate = g["act"][:, 0]
    assert np.all(gate >= 0) and np.all(gate <= 1)
    assert np.any(gate == 0) and np.any(gate == 1)
    assert np.mean(np.abs(g["act"][:, 1:]) == 1.0) > 0.3
    assert np.all(np.abs(g["h_hist"][1:]) <= 1.0)


# ---------------------------------------------------------------- single steps

@pytest.mark.parametrize("case", ["tiny", "pages", "ragged_scalar", "three_tiles", "sample_tiles", "no_input",
                                  "long_input48", "odd_channels"])
def test_fwd_step_matches_oracle(cfc, oracle_mod, case):
    d = CASES[case]
    say("fwd step parity", case)
    x = cfc_inputs(**d, seed=2, bias_scale=0.5)
    h_t, act_t = cfc.cfc_fwd_step(dev(x.u[0]), dev(x.h0), dev(x.W), dev(x.bias))
    rh, ra = oracle_mod.fwd_step(x.u[0], x.h0, x.W, x.bias, "f64")
    assert_ok(check_act("h_t", host(h_t), rh))
    assert_ok(check_act("act_t", host(act_t), ra))


@pytest.mark.parametrize("case", ["tiny", "pages", "ragged_scalar", "three_tiles", "sample_tiles", "no_input"])
@pytest.mark.parametrize("carry", [True, False])
def test_bwd_step_matches_oracle(cfc, oracle_mod, case, carry):
    d = CASES[case]
    say("bwd step parity", case, "carry" if carry else "zero carry")
    B, C, n_x = d["B"], d["C"], d["n_x"]
    n_in = n_x + C
    x = cfc_inputs(**d, seed=3, bias_scale=0.3)
    h_t, act_t = oracle_mod.fwd_step(x.u[0], x.h0, x.W, x.bias, "f32")
    dh_in = normal((B, C), 3, 1) if carry else None
    S0 = normal((B, 3, C, n_in), 3, 2)
    Sb0 = normal((B, 3, C), 3, 3)
    S_dev, Sb_dev = dev(S0), dev(Sb0)
    dh_out, du = cfc.cfc_bwd_step(dev(x.u[0]), dev(x.h0), dev(h_t), dev(x.y[0]), dev(x.W), dev(act_t),
                                  dev(dh_in) if carry else None, S_dev, Sb_dev, want_du=n_x > 0)
    zero = np.zeros((B, C), np.float32)
    r_dh, r_du, r_S, r_Sb, r_dp = oracle_mod.bwd_step(x.u[0], x.h0, h_t, x.y[0], x.W, act_t,
                                                      dh_in if carry else zero, S0, Sb0, "f64")
    adp = np.abs(r_dp)                                     # [3,B,C]
    z = np.concatenate([x.u[0], x.h0], axis=1).astype(np.float64)
    mdz = np.einsum("qbc,qck->bk", adp, np.abs(x.W.astype(np.float64)))
    mS = np.abs(S0) + adp.transpose(1, 0, 2)[..., None] * np.abs(z)[:, None, None, :]
    mSb = np.abs(Sb0) + adp.transpose(1, 0, 2)
    assert_ok(check_grad("dh_out", host(dh_out), r_dh, mdz[:, n_x:]))
    if n_x > 0:
        assert_ok(check_grad("du_t", host(du), r_du, mdz[:, :n_x]))
    assert_ok(check_grad("S", host(S_dev), r_S, mS))
    assert_ok(check_grad("Sb", host(Sb_dev), r_Sb, mSb))


def test_bwd_carry_bits_do_not_depend_on_du_request(cfc):
    d = CASES["pages"]
    say("bwd du request independence")
    x = cfc_inputs(**d, seed=4)
    h_t, act_t = cfc.cfc_fwd_step(dev(x.u[0]), dev(x.h0), dev(x.W), dev(x.bias))
    outs = []
    for want in (False, True):
        S = torch.zeros((d["B"], 3, d["C"], d["n_x"] + d["C"]), device="cuda")
        Sb = torch.zeros((d["B"], 3, d["C"]), device="cuda")
        dh, _ = cfc.cfc_bwd_step(dev(x.u[0]), dev(x.h0), h_t, dev(x.y[0]), dev(x.W), act_t, None, S, Sb,
                                 want_du=want)
        outs.append((host(dh), host(S)))
    np.testing.assert_array_equal(bits(outs[0][0]), bits(outs[1][0]))
    np.testing.assert_array_equal(bits(outs[0][1]), bits(outs[1][1]))


@pytest.mark.parametrize("case", ["tiny", "pages", "wide", "ragged_scalar", "no_input", "long_input48",
                                  "odd_channels"])
def test_input_projection_matches_oracle(cfc, oracle_mod, case):
    d = CASES[case]
    say("input projection parity", case)
    x = cfc_inputs(**d, seed=8, bias_scale=0.5)
    X = host(cfc.cfc_input_projection(dev(x.u), dev(x.W), dev(x.bias)))
    ref = oracle_mod.input_projection(x.u, x.W, x.bias, "f64")
    n_x = d["n_x"]
    Wx = np.abs(x.W[:, :, :n_x].reshape(3 * d["C"], n_x).astype(np.float64))
    mass = np.abs(x.bias.reshape(-1)).astype(np.float64) + np.abs(x.u.astype(np.float64)) @ Wx.T
    assert_ok(check_grad("X", X, ref, mass))


@pytest.mark.parametrize("case,rows", [("wide", 37), ("wide", 256), ("wide", 4000), ("odd_channels", 5)])
def test_input_projection_rows_do_not_depend_on_the_launch(cfc, case, rows):
    """Each row of X has one canonical value: the first rows projected on
    their own (a small grid, a ragged last row tile) equal the same rows of
    the full call (the wide shape's 16,384 rows), bit for bit."""
    d = CASES[case]
    say("input projection rows", case, rows)
    x = cfc_inputs(**d, seed=18, bias_scale=0.5)
    u = dev(x.u).reshape(-1, d["n_x"])
    W, bias = dev(x.W), dev(x.bias)
    full = host(cfc.cfc_input_projection(u, W, bias))
    part = host(cfc.cfc_input_projection(u[:rows].contiguous(), W, bias))
    np.testing.assert_array_equal(bits(part), bits(full[:rows]))


def persist_flag_region(B, C, K):
    """Words of the workspace's last region, the flags of a persistent launch
    that formed X itself: one per projection workgroup (one 64 x 64 tile of
    X each), the error word, then one per sample and backward chunk of 16
    steps (set when the launch also forms the scratch)."""
    n = -(-K * B // 64) * -(-3 * C // 64)
    return n, (n + 1 + B * -(-K // 16) + 63) // 64 * 64


def persist_projection_flags(ws, B, C, K):
    """(projection flags, error word) of that region."""
    n, region = persist_flag_region(B, C, K)
    f = host(ws[ws.numel() - region:]).view(np.int32)
    return f[:n], f[n]


def persist_chunk_flags(ws, B, C, K):
    """The chunk flags of that region, [B, ceil(K / 16)]."""
    n, region = persist_flag_region(B, C, K)
    f = host(ws[ws.numel() - region:]).view(np.int32)
    return f[n + 1:n + 1 + B * -(-K // 16)].reshape(B, -(-K // 16))


def test_persistent_wait_that_gives_up_is_reported(cfc):
    """The host forces the persistent launch's wait for its input projection
    to give up: it writes the next launch's number into the error word
    first, so the sample workgroups stop waiting at their first poll and the
    kernel finishes as usual.  cfc_kloop_status then reports CFC_EHIP; after
    a normal call on the same workspace it reports nothing again."""
    d = CASES["pages"]
    B, C, n_x, K = d["B"], d["C"], d["n_x"], d["K"]
    say("persistent wait forced to give up", d)
    x = cfc_inputs(**d, seed=5)
    u, y, h0, W, bias = [dev(a) for a in (x.u, x.y, x.h0, x.W, x.bias)]
    a = cfc.KloopBuffers.allocate(B, C, n_x, K, "cuda")
    assert cfc.cfc_kloop_path(B, C, n_x, K) == cfc.KLOOP_PERSISTENT
    cfc.cfc_kloop_fwd_bwd(u, y, h0, W, bias, out=a)
    cfc.cfc_kloop_status(a, B, C, n_x, K)
    flags, err = persist_projection_flags(a.ws, B, C, K)
    n, region = persist_flag_region(B, C, K)
    words = a.ws[a.ws.numel() - region:].view(torch.int32)
    words[n] = int(flags[0]) + 1   # the next launch's number (launch numbers count up by one)
    torch.cuda.synchronize()
    cfc.cfc_kloop_fwd_bwd(u, y, h0, W, bias, out=a)
    with pytest.raises(cfc.CfcError) as e:
        cfc.cfc_kloop_status(a, B, C, n_x, K)
    assert e.value.code == cfc.CFC_EHIP
    flags, err = persist_projection_flags(a.ws, B, C, K)
    assert err == flags[0]
    cfc.cfc_kloop_fwd_bwd(u, y, h0, W, bias, out=a)
    cfc.cfc_kloop_status(a, B, C, n_x, K)


@pytest.mark.parametrize("case", ["tiny", "pages", "long_input48", "long_ragged_k", "no_input", "single_step",
                                  "two_channel_groups"])
def test_persistent_step_forms_scratch_in_launch(cfc, case):
    """For B <= 128, rows of whole float4 and a launch whose workgroups fit
    the device's CUs one each, the persistent step's one launch also forms
    the per-sample scratch: fill units follow the backward one chunk of 16
    steps at a time, each after its sample's chunk flag.  After the step
    every chunk flag holds the launch's number (none does where the CUs are
    too few and the fill is a launch of its own), no wait gave up, and the
    scratch has the bits of cfc_scratch_fill (its own launch) over the same
    dp, h_hist and u."""
    d = CASES[case]
    B, C, n_x, K = d["B"], d["C"], d["n_x"], d["K"]
    say("scratch formed in the persistent launch", case)
    x = cfc_inputs(**d, seed=21, bias_scale=0.2)
    u, y, h0, W, bias = [dev(a) for a in (x.u, x.y, x.h0, x.W, x.bias)]
    assert cfc.cfc_kloop_path(B, C, n_x, K) == cfc.KLOOP_PERSISTENT
    # every workgroup of the launch resident at once: at most one per CU
    n_proj = -(-K * B // 64) * -(-3 * C // 64)
    fused = max(n_proj, B * -(-3 * C // 64)) + B <= torch.cuda.get_device_properties(0).multi_processor_count
    g = cfc.cfc_train_kloop(u, y, h0, W, bias)
    cfc.cfc_kloop_status(g, B, C, n_x, K)
    flags, err = persist_projection_flags(g.ws, B, C, K)
    chunks = persist_chunk_flags(g.ws, B, C, K)
    assert err != flags[0]
    if fused:
        np.testing.assert_array_equal(chunks, np.full_like(chunks, flags[0]))
    else:   # the scratch fill is a launch of its own: no chunk flag holds this launch's number
        assert not (chunks == flags[0]).any()
    dp = g.ws[:K * B * 3 * C].view(K, B, 3 * C)
    S = torch.full_like(g.gW_scratch, float("nan"))
    Sb = torch.full_like(g.gb_scratch, float("nan"))
    cfc.cfc_scratch_fill(dp, u, g.h_hist, S, Sb)
    np.testing.assert_array_equal(bits(host(S)), bits(host(g.gW_scratch)))
    np.testing.assert_array_equal(bits(host(Sb)), bits(host(g.gb_scratch)))
    # cfc_kloop_fwd_bwd_fill: the same launch without the reduction, same bits
    f = cfc.KloopBuffers.allocate(B, C, n_x, K, "cuda")
    f.gW_scratch.fill_(float("nan"))
    f.gb_scratch.fill_(float("nan"))
    cfc.cfc_kloop_fwd_bwd_fill(u, y, h0, W, bias, out=f)
    cfc.cfc_kloop_status(f, B, C, n_x, K)
    chunks_f = persist_chunk_flags(f.ws, B, C, K)
    if fused:
        np.testing.assert_array_equal(chunks_f, np.full_like(chunks_f, persist_projection_flags(f.ws, B, C, K)[0][0]))
    for k in ("h_hist", "act", "gW_scratch", "gb_scratch"):
        np.testing.assert_array_equal(bits(host(getattr(f, k))), bits(host(getattr(g, k))), err_msg=k)
    np.testing.assert_array_equal(bits(host(f.ws[:K * B * 3 * C])), bits(host(dp.reshape(-1))))


@pytest.mark.parametrize("case", ["pages", "ragged_scalar", "three_blocks", "odd_channels"])
def test_recurrence_composes_to_fwd_bwd(cfc, case):
    """cfc_input_projection then cfc_kloop_recurrence (two launches) gives
    the bits of cfc_kloop_fwd_bwd on the persistent path, whose one launch
    (B <= 128) also forms X: extra workgroups form it while the sample
    workgroups load W, and those wait for them.  Its bookkeeping afterwards:
    every projection workgroup's flag holds the launch's number and the
    error word, which a wait that gave up would have set to it, does not."""
    d = CASES[case]
    say("projection + recurrence == fwd_bwd", case)
    x = cfc_inputs(**d, seed=9, bias_scale=0.3)
    u, y, h0, W, bias = [dev(a) for a in (x.u, x.y, x.h0, x.W, x.bias)]
    cfc.cfc_set_kloop_mode(cfc.KLOOP_PERSISTENT)
    try:
        a = cfc.KloopBuffers.allocate(d["B"], d["C"], d["n_x"], d["K"], "cuda")
        a.ws.fill_(float("nan"))
        # first on other inputs, so that the flags and X of an earlier
        # launch are in place: X read before this launch formed it would
        # show in the bits
        cfc.cfc_kloop_fwd_bwd(dev(-0.5 * x.u), y, h0, W, bias, out=a)
        cfc.cfc_kloop_fwd_bwd(u, y, h0, W, bias, out=a)
        cfc.cfc_kloop_status(a, d["B"], d["C"], d["n_x"], d["K"])   # raises if a wait gave up
    finally:
        cfc.cfc_set_kloop_mode(cfc.KLOOP_AUTO)
    if d["B"] <= 128:
        flags, err = persist_projection_flags(a.ws, d["B"], d["C"], d["K"])
        assert flags[0] != 0 and err != flags[0], "a wait for the input projection gave up"
        np.testing.assert_array_equal(flags, np.full(flags.size, flags[0], np.int32))
    b = cfc.KloopBuffers.allocate(d["B"], d["C"], d["n_x"], d["K"], "cuda")
    X = cfc.cfc_input_projection(u, W, bias)
    cfc.cfc_kloop_recurrence(X, y, h0, W, out=b)
    n = d["K"] * d["B"] * 3 * d["C"]
    for k in ("h_hist", "act"):
        np.testing.assert_array_equal(bits(host(getattr(a, k))), bits(host(getattr(b, k))), err_msg=k)
    np.testing.assert_array_equal(bits(host(a.ws[:n])), bits(host(b.ws[:n])), err_msg="dp")


# ---------------------------------------------------------------- structure, bit for bit

@pytest.mark.parametrize("path", ["auto", "steps_valu", "steps_mfma", "resident"], indirect=True)
def test_kloop_is_deterministic_and_replay_stable(cfc, path):
    d = CASES["pages"]
    need_path(cfc, d)
    say("kloop determinism", path)
    x = cfc_inputs(**d, seed=5, bias_scale=0.1)
    a, _ = kloop_dev(cfc, x)
    first = {k: host(getattr(a, k)).copy() for k in ("h_hist", "act", "gW_scratch", "gb_scratch", "gW", "gb")}
    b, _ = kloop_dev(cfc, x)            # fresh buffers (step path: a new graph)
    for k, v in first.items():
        np.testing.assert_array_equal(bits(host(getattr(b, k))), bits(v), err_msg=k)
    t = [dev(v) for v in (x.u, x.y, x.h0, x.W, x.bias)]
    for i in range(4):                   # same buffers (step path: replays of one graph)
        # eager work of the program's own between replays: other kernels on the
        # stream, and the outputs overwritten, so a replay that skipped a node shows
        cfc.cfc_fwd_step(t[0][0], t[2], t[3], t[4])
        for k in ("gW", "gb", "gW_scratch", "h_hist"):
            getattr(a, k).fill_(float(i + 1))
        torch.cuda.synchronize()
        cfc.cfc_train_kloop(*t, out=a)
        torch.cuda.synchronize()
        for k, v in first.items():
            np.testing.assert_array_equal(bits(host(getattr(a, k))), bits(v), err_msg="%s, replay %d" % (k, i))


@pytest.mark.parametrize("path", ["auto", "steps_valu", "steps_mfma", "resident"], indirect=True)
@pytest.mark.parametrize("case", ["pages", "ragged_scalar", "sample_tiles", "three_tiles", "no_input",
                                  "long_input64", "two_channel_groups", "three_blocks", "odd_channels"])
def test_kloop_equals_eager_step_calls(cfc, case, path):
    """The K-loop step (persistent path: direct launches; step path: graph
    replay) gives the bits of the eager composition of single-step ABI calls
    with per-step scratch +=."""
    d = CASES[case]
    need_path(cfc, d)
    say("kloop == eager", case, path)
    B, C, n_x, K = d["B"], d["C"], d["n_x"], d["K"]
    x = cfc_inputs(**d, seed=6, bias_scale=0.2)
    g, (u, y, h0, W, bias) = kloop_dev(cfc, x)
    h = [h0]
    acts = []
    for t in range(K):
        ht, at = cfc.cfc_fwd_step(u[t], h[-1], W, bias)
        h.append(ht)
        acts.append(at)
    S = torch.zeros((B, 3, C, n_x + C), device="cuda")
    Sb = torch.zeros((B, 3, C), device="cuda")
    carry = None
    for t in range(K, 0, -1):
        carry, _ = cfc.cfc_bwd_step(u[t - 1], h[t - 1], h[t], y[t - 1], W, acts[t - 1], carry, S, Sb)
    gW = cfc.reduce_axis0(S.view(B, -1))
    gb = cfc.reduce_axis0(Sb.view(B, -1))
    np.testing.assert_array_equal(bits(host(torch.stack(h))), bits(host(g.h_hist)))
    np.testing.assert_array_equal(bits(host(torch.stack(acts))), bits(host(g.act)))
    np.testing.assert_array_equal(bits(host(S)), bits(host(g.gW_scratch)))
    np.testing.assert_array_equal(bits(host(Sb)), bits(host(g.gb_scratch)))
    np.testing.assert_array_equal(bits(host(gW)), bits(host(g.gW).reshape(-1)))
    np.testing.assert_array_equal(bits(host(gb)), bits(host(g.gb).reshape(-1)))


@pytest.mark.parametrize("case", ["tiny", "pages", "ragged_scalar", "three_tiles", "sample_tiles", "no_input",
                                  "long_input64", "long_input48", "two_channel_groups", "three_blocks",
                                  "odd_channels", "long_ragged_k", "single_step", "single_step_max_c",
                                  "one_channel", "mfma_long_k"])
def test_all_kloop_paths_agree_bitwise(cfc, case):
    """Persistent kernel, VALU step kernels, MFMA step kernels and the resident
    MFMA kernel: the same bits."""
    d = CASES[case]
    say("persistent == steps_valu == steps_mfma == resident", case)
    x = cfc_inputs(**d, seed=14, bias_scale=0.25)
    res = {}
    for mode in (cfc.KLOOP_PERSISTENT, cfc.KLOOP_STEPS_VALU, cfc.KLOOP_STEPS_MFMA, cfc.KLOOP_RESIDENT):
        cfc.cfc_set_kloop_mode(mode)
        try:
            if cfc.cfc_kloop_path(d["B"], d["C"], d["n_x"], d["K"]) < 0:
                continue
            out, _ = kloop_dev(cfc, x)
            res[mode] = {k: host(getattr(out, k)).copy()
                         for k in ("h_hist", "act", "gW_scratch", "gb_scratch", "gW", "gb")}
        finally:
            cfc.cfc_set_kloop_mode(cfc.KLOOP_AUTO)
    assert len(res) >= 2
    ref_mode = cfc.KLOOP_STEPS_VALU
    for mode, r in res.items():
        for k in r:
            np.testing.assert_array_equal(bits(r[k]), bits(res[ref_mode][k]), err_msg="%s %d" % (k, mode))


@pytest.mark.parametrize("case", ["wide", "mfma_long_k", "mfma_max"])
def test_resident_kernel_equals_step_kernels_and_finishes_its_waits(cfc, case):
    """The resident MFMA kernel against the MFMA step kernels, bit for bit,
    and its bookkeeping in the workspace afterwards: every workgroup's step
    counter at 2K - 1 (its last report, after backward step 2) and the error
    word, which a wait that gave up would have set, still 0."""
    d = CASES[case]
    B, C, n_x, K = d["B"], d["C"], d["n_x"], d["K"]
    say("resident == steps_mfma", case)
    x = cfc_inputs(**d, seed=21, bias_scale=0.3)
    res = {}
    for mode in (cfc.KLOOP_STEPS_MFMA, cfc.KLOOP_RESIDENT):
        cfc.cfc_set_kloop_mode(mode)
        try:
            if cfc.cfc_kloop_path(B, C, n_x, K) < 0:
                pytest.skip("the resident kernel does not fit this device at this shape")
            out, _ = kloop_dev(cfc, x)
            res[mode] = {k: host(getattr(out, k)).copy()
                         for k in ("h_hist", "act", "gW_scratch", "gb_scratch", "gW", "gb")}
            if mode == cfc.KLOOP_RESIDENT:
                ldf = (n_x + 15) // 16 * 16 + (C + 31) // 32 * 32
                wofs = (2 * K * B * 3 * C + 2 * B * C + 63) // 64 * 64
                nbt = (B + 15) // 16
                fofs = wofs + 3 * C * ldf + C * 64 * 16 + 32 * nbt * ((C + 31) // 32 * 32 + 1024)
                n = nbt * ((C + 15) // 16)
                flags = host(out.ws[fofs:fofs + 32 * (n + 1)]).view(np.int32)[::32]   # one per 128-byte line
                assert flags[n] == 0, "a wait of the resident kernel gave up"
                cfc.cfc_kloop_status(out, B, C, n_x, K)   # reads the same word
                np.testing.assert_array_equal(flags[:n], np.full(n, 2 * K - 1, np.int32))
        finally:
            cfc.cfc_set_kloop_mode(cfc.KLOOP_AUTO)
    for k in res[cfc.KLOOP_STEPS_MFMA]:
        np.testing.assert_array_equal(bits(res[cfc.KLOOP_RESIDENT][k]), bits(res[cfc.KLOOP_STEPS_MFMA][k]),
                                      err_msg=k)


@pytest.mark.parametrize("path", ["auto", "steps_valu", "steps_mfma", "resident"], indirect=True)
@pytest.mark.parametrize("case", ["pages", "three_tiles"])
def test_kloop_equals_its_phases(cfc, case, path):
    """cfc_train_kloop == cfc_kloop_fwd_bwd, then cfc_scratch_fill, then
    reduce_axis0 on each scratch tensor, bit for bit."""
    d = CASES[case]
    need_path(cfc, d)
    say("kloop == phases", case, path)
    B, C, n_x, K = d["B"], d["C"], d["n_x"], d["K"]
    x = cfc_inputs(**d, seed=15, bias_scale=0.2)
    g, t = kloop_dev(cfc, x)
    from recurrent_cell_amd.cfc import KloopBuffers
    ph = KloopBuffers.allocate(B, C, n_x, K, "cuda")
    cfc.cfc_kloop_fwd_bwd(*t, out=ph)
    dp = ph.ws[:K * B * 3 * C].view(K, B, 3 * C)
    cfc.cfc_scratch_fill(dp, t[0], ph.h_hist, ph.gW_scratch, ph.gb_scratch)
    cfc.reduce_axis0(ph.gW_scratch.view(B, -1), ph.gW.view(-1))
    cfc.reduce_axis0(ph.gb_scratch.view(B, -1), ph.gb.view(-1))
    for k in ("h_hist", "act", "gW_scratch", "gb_scratch", "gW", "gb"):
        np.testing.assert_array_equal(bits(host(getattr(ph, k))), bits(host(getattr(g, k))), err_msg=k)


@pytest.mark.parametrize("B,C,n_x,K", [(256, 128, 64, 64), (420, 100, 20, 37), (1400, 64, 0, 4),
                                        (32, 128, 64, 64), (30, 124, 64, 70), (30, 126, 62, 37),
                                        (256, 128, 64, 70), (256, 256, 128, 64), (420, 126, 62, 37)])
def test_scratch_fill_large_batch_equals_slices(cfc, B, C, n_x, K):
    """A sample's scratch depends on that sample alone: on large batches
    (thousands of tiles, ragged tiles, the fma tail, n_x = 0) the
    full-batch call equals calls on slices of 16 samples bit for bit, and
    both match fp64 sums.  Large batches give a workgroup several column
    tiles of its row tile (2 of 3 at B = 256, C = 128; all 6 at the wide
    shape; 3 on scalar staging at 3C = 378), slices one, so the two sides
    also cover both tile walks.  Shapes 4-6: the pages shape, then ragged
    tiles near it on 16-byte staging with two staging passes (K = 70), and
    on scalar staging (3C = 378) with the fma tail; shape 7 has two
    staging passes per tile with several tiles per workgroup."""
    say("scratch fill, large batch against slices", B, C, n_x, K)
    n_in = n_x + C
    dp = normal((K, B, 3 * C), 19, 1)
    u = normal((K, B, n_x), 19, 2)
    h_hist = normal((K + 1, B, C), 19, 3)
    S = torch.full((B, 3, C, n_in), float("nan"), device="cuda")
    Sb = torch.full((B, 3, C), float("nan"), device="cuda")
    cfc.cfc_scratch_fill(dev(dp), dev(u), dev(h_hist), S, Sb)
    S_ref = torch.full_like(S, float("nan"))
    Sb_ref = torch.full_like(Sb, float("nan"))
    for b0 in range(0, B, 16):
        b1 = min(B, b0 + 16)
        cfc.cfc_scratch_fill(dev(dp[:, b0:b1]), dev(u[:, b0:b1]), dev(h_hist[:, b0:b1]), S_ref[b0:b1], Sb_ref[b0:b1])
    np.testing.assert_array_equal(bits(host(S)), bits(host(S_ref)))
    np.testing.assert_array_equal(bits(host(Sb)), bits(host(Sb_ref)))
    z = np.concatenate([u, h_hist[:-1]], axis=2).astype(np.float64)              # [K,B,n_in]
    A = np.ascontiguousarray(dp.astype(np.float64).transpose(1, 2, 0))          # [B,3C,K]
    Z = np.ascontiguousarray(z.transpose(1, 0, 2))                              # [B,K,n_in]
    ref = np.matmul(A, Z).reshape(B, 3, C, -1)
    mass = np.matmul(np.abs(A), np.abs(Z)).reshape(B, 3, C, -1)
    assert_ok(check_grad("S", host(S), ref, mass))


@pytest.mark.parametrize("case", ["tiny", "pages", "ragged_scalar", "three_tiles", "no_input"])
def test_scratch_fill_matches_its_definition(cfc, case):
    """S[b,r,k] = sum_t dp[t,b,r] z_t[b,k], Sb[b,r] = sum_t dp[t,b,r] on
    arbitrary fp32 inputs, against fp64 sums (numpy matmul)."""
    d = CASES[case]
    say("scratch fill", case)
    B, C, n_x, K = d["B"], d["C"], d["n_x"], d["K"]
    x = cfc_inputs(**d, seed=16)
    dp = normal((K, B, 3 * C), 16, 1)
    h_hist = normal((K + 1, B, C), 16, 2)
    S = torch.full((B, 3, C, n_x + C), float("nan"), device="cuda")
    Sb = torch.full((B, 3, C), float("nan"), device="cuda")
    cfc.cfc_scratch_fill(dev(dp), dev(x.u), dev(h_hist), S, Sb)
    z = np.concatenate([x.u, h_hist[:-1]], axis=2).astype(np.float64)          # [K,B,n_in]
    A = np.ascontiguousarray(dp.astype(np.float64).transpose(1, 2, 0))          # [B,3C,K]
    Z = np.ascontiguousarray(z.transpose(1, 0, 2))                              # [B,K,n_in]
    ref = np.matmul(A, Z).reshape(B, 3, C, -1)
    mass = np.matmul(np.abs(A), np.abs(Z)).reshape(B, 3, C, -1)
    assert_ok(check_grad("S", host(S), ref, mass))
    refb = dp.astype(np.float64).sum(0).reshape(B, 3, C)
    assert_ok(check_grad("Sb", host(Sb), refb, np.abs(dp.astype(np.float64)).sum(0).reshape(B, 3, C)))


@pytest.mark.parametrize("entry", ["train_kloop", "noalloc"])
def test_persistent_step_replays_under_graph_capture(cfc, entry):
    """On a stream under capture the persistent path launches the input
    projection on its own (a replayed graph would repeat the number that the
    fused launch's projection flags are matched against).  One step captured
    with torch's graph API, replayed on three input sets with eager copies
    and synchronizations between the replays: every replay gives the bits of
    an eager step on the same inputs."""
    d = CASES["pages"]
    B, C, n_x, K = d["B"], d["C"], d["n_x"], d["K"]
    say("persistent step under graph capture", entry)
    keys = ("h_hist", "act", "gW_scratch", "gb_scratch", "gW", "gb")
    xs = [cfc_inputs(**d, seed=40 + i, bias_scale=0.2) for i in range(3)]
    ref = []
    for x in xs:
        out, _ = kloop_dev(cfc, x)
        ref.append({k: host(getattr(out, k)).copy() for k in keys})
    st = [dev(a) for a in (xs[0].u, xs[0].y, xs[0].h0, xs[0].W, xs[0].bias)]
    buf = cfc.KloopBuffers.allocate(B, C, n_x, K, "cuda")

    def step():
        if entry == "noalloc":
            cfc.cfc_train_kloop_noalloc(*st, out=buf)
        else:
            cfc.cfc_train_kloop(*st, out=buf)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()   # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in (1, 0, 2):
        for a, v in zip(st, (xs[i].u, xs[i].y, xs[i].h0, xs[i].W, xs[i].bias)):
            a.copy_(torch.from_numpy(np.ascontiguousarray(v)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in keys:
            np.testing.assert_array_equal(bits(host(getattr(buf, k))), bits(ref[i][k]), err_msg="%s %d" % (k, i))


def test_persistent_mode_refuses_shapes_it_cannot_hold(cfc):
    d = CASES["wide"]
    say("persistent refusal", d)
    cfc.cfc_set_kloop_mode(cfc.KLOOP_PERSISTENT)
    try:
        x = cfc_inputs(**dict(d, B=2, K=2), seed=1)
        with pytest.raises(cfc.CfcError):
            kloop_dev(cfc, x)
    finally:
        cfc.cfc_set_kloop_mode(cfc.KLOOP_AUTO)


@pytest.mark.parametrize("case", ["pages", "sample_tiles"])
def test_batched_rows_equal_single_sample_runs(cfc, case):
    d = CASES[case]
    say("batched row == B=1 run", case)
    x = cfc_inputs(**d, seed=7, bias_scale=0.2)
    full, _ = kloop_dev(cfc, x)
    fh, fa, fS, fSb = (host(full.h_hist), host(full.act), host(full.gW_scratch), host(full.gb_scratch))
    for b in sorted({0, 1, d["B"] // 2, d["B"] - 1}):
        xb = cfc_inputs(**d, seed=7, bias_scale=0.2)
        xb.u, xb.y, xb.h0 = x.u[:, b:b + 1].copy(), x.y[:, b:b + 1].copy(), x.h0[b:b + 1].copy()
        one, _ = kloop_dev(cfc, xb)
        np.testing.assert_array_equal(bits(host(one.h_hist)[:, 0]), bits(fh[:, b]))
        np.testing.assert_array_equal(bits(host(one.act)[:, :, 0]), bits(fa[:, :, b]))
        np.testing.assert_array_equal(bits(host(one.gW_scratch)[0]), bits(fS[b]))
        np.testing.assert_array_equal(bits(host(one.gb_scratch)[0]), bits(fSb[b]))
        np.testing.assert_array_equal(bits(host(one.gW)), bits(fS[b]))   # B = 1: exact copy


def test_scratch_clears_between_steps(cfc):
    d = CASES["pages"]
    say("scratch clears between steps")
    xa = cfc_inputs(**d, seed=8, bias_scale=0.1)
    xb = cfc_inputs(**d, seed=9, bias_scale=0.1)
    t = [dev(v) for v in (xa.u, xa.y, xa.h0, xa.W, xa.bias)]
    out = cfc.cfc_train_kloop(*t)
    torch.cuda.synchronize()
    for dst, src in zip(t, (xb.u, xb.y, xb.h0, xb.W, xb.bias)):
        dst.copy_(torch.from_numpy(src))
    cfc.cfc_train_kloop(*t, out=out)           # replay on step B's data
    ref, _ = kloop_dev(cfc, xb)                # step B alone, fresh buffers
    for k in ("gW_scratch", "gb_scratch", "gW", "gb", "h_hist"):
        np.testing.assert_array_equal(bits(host(getattr(out, k))), bits(host(getattr(ref, k))), err_msg=k)


def test_final_gradients_are_overwritten(cfc):
    d = CASES["tiny"]
    say("overwrite semantics")
    x = cfc_inputs(**d, seed=10)
    from recurrent_cell_amd.cfc import KloopBuffers
    out = KloopBuffers.allocate(d["B"], d["C"], d["n_x"], d["K"], "cuda")
    for tns in (out.gW, out.gb, out.gW_scratch, out.gb_scratch, out.h_hist, out.act, out.ws):
        tns.fill_(float("nan"))
    kloop_dev(cfc, x, out=out)
    ref, _ = kloop_dev(cfc, x)
    for k in ("gW", "gb", "gW_scratch", "gb_scratch", "h_hist", "act"):
        v = host(getattr(out, k))
        assert np.isfinite(v).all(), k
        np.testing.assert_array_equal(bits(v), bits(host(getattr(ref, k))))


def test_exact_special_cases(cfc):
    """W_f = 0, b_f = 0 gives gate = 0.5 exactly; W_g = W_h, b_g = b_h gives
    g == hh bit for bit and exactly zero f-head gradients."""
    d = CASES["pages"]
    say("special cases")
    x = cfc_inputs(**d, seed=11, bias_scale=0.3)
    x.W[0] = 0.0
    x.bias[0] = 0.0
    out, _ = kloop_dev(cfc, x)
    assert np.all(host(out.act)[:, 0] == 0.5)
    x = cfc_inputs(**d, seed=12, bias_scale=0.3)
    x.W[2] = x.W[1]
    x.bias[2] = x.bias[1]
    out, _ = kloop_dev(cfc, x)
    act = host(out.act)
    np.testing.assert_array_equal(bits(act[:, 1]), bits(act[:, 2]))
    assert np.all(host(out.gW)[0] == 0.0) and np.all(host(out.gb)[0] == 0.0)
    h = host(out.h_hist)[1:]
    assert np.all(np.abs(h) <= 1.0)
    gate = act[:, 0]
    assert np.all(gate > 0) and np.all(gate < 1)


@pytest.mark.parametrize("optimizer", ["sgd", "adamw"])
def test_training_loss_falls_at_batch_32(cfc, optimizer):
    """Training on the GPU's gradients at the pages shape (B = 32), the
    analogue of the pages' batch-32 training gate ("K-loop Parallelization",
    Tests + Acceptance: the first test that exercises the cross-batch
    reduction): a constant-direction target (+0.5 on even channels, -0.5 on
    odd ones, every step and sample), 50 steps of cfc_train_kloop, each
    followed by an update of W and the bias -- plain SGD (lr 1e-5) on the
    harness side, or cfc_adamw_step (lr 1e-2, no decay).  With SGD the loss
    (from h_hist and y) falls at every step; with either, the 50th loss is
    below a tenth of the first (the fp32 oracle run the same way goes from
    39,494 to 2,822 with SGD and to 143 with AdamW)."""
    d = CASES["pages"]
    say("training descent", optimizer, d)
    x = cfc_inputs(**d, seed=5)
    C = d["C"]
    tgt = np.where(np.arange(C) % 2 == 0, 0.5, -0.5).astype(np.float32)
    x.y = np.ascontiguousarray(np.broadcast_to(tgt, x.y.shape))
    t = [dev(a) for a in (x.u, x.y, x.h0, x.W, x.bias)]
    W, bias = t[3], t[4]
    ms = [torch.zeros_like(W), torch.zeros_like(bias)]
    vs = [torch.zeros_like(W), torch.zeros_like(bias)]
    out = None
    losses = []
    for step in range(1, 51):
        out = cfc.cfc_train_kloop(*t, out=out)
        losses.append(float(0.5 * ((out.h_hist[1:].double() - t[1].double()) ** 2).sum()))
        if optimizer == "sgd":
            W.sub_(1e-5 * out.gW)
            bias.sub_(1e-5 * out.gb)
        else:
            cfc.cfc_adamw_step([W, bias], [out.gW, out.gb], ms, vs, 1e-2, 0.9, 0.999, 1e-8, 0.0, step)
    torch.cuda.synchronize()
    losses = np.array(losses)
    say("  loss", "%.1f -> %.1f" % (losses[0], losses[-1]))
    assert np.all(np.isfinite(losses))
    if optimizer == "sgd":
        assert np.all(np.diff(losses) < 0), losses
    assert losses[-1] < 0.1 * losses[0], losses


def test_degenerate_sizes(cfc):
    say("K = 0 and B = 0")
    from recurrent_cell_amd.cfc import KloopBuffers
    x = cfc_inputs(B=3, C=16, n_x=4, K=0, seed=13)
    out = KloopBuffers.allocate(3, 16, 4, 0, "cuda")
    out.gW.fill_(float("nan"))
    out.gb.fill_(float("nan"))
    kloop_dev(cfc, x, out=out)
    np.testing.assert_array_equal(host(out.h_hist)[0], x.h0)
    assert np.all(host(out.gW) == 0) and np.all(host(out.gb) == 0)
    x = cfc_inputs(B=0, C=16, n_x=4, K=3, seed=13)
    out = KloopBuffers.allocate(0, 16, 4, 3, "cuda")
    out.gW.fill_(float("nan"))
    kloop_dev(cfc, x, out=out)
    assert np.all(host(out.gW) == 0)


# ---------------------------------------------------------------- reduce_axis0

SMALL_SHAPES = [(B, N) for B in (1, 2, 3, 31, 32, 33, 128, 256, 300) for N in (1, 3, 4, 5, 255, 1000, 4097)]


@pytest.mark.parametrize("B,N", SMALL_SHAPES)
def test_reduce_small_and_ragged(cfc, oracle_mod, B, N):
    say("reduce", B, N)
    x = reduce_rows(B, N, seed=B * 7 + N)
    xd = dev(x)
    out = torch.full((N,), float("nan"), device="cuda")
    cfc.reduce_axis0(xd, out)
    got = host(out)
    ref = oracle_mod.reduce_axis0_f64(x)
    assert_ok(check_reduce("reduce", got, ref, np.abs(x.astype(np.float64)).sum(0), B))
    again = host(cfc.reduce_axis0(xd))
    np.testing.assert_array_equal(bits(again), bits(got))


def test_reduce_integer_rows_exact(cfc):
    for B, N in ((256, 70001), (32, 4096), (3, 7)):
        say("reduce integer exact", B, N)
        x = small_int_rows(B, N, seed=B)
        got = host(cfc.reduce_axis0(dev(x)))
        np.testing.assert_array_equal(got, x.astype(np.int64).sum(0).astype(np.float32))
    ones = torch.ones((256, 1000), device="cuda")
    assert np.all(host(cfc.reduce_axis0(ones)) == 256.0)


def test_reduce_degenerate_and_unaligned(cfc):
    say("reduce degenerate / unaligned")
    x = reduce_rows(1, 999, seed=1)
    np.testing.assert_array_equal(bits(host(cfc.reduce_axis0(dev(x)))), bits(x[0]))
    out = torch.full((8,), float("nan"), device="cuda")
    cfc.reduce_axis0(torch.empty((0, 8), device="cuda"), out)
    assert np.all(host(out) == 0)
    # unaligned base (scalar path) gives the same bits as the aligned copy (vector path)
    x = reduce_rows(40, 1024, seed=2)
    flat = torch.zeros(40 * 1024 + 1, device="cuda")
    flat[1:] = dev(x).view(-1)
    mis = flat[1:].view(40, 1024)
    assert mis.data_ptr() % 16 != 0
    np.testing.assert_array_equal(bits(host(cfc.reduce_axis0(mis))), bits(host(cfc.reduce_axis0(dev(x)))))


FULL_B = (32, 128, 256)
FULL_N = (4096, 73728, 1048576, 8388608)


@pytest.mark.parametrize("B", FULL_B)
@pytest.mark.parametrize("N", FULL_N)
def test_reduce_full_size_sampled(cfc, oracle_mod, B, N):
    """Full-size shapes, as the benchmark launches them.  Inputs are N(0,1)
    from torch's seeded device generator.  Up to N = 2^20 every column is
    summed by the oracle from the host copy of the input; at N = 8M, 4096
    sampled columns (plus the first and last 64)."""
    say("reduce full size", B, N)
    gen = torch.Generator(device="cuda").manual_seed(1000 + B)
    x = torch.randn((B, N), device="cuda", generator=gen)
    out = torch.full((N,), float("nan"), device="cuda")
    cfc.reduce_axis0(x, out)
    if N <= (1 << 20):
        idx = np.arange(N)
        cols = host(x)
    else:
        rng = np.random.default_rng(N + B)
        idx = np.unique(np.concatenate([rng.integers(0, N, 4096), np.arange(64), np.arange(N - 64, N)]))
        cols = host(x[:, torch.from_numpy(idx).cuda()])
    ref = oracle_mod.reduce_axis0_f64(np.ascontiguousarray(cols))
    got = host(out)
    assert np.isfinite(got).all()
    assert_ok(check_reduce("reduce", got[idx], ref, np.abs(cols.astype(np.float64)).sum(0), B))
    again = torch.empty_like(out)
    cfc.reduce_axis0(x, again)
    assert torch.equal(again.view(torch.int32), out.view(torch.int32))
    del x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B", [32, 128])
def test_reduce_large_grid_ragged_and_column_bits(cfc, oracle_mod, B):
    """The largest grids take two column groups per lane.  A ragged tail
    (the last workgroup partly past N) is checked against the oracle, and
    every column's bits equal those of the same column reduced in a small
    launch (one group per lane): the bits depend on B alone."""
    N = 4 * (8388608 // 4 + 4 * 64 * 2 + 3)   # multiple of 4, not of a workgroup's columns
    say("reduce large grid", B, N)
    gen = torch.Generator(device="cuda").manual_seed(77 + B)
    x = torch.randn((B, N), device="cuda", generator=gen)
    out = torch.full((N,), float("nan"), device="cuda")
    cfc.reduce_axis0(x, out)
    idx = np.unique(np.concatenate([np.arange(N - 3000, N), np.random.default_rng(B).integers(0, N, 2048)]))
    cols = host(x[:, torch.from_numpy(idx).cuda()])
    ref = oracle_mod.reduce_axis0_f64(np.ascontiguousarray(cols))
    got = host(out)
    assert np.isfinite(got).all()
    assert_ok(check_reduce("reduce", got[idx], ref, np.abs(cols.astype(np.float64)).sum(0), B))
    for lo, hi in ((0, 4096), (N - 4096, N)):
        part = x[:, lo:hi].contiguous()
        small = torch.full((hi - lo,), float("nan"), device="cuda")
        cfc.reduce_axis0(part, small)
        assert torch.equal(small.view(torch.int32), out[lo:hi].view(torch.int32))
    del x
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- AdamW after the reducer

def f32(x):
    return float(np.float32(x))


@pytest.mark.parametrize("sizes,step,hp", [
    ((73728, 384), 1, (1e-3, 0.9, 0.999, 1e-8, 0.01)),           # W and bias of the 128-channel cell
    ((1, 3, 1000, 4097), 7, (3e-3, 0.8, 0.95, 1e-6, 0.1)),      # four ragged segments
    ((0, 5, 0), 1000, (1e-2, 0.9, 0.999, 1e-8, 0.0)),           # empty segments, late step, no decay
    ((2_000_003,), 3, (1e-4, 0.5, 0.5, 1e-3, 0.5)),             # grid-stride loop, odd length
])
def test_adamw_matches_oracle(cfc, oracle_mod, sizes, step, hp):
    say("adamw parity", sizes, step, hp)
    p, g, m, v = adamw_inputs(sizes, seed=31)
    tp, tg, tm, tv = ([dev(a) for a in xs] for xs in (p, g, m, v))
    lr, b1, b2, eps, wd = (f32(h) for h in hp)
    cfc.cfc_adamw_step(tp, tg, tm, tv, lr, b1, b2, eps, wd, step)
    for i in range(len(sizes)):
        ref = oracle_mod.adamw_step(p[i], g[i], m[i], v[i], lr, b1, b2, eps, wd, step)
        for rep in check_adamw(host(tp[i]), host(tm[i]), host(tv[i]), ref, p[i], m[i], g[i], lr, b1, b2, eps,
                               step):
            assert_ok(rep)


def test_adamw_reads_only_post_reducer_gradients(cfc):
    """The final gradient buffers hold the previous step's values until the
    reducer of this step overwrites them.  AdamW enqueued right after
    cfc_train_kloop on the same stream (no synchronisation) must apply this
    step's reduced gradients: the result equals, bit for bit, AdamW applied
    after a synchronisation to a snapshot of those gradients, and differs from
    AdamW on the previous step's gradients."""
    d = CASES["pages"]
    say("adamw after the reducer", d)
    xa = cfc_inputs(**d, seed=41)
    xb = cfc_inputs(**d, seed=42)
    out = cfc.KloopBuffers.allocate(d["B"], d["C"], d["n_x"], d["K"], "cuda")
    kloop_dev(cfc, xa, out=out)
    torch.cuda.synchronize()
    stale_gW, stale_gb = out.gW.clone(), out.gb.clone()
    W0, b0 = dev(xb.W), dev(xb.bias)
    state = lambda: ([W0.clone(), b0.clone()], [torch.zeros_like(W0), torch.zeros_like(b0)],  # noqa: E731
                     [torch.zeros_like(W0), torch.zeros_like(b0)])
    hp = (1e-3, 0.9, 0.999, 1e-8, 0.01)
    # the fused order: K-loop then AdamW on the same stream, nothing in between
    pa, ma, va = state()
    t = [dev(a) for a in (xb.u, xb.y, xb.h0)]
    cfc.cfc_train_kloop(t[0], t[1], t[2], W0, b0, out=out)
    cfc.cfc_adamw_step(pa, [out.gW, out.gb], ma, va, *hp, 2)
    torch.cuda.synchronize()
    # the same update from a snapshot taken after synchronising
    gW, gb = out.gW.clone(), out.gb.clone()
    pb, mb, vb = state()
    cfc.cfc_adamw_step(pb, [gW, gb], mb, vb, *hp, 2)
    for x, y in zip(pa + ma + va, pb + mb + vb):
        np.testing.assert_array_equal(bits(host(x)), bits(host(y)))
    # and not the stale gradients
    pc, mc, vc = state()
    cfc.cfc_adamw_step(pc, [stale_gW, stale_gb], mc, vc, *hp, 2)
    assert not np.array_equal(host(pa[0]), host(pc[0]))
    assert not torch.equal(gW, stale_gW)


# ---------------------------------------------------------------- GEMM-form weight gradient

@pytest.mark.parametrize("case", ["tiny", "pages", "wide", "ragged_scalar", "no_input", "odd_channels",
                                  "three_blocks", "long_input48"])
def test_kloop_gemm_matches_oracle(cfc, oracle_mod, case):
    """cfc_train_kloop_gemm (no scratch): activations as the K-loop's, gW and
    gb against the oracle at the gradient tolerance."""
    d = CASES[case]
    if cfc.cfc_kloop_path(d["B"], d["C"], d["n_x"], d["K"]) < 0:
        pytest.skip("no K-loop path takes this shape")
    say("kloop gemm-form parity", case, d)
    x = cfc_inputs(**d, seed=1, bias_scale=0.2)
    t = [dev(a) for a in (x.u, x.y, x.h0, x.W, x.bias)]
    out = cfc.cfc_train_kloop_gemm(*t)
    r = oracle_mod.train(x.u, x.y, x.h0, x.W, x.bias, "f64", want_dp=True)
    m = grad_mass(x.u, r["h_hist"], r["dp"])
    reps = [check_act("h_hist", host(out.h_hist), r["h_hist"]), check_act("act", host(out.act), r["act"]),
            check_grad("gW", host(out.gW), r["gW"], m["gW"]), check_grad("gb", host(out.gb), r["gb"], m["gb"])]
    for rep in reps:
        say("  ", describe(rep))
    for rep in reps:
        assert_ok(rep)


def test_kloop_gemm_composes_and_is_deterministic(cfc):
    """cfc_train_kloop_gemm == cfc_kloop_fwd_bwd then cfc_weight_grad_gemm on
    its dp, bit for bit, and repeated calls give the same bits; the
    activations equal cfc_train_kloop's."""
    d = CASES["pages"]
    say("kloop gemm-form composition", d)
    x = cfc_inputs(**d, seed=2, bias_scale=0.2)
    t = [dev(a) for a in (x.u, x.y, x.h0, x.W, x.bias)]
    a = cfc.cfc_train_kloop_gemm(*t)
    gW1, gb1 = host(a.gW).copy(), host(a.gb).copy()
    a.gW.fill_(float("nan"))
    cfc.cfc_train_kloop_gemm(*t, out=a)
    np.testing.assert_array_equal(bits(host(a.gW)), bits(gW1))
    np.testing.assert_array_equal(bits(host(a.gb)), bits(gb1))
    b = cfc.KloopBuffers.allocate(d["B"], d["C"], d["n_x"], d["K"], "cuda")
    cfc.cfc_kloop_fwd_bwd(*t, out=b)
    K, B, C = d["K"], d["B"], d["C"]
    dp = b.ws[:K * B * 3 * C].view(K, B, 3 * C)
    gW, gb = cfc.cfc_weight_grad_gemm(dp, t[0], b.h_hist)
    np.testing.assert_array_equal(bits(host(gW)), bits(gW1))
    np.testing.assert_array_equal(bits(host(gb)), bits(gb1))
    ref = cfc.cfc_train_kloop(*t)
    np.testing.assert_array_equal(bits(host(ref.h_hist)), bits(host(a.h_hist)))
    np.testing.assert_array_equal(bits(host(ref.act)), bits(host(a.act)))


def test_kloop_at_the_maximum_size(cfc, oracle_mod):
    """C = CFC_MAX_C, n_in = CFC_MAX_N_IN: the scratch K-loop and the
    GEMM-form step against the fp64 oracle, no worse than 4x the oracle's own
    fp32 evaluation (the stated tolerances are out of reach of fp32 sums of
    8,192 terms; see tests/tolerances.py)."""
    d = MAX_SIZE
    say("kloop at the maximum size", d)
    x = cfc_inputs(**d, seed=1, bias_scale=0.2)
    t = [dev(a) for a in (x.u, x.y, x.h0, x.W, x.bias)]
    out = cfc.cfc_train_kloop(*t)
    gem = cfc.cfc_train_kloop_gemm(*t)
    r = oracle_mod.train(x.u, x.y, x.h0, x.W, x.bias, "f64", want_dp=True)
    r32 = oracle_mod.train(x.u, x.y, x.h0, x.W, x.bias, "f32", want_dp=True)
    m = grad_mass(x.u, r["h_hist"], r["dp"])
    act_b = {k: 1e-6 + 1e-5 * np.abs(r[k]) for k in ("h_hist", "act")}
    grad_b = {k: 1e-6 + 1e-4 * np.abs(r[k]) + 16 * 2.0 ** -24 * m[k] for k in ("S", "Sb", "gW", "gb")}
    reps = [check_vs_fp32(k, host(getattr(out, k)), r[k], r32[k], act_b[k]) for k in ("h_hist", "act")]
    reps += [check_vs_fp32(k, host(getattr(out, a)), r[k], r32[k], grad_b[k])
             for k, a in (("S", "gW_scratch"), ("Sb", "gb_scratch"), ("gW", "gW"), ("gb", "gb"))]
    reps += [check_vs_fp32("gemm " + k, host(getattr(gem, k)), r[k], r32[k], grad_b[k]) for k in ("gW", "gb")]
    for rep in reps:
        say("  ", rep["name"], "worst", "%.3g" % rep["worst_ratio"], "fp32 oracle", "%.3g" % rep["worst_fp32"],
            "normwise", "%.3g" % rep["normwise"], "fp32", "%.3g" % rep["normwise_fp32"])
    for rep in reps:
        assert_ok(rep)


def test_fma_probe_runs_bounded_chains(cfc):
    """The FMA-rate probe: every chain x <- fma(x, 0.999, 0.001) stays in
    [0, 8] from its start and tends to 1, so each lane's sum of 8 chains lies
    in (0, 64) and, after many links, near 8."""
    out = torch.full((4 * 512,), float("nan"), device="cuda")
    cfc.cfc_probe_fma(out, 4, 512, 4096)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.isfinite(o).all()
    assert np.abs(o - 8.0).max() < 1e-2
