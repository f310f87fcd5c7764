"""Benchmark: CfC K-loop training steps per second on one MI355X.

A step is one cfc_train_kloop call: forward t = 1..K, BPTT t = K..1, the
per-sample scratch and reduce_axis0 of both scratch tensors (on the
persistent path two launches -- the persistent K-loop, whose launch also
forms the input projection and the scratch (extra workgroups, for B <= 128
and 16-byte shapes that fit the CUs; three or four launches otherwise), and
the reduction; on the step path one graph replay of 2K + 2 launches), on
the pages-shaped configuration B=32, C=128, n_x=64 (n_in=192), K=64, fp32,
inputs seeded and already resident in HBM.  Prints ONE JSON line.

Also measured in the same run:
  * the duration of each kernel of the step, live: one HIP event pair
    around back-to-back eager launches of each phase on the launch stream,
    pre-loaded by a spin kernel so the events time the GPU, not the host
    (pair_median_us: the median of per-launch event pairs, which also hold
    the event records' own cost);
    the kernel with the largest share of the step gives the roofline object;
  * the same step on the 2K-launch step-kernel path, for contrast;
  * graph-node latency (a graph of dependent one-element kernels), which
    gives the step's latency roofline;
  * the other two K-loop configurations (tiny B=4 C=16 n_x=8 K=4, and wide
    B=256 C=256 n_x=128 K=64) with their own rooflines, under "workloads";
  * reduce_axis0 GB/s on the standalone [B, N] shapes;
  * the batched MLP step and AdamW;
  * the CPU oracle on the host (cpu_baseline): fp64 and fp32 on one thread
    and fp32 on every usable host thread, for each K-loop configuration (the
    wide one on a bounded sample of its samples), and the reduction's column
    sums on one and on every thread.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CfC K=64 fwd+bwd train-steps/s at B=32,C=128; reduce_axis0 GB/s vs HBM peak"
HBM_PEAK = 8.0e12          # B/s, MI355X HBM3E
FP32_PEAK = 157.3e12       # flop/s, MI355X fp32 vector (256 CUs x 2.4 GHz x 256 flop/clk)


def step_bytes_flops(B, C, n_x, K):
    """Algorithmic bytes and flops of one K-loop training step."""
    n_in = n_x + C
    f = 4
    bytes_min = f * (K * B * n_x + K * B * C + B * C + 3 * C * n_in + 3 * C      # u, y, h0, W, bias
                     + (K + 1) * B * C + K * 3 * B * C                           # h_hist, act written
                     + K * B * C + K * 3 * B * C                                 # re-read in backward
                     + 2 * (3 * B * C * n_in + 3 * B * C)                        # scratch once + reduce read
                     + 3 * C * n_in + 3 * C)                                     # gW, gb
    flops = K * B * 3 * C * n_in * 2 * 3                                        # fwd, W^T dp, scratch
    return bytes_min, flops


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "kloop_persist_pages_hbm_traffic.md")
VALU_SUMMARY = os.path.join(ROOT, "profiles", "kloop_persist_pages_valu.md")
KERNEL_SOURCES = [os.path.join(ROOT, "recurrent_cell_amd", "csrc", f)
                  for f in ("cfc_kernels.hip", "cfc_kernels.h", "cfc_math.h")]


def kernel_source_digest():
    """sha256 of the persistent kernel's source: in each of KERNEL_SOURCES the
    text between "[persistent kernel source: begin]" and "... end]" markers
    (the whole file where it has none), in file order."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        text = open(f, "rb").read()
        parts = text.split(b"// [persistent kernel source: begin]\n")
        if len(parts) == 1:
            h.update(text)
            continue
        for p in parts[1:]:
            h.update(p.split(b"// [persistent kernel source: end]\n")[0])
    return h.hexdigest()


def profile_value(path, key):
    """A value recorded in a committed rocprofv3 counter summary ("key: value"
    under the kernel sources' sha256), or None if the summary is missing or
    the persistent kernel's sources changed since the counters were taken."""
    import re
    try:
        text = open(path).read()
        digest = kernel_source_digest()
    except OSError:
        return None
    m_hash = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"%s:\s*([0-9.]+)" % re.escape(key), text)
    if not m_hash or not m_val or m_hash.group(1) != digest:
        return None
    return float(m_val.group(1))


def measured_traffic():
    """HBM bytes per launch of the persistent kernel (FETCH_SIZE + WRITE_SIZE,
    calibrated), or None (see profile_value)."""
    v = profile_value(TRAFFIC_SUMMARY, "traffic_bytes_per_launch")
    return None if v is None else int(v)


def measured_valu_busy():
    """Fraction of time the VALU of the persistent kernel's CUs is busy
    (SQ_ACTIVE_INST_VALU / SQ_BUSY_CU_CYCLES), or None (see profile_value)."""
    return profile_value(VALU_SUMMARY, "valu_busy_fraction")


# The persistent launch forms the input projection itself (extra workgroups)
# up to this batch; above it the projection is a launch of its own.
PERSIST_FUSE_MAX_B = 128


def recurrence_flops(B, C, K):
    """Persistent kernel: W_h h_{t-1} forward and W_h^T dp (carry) backward."""
    return K * B * 3 * C * C * 2 * 2


def projection_flops(B, C, n_x, K):
    return K * B * 3 * C * n_x * 2


def fill_bytes(B, C, n_x, K):
    n_in = n_x + C
    return 4 * (K * B * 3 * C + K * B * n_x + K * B * C + B * 3 * C * n_in + B * 3 * C)


def fwd_launch_bytes(B, C, n_x):
    n_in = n_x + C
    return 4 * (B * n_x + B * C + 3 * C * n_in + 3 * C + B * C + 3 * B * C)


def bwd_launch_bytes(B, C, n_x):
    """One backward step launch of the K-loop: inputs read once, dp and carry written."""
    n_in = n_x + C
    return 4 * (6 * B * C + B * C + 3 * C * n_in + 3 * B * C + B * C)


class LaunchTimer:
    """Average GPU duration of one launch of fn: one event pair around n
    back-to-back launches, with the stream first kept busy by a spin kernel
    long enough for the host to enqueue them all (so the GPU never waits on
    the host and the pair times only the launches).  Per-launch event pairs
    are taken too, for context: each such pair also holds the event records'
    own cost (about 2 us on this GPU), so their figures run above the kernel
    durations a kernel trace reports, while the back-to-back mean agrees with
    them."""

    def __init__(self, torch):
        self.torch = torch
        try:
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            torch.cuda._sleep(1_000_000)
            b.record()
            torch.cuda.synchronize()
            self.cycles_per_s = 1_000_000 / max(a.elapsed_time(b) * 1e-3, 1e-6)
        except (AttributeError, RuntimeError):
            self.cycles_per_s = None   # no spin kernel: the pairs may include host time

    def _preload(self, seconds):
        if self.cycles_per_s is not None:
            self.torch.cuda._sleep(int(seconds * self.cycles_per_s) + 1000)

    def __call__(self, fn, n, host_us=80.0):
        torch = self.torch
        fn()
        torch.cuda.synchronize()
        ev = mean_s = None
        for _ in range(4):
            # back to back: the launch duration
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            self._preload(n * host_us * 1e-6)
            h0 = time.perf_counter()
            s.record()
            for _ in range(n):
                fn()
            e.record()
            host_s = time.perf_counter() - h0
            # per-launch pairs (context)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
            self._preload(n * host_us * 1e-6)
            for a, b in ev:
                a.record()
                fn()
                b.record()
            torch.cuda.synchronize()
            mean_s = s.elapsed_time(e) * 1e-3 / n
            if self.cycles_per_s is None or host_s < 0.5 * n * host_us * 1e-6:
                break
            host_us *= 3   # the enqueue took longer than the spin covered: spin longer
        ms = np.array([a.elapsed_time(b) for a, b in ev])
        gaps = np.array([ev[i][1].elapsed_time(ev[i + 1][0]) for i in range(n - 1)]) if n > 1 else np.zeros(1)
        return dict(mean_s=mean_s, pair_mean_s=float(ms.mean()) * 1e-3, pair_median_s=float(np.median(ms)) * 1e-3,
                    gap_median_us=float(np.median(gaps)) * 1e3, n=n)


def graph_node_latency(torch, n_nodes=130, reps=50):
    """Seconds per node of a graph of n_nodes dependent one-element kernels."""
    x = torch.zeros(1, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            x.add_(1.0)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(n_nodes):
            x.add_(1.0)
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / (reps * n_nodes)


def copy_peak(torch, mib=2048, reps=10):
    """Measured HBM rate of a plain fp32 device copy (mib MiB read + mib MiB
    written per copy), median over reps, in B/s."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty(n, device="cuda")
    dst.copy_(src)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n * 4 / float(np.median(ts))


def fma_rate(torch, cfc, blocks, threads=512, iters=8192, reps=5):
    """Measured non-packed fp32 FMA rate (flop/s) of `blocks` workgroups of
    `threads` lanes, one workgroup per CU (the FMA-chain probe of
    include/probe.h), median over reps launches."""
    out = torch.empty(blocks * threads, device="cuda")
    cfc.cfc_probe_fma(out, blocks, threads, 16)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        cfc.cfc_probe_fma(out, blocks, threads, iters)
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    if not bool(torch.isfinite(out).all()):
        raise RuntimeError("FMA probe produced non-finite values")
    return 2.0 * 64 * iters * blocks * threads / float(np.median(ts))


def host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = None
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "model": model}


def deterministic_runs(torch, cfc, t, n=3):
    """True iff n K-loop calls into fresh buffers give the same gradient bits."""
    ref = None
    for _ in range(n):
        o = cfc.cfc_train_kloop(*t)
        torch.cuda.synchronize()
        bits = (o.gW.view(torch.int32).cpu(), o.gb.view(torch.int32).cpu())
        if ref is None:
            ref = bits
        elif not (torch.equal(ref[0], bits[0]) and torch.equal(ref[1], bits[1])):
            return False
    return True


def time_calls(torch, fn, steps, warmup, trials):
    """Median over trials of the ms per call of fn, calls back to back."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    res = []
    for _ in range(trials):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) / steps)
    return float(np.median(res)), res


def time_steps(torch, cfc, t, out, steps, warmup, trials):
    return time_calls(torch, lambda: cfc.cfc_train_kloop(*t, out=out), steps, warmup, trials)


def bench_reduce(torch, cfc, timer, shapes):
    res = []
    for B, N in shapes:
        nbytes = (B + 1) * N * 4
        in_bytes = B * N * 4
        # launches rotate over copies of at least 2 GiB in total (8 times the 256 MB
        # Infinity Cache), so that their reads come from HBM
        copies = 1 if in_bytes >= 512 * 2 ** 20 else min(8192, -(-2 * 2 ** 30 // in_bytes))
        gen = torch.Generator(device="cuda").manual_seed(B * 31 + N)
        xs = [torch.randn((B, N), device="cuda", generator=gen) for _ in range(copies)]
        out = torch.empty(N, device="cuda")
        i = [0]

        def run():
            cfc.reduce_axis0(xs[i[0] % copies], out)
            i[0] += 1
        r = timer(run, max(10, copies))
        t_s = r["mean_s"]
        row = dict(B=B, N=N, bytes=nbytes, us=round(t_s * 1e6, 2), GBps=round(nbytes / t_s / 1e9, 1),
                   frac=round(nbytes / t_s / HBM_PEAK, 3), cold=copies * in_bytes >= 512 * 2 ** 20)
        if copies > 1:
            # the same buffer every launch: its reads can come from the Infinity Cache
            w = timer(lambda: cfc.reduce_axis0(xs[0], out), 20)["mean_s"]
            row["warm_us"] = round(w * 1e6, 2)
            row["warm_GBps"] = round(nbytes / w / 1e9, 1)
        res.append(row)
        del xs, out
        torch.cuda.empty_cache()
    return res


def bench_adamw(torch, cfc, timer, sizes_list):
    """AdamW after the reducer: one fused launch over the given segments.
    Algorithmic bytes per element: read p, g, m, v and write p, m, v (28 B)."""
    rows = []
    for sizes in sizes_list:
        segs = [[torch.randn(n, device="cuda") * s for n in sizes] for s in (0.5, 1e-2, 1e-2, 1e-2)]
        segs[3] = [v.square() for v in segs[3]]
        it = [0]

        def run():
            it[0] += 1
            cfc.cfc_adamw_step(*segs, 1e-3, 0.9, 0.999, 1e-8, 0.01, it[0])
        r = timer(run, 20 if sum(sizes) > (1 << 22) else 50)
        by = 28 * sum(sizes)
        rows.append(dict(sizes=list(sizes), bytes=by, mean_us=round(r["mean_s"] * 1e6, 3),
                         gbps=round(by / r["mean_s"] / 1e9, 1), frac=round(by / r["mean_s"] / HBM_PEAK, 4)))
        del segs
    return rows


def mlp_flops(B, dims):
    """Algorithmic flops of one MLP step: forward and weight gradient of every
    layer, upstream gradient of every layer but the first (2 per fma)."""
    f = sum(2 * B * dims[l] * dims[l + 1] for l in range(len(dims) - 1))
    dx = sum(2 * B * dims[l] * dims[l + 1] for l in range(1, len(dims) - 1))
    return 2 * f + dx


def bench_mlp(torch, timer, steps, trials, cpu_seconds):
    """The batched MLP training step (48-256-256-128-51, B = 16384): steps/s,
    the matrix-core roofline, per-launch timing, and the oracle's time for
    one step on the host."""
    from recurrent_cell_amd import mlp
    from recurrent_cell_amd.inputs import MLP_B, MLP_DIMS, MlpInputs
    B, dims = MLP_B, list(MLP_DIMS)
    x = MlpInputs(B, dims, seed=0)
    Xd, Td = torch.from_numpy(x.X).cuda(), torch.from_numpy(x.T).cuda()
    params = mlp.pack_params([torch.from_numpy(w).cuda() for w in x.W], [torch.from_numpy(b).cuda() for b in x.b],
                             dims)
    out = mlp.MlpBuffers.allocate(B, dims, "cuda")
    for _ in range(10):
        mlp.mlp_train_step(Xd, Td, dims, params, out=out)
    torch.cuda.synchronize()
    res = []
    for _ in range(trials):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            mlp.mlp_train_step(Xd, Td, dims, params, out=out)
        b.record()
        torch.cuda.synchronize()
        res.append(a.elapsed_time(b) / steps)
    ms = float(np.median(res))
    fl = mlp_flops(B, dims)
    # per launch: the layer products of one step, timed one by one
    L = len(dims) - 1
    Ws = [w for w, _ in mlp.unpack(params, dims)]
    bs = [b for _, b in mlp.unpack(params, dims)]
    acts = out.act
    kt = {}
    for l in range(L):
        xin = Xd if l == 0 else acts[l - 1]
        r = timer(lambda: mlp.mlp_linear_fwd(xin, Ws[l], bs[l], Y=acts[l], relu=l < L - 1), 30)
        kt["fwd%d" % l] = dict(us=round(r["mean_s"] * 1e6, 2), flops=2 * B * dims[l] * dims[l + 1])
    gy = [torch.randn((B, d), device="cuda") for d in dims[1:]]
    for l in range(1, L):
        r = timer(lambda: mlp.mlp_linear_bwd_data(gy[l], Ws[l], mask=acts[l - 1], dX=gy[l - 1]), 30)
        kt["dx%d" % l] = dict(us=round(r["mean_s"] * 1e6, 2), flops=2 * B * dims[l] * dims[l + 1])
    ws = torch.empty(mlp.lib().mlp_linear_bwd_weight_workspace_bytes(B, dims[1], dims[2]) // 4 + 1, device="cuda")
    gW = torch.empty((dims[2], dims[1]), device="cuda")
    gb = torch.empty((dims[2],), device="cuda")
    r = timer(lambda: mlp.mlp_linear_bwd_weight(gy[1], acts[0], gW=gW, gb=gb, ws=ws), 30)
    kt["dw1 (with its reduce)"] = dict(us=round(r["mean_s"] * 1e6, 2), flops=2 * B * dims[1] * dims[2])
    for v in kt.values():
        v["TFLOPs"] = round(v["flops"] / (v["us"] * 1e-6) / 1e12, 2)
    big = kt["fwd1"]
    roof = {"bound": "mfma", "achieved": big["TFLOPs"], "peak": FP32_PEAK / 1e12, "unit": "TFLOP/s",
            "frac": round(big["TFLOPs"] * 1e12 / FP32_PEAK, 4), "traffic": None,
            "kernel": "gemm_mfma_kernel (layer 1 forward, [16384 x 256] x [256 x 256])",
            "flops_per_launch": big["flops"], "launch_us": big["us"]}
    cpu = None
    if cpu_seconds > 0:
        # the numpy fp64 oracle with its BLAS on one thread, then on every
        # usable thread (threadpoolctl sets the BLAS pool)
        from threadpoolctl import threadpool_limits
        from oracle.mlp_oracle import mlp_train_step as oracle_step
        cpu = {}
        for key, th in (("fp64_1t", 1), ("fp64_all", host_threads())):
            with threadpool_limits(limits=th):
                n = 0
                t0 = time.perf_counter()
                while True:
                    oracle_step(x.X, x.T, x.W, x.b)
                    n += 1
                    if time.perf_counter() - t0 >= min(cpu_seconds, 4.0):
                        break
                el = time.perf_counter() - t0
            cpu[key] = {"value": round(n / el, 3), "unit": "train-steps/s", "cores": th, "kind": "oracle",
                        "sample": "%d whole steps, numpy fp64, BLAS on %d thread(s), %.1f s" % (n, th, el)}
    return {"workload": "batched MLP train step (forward, MSE loss, backward, every gradient), one mlp_train_step "
                        "call", "B": B, "dims": dims, "value": round(1000.0 / ms, 2), "unit": "train-steps/s",
            "ms_per_step": round(ms, 5), "trials_ms": [round(v, 5) for v in res], "flops_per_step": fl,
            "step_TFLOPs": round(fl / (ms * 1e-3) / 1e12, 2), "step_frac_fp32_peak": round(fl / (ms * 1e-3) /
                                                                                         FP32_PEAK, 4),
            "roofline": roof, "launches": kt, "cpu_oracle": cpu}


def _oracle_steps_per_s(oracle, x, precision, threads, budget_s, batch=None):
    """Whole training steps of the oracle per second on `threads` host threads
    (at least one call, then until budget_s has passed).  With batch=b', the
    first b' samples of the workload stand in for all B (samples are
    independent, so the per-step work is linear in B) and the rate is scaled
    by b'/B.  Returns (steps/s of the full workload, calls, seconds, threads used)."""
    B = x.h0.shape[0]
    u, y, h0 = x.u, x.y, x.h0
    if batch is not None and batch < B:
        u, y, h0 = (np.ascontiguousarray(a) for a in (x.u[:, :batch], x.y[:, :batch], x.h0[:batch]))
    else:
        batch = B
    args = (u, y, h0, x.W, x.bias)
    oracle.set_threads(threads)
    used = oracle.threads()
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.train(*args, precision)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return n / el * batch / B, n, el, used


def host_threads():
    """Host threads this process may use: its CPU affinity, capped by
    OMP_NUM_THREADS where that is set."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return max(1, n)


def cpu_baselines(configs, budget_s):
    """The oracle as it stands (plain C, gcc -O2, OpenMP over samples only),
    timed on the host beside the GPU: fp64 and fp32 on one thread and fp32 on
    every usable thread, for the tiny, pages and wide configurations (the wide
    one on a bounded sample of its samples), plus the batch-axis reduction's
    fp64 column sums on one thread and split over columns on every thread."""
    import oracle
    from recurrent_cell_amd.inputs import cfc_inputs
    allt = host_threads()
    before = oracle.threads()
    out = {"host_threads": allt}
    try:
        for name, plan in (("pages", [("fp64_1t", "f64", 1, None), ("fp32_1t", "f32", 1, None),
                                      ("fp32_all", "f32", allt, None)]),
                           ("tiny", [("fp32_1t", "f32", 1, None), ("fp32_all", "f32", allt, None)]),
                           ("wide", [("fp32_1t", "f32", 1, 8), ("fp32_all", "f32", allt, 8 * allt)])):
            d = configs[name]
            x = cfc_inputs(**d, seed=0)
            rows = {}
            for key, prec, th, batch in plan:
                v, n, el, used = _oracle_steps_per_s(oracle, x, prec, th, budget_s, batch)
                b = d["B"] if batch is None or batch >= d["B"] else batch
                rows[key] = {"value": round(v, 4), "unit": "train-steps/s", "cores": used, "kind": "oracle",
                             "sample": "%d whole train steps (B=%d C=%d n_x=%d K=%d), %s oracle, %d thread(s), "
                                       "%.1f s%s" % (n, b, d["C"], d["n_x"], d["K"], prec, used, el,
                                                     "" if b == d["B"] else
                                                     "; %d of the %d samples, rate scaled by %d/%d" %
                                                     (b, d["B"], b, d["B"]))}
            out[name] = rows
        B, N = 32, 1 << 20
        xr = np.random.default_rng(0).standard_normal((B, N), dtype=np.float32)
        by = (B + 1) * N * 4
        red = {}
        for key, th in (("fp64_1t", 1), ("fp64_all", allt)):
            oracle.set_threads(th)
            used = oracle.threads()
            n = 0
            t0 = time.perf_counter()
            while True:
                oracle.reduce_axis0_f64(xr)
                n += 1
                el = time.perf_counter() - t0
                if el >= min(budget_s, 2.0):
                    break
            red[key] = {"GBps": round(n * by / el / 1e9, 2), "cores": used, "kind": "oracle",
                        "sample": "%d calls on B=%d, N=%d (fp64 column sums in b order, columns split over %d "
                                  "thread(s)), %.1f s" % (n, B, N, used, el)}
        out["reduce_axis0"] = red
    finally:
        oracle.set_threads(before)
    return out


PATH_NAMES = {2: "persistent", 3: "steps_valu", 4: "steps_mfma", 5: "resident_mfma"}


def step_roofline(path, B, C, n_x, K, ms_per_step, t_node, persist_launches=None):
    """The step against its bounds.  The persistent path's headline ratio is
    the critical path at the non-packed fp32 rate: the 2K recurrence steps of
    a sample run in order on one CU, so they are bounded by one CU's rate, not
    the chip's; the parallel kernels by their whole-chip floors; plus one node
    latency per launch.  SURVEY's formula (node latencies plus the whole-chip
    floor of the flops or bytes) is given beside it, over this path's launches
    and, as context only, over the pages' 2K + 3 dependent launches."""
    bytes_min, flops = step_bytes_flops(B, C, n_x, K)
    nodes = {"persistent": persist_launches or (3 if B <= PERSIST_FUSE_MAX_B else 4),
             "steps_valu": 2 * K + 2, "steps_mfma": 2 * K + 3,
             "resident_mfma": 5}[path]
    t_formula = nodes * t_node + max(flops / FP32_PEAK, bytes_min / HBM_PEAK)
    pages_nodes = 2 * K + 3
    t_pages = pages_nodes * t_node + max(flops / FP32_PEAK, bytes_min / HBM_PEAK)
    r = {"path": path, "nodes": nodes, "t_node_us": round(t_node * 1e6, 3), "flops": flops, "bytes_min": bytes_min}
    if path == "persistent":
        cu_clk = 2.4e9
        t_rec = recurrence_flops(B, C, K) / B / (256 * cu_clk)
        par_flops = projection_flops(B, C, n_x, K) + 2 * K * B * 3 * C * (n_x + C)
        par_bytes = fill_bytes(B, C, n_x, K) + 4 * (B + 1) * 3 * C * (n_x + C) + 4 * K * B * (n_x + 3 * C)
        t_par = max(par_flops / FP32_PEAK, par_bytes / HBM_PEAK)
        t_np = nodes * t_node + 2 * t_rec + t_par
        t_pk = nodes * t_node + t_rec + t_par
        r.update({"roof": "critical path: per-CU recurrence at the non-packed fp32 rate (128 flop/clk/CU at "
                          "2.4 GHz) + parallel kernels at whole-chip floors + one node latency per launch",
                  "t_roof_ms": round(t_np * 1e3, 4), "step_over_roof": round(ms_per_step / (t_np * 1e3), 3),
                  "recurrence_floor_nonpacked_us": round(2 * t_rec * 1e6, 2),
                  "parallel_floor_us": round(t_par * 1e6, 2),
                  "packed_rate_roof_ms": round(t_pk * 1e3, 4),
                  "step_over_packed_rate_roof": round(ms_per_step / (t_pk * 1e3), 3)})
    else:
        r.update({"roof": "node latencies of this path's launches + whole-chip floor of the step's flops or bytes",
                  "t_roof_ms": round(t_formula * 1e3, 4), "step_over_roof": round(ms_per_step / (t_formula * 1e3), 3)})
    r["context"] = {"whole_chip_formula_ms": round(t_formula * 1e3, 4),
                    "step_over_whole_chip_formula": round(ms_per_step / (t_formula * 1e3), 3),
                    "pages_graph_nodes": pages_nodes, "pages_graph_roof_ms": round(t_pages * 1e3, 4),
                    "step_over_pages_graph_roof": round(ms_per_step / (t_pages * 1e3), 3),
                    "note": "the pages-graph figure charges the pages' 2K + 3 dependent launches, which this "
                            "path does not run when it is the persistent one: context only"}
    return r


def persist_fill_fused(torch, out, B, C, K):
    """Whether the persistent launch last made on out.ws also formed the
    scratch: the workspace's last region holds one flag per projection
    workgroup, the error word, then one per sample and chunk of 16 steps,
    which such a launch sets to its number (that of the projection flags)."""
    n = -(-K * B // 64) * -(-3 * C // 64)
    nc = -(-K // 16)
    region = (n + 1 + B * nc + 63) // 64 * 64
    f = out.ws[out.ws.numel() - region:].view(torch.int32).cpu().numpy()
    return bool(f[0] != 0 and f[n] != f[0] and (f[n + 1:n + 1 + B * nc] == f[0]).all())


def kloop_roofline(torch, cfc, path, kt, B, C, n_x, K, workload):
    """Roofline object of the K-loop's dominant kernel from live timings kt."""
    n_in = n_x + C
    if path == "persistent":
        # the step's launch: with B <= PERSIST_FUSE_MAX_B it also forms X,
        # and, when its workgroups fit the CUs, the per-sample scratch (their
        # flops counted); timed through cfc_kloop_fwd_bwd_fill (or
        # cfc_kloop_fwd_bwd), which is that one launch; the recurrence alone
        # (X given) is reported beside
        fused = B <= PERSIST_FUSE_MAX_B
        filled = fused and kt.get("fill_fused", False)
        dur = (kt["fwd_bwd_fill"]["mean_s"] if filled else kt["fwd_bwd"]["mean_s"]) if fused \
            else kt["recurrence"]["mean_s"]
        rec_fl = recurrence_flops(B, C, K)
        fl = rec_fl + (projection_flops(B, C, n_x, K) if fused else 0) + \
            (2 * K * B * 3 * C * (n_x + C) if filled else 0)
        achieved = fl / dur
        rec_achieved = rec_fl / dur
        traffic = measured_traffic() if workload == "pages" else None
        valu_busy = measured_valu_busy() if workload == "pages" else None
        # what the kernel can use: one CU per sample (B of 256), fp32 FMA
        # without packed math (4 SIMDs x 16 lanes x 2 flop per clock; half
        # the 256 flop per clock per CU of the published peak)
        usable = min(B, 256) * 2.4e9 * 4 * 16 * 2
        # the same rate measured: the FMA-chain probe on B workgroups of the
        # kernel's 512 lanes, one per CU, and on all 256 CUs
        meas_b = fma_rate(torch, cfc, min(B, 256))
        meas_chip = fma_rate(torch, cfc, 256)
        return {"bound": "alu", "achieved": round(achieved / 1e12, 3), "peak": FP32_PEAK / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, calibrated)",
                "kernel": "kloop_persist_kernel" + (" (its launch also forms X and the scratch)" if filled
                                                    else " (its launch also forms X)" if fused else ""),
                "flops_per_launch": fl, "flops_note": "recurrence (W_h h forward, W_h^T dp backward)" +
                                                      (" + input projection" if fused else "") +
                                                      (" + scratch fill" if filled else ""),
                "launch_us": round(dur * 1e6, 3),
                "recurrence_alone_us": round(kt["recurrence"]["mean_s"] * 1e6, 3),
                "recurrence_alone_note": "the same kernel given X (cfc_kloop_recurrence), one launch",
                "usable_peak": round(usable / 1e12, 3),
                "frac_of_usable": round(rec_achieved / usable, 4),
                "usable_note": "recurrence flops over the launch: one CU per sample (a sample's steps are "
                               "sequential), non-packed fp32 FMA",
                "usable_peak_measured": round(meas_b / 1e12, 3),
                "frac_of_usable_measured": round(rec_achieved / meas_b, 4),
                "fma_probe_chip_TFLOPs": round(meas_chip / 1e12, 2),
                "fma_probe_chip_GHz": round(meas_chip / (256 * 128) / 1e9, 3),
                "fma_probe_note": "v_fma_f32 chains, 512 lanes per workgroup, one workgroup per CU; "
                                  "GHz = chip rate / (256 CUs x 128 flop/clk)",
                "traffic_GBps": round(traffic / dur / 1e9, 1) if traffic else None,
                "traffic_frac_of_hbm_peak": round(traffic / dur / HBM_PEAK, 4) if traffic else None,
                "valu_busy_rocprof": valu_busy,
                "valu_busy_note": "SQ_ACTIVE_INST_VALU / SQ_BUSY_CU_CYCLES over the kernel's CUs "
                                  "(profiles/kloop_persist_pages_valu.md)"}
    if path == "steps_mfma":
        # the 2K step launches of the K-loop (and the one W re-layout), per launch on average
        dur = kt["fwd_bwd"]["mean_s"] / (2 * K)
        fl = K * B * 3 * C * (n_in + C) * 2 // (2 * K)
        achieved = fl / dur
        return {"bound": "mfma", "achieved": round(achieved / 1e12, 3), "peak": FP32_PEAK / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK, 4), "traffic": None,
                "kernel": "fwd_mfma_kernel + bwd_mfma_kernel (average over the 2K step launches)",
                "flops_per_launch": fl, "launch_us": round(dur * 1e6, 3)}
    if path == "resident_mfma":
        # one launch for all 2K steps (with the W re-layout and the exchange
        # clear before it, in the timed call)
        dur = kt["fwd_bwd"]["mean_s"]
        fl = K * B * 3 * C * (n_in + C) * 2
        achieved = fl / dur
        return {"bound": "mfma", "achieved": round(achieved / 1e12, 3), "peak": FP32_PEAK / 1e12,
                "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK, 4), "traffic": None,
                "kernel": "kloop_resident_kernel (all 2K steps; the call also holds the W re-layout)",
                "flops_per_launch": fl, "launch_us": round(dur * 1e6, 3),
                "us_per_step": round(dur * 1e6 / (2 * K), 3)}
    dur = kt["fwd_bwd"]["mean_s"] / (2 * K)
    fl = K * B * 3 * C * (n_in + C) * 2 // (2 * K)
    achieved = fl / dur
    return {"bound": "alu", "achieved": round(achieved / 1e12, 3), "peak": FP32_PEAK / 1e12,
            "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK, 4), "traffic": None,
            "kernel": "fwd_step_kernel + bwd_step_kernel (average over the 2K step launches)",
            "flops_per_launch": fl, "launch_us": round(dur * 1e6, 3)}


def time_kloop(torch, cfc, workload, steps, warmup, trials):
    """The train step of one configuration, timed alone: (ms_per_step, trials_ms)."""
    from recurrent_cell_amd.inputs import CONFIGS, cfc_inputs
    x = cfc_inputs(**CONFIGS[workload], seed=0)
    t = [torch.from_numpy(a).cuda() for a in (x.u, x.y, x.h0, x.W, x.bias)]
    out = cfc.cfc_train_kloop(*t)
    r = time_steps(torch, cfc, t, out, steps, warmup, trials)
    del out, t
    torch.cuda.empty_cache()
    return r


def bench_kloop(torch, cfc, workload, steps, warmup, trials, t_node, detail, timed=None):
    """One configuration of the K-loop: train steps/s of cfc_train_kloop, the
    live per-kernel timings and the roofline objects.  detail=True adds the
    contrast path, the GEMM-form step and the single-step kernels.  timed:
    (ms_per_step, trials_ms) measured beforehand (time_kloop), used instead
    of timing the steps here."""
    from recurrent_cell_amd.inputs import CONFIGS, cfc_inputs
    d = CONFIGS[workload]
    B, C, n_x, K = d["B"], d["C"], d["n_x"], d["K"]
    n_in = n_x + C
    x = cfc_inputs(**d, seed=0)
    t = [torch.from_numpy(a).cuda() for a in (x.u, x.y, x.h0, x.W, x.bias)]
    path = PATH_NAMES[cfc.cfc_kloop_path(B, C, n_x, K)]
    out = cfc.cfc_train_kloop(*t)
    ms_per_step, trials_ms = timed if timed is not None else time_steps(torch, cfc, t, out, steps, warmup, trials)
    res = {"workload": workload, "B": B, "C": C, "n_x": n_x, "n_in": n_in, "K": K, "path": path,
           "value": round(1000.0 / ms_per_step, 2), "unit": "train-steps/s", "ms_per_step": round(ms_per_step, 5),
           "trials_ms": [round(v, 5) for v in trials_ms]}

    timer = LaunchTimer(torch)
    kt = {}
    n_rep = 20 if K * B * C * n_in < (1 << 26) else 5
    kt["fwd_bwd"] = timer(lambda: cfc.cfc_kloop_fwd_bwd(*t, out=out), n_rep)
    if path == "persistent":
        kt["fwd_bwd_fill"] = timer(lambda: cfc.cfc_kloop_fwd_bwd_fill(*t, out=out), n_rep)
        kt["fill_fused"] = persist_fill_fused(torch, out, B, C, K)
        X = torch.empty((K, B, 3 * C), device="cuda")
        kt["input_projection"] = timer(lambda: cfc.cfc_input_projection(t[0], t[3], t[4], X), 50)
        kt["recurrence"] = timer(lambda: cfc.cfc_kloop_recurrence(X, t[1], t[2], t[3], out=out), 20)
    dp = out.ws[:K * B * 3 * C].view(K, B, 3 * C)
    kt["scratch_fill"] = timer(lambda: cfc.cfc_scratch_fill(dp, t[0], out.h_hist, out.gW_scratch,
                                                            out.gb_scratch), 20)
    gW_flat = out.gW_scratch.view(B, -1)
    red_out = torch.empty(3 * C * n_in, device="cuda")
    kt["reduce_axis0"] = timer(lambda: cfc.reduce_axis0(gW_flat, red_out), 20)

    if detail or path == "resident_mfma":
        # another path on the same inputs, for contrast: the step kernels after
        # the persistent path; the other step-kernel variant after a step
        # path; the MFMA step kernels (2K launches) after the resident kernel
        modes = {"persistent": cfc.KLOOP_STEPS, "steps_mfma": cfc.KLOOP_STEPS_VALU,
                 "steps_valu": cfc.KLOOP_STEPS_MFMA, "resident_mfma": cfc.KLOOP_STEPS_MFMA}
        cfc.cfc_set_kloop_mode(modes[path])
        try:
            taken = cfc.cfc_kloop_path(B, C, n_x, K)
            if taken >= 0:
                out_c = cfc.cfc_train_kloop(*t)
                ms_c, _ = time_steps(torch, cfc, t, out_c, max(20, steps // 10), 5, 3)
                res["contrast"] = {"path": PATH_NAMES[taken], "ms_per_step": round(ms_c, 5)}
                del out_c
        finally:
            cfc.cfc_set_kloop_mode(cfc.KLOOP_AUTO)
    if detail:
        # the K-loop step with the GEMM-form weight gradient in place of scratch + reducer
        og = cfc.cfc_train_kloop_gemm(*t)
        ms_g, _ = time_calls(torch, lambda: cfc.cfc_train_kloop_gemm(*t, out=og), max(20, steps // 5), 5, 3)
        res["gemm_form_weight_grad_ms_per_step"] = round(ms_g, 5)
        gws = torch.empty(cfc.lib().cfc_weight_grad_gemm_workspace_bytes(B, C, n_x, K) // 4 + 1, device="cuda")
        gWg, gbg = torch.empty((3, C, n_in), device="cuda"), torch.empty((3, C), device="cuda")
        kt["weight_grad_gemm"] = timer(lambda: cfc.cfc_weight_grad_gemm(dp, t[0], out.h_hist, gWg, gbg, gws), 50)
        # single-step kernels (the ABI calls, per-step += into the scratch)
        S = torch.zeros((B, 3, C, n_in), device="cuda")
        Sb = torch.zeros((B, 3, C), device="cuda")
        dh = [torch.zeros((B, C), device="cuda") for _ in range(2)]
        h_hist, act = out.h_hist, out.act
        it = [0]

        def fwd():
            k = it[0] % K
            cfc.cfc_fwd_step(t[0][k], h_hist[k], t[3], t[4], h_t=h_hist[k + 1], act_t=act[k])
            it[0] += 1

        def bwd():
            k = K - 1 - it[0] % K
            cfc.cfc_bwd_step(t[0][k], h_hist[k], h_hist[k + 1], t[1][k], t[3], act[k], dh[it[0] % 2], S, Sb,
                             dh_out=dh[(it[0] + 1) % 2])
            it[0] += 1
        kt["fwd_step"] = timer(fwd, 2 * K)
        it[0] = 0
        kt["bwd_step"] = timer(bwd, 2 * K)
        del S, Sb
    cfc.cfc_train_kloop(*t, out=out)   # restore the step's own state
    torch.cuda.synchronize()
    res["kernels"] = {k: dict(mean_us=round(v["mean_s"] * 1e6, 3), pair_median_us=round(v["pair_median_s"] * 1e6, 3),
                              n=v["n"]) for k, v in kt.items() if isinstance(v, dict)}
    if path == "persistent":
        res["persist_launch_forms_scratch"] = kt["fill_fused"]
    res["roofline"] = kloop_roofline(torch, cfc, path, kt, B, C, n_x, K, workload)
    res["step_roofline"] = step_roofline(path, B, C, n_x, K, ms_per_step, t_node,
                                         2 if kt.get("fill_fused") else None)
    if detail:
        res["deterministic_3_runs"] = deterministic_runs(torch, cfc, t)
    del out
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--trials", type=int, default=7)
    ap.add_argument("--cpu-seconds", type=float, default=2.5, help="seconds per CPU-oracle measurement")
    ap.add_argument("--no-reduce", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--workload", default="pages", choices=["tiny", "pages", "wide"],
                    help="the configuration of the headline line")
    ap.add_argument("--no-other-workloads", action="store_true", help="skip the tiny and wide legs")
    ap.add_argument("--no-mlp", action="store_true", help="skip the batched MLP step")
    ap.add_argument("--no-adamw", action="store_true", help="skip the AdamW timings")
    ap.add_argument("--only-mlp", action="store_true", help="run and print only the batched MLP step")
    ap.add_argument("--only-step", action="store_true",
                    help="time the headline workload's train step only (for profiling runs)")
    ap.add_argument("--only-reduce", action="store_true",
                    help="run and print only the reduce_axis0 shapes (for profiling runs)")
    ap.add_argument("--no-kernels", action="store_true", help="same as --only-step")
    ap.add_argument("--no-steps-path", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--no-gemm-form", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (a known-size reference for "
                         "hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path.  The K-loop "
              "would shard over the batch (B/G samples per GPU, W replicated), each GPU reducing its "
              "own scratch, then one all-gather of the G partial gradients and a fixed-order sum of "
              "them on every GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    from recurrent_cell_amd import cfc
    from recurrent_cell_amd.inputs import CONFIGS, REDUCE_B, REDUCE_N, cfc_inputs

    if args.only_mlp:
        print(json.dumps({"mlp": bench_mlp(torch, LaunchTimer(torch), args.steps, args.trials,
                                           0.0 if args.no_cpu else args.cpu_seconds)}), flush=True)
        return

    d = CONFIGS[args.workload]
    B, C, n_x, K = d["B"], d["C"], d["n_x"], d["K"]
    n_in = n_x + C
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty(n, device="cuda")
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.only_reduce:
        shapes = [(b, n) for b in REDUCE_B for n in REDUCE_N]
        print(json.dumps({"reduce_axis0": bench_reduce(torch, cfc, LaunchTimer(torch), shapes)}), flush=True)
        return
    if args.only_step or args.no_kernels:
        x = cfc_inputs(**d, seed=0)
        t = [torch.from_numpy(a).cuda() for a in (x.u, x.y, x.h0, x.W, x.bias)]
        out = cfc.cfc_train_kloop(*t)
        ms, tr = time_steps(torch, cfc, t, out, args.steps, args.warmup, args.trials)
        print(json.dumps({"workload": args.workload, "ms_per_step": round(ms, 5),
                          "value": round(1000.0 / ms, 2), "trials_ms": [round(v, 5) for v in tr]}), flush=True)
        return

    t_node = graph_node_latency(torch)
    # Every configuration's step is timed before any detail leg: the detail
    # legs (a forced step-path contrast captured as graphs, probes) measurably
    # slow a later cooperative launch in the same process (the wide step:
    # 0.88 against 0.73 ms).  The headline step first, then the others.
    head_timed = time_kloop(torch, cfc, args.workload, args.steps, args.warmup, args.trials)
    legs = {}
    if not args.no_other_workloads:
        for w in ("tiny", "pages", "wide"):
            if w == args.workload:
                continue
            legs[w] = bench_kloop(torch, cfc, w, 200 if w == "tiny" else 50, 10, 5, t_node, detail=False)
            print("[bench] %s step: %.5f ms" % (w, legs[w]["ms_per_step"]), file=sys.stderr, flush=True)
    head = bench_kloop(torch, cfc, args.workload, args.steps, args.warmup, args.trials, t_node, detail=True,
                       timed=head_timed)
    print("[bench] %s step: %.5f ms" % (args.workload, head["ms_per_step"]), file=sys.stderr, flush=True)

    result = {
        "metric": METRIC, "value": head["value"], "unit": "train-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "CfC K-loop train step (fwd + BPTT + scratch + reduce_axis0), one cfc_train_kloop call",
                   "B": B, "C": C, "n_x": n_x, "n_in": n_in, "K": K, "seed": 0, "path": head["path"]},
        "roofline": head["roofline"],
        "step_roofline": head["step_roofline"],
        "kernels": head["kernels"],
        "trials_ms": head["trials_ms"],
        "contrast": head.get("contrast"),
        "gemm_form_weight_grad_ms_per_step": head.get("gemm_form_weight_grad_ms_per_step"),
        "deterministic_3_runs": head.get("deterministic_3_runs"),
    }
    result["host"] = host_info()

    if not args.no_other_workloads:
        result["workloads"] = legs

    if not args.no_reduce:
        peak = copy_peak(torch)
        result["hbm_copy_peak"] = {"GBps": round(peak / 1e9, 1), "frac_of_datasheet": round(peak / HBM_PEAK, 4),
                                   "what": "torch fp32 device copy, 2 GiB read + 2 GiB written, median of 10"}
        timer = LaunchTimer(torch)
        shapes = [(b, n) for b in REDUCE_B for n in REDUCE_N]
        red = bench_reduce(torch, cfc, timer, shapes)
        for r in red:
            r["frac_copy"] = round(r["GBps"] / result["hbm_copy_peak"]["GBps"], 3)
        gate = [r for r in red if r["B"] * r["N"] * 4 >= 512 * 2 ** 20]
        result["reduce_axis0"] = {"shapes": red,
                                  "min_frac_large": min(r["frac"] for r in gate) if gate else None}
        print("[bench] reduce_axis0 done", file=sys.stderr, flush=True)

    if not args.no_mlp:
        result["mlp"] = bench_mlp(torch, LaunchTimer(torch), 50, 5, 0.0 if args.no_cpu else args.cpu_seconds)
        print("[bench] mlp done", file=sys.stderr, flush=True)

    if not args.no_adamw:
        # the optimizer step beside the path: W and bias of this cell, then large flat tensors
        result["adamw"] = bench_adamw(torch, cfc, LaunchTimer(torch),
                                      [(3 * C * n_in, 3 * C), (1 << 24,), (1 << 26,)])

    if not args.no_cpu:
        cb = cpu_baselines(CONFIGS, args.cpu_seconds)
        main_leg = cb[args.workload]
        best = main_leg["fp32_all"]
        result["cpu_baseline"] = dict(best)
        result["cpu_baseline"]["variants"] = {args.workload: main_leg}
        result["cpu_baseline"]["host_threads"] = cb["host_threads"]
        result["cpu_baseline"]["gpu_over_cpu"] = round(result["value"] / best["value"], 1)
        for w in ("tiny", "pages", "wide"):
            if w != args.workload:
                result["cpu_baseline"]["variants"][w] = cb[w]
                if "workloads" in result and w in result["workloads"]:
                    result["workloads"][w]["cpu_baseline"] = cb[w]
        if "reduce_axis0" in result:
            result["reduce_axis0"]["cpu_oracle"] = cb["reduce_axis0"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
