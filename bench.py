"""Benchmark: CfC K-loop training steps per second on one MI355X.

A step is one replay of the whole K-loop graph (forward t = 1..K, BPTT
t = K..1 into the per-sample scratch, reduce_axis0 of both scratch tensors)
on the pages-shaped configuration B=32, C=128, n_x=64 (n_in=192), K=64,
fp32, inputs seeded and already resident in HBM.  Prints ONE JSON line.

Also measured, in the same run:
  * per-launch durations of the forward and backward step kernels (HIP
    events around each launch on the launch stream) -> the roofline object
    of the kernel with the largest share of the step;
  * graph-node latency (a graph of dependent tiny kernels) -> the step's
    latency roofline;
  * reduce_axis0 GB/s on the standalone [B, N] shapes;
  * the CPU oracle on a bounded sample of the same workload (cpu_baseline).
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
FP32_PEAK = 157.3e12       # flop/s, MI355X fp32 vector


def step_bytes_flops(B, C, n_x, K):
    n_in = n_x + C
    f = 4
    bytes_min = f * (K * B * n_x + K * B * C + B * C + 3 * C * n_in + 3 * C      # u, y, h0, W, bias
                     + (K + 1) * B * C + K * 3 * B * C                           # h_hist, act written
                     + K * B * C + K * 3 * B * C                                 # re-read in backward
                     + 2 * (3 * B * C * n_in + 3 * B * C)                        # scratch once + reduce read
                     + 3 * C * n_in + 3 * C)                                     # gW, gb
    flops = K * B * 3 * C * n_in * 2 * 3                                        # fwd, scratch, W^T dp
    return bytes_min, flops


def bwd_launch_bytes(B, C, n_x):
    """Algorithmic bytes of one backward step launch: its inputs read once,
    the scratch read and written once, its outputs written once."""
    n_in = n_x + C
    return 4 * (B * n_x + 6 * B * C + B * C + 3 * C * n_in          # u_t h_prev h_t y_t dh_in act_t(3), W
                + 2 * 3 * B * C * n_in + 2 * 3 * B * C                # gW / gb scratch read + write
                + B * C)                                            # dh_out


def fwd_launch_bytes(B, C, n_x):
    n_in = n_x + C
    return 4 * (B * n_x + B * C + 3 * C * n_in + 3 * C + B * C + 3 * B * C)


def time_per_launch(torch, fn, n):
    """Average duration of fn's kernel: an event pair around each launch."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    ms = [s.elapsed_time(e) for s, e in ev]
    return float(np.mean(ms)) * 1e-3, float(np.median(ms)) * 1e-3


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


def bench_reduce(torch, cfc, shapes, reps=10):
    res = []
    for B, N in shapes:
        nbytes = (B + 1) * N * 4
        in_bytes = B * N * 4
        copies = 1 if in_bytes >= 512 * 2 ** 20 else min(64, -(-2 * 2 ** 30 // in_bytes))
        gen = torch.Generator(device="cuda").manual_seed(B * 31 + N)
        xs = [torch.randn((B, N), device="cuda", generator=gen) for _ in range(copies)]
        out = torch.empty(N, device="cuda")
        for i in range(2):
            cfc.reduce_axis0(xs[i % copies], out)
        i = [0]

        def run():
            cfc.reduce_axis0(xs[i[0] % copies], out)
            i[0] += 1
        mean_s, med_s = time_per_launch(torch, run, max(reps, copies))
        res.append(dict(B=B, N=N, bytes=nbytes, us=round(med_s * 1e6, 2),
                        GBps=round(nbytes / med_s / 1e9, 1), frac=round(nbytes / med_s / HBM_PEAK, 3),
                        cold=copies > 1 or in_bytes >= 512 * 2 ** 20))
        del xs, out
        torch.cuda.empty_cache()
    return res


def cpu_baseline(x, budget_s):
    """The fp64 oracle, single thread, on whole training steps of the same
    configuration until budget_s has passed."""
    import oracle
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.train(x.u, x.y, x.h0, x.W, x.bias, "f64")
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return n, el


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--trials", type=int, default=7)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-reduce", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--workload", default="pages", choices=["tiny", "pages", "wide"])
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(the K-loop would shard over the batch; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    from recurrent_cell_amd import cfc
    from recurrent_cell_amd.inputs import CONFIGS, REDUCE_B, REDUCE_N, cfc_inputs

    d = CONFIGS[args.workload]
    B, C, n_x, K = d["B"], d["C"], d["n_x"], d["K"]
    x = cfc_inputs(**d, seed=0)
    t = [torch.from_numpy(a).cuda() for a in (x.u, x.y, x.h0, x.W, x.bias)]
    out = cfc.cfc_train_kloop(*t)
    for _ in range(args.warmup):
        cfc.cfc_train_kloop(*t, out=out)
    torch.cuda.synchronize()

    trials = []
    for _ in range(args.trials):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(args.steps):
            cfc.cfc_train_kloop(*t, out=out)
        b.record()
        torch.cuda.synchronize()
        trials.append(a.elapsed_time(b) / args.steps)
    ms_per_step = float(np.median(trials))
    value = 1000.0 / ms_per_step

    # Per-launch durations of the step kernels, same shapes and state as the graph.
    n_in = n_x + C
    h_hist, act = out.h_hist, out.act
    S = torch.zeros((B, 3, C, n_in), device="cuda")
    Sb = torch.zeros((B, 3, C), device="cuda")
    dh = [torch.zeros((B, C), device="cuda") for _ in range(2)]
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
    nl = 4 * K
    fwd_mean, fwd_med = time_per_launch(torch, fwd, nl)
    it[0] = 0
    bwd_mean, bwd_med = time_per_launch(torch, bwd, nl)
    fwd_b, bwd_b = fwd_launch_bytes(B, C, n_x), bwd_launch_bytes(B, C, n_x)
    if bwd_mean * K >= fwd_mean * K:
        dom = dict(kernel="bwd_step_kernel", bytes=bwd_b, t=bwd_mean)
    else:
        dom = dict(kernel="fwd_step_kernel", bytes=fwd_b, t=fwd_mean)
    achieved = dom["bytes"] / dom["t"] / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                "frac": round(achieved * 1e9 / HBM_PEAK, 4), "traffic": None,
                "kernel": dom["kernel"], "bytes_per_launch": dom["bytes"],
                "launch_us": round(dom["t"] * 1e6, 3)}

    t_node = graph_node_latency(torch)
    n_nodes = 2 * K + 1
    bytes_min, flops = step_bytes_flops(B, C, n_x, K)
    t_roof = n_nodes * t_node + max(flops / FP32_PEAK, bytes_min / HBM_PEAK)
    step_roof = {"nodes": n_nodes, "t_node_us": round(t_node * 1e6, 3),
                 "t_roof_ms": round(t_roof * 1e3, 4), "step_over_roof": round(ms_per_step / (t_roof * 1e3), 3),
                 "flops": flops, "bytes_min": bytes_min,
                 "fwd_launch_us": round(fwd_mean * 1e6, 3), "bwd_launch_us": round(bwd_mean * 1e6, 3),
                 "fwd_launch_median_us": round(fwd_med * 1e6, 3), "bwd_launch_median_us": round(bwd_med * 1e6, 3)}

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "train-steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "CfC K-loop train step (fwd + BPTT + reduce_axis0), one hipGraph replay",
                   "B": B, "C": C, "n_x": n_x, "n_in": n_in, "K": K, "seed": 0},
        "roofline": roofline,
        "step_roofline": step_roof,
        "trials_ms": [round(v, 5) for v in trials],
    }

    if not args.no_reduce:
        shapes = [(b, n) for b in REDUCE_B for n in REDUCE_N]
        red = bench_reduce(torch, cfc, shapes)
        gate = [r for r in red if r["B"] * r["N"] * 4 >= 512 * 2 ** 20]
        result["reduce_axis0"] = {"shapes": red,
                                  "min_frac_large": min(r["frac"] for r in gate) if gate else None}

    if not args.no_cpu:
        n, el = cpu_baseline(x, args.cpu_seconds)
        result["cpu_baseline"] = {"value": round(n / el, 4), "unit": "train-steps/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": "%d whole train steps of the same workload (B=%d C=%d n_x=%d K=%d), "
                                            "fp64 oracle, one thread, %.1f s" % (n, B, C, n_x, K, el)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
