"""Benchmark of the verify-decode layer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one whole layer step (input boundary -> attention -> attention boundary ->
router/routing/pooler -> experts -> unpooler) of b = 8 verify rows at hidden 4096 with an
8192-token paged context, replayed from a HIP graph.  Inputs are resident in HBM before the
timed region.  To keep the 256 MB MALL and the L2s from serving repeat reads, steps rotate
over R independent copies of the weights and KV (R * touched bytes >= 1 GB); one graph holds
the R copies' steps back to back, as a serving graph holds consecutive layers.  For a
workload with a draft head (the 4-layer chain) a step is the whole chain: every layer, the
final boundary and the head.  Prints one JSON line.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBPS = 8000.0


def algorithmic_bytes(wk, counts_per_layer):
    """Weights + KV bytes one layer step must move (activations excluded; experts counted
    only if they received a routed row)."""
    d, w = wk["dims"], wk["workload"]
    H, Hq, Hkv, D = d["hidden"], d["n_q_heads"], d["n_kv_heads"], d["head_dim"]
    E, I, b = d["n_experts"], d["inter"], w.b
    dense = 2 * (2 * Hq + 2 * Hkv) * D * H + 2 * H * Hq * D + 2 * E * H + 4 * 4 * H
    per_expert = 3 * H * I * (0.5 + 1.0 / 16) + 8
    if w.dense_inter:  # a dense draft layer: no router, no experts; gate_up and down instead
        dense += 2 * 3 * H * w.dense_inter - 2 * E * H
        per_expert = 0.0
    total = 0.0
    for li, counts in enumerate(counts_per_layer):
        lens = wk["layers"][li]["seq_lens"].numpy().astype(np.int64)
        window = int(wk["layers"][li].get("window", 0))
        if window > 0:                          # a request's rows see its last w + q - 1 tokens
            lens = np.minimum(lens, window + w.q_rows - 1)
        kv = lens.sum() * Hkv * D * 2 * 2 + b * Hkv * D * 2 * 2
        total += dense + int((counts > 0).sum()) * per_expert + kv
    if wk.get("head") is not None and len(counts_per_layer) == len(wk["layers"]):
        V = wk["head"]["w_lm"].shape[0]
        total += 2 * V * H + 8 * V + 8 * H      # head weight, d2t, final and last post gains
    return total, int((counts_per_layer[0] > 0).sum()) * per_expert


TRAFFIC_FILE = "profiles/moe_experts_{workload}_traffic.txt"
KERNEL_SOURCES = ("speculative_verify_decode_amd/csrc/k_moe.hip",
                  "speculative_verify_decode_amd/csrc/sd_common.h")


def measured_traffic(workload):
    """HBM bytes per sd_moe_experts launch from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None if there is none for this workload or the expert kernels' sources
    have changed since the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, TRAFFIC_FILE.format(workload=workload))
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in ("traffic_bytes_per_launch", "source_sha256"):
            k, v = line.split(":", 1)
            fields[k] = v.split()[0]
    h = hashlib.sha256()
    for fn in KERNEL_SOURCES:
        with open(os.path.join(root, fn), "rb") as f:
            h.update(f.read())
    if fields.get("source_sha256") != h.hexdigest():
        return None
    return int(fields["traffic_bytes_per_launch"])


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or "unknown"."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def rotation_copies(K, step_bytes, requested=0):
    """Copies R of the weights and KV to rotate over: R divides the K timed steps, so every
    timed replay is one whole R-step graph; at least enough copies that R * step_bytes >= 1 GB
    (8 at the least, 16 at the most for that rule), at most 32.  Returns (R, remainder): a K
    with no such divisor keeps R = the lower bound and replays its K % R remaining steps as
    one graph of that many copies."""
    if requested:
        return requested, K % requested
    lo = min(max(math.ceil(1.0e9 / step_bytes), 8), 16, K)
    for R in range(lo, min(K, 32) + 1):
        if K % R == 0:
            return R, 0
    return lo, K % lo


def read_ceiling(dev, nbytes=1 << 30, reps=10):
    """A plain streaming read of a 1 GiB buffer (sd_debug_read_probe): the practical HBM read
    rate on this machine, timed with HIP events around reps back-to-back reads."""
    from speculative_verify_decode_amd import binding as B
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = B.read_probe_sink(dev)
    for _ in range(2):
        B.debug_read_probe(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        B.debug_read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    del buf
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"GBps": round(gbps, 1), "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "bytes": nbytes, "us": round(us, 3), "kernel": "sd_debug_read_probe"}


def cpu_baseline(wk):
    """The oracle, as it stands, on full layer steps of the workload, repeated until about
    10 s of host time (at most 4 steps); the mean per step."""
    import threadpoolctl
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import oracle
    from tests.helpers import np64, oracle_layer_inputs
    lay, act, d = wk["layers"][0], wk["act"], wk["dims"]
    inp = oracle_layer_inputs(lay, act)
    threads = max((p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()), default=1)
    times = []
    while len(times) < 4 and sum(times) < 10.0:
        t0 = time.perf_counter()
        oracle.layer_step(inp, d, branch_in=np64(act["branch_in"]))
        times.append(time.perf_counter() - t0)
    return {"value": float(np.mean(times)) * 1e6, "unit": "us per layer-step", "cores": int(threads),
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{len(times)} full layer steps of {wk['workload'].name} (fp64 NumPy oracle, "
                      f"{sum(times):.1f} s), {len(os.sched_getaffinity(0))} host cores visible"}


def print_dense(args, wk, R, us, per, hot_us, step_bytes, runners, st, timing):
    """The dense draft layer's line: the step (attention + dense SwiGLU, every weight byte
    once) and, beside it, the context-K/V store of the workload's context rows."""
    d, w = wk["dims"], wk["workload"]
    ctx_us = None
    if runners[0].ctx is not None:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(st):
            runners[0].context_kv(stream=st)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            runners[0].context_kv(stream=st)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(st):
            for _ in range(5):
                g.replay()
            e0.record(st)
            for _ in range(50):
                g.replay()
            e1.record(st)
        torch.cuda.synchronize()
        ctx_us = e0.elapsed_time(e1) * 1e3 / 50
    out = {
        "metric": "µs per dense draft layer-step (b=8 verify) + achieved HBM GB/s vs peak",
        "value": round(us, 3), "unit": "us", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": False,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "b": w.b, "hidden": d["hidden"], "dense_inter": w.dense_inter,
                   "context": int(wk["layers"][0]["seq_lens"].sum()), "rotation_copies": R},
        "step_bytes": int(step_bytes),
        "step_GBps": round(step_bytes / (us * 1e-6) / 1e9, 1),
        "step_frac_hbm": round(step_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "us_p10_p50_p90": [round(float(np.percentile(per, q)), 3) for q in (10, 50, 90)],
        **timing,
        "hot_cache_us": round(hot_us, 3),
        "roofline": {"bound": "hbm", "kernel": "whole dense layer step", "unit": "GB/s",
                     "achieved": round(step_bytes / (us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBPS,
                     "frac": round(step_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "traffic": None},
        "context_kv_us": None if ctx_us is None else round(ctx_us, 3),
        "context_kv_rows": None if runners[0].ctx is None else int(runners[0].ctx["states"].shape[0]),
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="h4096_b8_ctx8k")
    ap.add_argument("--copies", type=int, default=0,
                    help="rotation copies (0: auto: divides --steps, >= 1 GB)")
    ap.add_argument("--roofline-iters", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported (the layer step "
              "is measured on one GPU's share of a sharded layer)", file=sys.stderr)
        sys.exit(2)

    from speculative_verify_decode_amd import binding as B
    from speculative_verify_decode_amd import synth
    from speculative_verify_decode_amd.runner import StepRunner

    B.lib()                                   # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    t0 = time.time()
    wk = synth.make_workload(args.workload)
    print(f"[bench] generated {args.workload} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    # A step is one layer step, or for a workload with a draft head the whole chain (every
    # layer, the final boundary and the head).
    chain = wk.get("head") is not None
    H = wk["dims"]["hidden"]

    def make_runner():
        r = StepRunner(wk, dev)
        r.chain_bufs = [torch.empty(wk["workload"].b, H, dtype=torch.float32, device=dev)
                        for _ in r.layers]
        r.pool = r.pooled_buf()
        return r

    dense = wk["workload"].dense_inter > 0

    # The timed layer step is sd_layer_step (unpooler included, input given as the unpooled
    # branch).  pooled_step_us times sd_layer_step_pooled on the same copies, as in a stack:
    # its input boundary gathers the previous layer's expert outputs and it leaves its own
    # unpooled.  Its pooled input is the same branch in pooled form (pool_from_branch), so it
    # routes to the same experts as the timed step.
    def pool_from_branch(r):
        """r's unpooled input branch as a pooled one: row t in slot t k with weight 1, the
        row's other slots zero with weight 0, so the gather reproduces it exactly."""
        k, b = wk["dims"]["top_k"], r.b
        y, rt = r.pool["y"], r.pool["route_t"]
        y.zero_()
        y.view(b, k, H)[:, 0].copy_(r.act["branch_in"])
        rt["topk_w"].zero_()
        rt["topk_w"].view(b, k)[:, 0] = 1.0
        rt["slot_of"].copy_(torch.arange(b * k, device=dev).view(rt["slot_of"].shape))

    def run_step(r, sb, stream=None, pool=False):
        if chain:
            r.chain(sb, r.act["branch_in"], r.chain_bufs, with_tau=False, stream=stream)
        elif dense:
            r.dense_step(0, sb, stream=stream)
        elif pool:
            r.layer_step_pooled(0, sb, r.pool, r.pool, stream=stream)
        else:
            r.layer_step(0, sb, r.act["branch_in"], stream=stream)

    # first copy: eager layer steps to learn the routing (touched experts) and the byte count
    r0 = make_runner()
    s = r0.act["stream"].clone()
    u = r0.act["branch_in"]
    counts_per_layer = []
    for i in range(len(r0.layers) if chain else 1):
        if dense:
            counts_per_layer.append(np.zeros(wk["dims"]["n_experts"], dtype=np.int64))
            break
        u = r0.layer_step(i, s, u, branch_out=r0.chain_bufs[i])
        torch.cuda.synchronize()
        counts_per_layer.append(r0.route_t["expert_counts"].cpu().numpy())
    counts = counts_per_layer[0]
    step_bytes, expert_bytes = algorithmic_bytes(wk, counts_per_layer)
    # every replay is timed on its own (inputs are restored between replays), so the fixed
    # cost of starting a replay is shared by the R steps of one graph; R divides K, so every
    # timed replay is a whole R-step graph
    R, n_rest = rotation_copies(args.steps, step_bytes, args.copies)
    runners = [r0] + [make_runner() for _ in range(R - 1)]
    print(f"[bench] {R} rotation copies, {step_bytes / 1e6:.1f} MB algorithmic per step",
          file=sys.stderr, flush=True)

    # Every timed step sees the same inputs: a step updates its stream (and, pooled, its
    # pooled branch) in place, and an ever-growing stream would drift the routing and the
    # bytes a step moves, so each copy's inputs are restored from a snapshot between graph
    # replays, outside the timed intervals (events around each replay only).  Graphs run on
    # a side stream; one graph holds the R copies' steps back to back (as a serving graph
    # holds a model's consecutive layers).
    st = torch.cuda.Stream()
    streams = [r.act["stream"].clone() for r in runners]
    pooled = not chain and not dense
    with torch.cuda.stream(st):
        for r, sb in zip(runners, streams):
            run_step(r, sb, stream=st)      # warm (lazy module load)
            sb.copy_(r.act["stream"])
            if pooled:                      # warm the pooled form too
                run_step(r, sb, stream=st, pool=True)
                sb.copy_(r.act["stream"])
                pool_from_branch(r)
    torch.cuda.synchronize()
    snaps = []
    for r, sb in zip(runners, streams):
        sn = dict(s=sb.clone())
        if pooled:
            sn["y"] = r.pool["y"].clone()
            sn["rt"] = {k: v.clone() for k, v in r.pool["route_t"].items()}
        snaps.append(sn)

    def restore():
        for r, sb, sn in zip(runners, streams, snaps):
            sb.copy_(sn["s"])
            if pooled:
                r.pool["y"].copy_(sn["y"])
                for k, v in r.pool["route_t"].items():
                    v.copy_(sn["rt"][k])

    # bytes per step from each copy's own routing on exactly the timed inputs
    touched = [int((c > 0).sum()) for c in counts_per_layer] if chain else int((counts > 0).sum())
    if pooled:
        with torch.cuda.stream(st):
            for r, sb in zip(runners, streams):
                run_step(r, sb, stream=st)
        torch.cuda.synchronize()
        copy_counts = [r.route_t["expert_counts"].cpu().numpy() for r in runners]
        with torch.cuda.stream(st):
            restore()
        torch.cuda.synchronize()
        step_bytes = float(np.mean([algorithmic_bytes(wk, [c])[0] for c in copy_counts]))
        touched = [int((c > 0).sum()) for c in copy_counts]

    g_all = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all, stream=st):
        for r, sb in zip(runners, streams):
            run_step(r, sb, stream=st)
    g_rest = None
    if n_rest:  # only when K has no divisor in the copies' range: its last K % R steps
        g_rest = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_rest, stream=st):
            for r, sb in zip(runners[:n_rest], streams[:n_rest]):
                run_step(r, sb, stream=st)
    torch.cuda.synchronize()

    def timed_replays(graph, n):
        """Replays graph n times, inputs restored before each; us of each replay."""
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        with torch.cuda.stream(st):
            for e0_, e1_ in evs:
                restore()
                e0_.record(st)
                graph.replay()
                e1_.record(st)
        torch.cuda.synchronize()
        return np.array([a_.elapsed_time(b_) for a_, b_ in evs]) * 1e3

    # warm-up: W steps' worth of replays, and at least 3 (the first replays run slower)
    timed_replays(g_all, max(3, math.ceil(args.warmup / R)))
    K = args.steps
    n_all = K // R
    per_all = timed_replays(g_all, n_all) if n_all else np.zeros(0)
    rest = float(timed_replays(g_rest, 1)[0]) if g_rest is not None else 0.0
    us = (float(per_all.sum()) + rest) / K
    # percentiles of the per-step time over at least 10 whole replays (more replays than
    # the K timed steps hold are taken for these figures only)
    per = per_all / R
    if len(per) < 10:
        per = np.concatenate([per, timed_replays(g_all, 10 - len(per)) / R])
    timing = {"percentile_replays": int(len(per)),
              "timed_replays": {"steps_per_replay": R, "whole": n_all, "remainder_steps": n_rest},
              "hbm_read_ceiling": read_ceiling(dev)}

    # the pooled layer step (sd_layer_step_pooled) on the same copies and inputs
    pooled_us = None
    if pooled:
        # the maps the timed step left in each copy's route feed the roofline loop below
        plain_expert_bytes = [algorithmic_bytes(wk, [c])[1] for c in copy_counts]
        g_pool = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_pool, stream=st):
            for r, sb in zip(runners, streams):
                run_step(r, sb, stream=st, pool=True)
        torch.cuda.synchronize()
        timed_replays(g_pool, max(3, math.ceil(args.warmup / R)))
        pooled_us = float(timed_replays(g_pool, max(1, min(K, 200) // R)).mean()) / R

    # hot-cache number (copy 0, R steps per replay, inputs restored between replays),
    # labelled separately
    g_hot = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_hot, stream=st):
        for _ in range(R):
            run_step(runners[0], streams[0], stream=st)
    torch.cuda.synchronize()
    timed_replays(g_hot, 2)
    hot_us = float(timed_replays(g_hot, max(1, 50 // R)).mean()) / R

    # dominant kernels: the routed-expert GEMMs (sd_moe_experts_x16: k_moe_w13 then k_moe_w2,
    # the pair the layer step runs), timed live with HIP events on their launch stream,
    # rotating over the copies like the step; their input is a boundary's expert-input form
    # of the same rows
    d, b = wk["dims"], wk["workload"].b
    H = d["hidden"]
    if dense:
        print_dense(args, wk, R, us, per, hot_us, step_bytes, runners, st, timing)
        return
    y = torch.empty(b * d["top_k"], H, dtype=torch.float32, device=dev)
    x = []
    for r in runners:
        x16 = torch.empty(2, b, H, dtype=torch.float16, device=dev)
        hb = torch.empty(b, H, dtype=torch.bfloat16, device=dev)
        sb = r.act["stream"].clone()
        B.boundary_dualnorm(r.dims, b, sb, r.act["branch_in"], None, r.layers[0].t["g_post_prev"],
                            r.layers[0].t["g_pre_ffn"], hb, out16=x16)
        x.append(x16)
    torch.cuda.synchronize()
    n_it = args.roofline_iters
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(st):
        for i in range(10):
            r = runners[i % R]
            B.moe_experts_x16(r.dims, b, x[i % R], r.layers[0].moe_w, r.route, y, None, r.ws,
                              stream=st)
        e0.record(st)
        for i in range(n_it):
            r = runners[i % R]
            B.moe_experts_x16(r.dims, b, x[i % R], r.layers[0].moe_w, r.route, y, None, r.ws,
                              stream=st)
        e1.record(st)
    torch.cuda.synchronize()
    exp_us = e0.elapsed_time(e1) * 1e3 / n_it      # average per launch, back to back
    if pooled:  # each copy's own touched experts, in the loop's rotation
        expert_bytes = float(np.mean([plain_expert_bytes[i % R] for i in range(n_it)]))
    achieved = expert_bytes / (exp_us * 1e-6) / 1e9

    out = {
        "metric": ("µs per decode chain (every layer, final boundary, draft head) + achieved HBM "
                   "GB/s vs peak" if chain else
                   "µs per decode layer-step (b=8 verify) + achieved HBM GB/s vs peak"),
        "value": round(us, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "b": b, "hidden": d["hidden"],
                   "n_q_heads": d["n_q_heads"], "n_kv_heads": d["n_kv_heads"],
                   "head_dim": d["head_dim"], "experts": d["n_experts"], "top_k": d["top_k"],
                   "inter": d["inter"], "context": int(wk["layers"][0]["seq_lens"].sum()),
                   "touched_experts": touched,
                   "layers": len(counts_per_layer), "rotation_copies": R,
                   "layer_step": "chain" if chain else ("dense" if dense else "sd_layer_step")},
        "step_bytes": int(step_bytes),
        "step_GBps": round(step_bytes / (us * 1e-6) / 1e9, 1),
        "step_frac_hbm": round(step_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
        "tokens_per_s": round(b * 1e6 / us, 1),
        "pooled_step_us": None if pooled_us is None else round(pooled_us, 3),
        "us_p10_p50_p90": [round(float(np.percentile(per, q)), 3) for q in (10, 50, 90)],
        **timing,
        "hot_cache_us": round(hot_us, 3),
        "roofline": {"bound": "hbm",
                     "kernel": "routed-expert GEMMs (sd_moe_experts_x16: k_moe_w13 + k_moe_w2)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(args.workload),
                     "launch_us": round(exp_us, 3), "bytes_per_launch": int(expert_bytes)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on one layer step", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wk)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
