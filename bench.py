"""Benchmark of the blockwise ring-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--primary-only]
                    [--no-cpu-baseline]

Prints ONE JSON line.  The headline workload is the zigzag causal ring
prefill of one rank: seq 8192, cp 4 (8 chunks of 1024), rank 0 holding Q
chunks {0, 7}, 32 heads, d 128, bf16 with float32 accumulation.  A step is
one full ring sweep of that rank: 4 ring steps of one launch each, which
computes the (Q chunk, K/V chunk) pairs of the current block (7 FULL, 2 DIAG
and 7 SKIP pairs overall, merged in place) and copies the next K/V block
into the idle staging slot.
`value` is algorithmic causal-attention TFLOP/s: visible (q, k) pairs x
heads x (2 d_qk + 2 d_v) per sweep / time per sweep.  The K timed sweeps
are captured as one HIP graph (each sweep recomputes everything from the
same inputs) and replayed once between two synchronisations, after W
untimed sweeps.  Reported beside it under "launch": one graph per sweep
replayed K times, plain eager issue, and the same sweep with the staging
copies on a side stream (ring_stage_copy launches ordered by events).

Also reported in the same line (unless --primary-only): the long zigzag
prefill (rank 0 of cp=8 over 1M tokens), GQA decode over 8 sequence shards
(GB/s against HBM), the same decode over paged caches read through block
tables, segmented chunked prefill (MLA shape), a packed multi-request
(varlen) prefill, the all-gather-KV reorganisation gather, the tiny fp32
non-causal ring (a correctness workload, timed for completeness) and a
standalone LSE merge, each with the roofline of its dominant kernel, plus
the CPU oracle timed on the host (all its threads, and on one thread).
"""

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_F32_VALU_TFLOPS = 157.3   # MI355X fp32 vector ALU (published, packed FMA)
METRIC = "causal attn TFLOP/s per ring-step prefill + decode GB/s, % of roofline"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--primary-only", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default="", help="comma list of secondary workloads to run")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    p.add_argument("--sweep-only", type=int, default=0, metavar="K",
                   help="only replay the zigzag sweep graph K times (for counter passes)")
    p.add_argument("--decode-only", type=int, default=0, metavar="K",
                   help="only run the sharded decode kernel K times (for counter passes)")
    p.add_argument("--merge-only", type=int, default=0, metavar="K",
                   help="only run the standalone LSE merge K times (for counter passes)")
    p.add_argument("--long-step-only", type=int, default=0, metavar="K",
                   help="only run one FULL ring-step launch of the 1M-token prefill K times")
    return p.parse_args()


def sweep_only(reps):
    """Replays of the headline sweep alone, so per-dispatch counters average
    exactly over the sweep's launches (one of each per replay)."""
    import torch
    import workloads
    w = workloads.zigzag_setup(2)
    graph = w["ring"].capture(w["q_local"], w["o"], w["lse"])
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    print(json.dumps({"sweep_replays": reps, "launches_per_sweep": len(zigzag_launches(w))}),
          flush=True)


def decode_only(reps):
    """The sharded GQA decode kernel alone, K launches (no merge), so
    per-dispatch counters and durations cover exactly that kernel."""
    import torch
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.decode_setup()
    o_parts = torch.empty((w["n_shards"], w["B"], w["hq"], w["d"]), device="cuda")
    lse_parts = torch.empty((w["n_shards"], w["B"], w["hq"]), device="cuda")
    for _ in range(reps):
        ra.split_kv_decode(w["q"], w["ks"], w["vs"], shard_lens=w["lens"], o_parts=o_parts,
                           lse_parts=lse_parts)
    torch.cuda.synchronize()
    print(json.dumps({"decode_launches": reps, "kernel_bytes": decode_kernel_bytes(w)}), flush=True)


def decode_kernel_bytes(w):
    """Algorithmic bytes of one decode launch: K and V once, Q, partials written."""
    return w["kv_bytes"] + w["q"].numel() * 2 + w["n_shards"] * w["B"] * w["hq"] * (w["d"] + 1) * 4


def calibrate_copy():
    """A plain copy of known size, for scaling the HBM byte counters."""
    import torch
    n = 1 << 28                      # 2^28 float32 = 1 GiB
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(5):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "device-to-device copy", "bytes_read": n * 4,
                      "bytes_written": n * 4, "launches": 5}), flush=True)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_launch_stats(launch_list, reps):
    """Average duration (ms) of the attention kernel launches of one step.

    The step's kernel launches (no copies) are captured back to back in a HIP
    graph and replayed `reps` times between two HIP events on the replay
    stream, so the figure is kernel time plus the dispatch gaps between
    consecutive kernels -- no host overhead, no event per launch.
    """
    import torch
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for fn in launch_list:          # warm: first launch outside the graph
            fn()
        with torch.cuda.graph(graph, stream=stream):
            for fn in launch_list:
                fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        graph.replay()
        s.record()
        for _ in range(reps):
            graph.replay()
        e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / (reps * len(launch_list))


def zigzag_launches(w, cls_filter=None):
    """The ring_attn_step launches of one zigzag sweep, exactly as the ring issues
    them (collected from the sweep itself; K/V slots hold the staged data)."""
    import torch
    launches = []
    w["ring"].run(w["q_local"], w["o"], w["lse"],
                  on_launch=lambda t, qi, kj, cls, fn: launches.append((cls, fn)))
    torch.cuda.synchronize()
    # SKIP pairs launch no attention kernel
    return [fn for cls, fn in launches if cls != 2 and (cls_filter is None or cls == cls_filter)]


def graph_upload(graph):
    """Upload an instantiated graph to the device ahead of its first launch
    (hipGraphUpload), so the timed replay does not pay the one-time upload."""
    import ctypes
    import torch
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")      # the runtime torch has loaded
        rc = hip.hipGraphUpload(ctypes.c_void_p(graph.raw_cuda_graph_exec()),
                                ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    except (OSError, AttributeError, RuntimeError):
        rc = -1
    torch.cuda.synchronize()
    return rc == 0


def time_steps(step_fn, steps, warmup):
    import torch
    for _ in range(warmup):
        step_fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step_fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def profiled_traffic(summary, source, field="traffic_bytes_per_launch"):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the kernel source changed after the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        text = open(os.path.join(root, "profiles", summary)).read()
        src = open(os.path.join(root, "ring_attention_02_amd", "csrc", source), "rb").read()
    except OSError:
        return None
    sha = hashlib.sha256(src).hexdigest()[:16]
    key = f"kernel source sha256 prefix ({source})"
    fields = dict(line.split(": ", 1) for line in text.splitlines() if ": " in line and
                  line.split(": ", 1)[0] in (key, field))
    if fields.get(key, "").strip() != sha or field not in fields:
        return None
    return int(float(fields[field]))


def roofline_entry(bound, achieved, peak, unit, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def zigzag_bench(cfg_id, steps, warmup, use_graph=True):
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.zigzag_setup(cfg_id)
    ring, q, o, lse = w["ring"], w["q_local"], w["o"], w["lse"]
    eager = time_steps(lambda: ring.run(q, o, lse), steps, warmup)
    sec = eager
    side_sec = per_graph_sec = None
    if use_graph:
        # one graph per sweep, replayed once per step
        graph = ring.capture(q, o, lse)
        per_graph_sec = time_steps(graph.replay, steps, warmup)
        sec = per_graph_sec
        if cfg_id == 2:
            # the same sweep with the staging copies on a side stream
            side_graph = ring.capture(q, o, lse, side_copies=True)
            side_sec = time_steps(side_graph.replay, steps, warmup)
            del side_graph
            # the timed steps as one graph of `steps` sweeps: one graph launch
            # for the whole job (each sweep still recomputes everything)
            job = ring.capture(q, o, lse, sweeps=steps)
            graph_upload(job)
            for _ in range(warmup):
                graph.replay()
            sec = time_steps(job.replay, 1, 0) / steps
            del job
    launches = zigzag_launches(w)
    reps = max(2, min(steps, 20)) if cfg_id == 2 else 1
    mean_ms = kernel_launch_stats(launches, reps)
    flops_per_launch = w["flops"] / len(launches)
    achieved = flops_per_launch / (mean_ms * 1e-3) / 1e12
    full_ms = kernel_launch_stats(zigzag_launches(w, ra.FULL), reps)
    diag_ms = kernel_launch_stats(zigzag_launches(w, ra.DIAG), reps)
    return w, sec, dict(mean_launch_ms=mean_ms, launches_per_step=len(launches),
                        flops_per_launch=flops_per_launch, achieved_tflops=achieved,
                        full_ms=full_ms, diag_ms=diag_ms, eager_ms=eager * 1e3,
                        side_ms=None if side_sec is None else side_sec * 1e3,
                        per_graph_ms=None if per_graph_sec is None else per_graph_sec * 1e3)


def tiny_bench(steps, warmup):
    """C1: the fp32 non-causal ring, 512 tokens in 4 blocks of 128, 4 heads,
    d 64: 16 ring-step launches and one 4-part LSE merge per sweep, issued
    eagerly (a correctness workload: the figure is mostly launch cost)."""
    import torch
    import ring_attention_02_amd as ra
    import workloads
    from seeded_inputs import CONFIGS, Q_ID, K_ID, V_ID
    c = CONFIGS[1]
    shape = (c["batch"], c["seq"], c["heads"], c["d"])
    q, k, v = (workloads.host_tensor(1, t, 0, shape, torch.float32) for t in (Q_ID, K_ID, V_ID))
    flops = c["batch"] * c["seq"] * c["seq"] * c["heads"] * 4 * c["d"]
    sec = time_steps(lambda: ra.noncausal_ring_sweep(q, k, v, c["n_blocks"]), steps, warmup)
    return flops, sec


def decode_bench(steps, warmup, paged=False):
    import torch
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.decode_paged_setup() if paged else workloads.decode_setup()
    o_parts = torch.empty((w["n_shards"], w["B"], w["hq"], w["d"]), device="cuda")
    lse_parts = torch.empty((w["n_shards"], w["B"], w["hq"]), device="cuda")
    o = torch.empty((w["B"], w["hq"], w["d"]), device="cuda")
    lse = torch.empty((w["B"], w["hq"]), device="cuda")

    def decode():
        if paged:
            ra.split_kv_decode_paged(w["q"], w["kp"], w["vp"], w["tables"], w["lens"],
                                     o_parts=o_parts, lse_parts=lse_parts)
        else:
            ra.split_kv_decode(w["q"], w["ks"], w["vs"], shard_lens=w["lens"], o_parts=o_parts,
                               lse_parts=lse_parts)

    def step():
        decode()
        ra.lse_merge(o_parts, lse_parts, o_out=o, lse_out=lse)

    sec = time_steps(step, steps, warmup)
    # the decode kernel alone, HIP events on its stream
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    durs = []
    for _ in range(max(3, min(steps, 10))):
        s.record()
        decode()
        e.record()
        torch.cuda.synchronize()
        durs.append(s.elapsed_time(e))
    kern_ms = float(np.mean(durs))
    kern_bytes = decode_kernel_bytes(w)
    return w, sec, dict(kernel_ms=kern_ms, kernel_bytes=kern_bytes,
                        kernel_gbs=kern_bytes / (kern_ms * 1e-3) / 1e9)


def segmented_bench(steps, warmup):
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.segmented_setup()
    launches = []

    def collect(step, qi, kj, cls, fn):
        launches.append(fn)

    def run(cb=None):
        ra.segmented_prefill(w["q"], w["k"], w["v"], w["o"], w["lse"], q_pos0=w["q_pos0"],
                             segment=w["segment"], on_launch=cb)

    sec = time_steps(run, steps, warmup)
    run(collect)
    mean_ms = kernel_launch_stats(launches, 1)
    achieved = w["flops"] / len(launches) / (mean_ms * 1e-3) / 1e12
    return w, sec, dict(mean_launch_ms=mean_ms, launches_per_step=len(launches),
                        achieved_tflops=achieved)


def varlen_bench(steps, warmup):
    import torch
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.varlen_setup()

    def step():
        ra.ring_attn_step_varlen(w["q"], w["k"], w["v"], w["cu"], w["cu"], w["pos"], w["pos"],
                                 o=w["o"], lse=w["lse"], causal=True)

    sec = time_steps(step, steps, warmup)
    ms = kernel_launch_stats([step], max(2, min(steps, 10)))
    return w, sec, dict(mean_launch_ms=ms, achieved_tflops=w["flops"] / (ms * 1e-3) / 1e12)


def reorg_bench(steps, warmup):
    import torch
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.reorg_setup()
    ok = torch.empty_like(w["gk"])
    ov = torch.empty_like(w["gv"])

    def step():
        ra.gather_rows(w["gk"], w["idx"], dst=ok)
        ra.gather_rows(w["gv"], w["idx"], dst=ov)

    sec = time_steps(step, steps, warmup)
    return w, sec


def merge_setup():
    import torch
    rows, dv, n = 131072 * 64, 128, 2       # the long prefill's rows, two partials
    o_parts = torch.randn((n, rows, dv), device="cuda")
    lse_parts = torch.randn((n, rows), device="cuda")
    o = torch.empty((rows, dv), device="cuda")
    lse = torch.empty((rows,), device="cuda")
    nbytes = (n * rows * (dv + 1) + rows * (dv + 1)) * 4   # parts read, result written
    return o_parts, lse_parts, o, lse, nbytes


def merge_bench(steps, warmup):
    import ring_attention_02_amd as ra
    o_parts, lse_parts, o, lse, nbytes = merge_setup()
    sec = time_steps(lambda: ra.lse_merge(o_parts, lse_parts, o_out=o, lse_out=lse), steps, warmup)
    return sec, nbytes


def long_step_only(reps):
    """One FULL ring step of the 1M-token zigzag prefill (rank 0, cp 8): the
    launch that attends the tail query part to a whole staged block and
    forwards the next one, K times, for counter passes."""
    import torch
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.zigzag_setup(4)
    fn = zigzag_launches(w, ra.FULL)[0]
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    print(json.dumps({"long_step_launches": reps}), flush=True)


def merge_only(reps):
    """The standalone LSE merge alone, K launches, for counter passes."""
    import torch
    import ring_attention_02_amd as ra
    o_parts, lse_parts, o, lse, nbytes = merge_setup()
    for _ in range(reps):
        ra.lse_merge(o_parts, lse_parts, o_out=o, lse_out=lse)
    torch.cuda.synchronize()
    print(json.dumps({"merge_launches": reps, "bytes_per_launch": nbytes}), flush=True)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host, on a bounded sample of the workload
# ---------------------------------------------------------------------------

def cpu_baseline(w):
    import oracle
    import workloads
    k = w["k_full"][0].float().cpu().numpy().astype(np.float64)
    v = w["v_full"][0].float().cpu().numpy().astype(np.float64)
    q = w["q_local"][0].float().cpu().numpy().astype(np.float64)
    q_pos = np.asarray(w["local"], dtype=np.int64)
    heads_done, pairs_done, t_used = 0, 0, 0.0
    budget = 15.0
    for h in range(w["hq"]):
        t0 = time.perf_counter()
        oracle.attention_ref(q[None, :, h:h + 1], k[None, :, h:h + 1], v[None, :, h:h + 1],
                             q_pos, np.arange(k.shape[0]), causal=True)
        t_used += time.perf_counter() - t0
        heads_done += 1
        if t_used > budget:
            break
    flops = w["pairs"] * heads_done * (2 * w["d"] + 2 * w["d"])
    out = {"value": round(flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
           "kind": "oracle",
           "sample": f"rank-0 local queries (2048 tokens) x all 8192 keys for {heads_done} of "
                     f"{w['hq']} heads, float64 numpy, {t_used:.1f} s"}
    # the same oracle on one thread: one head of this workload, and the whole
    # tiny fp32 ring workload (512 tokens, 4 heads, d 64, no mask)
    from threadpoolctl import threadpool_limits
    from seeded_inputs import CONFIGS, Q_ID, K_ID, V_ID
    c1 = CONFIGS[1]
    shape1 = (c1["batch"], c1["seq"], c1["heads"], c1["d"])
    import torch
    q1, k1, v1 = (workloads.host_tensor(1, t, 0, shape1, torch.float32).cpu().numpy()
                  for t in (Q_ID, K_ID, V_ID))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        oracle.attention_ref(q[None, :, :1], k[None, :, :1], v[None, :, :1], q_pos,
                             np.arange(k.shape[0]), causal=True)
        t_head = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.attention_ref(q1, k1, v1, causal=False)
        t_c1 = time.perf_counter() - t0
    f_head = w["pairs"] * (2 * w["d"] + 2 * w["d"])
    f_c1 = c1["batch"] * c1["seq"] * c1["seq"] * c1["heads"] * 4 * c1["d"]
    out["single_thread"] = {
        "zigzag_one_head": {"value": round(f_head / t_head / 1e12, 6), "unit": "TFLOP/s",
                            "seconds": round(t_head, 3)},
        "tiny_noncausal_ring_f32": {"value": round(f_c1 / t_c1 / 1e12, 6), "unit": "TFLOP/s",
                                    "seconds": round(t_c1, 4)}}
    return out



def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is one "
              f"GPU's share of the ring and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import torch
    import ring_attention_02_amd  # noqa: F401  (fails loudly if the library is missing)
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.sweep_only:
        sweep_only(args.sweep_only)
        return
    if args.decode_only:
        decode_only(args.decode_only)
        return
    if args.merge_only:
        merge_only(args.merge_only)
        return
    if args.long_step_only:
        long_step_only(args.long_step_only)
        return

    log("C2: zigzag causal prefill, seq 8192, cp 4, rank 0")
    w2, sec2, l2 = zigzag_bench(2, args.steps, args.warmup)
    value = w2["flops"] / sec2 / 1e12
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec2 * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "zigzag causal ring prefill, one rank's share: seq 8192, cp 4 "
                               "(8 chunks of 1024), rank 0 holds Q chunks {0,7}, 32 heads, "
                               "d 128, bf16",
                   "global_batch": 1, "seq_len": 8192, "parallelism": "cp4 ring emulated on 1 GPU",
                   "flops_per_step": w2["flops"]},
        "roofline": roofline_entry("mfma", l2["achieved_tflops"], PEAK_BF16_TFLOPS, "TFLOP/s",
                                   profiled_traffic("attn_step_bf16_zigzag_seq8192_cp4.md",
                                                    "attn_step.hip")),
        "kernel": {"name": "attn_step_bf16_kernel<128,128>",
                   "mean_launch_ms": round(l2["mean_launch_ms"], 5),
                   "launches_per_step": l2["launches_per_step"],
                   "full_pair_ms": round(l2["full_ms"], 5), "diag_pair_ms": round(l2["diag_ms"], 5),
                   "timing": "HIP-graph replay of the step's kernels back to back, HIP events"},
        "launch": {"mode": "the K timed sweeps captured as one HIP graph and replayed once "
                           "(one launch per ring step, next block's copy inside it)",
                   "one_graph_per_sweep_ms_per_step": round(l2["per_graph_ms"], 4),
                   "eager_ms_per_step": round(l2["eager_ms"], 4),
                   "side_stream_copies_ms_per_step": round(l2["side_ms"], 4)},
    }
    del w2["ring"]
    if not args.no_cpu_baseline:
        log("CPU baseline (oracle on host)")
        out["cpu_baseline"] = cpu_baseline(w2)
    del w2
    torch.cuda.empty_cache()

    if not args.primary_only:
        only = set(filter(None, args.only.split(",")))
        sec = {}
        if not only or "c4" in only:
            log("C4: zigzag causal prefill, 1M tokens, cp 8, rank 0")
            w4, s4, l4 = zigzag_bench(4, max(1, min(args.steps, 2)), 1, use_graph=False)
            sec["long_prefill_1M_cp8"] = {
                "value": round(w4["flops"] / s4 / 1e12, 3), "unit": "TFLOP/s",
                "ms_per_step": round(s4 * 1e3, 3), "flops_per_step": w4["flops"],
                "roofline": roofline_entry("mfma", l4["achieved_tflops"], PEAK_BF16_TFLOPS, "TFLOP/s"),
                "full_pair_ms": round(l4["full_ms"], 3), "diag_pair_ms": round(l4["diag_ms"], 3),
                "full_step_traffic_bytes": profiled_traffic(
                    "attn_step_bf16_long_prefill_1M_cp8_full_step.md", "attn_step.hip",
                    field="full_step_traffic_bytes_per_launch")}
            del w4
            torch.cuda.empty_cache()
        if not only or "c3" in only:
            log("C3: GQA decode, 64 x 131072 context, 8 shards")
            w3, s3, l3 = decode_bench(max(3, min(args.steps, 10)), 2)
            sec["decode_gqa_8_shards"] = {
                "value": round(w3["bytes"] / s3 / 1e9, 1), "unit": "GB/s",
                "ms_per_step": round(s3 * 1e3, 4), "bytes_per_step": w3["bytes"],
                "roofline": roofline_entry("hbm", l3["kernel_gbs"], PEAK_HBM_GBS, "GB/s",
                                           profiled_traffic("decode_bf16_gqa_8shards.md", "decode.hip")),
                "kernel_ms": round(l3["kernel_ms"], 4)}
            del w3
            torch.cuda.empty_cache()
        if not only or "c3p" in only:
            log("C3 paged: the same decode through per-request block tables")
            w3p, s3p, l3p = decode_bench(max(3, min(args.steps, 10)), 2, paged=True)
            sec["decode_gqa_8_shards_paged"] = {
                "value": round(w3p["bytes"] / s3p / 1e9, 1), "unit": "GB/s",
                "ms_per_step": round(s3p * 1e3, 4), "bytes_per_step": w3p["bytes"],
                "roofline": roofline_entry("hbm", l3p["kernel_gbs"], PEAK_HBM_GBS, "GB/s"),
                "kernel_ms": round(l3p["kernel_ms"], 4)}
            del w3p
            torch.cuda.empty_cache()
        if not only or "c5" in only:
            log("C5: segmented chunked prefill, MLA shape")
            w5, s5, l5 = segmented_bench(max(2, min(args.steps, 5)), 1)
            sec["segmented_prefill_mla"] = {
                "value": round(w5["flops"] / s5 / 1e12, 3), "unit": "TFLOP/s",
                "ms_per_step": round(s5 * 1e3, 3), "flops_per_step": w5["flops"],
                "roofline": roofline_entry("mfma", l5["achieved_tflops"], PEAK_BF16_TFLOPS, "TFLOP/s"),
                "mean_launch_ms": round(l5["mean_launch_ms"], 4)}
            del w5
            torch.cuda.empty_cache()
        if not only or "varlen" in only:
            log("varlen: 16 packed requests (512..8192 tokens), self-causal, GQA 32/8, d 128")
            w7, s7, l7 = varlen_bench(max(3, min(args.steps, 10)), 2)
            sec["varlen_packed_prefill"] = {
                "value": round(w7["flops"] / s7 / 1e12, 3), "unit": "TFLOP/s",
                "ms_per_step": round(s7 * 1e3, 4), "flops_per_step": w7["flops"],
                "tokens": int(w7["cu"][-1]),
                "roofline": roofline_entry("mfma", l7["achieved_tflops"], PEAK_BF16_TFLOPS, "TFLOP/s"),
                "mean_launch_ms": round(l7["mean_launch_ms"], 4)}
            del w7
            torch.cuda.empty_cache()
        if not only or "reorg" in only:
            log("reorg_kvcache: all-gathered K/V of 135,168 tokens (4 requests, 8 devices) to request order")
            w8, s8 = reorg_bench(max(3, min(args.steps, 10)), 2)
            sec["reorg_kvcache_gather"] = {
                "value": round(w8["bytes"] / s8 / 1e9, 1), "unit": "GB/s",
                "ms_per_step": round(s8 * 1e3, 4), "bytes_per_step": w8["bytes"],
                "roofline": roofline_entry("hbm", w8["bytes"] / s8 / 1e9, PEAK_HBM_GBS, "GB/s")}
            del w8
            torch.cuda.empty_cache()
        if not only or "c1" in only:
            log("C1: tiny non-causal ring, fp32, 512 tokens in 4 blocks")
            f1, s1 = tiny_bench(max(10, args.steps), 5)
            sec["tiny_noncausal_ring_f32"] = {
                "value": round(f1 / s1 / 1e12, 4), "unit": "TFLOP/s", "ms_per_step": round(s1 * 1e3, 4),
                "flops_per_step": f1,
                "roofline": roofline_entry("alu", f1 / s1 / 1e12, PEAK_F32_VALU_TFLOPS, "TFLOP/s"),
                "note": "correctness workload: 16 launches and one merge per sweep, issued eagerly"}
        if not only or "merge" in only:
            log("lse_merge: 2 partials x 8.4M rows x 128")
            s6, b6 = merge_bench(max(5, args.steps), 2)
            sec["lse_merge_2x8M"] = {
                "value": round(b6 / s6 / 1e9, 1), "unit": "GB/s", "ms_per_step": round(s6 * 1e3, 4),
                "roofline": roofline_entry("hbm", b6 / s6 / 1e9, PEAK_HBM_GBS, "GB/s",
                                           profiled_traffic("lse_merge_2x8M.md", "lse_merge.hip"))}
        out["secondary"] = sec
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
