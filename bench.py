"""Benchmark of the blockwise ring-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--primary-only]
                    [--no-cpu-baseline]

Prints ONE JSON line.  The headline workload is the long zigzag causal ring
prefill of one rank: a 1,048,576-token sequence at cp 8 (16 chunks of
65,536), rank 0 holding Q chunks {0, 15} (131,072 local queries), 64 query
heads over 8 kv heads, d 128, bf16 with float32 accumulation.  A step is one
full ring sweep of that rank: 8 ring steps of one launch each, which compute
the (Q chunk, K/V chunk) pairs of the block the rank holds (15 FULL, 2 DIAG
and 15 SKIP pairs overall, merged in place) and copy the next K/V block
into the idle staging slot.  W untimed sweeps, then exactly K timed sweeps
between two device synchronisations.
`value` is algorithmic causal-attention TFLOP/s: visible (q, k) pairs x
heads x (2 d_qk + 2 d_v) per sweep / time per sweep.  The roofline entry
averages the ring-step kernel's launches of the timed sweeps, each timed
with HIP events on the stream it is launched on.

Also reported in the same line (unless --primary-only): the short zigzag
prefill (rank 0 of cp 4 over 8192 tokens, with its copy/compute overlap),
GQA decode over 8 sequence shards (GB/s against HBM), the same decode over
paged caches read through block tables, segmented chunked prefill (MLA
shape), a packed multi-request (varlen) prefill, the all-gather-KV
reorganisation gather, the tiny fp32 non-causal ring (a correctness
workload, timed for completeness) and a standalone LSE merge, each with the
roofline of its dominant kernel; and the CPU oracle timed on the host on a
bounded sample of the headline workload (extrapolated by visible pairs),
with the same for the other workloads beside it.
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
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
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
    p.add_argument("--long-sweep-only", type=int, default=0, metavar="K",
                   help="only run K sweeps of the 1M-token prefill (for counter passes)")
    p.add_argument("--paged-only", type=int, default=0, metavar="K",
                   help="only run the paged decode kernel K times (for counter passes)")
    p.add_argument("--segmented-only", type=int, default=0, metavar="K",
                   help="only run the chunked prefill (MLA shape) K times (for counter passes)")
    p.add_argument("--varlen-only", type=int, default=0, metavar="K",
                   help="only run the packed 16-request prefill launch K times (for counter passes)")
    p.add_argument("--reorg-only", type=int, default=0, metavar="K",
                   help="only run the reorganisation gather (K then V) K times (for counter passes)")
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


def paged_only(reps):
    """The paged decode kernel alone, K launches (no merge)."""
    import torch
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.decode_paged_setup()
    o_parts = torch.empty((w["n_shards"], w["B"], w["hq"], w["d"]), device="cuda")
    lse_parts = torch.empty((w["n_shards"], w["B"], w["hq"]), device="cuda")
    for _ in range(reps):
        ra.split_kv_decode_paged(w["q"], w["kp"], w["vp"], w["tables"], w["lens"], o_parts=o_parts,
                                 lse_parts=lse_parts)
    torch.cuda.synchronize()
    print(json.dumps({"paged_decode_launches": reps, "kernel_bytes": decode_kernel_bytes(w)}), flush=True)


def segmented_only(reps):
    """The chunked prefill (MLA shape) alone, K times (5 ring-step launches each)."""
    import torch
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.segmented_setup()
    for _ in range(reps):
        ra.segmented_prefill(w["q"], w["k"], w["v"], w["o"], w["lse"], q_pos0=w["q_pos0"], segment=w["segment"])
    torch.cuda.synchronize()
    print(json.dumps({"segmented_runs": reps, "bytes_per_run": segmented_bytes(w)}), flush=True)


def segmented_bytes(w):
    """Algorithmic bytes of one chunked prefill: Q once per launch (up to four
    segments each), every K/V byte once, O and LSE written by the first launch
    and read and written by each later one."""
    n_seg = -(-w["skv"] // w["segment"])
    launches = -(-n_seg // 4)
    q = w["sq"] * w["h"] * w["dqk"] * 2
    kv = w["skv"] * w["h"] * (w["dqk"] + w["dv"]) * 2
    ol = w["sq"] * w["h"] * (w["dv"] + 1) * 4
    return launches * q + kv + ol + (launches - 1) * 2 * ol


def varlen_only(reps):
    """The packed 16-request prefill launch alone, K times."""
    import torch
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.varlen_setup()
    for _ in range(reps):
        ra.ring_attn_step_varlen(w["q"], w["k"], w["v"], w["cu"], w["cu"], w["pos"], w["pos"],
                                 o=w["o"], lse=w["lse"], causal=True)
    torch.cuda.synchronize()
    print(json.dumps({"varlen_launches": reps, "bytes_per_launch": varlen_bytes(w)}), flush=True)


def varlen_bytes(w):
    """Algorithmic bytes of the packed launch: Q, K and V read once, O and LSE written."""
    t = int(w["cu"][-1])
    return t * (w["hq"] * w["d"] * 2 + 2 * w["hkv"] * w["d"] * 2 + w["hq"] * (w["d"] + 1) * 4)


def reorg_only(reps):
    """The reorganisation gather alone: K then V rows, K times."""
    import torch
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.reorg_setup()
    ok = torch.empty_like(w["gk"])
    ov = torch.empty_like(w["gv"])
    for _ in range(reps):
        ra.gather_rows(w["gk"], w["idx"], dst=ok)
        ra.gather_rows(w["gv"], w["idx"], dst=ov)
    torch.cuda.synchronize()
    print(json.dumps({"gather_pairs": reps, "bytes_per_pair": w["bytes"]}), flush=True)


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


def build_digest(source):
    """The build digest of a kernel source file (its bytes and device flags),
    as the package's build script computes it."""
    import importlib.util
    root = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location(
        "_ringattn_build", os.path.join(root, "ring_attention_02_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.build_digest(source)


def profiled_traffic(summary, source, field="traffic_bytes_per_launch"):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    when the kernel's source or its compile flags changed after the counters
    were taken."""
    root = os.path.dirname(os.path.abspath(__file__))
    try:
        text = open(os.path.join(root, "profiles", summary)).read()
        sha = build_digest(source)
    except OSError:
        return None
    key = f"kernel build sha256 prefix ({source})"
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

def graph_ms(fns, sweeps, reps=3):
    """Milliseconds per call sequence: `sweeps` copies of the launch list fns
    captured back to back as one HIP graph (uploaded before its first launch),
    replayed `reps` times between two HIP events on the replay stream."""
    import torch
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for fn in fns:                  # warm: first launch outside the graph
            fn()
        with torch.cuda.graph(graph, stream=stream):
            for _ in range(sweeps):
                for fn in fns:
                    fn()
    torch.cuda.synchronize()
    graph_upload(graph)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        graph.replay()
        s.record()
        for _ in range(reps):
            graph.replay()
        e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / (reps * sweeps)


def long_headline(steps, warmup):
    """The 1M-token zigzag sweep of rank 0: W untimed sweeps, then exactly K
    timed sweeps (one launch per ring step, issued from the host; at ~0.25 s
    per launch issue cost is nil).  Every launch of the timed sweeps is
    bracketed by HIP events on its own stream (the current stream, which the
    binding launches on)."""
    import torch
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.zigzag_setup(4)
    ring, q, o, lse = w["ring"], w["q_local"], w["o"], w["lse"]
    for _ in range(warmup):
        ring.run(q, o, lse)
    events = []

    def timed(t, qi, kj, cls, fn):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        events.append((cls, s, e))

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ring.run(q, o, lse, on_launch=timed)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    durs = [(cls, s.elapsed_time(e)) for cls, s, e in events]
    launches = len(durs) // steps
    mean_ms = float(np.mean([d for _, d in durs]))
    full_ms = float(np.mean([d for c, d in durs if c == ra.FULL]))
    diag = [d for c, d in durs if c == ra.DIAG]
    flops_per_launch = w["flops"] / launches
    # The ring transfer's share: the sweep's forwarded blocks copied alone
    # (ring_stage_copy launches, one HIP graph), against the sweep.
    copies = [lambda u=u: ra.stage_copy(ring.forward_pairs(u)) for u in range(1, ring.cp)]
    t_copy_ms = graph_ms(copies, 1, 3)
    # one sweep of every other rank's share (same K/V, its own Q parts and
    # ring order) after one untimed sweep of it, timed like the headline's:
    # the zigzag partition gives every rank the same visible pairs in other
    # step shapes
    per_rank = [sec * 1e3]
    for r in range(1, ring.cp):
        wr = workloads.zigzag_setup(4, rank=r)
        wr["ring"].run(wr["q_local"], wr["o"], wr["lse"])
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        wr["ring"].run(wr["q_local"], wr["o"], wr["lse"])
        torch.cuda.synchronize()
        per_rank.append((time.perf_counter() - t0) * 1e3)
        del wr
        torch.cuda.empty_cache()
    return w, sec, dict(mean_launch_ms=mean_ms, launches_per_step=launches,
                        flops_per_launch=flops_per_launch, t_copy_ms=t_copy_ms, per_rank_ms=per_rank,
                        achieved_tflops=flops_per_launch / (mean_ms * 1e-3) / 1e12,
                        full_ms=full_ms, diag_ms=float(np.mean(diag)) if diag else None)


def short_zigzag_bench(sweeps=50, warmup=20):
    """C2, the 8192-token sweep of rank 0 (cp 4): `sweeps` timed sweeps captured
    as one HIP graph after `warmup` untimed ones (fixed counts, independent of
    the headline's), plus other launch modes and the copy/compute overlap.

    Overlap efficiency, (T_compute + T_copies - T_sweep) / T_copies: T_sweep
    is the sweep as run (each step's launch also forwards the next block),
    T_compute the same attention launches given no forwarded ranges, T_copies
    the three block copies alone (ring_stage_copy launches); all three as
    graphs of `sweeps` sequences."""
    import torch
    import ring_attention_02_amd as ra
    import workloads
    w = workloads.zigzag_setup(2)
    ring, q, o, lse = w["ring"], w["q_local"], w["o"], w["lse"]
    eager = time_steps(lambda: ring.run(q, o, lse), sweeps, warmup)
    graph = ring.capture(q, o, lse)                   # one graph per sweep
    per_graph = time_steps(graph.replay, sweeps, warmup)
    side_graph = ring.capture(q, o, lse, side_copies=True)
    side = time_steps(side_graph.replay, sweeps, warmup)
    del side_graph
    job = ring.capture(q, o, lse, sweeps=sweeps)      # the timed sweeps as one graph
    graph_upload(job)
    for _ in range(warmup):
        graph.replay()
    sec = time_steps(job.replay, 1, 0) / sweeps
    del job
    fns = []
    ring.run(q, o, lse, on_launch=lambda t, qi, kj, cls, fn: fns.append((cls, fn)))
    torch.cuda.synchronize()
    launches = [fn for _, fn in fns]
    reps = 20
    mean_ms = graph_ms(launches, 1, reps) / len(launches)
    full_ms = graph_ms([fn for c, fn in fns if c == ra.FULL], 1, reps) / sum(c == ra.FULL for c, _ in fns)
    diag_ms = graph_ms([fn for c, fn in fns if c == ra.DIAG], 1, reps)
    t_sweep = graph_ms(launches, sweeps)
    compute = [lambda j=fn.jobs: ra.ring_attn_step_jobs(j, causal=True) for fn in launches]
    t_compute = graph_ms(compute, sweeps)
    copies = [lambda u=u: ra.stage_copy(ring.forward_pairs(u)) for u in range(1, ring.cp)]
    t_copy = graph_ms(copies, sweeps)
    # every rank of the ring, the same way (50 sweeps as one graph): the
    # zigzag partition gives each the same visible pairs, in other step shapes
    per_rank = []
    for r in range(ring.cp):
        wr = w if r == w["rank"] else workloads.zigzag_setup(2, rank=r)
        g = wr["ring"].capture(wr["q_local"], wr["o"], wr["lse"], sweeps=sweeps)
        graph_upload(g)
        wr["ring"].run(wr["q_local"], wr["o"], wr["lse"])
        per_rank.append(time_steps(g.replay, 1, 1) / sweeps * 1e3)
        del g, wr
    flops_per_launch = w["flops"] / len(launches)
    return w, sec, dict(mean_launch_ms=mean_ms, launches_per_step=len(launches),
                        achieved_tflops=flops_per_launch / (mean_ms * 1e-3) / 1e12,
                        full_ms=full_ms, diag_ms=diag_ms, eager_ms=eager * 1e3,
                        side_ms=side * 1e3, per_graph_ms=per_graph * 1e3,
                        t_sweep_ms=t_sweep, t_compute_ms=t_compute, t_copy_ms=t_copy, per_rank_ms=per_rank,
                        overlap=(t_compute + t_copy - t_sweep) / t_copy)


def tiny_bench(steps, warmup):
    """C1: the fp32 non-causal ring, 512 tokens in 4 blocks of 128, 4 heads,
    d 64: 16 ring-step launches and one 4-part LSE merge per sweep (a
    correctness workload: each fp32 launch is 8 workgroups of 64 rows, so
    the sweep is bound by latency, not by the ALU or by launch issue).
    Returns the graph-replayed and the eager seconds per sweep."""
    import torch
    import ring_attention_02_amd as ra
    import workloads
    from seeded_inputs import CONFIGS, Q_ID, K_ID, V_ID
    c = CONFIGS[1]
    shape = (c["batch"], c["seq"], c["heads"], c["d"])
    q, k, v = (workloads.host_tensor(1, t, 0, shape, torch.float32) for t in (Q_ID, K_ID, V_ID))
    flops = c["batch"] * c["seq"] * c["seq"] * c["heads"] * 4 * c["d"]
    sweep = lambda: ra.noncausal_ring_sweep(q, k, v, c["n_blocks"])
    eager = time_steps(sweep, steps, warmup)
    # the same sweep (its 16 step launches, their K/V block copies and the
    # merge) recorded once as a HIP graph and replayed once per timed step
    torch.cuda.synchronize()
    graph, stream = torch.cuda.CUDAGraph(), torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        sweep()
        with torch.cuda.graph(graph, stream=stream):
            sweep()
    torch.cuda.synchronize()
    graph_upload(graph)
    sec = time_steps(graph.replay, steps, warmup)
    return flops, sec, eager


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


def context_bench():
    """What the same GPU reaches on work with nothing but the roofline in the
    way, measured in the same run: a bf16 GEMM of 8192^3 through torch.matmul
    (the vendor BLAS; 300 back-to-back calls after 100 warm-up calls, long
    enough for the clock to settle as under the prefill sweeps) and a plain
    1 GiB device-to-device copy (read + write bytes).  Not part of the path:
    it puts the kernels' roofline fractions next to a practical ceiling."""
    import torch
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn((n, n), device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn((n, n), device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    for _ in range(100):
        torch.matmul(a, b, out=c)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    calls = 300
    s.record()
    for _ in range(calls):
        torch.matmul(a, b, out=c)
    e.record()
    torch.cuda.synchronize()
    gemm_tflops = 2 * n ** 3 / (s.elapsed_time(e) * 1e-3 / calls) / 1e12
    del a, b, c
    src = torch.empty(1 << 29, device="cuda", dtype=torch.int16)
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    s.record()
    for _ in range(20):
        dst.copy_(src)
    e.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) / (s.elapsed_time(e) * 1e-3 / 20) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"bf16_gemm_8192": {"tflops": round(gemm_tflops, 1),
                               "frac_of_peak": round(gemm_tflops / PEAK_BF16_TFLOPS, 4),
                               "what": "torch.matmul bf16 8192x8192x8192, 300 calls after 100 warm-up"},
            "d2d_copy_1GiB": {"gbs": round(copy_gbs, 1), "frac_of_peak": round(copy_gbs / PEAK_HBM_GBS, 4),
                              "what": "1 GiB device-to-device tensor copy, read + write bytes"}}


def host_index_bench():
    """The host-side index calls at the workloads' sizes, as tokens per second
    (they run on the host, with no device roofline): the head-tail partition
    of the 1M-token sequence for every rank of cp 8, the slot mapping of the
    decode workload's 64 x 131,072 positions over 8 devices, and the
    reorganisation index of the 135,168-token all-gathered context (4
    requests, 8 devices).  Each is the median of 5 calls through the
    binding (ctypes and numpy allocation included), on one host thread."""
    import ring_attention_02_amd as ra

    def med(fn, reps=5):
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return float(np.median(ts))

    seq, cp = 1 << 20, 8
    t_part = med(lambda: [ra.partition([seq], cp, r) for r in range(cp)])
    pos = np.arange(131072, dtype=np.int64)
    t_slot = med(lambda: [ra.slot_mapping(pos, 128, 16, 8, 1) for _ in range(64)])
    lens = [50000, 40000, 30000, 15168]
    t_reorg = med(lambda: ra.reorg_index(lens, 128, 16, 1, 8))
    return {"cp_partition": {"value": round(cp * seq / t_part / 1e6, 2), "unit": "M tokens/s",
                             "what": "1,048,576 tokens, cp 8, all 8 ranks (local list + restore index)"},
            "cp_slot_mapping": {"value": round(64 * 131072 / t_slot / 1e6, 2), "unit": "M tokens/s",
                                "what": "64 requests x 131,072 positions, block 128, interleave 16, 8 devices"},
            "cp_reorg_index": {"value": round(sum(lens) / t_reorg / 1e6, 2), "unit": "M tokens/s",
                               "what": "135,168 tokens of 4 requests on 8 devices, block 128, interleave 16"}}


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


def long_sweep_only(reps):
    """K whole sweeps of the 1M-token zigzag prefill (rank 0, cp 8), nothing
    else on the GPU after the input setup: for counter passes over the
    headline's launches (8 per sweep: 7 FULL steps and the paired diagonal
    step)."""
    import torch
    import workloads
    w = workloads.zigzag_setup(4)
    for _ in range(reps):
        w["ring"].run(w["q_local"], w["o"], w["lse"])
    torch.cuda.synchronize()
    print(json.dumps({"long_sweeps": reps, "launches_per_sweep": 8, "flops_per_sweep": w["flops"]}),
          flush=True)


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
# CPU baseline: the oracle on the host, on bounded samples of the workloads
# ---------------------------------------------------------------------------

def host_cores():
    """Host cores as the OS reports them, those this process may run on, and
    the BLAS threads numpy's oracle actually uses."""
    return {"os_cpu_count": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "blas_threads": blas_threads()}


def _host64(t):
    return t.float().cpu().numpy().astype(np.float64)


def cpu_baseline_long(w):
    """The oracle on 3,072 sampled (token, head) rows of the 1M-token rank-0
    share (about 10 s of host work), extrapolated to the whole sweep by
    visible-pair count.

    Rows: 4 kv heads (0, 3, 4 and 7) x 4 of their query heads x 192 tokens,
    96 of each local Q chunk at seeded random offsets, in batches of 32.
    Each batch goes to the oracle with the keys up to its last row's
    position, causal by absolute position, so it computes (and masks) at
    least the visible pairs it is credited with.  Only the oracle calls are
    timed."""
    import torch
    import oracle
    rng = np.random.default_rng(40404)
    c, d, hq, hkv = w["chunk"], w["d"], w["hq"], w["hkv"]
    group = hq // hkv
    t_used, flops, rows = 0.0, 0, 0
    kv_heads = sorted({0, (hkv - 1) // 2, hkv // 2, hkv - 1})
    for kvh in kv_heads:
        k = _host64(w["k_full"][0, :, kvh])
        v = _host64(w["v_full"][0, :, kvh])
        for h in kvh * group + np.array([0, 3, 5, 7]) % group:
            for i, part in enumerate(w["local_parts"]):
                offs = np.sort(rng.choice(c, 96, replace=False))
                for off in np.split(offs, 3):
                    idx = torch.from_numpy(i * c + off).to(w["q_local"].device)
                    qr = _host64(w["q_local"][0, idx, int(h)])               # [32, d]
                    pos = part * c + off
                    n = int(pos.max()) + 1
                    t0 = time.perf_counter()
                    oracle.attention_ref(qr[None, :, None, :], k[None, :n, None, :], v[None, :n, None, :],
                                         pos, np.arange(n), causal=True)
                    t_used += time.perf_counter() - t0
                    flops += int((pos + 1).sum()) * (2 * d + 2 * d)
                    rows += len(pos)
        del k, v
    rate = flops / t_used
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{rows} (token, head) rows of the 1M-token rank-0 share ({len(kv_heads)} kv heads x 4 "
                      f"query heads x 96 tokens of each local chunk), float64 numpy, {t_used:.1f} s; the "
                      f"rate is extrapolated to the whole sweep by visible pairs",
            "extrapolated": True, "extrapolated_seconds_per_sweep": round(w["flops"] / rate, 1),
            **host_cores()}


def cpu_baseline_short(w):
    """The oracle on the whole 8192-token rank-0 share (every head, all its
    threads), and on one thread for one head of it and for the whole tiny
    fp32 ring workload."""
    import oracle
    import workloads
    k = w["k_full"][0].float().cpu().numpy().astype(np.float64)
    v = w["v_full"][0].float().cpu().numpy().astype(np.float64)
    q = w["q_local"][0].float().cpu().numpy().astype(np.float64)
    q_pos = np.asarray(w["local"], dtype=np.int64)
    t0 = time.perf_counter()
    oracle.attention_ref(q[None], k[None], v[None], q_pos, np.arange(k.shape[0]), causal=True)
    t_all = time.perf_counter() - t0
    out = {"value": round(w["flops"] / t_all / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(),
           "kind": "oracle", "extrapolated": False,
           "sample": f"the whole workload: rank-0 local queries (2048 tokens) x all 8192 keys, "
                     f"{w['hq']} heads, float64 numpy, {t_all:.1f} s"}
    from threadpoolctl import threadpool_limits
    from seeded_inputs import CONFIGS, Q_ID, K_ID, V_ID
    import torch
    c1 = CONFIGS[1]
    shape1 = (c1["batch"], c1["seq"], c1["heads"], c1["d"])
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


def cpu_baseline_decode():
    """The oracle on one whole request of the decode workload (131,072 cached
    tokens over 8 shards, 64 query heads): per-shard attention and the merge.
    Rate in GB/s of the request's algorithmic bytes; the 64-request time is
    extrapolated (x 64)."""
    import torch
    import ring_attention_02_amd as ra
    import oracle
    import workloads
    from seeded_inputs import CONFIGS, Q_ID
    c = CONFIGS[3]
    B, hq, hkv, d, ctx = c["batch"], c["hq"], c["hkv"], c["d"], c["ctx"]
    n_sh = c["pcp"] * c["dcp"]
    kc, vc = workloads.decode_context(0)
    k64, v64 = _host64(kc)[None], _host64(vc)[None]
    del kc, vc
    q64 = _host64(workloads.host_tensor(3, Q_ID, 0, (B, hq, d), torch.bfloat16)[:1])
    dev, _ = ra.slot_mapping(np.arange(ctx), c["block_size"], c["interleave"], c["pcp"], c["dcp"])
    t0 = time.perf_counter()
    oracle.decode_shards_ref(q64, k64, v64, dev, n_sh)
    t = time.perf_counter() - t0
    nbytes = 2 * ctx * hkv * d * 2 + hq * d * 2 + 2 * n_sh * hq * (d + 1) * 4 + hq * (d + 1) * 4
    return {"value": round(nbytes / t / 1e9, 3), "unit": "GB/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"request 0 of 64 (all 64 heads, 8 shards and the merge), float64 numpy, {t:.1f} s",
            "extrapolated": True, "extrapolated_seconds_per_step": round(64 * t, 1)}


def cpu_baseline_segmented(w):
    """The oracle on 256 sampled (token, head) rows of the chunked-prefill
    workload (4 heads x 64 query tokens, all keys up to the last row's
    position), extrapolated to the whole workload by visible pairs."""
    import torch
    import oracle
    rng = np.random.default_rng(50505)
    t_used, flops, rows = 0.0, 0, 0
    for h in (0, 41, 86, w["h"] - 1):
        k = _host64(w["k"][0, :, h])
        v = _host64(w["v"][0, :, h])
        off = np.sort(rng.choice(w["sq"], 64, replace=False))
        qr = _host64(w["q"][0, torch.from_numpy(off).to(w["q"].device), h])
        pos = w["q_pos0"] + off
        n = int(pos.max()) + 1
        t0 = time.perf_counter()
        oracle.attention_ref(qr[None, :, None, :], k[None, :n, None, :], v[None, :n, None, :], pos,
                             np.arange(n), causal=True)
        t_used += time.perf_counter() - t0
        flops += int((pos + 1).sum()) * (2 * w["dqk"] + 2 * w["dv"])
        rows += len(pos)
    rate = flops / t_used
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{rows} (token, head) rows (4 heads x 64 tokens), float64 numpy, {t_used:.1f} s",
            "extrapolated": True, "extrapolated_seconds_per_step": round(w["flops"] / rate, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path is one "
              f"GPU's share of the ring and has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)
    import torch
    import ring_attention_02_amd  # noqa: F401  (fails loudly if the library is missing)
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    for flag, fn in ((args.calibrate_copy, calibrate_copy), (args.sweep_only, sweep_only),
                     (args.decode_only, decode_only), (args.merge_only, merge_only),
                     (args.long_step_only, long_step_only), (args.long_sweep_only, long_sweep_only),
                     (args.paged_only, paged_only), (args.segmented_only, segmented_only),
                     (args.varlen_only, varlen_only), (args.reorg_only, reorg_only)):
        if flag:
            fn() if flag is True else fn(flag)
            return

    log(f"C4 (headline): zigzag causal prefill, 1M tokens, cp 8, rank 0: {args.warmup} + {args.steps} sweeps")
    w4, sec4, l4 = long_headline(args.steps, args.warmup)
    out = {
        "metric": METRIC, "value": round(w4["flops"] / sec4 / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(sec4 * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "zigzag causal ring prefill, one rank's share of a 1,048,576-token "
                               "sequence: cp 8 (16 chunks of 65,536), rank 0 holds Q chunks {0,15} "
                               "(131,072 queries), 64 q-heads / 8 kv-heads, d 128, bf16",
                   "global_batch": 1, "seq_len": 1048576, "parallelism": "cp8 ring emulated on 1 GPU",
                   "flops_per_step": w4["flops"]},
        "roofline": roofline_entry("mfma", l4["achieved_tflops"], PEAK_BF16_TFLOPS, "TFLOP/s",
                                   profiled_traffic("attn_step_bf16_long_prefill_1M_cp8_sweep.md",
                                                    "attn_step.hip")),
        "kernel": {"name": "attn_step_bf16_kernel<128,128,1,*,false,2> (7 FULL steps, 1 paired diagonal step)",
                   "mean_launch_ms": round(l4["mean_launch_ms"], 3),
                   "launches_per_step": l4["launches_per_step"],
                   "full_step_ms": round(l4["full_ms"], 3), "diag_step_ms": round(l4["diag_ms"], 3),
                   "timing": "HIP events around every launch of the timed sweeps, on the launch stream"},
        "launch": {"mode": "one ring_attn_step_jobs launch per ring step, issued eagerly; each launch "
                           "also copies the next K/V block into the idle staging slot",
                   "per_rank_sweep_ms": [round(x, 1) for x in l4["per_rank_ms"]],
                   "forwarded_blocks_alone_ms": round(l4["t_copy_ms"], 3),
                   "forwarded_share_of_sweep": round(l4["t_copy_ms"] / (sec4 * 1e3), 5),
                   "full_step_traffic_bytes": profiled_traffic(
                       "attn_step_bf16_long_prefill_1M_cp8_full_step.md", "attn_step.hip",
                       field="full_step_traffic_bytes_per_launch")},
    }
    cpu = None
    if not args.no_cpu_baseline:
        log("CPU baseline: oracle on sampled rows of the 1M-token share")
        cpu = cpu_baseline_long(w4)
        out["cpu_baseline"] = cpu
    del w4
    torch.cuda.empty_cache()

    if not args.primary_only:
        only = set(filter(None, args.only.split(",")))
        sec, others = {}, {}
        if not only or "c2" in only:
            log("C2: zigzag causal prefill, seq 8192, cp 4, rank 0 (50 sweeps as one graph, 20 warm-up)")
            w2, s2, l2 = short_zigzag_bench()
            sec["short_prefill_8192_cp4"] = {
                "value": round(w2["flops"] / s2 / 1e12, 3), "unit": "TFLOP/s", "ms_per_step": round(s2 * 1e3, 4),
                "flops_per_step": w2["flops"],
                "roofline": roofline_entry("mfma", l2["achieved_tflops"], PEAK_BF16_TFLOPS, "TFLOP/s",
                                           profiled_traffic("attn_step_bf16_zigzag_seq8192_cp4.md",
                                                            "attn_step.hip")),
                "mean_launch_ms": round(l2["mean_launch_ms"], 5), "full_step_ms": round(l2["full_ms"], 5),
                "diag_step_ms": round(l2["diag_ms"], 5),
                "one_graph_per_sweep_ms": round(l2["per_graph_ms"], 4), "eager_ms": round(l2["eager_ms"], 4),
                "side_stream_copies_ms": round(l2["side_ms"], 4),
                "per_rank_sweep_ms": [round(x, 4) for x in l2["per_rank_ms"]],
                "overlap": {"efficiency": round(l2["overlap"], 3), "t_sweep_ms": round(l2["t_sweep_ms"], 4),
                            "t_compute_only_ms": round(l2["t_compute_ms"], 4),
                            "t_copies_only_ms": round(l2["t_copy_ms"], 4),
                            "definition": "(T_compute + T_copies - T_sweep) / T_copies, graph replays"}}
            if cpu is not None:
                log("CPU baseline: oracle on the whole 8192-token share")
                others["short_prefill_8192_cp4"] = cpu_baseline_short(w2)
            del w2
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
            if cpu is not None:
                log("CPU baseline: oracle on one decode request")
                others["decode_gqa_8_shards"] = cpu_baseline_decode()
                torch.cuda.empty_cache()
        if not only or "c3p" in only:
            log("C3 paged: the same decode through per-request block tables")
            w3p, s3p, l3p = decode_bench(max(3, min(args.steps, 10)), 2, paged=True)
            sec["decode_gqa_8_shards_paged"] = {
                "value": round(w3p["bytes"] / s3p / 1e9, 1), "unit": "GB/s",
                "ms_per_step": round(s3p * 1e3, 4), "bytes_per_step": w3p["bytes"],
                "roofline": roofline_entry("hbm", l3p["kernel_gbs"], PEAK_HBM_GBS, "GB/s",
                                           profiled_traffic("decode_bf16_gqa_8shards_paged.md", "decode.hip")),
                "kernel_ms": round(l3p["kernel_ms"], 4)}
            del w3p
            torch.cuda.empty_cache()
        if not only or "c5" in only:
            log("C5: segmented chunked prefill, MLA shape")
            w5, s5, l5 = segmented_bench(max(2, min(args.steps, 5)), 1)
            sec["segmented_prefill_mla"] = {
                "value": round(w5["flops"] / s5 / 1e12, 3), "unit": "TFLOP/s",
                "ms_per_step": round(s5 * 1e3, 3), "flops_per_step": w5["flops"],
                "roofline": roofline_entry("mfma", l5["achieved_tflops"], PEAK_BF16_TFLOPS, "TFLOP/s",
                                           profiled_traffic("attn_step_bf16_segmented_prefill_mla.md",
                                                            "attn_step.hip")),
                "mean_launch_ms": round(l5["mean_launch_ms"], 4)}
            if cpu is not None:
                log("CPU baseline: oracle on sampled chunked-prefill rows")
                others["segmented_prefill_mla"] = cpu_baseline_segmented(w5)
            del w5
            torch.cuda.empty_cache()
        if not only or "varlen" in only:
            log("varlen: 16 packed requests (512..8192 tokens), self-causal, GQA 32/8, d 128")
            w7, s7, l7 = varlen_bench(max(3, min(args.steps, 10)), 2)
            sec["varlen_packed_prefill"] = {
                "value": round(w7["flops"] / s7 / 1e12, 3), "unit": "TFLOP/s",
                "ms_per_step": round(s7 * 1e3, 4), "flops_per_step": w7["flops"],
                "tokens": int(w7["cu"][-1]),
                "roofline": roofline_entry("mfma", l7["achieved_tflops"], PEAK_BF16_TFLOPS, "TFLOP/s",
                                           profiled_traffic("attn_step_bf16_varlen_16req.md", "attn_step.hip")),
                "mean_launch_ms": round(l7["mean_launch_ms"], 4)}
            del w7
            torch.cuda.empty_cache()
        if not only or "reorg" in only:
            log("reorg_kvcache: all-gathered K/V of 135,168 tokens (4 requests, 8 devices) to request order")
            w8, s8 = reorg_bench(max(3, min(args.steps, 10)), 2)
            sec["reorg_kvcache_gather"] = {
                "value": round(w8["bytes"] / s8 / 1e9, 1), "unit": "GB/s",
                "ms_per_step": round(s8 * 1e3, 4), "bytes_per_step": w8["bytes"],
                "roofline": roofline_entry("hbm", w8["bytes"] / s8 / 1e9, PEAK_HBM_GBS, "GB/s",
                                           profiled_traffic("gather_rows_reorg_kvcache.md", "stage.hip"))}
            del w8
            torch.cuda.empty_cache()
        if not only or "c1" in only:
            log("C1: tiny non-causal ring, fp32, 512 tokens in 4 blocks")
            f1, s1, e1 = tiny_bench(max(10, args.steps), 5)
            sec["tiny_noncausal_ring_f32"] = {
                "value": round(f1 / s1 / 1e12, 4), "unit": "TFLOP/s", "ms_per_step": round(s1 * 1e3, 4),
                "flops_per_step": f1, "eager_ms": round(e1 * 1e3, 4),
                "roofline": roofline_entry("alu", f1 / s1 / 1e12, PEAK_F32_VALU_TFLOPS, "TFLOP/s"),
                "note": "correctness workload: 16 step launches of 8 workgroups (64 rows, 4 key-split "
                        "waves) and one merge per sweep, replayed as one HIP graph per sweep (eager_ms: "
                        "the same sweep issued eagerly)"}
        if not only or "merge" in only:
            log("lse_merge: 2 partials x 8.4M rows x 128")
            s6, b6 = merge_bench(max(5, args.steps), 2)
            sec["lse_merge_2x8M"] = {
                "value": round(b6 / s6 / 1e9, 1), "unit": "GB/s", "ms_per_step": round(s6 * 1e3, 4),
                "roofline": roofline_entry("hbm", b6 / s6 / 1e9, PEAK_HBM_GBS, "GB/s",
                                           profiled_traffic("lse_merge_2x8M.md", "lse_merge.hip"))}
        out["secondary"] = sec
        if not only or "host" in only:
            log("host index calls: partition, slot mapping, reorganisation index")
            out["host_index"] = host_index_bench()
        if not only or "context" in only:
            log("context: vendor bf16 GEMM and a plain device copy on the same GPU")
            out["context"] = context_bench()
        if cpu is not None and others:
            cpu["others"] = others
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
