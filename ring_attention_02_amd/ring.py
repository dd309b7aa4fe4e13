"""Ring schedules on one GPU: the zigzag causal ring, segmented prefill and
the plain (non-causal) ring sweep, all built on the library's calls.

Ring rule (guijiagi.com "Ring Attention", ring-topology excerpt): at step t
rank i computes with the K/V block that started on rank (i - t) mod N while
that block travels on to rank i + 1; after N steps its partial output is the
final result.  With the head-tail partition (vLLM-Ascend "Context Parallel
(CP)", PCP head-tail token partition paragraph) the block of rank s holds
sequence parts s and 2N-1-s.

On one GPU the other ranks' K/V live in one full-sequence buffer.  Receiving
a block is a copy into one of two staging slots, made one step ahead so it
overlaps the attention of the current block: the double buffering of the
video "How Context Parallelism Splits Long Sequences Across GPUs" (chapter
on the wire budget) and of the Excalidraw "Context Parallel (CP) / Ring
Attention" diagram (rotation overlapped with local attention).  By default
the copy rides in the ring step's own launch (its forwarded ranges), so a
sweep is one stream of one launch per step.  With a copy stream the copies
run there instead, ordered by events: block t+1 lands before step t+1 and
is written only after the step that last read its slot.  Step 0 uses the
rank's own block in place.
"""

import math

from . import (ring_attn_step, ring_attn_step_jobs, lse_merge, classify, stage_copy, ring_schedule,
               FULL, DIAG, SKIP)


def _torch():
    import torch
    return torch


class ZigzagRing:
    """One rank's share of a zigzag causal ring prefill, emulated on one GPU.

    k_full / v_full: [1, seq, hkv, d] (bf16 or f32) -- every rank's K/V.
    The local queries are the rank's two parts, [1, 2*chunk, hq, d_qk].
    """

    def __init__(self, k_full, v_full, cp_size, rank):
        torch = _torch()
        seq = k_full.shape[1]
        if k_full.shape[0] != 1 or seq % (2 * cp_size) != 0:
            raise ValueError("k_full must be [1, seq, hkv, d] with seq a multiple of 2*cp_size")
        self.k_full, self.v_full = k_full, v_full
        self.cp, self.rank = cp_size, rank
        self.chunk = seq // (2 * cp_size)
        c = self.chunk
        # the block's (head, tail) parts at each step, from the library's ring
        # order; step 0 is the rank's own block, whose parts are its queries
        self.steps = [tuple(int(p) for p in pair) for pair in ring_schedule(cp_size, rank)[1]]
        self.q_parts = self.steps[0]
        dev = k_full.device
        self.kbuf = [torch.empty((2, 1, c, *k_full.shape[2:]), dtype=k_full.dtype, device=dev)
                     for _ in range(2)]
        self.vbuf = [torch.empty((2, 1, c, *v_full.shape[2:]), dtype=v_full.dtype, device=dev)
                     for _ in range(2)]

    def local_slices(self, t):
        return [self.k_full[:, p * self.chunk:(p + 1) * self.chunk] for p in self.steps[t]], \
               [self.v_full[:, p * self.chunk:(p + 1) * self.chunk] for p in self.steps[t]]

    def forward_pairs(self, t):
        """(dst, src) pieces that 'receive' the block of step t into slot t % 2."""
        slot = t % 2
        ks, vs = self.local_slices(t)
        return [(self.kbuf[slot][0], ks[0]), (self.kbuf[slot][1], ks[1]),
                (self.vbuf[slot][0], vs[0]), (self.vbuf[slot][1], vs[1])]

    def pairs(self):
        """(step, q part index, kv part index, class) for every pair of the sweep."""
        c = self.chunk
        out = []
        for t, kv_parts in enumerate(self.steps):
            for qi, qp in enumerate(self.q_parts):
                for kj, kp in enumerate(kv_parts):
                    out.append((t, qi, kj, classify(qp * c, c, kp * c, c, True)))
        return out

    def run(self, q_local, o, lse, scale=None, on_launch=None, copy_stream=None):
        """Sweep every ring step; o [1, 2c, hq, dv] / lse [1, 2c, hq] end final.

        Step t's launch computes with the block of step t and carries the
        copy of the block of step t + 1 into the other slot.  With
        copy_stream (a torch stream) the copies run on it instead, in
        ring_stage_copy launches ordered against the steps by events.
        on_launch(step, q_index, kv_index, cls, fn) may wrap each launch (the
        bench uses it to time launches); fn() performs the launch, and
        fn.jobs / fn.forward are the jobs and forwarded (dst, src) pairs it
        passes to ring_attn_step_jobs.
        """
        c = self.chunk
        first = [True, True]
        side = copy_stream is not None
        if side:
            torch = _torch()
            main = torch.cuda.current_stream()
            copied = {}                              # block t -> event after its copy
            read_done = {}                           # step t -> event after its launch
            copy_stream.wait_stream(main)

            def issue_copy(u):
                # block u goes to slot u % 2, last read by step u - 2
                with torch.cuda.stream(copy_stream):
                    if u - 2 >= 1:
                        copy_stream.wait_event(read_done[u - 2])
                    stage_copy(self.forward_pairs(u))
                    copied[u] = torch.cuda.Event()
                    copied[u].record(copy_stream)

            for u in (1, 2):
                if u < self.cp:
                    issue_copy(u)
        for t, kv_parts in enumerate(self.steps):
            if t == 0:
                ks, vs = self.local_slices(0)
            else:
                ks, vs = self.kbuf[t % 2], self.vbuf[t % 2]
                if side:
                    main.wait_event(copied[t])
            fwd = self.forward_pairs(t + 1) if t + 1 < self.cp and not side else []
            # One launch per ring step: each local Q part is a job over the
            # block's parts it can see (SKIP parts are left out).
            jobs, step_cls = [], FULL
            for qi, qp in enumerate(self.q_parts):
                qs = slice(qi * c, (qi + 1) * c)
                segs = []
                for kj, kp in enumerate(kv_parts):
                    cls = classify(qp * c, c, kp * c, c, True)
                    if cls != SKIP:
                        segs.append((ks[kj], vs[kj], kp * c))
                        step_cls = DIAG if cls == DIAG else step_cls
                acc = not first[qi]
                first[qi] = False
                if segs or not acc:
                    jobs.append(dict(q=q_local[:, qs], o=o[:, qs], lse=lse[:, qs],
                                     q_pos0=qp * c, accumulate=acc, segments=segs))
            if jobs:
                def fn(j=jobs, f=fwd):
                    ring_attn_step_jobs(j, causal=True, scale=scale, forward=f)
                fn.jobs, fn.forward = jobs, fwd
                if on_launch is None:
                    fn()
                else:
                    on_launch(t, 0, 0, step_cls, fn)
            elif fwd:
                stage_copy(fwd)
            if side:
                read_done[t] = torch.cuda.Event()
                read_done[t].record(main)
                if t >= 1 and t + 2 < self.cp:
                    issue_copy(t + 2)
        if side:
            main.wait_stream(copy_stream)
        return o, lse

    def capture(self, q_local, o, lse, scale=None, side_copies=False, sweeps=1):
        """Record whole sweeps as a HIP graph.

        Replaying the graph runs the same launches as run() without the
        host-side cost of issuing them one by one; the buffers passed here
        are the ones every replay reads and writes.  side_copies records the
        copy-stream form (two streams joined in the graph); sweeps > 1
        records that many complete sweeps back to back (each one recomputes
        o / lse from the same inputs), so a replay pays one graph launch for
        all of them.
        """
        torch = _torch()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        stream = torch.cuda.Stream()                      # default priority
        side = torch.cuda.Stream() if side_copies else None
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            with torch.cuda.graph(graph, stream=stream):
                for _ in range(sweeps):
                    self.run(q_local, o, lse, scale=scale, copy_stream=side)
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        return graph


def segmented_prefill(q, k, v, o, lse, q_pos0, segment, k_pos0=0, causal=True, scale=None,
                      on_launch=None):
    """Attend q to k/v one KV segment at a time with an online-softmax merge.

    vLLM-Ascend "Context Parallel (CP)", PCP chunked-prefill paragraph: with a
    cap on the KV processed per round, the segments are attended in order and
    each result is folded into the running one.  q [1, Sq, H, Dqk] at
    positions q_pos0.., k/v [1, Sk, Hkv, *] at positions k_pos0.. (read in
    place); o/lse are overwritten with the result.
    """
    sk = k.shape[1]
    n_seg = max(1, math.ceil(sk / segment))
    bounds = [(s_ * segment, min(sk, (s_ + 1) * segment)) for s_ in range(n_seg)]
    if q.dtype != _torch().bfloat16:
        # float32: one ring step per segment, each merged into the running result
        for s_, (a, b) in enumerate(bounds):
            ring_attn_step(q, k[:, a:b], v[:, a:b], o, lse, q_pos0=q_pos0, k_pos0=k_pos0 + a,
                           causal=causal, scale=scale, accumulate=s_ > 0)
        return o, lse
    # up to four segments per launch; the first launch overwrites o / lse
    for g in range(0, n_seg, 4):
        group = bounds[g:g + 4]
        segs = [(k[:, a:b], v[:, a:b], k_pos0 + a) for a, b in group]
        job = [dict(q=q, o=o, lse=lse, q_pos0=q_pos0, accumulate=g > 0, segments=segs)]
        if on_launch is None:
            ring_attn_step_jobs(job, causal=causal, scale=scale)
        else:
            cls = DIAG if any(classify(q_pos0, q.shape[1], k_pos0 + a, b - a, causal) == DIAG
                              for a, b in group) else FULL
            on_launch(g, 0, g, cls, lambda j=job: ring_attn_step_jobs(j, causal=causal, scale=scale))
    return o, lse


def noncausal_ring_sweep(q, k, v, n_blocks, scale=None):
    """Plain ring over n_blocks sequence blocks, no mask, fresh partial per step.

    Block qb meets K/V block (qb - t) mod n at step t; the n partials of every
    query row are combined with lse_merge.  Returns (o, lse) for all rows.
    """
    torch = _torch()
    B, S, H, D = q.shape
    dv = v.shape[3]
    blk = S // n_blocks
    if blk * n_blocks != S:
        raise ValueError("sequence must split into n_blocks equal blocks")
    o_parts = torch.empty((n_blocks, B, S, H, dv), dtype=torch.float32, device=q.device)
    lse_parts = torch.empty((n_blocks, B, S, H), dtype=torch.float32, device=q.device)
    for qb in range(n_blocks):
        qs = slice(qb * blk, (qb + 1) * blk)
        order = ring_schedule(n_blocks, qb)[0]        # block of each ring step
        for t in range(n_blocks):
            kb = int(order[t])
            ks = slice(kb * blk, (kb + 1) * blk)
            ring_attn_step(q[:, qs], k[:, ks].contiguous(), v[:, ks].contiguous(),
                           o_parts[t][:, qs], lse_parts[t][:, qs], q_pos0=qb * blk,
                           k_pos0=kb * blk, causal=False, scale=scale, accumulate=False)
    return lse_merge(o_parts, lse_parts)
