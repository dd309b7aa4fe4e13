"""GPU parity of the launch forms that the benchmarked workloads select, and
of reads at a segment's end.

* Keys past the end of a K/V segment must take no part even when the memory
  after the segment holds NaN: the ring step loads whole 64-key tiles with
  bounded buffer loads, and a partial last tile must read zeros there (a
  masked score gives P = 0, but 0 * NaN from V would still poison O).
* The paged decode at the decode workload's scale (8 shards x 32 requests x
  8 kv heads = 2,048 work items) runs without key splits and writes the
  partials directly.
* The packed (varlen) prefill at d 128 with at least two workgroups per CU
  runs the 4-wave, 128-row form.

Every result is compared element by element with the oracle."""

import numpy as np
import pytest

import oracle
from gpu_util import tensor, host64, compare, say, BF16_O, BF16_LSE

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    import ring_attention_02_amd as ra
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return ra


def _nan_padded(t, extra_rows=64):
    """A copy of t [B, S, H, D] inside a larger buffer whose rows after the
    last one hold NaN; returns the [B, S, H, D] view (contiguous) of it."""
    B, S, H, D = t.shape
    buf = torch.full((B * S + extra_rows, H, D), float("nan"), dtype=t.dtype, device=t.device)
    buf[:B * S] = t.reshape(B * S, H, D)
    return buf[:B * S].view(B, S, H, D)


# (B, sq, sk, hq, hkv, dqk, dv, q_pos0, k_pos0, causal): the launch form each
# selects on 256 CUs, and which way its workgroups sweep the keys.
NAN_TAIL_CASES = [
    (2, 200, 333, 4, 2, 128, 128, 0, 0, False),       # 8-wave key split (16 WGs), forward
    (1, 384, 700, 96, 96, 128, 128, 300, 0, True),    # 8-wave key split, 2 rounds: odd ones backward
    (1, 768, 650, 128, 16, 64, 64, 400, 100, True),   # 4-wave, 2 rounds
    (1, 1000, 520, 256, 32, 128, 128, 200, 0, True),  # 256-row, 4 rounds, tail tile read first backward
    (2, 130, 77, 8, 1, 192, 128, 0, 0, False),        # d 192, 8-wave
]


@pytest.mark.parametrize("idx", range(len(NAN_TAIL_CASES)))
def test_nan_after_segment_end(ra, idx):
    B, sq, sk, hq, hkv, dqk, dv, q0, k0, causal = NAN_TAIL_CASES[idx]
    say(f"NaN tail case {idx}: B={B} sq={sq} sk={sk} hq={hq} hkv={hkv} d=({dqk},{dv}) q0={q0} "
        f"k0={k0} causal={causal}")
    cfg = 400 + idx
    q, q64 = tensor(cfg, 1, 0, (B, sq, hq, dqk), torch.bfloat16)
    k, k64 = tensor(cfg, 2, 0, (B, sk, hkv, dqk), torch.bfloat16)
    v, v64 = tensor(cfg, 3, 0, (B, sk, hkv, dv), torch.bfloat16)
    kn, vn = _nan_padded(k), _nan_padded(v)
    o = torch.empty((B, sq, hq, dv), device="cuda")
    lse = torch.empty((B, sq, hq), device="cuda")
    scale = 1.0 / np.sqrt(dqk)
    ra.ring_attn_step(q, kn, vn, o, lse, q0, k0, causal, scale, accumulate=False)
    torch.cuda.synchronize()
    o_h, lse_h = host64(o), host64(lse)
    assert np.all(np.isfinite(o_h)), "NaN past the segment's end reached O"
    group = hq // hkv
    heads = sorted({0, hq // 2 + 1, hq - 1})
    for h in heads:
        kv = slice(h // group, h // group + 1)
        ro, rl = oracle.attention_ref(q64[:, :, h:h + 1], k64[:, :, kv], v64[:, :, kv],
                                      q0 + np.arange(sq), k0 + np.arange(sk), causal, scale)
        compare(o_h[:, :, h:h + 1], lse_h[:, :, h:h + 1], ro, rl, BF16_O, BF16_LSE,
                f"NaN tail {idx} head {h}")


def test_nan_after_segment_end_jobs_and_varlen(ra):
    """Multi-segment jobs whose every segment is followed by NaN rows, and a
    packed launch whose last request's keys end where NaN rows begin."""
    hq, hkv, d = 8, 2, 128
    say("NaN tails: two jobs over three ragged segments; varlen last request")
    c = 333
    q, q64 = tensor(410, 1, 0, (1, 2 * c, hq, d), torch.bfloat16)
    segs, k64s, v64s, kpos = [], [], [], []
    for i, (sk, k0) in enumerate([(200, 0), (97, 300), (150, 500)]):
        k, k64 = tensor(410, 2, i, (1, sk, hkv, d), torch.bfloat16)
        v, v64 = tensor(410, 3, i, (1, sk, hkv, d), torch.bfloat16)
        segs.append((_nan_padded(k), _nan_padded(v), k0))
        k64s.append(k64); v64s.append(v64); kpos.append(k0 + np.arange(sk))
    o = torch.empty((1, 2 * c, hq, d), device="cuda")
    lse = torch.empty((1, 2 * c, hq), device="cuda")
    jobs = [dict(q=q[:, :c], o=o[:, :c], lse=lse[:, :c], q_pos0=100, accumulate=False, segments=segs),
            dict(q=q[:, c:], o=o[:, c:], lse=lse[:, c:], q_pos0=450, accumulate=False, segments=segs)]
    ra.ring_attn_step_jobs(jobs, causal=True)
    torch.cuda.synchronize()
    o_h, lse_h = host64(o), host64(lse)
    assert np.all(np.isfinite(o_h))
    k_all, v_all, p_all = np.concatenate(k64s, 1), np.concatenate(v64s, 1), np.concatenate(kpos)
    for part, q0 in ((slice(0, c), 100), (slice(c, 2 * c), 450)):
        ro, rl = oracle.attention_ref(q64[:, part], k_all, v_all, q0 + np.arange(c), p_all, True)
        compare(o_h[:, part], lse_h[:, part], ro, rl, BF16_O, BF16_LSE, f"jobs q0={q0}")

    reqs = [(300, 300, 0, 0), (130, 1131, 1001, 0), (129, 205, 3000, 2900)]   # (lq, lk, q0, k0)
    cq = np.concatenate([[0], np.cumsum([r[0] for r in reqs])]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum([r[1] for r in reqs])]).astype(np.int64)
    qv, qv64 = tensor(411, 1, 0, (int(cq[-1]), hq, d), torch.bfloat16)
    kv_, kv64 = tensor(411, 2, 0, (1, int(ck[-1]), hkv, d), torch.bfloat16)
    vv_, vv64 = tensor(411, 3, 0, (1, int(ck[-1]), hkv, d), torch.bfloat16)
    kn, vn = _nan_padded(kv_)[0], _nan_padded(vv_)[0]
    ov, lv = ra.ring_attn_step_varlen(qv, kn, vn, cq, ck, [r[2] for r in reqs], [r[3] for r in reqs])
    torch.cuda.synchronize()
    ov_h, lv_h = host64(ov), host64(lv)
    assert np.all(np.isfinite(ov_h))
    for i, (lq, lk, q0, k0) in enumerate(reqs):
        rows, keys = slice(int(cq[i]), int(cq[i + 1])), slice(int(ck[i]), int(ck[i + 1]))
        ro, rl = oracle.attention_ref(qv64[None, rows], kv64[:, keys], vv64[:, keys], q0 + np.arange(lq),
                                      k0 + np.arange(lk), True)
        compare(ov_h[None, rows], lv_h[None, rows], ro, rl, BF16_O, BF16_LSE, f"varlen NaN tail {i}")


def test_split_kv_decode_paged_without_key_splits(ra):
    """The benchmarked paged form: 8 shards x 32 requests x 8 kv heads = 2,048
    work items, so the launch takes no key splits and the kernel writes the
    per-shard partials directly (no workspace).  Random block tables, one
    ragged request, GQA 64/8, blocks of 128 interleaved by 16."""
    n_shards, B, hq, hkv, d, bs, il = 8, 32, 64, 8, 128, 128, 16
    rng = np.random.default_rng(520)
    ctx = [int(x) for x in rng.integers(512, 3072, B)]
    ctx[5] = 2048 - 77                              # ragged inside a block
    ctx[17] = 1                                     # a single cached token
    vbs = bs * n_shards
    n_vb = [-(-L // vbs) for L in ctx]
    num_blocks = sum(n_vb) + 9
    max_blocks = max(n_vb)
    assert ra.split_kv_decode_workspace(n_shards, B, hq, hkv, d, max_blocks * bs) == 0
    say(f"paged decode without splits: {n_shards * B * hkv} work items, contexts {min(ctx)}..{max(ctx)}")
    perm = rng.permutation(num_blocks).astype(np.int32)
    q, q64 = tensor(521, 1, 0, (B, hq, d), torch.bfloat16)
    tmax = max(ctx)
    k_ctx, k64 = tensor(521, 2, 0, (B, tmax, hkv, d), torch.bfloat16)
    v_ctx, v64 = tensor(521, 3, 0, (B, tmax, hkv, d), torch.bfloat16)
    kp = torch.zeros((n_shards, num_blocks, bs, hkv, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    tables = np.full((n_shards, B, max_blocks), -1, dtype=np.int32)
    lens = np.zeros((n_shards, B), dtype=np.int64)
    used = 0
    for b, L in enumerate(ctx):
        table = perm[used:used + n_vb[b]]
        used += n_vb[b]
        dev, slot = ra.slot_mapping(np.arange(L), bs, il, n_shards, 1, block_table=table)
        lens[:, b] = np.bincount(dev, minlength=n_shards)
        tables[:, b, :n_vb[b]] = table
        dev_t, slot_t = torch.from_numpy(dev.astype(np.int64)).cuda(), torch.from_numpy(slot).cuda()
        kp.view(n_shards, num_blocks * bs, hkv, d)[dev_t, slot_t] = k_ctx[b, :L]
        vp.view(n_shards, num_blocks * bs, hkv, d)[dev_t, slot_t] = v_ctx[b, :L]
    o_parts, lse_parts = ra.split_kv_decode_paged(q, kp, vp, torch.from_numpy(tables).cuda(),
                                                  torch.from_numpy(lens).cuda())
    o, lse = ra.lse_merge(o_parts, lse_parts)
    torch.cuda.synchronize()
    op_h, lp_h, o_h, l_h = host64(o_parts), host64(lse_parts), host64(o), host64(lse)
    for b, L in enumerate(ctx):
        dev_ref, _ = oracle.slot_mapping_ref(np.arange(L), bs, il, n_shards, 1)
        po, pl, mo, ml = oracle.decode_shards_ref(q64[b:b + 1], k64[b:b + 1, :L], v64[b:b + 1, :L],
                                                  np.asarray(dev_ref), n_shards)
        compare(op_h[:, b], lp_h[:, b], po[:, 0], pl[:, 0], BF16_O, BF16_LSE, f"partials b={b}")
        compare(o_h[b], l_h[b], mo[0], ml[0], BF16_O, BF16_LSE, f"merged b={b}")


def test_varlen_four_wave_form(ra):
    """The benchmarked packed form: 16 self-causal requests of 512..2048
    tokens, GQA 32/8, d 128.  The grid (16 query tiles x 16 requests x 32
    heads = 8,192 workgroups) is far above two per CU, so it runs the 4-wave
    128-row kernel, longest tiles first.  Sampled heads per request."""
    rng = np.random.default_rng(530)
    lens = [int(x) for x in rng.integers(8, 33, 16) * 64]
    lens[3] = 2048
    lens[9] = 512 + 37                               # ragged last tile
    hq, hkv, d = 32, 8, 128
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    pos = np.zeros(len(lens), dtype=np.int64)
    say(f"varlen 4-wave form: {len(lens)} requests, {int(cu[-1])} tokens")
    q, q64 = tensor(531, 1, 0, (int(cu[-1]), hq, d), torch.bfloat16)
    k, k64 = tensor(531, 2, 0, (int(cu[-1]), hkv, d), torch.bfloat16)
    v, v64 = tensor(531, 3, 0, (int(cu[-1]), hkv, d), torch.bfloat16)
    o, lse = ra.ring_attn_step_varlen(q, k, v, cu, cu, pos, pos, causal=True)
    torch.cuda.synchronize()
    o_h, l_h = host64(o), host64(lse)
    group = hq // hkv
    for i, L in enumerate(lens):
        rows = slice(int(cu[i]), int(cu[i + 1]))
        heads = sorted({int(rng.integers(0, hq)), hq - 1 - i % hq})
        for h in heads:
            kvh = slice(h // group, h // group + 1)
            ro, rl = oracle.attention_ref(q64[None, rows, h:h + 1], k64[None, rows, kvh],
                                          v64[None, rows, kvh], np.arange(L), np.arange(L), True)
            compare(o_h[None, rows, h:h + 1], l_h[None, rows, h:h + 1], ro, rl, BF16_O, BF16_LSE,
                    f"request {i} (L={L}) head {h}")
