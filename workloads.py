"""Device inputs of the five workloads, shared by bench.py and the GPU tests.

Inputs come from seeded_inputs (host draws for the small workloads, seeded
device draws for the large ones); sequence placement uses the library's own
partition and slot mapping.  Nothing here computes attention.

  C1  tiny non-causal ring: 1 x 512 tokens, 4 heads, d 64, fp32, 4 blocks
  C2  zigzag causal prefill, rank 0 of cp=4 over 8192 tokens, 32 heads, d 128
  C3  GQA decode: 64 requests x 131072 context, 64 q / 8 kv heads, 8 shards
  C4  zigzag causal prefill, rank 0 of cp=8 over 1048576 tokens, 64 q / 8 kv heads
  C5  segmented chunked prefill: 4096 queries at 131072.., 128 heads, d 192/128
"""

import numpy as np

import seeded_inputs as si
from seeded_inputs import Q_ID, K_ID, V_ID, CONFIGS


def _torch():
    import torch
    return torch


def host_tensor(cfg, tid, chunk, shape, dtype):
    torch = _torch()
    if dtype == torch.float32:
        return torch.from_numpy(si.normal_f32(cfg, tid, chunk, shape)).cuda()
    bits = si.normal_bf16_bits(cfg, tid, chunk, shape)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def causal_pairs(q_pos0, sq, k_pos0, sk):
    """Visible (q, k) pairs of a causal block pair: sum_i clip(q0+i-k0+1, 0, sk)."""
    def tri(n):  # sum_{j=1..n} j
        return n * (n + 1) // 2
    lo = q_pos0 - k_pos0 + 1            # visible keys of row 0 before clipping
    total = 0
    # rows where the count is between 1 and sk-1 form an arithmetic run
    first_pos = max(0, 1 - lo)          # first row with >= 1 visible key
    first_full = max(0, sk - lo)        # first row that sees all sk keys
    first_pos, first_full = min(first_pos, sq), min(first_full, sq)
    if first_full > first_pos:
        a, b = lo + first_pos, lo + first_full - 1
        total += tri(b) - tri(a - 1)
    total += (sq - first_full) * sk
    return total


def zigzag_setup(cfg_id, rank=None):
    """C2 / C4: a rank's local Q (the workload's rank 0 unless another is
    named), every rank's K/V, the ring and its FLOP count."""
    import ring_attention_02_amd as ra
    torch = _torch()
    c = CONFIGS[cfg_id]
    seq, cp, hq, hkv, d = c["seq"], c["cp"], c["hq"], c["hkv"], c["d"]
    rank = c["rank"] if rank is None else rank
    parts = 2 * cp
    chunk = seq // parts
    big = cfg_id == 4
    shape_k = (1, chunk, hkv, d)
    gen = (lambda tid, p, shp: si.device_normal(cfg_id, tid, p, shp, torch.bfloat16, "cuda")) if big \
        else (lambda tid, p, shp: host_tensor(cfg_id, tid, p, shp, torch.bfloat16))
    k_full = torch.cat([gen(K_ID, p, shape_k) for p in range(parts)], 1)
    v_full = torch.cat([gen(V_ID, p, shape_k) for p in range(parts)], 1)
    local, restore = ra.partition([seq], cp, rank)
    # Q part p holds tokens [p*chunk, (p+1)*chunk); the local list names which
    # parts (and in which order) this rank holds.
    local_parts = [int(local[i * chunk]) // chunk for i in range(len(local) // chunk)]
    for i, p in enumerate(local_parts):
        assert np.array_equal(local[i * chunk:(i + 1) * chunk], np.arange(p * chunk, (p + 1) * chunk))
    q_local = torch.cat([gen(Q_ID, p, (1, chunk, hq, d)) for p in local_parts], 1).contiguous()
    ring = ra.ZigzagRing(k_full, v_full, cp, rank)
    o = torch.empty((1, q_local.shape[1], hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, q_local.shape[1], hq), dtype=torch.float32, device="cuda")
    pairs = 0
    for p in local_parts:
        for kp in range(parts):
            pairs += causal_pairs(p * chunk, chunk, kp * chunk, chunk)
    flops = pairs * hq * (2 * d + 2 * d)
    return dict(cfg=cfg_id, k_full=k_full, v_full=v_full, q_local=q_local, local=local,
                restore=restore, local_parts=local_parts, chunk=chunk, ring=ring, o=o, lse=lse,
                flops=flops, pairs=pairs, hq=hq, hkv=hkv, d=d, seq=seq, cp=cp, rank=rank)


def decode_setup(requests=None):
    """C3: per-shard K/V caches filled through the slot mapping; q; shard lengths."""
    import ring_attention_02_amd as ra
    torch = _torch()
    c = CONFIGS[3]
    B, hq, hkv, d, ctx = c["batch"], c["hq"], c["hkv"], c["d"], c["ctx"]
    bs, il, n_sh = c["block_size"], c["interleave"], c["pcp"] * c["dcp"]
    dev, slot = ra.slot_mapping(np.arange(ctx), bs, il, c["pcp"], c["dcp"])
    t_shard = int(slot.max()) + 1
    counts = np.bincount(dev, minlength=n_sh)
    dev_t = torch.from_numpy(dev.astype(np.int64)).cuda()
    slot_t = torch.from_numpy(slot).cuda()
    ks = torch.empty((n_sh, B, t_shard, hkv, d), dtype=torch.bfloat16, device="cuda")
    vs = torch.empty_like(ks)
    for b in range(B):
        kc = si.device_normal(3, K_ID, b, (ctx, hkv, d), torch.bfloat16, "cuda")
        ks[dev_t, b, slot_t] = kc
        del kc
        vc = si.device_normal(3, V_ID, b, (ctx, hkv, d), torch.bfloat16, "cuda")
        vs[dev_t, b, slot_t] = vc
        del vc
    q = host_tensor(3, Q_ID, 0, (B, hq, d), torch.bfloat16)
    lens = torch.from_numpy(np.repeat(counts[:, None], B, axis=1).astype(np.int64)).cuda()
    kv_bytes = 2 * n_sh * B * t_shard * hkv * d * 2
    return dict(q=q, ks=ks, vs=vs, lens=lens, dev=dev, slot=slot, t_shard=t_shard, B=B, hq=hq,
                hkv=hkv, d=d, ctx=ctx, n_shards=n_sh, kv_bytes=kv_bytes,
                # algorithmic bytes: K+V once, Q, partials written then read by the merge,
                # merged output written
                bytes=kv_bytes + q.numel() * 2 + 2 * n_sh * B * hq * (d + 1) * 4 + B * hq * (d + 1) * 4)


def decode_paged_setup():
    """C3 in a paged layout: each shard's cache is a pool of 128-token blocks;
    request b's virtual blocks take a seeded random choice of physical blocks
    (the same ids in every shard), and the slot mapping places each token at
    table[vb] * block_size + loc of its shard's pool."""
    import ring_attention_02_amd as ra
    torch = _torch()
    c = CONFIGS[3]
    B, hq, hkv, d, ctx = c["batch"], c["hq"], c["hkv"], c["d"], c["ctx"]
    bs, il, n_sh = c["block_size"], c["interleave"], c["pcp"] * c["dcp"]
    n_vb = -(-ctx // (bs * n_sh))
    num_blocks = B * n_vb
    perm = np.random.default_rng(si.device_seed(3, 9, 0)).permutation(num_blocks).astype(np.int32)
    kp = torch.empty((n_sh, num_blocks * bs, hkv, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    tables = np.empty((n_sh, B, n_vb), dtype=np.int32)
    lens = np.empty((n_sh, B), dtype=np.int64)
    for b in range(B):
        table = perm[b * n_vb:(b + 1) * n_vb]
        dev, slot = ra.slot_mapping(np.arange(ctx), bs, il, c["pcp"], c["dcp"], block_table=table)
        tables[:, b] = table
        lens[:, b] = np.bincount(dev, minlength=n_sh)
        dev_t = torch.from_numpy(dev.astype(np.int64)).cuda()
        slot_t = torch.from_numpy(slot).cuda()
        kc = si.device_normal(3, K_ID, b, (ctx, hkv, d), torch.bfloat16, "cuda")
        kp[dev_t, slot_t] = kc
        del kc
        vc = si.device_normal(3, V_ID, b, (ctx, hkv, d), torch.bfloat16, "cuda")
        vp[dev_t, slot_t] = vc
        del vc
    q = host_tensor(3, Q_ID, 0, (B, hq, d), torch.bfloat16)
    kv_bytes = 2 * n_sh * B * n_vb * bs * hkv * d * 2
    return dict(q=q, kp=kp.view(n_sh, num_blocks, bs, hkv, d), vp=vp.view(n_sh, num_blocks, bs, hkv, d),
                tables=torch.from_numpy(tables).cuda(), lens=torch.from_numpy(lens).cuda(), B=B, hq=hq,
                hkv=hkv, d=d, ctx=ctx, n_shards=n_sh, kv_bytes=kv_bytes,
                bytes=kv_bytes + q.numel() * 2 + 2 * n_sh * B * hq * (d + 1) * 4 + B * hq * (d + 1) * 4)


def decode_context(b, ctx=None):
    """Token-order K/V context of request b (regenerated from its seed)."""
    torch = _torch()
    c = CONFIGS[3]
    ctx = ctx or c["ctx"]
    kc = si.device_normal(3, K_ID, b, (c["ctx"], c["hkv"], c["d"]), torch.bfloat16, "cuda")
    vc = si.device_normal(3, V_ID, b, (c["ctx"], c["hkv"], c["d"]), torch.bfloat16, "cuda")
    return kc[:ctx], vc[:ctx]


def segmented_setup():
    """C5: q at 131072.., K/V over the whole 135168-token context."""
    torch = _torch()
    c = CONFIGS[5]
    sq, q0, h, dqk, dv, skv = c["q_len"], c["q_pos0"], c["heads"], c["d_qk"], c["d_v"], c["kv_len"]
    q = si.device_normal(5, Q_ID, 0, (1, sq, h, dqk), torch.bfloat16, "cuda")
    k = si.device_normal(5, K_ID, 0, (1, skv, h, dqk), torch.bfloat16, "cuda")
    v = si.device_normal(5, V_ID, 0, (1, skv, h, dv), torch.bfloat16, "cuda")
    o = torch.empty((1, sq, h, dv), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, sq, h), dtype=torch.float32, device="cuda")
    pairs = causal_pairs(q0, sq, 0, skv)
    return dict(q=q, k=k, v=v, o=o, lse=lse, q_pos0=q0, segment=c["segment"], sq=sq, h=h,
                dqk=dqk, dv=dv, skv=skv, pairs=pairs, flops=pairs * h * (2 * dqk + 2 * dv))


def varlen_setup(n_req=16, hq=32, hkv=8, d=128, seed_cfg=6):
    """Packed multi-request prefill: n_req requests whose lengths are a
    seeded uniform draw in [512, 8192] tokens (multiples of 64), each
    attending causally to itself; GQA 32/8, d 128, bf16 N(0, 1)."""
    torch = _torch()
    rng = np.random.default_rng(si.device_seed(seed_cfg, 0, 0))
    lens = (rng.integers(512 // 64, 8192 // 64 + 1, size=n_req) * 64).astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    total = int(cu[-1])
    q = si.device_normal(seed_cfg, Q_ID, 0, (total, hq, d), torch.bfloat16, "cuda")
    k = si.device_normal(seed_cfg, K_ID, 0, (total, hkv, d), torch.bfloat16, "cuda")
    v = si.device_normal(seed_cfg, V_ID, 0, (total, hkv, d), torch.bfloat16, "cuda")
    o = torch.empty((total, hq, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((total, hq), dtype=torch.float32, device="cuda")
    pairs = int(sum(int(L) * (int(L) + 1) // 2 for L in lens))
    zeros = np.zeros(n_req, dtype=np.int64)
    return dict(q=q, k=k, v=v, o=o, lse=lse, cu=cu, pos=zeros, lens=lens, hq=hq, hkv=hkv, d=d,
                pairs=pairs, flops=pairs * hq * 4 * d)


def reorg_setup():
    """All-gather-KV reorganisation at the chunked-prefill (MLA) scale: the
    135,168-token context split into 4 requests, placed on 8 devices
    (block 128, interleave 16), all-gathered: K [N, 128, 192] and
    V [N, 128, 128] bf16 in gathered order, and the request-order row index."""
    import ring_attention_02_amd as ra
    torch = _torch()
    c = CONFIGS[5]
    lens = [50000, 40000, 30000, c["kv_len"] - 120000]
    n = sum(lens)
    gk = si.device_normal(5, K_ID, 7, (n, c["heads"], c["d_qk"]), torch.bfloat16, "cuda")
    gv = si.device_normal(5, V_ID, 7, (n, c["heads"], c["d_v"]), torch.bfloat16, "cuda")
    src, _ = ra.reorg_index(lens, 128, 16, 1, 8)
    return dict(gk=gk, gv=gv, idx=torch.from_numpy(src).cuda(), lens=lens, n=n,
                bytes=2 * (gk.numel() + gv.numel()) * 2 + src.size * 8)
