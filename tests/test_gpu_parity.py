"""GPU parity of every entry point against the CPU oracle, element by element,
on seeded inputs small enough for the oracle (several tiles plus ragged
tails), with the edge cases of the method: empty rows, SKIP pairs, single
keys, GQA groups, every supported head-dim pair, accumulate on and off."""

import numpy as np
import pytest

import oracle
from gpu_util import tensor, host64, compare, say, F32_O, BF16_O, BF16_LSE

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    import ring_attention_02_amd as ra
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return ra


CASES = [
    # (B, sq, sk, hq, hkv, dqk, dv, q_pos0, k_pos0, causal)
    (1, 128, 64, 2, 2, 128, 128, 0, 0, False),
    (1, 200, 333, 4, 2, 128, 128, 0, 0, False),          # ragged tails, GQA 2
    (2, 130, 70, 8, 1, 64, 64, 0, 0, False),             # GQA 8, batch 2
    (1, 257, 257, 4, 4, 128, 128, 0, 0, True),           # self-causal diagonal, ragged
    (1, 300, 200, 2, 1, 192, 128, 500, 250, True),       # MLA shape, diagonal offset
    (1, 100, 64, 2, 2, 128, 128, 100, 150, True),        # rows 100..149 see nothing
    (1, 1, 1, 1, 1, 64, 64, 0, 0, True),                 # one query, one key
    (1, 1, 500, 16, 2, 128, 128, 1000, 0, True),         # one query sees all (FULL)
    (1, 64, 1024, 4, 1, 64, 64, 2000, 1500, True),       # partial diagonal, many tiles
    (1, 384, 128, 16, 16, 192, 128, 128, 0, True),       # FULL (every pair visible)
]


def _run_case(ra, idx, case, dtype, accumulate):
    B, sq, sk, hq, hkv, dqk, dv, q0, k0, causal = case
    say(f"case {idx}: B={B} sq={sq} sk={sk} hq={hq} hkv={hkv} d=({dqk},{dv}) q0={q0} k0={k0} "
        f"causal={causal} dtype={dtype} acc={accumulate}")
    cfg = 100 + idx
    q, q64 = tensor(cfg, 1, 0, (B, sq, hq, dqk), dtype)
    k, k64 = tensor(cfg, 2, 0, (B, sk, hkv, dqk), dtype)
    v, v64 = tensor(cfg, 3, 0, (B, sk, hkv, dv), dtype)
    scale = 1.0 / np.sqrt(dqk)
    q_pos, k_pos = q0 + np.arange(sq), k0 + np.arange(sk)
    o = torch.full((B, sq, hq, dv), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((B, sq, hq), 7.0, dtype=torch.float32, device="cuda")
    if accumulate:
        # a previous ring step against another K/V block sitting just before this one
        sk2 = 96
        k2, k2_64 = tensor(cfg, 4, 0, (B, sk2, hkv, dqk), dtype)
        v2, v2_64 = tensor(cfg, 5, 0, (B, sk2, hkv, dv), dtype)
        ra.ring_attn_step(q, k2, v2, o, lse, q0, k0 - sk2, causal, scale, accumulate=False)
        cls = ra.ring_attn_step(q, k, v, o, lse, q0, k0, causal, scale, accumulate=True)
        o_ref, lse_ref = oracle.attention_ref(
            q64, np.concatenate([k2_64, k64], 1), np.concatenate([v2_64, v64], 1), q_pos,
            np.concatenate([k0 - sk2 + np.arange(sk2), k_pos]), causal, scale)
    else:
        cls = ra.ring_attn_step(q, k, v, o, lse, q0, k0, causal, scale, accumulate=False)
        o_ref, lse_ref = oracle.attention_ref(q64, k64, v64, q_pos, k_pos, causal, scale)
    torch.cuda.synchronize()
    assert cls == oracle.classify_ref(q0, sq, k0, sk, causal)
    tol_o = F32_O if dtype == torch.float32 else BF16_O
    tol_l = F32_O if dtype == torch.float32 else BF16_LSE
    compare(host64(o), host64(lse), o_ref, lse_ref, tol_o, tol_l, f"case {idx}")


@pytest.mark.parametrize("idx", range(len(CASES)))
@pytest.mark.parametrize("accumulate", [False, True])
def test_ring_attn_step_bf16(ra, idx, accumulate):
    _run_case(ra, idx, CASES[idx], torch.bfloat16, accumulate)


@pytest.mark.parametrize("idx", [0, 1, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("accumulate", [False, True])
def test_ring_attn_step_f32(ra, idx, accumulate):
    _run_case(ra, idx, CASES[idx], torch.float32, accumulate)


def test_skip_pair_writes_identity_or_nothing(ra):
    q, _ = tensor(7, 1, 0, (1, 64, 2, 128), torch.bfloat16)
    k, _ = tensor(7, 2, 0, (1, 64, 2, 128), torch.bfloat16)
    v, _ = tensor(7, 3, 0, (1, 64, 2, 128), torch.bfloat16)
    o = torch.full((1, 64, 2, 128), 3.0, device="cuda")
    lse = torch.full((1, 64, 2), 5.0, device="cuda")
    cls = ra.ring_attn_step(q, k, v, o, lse, q_pos0=0, k_pos0=64, causal=True, accumulate=True)
    torch.cuda.synchronize()
    assert cls == ra.SKIP
    assert torch.all(o == 3.0) and torch.all(lse == 5.0)
    cls = ra.ring_attn_step(q, k, v, o, lse, q_pos0=0, k_pos0=64, causal=True, accumulate=False)
    torch.cuda.synchronize()
    assert cls == ra.SKIP
    assert torch.all(o == 0.0) and torch.all(torch.isneginf(lse))


def _random_cases(n, seed):
    """Seeded random shapes across every supported head-dim pair, GQA group,
    causal offset (FULL / DIAG / partly empty rows), batch and ragged size."""
    rng = np.random.default_rng(seed)
    pairs = [(64, 64), (128, 128), (192, 128)]
    out = []
    for i in range(n):
        dqk, dv = pairs[i % 3]
        hkv = int(rng.choice([1, 2, 4]))
        hq = hkv * int(rng.choice([1, 2, 4, 8]))
        B = int(rng.choice([1, 1, 2]))
        sq = int(rng.integers(1, 300))
        sk = int(rng.integers(1, 400))
        causal = bool(rng.integers(0, 2))
        q0 = int(rng.integers(0, 600))
        k0 = int(rng.integers(0, 600))
        out.append((B, sq, sk, hq, hkv, dqk, dv, q0, k0, causal))
    return out


RANDOM_CASES = _random_cases(24, 2026)


@pytest.mark.parametrize("idx", range(len(RANDOM_CASES)))
def test_ring_attn_step_random_shapes(ra, idx):
    """bf16 ring step on seeded random shapes, accumulate alternating."""
    _run_case(ra, 200 + idx, RANDOM_CASES[idx], torch.bfloat16, accumulate=bool(idx % 2))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_empty_key_and_query_blocks(ra, dtype):
    """sk = 0: a non-accumulating step writes O = 0 and LSE = -inf (the oracle
    over no keys), an accumulating one leaves the running result untouched;
    sq = 0 is a no-op."""
    say(f"empty blocks: dtype={dtype}")
    q, q64 = tensor(71, 1, 0, (1, 37, 4, 128), dtype)
    k0 = torch.empty((1, 0, 2, 128), dtype=dtype, device="cuda")
    o = torch.full((1, 37, 4, 128), 7.0, device="cuda")
    lse = torch.full((1, 37, 4), 7.0, device="cuda")
    cls = ra.ring_attn_step(q, k0, k0, o, lse, 0, 0, True, 0.1, accumulate=False)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q64, np.zeros((1, 0, 2, 128)), np.zeros((1, 0, 2, 128)),
                                          np.arange(37), np.arange(0), True, 0.1)
    assert cls == ra.SKIP == oracle.classify_ref(0, 37, 0, 0, True)
    assert np.array_equal(host64(o), o_ref) and np.array_equal(host64(lse), lse_ref)
    o.fill_(3.0)
    lse.fill_(2.0)
    ra.ring_attn_step(q, k0, k0, o, lse, 0, 0, True, 0.1, accumulate=True)
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((lse == 2.0).all())
    k, _ = tensor(71, 2, 0, (1, 50, 2, 128), dtype)
    q0 = torch.empty((1, 0, 4, 128), dtype=dtype, device="cuda")
    o0 = torch.empty((1, 0, 4, 128), device="cuda")
    l0 = torch.empty((1, 0, 4), device="cuda")
    ra.ring_attn_step(q0, k, k, o0, l0, 0, 0, True, 0.1, accumulate=False)
    torch.cuda.synchronize()


def test_deterministic(ra):
    q, _ = tensor(8, 1, 0, (1, 300, 4, 128), torch.bfloat16)
    k, _ = tensor(8, 2, 0, (1, 500, 2, 128), torch.bfloat16)
    v, _ = tensor(8, 3, 0, (1, 500, 2, 128), torch.bfloat16)
    outs = []
    for _ in range(2):
        o = torch.empty((1, 300, 4, 128), device="cuda")
        lse = torch.empty((1, 300, 4), device="cuda")
        ra.ring_attn_step(q, k, v, o, lse, q_pos0=400, k_pos0=0, causal=True)
        outs.append((o.clone(), lse.clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("n,rows,dv,out_bf16", [(1, 37, 64, False), (4, 512, 64, False),
                                                (8, 4096, 128, False), (3, 1000, 128, True),
                                                (2, 65, 192, False), (3, 100, 36, False),
                                                (5, 77, 12, True)])
def test_lse_merge(ra, n, rows, dv, out_bf16):
    say(f"lse_merge n={n} rows={rows} dv={dv} bf16={out_bf16}")
    r = np.random.default_rng(n * 1000 + rows)
    o_parts = r.standard_normal((n, rows, dv)).astype(np.float32)
    lse_parts = (r.standard_normal((n, rows)) * 3).astype(np.float32)
    lse_parts[:, :5] = -np.inf                  # rows with nothing anywhere
    o_parts[:, :5] = 0.0
    if n > 1:
        lse_parts[0, 5:20] = -np.inf            # one empty part
        o_parts[0, 5:20] = 0.0
    o_ref, lse_ref = oracle.lse_merge_ref(list(o_parts.astype(np.float64)),
                                          list(lse_parts.astype(np.float64)))
    od, ld = ra.lse_merge(torch.from_numpy(o_parts).cuda(), torch.from_numpy(lse_parts).cuda(),
                          out_dtype=torch.bfloat16 if out_bf16 else torch.float32)
    torch.cuda.synchronize()
    o_gpu = host64(od)
    compare(o_gpu, host64(ld), o_ref, lse_ref, BF16_O if out_bf16 else 1e-5, 1e-5, "lse_merge")
    if out_bf16:
        # bf16 output: round-to-nearest-even leaves at most half an ulp, i.e.
        # 2^-8 of the value, on top of the float32 merge
        assert np.all(np.abs(o_gpu - o_ref) <= 2.0 ** -8 * np.abs(o_ref) + 1e-5)


def test_zigzag_all_ranks_restore(ra):
    """Every rank of a small zigzag ring; gathered outputs put back in order
    with the restore index equal full causal attention."""
    seq, cp, h, d = 2048, 4, 4, 128
    k, k64 = tensor(21, 2, 0, (1, seq, h, d), torch.bfloat16)
    v, v64 = tensor(21, 3, 0, (1, seq, h, d), torch.bfloat16)
    q_all, q64 = tensor(21, 1, 0, (1, seq, h, d), torch.bfloat16)
    gathered_o, gathered_l = [], []
    restore = None
    for rank in range(cp):
        local, restore = ra.partition([seq], cp, rank)
        idx = torch.from_numpy(local).cuda()
        q_local = q_all.index_select(1, idx).contiguous()
        ring = ra.ZigzagRing(k, v, cp, rank)
        o = torch.empty((1, len(local), h, d), device="cuda")
        lse = torch.empty((1, len(local), h), device="cuda")
        ring.run(q_local, o, lse)
        gathered_o.append(o)
        gathered_l.append(lse)
    restore_t = torch.from_numpy(restore).cuda()          # applied on the device
    o = ra.gather_rows(torch.cat(gathered_o, 1)[0], restore_t)[None]
    lse = ra.gather_rows(torch.cat(gathered_l, 1)[0], restore_t)[None]
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q64, k64, v64, causal=True)
    compare(host64(o), host64(lse), o_ref, lse_ref, BF16_O, BF16_LSE, "zigzag all ranks")


def test_noncausal_ring_sweep_f32(ra):
    q, q64 = tensor(1, 1, 0, (1, 512, 4, 64), torch.float32)
    k, k64 = tensor(1, 2, 0, (1, 512, 4, 64), torch.float32)
    v, v64 = tensor(1, 3, 0, (1, 512, 4, 64), torch.float32)
    o, lse = ra.noncausal_ring_sweep(q, k, v, 4)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q64, k64, v64, causal=False)
    compare(host64(o), host64(lse), o_ref, lse_ref, F32_O, F32_O, "tiny ring fp32")


def test_segmented_prefill_small(ra):
    sq, h, dqk, dv, q0 = 256, 4, 192, 128, 1000
    skv = q0 + sq
    q, q64 = tensor(31, 1, 0, (1, sq, h, dqk), torch.bfloat16)
    k, k64 = tensor(31, 2, 0, (1, skv, h, dqk), torch.bfloat16)
    v, v64 = tensor(31, 3, 0, (1, skv, h, dv), torch.bfloat16)
    o = torch.empty((1, sq, h, dv), device="cuda")
    lse = torch.empty((1, sq, h), device="cuda")
    ra.segmented_prefill(q, k, v, o, lse, q_pos0=q0, segment=300)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(q64, k64, v64, q0 + np.arange(sq), np.arange(skv), True)
    compare(host64(o), host64(lse), o_ref, lse_ref, BF16_O, BF16_LSE, "segmented")


def _decode_case(ra, cfg, B, ctx_lens, n_shards, hq, hkv, bs=128, il=16, fill=0.0):
    d = 128
    tmax = max(ctx_lens)
    vbs = bs * n_shards
    t_shard = -(-tmax // vbs) * bs
    q, q64 = tensor(cfg, 1, 0, (B, hq, d), torch.bfloat16)
    k_ctx, k64 = tensor(cfg, 2, 0, (B, tmax, hkv, d), torch.bfloat16)
    v_ctx, v64 = tensor(cfg, 3, 0, (B, tmax, hkv, d), torch.bfloat16)
    # rows past each shard's length hold `fill` (NaN: they must never be read)
    ks = torch.full((n_shards, B, t_shard, hkv, d), fill, dtype=torch.bfloat16, device="cuda")
    vs = torch.full_like(ks, fill)
    lens = np.zeros((n_shards, B), dtype=np.int64)
    for b, L in enumerate(ctx_lens):
        dev, slot = ra.slot_mapping(np.arange(L), bs, il, n_shards, 1)
        lens[:, b] = np.bincount(dev, minlength=n_shards)
        dev_t = torch.from_numpy(dev.astype(np.int64)).cuda()
        slot_t = torch.from_numpy(slot).cuda()
        ks[dev_t, b, slot_t] = k_ctx[b, :L]
        vs[dev_t, b, slot_t] = v_ctx[b, :L]
    lens_t = torch.from_numpy(lens).cuda()
    o_parts, lse_parts = ra.split_kv_decode(q, ks, vs, shard_lens=lens_t)
    o, lse = ra.lse_merge(o_parts, lse_parts)
    torch.cuda.synchronize()
    for b, L in enumerate(ctx_lens):
        dev_ref, _ = oracle.slot_mapping_ref(np.arange(L), bs, il, n_shards, 1)
        po, pl, mo, ml = oracle.decode_shards_ref(q64[b:b + 1], k64[b:b + 1, :L], v64[b:b + 1, :L],
                                                  dev_ref, n_shards)
        compare(host64(o_parts[:, b]), host64(lse_parts[:, b]), po[:, 0], pl[:, 0], BF16_O,
                BF16_LSE, f"decode partials b={b}")
        compare(host64(o[b]), host64(lse[b]), mo[0], ml[0], BF16_O, BF16_LSE, f"decode b={b}")


def test_split_kv_decode_small(ra):
    say("decode: 8 shards, 3 requests (one ragged), GQA 8")
    _decode_case(ra, 41, 3, [4096, 1500, 4096], 8, 16, 2)


def test_split_kv_decode_with_splits(ra):
    # few work items -> the kernel splits each shard's keys and merges the splits
    assert ra.split_kv_decode_workspace(2, 1, 4, 1, 128, 8192) > 0
    say("decode: 2 shards, 1 request, splits")
    _decode_case(ra, 42, 1, [16384 - 100], 2, 4, 1)


def test_split_kv_decode_group16_and_empty_shard(ra):
    say("decode: group 16, shard with no tokens")
    _decode_case(ra, 43, 2, [100, 2048], 8, 16, 1)


def test_split_kv_decode_nan_past_shard_ends(ra):
    # every K/V row past a shard's length is NaN; ragged last tiles everywhere
    say("decode: NaN rows past every shard's end")
    _decode_case(ra, 47, 3, [4096, 1500, 77], 8, 16, 2, fill=float("nan"))


def test_zigzag_graph_replay_matches_eager(ra):
    """The captured sweep, replayed several times with eager work and
    synchronisations in between, reproduces the eager sweep bit for bit."""
    seq, cp, rank, h, d = 2048, 4, 1, 4, 128
    k, _ = tensor(22, 2, 0, (1, seq, h, d), torch.bfloat16)
    v, _ = tensor(22, 3, 0, (1, seq, h, d), torch.bfloat16)
    q_all, _ = tensor(22, 1, 0, (1, seq, h, d), torch.bfloat16)
    local, _ = ra.partition([seq], cp, rank)
    q_local = q_all.index_select(1, torch.from_numpy(local).cuda()).contiguous()
    ring = ra.ZigzagRing(k, v, cp, rank)
    o = torch.empty((1, len(local), h, d), device="cuda")
    lse = torch.empty((1, len(local), h), device="cuda")
    ring.run(q_local, o, lse)
    torch.cuda.synchronize()
    o_eager, lse_eager = o.clone(), lse.clone()
    graph = ring.capture(q_local, o, lse)
    for i in range(3):
        o.fill_(float(i + 1))
        lse.fill_(-float(i + 1))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager) and torch.equal(lse, lse_eager), f"replay {i}"
        ring.run(q_local, o, lse)        # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager)


def test_zigzag_copy_stream_matches_in_launch_copies(ra):
    """Staging copies on a side stream (eager, and captured as a two-stream
    graph replayed several times) give the same sweep bit for bit as the
    copies carried in the step launches; cp 4 exercises the slot reuse
    (block 3 waits for step 1 to finish reading slot 1)."""
    seq, cp, rank, h, d = 4096, 4, 0, 4, 128
    say(f"zigzag copy stream: seq {seq} cp {cp} rank {rank}")
    k, _ = tensor(23, 2, 0, (1, seq, h, d), torch.bfloat16)
    v, _ = tensor(23, 3, 0, (1, seq, h, d), torch.bfloat16)
    q_all, _ = tensor(23, 1, 0, (1, seq, h, d), torch.bfloat16)
    local, _ = ra.partition([seq], cp, rank)
    q_local = q_all.index_select(1, torch.from_numpy(local).cuda()).contiguous()
    ring = ra.ZigzagRing(k, v, cp, rank)
    o = torch.empty((1, len(local), h, d), device="cuda")
    lse = torch.empty((1, len(local), h), device="cuda")
    ring.run(q_local, o, lse)
    torch.cuda.synchronize()
    o_ref, lse_ref = o.clone(), lse.clone()
    side = torch.cuda.Stream()
    o.zero_()
    ring.run(q_local, o, lse, copy_stream=side)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), "eager copy stream"
    graph = ring.capture(q_local, o, lse, side_copies=True)
    for i in range(3):
        o.fill_(float(i + 1))
        lse.fill_(-float(i + 1))
        for buf in ring.kbuf + ring.vbuf:           # stale slots must be rewritten
            buf.fill_(float(i))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref), f"replay {i}"
        ring.run(q_local, o, lse)
        torch.cuda.synchronize()


@pytest.mark.parametrize("causal", [False, True])
def test_peaked_scores_exercise_max_raises(ra, causal):
    """Large score range (queries scaled x8, some keys planted equal to a
    query): the running max is raised many times inside a block, and the
    result must still match the oracle."""
    sq, sk, hq, hkv, d = 200, 700, 4, 2, 128
    q, _ = tensor(61, 1, 0, (1, sq, hq, d), torch.float32)
    k, _ = tensor(61, 2, 0, (1, sk, hkv, d), torch.float32)
    v, _ = tensor(61, 3, 0, (1, sk, hkv, d), torch.bfloat16)
    q = q * 8.0
    k[0, 650:660, 0] = q[0, 190:200, 0] / 8.0       # very large scores late in the block
    k[0, 3, 1] = q[0, 5, 2] / 8.0
    qb, kb = q.to(torch.bfloat16), k.to(torch.bfloat16)
    o = torch.empty((1, sq, hq, d), device="cuda")
    lse = torch.empty((1, sq, hq), device="cuda")
    ra.ring_attn_step(qb, kb, v, o, lse, q_pos0=600, k_pos0=0, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(host64(qb), host64(kb), host64(v), 600 + np.arange(sq),
                                          np.arange(sk), causal)
    compare(host64(o), host64(lse), o_ref, lse_ref, BF16_O, BF16_LSE, "peaked")


@pytest.mark.parametrize("causal", [False, True])
def test_score_jump_beyond_the_exp2_range(ra, causal):
    """Keys planted equal to a query (queries scaled x8) late in the block:
    their scores exceed every earlier score of the row by about 1000 in log2
    units, so exponentials taken against the earlier running max would
    overflow float32; the result must still match the oracle."""
    sq, sk, hq, hkv, d = 130, 700, 2, 1, 128
    q, _ = tensor(62, 1, 0, (1, sq, hq, d), torch.float32)
    k, _ = tensor(62, 2, 0, (1, sk, hkv, d), torch.float32)
    v, _ = tensor(62, 3, 0, (1, sk, hkv, d), torch.bfloat16)
    q = q * 8.0
    k[0, 650, 0] = q[0, 100, 0]                    # row 100 of head 0: score |q|^2
    k[0, 690:700, 0] = q[0, 120:130, 1] * 1.5      # rows 120..129 of head 1, later still
    qb, kb = q.to(torch.bfloat16), k.to(torch.bfloat16)
    o = torch.empty((1, sq, hq, d), device="cuda")
    lse = torch.empty((1, sq, hq), device="cuda")
    ra.ring_attn_step(qb, kb, v, o, lse, q_pos0=600, k_pos0=0, causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(host64(qb), host64(kb), host64(v), 600 + np.arange(sq),
                                          np.arange(sk), causal)
    assert lse_ref[0, 100, 0] > 600.0          # the planted score (natural-log units) dominates its row
    compare(host64(o), host64(lse), o_ref, lse_ref, BF16_O, BF16_LSE, "score jump")


def test_stage_copy_pieces(ra):
    src = [torch.randn(n, device="cuda") for n in (4096, 4, 100000 * 4, 12)]
    dst = [torch.full_like(x, -1.0) for x in src]
    big = torch.randn((2, 1000, 8, 128), device="cuda").to(torch.bfloat16)
    big_dst = torch.zeros_like(big)
    ra.stage_copy(list(zip(dst, src)) + [(big_dst[0], big[1]), (big_dst[1], big[0])])
    torch.cuda.synchronize()
    for d, s_ in zip(dst, src):
        assert torch.equal(d, s_)
    assert torch.equal(big_dst[0], big[1]) and torch.equal(big_dst[1], big[0])


@pytest.mark.parametrize("dqk,dv,hq,hkv", [(128, 128, 4, 2), (64, 64, 2, 2), (192, 128, 2, 1)])
def test_jobs_union_of_segments(ra, dqk, dv, hq, hkv):
    """Several query chunks in one launch, each over scattered K/V segments
    (one of them invisible, one job with no segment), against the oracle on
    the union of keys; accumulate on one job."""
    sq = 200
    def seg(cfg, sk):
        k, k64 = tensor(cfg, 2, sk, (1, sk, hkv, dqk), torch.bfloat16)
        v, v64 = tensor(cfg, 3, sk, (1, sk, hkv, dv), torch.bfloat16)
        return k, v, k64, v64
    segs = {n: seg(70 + i, n) for i, n in enumerate((100, 257, 64, 130))}
    layout = [  # (q_pos0, [(segment size, k_pos0)], accumulate)
        (1000, [(100, 0), (257, 990), (64, 5000)], False),   # FULL, DIAG, invisible
        (300, [(130, 250), (64, 0)], True),                   # DIAG, FULL; merged into previous
        (50, [], False),                                      # no keys: empty partial
    ]
    jobs, refs = [], []
    for i, (q0, sg, acc) in enumerate(layout):
        q, q64 = tensor(80 + i, 1, 0, (1, sq, hq, dqk), torch.bfloat16)
        o = torch.full((1, sq, hq, dv), 3.0, device="cuda")
        lse = torch.full((1, sq, hq), 1.0, device="cuda")
        kk = [segs[n][2] for n, _ in sg]
        vv = [segs[n][3] for n, _ in sg]
        kp = [p0 + np.arange(n) for n, p0 in sg]
        if acc:   # a previous partial over 40 keys just before the segments
            k2, k2_64 = tensor(90, 2, 0, (1, 40, hkv, dqk), torch.bfloat16)
            v2, v2_64 = tensor(90, 3, 0, (1, 40, hkv, dv), torch.bfloat16)
            ra.ring_attn_step(q, k2, v2, o, lse, q_pos0=q0, k_pos0=200, causal=True)
            kk, vv, kp = [k2_64] + kk, [v2_64] + vv, [200 + np.arange(40)] + kp
        jobs.append(dict(q=q, o=o, lse=lse, q_pos0=q0, accumulate=acc,
                         segments=[(segs[n][0], segs[n][1], p0) for n, p0 in sg]))
        if kk:
            ro, rl = oracle.attention_ref(q64, np.concatenate(kk, 1), np.concatenate(vv, 1),
                                          q0 + np.arange(sq), np.concatenate(kp), True)
        else:
            ro, rl = np.zeros((1, sq, hq, dv)), np.full((1, sq, hq), -np.inf)
        refs.append((o, lse, ro, rl))
    # the same launch forwards four ranges of odd sizes (copied bit for bit)
    src = [torch.randn(n, device="cuda") for n in (4096, 4, 100004, 12)]
    dst = [torch.full_like(x, -1.0) for x in src]
    ra.ring_attn_step_jobs(jobs, causal=True, forward=list(zip(dst, src)))
    torch.cuda.synchronize()
    for i, (o, lse, ro, rl) in enumerate(refs):
        compare(host64(o), host64(lse), ro, rl, BF16_O, BF16_LSE, f"job {i}")
    for d, s_ in zip(dst, src):
        assert torch.equal(d, s_)


def test_jobs_forward_without_attention_work(ra):
    """A launch whose only job has no visible key and accumulates still moves
    its forwarded ranges (and leaves o / lse as they were)."""
    q = torch.randn((1, 64, 2, 128), device="cuda").to(torch.bfloat16)
    k = torch.randn((1, 64, 2, 128), device="cuda").to(torch.bfloat16)
    o = torch.full((1, 64, 2, 128), 5.0, device="cuda")
    lse = torch.full((1, 64, 2), 2.0, device="cuda")
    src = torch.randn((3, 1000, 8), device="cuda")
    dst = torch.zeros_like(src)
    ra.ring_attn_step_jobs([dict(q=q, o=o, lse=lse, q_pos0=0, accumulate=True,
                                 segments=[(k, k, 1000)])],
                           causal=True, forward=[(dst[0], src[2]), (dst[2], src[0])])
    torch.cuda.synchronize()
    assert torch.equal(dst[0], src[2]) and torch.equal(dst[2], src[0])
    assert bool((dst[1] == 0).all())
    assert bool((o == 5.0).all()) and bool((lse == 2.0).all())


@pytest.mark.parametrize("accumulate", [False, True])
def test_jobs_paired_diagonal_step(ra, accumulate):
    """The head-tail diagonal step in one launch: job 0 = the head part over its
    own chunk (DIAG), job 1 = the tail part over the head chunk (FULL) and its
    own chunk (DIAG).  With 64 heads and 4 query tiles the plain grid is 512
    workgroups, so on a 256-CU device the launch pairs tile p of job 0 with
    tile 3-p of job 1 in one 8-wave workgroup; results must not change.
    With accumulate, both jobs merge into a partial over 96 earlier keys."""
    c, hq, d, pre = 512, 64, 128, 96
    q, _ = tensor(91, 1, 0, (1, 2 * c, hq, d), torch.bfloat16)
    k, _ = tensor(91, 2, 0, (1, 2 * c, hq, d), torch.bfloat16)
    v, _ = tensor(91, 3, 0, (1, 2 * c, hq, d), torch.bfloat16)
    k_pre, _ = tensor(91, 4, 0, (1, pre, hq, d), torch.bfloat16)
    v_pre, _ = tensor(91, 5, 0, (1, pre, hq, d), torch.bfloat16)
    o = torch.empty((1, 2 * c, hq, d), device="cuda")
    lse = torch.empty((1, 2 * c, hq), device="cuda")
    # positions: earlier keys 0..pre-1, head part pre.., tail part pre+7c..
    head0, tail0 = pre, pre + 7 * c
    k_head, v_head = k[:, :c].contiguous(), v[:, :c].contiguous()
    k_tail, v_tail = k[:, c:].contiguous(), v[:, c:].contiguous()
    if accumulate:
        for part, q0 in ((slice(0, c), head0), (slice(c, 2 * c), tail0)):
            ra.ring_attn_step(q[:, part], k_pre, v_pre, o[:, part], lse[:, part], q_pos0=q0,
                              k_pos0=0, causal=True)
    jobs = [dict(q=q[:, :c], o=o[:, :c], lse=lse[:, :c], q_pos0=head0, accumulate=accumulate,
                 segments=[(k_head, v_head, head0)]),
            dict(q=q[:, c:], o=o[:, c:], lse=lse[:, c:], q_pos0=tail0, accumulate=accumulate,
                 segments=[(k_head, v_head, head0), (k_tail, v_tail, tail0)])]
    ra.ring_attn_step_jobs(jobs, causal=True)
    torch.cuda.synchronize()
    heads = [0, 17, 63]
    q64 = host64(q)[:, :, heads]
    k64, v64 = host64(k)[:, :, heads], host64(v)[:, :, heads]
    pos = np.concatenate([head0 + np.arange(c), tail0 + np.arange(c)])
    kpos = pos
    if accumulate:
        k64 = np.concatenate([host64(k_pre)[:, :, heads], k64], 1)
        v64 = np.concatenate([host64(v_pre)[:, :, heads], v64], 1)
        kpos = np.concatenate([np.arange(pre), pos])
    ro, rl = oracle.attention_ref(q64, k64, v64, pos, kpos, True)
    compare(host64(o)[:, :, heads], host64(lse)[:, :, heads], ro, rl, BF16_O, BF16_LSE, "paired")


@pytest.mark.parametrize("c,accumulate", [(2048, False), (2048, True), (2200, False)])
def test_jobs_paired_diagonal_step_large_grid(ra, c, accumulate):
    """The head-tail diagonal step on a large grid: 2048-token parts, 64 query
    heads over 8 kv heads.  The paired grid is 8 query tiles of 256 rows x 64
    heads = 512 workgroups (two per CU on a 256-CU device), whose loads the
    pairing evens out (head tile p sees 4(p+1) key tiles, tail tile 7-p sees
    32 + 4(8-p)); results must match the oracle on sampled heads.  2200-token
    parts give 9 tiles (the middle one meets itself across the two jobs) and
    a ragged last tile of 152 rows."""
    hq, hkv, d, pre = 64, 8, 128, 96
    q, _ = tensor(92, 1, 0, (1, 2 * c, hq, d), torch.bfloat16)
    k, _ = tensor(92, 2, 0, (1, 2 * c, hkv, d), torch.bfloat16)
    v, _ = tensor(92, 3, 0, (1, 2 * c, hkv, d), torch.bfloat16)
    k_pre, _ = tensor(92, 4, 0, (1, pre, hkv, d), torch.bfloat16)
    v_pre, _ = tensor(92, 5, 0, (1, pre, hkv, d), torch.bfloat16)
    o = torch.empty((1, 2 * c, hq, d), device="cuda")
    lse = torch.empty((1, 2 * c, hq), device="cuda")
    head0, tail0 = pre, pre + 7 * c
    k_head, v_head = k[:, :c].contiguous(), v[:, :c].contiguous()
    k_tail, v_tail = k[:, c:].contiguous(), v[:, c:].contiguous()
    if accumulate:
        for part, q0 in ((slice(0, c), head0), (slice(c, 2 * c), tail0)):
            ra.ring_attn_step(q[:, part], k_pre, v_pre, o[:, part], lse[:, part], q_pos0=q0,
                              k_pos0=0, causal=True)
    jobs = [dict(q=q[:, :c], o=o[:, :c], lse=lse[:, :c], q_pos0=head0, accumulate=accumulate,
                 segments=[(k_head, v_head, head0)]),
            dict(q=q[:, c:], o=o[:, c:], lse=lse[:, c:], q_pos0=tail0, accumulate=accumulate,
                 segments=[(k_head, v_head, head0), (k_tail, v_tail, tail0)])]
    ra.ring_attn_step_jobs(jobs, causal=True)
    torch.cuda.synchronize()
    heads, kv_heads = [5, 62], [0, 7]            # q-head h reads kv-head h // 8
    q64 = host64(q)[:, :, heads]
    k64, v64 = host64(k)[:, :, kv_heads], host64(v)[:, :, kv_heads]
    pos = np.concatenate([head0 + np.arange(c), tail0 + np.arange(c)])
    kpos = pos
    if accumulate:
        k64 = np.concatenate([host64(k_pre)[:, :, kv_heads], k64], 1)
        v64 = np.concatenate([host64(v_pre)[:, :, kv_heads], v64], 1)
        kpos = np.concatenate([np.arange(pre), pos])
    ro, rl = oracle.attention_ref(q64, k64, v64, pos, kpos, True)
    compare(host64(o)[:, :, heads], host64(lse)[:, :, heads], ro, rl, BF16_O, BF16_LSE,
            "paired large grid")


# Seeds chosen so that, on a 256-CU device, the launches cover the large-grid
# paired (49, 1), 4-wave plain (5, 32), 8-wave paired (114, 159, 338) and
# 8-wave plain (13, 3) forms, with both head dims and accumulate on and off.
@pytest.mark.parametrize("seed", [49, 1, 5, 32, 114, 159, 338, 13, 3])
def test_jobs_random_diagonal_steps(ra, seed):
    """Seeded random head-tail diagonal steps (two jobs, the tail job over two
    segments): part lengths 64..2400, 16..64 query heads, MHA or GQA, d 64
    or 128, fresh or accumulating.  Small and large grids, paired and not,
    as the host's cost model decides; sampled heads against the oracle."""
    rng = np.random.default_rng(1000 + seed)
    c = int(rng.integers(64, 2401))
    d = int(rng.choice([64, 128]))
    hq = int(rng.choice([16, 32, 64]))
    hkv = int(rng.choice([hq, 8]))
    accumulate = bool(rng.integers(0, 2))
    pre = int(rng.integers(1, 130))
    gap = int(rng.integers(1, 8))            # the tail part sits gap parts after the head
    say(f"seed {seed}: c={c} d={d} hq={hq} hkv={hkv} acc={accumulate} pre={pre} gap={gap}")
    cfg = 300 + seed
    q, _ = tensor(cfg, 1, 0, (1, 2 * c, hq, d), torch.bfloat16)
    k, _ = tensor(cfg, 2, 0, (1, 2 * c, hkv, d), torch.bfloat16)
    v, _ = tensor(cfg, 3, 0, (1, 2 * c, hkv, d), torch.bfloat16)
    k_pre, _ = tensor(cfg, 4, 0, (1, pre, hkv, d), torch.bfloat16)
    v_pre, _ = tensor(cfg, 5, 0, (1, pre, hkv, d), torch.bfloat16)
    o = torch.empty((1, 2 * c, hq, d), device="cuda")
    lse = torch.empty((1, 2 * c, hq), device="cuda")
    head0, tail0 = pre, pre + gap * c
    k_head, v_head = k[:, :c].contiguous(), v[:, :c].contiguous()
    k_tail, v_tail = k[:, c:].contiguous(), v[:, c:].contiguous()
    if accumulate:
        for part, q0 in ((slice(0, c), head0), (slice(c, 2 * c), tail0)):
            ra.ring_attn_step(q[:, part], k_pre, v_pre, o[:, part], lse[:, part], q_pos0=q0,
                              k_pos0=0, causal=True)
    jobs = [dict(q=q[:, :c], o=o[:, :c], lse=lse[:, :c], q_pos0=head0, accumulate=accumulate,
                 segments=[(k_head, v_head, head0)]),
            dict(q=q[:, c:], o=o[:, c:], lse=lse[:, c:], q_pos0=tail0, accumulate=accumulate,
                 segments=[(k_head, v_head, head0), (k_tail, v_tail, tail0)])]
    ra.ring_attn_step_jobs(jobs, causal=True)
    torch.cuda.synchronize()
    group = hq // hkv
    heads = sorted({0, int(rng.integers(0, hq)), hq - 1})
    kv_heads = [h // group for h in heads]
    q64 = host64(q)[:, :, heads]
    k64, v64 = host64(k)[:, :, kv_heads], host64(v)[:, :, kv_heads]
    pos = np.concatenate([head0 + np.arange(c), tail0 + np.arange(c)])
    kpos = pos
    if accumulate:
        k64 = np.concatenate([host64(k_pre)[:, :, kv_heads], k64], 1)
        v64 = np.concatenate([host64(v_pre)[:, :, kv_heads], v64], 1)
        kpos = np.concatenate([np.arange(pre), pos])
    ro, rl = oracle.attention_ref(q64, k64, v64, pos, kpos, True)
    compare(host64(o)[:, :, heads], host64(lse)[:, :, heads], ro, rl, BF16_O, BF16_LSE,
            f"random diagonal step {seed}")


def _decode_paged_case(ra, cfg, B, ctx_lens, n_shards, hq, hkv, bs, il, spare_blocks,
                       drop=None, fill=0.0):
    """Paged caches: each request has its own block table (a random choice of
    physical blocks, the same ids in every shard's pool, as the slot mapping
    places them); tokens go to pool[dev, table[vb] * bs + loc].  drop=(s, b, j)
    points entry j of (shard s, request b) outside the pool: those tokens
    must take no part."""
    d = 128
    tmax = max(ctx_lens)
    vbs = bs * n_shards
    n_vb = [-(-L // vbs) for L in ctx_lens]
    num_blocks = sum(n_vb) + spare_blocks
    max_blocks = max(n_vb) + 1
    rng = np.random.default_rng(cfg)
    perm = rng.permutation(num_blocks).astype(np.int32)
    q, q64 = tensor(cfg, 1, 0, (B, hq, d), torch.bfloat16)
    k_ctx, k64 = tensor(cfg, 2, 0, (B, tmax, hkv, d), torch.bfloat16)
    v_ctx, v64 = tensor(cfg, 3, 0, (B, tmax, hkv, d), torch.bfloat16)
    kp = torch.full((n_shards, num_blocks, bs, hkv, d), fill, dtype=torch.bfloat16, device="cuda")
    vp = torch.full_like(kp, fill)
    tables = np.full((n_shards, B, max_blocks), -1, dtype=np.int32)
    lens = np.zeros((n_shards, B), dtype=np.int64)
    devs, used = [], 0
    for b, L in enumerate(ctx_lens):
        table = perm[used:used + n_vb[b]]
        used += n_vb[b]
        dev, slot = ra.slot_mapping(np.arange(L), bs, il, n_shards, 1, block_table=table)
        devs.append(dev)
        lens[:, b] = np.bincount(dev, minlength=n_shards)
        tables[:, b, :n_vb[b]] = table
        dev_t = torch.from_numpy(dev.astype(np.int64)).cuda()
        slot_t = torch.from_numpy(slot).cuda()
        kp.view(n_shards, num_blocks * bs, hkv, d)[dev_t, slot_t] = k_ctx[b, :L]
        vp.view(n_shards, num_blocks * bs, hkv, d)[dev_t, slot_t] = v_ctx[b, :L]
    if drop is not None:
        s, b, j = drop
        tables[s, b, j] = num_blocks + 5          # outside the pool
    tables_t = torch.from_numpy(tables).cuda()
    lens_t = torch.from_numpy(lens).cuda()
    o_parts, lse_parts = ra.split_kv_decode_paged(q, kp, vp, tables_t, lens_t)
    o, lse = ra.lse_merge(o_parts, lse_parts)
    torch.cuda.synchronize()
    for b, L in enumerate(ctx_lens):
        dev_ref, slot_ref = oracle.slot_mapping_ref(np.arange(L), bs, il, n_shards, 1)
        dev_ref = np.asarray(dev_ref).copy()
        if drop is not None and drop[1] == b:
            s, _, j = drop
            # local block j of shard s holds the tokens with local index in [j*bs, (j+1)*bs)
            dev_ref[(dev_ref == s) & (np.asarray(slot_ref) // bs == j)] = -1
        po, pl, mo, ml = oracle.decode_shards_ref(q64[b:b + 1], k64[b:b + 1, :L], v64[b:b + 1, :L],
                                                  dev_ref, n_shards)
        compare(host64(o_parts[:, b]), host64(lse_parts[:, b]), po[:, 0], pl[:, 0], BF16_O,
                BF16_LSE, f"paged partials b={b}")
        compare(host64(o[b]), host64(lse[b]), mo[0], ml[0], BF16_O, BF16_LSE, f"paged b={b}")


def test_split_kv_decode_paged(ra):
    say("paged decode: 8 shards, 3 ragged requests, random block tables, GQA 8")
    _decode_paged_case(ra, 44, 3, [4096, 1500, 3000], 8, 16, 2, 128, 16, spare_blocks=7)


def test_split_kv_decode_paged_splits_and_small_blocks(ra):
    say("paged decode: 2 shards, blocks of 32, key splits")
    assert ra.split_kv_decode_workspace(2, 1, 4, 1, 128, 300 * 32) > 0
    _decode_paged_case(ra, 45, 1, [16384 - 77], 2, 4, 1, 32, 8, spare_blocks=40)


def test_split_kv_decode_paged_entry_outside_pool(ra):
    say("paged decode: one table entry outside the pool is an empty block")
    _decode_paged_case(ra, 46, 2, [2048, 1000], 4, 8, 1, 64, 16, spare_blocks=3, drop=(1, 0, 2))


def test_split_kv_decode_paged_nan_past_shard_ends(ra):
    # pool rows no token occupies (block tails, spare blocks) are NaN
    say("paged decode: NaN in every unoccupied pool row")
    _decode_paged_case(ra, 48, 3, [4096, 1500, 77], 8, 16, 2, 128, 16, spare_blocks=5, fill=float("nan"))



def test_gather_rows_out_of_range_is_zero(ra):
    src = torch.randn((50, 3, 8), device="cuda")
    idx = torch.tensor([4, -1, 49, 50, 0, 4], dtype=torch.int64, device="cuda")
    out = ra.gather_rows(src, idx)
    torch.cuda.synchronize()
    for i, j in enumerate([4, -1, 49, 50, 0, 4]):
        want = src[j] if 0 <= j < 50 else torch.zeros_like(src[0])
        assert torch.equal(out[i], want)


# (rows, bytes per row): more rows than the grid's 262,144 waves (waves loop
# over rows); a row just past one 48 KiB burst per wave (a ragged second
# round); rows of several bursts
@pytest.mark.parametrize("n,row_bytes", [(300001, 16), (37, 48 * 1024 + 16), (5, 200 * 1024 + 48)])
def test_gather_rows_bursts_and_grid_stride(ra, n, row_bytes):
    say(f"gather rows n={n} row_bytes={row_bytes}")
    g = torch.Generator(device="cuda").manual_seed(n)
    src = torch.randint(-2**31, 2**31 - 1, (n, row_bytes // 4), dtype=torch.int32, device="cuda", generator=g)
    idx = torch.randint(0, n, (n,), dtype=torch.int64, device="cuda", generator=g)
    idx[0], idx[-1] = n - 1, -3                    # the last source row; one index out of range
    out = ra.gather_rows(src, idx)
    torch.cuda.synchronize()
    want = src[idx.clamp(min=0)]
    want[-1] = 0
    assert torch.equal(out, want)


# (q_len, k_len, q_pos0, k_pos0) of packed requests: self-causal, single
# token, no queries, chunk tail over a long prefix, no keys, all keys later
# (nothing visible), ragged tails past the tile size.
VARLEN_REQS = [(300, 300, 0, 0), (1, 1, 7, 7), (0, 50, 0, 0), (130, 1131, 1001, 0), (64, 0, 0, 0),
               (257, 100, 0, 500), (129, 200, 3000, 2900)]


def _varlen_case(ra, cfg, reqs, hq, hkv, dqk, dv, causal=True, split_keys=False):
    n = len(reqs)
    cq = np.concatenate([[0], np.cumsum([r[0] for r in reqs])]).astype(np.int64)
    ck = np.concatenate([[0], np.cumsum([r[1] for r in reqs])]).astype(np.int64)
    pq = np.array([r[2] for r in reqs], dtype=np.int64)
    pk = np.array([r[3] for r in reqs], dtype=np.int64)
    q, q64 = tensor(cfg, 1, 0, (int(cq[-1]), hq, dqk), torch.bfloat16)
    k, k64 = tensor(cfg, 2, 0, (int(ck[-1]), hkv, dqk), torch.bfloat16)
    v, v64 = tensor(cfg, 3, 0, (int(ck[-1]), hkv, dv), torch.bfloat16)
    if not split_keys:
        o, lse = ra.ring_attn_step_varlen(q, k, v, cq, ck, pq, pk, causal=causal)
    else:
        # first half of every request's keys, then the second half merged in
        half = np.array([r[1] // 2 for r in reqs], dtype=np.int64)
        ck1 = np.concatenate([[0], np.cumsum(half)])
        ck2 = np.concatenate([[0], np.cumsum([r[1] - h for r, h in zip(reqs, half)])])
        sel1 = np.concatenate([np.arange(ck[i], ck[i] + half[i]) for i in range(n)]).astype(np.int64)
        sel2 = np.concatenate([np.arange(ck[i] + half[i], ck[i + 1]) for i in range(n)]).astype(np.int64)
        k1, v1 = k[torch.from_numpy(sel1).cuda()].contiguous(), v[torch.from_numpy(sel1).cuda()].contiguous()
        k2, v2 = k[torch.from_numpy(sel2).cuda()].contiguous(), v[torch.from_numpy(sel2).cuda()].contiguous()
        o, lse = ra.ring_attn_step_varlen(q, k1, v1, cq, ck1, pq, pk, causal=causal)
        ra.ring_attn_step_varlen(q, k2, v2, cq, ck2, pq, pk + half, o=o, lse=lse, causal=causal,
                                 accumulate=True)
    torch.cuda.synchronize()
    o64, l64 = host64(o), host64(lse)
    for i, (lq, lk, q0, k0) in enumerate(reqs):
        if lq == 0:
            continue
        rows = slice(int(cq[i]), int(cq[i + 1]))
        keys = slice(int(ck[i]), int(ck[i + 1]))
        if lk:
            ro, rl = oracle.attention_ref(q64[None, rows], k64[None, keys], v64[None, keys],
                                          q0 + np.arange(lq), k0 + np.arange(lk), causal)
        else:
            ro, rl = np.zeros((1, lq, hq, dv)), np.full((1, lq, hq), -np.inf)
        compare(o64[None, rows], l64[None, rows], ro, rl, BF16_O, BF16_LSE, f"varlen request {i}")


@pytest.mark.parametrize("dqk,dv,hq,hkv", [(128, 128, 4, 2), (64, 64, 2, 2), (192, 128, 2, 1)])
def test_varlen_packed_requests(ra, dqk, dv, hq, hkv):
    say(f"varlen: {len(VARLEN_REQS)} packed requests, d {dqk}/{dv}")
    _varlen_case(ra, 61, VARLEN_REQS, hq, hkv, dqk, dv)


def test_varlen_noncausal_and_accumulate(ra):
    _varlen_case(ra, 62, VARLEN_REQS, 4, 1, 128, 128, causal=False)
    _varlen_case(ra, 63, VARLEN_REQS, 4, 2, 128, 128, split_keys=True)


def test_varlen_more_requests_than_one_launch(ra):
    rng = np.random.default_rng(64)
    reqs = [(int(rng.integers(0, 90)), int(rng.integers(0, 150)), int(rng.integers(0, 200)),
             int(rng.integers(0, 200))) for _ in range(150)]
    _varlen_case(ra, 64, reqs, 2, 1, 128, 128)


def test_allgather_kv_reorg_then_segmented_prefill(ra):
    """All-gather-KV chunked prefill: each device's KV buffer lists the
    requests in order (tokens by slot), the all-gather concatenates the
    devices, the reorganisation gathers every request back into one
    contiguous, in-order block (bit for bit), and the chunk's queries then
    attend segment by segment over it."""
    lens, bs, il, pcp, dcp, hq, hkv, d = [700, 257, 1500], 32, 8, 1, 4, 4, 2, 128
    W = pcp * dcp
    ks, vs, k64s, v64s = [], [], [], []
    for r, L in enumerate(lens):
        k, k64 = tensor(70 + r, 2, 0, (L, hkv, d), torch.bfloat16)
        v, v64 = tensor(70 + r, 3, 0, (L, hkv, d), torch.bfloat16)
        ks.append(k); vs.append(v); k64s.append(k64); v64s.append(v64)
    dev_k, dev_v = [], []
    for dv_ in range(W):                     # each device's buffer, built by concatenation
        pk, pv = [], []
        for r, L in enumerate(lens):
            dev, slot = ra.slot_mapping(np.arange(L), bs, il, pcp, dcp)
            mine = np.nonzero(dev == dv_)[0]
            order = torch.from_numpy(mine[np.argsort(slot[mine], kind="stable")]).cuda()
            pk.append(ks[r][order]); pv.append(vs[r][order])
        dev_k.append(torch.cat(pk)); dev_v.append(torch.cat(pv))
    gathered_k, gathered_v = torch.cat(dev_k).contiguous(), torch.cat(dev_v).contiguous()   # all-gather
    src, _ = ra.reorg_index(lens, bs, il, pcp, dcp)
    src_t = torch.from_numpy(src).cuda()
    k_r = ra.gather_rows(gathered_k, src_t)
    v_r = ra.gather_rows(gathered_v, src_t)
    torch.cuda.synchronize()
    assert torch.equal(k_r, torch.cat(ks)) and torch.equal(v_r, torch.cat(vs))
    # the last request's final 200 tokens are the chunk: causal over its whole context
    r, L, sq = 2, lens[2], 200
    off = sum(lens[:r])
    q, q64 = tensor(79, 1, 0, (1, sq, hq, d), torch.bfloat16)
    o = torch.empty((1, sq, hq, d), device="cuda")
    lse = torch.empty((1, sq, hq), device="cuda")
    ra.segmented_prefill(q, k_r[None, off:off + L], v_r[None, off:off + L], o, lse, q_pos0=L - sq,
                         segment=512)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_ref(q64, k64s[r][None], v64s[r][None], L - sq + np.arange(sq), np.arange(L),
                                  True)
    compare(host64(o), host64(lse), ro, rl, BF16_O, BF16_LSE, "reorganised chunk")


# Launch shapes that give an XCD more than one round of workgroups, so the
# workgroups of odd rounds sweep their keys backwards (serpentine order):
# the 8-wave key-split mode (288 workgroups), the 4-wave mode (768) and the
# 256-row mode (1,024), causal with a diagonal and ragged tails.  The oracle
# runs on a few heads of each.
SERPENTINE = [
    # (sq, sk, hq, hkv, dqk, dv, q_pos0, k_pos0)
    (384, 700, 96, 96, 128, 128, 300, 0),      # 8-wave key split, 2 rounds
    (768, 650, 128, 16, 64, 64, 400, 100),     # 4-wave, 2 rounds
    (1000, 520, 256, 32, 128, 128, 200, 0),    # 256-row, 4 rounds, ragged rows
    (1000, 300, 256, 256, 192, 128, 250, 100), # 256-row d 192
    # the same launch forms with whole 64-key tiles only (the kernels that keep
    # one descriptor per segment; the ragged cases above run the per-tile ones)
    (384, 704, 96, 96, 128, 128, 300, 0),
    (768, 640, 128, 16, 64, 64, 400, 100),
    (1000, 512, 256, 32, 128, 128, 200, 0),
    (1000, 320, 256, 256, 192, 128, 250, 100),
]


@pytest.mark.parametrize("idx", range(len(SERPENTINE)))
def test_serpentine_rounds_match_oracle(ra, idx):
    sq, sk, hq, hkv, dqk, dv, q0, k0 = SERPENTINE[idx]
    say(f"serpentine case {idx}: sq={sq} sk={sk} hq={hq} hkv={hkv} d=({dqk},{dv}) q0={q0} k0={k0}")
    cfg = 300 + idx
    q, q64 = tensor(cfg, 1, 0, (1, sq, hq, dqk), torch.bfloat16)
    k, k64 = tensor(cfg, 2, 0, (1, sk, hkv, dqk), torch.bfloat16)
    v, v64 = tensor(cfg, 3, 0, (1, sk, hkv, dv), torch.bfloat16)
    o = torch.empty((1, sq, hq, dv), device="cuda")
    lse = torch.empty((1, sq, hq), device="cuda")
    scale = 1.0 / np.sqrt(dqk)
    ra.ring_attn_step(q, k, v, o, lse, q0, k0, True, scale, accumulate=False)
    torch.cuda.synchronize()
    o_h, lse_h = host64(o), host64(lse)
    group = hq // hkv
    for h in sorted({0, 1, hq // 2 + 3, hq - 1}):
        o_ref, lse_ref = oracle.attention_ref(q64[:, :, h:h + 1], k64[:, :, h // group:h // group + 1],
                                              v64[:, :, h // group:h // group + 1], q0 + np.arange(sq),
                                              k0 + np.arange(sk), True, scale)
        compare(o_h[:, :, h:h + 1], lse_h[:, :, h:h + 1], o_ref, lse_ref, BF16_O, BF16_LSE,
                f"serpentine {idx} head {h}")
