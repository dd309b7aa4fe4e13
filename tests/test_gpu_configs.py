"""Parity at the five workloads' full sizes, in the launch configuration the
bench times, checked against the oracle on sampled outputs.

Each sampled row of attention depends only on its own query row and the keys
visible to it, so the oracle evaluated on those rows is exact for them.
  C1  tiny non-causal ring, fp32: every row.
  C2  zigzag rank 0, seq 8192, cp 4: every row of 6 of the 32 heads, plus
      the restore index bit for bit; all four ranks gathered and restored
      on the device: every row of 4 heads.
  C3  GQA decode over 8 shards, 64 x 131072: per-shard partials and merged
      output of 3 whole requests (all heads), over contiguous shards and over
      paged pools read through block tables.
  C4  zigzag rank 0 of 1M tokens, cp 8: 512 (token, head) rows covering both
      Q chunks, chunk edges, tile edges, the diagonal, and all 64 heads of a
      few tokens; rank 7 of the same ring (both query parts busy at every
      step): 162 rows.
  C5  segmented chunked prefill (MLA shape): 541 (token, head) rows.
The standalone merge (2 x 8,388,608 rows x 128), the reorganisation gather
(135,168 K and V rows) and the packed 16-request prefill (69,952 tokens) are
checked at the sizes the bench times.
C4 (ranks 0 and 7) and C5 are also checked over every row, on the device, for properties any
correct output has (finite; inside the range of its kv head's V; LSE between
the score of a key every row sees and the largest possible score plus the
log of the number of keys seen).
"""

import numpy as np
import pytest

import oracle
from gpu_util import host64, compare, say, tensor, whole_output_properties, F32_O, BF16_O, BF16_LSE

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    import ring_attention_02_amd as ra
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    return ra


def _release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_c1_tiny_noncausal_ring(ra):
    import workloads
    from seeded_inputs import CONFIGS
    c = CONFIGS[1]
    shape = (c["batch"], c["seq"], c["heads"], c["d"])
    q = workloads.host_tensor(1, 1, 0, shape, torch.float32)
    k = workloads.host_tensor(1, 2, 0, shape, torch.float32)
    v = workloads.host_tensor(1, 3, 0, shape, torch.float32)
    o, lse = ra.noncausal_ring_sweep(q, k, v, c["n_blocks"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ref(host64(q), host64(k), host64(v), causal=False)
    compare(host64(o), host64(lse), o_ref, lse_ref, F32_O, F32_O, "C1")


def _sampled_rows_check(o, lse, q64_rows, k_of, v_of, q_pos, heads, groups, what,
                        k_pos=None):
    """Compare sampled (row, head) outputs: rows grouped by kv head.

    q64_rows: [n, d] float64 query rows; heads: [n] query head of each row;
    k_of(kvh) / v_of(kvh): float64 [Sk, d] keys / values of that kv head.
    """
    kvh_of = heads // groups
    for kvh in np.unique(kvh_of):
        sel = np.nonzero(kvh_of == kvh)[0]
        kk, vv = k_of(int(kvh)), v_of(int(kvh))
        pos = np.arange(kk.shape[0]) if k_pos is None else k_pos
        ro, rl = oracle.attention_ref(q64_rows[sel][None, :, None, :], kk[None, :, None, :],
                                      vv[None, :, None, :], q_pos[sel], pos, causal=True)
        compare(o[sel], lse[sel], ro[0, :, 0], rl[0, :, 0], BF16_O, BF16_LSE,
                f"{what} kv head {kvh} ({len(sel)} rows)")


def test_c2_zigzag_full(ra):
    import workloads
    w = workloads.zigzag_setup(2)
    ref_local, ref_restore = oracle.partition_ref([w["seq"]], w["cp"])
    assert np.array_equal(w["local"], ref_local[w["rank"]])
    assert np.array_equal(w["restore"], ref_restore)
    graph = w["ring"].capture(w["q_local"], w["o"], w["lse"])     # the bench's launch mode
    w["o"].fill_(5.0)
    graph.replay()
    torch.cuda.synchronize()
    o, lse = host64(w["o"][0]), host64(w["lse"][0])
    q, k, v = host64(w["q_local"][0]), host64(w["k_full"][0]), host64(w["v_full"][0])
    q_pos = np.asarray(w["local"])
    for h in (0, 5, 13, 20, 27, 31):
        ro, rl = oracle.attention_ref(q[None, :, h:h + 1], k[None, :, h:h + 1], v[None, :, h:h + 1],
                                      q_pos, np.arange(w["seq"]), causal=True)
        compare(o[:, h], lse[:, h], ro[0, :, 0], rl[0, :, 0], BF16_O, BF16_LSE, f"C2 head {h}")
    del w, graph
    _release()


def test_c2_every_rank_restored_on_device(ra):
    """All four ranks of the 8192-token ring at full size (each in its own
    ring order and step shapes), their outputs gathered in rank order and
    put back in token order with the restore index on the device; every row
    of 4 heads against full causal attention over the sequence."""
    import workloads
    outs_o, outs_l, restore = [], [], None
    q_full = None
    for r in range(4):
        w = workloads.zigzag_setup(2, rank=r)
        w["ring"].run(w["q_local"], w["o"], w["lse"])
        outs_o.append(w["o"][0])
        outs_l.append(w["lse"][0])
        if q_full is None:
            q_full = torch.empty((w["seq"], w["hq"], w["d"]), dtype=torch.bfloat16, device="cuda")
            k_full, v_full, restore = w["k_full"][0], w["v_full"][0], w["restore"]
        q_full[torch.as_tensor(np.asarray(w["local"]), device="cuda")] = w["q_local"][0]
        say(f"C2 rank {r}: {w['q_local'].shape[1]} local tokens")
    idx = torch.from_numpy(np.asarray(restore)).cuda()
    o = ra.gather_rows(torch.cat(outs_o, 0), idx)
    lse = ra.gather_rows(torch.cat(outs_l, 0), idx)
    torch.cuda.synchronize()
    seq = q_full.shape[0]
    for h in (0, 9, 22, 31):
        ro, rl = oracle.attention_ref(host64(q_full[None, :, h:h + 1]), host64(k_full[None, :, h:h + 1]),
                                      host64(v_full[None, :, h:h + 1]), np.arange(seq), np.arange(seq), causal=True)
        compare(host64(o[:, h]), host64(lse[:, h]), ro[0, :, 0], rl[0, :, 0], BF16_O, BF16_LSE,
                f"C2 all ranks head {h}")
    _release()


def test_c3_decode_full(ra):
    import workloads
    w = workloads.decode_setup()
    o_parts, lse_parts = ra.split_kv_decode(w["q"], w["ks"], w["vs"], shard_lens=w["lens"])
    o, lse = ra.lse_merge(o_parts, lse_parts)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    dev_ref, slot_ref = oracle.slot_mapping_ref(np.arange(w["ctx"]), 128, 16, 8, 1)
    assert np.array_equal(w["dev"], dev_ref) and np.array_equal(w["slot"], slot_ref)
    q64 = host64(w["q"])
    for b in (0, 37, 63):
        kc, vc = workloads.decode_context(b)
        k64, v64 = host64(kc)[None], host64(vc)[None]
        del kc, vc
        po, pl, mo, ml = oracle.decode_shards_ref(q64[b:b + 1], k64, v64, dev_ref, w["n_shards"])
        compare(host64(o_parts[:, b]), host64(lse_parts[:, b]), po[:, 0], pl[:, 0], BF16_O,
                BF16_LSE, f"C3 request {b} shard partials")
        compare(host64(o[b]), host64(lse[b]), mo[0], ml[0], BF16_O, BF16_LSE, f"C3 request {b}")
    del w
    _release()


def test_c3_decode_paged_full(ra):
    """C3 as benched in the paged layout: 8 pools of 128-token blocks, each
    request's virtual blocks at a seeded random choice of physical blocks,
    4,096 work items (no key splits: partials straight to o_parts).  Sampled
    requests against the oracle, shard partials and merged result."""
    import workloads
    w = workloads.decode_paged_setup()
    assert ra.split_kv_decode_workspace(w["n_shards"], w["B"], w["hq"], w["hkv"], w["d"],
                                        w["tables"].shape[2] * w["kp"].shape[2]) == 0
    o_parts, lse_parts = ra.split_kv_decode_paged(w["q"], w["kp"], w["vp"], w["tables"], w["lens"])
    o, lse = ra.lse_merge(o_parts, lse_parts)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    tables = w["tables"].cpu().numpy()
    q64 = host64(w["q"])
    for b in (0, 37, 63):
        # the pools were filled through the library's slot mapping; the oracle's agrees
        dev_ref, slot_ref = oracle.slot_mapping_ref(np.arange(w["ctx"]), 128, 16, 8, 1,
                                                    block_table=tables[0, b])
        dev, slot = ra.slot_mapping(np.arange(w["ctx"]), 128, 16, 8, 1, block_table=tables[0, b])
        assert np.array_equal(dev, dev_ref) and np.array_equal(slot, slot_ref)
        kc, vc = workloads.decode_context(b)
        k64, v64 = host64(kc)[None], host64(vc)[None]
        del kc, vc
        po, pl, mo, ml = oracle.decode_shards_ref(q64[b:b + 1], k64, v64, dev_ref, w["n_shards"])
        compare(host64(o_parts[:, b]), host64(lse_parts[:, b]), po[:, 0], pl[:, 0], BF16_O,
                BF16_LSE, f"C3 paged request {b} shard partials")
        compare(host64(o[b]), host64(lse[b]), mo[0], ml[0], BF16_O, BF16_LSE, f"C3 paged request {b}")
    del w
    _release()


def test_c4_long_zigzag_sampled(ra):
    import workloads
    w = workloads.zigzag_setup(4)
    w["ring"].run(w["q_local"], w["o"], w["lse"])
    torch.cuda.synchronize()
    c, hq, hkv = w["chunk"], w["hq"], w["hkv"]
    n_local = w["q_local"].shape[1]
    rng = np.random.default_rng(4)
    toks = {0, 1, 63, 64, 127, 128, c - 1, c, c + 1, c + 63, c + 64, 2 * c - 1, c // 2}
    toks |= set(rng.integers(0, n_local, 30).tolist())
    rows = []
    for t in sorted(toks):
        for h in rng.choice(hq, 8, replace=False):
            rows.append((t, int(h)))
    for t in (0, c - 1, 2 * c - 1):            # every head of a few tokens
        rows += [(t, h) for h in range(hq)]
    rows = sorted(set(rows))
    assert len(rows) >= 512
    tt = np.array([r[0] for r in rows])
    hh = np.array([r[1] for r in rows])
    ti, hi = torch.from_numpy(tt).cuda(), torch.from_numpy(hh).cuda()
    o = host64(w["o"][0][ti, hi])
    lse = host64(w["lse"][0][ti, hi])
    q_rows = host64(w["q_local"][0][ti, hi])
    q_pos = np.asarray(w["local"])[tt]
    say(f"C4: {len(rows)} sampled rows")
    k_full, v_full = w["k_full"], w["v_full"]
    _sampled_rows_check(o, lse, q_rows, lambda g: host64(k_full[0, :, g]),
                        lambda g: host64(v_full[0, :, g]), q_pos, hh, hq // hkv, "C4")
    qp = torch.as_tensor(np.asarray(w["local"]), device="cuda")
    whole_output_properties(w["o"][0], w["lse"][0], w["q_local"][0], k_full[0], v_full[0], qp, 0,
                             hq // hkv, 1.0 / np.sqrt(w["d"]), "C4")
    del w, k_full, v_full
    _release()


def test_c4_last_rank_sampled(ra):
    """Rank 7 of the same 1M-token ring: its head part (chunk 7) sees a part
    of every block it receives and its tail part (chunk 8) only the head
    chunks, so every step runs both query parts (rank 0's head part is done
    after step 0).  Sampled rows against the oracle, every row checked for
    the whole-output properties."""
    import workloads
    w = workloads.zigzag_setup(4, rank=7)
    w["ring"].run(w["q_local"], w["o"], w["lse"])
    torch.cuda.synchronize()
    c, hq, hkv = w["chunk"], w["hq"], w["hkv"]
    n_local = w["q_local"].shape[1]
    rng = np.random.default_rng(47)
    toks = {0, 1, 64, c - 1, c, c + 1, 2 * c - 1} | set(rng.integers(0, n_local, 20).tolist())
    rows = sorted({(t, int(h)) for t in toks for h in rng.choice(hq, 6, replace=False)})
    tt = np.array([r[0] for r in rows])
    hh = np.array([r[1] for r in rows])
    ti, hi = torch.from_numpy(tt).cuda(), torch.from_numpy(hh).cuda()
    o, lse = host64(w["o"][0][ti, hi]), host64(w["lse"][0][ti, hi])
    q_rows = host64(w["q_local"][0][ti, hi])
    q_pos = np.asarray(w["local"])[tt]
    say(f"C4 rank 7: {len(rows)} sampled rows")
    k_full, v_full = w["k_full"], w["v_full"]
    _sampled_rows_check(o, lse, q_rows, lambda g: host64(k_full[0, :, g]),
                        lambda g: host64(v_full[0, :, g]), q_pos, hh, hq // hkv, "C4 rank 7")
    qp = torch.as_tensor(np.asarray(w["local"]), device="cuda")
    whole_output_properties(w["o"][0], w["lse"][0], w["q_local"][0], k_full[0], v_full[0], qp, 0,
                            hq // hkv, 1.0 / np.sqrt(w["d"]), "C4 rank 7")
    del w, k_full, v_full
    _release()


def test_c5_segmented_sampled(ra):
    import workloads
    w = workloads.segmented_setup()
    ra.segmented_prefill(w["q"], w["k"], w["v"], w["o"], w["lse"], q_pos0=w["q_pos0"],
                         segment=w["segment"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    sq, h = w["sq"], w["h"]
    heads = rng.choice(h, 16, replace=False)
    rows = []
    for hd in heads:
        toks = {0, 1, 63, 64, 127, sq - 1, sq // 2} | set(rng.integers(0, sq, 27).tolist())
        rows += [(t, int(hd)) for t in sorted(toks)]
    rows = sorted(set(rows))
    assert len(rows) >= 512
    tt = np.array([r[0] for r in rows])
    hh = np.array([r[1] for r in rows])
    ti, hi = torch.from_numpy(tt).cuda(), torch.from_numpy(hh).cuda()
    o = host64(w["o"][0][ti, hi])
    lse = host64(w["lse"][0][ti, hi])
    q_rows = host64(w["q"][0][ti, hi])
    q_pos = w["q_pos0"] + tt
    say(f"C5: {len(rows)} sampled rows")
    k, v = w["k"], w["v"]
    _sampled_rows_check(o, lse, q_rows, lambda g: host64(k[0, :, g]), lambda g: host64(v[0, :, g]),
                        q_pos, hh, 1, "C5")
    qp = w["q_pos0"] + torch.arange(sq, device="cuda")
    whole_output_properties(w["o"][0], w["lse"][0], w["q"][0], k[0], v[0], qp, 0, 1,
                             1.0 / np.sqrt(w["dqk"]), "C5")
    del w, k, v
    _release()


@pytest.mark.parametrize("dqk,dv,hq,hkv", [(128, 128, 4, 2), (64, 64, 4, 4), (192, 128, 4, 1)])
def test_large_grid_ragged_sampled(ra, dqk, dv, hq, hkv):
    """A grid large enough for the 256-row workgroups (130 full row tiles and
    a ragged 37-row tail, 4 heads), causal with a position offset between Q
    and K; sampled rows against the oracle (tile edges, the tail, random)."""
    sq, sk, q0 = 256 * 130 + 37, 256 * 130 + 37 + 500, 500
    q, _ = tensor(81, 1, 0, (1, sq, hq, dqk), torch.bfloat16)
    k, _ = tensor(81, 2, 0, (1, sk, hkv, dqk), torch.bfloat16)
    v, _ = tensor(81, 3, 0, (1, sk, hkv, dv), torch.bfloat16)
    o = torch.empty((1, sq, hq, dv), device="cuda")
    lse = torch.empty((1, sq, hq), device="cuda")
    ra.ring_attn_step(q, k, v, o, lse, q_pos0=q0, k_pos0=0, causal=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(81)
    toks = sorted({0, 1, 31, 32, 127, 128, 255, 256, 511, sq - 38, sq - 37, sq - 1}
                  | set(rng.integers(0, sq, 20).tolist()))
    rows = [(t, hd) for t in toks for hd in range(hq)]
    tt = np.array([r[0] for r in rows])
    hh = np.array([r[1] for r in rows])
    ti, hi = torch.from_numpy(tt).cuda(), torch.from_numpy(hh).cuda()
    say(f"large grid d {dqk}/{dv}: {len(rows)} sampled rows")
    _sampled_rows_check(host64(o[0][ti, hi]), host64(lse[0][ti, hi]), host64(q[0][ti, hi]),
                        lambda g: host64(k[0, :, g]), lambda g: host64(v[0, :, g]), q0 + tt, hh,
                        hq // hkv, "large grid")
    del q, k, v, o, lse
    _release()


def test_lse_merge_at_the_benched_size(ra):
    """The standalone merge as benched: 2 partials of the 1M-token share's
    8,388,608 rows x 128 (8.6 GB in).  Sampled rows (the first, the last and
    seeded random ones) against the oracle, every row finite."""
    import seeded_inputs as si
    rows, dv, n = 131072 * 64, 128, 2
    o_parts = si.device_normal(7, 1, 0, (n, rows, dv), torch.float32, "cuda")
    lse_parts = si.device_normal(7, 2, 0, (n, rows), torch.float32, "cuda") * 3
    lse_parts[1, rows - 5:] = float("-inf")             # the last rows: one part empty
    o_parts[1, rows - 5:] = 0.0
    o, lse = ra.lse_merge(o_parts, lse_parts)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(8)
    pick = np.unique(np.concatenate([[0, 1, rows // 2, rows - 6, rows - 5, rows - 1],
                                     rng.integers(0, rows, 2000)]))
    idx = torch.from_numpy(pick).cuda()
    op, lp = host64(o_parts[:, idx]), host64(lse_parts[:, idx])
    o_ref, lse_ref = oracle.lse_merge_ref(list(op), list(lp))
    compare(host64(o[idx]), host64(lse[idx]), o_ref, lse_ref, 1e-5, 1e-5,
            f"merge of 2 x {rows} rows ({len(pick)} sampled)")
    del o_parts, lse_parts, o, lse
    _release()


def test_reorg_gather_at_the_benched_size(ra):
    """The all-gather-KV reorganisation as benched (135,168 tokens of 4
    requests on 8 devices, K 128 x 192 and V 128 x 128 bf16): the row index
    bit for bit against the oracle, and the gathered K and V rows, all of
    them, equal to the source rows the index names (compared on the device,
    byte for byte)."""
    import workloads
    w = workloads.reorg_setup()
    src_ref, _ = oracle.reorg_index_ref(w["lens"], 128, 16, 1, 8)
    assert np.array_equal(w["idx"].cpu().numpy(), src_ref)
    ok = ra.gather_rows(w["gk"], w["idx"])
    ov = ra.gather_rows(w["gv"], w["idx"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    pick = np.unique(np.concatenate([[0, 1, w["n"] - 1], rng.integers(0, w["n"], 2000)]))
    for got, src, name in ((ok, w["gk"], "K"), (ov, w["gv"], "V")):
        # sampled rows on the host, against the oracle's index
        g = got[torch.from_numpy(pick).cuda()].view(torch.int16).cpu().numpy()
        e = src[torch.from_numpy(src_ref[pick]).cuda()].view(torch.int16).cpu().numpy()
        assert np.array_equal(g, e), f"{name}: sampled rows differ"
        # every row: dst[i] is src[idx[i]] (the definition), byte for byte on the device
        ref_idx = torch.from_numpy(src_ref).cuda()
        for a0 in range(0, w["n"], 16384):
            exp = src.view(torch.int16)[ref_idx[a0:a0 + 16384]]
            assert torch.equal(got.view(torch.int16)[a0:a0 + 16384], exp), f"{name} rows {a0}.."
    say(f"  reorg gather: {w['n']} K and V rows equal to their source rows")
    del w, ok, ov
    _release()


def test_varlen_at_the_benched_size(ra):
    """The packed 16-request prefill as benched (lengths 512..8192, 69,952
    tokens, self-causal, GQA 32/8, d 128): per request, sampled rows against
    the oracle and every row checked for the whole-output properties."""
    import workloads
    w = workloads.varlen_setup()
    ra.ring_attn_step_varlen(w["q"], w["k"], w["v"], w["cu"], w["cu"], w["pos"], w["pos"],
                             o=w["o"], lse=w["lse"], causal=True)
    torch.cuda.synchronize()
    hq, hkv, d = w["hq"], w["hkv"], w["d"]
    group, scale = hq // hkv, 1.0 / np.sqrt(d)
    rng = np.random.default_rng(12)
    for r, L in enumerate(w["lens"]):
        a0, L = int(w["cu"][r]), int(L)
        sl = slice(a0, a0 + L)
        whole_output_properties(w["o"][sl], w["lse"][sl], w["q"][sl], w["k"][sl], w["v"][sl],
                                torch.arange(L, device="cuda"), 0, group, scale, f"varlen request {r}")
        toks = np.unique(np.array([0, 1, 63, 64, L // 2, L - 1] + rng.integers(0, L, 4).tolist()))
        heads = np.array([0, hq - 1, int(rng.integers(0, hq))])
        for h in np.unique(heads):
            kvh = int(h) // group
            k64, v64 = host64(w["k"][sl, kvh]), host64(w["v"][sl, kvh])
            ti = torch.from_numpy(a0 + toks).cuda()
            q64 = host64(w["q"][ti, int(h)])
            ro, rl = oracle.attention_ref(q64[None, :, None, :], k64[None, :, None, :], v64[None, :, None, :],
                                          toks, np.arange(L), causal=True)
            compare(host64(w["o"][ti, int(h)]), host64(w["lse"][ti, int(h)]), ro[0, :, 0], rl[0, :, 0],
                    BF16_O, BF16_LSE, f"varlen request {r} (L={L}) head {h}")
    del w
    _release()
