"""Pins of the CPU oracle against facts other than itself.

Each test ties an oracle function to something the pages or the
mathematics fix: brute force written with pure-Python loops, closed forms,
a library routine for a special case, the pages' worked rules (fixtures in
tests/golden/) and invariants such as "any blockwise LSE merge equals the
full softmax".  The cases are chosen so that a dropped term, a wrong sign,
index or head mapping, or a transposed operand fails at least one test.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import (attention_ref, lse_merge_ref, decode_shards_ref, partition_ref,
                    slot_mapping_ref, classify_ref, visible_pairs_ref,
                    ring_schedule_ref, zigzag_ring_chunks_ref, FULL, DIAG, SKIP)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


# ----------------------------------------------------------------------------
# attention_ref: brute force
# ----------------------------------------------------------------------------

def brute_attention(q, k, v, q_pos, k_pos, causal, scale):
    """Direct per-row softmax with math.exp / math.fsum, no numpy reductions."""
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, Dv = v.shape
    group = Hq // Hkv
    o = [[[[0.0] * Dv for _ in range(Hq)] for _ in range(Sq)] for _ in range(B)]
    lse = [[[-math.inf] * Hq for _ in range(Sq)] for _ in range(B)]
    for b in range(B):
        for i in range(Sq):
            for h in range(Hq):
                kvh = h // group
                js = [j for j in range(Sk) if (not causal) or k_pos[j] <= q_pos[i]]
                if not js:
                    continue
                s = {j: scale * math.fsum(float(q[b, i, h, c]) * float(k[b, j, kvh, c])
                                          for c in range(D)) for j in js}
                m = max(s.values())
                w = {j: math.exp(s[j] - m) for j in js}
                tot = math.fsum(w.values())
                for c in range(Dv):
                    o[b][i][h][c] = math.fsum(w[j] * float(v[b, j, kvh, c]) for j in js) / tot
                lse[b][i][h] = m + math.log(tot)
    return np.array(o), np.array(lse)


@pytest.mark.parametrize("seed", range(12))
def test_attention_matches_brute_force(seed):
    r = np.random.default_rng(1000 + seed)
    B = int(r.integers(1, 3))
    Hkv = int(r.choice([1, 2]))
    Hq = Hkv * int(r.choice([1, 2]))
    Sq, Sk = int(r.integers(1, 13)), int(r.integers(1, 13))
    D, Dv = int(r.integers(1, 9)), int(r.integers(1, 9))
    causal = bool(seed % 3 != 0)
    q = r.standard_normal((B, Sq, Hq, D)) * 1.5
    k = r.standard_normal((B, Sk, Hkv, D))
    v = r.standard_normal((B, Sk, Hkv, Dv))
    q_pos = int(r.integers(0, 20)) + np.arange(Sq)
    k_pos = int(r.integers(0, 20)) + np.arange(Sk)
    scale = float(r.uniform(0.2, 1.2))
    o, lse = attention_ref(q, k, v, q_pos, k_pos, causal, scale)
    ob, lseb = brute_attention(q, k, v, q_pos, k_pos, causal, scale)
    np.testing.assert_allclose(o, ob, rtol=0, atol=TOL)
    fin = np.isfinite(lseb)
    assert np.array_equal(fin, np.isfinite(lse))
    np.testing.assert_allclose(lse[fin], lseb[fin], rtol=0, atol=TOL)
    assert np.all(o[~fin] == 0.0)


# ----------------------------------------------------------------------------
# attention_ref: closed forms
# ----------------------------------------------------------------------------

def test_single_key_returns_its_value():
    r = np.random.default_rng(1)
    q = r.standard_normal((1, 3, 2, 5))
    k = r.standard_normal((1, 1, 2, 5))
    v = r.standard_normal((1, 1, 2, 4))
    o, lse = attention_ref(q, k, v, scale=0.7)
    for h in range(2):
        np.testing.assert_allclose(o[0, :, h, :], np.broadcast_to(v[0, 0, h], (3, 4)), atol=TOL)
        np.testing.assert_allclose(lse[0, :, h], 0.7 * (q[0, :, h, :] @ k[0, 0, h]), atol=TOL)


def test_identical_keys_give_mean_value_and_log_n():
    r = np.random.default_rng(2)
    n = 7
    q = r.standard_normal((1, 2, 1, 6))
    k = np.broadcast_to(r.standard_normal(6), (1, n, 1, 6)).copy()
    v = r.standard_normal((1, n, 1, 3))
    o, lse = attention_ref(q, k, v, scale=0.3)
    np.testing.assert_allclose(o[0, :, 0], np.broadcast_to(v[0, :, 0].mean(0), (2, 3)), atol=TOL)
    s = 0.3 * (q[0, :, 0] @ k[0, 0, 0])
    np.testing.assert_allclose(lse[0, :, 0], s + math.log(n), atol=TOL)


def test_zero_query_averages_visible_values_causal_offsets():
    r = np.random.default_rng(3)
    Sq, Sk = 5, 9
    q = np.zeros((1, Sq, 1, 4))
    k = r.standard_normal((1, Sk, 1, 4))
    v = r.standard_normal((1, Sk, 1, 2))
    q_pos = np.arange(Sq) + 10
    k_pos = np.arange(Sk) + 8          # row i sees keys 0 .. i+2
    o, lse = attention_ref(q, k, v, q_pos, k_pos, causal=True)
    for i in range(Sq):
        nvis = i + 3
        np.testing.assert_allclose(o[0, i, 0], v[0, :nvis, 0].mean(0), atol=TOL)
        np.testing.assert_allclose(lse[0, i, 0], math.log(nvis), atol=TOL)


def test_first_causal_row_sees_only_first_key_and_empty_rows():
    r = np.random.default_rng(4)
    q = r.standard_normal((1, 4, 1, 3))
    k = r.standard_normal((1, 4, 1, 3))
    v = r.standard_normal((1, 4, 1, 3))
    # queries at 5..8, keys at 6..9: row 0 sees nothing, row 1 sees only key 0
    o, lse = attention_ref(q, k, v, np.arange(5, 9), np.arange(6, 10), causal=True, scale=1.0)
    assert np.all(o[0, 0, 0] == 0.0) and lse[0, 0, 0] == -np.inf
    np.testing.assert_allclose(o[0, 1, 0], v[0, 0, 0], atol=TOL)
    np.testing.assert_allclose(lse[0, 1, 0], q[0, 1, 0] @ k[0, 0, 0], atol=TOL)


def test_gqa_uses_contiguous_head_groups():
    # one key per kv head with a distinct value: O[h] must be V[h // (Hq/Hkv)]
    Hq, Hkv = 6, 2
    q = np.ones((1, 1, Hq, 2))
    k = np.ones((1, 1, Hkv, 2))
    v = np.array([[[[10.0], [20.0]]]])
    o, _ = attention_ref(q, k, v)
    assert o[0, 0, :, 0].tolist() == [10.0, 10.0, 10.0, 20.0, 20.0, 20.0]


def test_default_scale_is_inverse_sqrt_dqk():
    # two keys with known dot products; softmax weight of the first key in closed form
    d = 16
    q = np.zeros((1, 1, 1, d)); q[..., 0] = 1.0
    k = np.zeros((1, 2, 1, d)); k[0, 0, 0, 0] = 4.0; k[0, 1, 0, 0] = 0.0
    v = np.array([[[[1.0]], [[0.0]]]])
    o, lse = attention_ref(q, k, v)
    a = 4.0 / math.sqrt(d)
    np.testing.assert_allclose(o[0, 0, 0, 0], math.exp(a) / (math.exp(a) + 1.0), atol=TOL)
    np.testing.assert_allclose(lse[0, 0, 0], math.log(math.exp(a) + 1.0), atol=TOL)


def test_matches_torch_sdpa_float64_with_explicit_mask():
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(5)
    B, Sq, Sk, Hq, Hkv, D, Dv = 2, 11, 17, 4, 2, 8, 6
    q = r.standard_normal((B, Sq, Hq, D))
    k = r.standard_normal((B, Sk, Hkv, D))
    v = r.standard_normal((B, Sk, Hkv, Dv))
    q_pos, k_pos = np.arange(Sq) + 9, np.arange(Sk)
    o, lse = attention_ref(q, k, v, q_pos, k_pos, causal=True, scale=0.4)
    mask = torch.from_numpy(k_pos[None, :] <= q_pos[:, None])
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(k, Hq // Hkv, axis=2)).permute(0, 2, 1, 3)
    tv = torch.from_numpy(np.repeat(v, Hq // Hkv, axis=2)).permute(0, 2, 1, 3)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=0.4)
    np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=TOL)
    scores = (tq @ tk.transpose(-1, -2)) * 0.4
    scores = scores.masked_fill(~mask, float("-inf"))
    ref_lse = torch.logsumexp(scores, dim=-1).permute(0, 2, 1).numpy()
    np.testing.assert_allclose(lse, ref_lse, atol=TOL)


# ----------------------------------------------------------------------------
# lse_merge_ref: blockwise merge equals the full softmax
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(8))
def test_blockwise_merge_equals_full_attention(seed):
    r = np.random.default_rng(200 + seed)
    Sq, Sk, Hq, Hkv, D = 6, 23, 4, 2, 5
    q = r.standard_normal((1, Sq, Hq, D)) * 2
    k = r.standard_normal((1, Sk, Hkv, D))
    v = r.standard_normal((1, Sk, Hkv, 3))
    causal = seed % 2 == 1
    q_pos, k_pos = np.arange(Sq) + 12, np.arange(Sk)
    full_o, full_lse = attention_ref(q, k, v, q_pos, k_pos, causal)
    # random cut points (allowing empty and single-key blocks), random order
    cuts = np.sort(r.integers(0, Sk + 1, size=6))
    bounds = [0, *cuts.tolist(), Sk]
    blocks = [(a, b) for a, b in zip(bounds[:-1], bounds[1:])]
    r.shuffle(blocks)
    parts_o, parts_lse = [], []
    for a, b in blocks:
        po, pl = attention_ref(q, k[:, a:b], v[:, a:b], q_pos, k_pos[a:b], causal)
        parts_o.append(po); parts_lse.append(pl)
    o, lse = lse_merge_ref(parts_o, parts_lse)
    np.testing.assert_allclose(o, full_o, atol=TOL)
    np.testing.assert_allclose(lse, full_lse, atol=TOL)


def test_merge_identity_commutativity_associativity():
    r = np.random.default_rng(7)
    o = [r.standard_normal((5, 4)) for _ in range(3)]
    l = [r.standard_normal(5) for _ in range(3)]
    ident_o, ident_l = np.zeros((5, 4)), np.full(5, -np.inf)
    mo, ml = lse_merge_ref([o[0], ident_o], [l[0], ident_l])
    np.testing.assert_allclose(mo, o[0], atol=TOL); np.testing.assert_allclose(ml, l[0], atol=TOL)
    a = lse_merge_ref(o, l)
    b = lse_merge_ref(o[::-1], l[::-1])
    ab = lse_merge_ref(o[:2], l[:2])
    c = lse_merge_ref([ab[0], o[2]], [ab[1], l[2]])
    for x in (b, c):
        np.testing.assert_allclose(x[0], a[0], atol=TOL)
        np.testing.assert_allclose(x[1], a[1], atol=TOL)
    e = lse_merge_ref([ident_o, ident_o], [ident_l, ident_l])
    assert np.all(e[0] == 0) and np.all(np.isneginf(e[1]))


def test_merge_two_parts_closed_form_weights():
    # LSE values log(1) and log(3): weights 1/4 and 3/4, total log(4)
    o, lse = lse_merge_ref([np.array([[4.0]]), np.array([[8.0]])],
                           [np.array([0.0]), np.array([math.log(3.0)])])
    np.testing.assert_allclose(o, [[7.0]], atol=TOL)
    np.testing.assert_allclose(lse, [math.log(4.0)], atol=TOL)


# ----------------------------------------------------------------------------
# ring schedule
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 4, 8])
def test_ring_schedule_matches_simulated_message_passing(n):
    holding = list(range(n))            # step 0: every rank holds its own block
    seen = {r: [] for r in range(n)}
    for _ in range(n):
        for r in range(n):
            seen[r].append(holding[r])
        holding = [holding[(r - 1) % n] for r in range(n)]   # each rank passes to r+1
    for r in range(n):
        assert ring_schedule_ref(r, n) == seen[r]
        assert sorted(seen[r]) == list(range(n)) and seen[r][0] == r


def test_zigzag_ring_chunks_rank0_cp8():
    assert zigzag_ring_chunks_ref(0, 8) == [(0, 15), (7, 8), (6, 9), (5, 10), (4, 11),
                                            (3, 12), (2, 13), (1, 14)]
    assert zigzag_ring_chunks_ref(0, 4) == [(0, 7), (3, 4), (2, 5), (1, 6)]


# ----------------------------------------------------------------------------
# partition
# ----------------------------------------------------------------------------

def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_partition_worked_examples():
    g = _load("partition_examples.json")
    for ex in g["examples"]:
        local, restore = partition_ref(ex["seq_lens"], ex["cp_size"])
        assert [x.tolist() for x in local] == ex["local"], ex["name"]
        assert restore.tolist() == ex["restore"], ex["name"]
    for ex in g["sampled"]:
        local, restore = partition_ref(ex["seq_lens"], ex["cp_size"])
        assert [int(local[0][i]) for i in ex["rank0_at"]] == ex["rank0_first"]
        for t, want in ex["restore_at"].items():
            assert int(restore[int(t)]) == want


@pytest.mark.parametrize("seq_lens,cp", [([8192], 4), ([10], 2), ([4, 8], 2), ([1, 0, 37, 5], 3),
                                         ([64], 8), ([3], 4)])
def test_partition_invariants(seq_lens, cp):
    local, restore = partition_ref(seq_lens, cp)
    total = sum(seq_lens)
    gathered = np.concatenate(local)
    assert len({len(x) for x in local}) == 1                    # equal local lengths
    assert np.array_equal(gathered[restore], np.arange(total))  # gather restores order
    assert len(set(restore.tolist())) == total                  # injective
    assert sorted(gathered[gathered >= 0].tolist()) == list(range(total))


@pytest.mark.parametrize("cp", [1, 2, 4, 8])
def test_partition_balances_causal_work(cp):
    # one request of 2*cp*c tokens; count visible causal pairs of each rank's Q
    # against the whole sequence: all ranks must do the same work
    c = 5
    L = 2 * cp * c
    local, _ = partition_ref([L], cp)
    work = [int(sum(t + 1 for t in x.tolist())) for x in local]
    assert len(set(work)) == 1


# ----------------------------------------------------------------------------
# slot mapping
# ----------------------------------------------------------------------------

def test_slot_mapping_worked_examples():
    g = _load("slot_mapping_examples.json")
    for c in g["cases"]:
        dev, slot = slot_mapping_ref(c["positions"], c["block_size"], c["interleave"],
                                     c["pcp_size"], c["dcp_size"])
        assert dev.tolist() == c["device"]
        assert slot.tolist() == c["slot"]
        assert (slot % c["block_size"]).tolist() == c["in_block"]
    for c in g["invalid"]:
        with pytest.raises(ValueError):
            slot_mapping_ref([0], c["block_size"], c["interleave"], c["pcp_size"], c["dcp_size"])


@pytest.mark.parametrize("bs,il,pcp,dcp", [(128, 16, 8, 1), (4, 2, 2, 1), (8, 8, 3, 1),
                                           (16, 4, 2, 2), (6, 3, 1, 1), (32, 1, 4, 1)])
def test_slot_mapping_invariants(bs, il, pcp, dcp):
    W = pcp * dcp
    n_vb = 5
    x = np.arange(n_vb * bs * W)
    dev, slot = slot_mapping_ref(x, bs, il, pcp, dcp)
    in_blk = slot % bs
    vb = slot // bs
    assert np.all((0 <= dev) & (dev < W))
    # bijection between x and (vb, dev, in-block offset)
    assert len(set(zip(vb.tolist(), dev.tolist(), in_blk.tolist()))) == len(x)
    # each device holds exactly block_size tokens of every virtual block
    for v_ in range(n_vb):
        sel = x // (bs * W) == v_
        assert np.bincount(dev[sel], minlength=W).tolist() == [bs] * W
    if il == bs:      # whole blocks dealt round-robin
        assert np.array_equal(dev, (x // bs) % W) and np.array_equal(in_blk, x % bs)
    if W == 1:        # one device: identity placement
        assert np.all(dev == 0) and np.array_equal(slot, x)
    # a block table remaps the virtual block only
    table = np.arange(n_vb)[::-1] * 3 + 1
    dev2, slot2 = slot_mapping_ref(x, bs, il, pcp, dcp, block_table=table)
    assert np.array_equal(dev2, dev)
    assert np.array_equal(slot2, table[x // (bs * W)] * bs + in_blk)


# ----------------------------------------------------------------------------
# classification and visible-pair counts
# ----------------------------------------------------------------------------

def _brute_visible(q0, sq, k0, sk, causal):
    return [[(not causal) or (k0 + j <= q0 + i) for j in range(sk)] for i in range(sq)]


def test_classify_and_pair_count_against_enumeration():
    for q0, sq, k0, sk in itertools.product([0, 3, 7], [1, 4, 6], [0, 2, 5, 9], [1, 3, 8]):
        for causal in (False, True):
            vis = _brute_visible(q0, sq, k0, sk, causal)
            flat = [x for row in vis for x in row]
            want = FULL if all(flat) else SKIP if not any(flat) else DIAG
            assert classify_ref(q0, sq, k0, sk, causal) == want
            assert visible_pairs_ref(q0, sq, k0, sk, causal) == sum(flat)
    assert classify_ref(0, 0, 0, 5, True) == SKIP and visible_pairs_ref(0, 5, 0, 0, True) == 0


def test_zigzag_rank0_pair_classes_cp4_and_cp8():
    # rank 0's Q parts {0, 2cp-1} against every K/V part, as the pages' workloads
    for cp, c, want in [(4, 1024, (7, 2, 7)), (8, 65536, (15, 2, 15))]:
        counts = [0, 0, 0]
        for qp in (0, 2 * cp - 1):
            for kp in range(2 * cp):
                counts[classify_ref(qp * c, c, kp * c, c, True)] += 1
        assert tuple(counts) == want


# ----------------------------------------------------------------------------
# decode over sharded KV
# ----------------------------------------------------------------------------

def test_sharded_decode_merge_equals_unsharded():
    r = np.random.default_rng(9)
    B, T, Hq, Hkv, D = 2, 64, 4, 2, 8
    q = r.standard_normal((B, Hq, D))
    k = r.standard_normal((B, T, Hkv, D))
    v = r.standard_normal((B, T, Hkv, D))
    dev, _ = slot_mapping_ref(np.arange(T), 4, 2, 4, 1)
    _, _, o, lse = decode_shards_ref(q, k, v, dev, 4)
    fo, fl = attention_ref(q[:, None], k, v)
    np.testing.assert_allclose(o, fo[:, 0], atol=TOL)
    np.testing.assert_allclose(lse, fl[:, 0], atol=TOL)


def test_reorg_index_golden():
    from oracle import reorg_index_ref
    g = _load("reorg_examples.json")
    for c in g["cases"]:
        src, dev_lens = reorg_index_ref(c["seq_lens"], c["block_size"], c["interleave"],
                                        c["pcp_size"], c["dcp_size"])
        assert src.tolist() == c["src_idx"], c["derivation"]
        assert dev_lens.tolist() == c["dev_lens"]


@pytest.mark.parametrize("lens,bs,il,pcp,dcp", [([1000, 37, 0, 513], 16, 4, 2, 2), ([4096], 128, 16, 8, 1),
                                                ([5, 9], 6, 3, 3, 1), ([300, 300], 32, 8, 1, 1)])
def test_reorg_index_invariants(lens, bs, il, pcp, dcp):
    from oracle import reorg_index_ref
    src, dev_lens = reorg_index_ref(lens, bs, il, pcp, dcp)
    n = sum(lens)
    assert sorted(src.tolist()) == list(range(n))            # a permutation of the gathered rows
    assert dev_lens.sum(0).tolist() == list(lens)            # every token on exactly one device
    if pcp * dcp == 1:
        assert src.tolist() == list(range(n))                # one device: already contiguous
    # rebuild the gathered buffer from the placement alone and read it back
    W = pcp * dcp
    bufs = [[] for _ in range(W)]
    for r, L in enumerate(lens):
        dev, slot = slot_mapping_ref(np.arange(L), bs, il, pcp, dcp)
        for d in range(W):
            order = np.argsort(slot[dev == d], kind="stable")
            bufs[d].extend(("tok", r, int(x)) for x in np.arange(L)[dev == d][order])
    gathered = [e for d in range(W) for e in bufs[d]]
    assert [gathered[i] for i in src] == [("tok", r, x) for r, L in enumerate(lens) for x in range(L)]
