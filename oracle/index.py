"""Oracle: the integer side of context parallelism.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  Plain Python and
numpy integers; every result is exact.

Sources (the pages):
* vLLM-Ascend developer guide "Context Parallel (CP)", section "Prefill
  context parallel (PCP)", paragraph on the head-tail token partition: the
  sequence is padded, cut into 2*pcp_size equal parts, and part i is
  paired with part 2*pcp_size-1-i so that every device gets the same causal
  work; an all-gather of the devices' token lists interleaves requests, so
  an index (pcp_allgather_restore_idx) recovers the original order.
* same guide, section "How it works / Block table": the interleaved
  virtual-block KV placement (virtual block size, local block index,
  device id and in-block offset) and the requirement that block_size be a
  multiple of cp_kv_cache_interleave_size.
* guijiagi.com tag page "Ring Attention", excerpt on the ring topology: at
  step t device i works on the K/V block that started on device (i - t)
  mod N and passes it on to device (i + 1) mod N.
* video page "How Context Parallelism Splits Long Sequences Across GPUs",
  chapter list: causal masking is applied per block.

Readings of what the pages leave open:
* the garbled padding target is read as "the smallest multiple of
  2*cp_size that is >= the request length"; padding sits at the tail and
  is marked -1 in local lists and is absent from the restore index;
* the restore index has gather semantics: original token t sits at
  gathered[restore_idx[t]], where the gathered list is the ranks' local
  lists concatenated in rank order;
* rank r holds part r first, then part 2*cp-1-r; several requests are
  partitioned one by one and concatenated per rank in request order;
* slot = block_table[virtual block] * block_size + in-block offset, with
  an identity block table by default; the device id is flat in
  [0, pcp_size*dcp_size);
* a (query range, key range) pair with no (q, k) pair at all is SKIP;
* (reorg_kvcache, MLA chunked prefill with all-gather KV in the same guide)
  each device's KV buffer lists the requests in order, each request's tokens
  at their local slots 0..n-1 (identity block table); the all-gather
  concatenates the devices' buffers in device order; the reorganised KV
  lists every request's tokens contiguously in their original order.
"""

import numpy as np

FULL, DIAG, SKIP = 0, 1, 2


def partition_ref(seq_lens, cp_size):
    """Head-tail (zigzag) partition of one or more requests over cp_size ranks.

    Returns (local, restore):
      local[r]  -- int64 array of global token ids held by rank r, padding -1;
      restore   -- int64 array, restore[t] = position of original token t in
                   the concatenation local[0] + local[1] + ... + local[cp-1].
    Global token ids number the requests' tokens consecutively, request by
    request.
    """
    if cp_size <= 0:
        raise ValueError("cp_size must be positive")
    parts = 2 * cp_size
    local = [[] for _ in range(cp_size)]
    offset = 0
    for L in seq_lens:
        L = int(L)
        if L < 0:
            raise ValueError("negative sequence length")
        padded = -(-L // parts) * parts          # smallest multiple of 2*cp >= L
        c = padded // parts                      # tokens per part
        for r in range(cp_size):
            for part in (r, parts - 1 - r):      # head part, then its tail partner
                for pos in range(part * c, (part + 1) * c):
                    local[r].append(offset + pos if pos < L else -1)
        offset += L
    gathered = [tok for r in range(cp_size) for tok in local[r]]
    restore = np.full(offset, -1, dtype=np.int64)
    for where, tok in enumerate(gathered):
        if tok >= 0:
            restore[tok] = where
    return [np.asarray(x, dtype=np.int64) for x in local], restore


def slot_mapping_ref(positions, block_size, interleave, pcp_size, dcp_size,
                     block_table=None):
    """Interleaved virtual-block placement of tokens over pcp_size*dcp_size devices.

    For token position x (block table section of the CP guide):
      virtual_block_size = block_size * pcp_size * dcp_size
      vb      = x // virtual_block_size
      off     = x %  virtual_block_size
      lbi     = off // interleave
      device  = lbi %  (pcp_size * dcp_size)
      in_blk  = (lbi // (pcp_size * dcp_size)) * interleave + off % interleave
      slot    = block_table[vb] * block_size + in_blk
    Returns (device int32[n], slot int64[n]).  Raises ValueError when
    block_size is not a multiple of interleave.
    """
    if block_size <= 0 or interleave <= 0 or pcp_size <= 0 or dcp_size <= 0:
        raise ValueError("sizes must be positive")
    if block_size % interleave != 0:
        raise ValueError("block_size must be a multiple of cp_kv_cache_interleave_size")
    world = pcp_size * dcp_size
    vbs = block_size * world
    device, slot = [], []
    for x in np.asarray(positions, dtype=np.int64).tolist():
        if x < 0:
            raise ValueError("negative position")
        vb = x // vbs
        off = x % vbs
        lbi = off // interleave
        dev = lbi % world
        in_blk = (lbi // world) * interleave + off % interleave
        phys = vb if block_table is None else int(block_table[vb])
        device.append(dev)
        slot.append(phys * block_size + in_blk)
    return np.asarray(device, dtype=np.int32), np.asarray(slot, dtype=np.int64)


def _visible_per_row(q_pos0, sq, k_pos0, sk, causal):
    """Number of keys of the block [k_pos0, k_pos0+sk) each query row sees.

    Causal: query at position p sees exactly the keys with position <= p,
    which are the first clip(p - k_pos0 + 1, 0, sk) keys of the block.
    """
    if not causal:
        return np.full(sq, sk, dtype=np.int64)
    q_positions = q_pos0 + np.arange(sq, dtype=np.int64)
    return np.clip(q_positions - k_pos0 + 1, 0, sk)


def classify_ref(q_pos0, sq, k_pos0, sk, causal):
    """FULL if every (q, k) pair is visible, SKIP if none is, DIAG otherwise."""
    if sq <= 0 or sk <= 0:
        return SKIP
    n = _visible_per_row(q_pos0, sq, k_pos0, sk, causal)
    if np.all(n == sk):
        return FULL
    if np.all(n == 0):
        return SKIP
    return DIAG


def visible_pairs_ref(q_pos0, sq, k_pos0, sk, causal):
    """Exact count of visible (q, k) pairs of one block pair."""
    if sq <= 0 or sk <= 0:
        return 0
    return int(_visible_per_row(q_pos0, sq, k_pos0, sk, causal).sum())


def ring_schedule_ref(rank, n):
    """K/V block index that rank `rank` computes with at ring steps 0..n-1."""
    return [(rank - t) % n for t in range(n)]


def zigzag_ring_chunks_ref(rank, cp_size):
    """Sequence parts (of 2*cp_size) held by the K/V block seen at each step.

    With the head-tail partition, the block that started on rank s carries
    parts s and 2*cp_size-1-s.
    """
    return [(s, 2 * cp_size - 1 - s) for s in ring_schedule_ref(rank, cp_size)]


def reorg_index_ref(seq_lens, block_size, interleave, pcp_size, dcp_size):
    """Rows of the all-gathered KV buffer, request by request, token by token.

    MLA chunked prefill with all-gather KV (CP guide, PCP chunked-prefill
    paragraph and MLA prefill note): the context KV is all-gathered, which
    interleaves requests, and reorg_kvcache stores each request's KV
    contiguously.  Simulated in that order: every device's buffer of
    (request, token) entries by local slot, the all-gather, then each
    request's tokens looked up in the gathered buffer.
    Returns (src_idx int64[sum seq_lens], dev_lens int64[W, num_reqs]).
    """
    world = pcp_size * dcp_size
    per_dev = [[] for _ in range(world)]
    dev_lens = np.zeros((world, len(seq_lens)), dtype=np.int64)
    for r, L in enumerate(seq_lens):
        dev, slot = slot_mapping_ref(np.arange(int(L)), block_size, interleave, pcp_size, dcp_size)
        for d in range(world):
            mine = sorted((int(s_), x) for x, (dv, s_) in enumerate(zip(dev, slot)) if dv == d)
            assert [s_ for s_, _ in mine] == list(range(len(mine))), "local slots must be 0..n-1"
            per_dev[d].extend((r, x) for _, x in mine)
            dev_lens[d, r] = len(mine)
    gathered = [entry for d in range(world) for entry in per_dev[d]]      # the all-gather
    where = {entry: row for row, entry in enumerate(gathered)}
    src = [where[(r, x)] for r, L in enumerate(seq_lens) for x in range(int(L))]
    return np.asarray(src, dtype=np.int64), dev_lens
