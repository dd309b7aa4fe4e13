"""Plain CPU oracle for blockwise ring attention / context parallelism.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the package
``ring_attention_02_amd``) may import, call or link anything in this
directory; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP path: no kernels, headers, helpers, tables or constants.

Everything is numpy float64 (integers for the index functions), written
for a reader who checks it against the pages by eye:

* ``attention``  -- the plain definition softmax(scale * Q K^T) V with an
  absolute-position causal mask, its log-sum-exp, the LSE merge of
  partials, and decode over a sequence-sharded KV cache.
* ``index``      -- the head-tail (zigzag) partition and restore index, the
  interleaved virtual-block slot mapping, the ring step schedule, the
  full / diagonal / skip block classification and the reorganisation index
  of an all-gathered KV cache.

Every function is pinned by tests in ``tests/test_oracle.py`` against
closed forms, brute force, worked examples derived from the pages' rules
(``tests/golden/``) and invariants.  No function here is "parity unpinned".
"""

from .attention import attention_ref, lse_merge_ref, decode_shards_ref
from .index import (partition_ref, slot_mapping_ref, classify_ref,
                    ring_schedule_ref, zigzag_ring_chunks_ref,
                    visible_pairs_ref, reorg_index_ref, FULL, DIAG, SKIP)

__all__ = [
    "attention_ref", "lse_merge_ref", "decode_shards_ref",
    "partition_ref", "slot_mapping_ref", "classify_ref", "ring_schedule_ref",
    "zigzag_ring_chunks_ref", "visible_pairs_ref", "reorg_index_ref", "FULL", "DIAG", "SKIP",
]
