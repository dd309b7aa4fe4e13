"""Oracle: attention, its log-sum-exp, the LSE merge and sharded decode.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.  numpy float64.

Sources (the pages):
* guijiagi.com tag page "Ring Attention", excerpt on the memory wall of
  plain attention (its formula and "key insight" paragraph): attention is
  softmax(Q K^T / sqrt(d)) V, and its numerator and denominator are both
  sums over keys, so they can be accumulated one key block at a time with
  a per-row maximum and sum carried between blocks.
* same page, excerpt on the ring topology: once a device has met every
  K/V block, its accumulated partial output is the final answer.
* vLLM-Ascend developer guide "Context Parallel (CP)", section "Decode
  context parallel (DCP)": the per-device attention outputs and their LSEs,
  each over that device's slice of the KV cache, are combined into the
  result.

Because the blockwise / ring method is an exact re-association of the plain
definition, the oracle computes the plain definition directly and never
blocks, fuses or reorders beyond it.

Readings of what the pages leave open (each listed in the design notes):
* the log-sum-exp is the natural log and includes the softmax scale;
* the scale is a parameter, defaulting to 1/sqrt(d_qk);
* the causal mask uses absolute positions: key j is visible to query i iff
  k_pos[j] <= q_pos[i];
* a query row with no visible key has O = 0 and LSE = -inf, and merging
  such a partial changes nothing;
* grouped-query attention uses contiguous groups: query head h reads
  kv head h // (Hq // Hkv).
"""

import numpy as np


def attention_ref(q, k, v, q_pos=None, k_pos=None, causal=False, scale=None):
    """Plain attention with its log-sum-exp, in float64.

    q: [B, Sq, Hq, Dqk]; k: [B, Sk, Hkv, Dqk]; v: [B, Sk, Hkv, Dv]
    (any real dtype; bf16 inputs are passed as their exact float values).
    q_pos: [Sq] absolute query positions (default 0..Sq-1).
    k_pos: [Sk] absolute key positions (default 0..Sk-1).
    Returns O [B, Sq, Hq, Dv] and LSE [B, Sq, Hq], both float64, where for
    every row  O = sum_j softmax_j * V_j  over the visible keys and
    LSE = log(sum_j exp(scale * q . k_j)).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, Hq, Dqk = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    assert Bk == B and Dk == Dqk and v.shape[:3] == (B, Sk, Hkv)
    assert Hq % Hkv == 0, "query heads must be a multiple of kv heads"
    Dv = v.shape[3]
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(Dqk)
    q_pos = np.arange(Sq) if q_pos is None else np.asarray(q_pos, dtype=np.int64)
    k_pos = np.arange(Sk) if k_pos is None else np.asarray(k_pos, dtype=np.int64)

    if causal:
        visible = k_pos[None, :] <= q_pos[:, None]          # [Sq, Sk]
    else:
        visible = np.ones((Sq, Sk), dtype=bool)
    any_visible = visible.any(axis=1)                        # [Sq]

    o = np.zeros((B, Sq, Hq, Dv), dtype=np.float64)
    lse = np.full((B, Sq, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            kvh = h // group
            s = scale * (q[b, :, h, :] @ k[b, :, kvh, :].T)  # [Sq, Sk]
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1, initial=-np.inf)               # running max, all keys at once
            m_safe = np.where(any_visible, m, 0.0)
            p = np.where(visible, np.exp(s - m_safe[:, None]), 0.0)
            l = p.sum(axis=1)                                # running sum, all keys at once
            l_safe = np.where(any_visible, l, 1.0)
            o[b, :, h, :] = np.where(any_visible[:, None],
                                     (p @ v[b, :, kvh, :]) / l_safe[:, None], 0.0)
            lse[b, :, h] = np.where(any_visible, m_safe + np.log(l_safe), -np.inf)
    return o, lse


def lse_merge_ref(o_parts, lse_parts):
    """Combine partial (O_k, LSE_k) into the result over the union of keys.

    o_parts: sequence of arrays [..., Dv]; lse_parts: matching [...] arrays.
    With M = max_k LSE_k:  LSE = M + log(sum_k exp(LSE_k - M)) and
    O = sum_k exp(LSE_k - LSE) * O_k.  Rows where every part is -inf (no
    visible key anywhere) give O = 0 and LSE = -inf.
    """
    o_parts = [np.asarray(o, dtype=np.float64) for o in o_parts]
    lse_parts = [np.asarray(x, dtype=np.float64) for x in lse_parts]
    assert len(o_parts) == len(lse_parts) and len(o_parts) > 0
    lse_stack = np.stack(lse_parts)                  # [n, ...]
    o_stack = np.stack(o_parts)                      # [n, ..., Dv]
    m = lse_stack.max(axis=0)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_stack - m_safe)                   # exp(-inf) = 0 for empty parts
    total = w.sum(axis=0)
    total_safe = np.where(empty, 1.0, total)
    lse = np.where(empty, -np.inf, m_safe + np.log(total_safe))
    weights = w / total_safe                         # = exp(LSE_k - LSE)
    o = (weights[..., None] * o_stack).sum(axis=0)
    o = np.where(empty[..., None], 0.0, o)
    return o, lse


def decode_shards_ref(q, k_ctx, v_ctx, token_device, n_shards, scale=None):
    """Decode (one new query per request) over a KV cache sharded by sequence.

    q: [B, Hq, Dqk]; k_ctx: [B, T, Hkv, Dqk]; v_ctx: [B, T, Hkv, Dv] hold the
    whole context in token order; token_device: [T] gives the shard that
    stores each token (the interleaved placement).  The query attends to
    every cached token with no mask.

    Returns per-shard partials O [n_shards, B, Hq, Dv], LSE [n_shards, B, Hq]
    and their merge O [B, Hq, Dv], LSE [B, Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    token_device = np.asarray(token_device)
    B, Hq, _ = q.shape
    Dv = np.asarray(v_ctx).shape[3]
    o_parts = np.zeros((n_shards, B, Hq, Dv))
    lse_parts = np.full((n_shards, B, Hq), -np.inf)
    for s in range(n_shards):
        sel = np.nonzero(token_device == s)[0]
        if sel.size == 0:
            continue
        o, lse = attention_ref(q[:, None, :, :], np.asarray(k_ctx)[:, sel],
                               np.asarray(v_ctx)[:, sel], causal=False, scale=scale)
        o_parts[s] = o[:, 0]
        lse_parts[s] = lse[:, 0]
    o, lse = lse_merge_ref(list(o_parts), list(lse_parts))
    return o_parts, lse_parts, o, lse
