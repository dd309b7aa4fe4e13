// Host-side index logic of context parallelism: the head-tail (zigzag)
// partition with its restore index, the interleaved virtual-block slot
// mapping, the row index that reorganises an all-gathered KV cache by
// request, and the full / diagonal / skip classification of block pairs.
//
// Partition: vLLM-Ascend developer guide "Context Parallel (CP)", section
// "Prefill context parallel (PCP)", head-tail token partition paragraph.
// Slot mapping: same guide, section "How it works / Block table".
// Reorganisation: same guide, PCP chunked-prefill paragraph and the MLA
// prefill note on all-gather KV.
// Classification: causal masking per block, video "How Context Parallelism
// Splits Long Sequences Across GPUs" (chapter on kernels, overlap and causal
// masks), with absolute positions so any Q range meets any KV range.
#include <cstdint>
#include <algorithm>
#include <limits>
#include <vector>

#include "status.h"

using ringattn::fail;
using ringattn::ok;

namespace {

// Tokens per part and padded length for one request of `len` tokens.
inline void part_geometry(int64_t len, int64_t parts, int64_t* part_len) {
  const int64_t padded = (len + parts - 1) / parts * parts;
  *part_len = padded / parts;
}

}  // namespace

extern "C" int32_t cp_partition(const int64_t* seq_lens, int32_t num_reqs, int32_t cp_size,
                                int32_t rank, int64_t* local_token_idx, int64_t* local_len,
                                int64_t* restore_idx, int64_t* restore_len) {
  RA_CHECK(num_reqs >= 0, CP_EINVAL, "cp_partition: num_reqs=%d < 0", num_reqs);
  RA_CHECK(num_reqs == 0 || seq_lens != nullptr, CP_EINVAL, "cp_partition: seq_lens is NULL");
  RA_CHECK(cp_size > 0, CP_EINVAL, "cp_partition: cp_size=%d must be > 0", cp_size);
  RA_CHECK(rank >= 0 && rank < cp_size, CP_EINVAL, "cp_partition: rank=%d outside [0,%d)", rank,
           cp_size);
  RA_CHECK(local_len != nullptr && restore_len != nullptr, CP_EINVAL,
           "cp_partition: local_len and restore_len must not be NULL");
  const int64_t parts = 2 * static_cast<int64_t>(cp_size);
  int64_t total = 0, per_rank = 0;
  for (int32_t r = 0; r < num_reqs; ++r) {
    RA_CHECK(seq_lens[r] >= 0, CP_EINVAL, "cp_partition: seq_lens[%d]=%lld < 0", r,
             static_cast<long long>(seq_lens[r]));
    RA_CHECK(seq_lens[r] <= (std::numeric_limits<int64_t>::max() / 4) - total, CP_EINVAL,
             "cp_partition: total length overflows");
    int64_t c;
    part_geometry(seq_lens[r], parts, &c);
    total += seq_lens[r];
    per_rank += 2 * c;
  }
  if (local_token_idx != nullptr)
    RA_CHECK(*local_len >= per_rank, CP_EINVAL,
             "cp_partition: local capacity %lld < needed %lld",
             static_cast<long long>(*local_len), static_cast<long long>(per_rank));
  if (restore_idx != nullptr)
    RA_CHECK(*restore_len >= total, CP_EINVAL,
             "cp_partition: restore capacity %lld < needed %lld",
             static_cast<long long>(*restore_len), static_cast<long long>(total));

  // Walk every rank's list in gathered order: rank-major, then request, then
  // head part followed by its tail partner.  Position `where` in that walk is
  // the token's index after an all-gather of the local lists.
  if (local_token_idx != nullptr || restore_idx != nullptr) {
    int64_t where = 0;
    for (int32_t r = 0; r < cp_size; ++r) {
      int64_t req_offset = 0, local_pos = 0;
      for (int32_t q = 0; q < num_reqs; ++q) {
        const int64_t len = seq_lens[q];
        int64_t c;
        part_geometry(len, parts, &c);
        const int64_t owned[2] = {r, parts - 1 - r};
        for (int64_t which : owned) {
          const int64_t first = which * c;
          for (int64_t p = first; p < first + c; ++p, ++where, ++local_pos) {
            const int64_t tok = p < len ? req_offset + p : -1;
            if (r == rank && local_token_idx != nullptr) local_token_idx[local_pos] = tok;
            if (tok >= 0 && restore_idx != nullptr) restore_idx[tok] = where;
          }
        }
        req_offset += len;
      }
    }
  }
  *local_len = per_rank;
  *restore_len = total;
  return ok();
}

extern "C" int32_t cp_slot_mapping(const int64_t* positions, int64_t n, int32_t block_size,
                                   int32_t interleave, int32_t pcp_size, int32_t dcp_size,
                                   const int32_t* block_table, int64_t block_table_len,
                                   int32_t* device_out, int64_t* slot_out) {
  RA_CHECK(n >= 0, CP_EINVAL, "cp_slot_mapping: n=%lld < 0", static_cast<long long>(n));
  RA_CHECK(n == 0 || (positions && device_out && slot_out), CP_EINVAL,
           "cp_slot_mapping: NULL array");
  RA_CHECK(block_size > 0 && interleave > 0 && pcp_size > 0 && dcp_size > 0, CP_EINVAL,
           "cp_slot_mapping: sizes must be positive (block_size=%d interleave=%d pcp=%d dcp=%d)",
           block_size, interleave, pcp_size, dcp_size);
  RA_CHECK(block_size % interleave == 0, CP_EINVAL,
           "cp_slot_mapping: block_size %d is not a multiple of interleave %d", block_size,
           interleave);
  RA_CHECK(block_table == nullptr || block_table_len >= 0, CP_EINVAL,
           "cp_slot_mapping: negative block_table_len");
  const int64_t world = static_cast<int64_t>(pcp_size) * dcp_size;
  const int64_t vbs = static_cast<int64_t>(block_size) * world;
  // Validate everything before writing anything.
  for (int64_t i = 0; i < n; ++i) {
    RA_CHECK(positions[i] >= 0, CP_EINVAL, "cp_slot_mapping: positions[%lld] < 0",
             static_cast<long long>(i));
    if (block_table != nullptr) {
      const int64_t vb = positions[i] / vbs;
      RA_CHECK(vb < block_table_len, CP_EINVAL,
               "cp_slot_mapping: virtual block %lld beyond block table of %lld",
               static_cast<long long>(vb), static_cast<long long>(block_table_len));
      RA_CHECK(block_table[vb] >= 0, CP_EINVAL, "cp_slot_mapping: negative block_table[%lld]",
               static_cast<long long>(vb));
    }
  }
  for (int64_t i = 0; i < n; ++i) {
    const int64_t x = positions[i];
    const int64_t vb = x / vbs;
    const int64_t off = x % vbs;
    const int64_t lbi = off / interleave;
    const int64_t in_block = (lbi / world) * interleave + off % interleave;
    const int64_t phys = block_table ? static_cast<int64_t>(block_table[vb]) : vb;
    device_out[i] = static_cast<int32_t>(lbi % world);
    slot_out[i] = phys * block_size + in_block;
  }
  return ok();
}

// vLLM-Ascend "Context Parallel (CP)", MLA chunked prefill with all-gather
// KV: each device holds, request after request, its slots of the context
// (placed by the slot mapping); an all-gather concatenates the devices'
// buffers, so the gathered KV interleaves requests and devices, and
// reorg_kvcache makes every request's KV contiguous again.  This computes,
// for every token of every request in original order, its row in the
// gathered buffer; the device gather (cp_gather_rows) then moves the rows.
extern "C" int32_t cp_reorg_index(const int64_t* seq_lens, int32_t num_reqs, int32_t block_size,
                                  int32_t interleave, int32_t pcp_size, int32_t dcp_size,
                                  int64_t* src_idx, int64_t* src_len, int64_t* dev_lens,
                                  int64_t dev_lens_len) {
  RA_CHECK(num_reqs >= 0, CP_EINVAL, "cp_reorg_index: num_reqs=%d < 0", num_reqs);
  RA_CHECK(num_reqs == 0 || seq_lens, CP_EINVAL, "cp_reorg_index: NULL seq_lens");
  RA_CHECK(block_size > 0 && interleave > 0 && pcp_size > 0 && dcp_size > 0, CP_EINVAL,
           "cp_reorg_index: sizes must be positive (block_size=%d interleave=%d pcp=%d dcp=%d)",
           block_size, interleave, pcp_size, dcp_size);
  RA_CHECK(block_size % interleave == 0, CP_EINVAL,
           "cp_reorg_index: block_size %d is not a multiple of interleave %d", block_size, interleave);
  RA_CHECK(src_idx == nullptr || src_len != nullptr, CP_EINVAL,
           "cp_reorg_index: src_len (the capacity of src_idx) must not be NULL");
  int64_t total = 0;
  for (int32_t r = 0; r < num_reqs; ++r) {
    RA_CHECK(seq_lens[r] >= 0, CP_EINVAL, "cp_reorg_index: seq_lens[%d] < 0", r);
    RA_CHECK(seq_lens[r] <= std::numeric_limits<int64_t>::max() / 4 - total, CP_EINVAL,
             "cp_reorg_index: total length overflows");
    total += seq_lens[r];
  }
  const int64_t world = static_cast<int64_t>(pcp_size) * dcp_size;
  const int64_t vbs = static_cast<int64_t>(block_size) * world;
  // capacities are checked before anything is written
  if (src_idx != nullptr)
    RA_CHECK(*src_len >= total, CP_EINVAL, "cp_reorg_index: src_idx capacity %lld < needed %lld",
             static_cast<long long>(*src_len), static_cast<long long>(total));
  if (dev_lens != nullptr)
    RA_CHECK(dev_lens_len >= world * num_reqs, CP_EINVAL,
             "cp_reorg_index: dev_lens capacity %lld < needed %lld", static_cast<long long>(dev_lens_len),
             static_cast<long long>(world * num_reqs));
  if (src_len) *src_len = total;
  // tokens of request r on device d
  std::vector<int64_t> len(static_cast<size_t>(world * num_reqs), 0);
  for (int32_t r = 0; r < num_reqs; ++r)
    for (int64_t x = 0; x < seq_lens[r]; ++x) ++len[((x % vbs) / interleave % world) * num_reqs + r];
  if (dev_lens) std::copy(len.begin(), len.end(), dev_lens);
  if (src_idx == nullptr) return ok();
  // gathered row of (device d, request r, local slot s) = base[d][r] + s
  std::vector<int64_t> base(len.size(), 0);
  int64_t run = 0;
  for (int64_t d = 0; d < world; ++d)
    for (int32_t r = 0; r < num_reqs; ++r) {
      base[d * num_reqs + r] = run;
      run += len[d * num_reqs + r];
    }
  int64_t out = 0;
  for (int32_t r = 0; r < num_reqs; ++r)
    for (int64_t x = 0; x < seq_lens[r]; ++x) {
      const int64_t off = x % vbs, lbi = off / interleave;
      const int64_t dev = lbi % world;
      const int64_t slot = (x / vbs) * block_size + (lbi / world) * interleave + off % interleave;
      src_idx[out++] = base[dev * num_reqs + r] + slot;
    }
  return ok();
}

// Ring order: guijiagi.com "Ring Attention", ring-topology excerpt -- at
// step t device i computes with the K/V block that started on device
// (i - t) mod N, received from its predecessor, and passes it on to its
// successor; after N steps it has met every block once.  With the head-tail
// partition (vLLM-Ascend "Context Parallel (CP)", PCP head-tail token
// partition paragraph) the block of rank s carries parts s and 2N-1-s.
extern "C" int32_t cp_ring_schedule(int32_t rank, int32_t cp_size, int32_t* src_rank,
                                    int32_t* parts) {
  RA_CHECK(cp_size > 0, CP_EINVAL, "cp_ring_schedule: cp_size=%d must be > 0", cp_size);
  RA_CHECK(rank >= 0 && rank < cp_size, CP_EINVAL, "cp_ring_schedule: rank=%d outside [0,%d)", rank,
           cp_size);
  RA_CHECK(src_rank != nullptr || parts != nullptr, CP_EINVAL,
           "cp_ring_schedule: src_rank and parts are both NULL");
  for (int32_t t = 0; t < cp_size; ++t) {
    // the block moves one rank per step, so after t steps rank `rank` holds
    // the one that started t ranks before it (mod N)
    const int32_t s = static_cast<int32_t>((static_cast<int64_t>(rank) - t + cp_size) % cp_size);
    if (src_rank) src_rank[t] = s;
    if (parts) {
      parts[2 * t] = s;
      parts[2 * t + 1] = 2 * cp_size - 1 - s;
    }
  }
  return ok();
}

namespace ringattn {
// Shared with the device entry point so both classify identically.
int32_t classify_pair(int64_t q_pos0, int64_t sq, int64_t k_pos0, int64_t sk, int32_t mask) {
  if (sq <= 0 || sk <= 0) return CP_CLASS_SKIP;
  if (mask == CP_MASK_NONE) return CP_CLASS_FULL;
  // Causal: the last key is visible to the first query -> every pair visible.
  if (k_pos0 + sk - 1 <= q_pos0) return CP_CLASS_FULL;
  // The first key is beyond the last query -> nothing visible.
  if (k_pos0 > q_pos0 + sq - 1) return CP_CLASS_SKIP;
  return CP_CLASS_DIAG;
}
}  // namespace ringattn

extern "C" int32_t cp_classify(int64_t q_pos0, int64_t sq, int64_t k_pos0, int64_t sk,
                               int32_t mask, int32_t* class_out) {
  RA_CHECK(class_out != nullptr, CP_EINVAL, "cp_classify: class_out is NULL");
  RA_CHECK(sq >= 0 && sk >= 0, CP_EINVAL, "cp_classify: negative length");
  RA_CHECK(mask == CP_MASK_NONE || mask == CP_MASK_CAUSAL, CP_EINVAL, "cp_classify: mask=%d",
           mask);
  *class_out = ringattn::classify_pair(q_pos0, sq, k_pos0, sk, mask);
  return ok();
}
