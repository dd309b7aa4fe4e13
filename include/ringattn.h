/*
 * ringattn.h -- C ABI of the MI355X (gfx950) blockwise ring-attention library.
 *
 * One GPU's share of ring attention / context parallelism: the head-tail
 * (zigzag) sequence partition, the interleaved KV-cache slot mapping, one
 * (Q chunk, KV block) ring step of blockwise attention that returns the
 * partial output O with its log-sum-exp (LSE), the LSE merge of partials,
 * and grouped-query decode over a sequence-sharded KV cache.
 *
 * Sources for the operations (web pages; section names given so a reader
 * can find the passage):
 *   [CP]   vLLM-Ascend developer guide, "Context Parallel (CP)" (v0.13.0):
 *          "How it works / Block table", "Decode context parallel (DCP)",
 *          "Prefill context parallel (PCP)" with its paragraphs on the
 *          head-tail token partition, prefill, decode and chunked prefill.
 *   [RA]   guijiagi.com tag page "Ring Attention": excerpts on the ring
 *          topology and on the memory wall of plain attention (formula and
 *          "key insight").
 *   [VID]  video page "How Context Parallelism Splits Long Sequences Across
 *          GPUs", chapter list (online softmax, double buffering, causal
 *          masks).
 *   [DIAG] Excalidraw diagram "Context Parallel (CP) / Ring Attention":
 *          K/V rotate around the ring while local attention runs.
 *
 * Conventions shared by every call:
 *   - Every function returns a cp_status_t value (as int32_t).  On any
 *     status other than CP_OK nothing has been written and nothing launched
 *     (except CP_EHIP, reported after a launch failed).  A short detail
 *     string for the calling thread is available from cp_last_error().
 *   - The library never prints, never throws across this boundary, keeps no
 *     global mutable state besides the thread-local error string and a
 *     per-device cache of the compute-unit count, and allocates no device
 *     memory: the caller owns every buffer.
 *   - Host functions are synchronous and take host pointers.  Device
 *     functions take device pointers (16-byte aligned, densely packed in the
 *     layouts stated), are asynchronous on `stream` (a hipStream_t passed as
 *     void*; NULL is the null stream) and return after the launch.
 *   - Integer sizes are int64_t where they can exceed 2^31; all device
 *     offsets are computed in 64 bits.
 */
#ifndef RINGATTN_H
#define RINGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RINGATTN_ABI_VERSION 3

typedef enum {
  CP_OK = 0,
  CP_EINVAL = 1,        /* bad argument: null pointer, bad size, constraint violated */
  CP_EDTYPE = 2,        /* dtype code not known */
  CP_EUNSUPPORTED = 3,  /* valid request this build has no kernel for (head dims, group size) */
  CP_EHIP = 4           /* HIP runtime reported an error at launch */
} cp_status_t;

typedef enum { CP_BF16 = 0, CP_F32 = 1 } cp_dtype_t;
typedef enum { CP_MASK_NONE = 0, CP_MASK_CAUSAL = 1 } cp_mask_t;
typedef enum { CP_CLASS_FULL = 0, CP_CLASS_DIAG = 1, CP_CLASS_SKIP = 2 } cp_class_t;

/* RINGATTN_ABI_VERSION of the loaded library. */
int32_t cp_abi_version(void);
/* Static, human-readable name of a status code. */
const char* cp_status_string(int32_t status);
/* Detail of the calling thread's last failing call ("" if none). */
const char* cp_last_error(void);

/* ------------------------------------------------------------------------
 * cp_partition -- head-tail (zigzag) token partition and restore index.
 * [CP] "Prefill context parallel (PCP)", head-tail token partition.
 *
 * Each request of length L is padded at its tail to the smallest multiple
 * of 2*cp_size, cut into 2*cp_size equal parts of c tokens, and rank r
 * takes part r followed by part 2*cp_size-1-r.  Requests are processed in
 * order and concatenated per rank.  Tokens are numbered globally, request
 * after request; padding is -1.
 *
 *   seq_lens        [num_reqs] request lengths (>= 0), host.
 *   rank            rank whose local list is produced, 0 <= rank < cp_size.
 *   local_token_idx [*local_len] out: global token ids held by `rank`.
 *   local_len       in: capacity of local_token_idx; out: entries needed.
 *   restore_idx     [*restore_len] out: restore_idx[t] is the position of
 *                   original token t in the rank-ordered concatenation of all
 *                   ranks' local lists (what an all-gather produces).
 *   restore_len     in: capacity; out: entries needed (= sum of seq_lens).
 * Pass local_token_idx == NULL and restore_idx == NULL to query the two
 * lengths only.  Either array may be NULL to skip it.  A capacity smaller
 * than needed is CP_EINVAL.
 * ---------------------------------------------------------------------- */
int32_t cp_partition(const int64_t* seq_lens, int32_t num_reqs, int32_t cp_size, int32_t rank,
                     int64_t* local_token_idx, int64_t* local_len,
                     int64_t* restore_idx, int64_t* restore_len);

/* ------------------------------------------------------------------------
 * cp_slot_mapping -- interleaved virtual-block KV placement.
 * [CP] "How it works / Block table".
 *
 * With W = pcp_size*dcp_size, a virtual block holds block_size*W tokens.
 * For token position x:  vb = x / (block_size*W),  off = x % (block_size*W),
 * lbi = off / interleave,  device = lbi % W,
 * in_block = (lbi / W) * interleave + off % interleave,
 * slot = block_table[vb] * block_size + in_block  (identity table if NULL).
 *
 *   positions   [n] token positions (>= 0), host.
 *   block_table [block_table_len] physical block of each virtual block, or
 *               NULL for the identity; every vb reached must be < len.
 *   device_out  [n] out: device id in [0, W).
 *   slot_out    [n] out: slot on that device.
 * block_size % interleave != 0 is CP_EINVAL (the page requires it).
 * ---------------------------------------------------------------------- */
int32_t cp_slot_mapping(const int64_t* positions, int64_t n, int32_t block_size,
                        int32_t interleave, int32_t pcp_size, int32_t dcp_size,
                        const int32_t* block_table, int64_t block_table_len,
                        int32_t* device_out, int64_t* slot_out);

/* ------------------------------------------------------------------------
 * cp_reorg_index -- rows of an all-gathered KV buffer in request order.
 * [CP] PCP chunked-prefill paragraph (AllGatherKV in the MLA backend) and
 * the MLA prefill note: after the all-gather the KV of several requests is
 * interleaved, and reorg_kvcache stores each request's KV contiguously.
 *
 * Gathered layout assumed: device d = 0..W-1 (W = pcp_size * dcp_size) in
 * order, each holding requests 0..num_reqs-1 in order, each request's tokens
 * at their local slots 0..n-1 (the slot mapping with an identity block
 * table).  For request r and token x < seq_lens[r] (requests in order,
 * tokens in original order), src_idx gets the gathered row of that token.
 *
 *   seq_lens  host int64 [num_reqs] context lengths.
 *   src_idx   host int64 [*src_len] out, or NULL to query the length.
 *   src_len   host int64 in: capacity of src_idx (required when src_idx is
 *             not NULL); out: sum of seq_lens.  May be NULL when src_idx is.
 *   dev_lens  host int64 [dev_lens_len] out, device-major: dev_lens[d *
 *             num_reqs + r] = tokens of request r on device d (may be NULL).
 *   dev_lens_len  capacity of dev_lens (at least W * num_reqs when given).
 * CP_EINVAL as cp_slot_mapping for the sizes; negative lengths and a
 * capacity smaller than needed are CP_EINVAL (nothing is written).
 * ---------------------------------------------------------------------- */
int32_t cp_reorg_index(const int64_t* seq_lens, int32_t num_reqs, int32_t block_size,
                       int32_t interleave, int32_t pcp_size, int32_t dcp_size, int64_t* src_idx,
                       int64_t* src_len, int64_t* dev_lens, int64_t dev_lens_len);

/* ------------------------------------------------------------------------
 * cp_ring_schedule -- which K/V block a rank computes with at each ring step.
 * [RA] ring-topology excerpt: at step t device i holds the block that
 * started on device (i - t) mod N, received from device i - 1 while it
 * passes its previous block on to device i + 1; after N steps every device
 * has met every block once.  [CP] head-tail partition: the block of rank s
 * carries sequence parts s and 2N-1-s (of 2N).
 *
 *   rank, cp_size  0 <= rank < cp_size.
 *   src_rank  host int32 [cp_size] out, or NULL: src_rank[t] = rank whose
 *             block `rank` computes with at step t (step 0 is its own).
 *   parts     host int32 [2 * cp_size] out, or NULL: parts[2t], parts[2t+1]
 *             = the head and tail part of that block.
 * At least one output must be given (CP_EINVAL otherwise).
 * ---------------------------------------------------------------------- */
int32_t cp_ring_schedule(int32_t rank, int32_t cp_size, int32_t* src_rank, int32_t* parts);

/* ------------------------------------------------------------------------
 * cp_classify -- class of one (Q range, KV range) block pair.
 * [VID] chapter on kernels, overlap and causal masks; [RA] ring topology.
 *
 * Queries sit at positions [q_pos0, q_pos0+sq), keys at [k_pos0, k_pos0+sk).
 * Under CP_MASK_CAUSAL key k is visible to query q iff k <= q.
 * *class_out = CP_CLASS_FULL if every pair is visible, CP_CLASS_SKIP if none
 * is (or the block is empty), CP_CLASS_DIAG otherwise.
 * ---------------------------------------------------------------------- */
int32_t cp_classify(int64_t q_pos0, int64_t sq, int64_t k_pos0, int64_t sk, int32_t mask,
                    int32_t* class_out);

/* ------------------------------------------------------------------------
 * ring_attn_step -- blockwise attention of one Q chunk against one KV block.
 * [RA] memory-wall excerpt (softmax(Q K^T / sqrt(d)) V accumulated block by
 * block with a running max and running sum) and ring-topology excerpt;
 * [CP] DCP section (attn_output with attn_lse, combined by the LSE rule).
 *
 *   q     [batch, sq, hq, d_qk]   dtype (CP_BF16 or CP_F32), device.
 *   k     [batch, sk, hkv, d_qk]  dtype, device.
 *   v     [batch, sk, hkv, d_v]   dtype, device.
 *   o     [batch, sq, hq, d_v]    float32, device, in/out.
 *   lse   [batch, sq, hq]         float32, device, in/out; natural log of
 *         sum_k exp(scale * q.k) over the visible keys.
 *   class_out  optional host int32: the block pair's cp_class_t.
 * Query row i is at absolute position q_pos0+i and key j at k_pos0+j; with
 * CP_MASK_CAUSAL key j is visible to row i iff k_pos0+j <= q_pos0+i.  Query
 * head h reads kv head h / (hq/hkv) (hq must be a multiple of hkv).
 * accumulate == 0: o/lse are overwritten with this block's normalised
 *   partial; rows that see no key get O = 0, LSE = -inf (a SKIP pair writes
 *   that for every row).
 * accumulate == 1: this block's partial is LSE-merged into the running
 *   (o, lse) in place; a SKIP pair launches nothing.
 * Supported (d_qk, d_v): (64,64), (128,128), (192,128); others are
 * CP_EUNSUPPORTED.  bf16 runs on MFMA with float32 accumulation; float32
 * inputs run a float32 vector path.
 * ---------------------------------------------------------------------- */
int32_t ring_attn_step(const void* q, const void* k, const void* v, int32_t dtype,
                       int32_t batch, int64_t sq, int64_t sk, int32_t hq, int32_t hkv,
                       int32_t d_qk, int32_t d_v, int64_t q_pos0, int64_t k_pos0,
                       int32_t mask, float scale, int32_t accumulate,
                       float* o, float* lse, int32_t* class_out, void* stream);

/* ------------------------------------------------------------------------
 * ring_attn_step_jobs -- one ring step for several local query chunks at once.
 * [RA] ring-topology excerpt (each step, the device's query chunks meet the
 * K/V block it holds) and memory-wall excerpt (one running max and sum per
 * row); [CP] head-tail partition (a device holds two query parts and a K/V
 * block carries two parts, each with its own positions).
 *
 * Each job is one query chunk q [batch, sq, hq, d_qk] at absolute positions
 * q_pos0.. with its outputs o [batch, sq, hq, d_v] / lse [batch, sq, hq]
 * (float32).  It attends to the union of its segments' keys; segment s is
 * k/v [batch, sk_s, hkv, d] at positions k_pos0_s..  With accumulate == 0
 * the job's (o, lse) are overwritten with that attention (O = 0, LSE = -inf
 * where no key is visible); with accumulate == 1 it is LSE-merged into them.
 * Masking, GQA mapping and scale are as for ring_attn_step.  All jobs run
 * in one launch: they share sq and must write disjoint o / lse buffers
 * (CP_EINVAL otherwise).  1 <= n_jobs <= 4, 0 <= n_segments <= 4, bf16
 * only.  Segments that no query can see are skipped on the host.
 *
 * forward / n_forward (0 <= n_forward <= 4; forward may be NULL when 0):
 * byte ranges the same launch copies src -> dst while it computes -- the
 * K/V block that moves on around the ring ([RA] ring-topology excerpt: a
 * device passes its block on while it computes with it; [VID] chapter on
 * the wire budget: the transfer overlaps the step).  On one GPU the next
 * step's block is copied into the idle staging slot; the workgroups of the
 * attention launch each move a slice (half of them before their attention
 * work, half after it), so no second stream, event or copy kernel is
 * needed.  dst / src are device pointers,
 * 16-byte aligned, bytes a multiple of 16.  A dst range may overlap no
 * other forward range (src or dst) and no q / o / lse / k / v buffer of the
 * jobs, and a src range no o / lse buffer of the jobs (CP_EINVAL).  The
 * copies complete with the launch (stream order), also when no job has any
 * visible key.
 * ---------------------------------------------------------------------- */
typedef struct {
  const void* k;   /* [batch, sk, hkv, d_qk] */
  const void* v;   /* [batch, sk, hkv, d_v]  */
  int64_t sk;
  int64_t k_pos0;
} cp_kv_segment_t;

typedef struct {
  const void* q;   /* [batch, sq, hq, d_qk] */
  float* o;        /* [batch, sq, hq, d_v]  */
  float* lse;      /* [batch, sq, hq]       */
  int64_t q_pos0;
  int32_t accumulate;
  int32_t n_segments;
  cp_kv_segment_t segments[4];
} cp_attn_job_t;

typedef struct {
  void* dst;
  const void* src;
  int64_t bytes;
} cp_copy_t;

int32_t ring_attn_step_jobs(const cp_attn_job_t* jobs, int32_t n_jobs,
                            const cp_copy_t* forward, int32_t n_forward, int32_t dtype,
                            int32_t batch, int64_t sq, int32_t hq, int32_t hkv, int32_t d_qk,
                            int32_t d_v, int32_t mask, float scale, void* stream);

/* ------------------------------------------------------------------------
 * ring_attn_step_varlen -- one ring step for several packed requests.
 * [CP] PCP head-tail partition paragraph (several requests are split and
 * laid out one after the other on each device) and chunked-prefill
 * paragraph; [VID] chapter on kernels and causal masks (per-block masks).
 *
 *   q   [total_q, hq, d_qk]  dtype, device (requests packed along tokens).
 *   k   [total_k, hkv, d_qk], v [total_k, hkv, d_v]  dtype, device.
 *   o   [total_q, hq, d_v] float32, lse [total_q, hq] float32, device.
 *   cu_seqlens_q, cu_seqlens_k  HOST int64 [n_req + 1]: request r owns
 *       query rows [cu_q[r], cu_q[r+1]) and key rows [cu_k[r], cu_k[r+1]);
 *       total_q = cu_q[n_req], total_k = cu_k[n_req].
 *   q_pos0, k_pos0  HOST int64 [n_req]: absolute position of each request's
 *       first query / key.
 * Every request is an independent ring_attn_step over its own rows: keys of
 * other requests are never visible; masking, GQA, scale and accumulate are as
 * for ring_attn_step (a request without visible keys gets O = 0, LSE = -inf,
 * or is left unchanged when accumulating).  The offsets must start >= 0 and
 * not decrease, packed lengths stay below 2^31 (CP_EINVAL / CP_EUNSUPPORTED).
 * bf16 only.  One launch covers up to 64 requests.
 * ---------------------------------------------------------------------- */
int32_t ring_attn_step_varlen(const void* q, const void* k, const void* v, int32_t dtype,
                              int32_t n_req, const int64_t* cu_seqlens_q,
                              const int64_t* cu_seqlens_k, const int64_t* q_pos0,
                              const int64_t* k_pos0, int32_t hq, int32_t hkv, int32_t d_qk,
                              int32_t d_v, int32_t mask, float scale, int32_t accumulate, float* o,
                              float* lse, void* stream);

/* ------------------------------------------------------------------------
 * cp_gather_rows -- dst row i = src row idx[i] (device).
 * [CP] PCP head-tail partition paragraph: after the ranks' outputs are
 * gathered, the restore index puts the tokens back in their original order;
 * this applies it on the device.
 *
 *   dst  [n, row_bytes], src [n_src, row_bytes]: device, 16-byte aligned,
 *        row_bytes a positive multiple of 16; dst and src must not overlap.
 *   idx  device int64 [n].  An index outside [0, n_src) gives a zero row
 *        (it is never dereferenced).
 * ---------------------------------------------------------------------- */
int32_t cp_gather_rows(void* dst, const void* src, const int64_t* idx, int64_t n, int64_t n_src,
                       int64_t row_bytes, void* stream);

/* ------------------------------------------------------------------------
 * lse_merge -- combine n partial (O, LSE) results of the same rows.
 * [CP] DCP section (output and LSE combined to update the result);
 * [RA] memory-wall excerpt (running max and running sum).
 *
 *   o_parts   [n_parts, rows, d_v] float32, device.
 *   lse_parts [n_parts, rows]      float32, device.
 *   o_out     [rows, d_v]          float32 or bf16 (out_dtype), device.
 *   lse_out   [rows]               float32, device, or NULL.
 * With M = max_k LSE_k: LSE = M + ln sum_k exp(LSE_k - M) and
 * O = sum_k exp(LSE_k - LSE) * O_k.  Rows whose parts are all -inf give
 * O = 0, LSE = -inf.  d_v must be a multiple of 4 and at most 512.
 * o_out may alias nothing in o_parts.
 * ---------------------------------------------------------------------- */
int32_t lse_merge(const float* o_parts, const float* lse_parts, int32_t n_parts, int64_t rows,
                  int32_t d_v, void* o_out, int32_t out_dtype, float* lse_out, void* stream);

/* ------------------------------------------------------------------------
 * split_kv_decode -- one-token GQA decode over a sequence-sharded KV cache.
 * [CP] "Decode context parallel (DCP)" and the PCP decode paragraph: each
 * device attends with its slice of the KV cache, then the partial outputs
 * and LSEs are combined (here: lse_merge with n_parts = n_shards).
 *
 *   q          [batch, hq, d_qk]                        dtype, device.
 *   k_shards   [n_shards, batch, t_shard, hkv, d_qk]    dtype, device.
 *   v_shards   [n_shards, batch, t_shard, hkv, d_v]     dtype, device.
 *   shard_lens device int64 [n_shards*batch]: valid tokens of each
 *              (shard, request), slots [0, len) (<= t_shard); NULL = t_shard.
 *   o_parts    [n_shards, batch, hq, d_v] float32, device, out.
 *   lse_parts  [n_shards, batch, hq]      float32, device, out.
 *   workspace  device scratch of at least split_kv_decode_workspace(...)
 *              bytes (may be NULL when that size is 0).
 * The query attends to every valid token with no mask; the order of tokens
 * inside a shard does not matter.  Only CP_BF16 with d_qk = d_v = 128 and
 * 1 <= hq/hkv <= 16 is supported in this build.
 * ---------------------------------------------------------------------- */
size_t split_kv_decode_workspace(int32_t n_shards, int32_t batch, int32_t hq, int32_t hkv,
                                 int32_t d_v, int64_t t_shard);
int32_t split_kv_decode(const void* q, const void* k_shards, const void* v_shards, int32_t dtype,
                        int32_t n_shards, int32_t batch, int64_t t_shard,
                        const int64_t* shard_lens, int32_t hq, int32_t hkv, int32_t d_qk,
                        int32_t d_v, float scale, float* o_parts, float* lse_parts,
                        void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * split_kv_decode_noalloc -- split_kv_decode without a caller workspace.
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the
 * key-split partials go to a static device array of the library instead
 * (40 MiB, held by each GPU the library runs on until the process ends),
 * and the call itself allocates nothing.  Arguments, layouts, results and
 * errors are those of split_kv_decode (same kernels); a shape whose splits
 * would need more than the array is CP_EUNSUPPORTED (no supported shape
 * does).  Calls on one GPU share its array: calls that overlap in time on
 * one GPU (different streams without ordering) race; calls ordered on one
 * stream are safe, since every call rewrites what it reads.
 * ---------------------------------------------------------------------- */
int32_t split_kv_decode_noalloc(const void* q, const void* k_shards, const void* v_shards,
                                int32_t dtype, int32_t n_shards, int32_t batch, int64_t t_shard,
                                const int64_t* shard_lens, int32_t hq, int32_t hkv, int32_t d_qk,
                                int32_t d_v, float scale, float* o_parts, float* lse_parts,
                                void* stream);

/* ------------------------------------------------------------------------
 * split_kv_decode_paged -- split_kv_decode over a paged KV cache.
 * [CP] "How it works / Block table": a request's logical KV blocks map to
 * physical blocks of the device's cache through its block table, and the
 * slot mapping places every token at block_table[vb] * block_size + offset.
 * Each shard is one device's cache pool; the decode reads through the table.
 *
 *   k_pool, v_pool  [n_shards, num_blocks, block_size, hkv, 128]  bf16, device.
 *   block_tables    device int32 [n_shards, batch, max_blocks]: physical
 *                   block of logical block j of (shard, request).  An entry
 *                   outside [0, num_blocks) is read as an empty block (its
 *                   tokens take no part), never dereferenced.
 *   shard_lens      device int64 [n_shards*batch]: local tokens of each
 *                   (shard, request); token i is row i % block_size of block
 *                   block_tables[.., i / block_size].  Clipped to
 *                   [0, max_blocks * block_size].  Required.
 *   q, o_parts, lse_parts, scale, workspace: as split_kv_decode, with the
 *   workspace sized by split_kv_decode_workspace(..., t_shard =
 *   max_blocks * block_size).
 * block_size must be a positive multiple of 32 (CP_EINVAL).  Same dtype and
 * head-size support as split_kv_decode.
 * ---------------------------------------------------------------------- */
int32_t split_kv_decode_paged(const void* q, const void* k_pool, const void* v_pool, int32_t dtype,
                              int32_t n_shards, int32_t batch, int32_t num_blocks,
                              int32_t block_size, const int32_t* block_tables, int32_t max_blocks,
                              const int64_t* shard_lens, int32_t hq, int32_t hkv, int32_t d_qk,
                              int32_t d_v, float scale, float* o_parts, float* lse_parts,
                              void* workspace, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * ring_stage_copy -- receive a ring step's K/V block into a staging slot.
 * [RA] ring-topology excerpt (each step a device takes over the K/V block of
 * its predecessor while computing); [VID] chapter on the wire budget and
 * double buffering.  On one GPU the transfer is a device-to-device copy.
 *
 *   dsts, srcs  host arrays of n device pointers (16-byte aligned).
 *   bytes       host array of n byte counts (multiples of 16).
 * Copies piece i from srcs[i] to dsts[i] for all 1 <= n <= 8 pieces in one
 * launch, asynchronously on `stream`.  Pieces must not overlap each other.
 * ---------------------------------------------------------------------- */
int32_t ring_stage_copy(void* const* dsts, const void* const* srcs, const int64_t* bytes,
                        int32_t n, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* RINGATTN_H */
