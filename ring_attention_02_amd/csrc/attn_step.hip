// One ring step of blockwise attention: a Q chunk against one K/V block,
// producing the normalised partial output O and its log-sum-exp, optionally
// merged in place into a running (O, LSE).
//
// Method: attention softmax(scale * Q K^T) V accumulated over key tiles with
// a per-row running maximum and running sum (guijiagi.com "Ring Attention",
// memory-wall excerpt, formula and "key insight"); each ring step's result is
// folded into the device's partial output (same page, ring-topology excerpt)
// with the output/LSE combine rule (vLLM-Ascend "Context Parallel (CP)",
// DCP section).  Causal masking uses absolute positions, so any Q chunk can
// meet any K/V block of a zigzag partition.
//
// gfx950 design (bf16 path):
//  * one launch is one ring step: up to 4 query chunks ("jobs"), each over up
//    to 4 K/V segments at their own positions, or up to 64 packed requests
//    (varlen); it can also copy the ring's next K/V block into the idle
//    staging slot (forwarded ranges);
//  * workgroup = 4 waves = 128 query rows of one (job, batch, query head);
//    each wave owns 32 rows whose Q fragment stays in registers for the
//    sweep; grids under two workgroups per CU use 8 waves (two key-split
//    halves that swap half their output blocks through LDS, then each
//    finalise and store half of the d_v columns), grids with at least two
//    256-row workgroups per CU use 8 waves on 256 rows sharing every K/V
//    tile, and a complementary two-job step can pair two query tiles in one
//    workgroup (on small and large grids);
//  * K/V tiles of 64 keys go HBM -> LDS with bounded buffer loads (one
//    descriptor per segment, the tile offset in soffset; rows past a segment
//    read as zero), two stages each, XOR-swizzled 16-byte chunks for
//    conflict-free b128 and transposed reads, one barrier per tile;
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand,
//    Q^T as B), so each lane holds 32 scores of ONE query row: the row max
//    and row sum are in-register plus one cross-half exchange;
//  * P^T stays in registers and is the B operand of O^T += V^T P^T; the
//    contraction order over keys is permuted to match the score layout, and
//    V^T is read with ds_read_b64_tr_b16 from row-major V in LDS;
//  * the next tile's S^T MFMAs are interleaved with this tile's
//    exponentials at raised wave priority, then P V runs with its LDS reads
//    kept ahead of the MFMAs;
//  * exp2-domain online softmax with a lazily raised running max; tiles that
//    need no mask skip it with one compare.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "kernels_common.h"
#include "status.h"

namespace ringattn {

int32_t classify_pair(int64_t q_pos0, int64_t sq, int64_t k_pos0, int64_t sk, int32_t mask);

namespace {

struct StepArgs {
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  int64_t sq, sk;
  int64_t q_pos0, k_pos0;
  int32_t hq, hkv, group;
  int32_t n_qtiles, total_wgs;
  int32_t causal, accumulate, reverse_q;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
};

// A ring step of the bf16 kernel: up to kMaxJobs query chunks (same length
// sq), each attending to up to kMaxSegs K/V segments with their own absolute
// positions.  A job's segments are swept in order with one online softmax,
// so its result is attention over the union of their keys.
constexpr int kMaxJobs = 4;
constexpr int kMaxSegs = 4;
struct KvSeg {
  const void* k;
  const void* v;
  int64_t sk, k_pos0;
};
struct QJob {
  const void* q;
  float* o;
  float* lse;
  int64_t q_pos0;
  int32_t accumulate, n_seg;
  KvSeg seg[kMaxSegs];
};
// Packed variable-length requests (one launch covers up to kMaxReq): request
// r's queries are rows [q_start, q_start + q_len) of the packed Q / O / LSE
// (whose base pointers are job 0's) at absolute positions q_pos0.., its keys
// rows [k_start, k_start + k_len) of the packed K / V (job 0's segment 0) at
// positions k_pos0..; attention never crosses requests.
constexpr int kMaxReq = 64;
struct ReqDesc {
  int32_t q_start, q_len, k_start, k_len;
  int64_t q_pos0, k_pos0;
};

// Byte ranges the launch forwards around the ring while it computes, in
// 16-byte units; fwd_end holds inclusive prefix sums (entries past n_fwd
// repeat the total) and each workgroup moves fwd_per_wg consecutive units.
constexpr int kMaxFwd = 4;
struct FwdCopy {
  u32x4* dst;
  const u32x4* src;
};
struct JobArgs {
  QJob job[kMaxJobs];
  FwdCopy fwd[kMaxFwd];
  int64_t fwd_end[kMaxFwd];
  int64_t fwd_per_wg;
  int32_t n_fwd;
  int32_t paired;   // two jobs, tile p of job 0 and tile n_qtiles-1-p of job 1 per workgroup
  int64_t sq;
  int32_t n_jobs, hq, hkv, group;
  int32_t n_qtiles, total_wgs;
  int32_t causal, reverse_q;
  int32_t serp_w;   // > 0: workgroups of odd rounds of serp_w per XCD sweep keys backwards
  float scale, scale_log2;
};
struct VarlenArgs {
  JobArgs base;
  ReqDesc req[kMaxReq];
  int32_t n_req;
  // causal launches: request r's workgroups are [wg_start[r], wg_start[r+1])
  int32_t wg_start[kMaxReq + 1];
};
template <bool VARLEN>
struct KernelArgs {
  using type = JobArgs;
};
template <>
struct KernelArgs<true> {
  using type = VarlenArgs;
};
__device__ __forceinline__ const JobArgs& base_args(const JobArgs& x) { return x; }
__device__ __forceinline__ const JobArgs& base_args(const VarlenArgs& x) { return x.base; }


// Folds a block partial (o_blk, lse_blk) into the running (o, lse) of one
// row.  Returns the merged LSE and the weights of the old and the new part.
__device__ __forceinline__ float merge_weights(float lse_old, float lse_blk, float* w_old,
                                               float* w_blk) {
  const float mx = fmaxf(lse_old, lse_blk);
  if (mx == kNegInf) {
    *w_old = 1.f;
    *w_blk = 0.f;
    return kNegInf;
  }
  const float e_old = fast_exp2((lse_old - mx) * kLog2e);
  const float e_blk = fast_exp2((lse_blk - mx) * kLog2e);
  const float s = e_old + e_blk;
  const float inv = 1.f / s;
  *w_old = e_old * inv;
  *w_blk = e_blk * inv;
  return mx + fast_log2(s) * kLn2;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
constexpr int kBM = 128;  // query rows per workgroup (4 waves x 32)
constexpr int kBN = 64;   // keys per tile
constexpr int kThreads = 256;
constexpr float kTau = 8.f;  // log2 headroom before the running max must be raised

template <int DQK, int DV>
struct Bf16Cfg {
  static constexpr int KCPR = DQK / 8;               // 16-byte chunks per K row
  static constexpr int VCPR = DV / 8;                // 16-byte chunks per V row
  static constexpr int KTILE = kBN * DQK;            // bf16 elements of one K stage
  static constexpr int VTILE = kBN * DV;             // bf16 elements of one V stage
  static constexpr int KDMA = kBN * KCPR / kThreads;  // 16-B direct loads per thread per K tile
  static constexpr int VDMA = kBN * VCPR / kThreads;
  static constexpr int QC = DQK / 16;  // MFMA steps of S^T = K Q^T
  static constexpr int DB = DV / 32;   // 32-row d_v blocks of O^T
  static_assert(KDMA * kThreads == kBN * KCPR && VDMA * kThreads == kBN * VCPR, "tile split");
};

// XOR swizzles of the 16-byte chunks inside a K / V row of LDS (self-inverse).
// K: the 16 lanes of a read quarter hold 16 consecutive keys and one chunk
// index; the swizzle spreads them over all 64 banks.
template <int CPR>
__device__ __forceinline__ int kswz(int c, int r) {
  if constexpr (CPR == 16) return c ^ (r & 15);
  else return (c & ~7) | ((c & 7) ^ ((r >> 1) & 7));   // rows of 128 or 384 bytes
}
// V: a transposed read takes 4 consecutive rows x 2 (per 16 lanes) or x 4
// (per 32 lanes) chunks; the swizzle puts those on distinct banks.
template <int CPR>
__device__ __forceinline__ int vswz(int c, int r) {
  if constexpr (CPR == 16) return c ^ (4 * (r & 3));
  else return c ^ (4 * ((r >> 1) & 1));                // rows of 128 bytes
}

// This workgroup's slice of the forwarded ranges: 16-byte units
// [wg * fwd_per_wg, ...) of their concatenation.  Half of the workgroups
// (alternate ones on each XCD) move their slice before their attention work,
// the other half after it, so each half's copy runs while the other half
// computes (the 8192-token ring sweep, one workgroup per CU, 2 % faster than
// with every slice at the start).  An early slice's first round (four units
// per thread) is split in two: its loads are issued on entry and its stores
// after the workgroup has mapped itself to its work, before the prologue's
// own loads (issuing those first was measured slower on long launches); any
// further rounds run range by range.  Lanes past the end load an in-bounds
// unit and store nothing, so the loads need no branches.
template <int NT>
struct FwdSlice {
  u32x4 x[4];
  u32x4* d[4];

  __device__ __forceinline__ void load_first(const JobArgs& a, int wg, int tid) {
    const int64_t u0 = static_cast<int64_t>(wg) * a.fwd_per_wg;
    const int64_t u1 = min(u0 + a.fwd_per_wg, a.fwd_end[kMaxFwd - 1]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t u = u0 + r * NT + tid;
      const bool valid = u < u1;
      const int64_t uc = valid ? u : u1 - 1;   // u1 >= 1: every launch forwards >= 1 unit
      const u32x4* src = a.fwd[0].src;
      u32x4* dst = a.fwd[0].dst;
      int64_t start = 0;
#pragma unroll
      for (int i = 1; i < kMaxFwd; ++i) {
        const bool later = uc >= a.fwd_end[i - 1];
        src = later ? a.fwd[i].src : src;
        dst = later ? a.fwd[i].dst : dst;
        start = later ? a.fwd_end[i - 1] : start;
      }
      x[r] = src[uc - start];
      d[r] = valid ? dst + (uc - start) : nullptr;
    }
  }

  __device__ __forceinline__ void store_first_and_rest(const JobArgs& a, int wg, int tid) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (d[r] != nullptr) *d[r] = x[r];
    const int64_t u0 = static_cast<int64_t>(wg) * a.fwd_per_wg + 4 * NT;
    const int64_t u1 = min(static_cast<int64_t>(wg) * a.fwd_per_wg + a.fwd_per_wg, a.fwd_end[kMaxFwd - 1]);
    if (u0 >= u1) return;
#pragma unroll
    for (int f = 0; f < kMaxFwd; ++f) {
      const int64_t start = f == 0 ? 0 : a.fwd_end[f - 1];
      const int64_t lo = max(u0, start) - start, hi = min(u1, a.fwd_end[f]) - start;
      if (lo >= hi) continue;
      const u32x4* __restrict__ src = a.fwd[f].src;
      u32x4* __restrict__ dst = a.fwd[f].dst;
      for (int64_t base = lo + tid; base < hi + tid; base += 4 * NT) {
        u32x4 y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = src[min(base + r * NT, hi - 1)];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (base + r * NT < hi) dst[base + r * NT] = y[r];
      }
    }
  }
};

// SPLIT = 2 doubles the waves of a workgroup: waves 4-7 sweep the odd key
// tiles of the same 128 query rows while waves 0-3 sweep the even ones, and
// the two softmax states are merged through LDS at the end.  This keeps two
// waves per SIMD even when a launch has only one workgroup per CU.
// ROWS = 2 (large grids): 8 waves own 256 query rows and share every K/V
// tile, halving the tile loads and LDS writes per FLOP.
template <int DQK, int DV, int SPLIT, bool PAIRED, bool VARLEN, int ROWS, bool TAILS>
__global__ void __launch_bounds__(kThreads * SPLIT * ROWS, 2)
attn_step_bf16_kernel(typename KernelArgs<VARLEN>::type args) {
#if defined(__HIP_DEVICE_COMPILE__)   // the host pass only needs the launch stub
  const JobArgs& a = base_args(args);
  using C = Bf16Cfg<DQK, DV>;
  // K stages of both halves, then V stages of both halves; after the sweep
  // the key-split halves swap their states through the same memory.
  constexpr int kStageElems = SPLIT * 2 * (C::KTILE + C::VTILE);
  constexpr int kSwapElems = SPLIT == 2 ? 8 * (16 * (C::DB / 2) + 2) * 64 * 2 : 0;   // floats as uint16 pairs
  __shared__ __attribute__((aligned(16))) uint16_t smem[kStageElems > kSwapElems ? kStageElems : kSwapElems];
  // (d_qk = 192: V stages first, so the transposed V reads keep their whole
  // offset in the 16-bit immediate; only K stage 1's second half reaches past
  // 64 KB)
  uint16_t* const Ks = smem + (DQK > 128 ? SPLIT * 2 * C::VTILE : 0);
  uint16_t* const Vs = smem + (DQK > 128 ? 0 : SPLIT * 2 * C::KTILE);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
  static_assert(ROWS == 1 || SPLIT == 1, "256-row tiles use one key sweep");
  constexpr int BM = kBM * ROWS;                  // query rows per workgroup
  constexpr int LW = 4 * ROWS;                    // waves that load (and read) each tile
  const int wave = ROWS == 2 ? wave_all : (wave_all & 3);  // owns 32 query rows
  const int half = SPLIT == 1 ? 0 : wave_all >> 2;  // which alternate key tiles it sweeps
  uint16_t* const Kh = Ks + half * 2 * C::KTILE;
  uint16_t* const Vh = Vs + half * 2 * C::VTILE;
  // An early workgroup's loads of its slice of the forwarded block go out
  // first; a late one moves its slice after its work items.
  FwdSlice<kThreads * SPLIT * ROWS> fwd;
  const bool fwd_late = ((blockIdx.x >> 3) & 1) != 0;
  if (a.n_fwd > 0 && !fwd_late) fwd.load_first(a, blockIdx.x, tid);

  const int col = lane & 31;  // query row within the wave (B / C column)
  const int hh = lane >> 5;   // which half of each contraction slice this lane holds
  const int g = lane >> 4;    // 16-lane group (transposed V reads)
  const int i16 = lane & 15;

  // Workgroup -> work items (job, query tile) of one (head, batch).  Plain
  // launches: one item, job fastest so every XCD's contiguous range mixes
  // all jobs and tile weights.  Paired launches (two jobs whose tile loads
  // are complementary, as the two query parts of a head-tail rank at the
  // diagonal step): item 0 is query tile p of job 0, item 1 is tile
  // n_qtiles-1-p of job 1, run one after the other.
  const int logical = xcd_contiguous_id(blockIdx.x, a.total_wgs);
  // Serpentine key order: the workgroups an XCD runs together sweep a kv
  // head's tiles in step and share its L2; one that starts after another
  // finished sweeps the other way, from where the running ones still are.
  const bool rev = a.serp_w > 0 && ((blockIdx.x / 8) / a.serp_w) % 2 == 1;
  int jb0, qt0, rest;
  if constexpr (PAIRED) {
    jb0 = 0;
    qt0 = logical % a.n_qtiles;
    rest = logical / a.n_qtiles;
  } else if constexpr (VARLEN) {
    // (jb0 names the request here)
    if (a.reverse_q) {
      // Causal requests, request by request (the host orders them longest
      // first), each request's query tiles longest first (a tile's load
      // grows with its index), then the query head within its kv group, kv
      // head fastest.  Consecutive ids go to consecutive XCDs, so with 8 kv
      // heads each XCD keeps to one of them, and the workgroups it runs
      // together are neighbouring tiles of one request: they sweep the same
      // keys and share the XCD's L2.
      const int id = static_cast<int>(blockIdx.x);
      int r = 0;
      while (r + 1 < args.n_req && args.wg_start[r + 1] <= id) ++r;
      int local = id - args.wg_start[r];
      const int kv = local % a.hkv;
      local /= a.hkv;
      const int gq = local % a.group;
      local /= a.group;
      jb0 = r;
      qt0 = (args.req[r].q_len + BM - 1) / BM - 1 - local;
      rest = kv * a.group + gq;   // the query head (packed requests: batch 0)
    } else {
      // query tile fastest, then request
      qt0 = logical % a.n_qtiles;
      rest = logical / a.n_qtiles;
      jb0 = rest % args.n_req;
      rest /= args.n_req;
    }
  } else {
    jb0 = logical % a.n_jobs;
    rest = logical / a.n_jobs;
    qt0 = rest % a.n_qtiles;
    rest /= a.n_qtiles;
    if (a.reverse_q) qt0 = a.n_qtiles - 1 - qt0;
  }
  const int h = rest % a.hq;
  const int b = rest / a.hq;
  const int kvh = h / a.group;
  if (a.n_fwd > 0 && !fwd_late) fwd.store_first_and_rest(a, blockIdx.x, tid);
#pragma unroll
  for (int item = 0; item < (PAIRED ? 2 : 1); ++item) {
  if (item > 0) __syncthreads();   // the previous item is done with the LDS stages
  // Large-grid pairs run the tail tile first: the workgroups an XCD runs
  // together then sweep the shared head chunk in step before their lengths
  // diverge (1M-token diagonal step 4 % faster; the 8-wave pairs measured
  // better in the written order).
  constexpr bool kLongFirst = PAIRED && ROWS == 2;
  const bool second = kLongFirst ? item == 0 : item == 1;
  const int jb = second ? 1 : jb0;
  const int qt = second ? a.n_qtiles - 1 - qt0 : qt0;
  const QJob& job = a.job[VARLEN ? 0 : jb];
  // The job's fields: its own, or a packed request's slice of job 0's
  // buffers (one segment).  Read where they are used (no copies held live).
  auto j_sq = [&]() -> int64_t {
    if constexpr (VARLEN) return args.req[jb].q_len;
    else return a.sq;
  };
  auto j_qpos0 = [&]() -> int64_t {
    if constexpr (VARLEN) return args.req[jb].q_pos0;
    else return job.q_pos0;
  };
  auto j_o = [&]() -> float* {
    if constexpr (VARLEN) return job.o + static_cast<int64_t>(args.req[jb].q_start) * a.hq * DV;
    else return job.o;
  };
  auto j_lse = [&]() -> float* {
    if constexpr (VARLEN) return job.lse + static_cast<int64_t>(args.req[jb].q_start) * a.hq;
    else return job.lse;
  };
  auto j_nseg = [&]() -> int {
    if constexpr (VARLEN) return 1;
    else return job.n_seg;
  };
  auto seg_base = [&](int sg, bool is_k) -> const uint16_t* {
    if constexpr (VARLEN)
      return static_cast<const uint16_t*>(is_k ? job.seg[0].k : job.seg[0].v) +
             static_cast<int64_t>(args.req[jb].k_start) * a.hkv * (is_k ? DQK : DV);
    else
      return static_cast<const uint16_t*>(is_k ? job.seg[sg].k : job.seg[sg].v);
  };
  auto seg_sk = [&](int sg) -> int64_t {
    if constexpr (VARLEN) return args.req[jb].k_len;
    else return job.seg[sg].sk;
  };
  auto seg_kpos0 = [&](int sg) -> int64_t {
    if constexpr (VARLEN) return args.req[jb].k_pos0;
    else return job.seg[sg].k_pos0;
  };
  const int64_t sq = j_sq();
  if (VARLEN && static_cast<int64_t>(qt) * BM >= sq) continue;   // past this request's queries
  const uint16_t* jq = static_cast<const uint16_t*>(job.q);
  if constexpr (VARLEN) jq += static_cast<int64_t>(args.req[jb].q_start) * a.hq * DQK;

  const uint16_t* __restrict__ qg = jq;

  const int64_t q_first = static_cast<int64_t>(qt) * BM;
  const int64_t q_last = min(sq, q_first + BM) - 1;  // last valid local row of the WG
  const int64_t wq0 = q_first + wave * 32;              // first row of this wave
  const int64_t my_row = wq0 + col;
  const bool row_valid = my_row < sq;
  const int64_t qpos = j_qpos0() + my_row;

  // The job's segments, each with the number of its tiles that some row of
  // this workgroup can see; the sweep walks them segment after segment
  // ("virtual" tile numbers).  The cursors below read a segment's fields
  // from the argument block (uniform scalar loads) only when the sweep
  // enters it, so no segment state occupies registers in between.
  auto seg_tiles = [&](int sg) -> int {
    if (sg >= j_nseg()) return 0;
    int64_t nkeys = seg_sk(sg);
    if (a.causal) {
      const int64_t lim = j_qpos0() + q_last - seg_kpos0(sg) + 1;
      nkeys = lim < 0 ? 0 : (lim < nkeys ? lim : nkeys);
    }
    return static_cast<int>((nkeys + kBN - 1) / kBN);
  };
  static_assert(kMaxSegs == 4, "four segment slots per job");
  const int ntiles = seg_tiles(0) + seg_tiles(1) + seg_tiles(2) + seg_tiles(3);
  // Moves a cursor (segment sg covering virtual tiles [start, end)) forward
  // to the segment that holds virtual tile vt < ntiles.
  auto advance = [&](int& sg, int& start, int& end, int vt) {
    if (vt < start) {   // a backward sweep left the segment: start over
      sg = -1;
      start = end = 0;
    }
    while (vt >= end && sg < kMaxSegs - 1) {
      ++sg;
      start = end;
      end = start + seg_tiles(sg);
    }
  };

  // Q^T fragment (B operand): for step c the lane holds Q[row][16c + 8hh .. +7].
  bf16x8 qf[C::QC];
  {
    const uint16_t* qp = qg + ((static_cast<int64_t>(b) * sq + (row_valid ? my_row : 0)) * a.hq + h) * DQK;
#pragma unroll
    for (int c = 0; c < C::QC; ++c) {
      u32x4 raw = *reinterpret_cast<const u32x4*>(qp + 16 * c + 8 * hh);
      if (!row_valid) raw = u32x4{0u, 0u, 0u, 0u};
      qf[c] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 oacc[C::DB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  float m_run = kNegInf;  // running max of raw scores of this lane's row (possibly stale by < tau)
  float l_run = 0.f;      // running sum over this lane's half of the keys

  // Direct buffer->LDS loads.  Each of K and V has a cursor on the segment
  // that holds the current tile; the segment's fields are read from the
  // argument block only when the sweep enters it.  Wave-instruction i fills
  // 64 consecutive 16-byte LDS slots; each lane fetches the logical chunk
  // the swizzle maps to its slot, at a loop-invariant byte offset inside the
  // tile.  Rows past the end of a segment must read as zeros (their scores
  // are masked, but 0 * NaN in P V would still poison O), and the range
  // check of a raw buffer load covers the per-lane offset only, not the
  // uniform soffset:
  //  * launches whose segments all hold whole 64-key tiles (TAILS false):
  //    one descriptor per segment, based at some tile of it, the tile offset
  //    in soffset; it is rebuilt when the sweep enters a segment or has
  //    moved 2^30 bytes past its base.  No tile reaches past its segment.
  //  * launches with a partial last tile somewhere (TAILS true): every tile
  //    load uses a descriptor based at that tile, whose record count ends at
  //    the segment's last key, so the rows past the end are out of range.
  // (Building a descriptor per tile costs 0.5 scalar instructions per MFMA,
  // which measured 4 % on long launches; hence the two forms.)
  const int64_t row_elems_k = static_cast<int64_t>(a.hkv) * DQK;
  const int64_t row_elems_v = static_cast<int64_t>(a.hkv) * DV;
  constexpr int KDMA_W = C::KDMA / ROWS, VDMA_W = C::VDMA / ROWS;   // per wave
  static_assert(KDMA_W * ROWS == C::KDMA && VDMA_W * ROWS == C::VDMA, "tile loads split evenly");
  uint32_t koffb[KDMA_W], voffb[VDMA_W];
#pragma unroll
  for (int i = 0; i < KDMA_W; ++i) {
    const int p = (i * LW + wave) * 64 + lane;
    const int row = p / C::KCPR;
    koffb[i] = static_cast<uint32_t>((row * row_elems_k + kswz<C::KCPR>(p % C::KCPR, row) * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < VDMA_W; ++i) {
    const int p = (i * LW + wave) * 64 + lane;
    const int row = p / C::VCPR;
    voffb[i] = static_cast<uint32_t>((row * row_elems_v + vswz<C::VCPR>(p % C::VCPR, row) * 8) * 2);
  }
  const int tile_bytes_k = static_cast<int>(kBN * row_elems_k * 2);
  const int tile_bytes_v = static_cast<int>(kBN * row_elems_v * 2);
  const int rebase_k = (1 << 30) / tile_bytes_k, rebase_v = (1 << 30) / tile_bytes_v;
  struct DmaCursor {
    int sg, start, end;
    int base_vt;                    // whole tiles: the descriptor's base tile
    __amdgpu_buffer_rsrc_t rsrc;    // whole tiles: the segment's descriptor
    const char* base;               // tails: the segment's key 0, this (batch, kv head)
    int64_t valid;                  // tails: bytes from base to the end of key sk-1's row
  };
  auto seek = [&](DmaCursor& c, int vt, bool is_k) {
    advance(c.sg, c.start, c.end, vt);
    const int64_t sk = seg_sk(c.sg);
    const int64_t row_elems = is_k ? row_elems_k : row_elems_v;
    const int width = is_k ? DQK : DV;
    const uint16_t* base = seg_base(c.sg, is_k) + (static_cast<int64_t>(b) * sk * a.hkv + kvh) * width;
    if constexpr (TAILS) {
      c.base = reinterpret_cast<const char*>(base);
      c.valid = ((sk - 1) * row_elems + width) * 2;
    } else {
      // a backward sweep bases the descriptor below vt so the next tiles reuse it
      const int rebase = is_k ? rebase_k : rebase_v;
      const int base_vt = rev ? max(c.start, vt - rebase + 1) : vt;
      const int64_t key0 = static_cast<int64_t>(base_vt - c.start) * kBN;
      // bytes from the base tile to the end of key sk-1's row of this head
      const int64_t valid = ((sk - 1 - key0) * row_elems + width) * 2;
      const int nrec = valid > 0x7FFFFFF0 ? 0x7FFFFFF0 : static_cast<int>(valid);
      c.base_vt = base_vt;
      c.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base + key0 * row_elems),
                                                 static_cast<short>(0), nrec, 0x00020000);
    }
  };
  // The descriptor and soffset of tile vt (moving the cursor first if needed).
  auto tile_src = [&](DmaCursor& c, int vt, bool is_k, int* soff) {
    if constexpr (TAILS) {
      if (vt >= c.end || vt < c.start) seek(c, vt, is_k);
      const int64_t off = static_cast<int64_t>(vt - c.start) * (is_k ? tile_bytes_k : tile_bytes_v);
      const uint64_t left = static_cast<uint64_t>(c.valid - off);   // > 0: the tile holds a key
      const int nrec = (left >> 31) != 0 ? 0x7FFFFFF0 : static_cast<int>(left);
      *soff = 0;
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(c.base + off), static_cast<short>(0), nrec,
                                               0x00020000);
    } else {
      if (vt >= c.end || vt < c.base_vt || vt - c.base_vt >= (is_k ? rebase_k : rebase_v)) seek(c, vt, is_k);
      *soff = (vt - c.base_vt) * (is_k ? tile_bytes_k : tile_bytes_v);
      return c.rsrc;
    }
  };
  const auto no_rsrc = __builtin_amdgcn_make_buffer_rsrc(static_cast<void*>(nullptr), static_cast<short>(0), 0, 0);
  DmaCursor kcur{-1, 0, 0, 0, no_rsrc, nullptr, 0}, vcur{-1, 0, 0, 0, no_rsrc, nullptr, 0};
  auto dma_k = [&](int vt, int stage) {
    int soff;
    const auto rsrc = tile_src(kcur, vt, true, &soff);
    uint16_t* dst = Kh + stage * C::KTILE;
#pragma unroll
    for (int i = 0; i < KDMA_W; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(dst + (i * LW + wave) * 64 * 8), 16,
          static_cast<int>(koffb[i]), soff, 0, 0);
  };
  auto dma_v = [&](int vt, int stage) {
    int soff;
    const auto rsrc = tile_src(vcur, vt, false, &soff);
    uint16_t* dst = Vh + stage * C::VTILE;
#pragma unroll
    for (int i = 0; i < VDMA_W; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(dst + (i * LW + wave) * 64 * 8), 16,
          static_cast<int>(voffb[i]), soff, 0, 0);
  };

  // One K fragment (A operand of S^T = K Q^T): key 32kb + col, d chunk 2c + hh.
  auto k_frag = [&](const uint16_t* kst, int kb, int c) -> bf16x8 {
    const int key = kb * 32 + col;
    const int slot = kswz<C::KCPR>(2 * c + hh, key);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kst + (key * C::KCPR + slot) * 8));
  };
  // One V^T fragment (A operand of O^T += V^T P^T) for d_v block d and
  // 16-key chunk kc, from row-major V through two transposed LDS reads of
  // rows r0 = 16kc + 4(g/2) + i16/4 and r0 + 8.  The V swizzle reads bits
  // of r0 that 16kc and +8 leave alone, so each d_v block also has a single
  // per-lane base, with the chunk, the second read and the stage as constant
  // offsets.  The d_qk = 192 kernels use that form: it takes the
  // transposed-read addresses out of the registers their fast loop would
  // otherwise spill (the d_qk <= 128 kernels measured faster with the
  // addresses formed per read).
  constexpr bool kVBase = DQK > 128;
  int vbase[C::DB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d) {
    const int r = 4 * (g >> 1) + (i16 >> 2);
    const int cc = 4 * d + 2 * (g & 1) + ((i16 & 3) >> 1);
    vbase[d] = (r * C::VCPR + vswz<C::VCPR>(cc, r)) * 8 + 4 * (i16 & 1);
  }
  auto v_frag = [&](const uint16_t* vst, int d, int kc) -> bf16x8 {
    if constexpr (kVBase) {
      const uint16_t* p = vst + vbase[d] + kc * 16 * C::VCPR * 8;
      return join_bf16x4(lds_read_tr16(p), lds_read_tr16(p + 8 * C::VCPR * 8));
    } else {
      const int r0 = kc * 16 + 4 * (g >> 1) + (i16 >> 2);
      const int r1 = r0 + 8;
      const int cc = 4 * d + 2 * (g & 1) + ((i16 & 3) >> 1);
      const int half = 4 * (i16 & 1);
      const s16x4 lo = lds_read_tr16(vst + (r0 * C::VCPR + vswz<C::VCPR>(cc, r0)) * 8 + half);
      const s16x4 hi = lds_read_tr16(vst + (r1 * C::VCPR + vswz<C::VCPR>(cc, r1)) * 8 + half);
      return join_bf16x4(lo, hi);
    }
  };
  // Scores of a whole tile: s[kb][i] is key 32kb + 8(i/4) + 4hh + i%4.
  auto qk = [&](int stage, f32x16* s) {
    const uint16_t* kst = Kh + stage * C::KTILE;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int c = 0; c < C::QC; ++c)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag(kst, kb, c), qf[c], s[kb], 0, 0, 0);
  };
  auto pv = [&](int stage, const bf16x8* pb) {
    const uint16_t* vst = Vh + stage * C::VTILE;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc)
#pragma unroll
      for (int d = 0; d < C::DB; ++d)
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_frag(vst, d, kc), pb[kc], oacc[d], 0, 0, 0);
    // keep a few transposed reads in flight ahead of each MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 4 * C::DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i + 2 < 4 * C::DB) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };
  // Masking cursor of this wave: the segment of the tile being softmaxed and
  // the first of its tiles in which some key is past the segment end or, for
  // a causal mask, later than this wave's first query.
  struct MaskCursor {
    int sg, start, end, mask_from;
    int64_t sk, k_pos0;
  };
  MaskCursor mcur{-1, 0, 0, 0, 0, 0};
  auto mask_tile = [&](int vt, f32x16* s) {
    if (vt >= mcur.end || vt < mcur.start) {
      advance(mcur.sg, mcur.start, mcur.end, vt);
      mcur.sk = seg_sk(mcur.sg);
      mcur.k_pos0 = seg_kpos0(mcur.sg);
      int64_t from = mcur.sk / kBN;                       // the partial last tile, if any
      if (a.causal) {
        // key0 + kBN - 1 > q_pos0 + wq0 - k_pos0  <=>  key0 >= that - kBN + 2
        const int64_t d = j_qpos0() + wq0 - mcur.k_pos0 - kBN + 2;
        const int64_t tc = d <= 0 ? 0 : (d + kBN - 1) / kBN;
        from = min(from, tc);
      }
      mcur.mask_from = mcur.start + static_cast<int>(min(from, static_cast<int64_t>(1) << 30));
    }
    if (vt < mcur.mask_from) return;
    const int64_t key0 = static_cast<int64_t>(vt - mcur.start) * kBN;
    // visible iff local key < min(sk, qpos - k_pos0 + 1)
    const int64_t lim64 = a.causal ? min(mcur.sk, qpos - mcur.k_pos0 + 1) : mcur.sk;
    const int lim = static_cast<int>(max(min(lim64 - key0, static_cast<int64_t>(kBN)), static_cast<int64_t>(0)));
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb * 32 + 8 * (i / 4) + 4 * hh + (i % 4) >= lim) s[kb][i] = kNegInf;
  };
  // Exponentials of one tile against the (possibly stale) running max, their
  // sum, and P in bf16 for the PV product.
  auto exps = [&](const f32x16* s, bf16x8* pb, float neg_mc) -> float {
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(fmaf(s[kb][8 * mm + e], a.scale_log2, neg_mc));
          psum += p;
          pb[kb * 2 + mm][e] = static_cast<__bf16>(p);
        }
    return psum;
  };

  // This half sweeps tiles half, half + SPLIT, ...: my_n of them.  Every wave
  // runs the same number of iterations (barriers stay uniform); a half with
  // fewer tiles idles through its last one.
  const int my_n = ntiles > half ? (ntiles - half + SPLIT - 1) / SPLIT : 0;
  const int n_iter = (ntiles + SPLIT - 1) / SPLIT;
  auto tile = [&](int j) { return rev ? ntiles - 1 - (j * SPLIT + half) : j * SPLIT + half; };
  // Online softmax of tile j (exp2 domain) plus the scores of tile j+1 on
  // MFMA interleaved with the exponentials.  The next scores are computed
  // even after the last tile (from a stale stage, then dropped): with no
  // branch around them the exponentials and the MFMAs share one basic block
  // and the interleave holds.  Both halves of a
  // row share m_run.  It is raised only when some row of the wave gained more
  // than tau (log2 units); otherwise the stale max stays, which is exact
  // because numerator and denominator share it, and P stays below 2^tau.
  // The loop is unrolled by two so the score buffers swap without copies
  // (paired kernels also unroll their two work items, which keeps them free
  // of spills).
  // The interleave is written out chunk by chunk in every kernel but the
  // 8-wave paired one at d_qk <= 128, where the scheduler's group pattern
  // (below) spills less.  Timed side by side against the group pattern: the
  // 1M-token sweep 1 % faster, the chunked prefill (d_qk 192, whose
  // exponentials the pattern left after all 24 MFMAs) 4 % faster.
  constexpr bool kChunked = !(PAIRED && SPLIT == 2) || DQK > 128;
  auto softmax_and_next_scores = [&](int j, f32x16* s_cur, f32x16* s_nxt, bf16x8* pb, int next_stage) {
    mask_tile(tile(j), s_cur);
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s_cur[kb][i]);
    if (__ballot((mx - m_run) * a.scale_log2 > kTau) != 0) {   // false for -inf - -inf
      const float full = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, full);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * a.scale_log2);   // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < C::DB; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;
      m_run = m_new;
    }
    const float neg_mc = -(m_run == kNegInf ? 0.f : m_run) * a.scale_log2;
    // Raised wave priority over the interleaved block: when both waves of a
    // SIMD are ready, the one in this block issues first (measured +2 % on
    // long launches; the same around the PV block gained nothing).
    __builtin_amdgcn_s_setprio(1);
    if constexpr (kChunked) {
      // Written out d_qk chunk by chunk: per chunk c the two score MFMAs of
      // tile j+1, the LDS reads of chunk c+2's K fragments (two chunks
      // ahead: the chunked prefill at d_qk 192 1.7 % faster than one ahead,
      // the others within noise), and the exponentials of 16/QC score pairs
      // of tile j, each chunk held in place (its row sum pinned to it, so
      // the adds do not sink to the end).
      const uint16_t* kst = Kh + next_stage * C::KTILE;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s_nxt[kb][i] = 0.f;
      bf16x8 f0 = k_frag(kst, 0, 0), f1 = k_frag(kst, 1, 0);
      bf16x8 g0 = k_frag(kst, 0, 1), g1 = k_frag(kst, 1, 1);
      float psum = 0.f;
#pragma unroll
      for (int c = 0; c < C::QC; ++c) {
        bf16x8 n0 = g0, n1 = g1;
        if (c + 2 < C::QC) {
          g0 = k_frag(kst, 0, c + 2);
          g1 = k_frag(kst, 1, c + 2);
        }
        s_nxt[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0, qf[c], s_nxt[0], 0, 0, 0);
        s_nxt[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1, qf[c], s_nxt[1], 0, 0, 0);
#pragma unroll
        for (int t = 2 * ((16 * c) / C::QC); t < 2 * ((16 * (c + 1)) / C::QC); ++t) {
          const int kb = t / 16, mm = (t / 8) % 2, e = t % 8;
          const float p = fast_exp2(fmaf(s_cur[kb][8 * mm + e], a.scale_log2, neg_mc));
          psum += p;
          pb[kb * 2 + mm][e] = static_cast<__bf16>(p);
        }
        asm volatile("" : "+v"(psum));
        __builtin_amdgcn_sched_barrier(0);
        f0 = n0;
        f1 = n1;
      }
      l_run += psum;
    } else {
      qk(next_stage, s_nxt);               // MFMA: scores of tile j+1 ...
      l_run += exps(s_cur, pb, neg_mc);    // ... interleaved with the VALU exponentials of tile j
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 0; i < 2 * C::QC; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 112 / (2 * C::QC), 0);
        if (i + 2 < 2 * C::QC) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // prologue: K of this half's tiles 0 and 1 and V of tile 0 in flight
  if (my_n > 0) dma_k(tile(0), 0);
  if (my_n > 1) dma_k(tile(1), 1);
  if (my_n > 0) dma_v(tile(0), 0);

  if (n_iter > 0) {
    f32x16 s_cur[2], s_nxt[2];
    bf16x8 pb[4];
    // Iteration j: [scores of tile j+1 on MFMA + softmax of tile j] then
    // [P_j V_j].  (Running the two key-split halves in opposite phase orders
    // was measured slower on gfx950 than this lock-step order.)
    // scores of tile 0 once the prologue's loads have landed
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (my_n > 0) qk(0, s_cur);
    // One iteration; P = j & 1 is the parity of j, so the stage offsets are
    // constants and the two score buffers swap roles without copies.
    auto iteration = [&](int j, auto parity, f32x16* sc, f32x16* sn) {
      constexpr int P = decltype(parity)::value;
      // The loads issued at the start of iteration j-1 have landed for every
      // wave, and every wave is done with iteration j-1.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (j + 2 < my_n) dma_k(tile(j + 2), P);        // K stage j%2 held K_j (read in j-1)
      if (j + 1 < my_n) dma_v(tile(j + 1), P ^ 1);    // V stage (j+1)%2 held V_{j-1}
      if (j < my_n) {
        softmax_and_next_scores(j, sc, sn, pb, P ^ 1);
        pv(P, pb);                                     // MFMA: O += P_j V_j
      }
    };
    for (int j = 0; j < n_iter; j += 2) {
      iteration(j, std::integral_constant<int, 0>{}, s_cur, s_nxt);
      if (j + 1 < n_iter) iteration(j + 1, std::integral_constant<int, 1>{}, s_nxt, s_cur);
    }
  }

  // ---- epilogue: normalise, LSE, optional merge into the running result.
  // In the key-split variant each half finalises half of the d_v blocks
  // (half 0 the low ones), after the two halves have swapped the other
  // blocks and their (max, sum) through LDS; so all eight waves store.  The
  // running result of an accumulating launch is fetched before that swap,
  // so its latency hides behind it.
  constexpr int DH = SPLIT == 2 ? C::DB / 2 : C::DB;   // d_v blocks this wave finalises
  static_assert(DH * SPLIT == C::DB, "d_v blocks split evenly between the halves");
  const int64_t orow = (static_cast<int64_t>(b) * sq + (row_valid ? my_row : 0)) * a.hq + h;
  float* const op = j_o() + orow * DV + half * DH * 32;   // first column of my blocks
  const bool acc = job.accumulate != 0;
  float lse_old = kNegInf;
  f32x4 o_old[DH * 4];
  auto load_old = [&]() {
    if (!acc || !row_valid) return;
    lse_old = j_lse()[orow];
#pragma unroll
    for (int dd = 0; dd < DH; ++dd)
#pragma unroll
      for (int j = 0; j < 4; ++j) o_old[4 * dd + j] = *reinterpret_cast<const f32x4*>(op + dd * 32 + 8 * j + 4 * hh);
  };
  // (The paired kernel reads it at the stores: held across the swap, it spills.)
  constexpr bool kEarlyOld = !PAIRED;
  if constexpr (kEarlyOld) load_old();
  // Swap buffer of the key-split halves, lane by lane (the same query row
  // and key half hh in both waves): [wave_all][16*DH + 2][64 lanes].
  constexpr int NV = 16 * DH + 2;
  static_assert(SPLIT == 1 || 8 * NV * 64 * sizeof(float) <= sizeof(smem), "swap buffer fits the stages");
  float* const mine = reinterpret_cast<float*>(smem) + wave_all * NV * 64 + lane;
  const float* const theirs = reinterpret_cast<const float*>(smem) + (wave_all ^ 4) * NV * 64 + lane;
  // Register blocks are indexed with constants only: H is this wave's half.
  auto swap_out = [&](auto hc) {
    constexpr int P0 = (1 - decltype(hc)::value) * DH;   // the partner's blocks
#pragma unroll
    for (int dd = 0; dd < DH; ++dd)
#pragma unroll
      for (int i = 0; i < 16; ++i) mine[(16 * dd + i) * 64] = oacc[P0 + dd][i];
    mine[(NV - 2) * 64] = m_run;
    mine[(NV - 1) * 64] = l_run;
  };
  auto finish = [&](auto hc) {
    constexpr int H = decltype(hc)::value;
    constexpr int D0 = H * DH;   // my blocks
    if constexpr (SPLIT == 2) {
      const float m1 = theirs[(NV - 2) * 64];
      const float l1 = theirs[(NV - 1) * 64];
      const float m = fmaxf(m_run, m1);
      const float m_use = m == kNegInf ? 0.f : m;
      const float a0 = fast_exp2((m_run - m_use) * a.scale_log2);   // 0 for an empty side
      const float a1 = fast_exp2((m1 - m_use) * a.scale_log2);
#pragma unroll
      for (int dd = 0; dd < DH; ++dd)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[D0 + dd][i] = oacc[D0 + dd][i] * a0 + theirs[(16 * dd + i) * 64] * a1;
      l_run = l_run * a0 + l1 * a1;
      m_run = m;
    }
    if (!row_valid) return;
    if constexpr (!kEarlyOld) {
      if (acc) lse_old = j_lse()[orow];
    }
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const bool has = m_run != kNegInf && l_tot > 0.f;
    const float inv = has ? 1.f / l_tot : 0.f;
    const float lse_blk = has ? m_run * a.scale + fast_log2(l_tot) * kLn2 : kNegInf;
    float w_old = 0.f, w_blk = 1.f, lse_out = lse_blk;
    if (acc) lse_out = merge_weights(lse_old, lse_blk, &w_old, &w_blk);
    const float wb = w_blk * inv;
#pragma unroll
    for (int dd = 0; dd < DH; ++dd)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& oa = oacc[D0 + dd];
        f32x4 val = {oa[4 * j] * wb, oa[4 * j + 1] * wb, oa[4 * j + 2] * wb, oa[4 * j + 3] * wb};
        if (acc) {
          if constexpr (kEarlyOld) val += o_old[4 * dd + j] * w_old;
          else val += *reinterpret_cast<const f32x4*>(op + dd * 32 + 8 * j + 4 * hh) * w_old;
        }
        *reinterpret_cast<f32x4*>(op + dd * 32 + 8 * j + 4 * hh) = val;
      }
    if (H == 0 && hh == 0) j_lse()[orow] = lse_out;
  };
  if constexpr (SPLIT == 2) {
    __syncthreads();   // every wave is done with the K/V stages
    if (half == 0) swap_out(std::integral_constant<int, 0>{});
    else swap_out(std::integral_constant<int, 1>{});
    __syncthreads();
    if (half == 0) finish(std::integral_constant<int, 0>{});
    else finish(std::integral_constant<int, 1>{});
  } else {
    finish(std::integral_constant<int, 0>{});
  }
  }   // work items
  if (a.n_fwd > 0 && fwd_late) {
    fwd.load_first(a, blockIdx.x, tid);
    fwd.store_first_and_rest(a, blockIdx.x, tid);
  }
#endif
}

// ---------------------------------------------------------------------------
// float32 vector kernel (correctness path for float32 inputs)
// ---------------------------------------------------------------------------
// One query row per lane: a workgroup holds 64 rows of one (batch, head) in
// each of its 4 waves, and wave w sweeps key tiles w, w + 4, ... with its own
// running max, sum and output, staged through its own LDS tile.  The four
// states are merged by the running-max rule at the end (the same online
// softmax, applied across the key split).
constexpr int kF32Rows = 64;   // query rows per workgroup (one per lane)
constexpr int kF32Waves = 4;   // key-split waves per workgroup
constexpr int kF32Keys = 16;   // keys per tile

template <int DQK, int DV>
struct F32Smem {
  static constexpr int kTile = kF32Waves * kF32Keys * (DQK + DV);        // every wave's K and V tile
  static constexpr int kMerge = (kF32Waves - 1) * (DV + 2) * kF32Rows;   // waves 1..3: O, max, sum
  static constexpr int kFloats = kTile > kMerge ? kTile : kMerge;
};

template <int DQK, int DV>
__global__ void __launch_bounds__(kF32Rows * kF32Waves) attn_step_f32_kernel(StepArgs a) {
  __shared__ float smem[F32Smem<DQK, DV>::kFloats];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float* const Ks = smem + wave * kF32Keys * (DQK + DV);   // [kF32Keys][DQK]
  float* const Vs = Ks + kF32Keys * DQK;                    // [kF32Keys][DV]
  const int logical = xcd_contiguous_id(blockIdx.x, a.total_wgs);
  int qt = logical % a.n_qtiles;
  const int rest = logical / a.n_qtiles;
  const int h = rest % a.hq;
  const int b = rest / a.hq;
  if (a.reverse_q) qt = a.n_qtiles - 1 - qt;
  const int kvh = h / a.group;
  const float* qg = static_cast<const float*>(a.q);
  const float* kg = static_cast<const float*>(a.k);
  const float* vg = static_cast<const float*>(a.v);

  const int64_t q_first = static_cast<int64_t>(qt) * kF32Rows;
  const int64_t q_last = min(a.sq, q_first + kF32Rows) - 1;
  const int64_t my_row = q_first + lane;
  const bool row_valid = my_row < a.sq;
  const int64_t qpos = a.q_pos0 + my_row;
  int64_t nkeys = a.sk;
  if (a.causal) {
    const int64_t lim = a.q_pos0 + q_last - a.k_pos0 + 1;
    nkeys = lim < 0 ? 0 : (lim < a.sk ? lim : a.sk);
  }

  float qr[DQK];
  float acc[DV];
  const int64_t orow = (static_cast<int64_t>(b) * a.sq + my_row) * a.hq + h;
#pragma unroll
  for (int d = 0; d < DQK; ++d) qr[d] = row_valid ? qg[orow * DQK + d] : 0.f;
#pragma unroll
  for (int d = 0; d < DV; ++d) acc[d] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  // Every wave runs the same number of iterations (the barriers stay
  // uniform); a wave past the last tile idles through its last one.
  const int64_t ntiles = (nkeys + kF32Keys - 1) / kF32Keys;
  const int64_t n_iter = (ntiles + kF32Waves - 1) / kF32Waves;
  for (int64_t it = 0; it < n_iter; ++it) {
    const int64_t key0 = (it * kF32Waves + wave) * kF32Keys;
    const bool live = key0 < nkeys;
    __syncthreads();   // this wave is done reading its previous tile
    if (live) {
      for (int i = lane; i < kF32Keys * DQK; i += kF32Rows) {
        const int64_t key = key0 + i / DQK;
        Ks[i] = key < a.sk ? kg[((static_cast<int64_t>(b) * a.sk + key) * a.hkv + kvh) * DQK + i % DQK] : 0.f;
      }
      for (int i = lane; i < kF32Keys * DV; i += kF32Rows) {
        const int64_t key = key0 + i / DV;
        Vs[i] = key < a.sk ? vg[((static_cast<int64_t>(b) * a.sk + key) * a.hkv + kvh) * DV + i % DV] : 0.f;
      }
    }
    __syncthreads();
    if (!live) continue;
    float s[kF32Keys];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < DQK; ++d) dot = fmaf(qr[d], Ks[j * DQK + d], dot);
      const int64_t key = key0 + j;
      const bool vis = key < a.sk && (!a.causal || a.k_pos0 + key <= qpos);
      s[j] = vis ? dot : kNegInf;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f((m_run - m_use) * a.scale_log2);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      s[j] = exp2f((s[j] - m_use) * a.scale_log2);
      psum += s[j];
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int d = 0; d < DV; ++d) {
      float x = acc[d] * alpha;
#pragma unroll
      for (int j = 0; j < kF32Keys; ++j) x = fmaf(s[j], Vs[j * DV + d], x);
      acc[d] = x;
    }
  }

  // Merge the waves' states into wave 0 through LDS: [wave-1][DV + 2][lane].
  __syncthreads();   // every wave is done with its tiles
  if (wave > 0) {
    float* mine = smem + (wave - 1) * (DV + 2) * kF32Rows + lane;
#pragma unroll
    for (int d = 0; d < DV; ++d) mine[d * kF32Rows] = acc[d];
    mine[DV * kF32Rows] = m_run;
    mine[(DV + 1) * kF32Rows] = l_run;
  }
  __syncthreads();
  if (wave > 0 || !row_valid) return;
  float m_all = m_run;
#pragma unroll
  for (int w = 1; w < kF32Waves; ++w) m_all = fmaxf(m_all, smem[((w - 1) * (DV + 2) + DV) * kF32Rows + lane]);
  const float m_use = m_all == kNegInf ? 0.f : m_all;
  const float f0 = exp2f((m_run - m_use) * a.scale_log2);   // 0 for a wave that saw no key
  l_run *= f0;
#pragma unroll
  for (int d = 0; d < DV; ++d) acc[d] *= f0;
#pragma unroll
  for (int w = 1; w < kF32Waves; ++w) {
    const float* theirs = smem + (w - 1) * (DV + 2) * kF32Rows + lane;
    const float f = exp2f((theirs[DV * kF32Rows] - m_use) * a.scale_log2);
    l_run += theirs[(DV + 1) * kF32Rows] * f;
#pragma unroll
    for (int d = 0; d < DV; ++d) acc[d] += theirs[d * kF32Rows] * f;
  }
  m_run = m_all;

  const bool has = m_run != kNegInf && l_run > 0.f;
  const float inv = has ? 1.f / l_run : 0.f;
  const float lse_blk = has ? m_run * a.scale + logf(l_run) : kNegInf;
  float w_old = 0.f, w_blk = 1.f, lse_out = lse_blk;
  if (a.accumulate) {
    const float lse_old = a.lse[orow];
    const float mx = fmaxf(lse_old, lse_blk);
    if (mx == kNegInf) {
      w_old = 1.f; w_blk = 0.f; lse_out = kNegInf;
    } else {
      const float e_old = expf(lse_old - mx), e_blk = expf(lse_blk - mx);
      w_old = e_old / (e_old + e_blk);
      w_blk = e_blk / (e_old + e_blk);
      lse_out = mx + logf(e_old + e_blk);
    }
  }
  float* op = a.o + orow * DV;
#pragma unroll
  for (int d = 0; d < DV; ++d) {
    const float val = acc[d] * inv * w_blk;
    op[d] = a.accumulate ? fmaf(op[d], w_old, val) : val;
  }
  a.lse[orow] = lse_out;
}

// O = 0, LSE = -inf for every row: a non-accumulating step over a SKIP pair.
__global__ void fill_empty_kernel(float* o, float* lse, int64_t rows, int32_t dv) {
  const int64_t n = rows * dv;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    o[i] = 0.f;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < rows;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    lse[i] = kNegInf;
}

template <typename Kernel>
int32_t launch(Kernel kernel, int rows_per_wg, int threads, StepArgs args, int64_t batch,
               hipStream_t stream) {
  const int64_t n_qtiles = (args.sq + rows_per_wg - 1) / rows_per_wg;
  const int64_t total = n_qtiles * args.hq * batch;
  RA_CHECK(total < (int64_t{1} << 31), CP_EUNSUPPORTED,
           "ring_attn_step: %lld workgroups exceed the grid limit", static_cast<long long>(total));
  args.n_qtiles = static_cast<int32_t>(n_qtiles);
  args.total_wgs = static_cast<int32_t>(total);
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(total)), dim3(threads), 0, stream, args);
  const hipError_t err = hipGetLastError();
  RA_CHECK(err == hipSuccess, CP_EHIP, "ring_attn_step: launch failed: %s", hipGetErrorString(err));
  return CP_OK;
}

// Compute units of the current device (queried once per device).
int device_cus() {
  static std::atomic<int> cached[64];   // 0 = not queried yet; the value never changes
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus == 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// bf16 launch: a grid with fewer than two 4-wave workgroups per CU runs the
// 8-wave key-split variant so every SIMD still holds two waves.
template <int DQK, int DV, bool TAILS>
int32_t launch_bf16_t(JobArgs args, int64_t batch, hipStream_t stream) {
  const int64_t n_qtiles = (args.sq + kBM - 1) / kBM;
  const int64_t total = n_qtiles * (args.paired ? 1 : args.n_jobs) * args.hq * batch;
  RA_CHECK(total < (int64_t{1} << 31), CP_EUNSUPPORTED,
           "ring_attn_step: %lld workgroups exceed the grid limit", static_cast<long long>(total));
  args.n_qtiles = static_cast<int32_t>(n_qtiles);
  args.total_wgs = static_cast<int32_t>(total);
  if (args.n_fwd > 0) args.fwd_per_wg = (args.fwd_end[kMaxFwd - 1] + total - 1) / total;
  const dim3 grid(static_cast<unsigned>(total));
  const int xcd_cus = std::max(1, device_cus() / 8);
  if constexpr (DQK <= 128) {
    if (total < 2 * static_cast<int64_t>(device_cus())) {
      args.serp_w = xcd_cus;   // one 8-wave workgroup per CU
      if (args.paired)
        hipLaunchKernelGGL((attn_step_bf16_kernel<DQK, DV, 2, true, false, 1, TAILS>), grid, dim3(2 * kThreads), 0,
                           stream, args);
      else
        hipLaunchKernelGGL((attn_step_bf16_kernel<DQK, DV, 2, false, false, 1, TAILS>), grid, dim3(2 * kThreads), 0,
                           stream, args);
      const hipError_t err = hipGetLastError();
      RA_CHECK(err == hipSuccess, CP_EHIP, "ring_attn_step: launch failed: %s", hipGetErrorString(err));
      return CP_OK;
    }
  }
  // Large grids: 256-row workgroups while that still leaves two per CU
  // (paired launches: 256-row tile p of job 0, then tile n-1-p of job 1).
  const int64_t n_wide = (args.sq + 2 * kBM - 1) / (2 * kBM);
  const int64_t total_wide = n_wide * (args.paired ? 1 : args.n_jobs) * args.hq * batch;
  RA_CHECK(!args.paired || (DQK <= 128 && total_wide >= 2 * static_cast<int64_t>(device_cus())),
           CP_EUNSUPPORTED, "ring_attn_step: no paired variant for this grid");
  if (total_wide >= 2 * static_cast<int64_t>(device_cus())) {
    args.n_qtiles = static_cast<int32_t>(n_wide);
    args.total_wgs = static_cast<int32_t>(total_wide);
    args.serp_w = xcd_cus;       // one 8-wave workgroup per CU
    if (args.n_fwd > 0) args.fwd_per_wg = (args.fwd_end[kMaxFwd - 1] + total_wide - 1) / total_wide;
    const dim3 wide(static_cast<unsigned>(total_wide));
    bool launched = false;
    if constexpr (DQK <= 128) {
      if (args.paired) {
        hipLaunchKernelGGL((attn_step_bf16_kernel<DQK, DV, 1, true, false, 2, TAILS>), wide, dim3(2 * kThreads), 0,
                           stream, args);
        launched = true;
      }
    }
    if (!launched)
      hipLaunchKernelGGL((attn_step_bf16_kernel<DQK, DV, 1, false, false, 2, TAILS>), wide, dim3(2 * kThreads), 0,
                         stream, args);
  } else {
    args.serp_w = 2 * xcd_cus;   // two 4-wave workgroups per CU
    hipLaunchKernelGGL((attn_step_bf16_kernel<DQK, DV, 1, false, false, 1, TAILS>), grid, dim3(kThreads), 0, stream, args);
  }
  const hipError_t err = hipGetLastError();
  RA_CHECK(err == hipSuccess, CP_EHIP, "ring_attn_step: launch failed: %s", hipGetErrorString(err));
  return CP_OK;
}

// Does some segment end inside a 64-key tile?  Such launches run the
// kernels that base a descriptor at every tile (TAILS).
bool has_tails(const JobArgs& a) {
  for (int j = 0; j < a.n_jobs; ++j)
    for (int sg = 0; sg < a.job[j].n_seg; ++sg)
      if (a.job[j].seg[sg].sk % kBN != 0) return true;
  return false;
}
bool has_tails(const VarlenArgs& a) {
  for (int r = 0; r < a.n_req; ++r)
    if (a.req[r].k_len % kBN != 0) return true;
  return false;
}

template <int DQK, int DV>
int32_t launch_bf16(JobArgs args, int64_t batch, hipStream_t stream) {
  return has_tails(args) ? launch_bf16_t<DQK, DV, true>(args, batch, stream)
                         : launch_bf16_t<DQK, DV, false>(args, batch, stream);
}

// Varlen launch: every (query tile up to the longest request, request,
// head); tiles past a request's end exit at once.
template <int DQK, int DV, bool TAILS>
int32_t launch_bf16_varlen_t(VarlenArgs args, int64_t max_q, hipStream_t stream) {
  const int64_t n_qtiles = (max_q + kBM - 1) / kBM;
  int64_t total = n_qtiles * args.n_req * args.base.hq;
  if (args.base.reverse_q) {   // request-major grid: each request's own tiles
    int64_t acc = 0;
    for (int r = 0; r < args.n_req; ++r) {
      RA_CHECK(acc < (int64_t{1} << 31), CP_EUNSUPPORTED, "ring_attn_step_varlen: grid too large");
      args.wg_start[r] = static_cast<int32_t>(acc);
      acc += (static_cast<int64_t>(args.req[r].q_len) + kBM - 1) / kBM * args.base.hq;
    }
    RA_CHECK(acc < (int64_t{1} << 31), CP_EUNSUPPORTED, "ring_attn_step_varlen: grid too large");
    args.wg_start[args.n_req] = static_cast<int32_t>(acc);
    total = acc;
  }
  RA_CHECK(total < (int64_t{1} << 31), CP_EUNSUPPORTED,
           "ring_attn_step_varlen: %lld workgroups exceed the grid limit", static_cast<long long>(total));
  if (total == 0) return CP_OK;
  args.base.n_qtiles = static_cast<int32_t>(n_qtiles);
  args.base.total_wgs = static_cast<int32_t>(total);
  const dim3 grid(static_cast<unsigned>(total));
  const int xcd_cus = std::max(1, device_cus() / 8);
  if constexpr (DQK <= 128) {
    if (total < 2 * static_cast<int64_t>(device_cus())) {
      args.base.serp_w = xcd_cus;
      hipLaunchKernelGGL((attn_step_bf16_kernel<DQK, DV, 2, false, true, 1, TAILS>), grid, dim3(2 * kThreads), 0,
                         stream, args);
      const hipError_t err = hipGetLastError();
      RA_CHECK(err == hipSuccess, CP_EHIP, "ring_attn_step_varlen: launch failed: %s", hipGetErrorString(err));
      return CP_OK;
    }
  }
  // (128-row tiles here: packed requests end on ragged rows, which 256-row
  // tiles waste -- measured slower for the varlen mix.)
  args.base.serp_w = 2 * xcd_cus;
  hipLaunchKernelGGL((attn_step_bf16_kernel<DQK, DV, 1, false, true, 1, TAILS>), grid, dim3(kThreads), 0, stream, args);
  const hipError_t err = hipGetLastError();
  RA_CHECK(err == hipSuccess, CP_EHIP, "ring_attn_step_varlen: launch failed: %s", hipGetErrorString(err));
  return CP_OK;
}

template <int DQK, int DV>
int32_t launch_bf16_varlen(VarlenArgs args, int64_t max_q, hipStream_t stream) {
  return has_tails(args) ? launch_bf16_varlen_t<DQK, DV, true>(args, max_q, stream)
                         : launch_bf16_varlen_t<DQK, DV, false>(args, max_q, stream);
}

int32_t launch_bf16_any(int32_t d_qk, JobArgs args, int64_t batch, hipStream_t stream) {
  if (d_qk == 64) return launch_bf16<64, 64>(args, batch, stream);
  if (d_qk == 128) return launch_bf16<128, 128>(args, batch, stream);
  return launch_bf16<192, 128>(args, batch, stream);
}

bool head_dims_ok(int32_t d_qk, int32_t d_v) {
  return (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) || (d_qk == 192 && d_v == 128);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// Key tiles of one query tile (of `rows` rows) of a job: the tiles of each
// segment that its last row can see (the kernel's sweep length for that
// workgroup).
int job_tiles(const JobArgs& ja, int j, int64_t qt, int64_t rows = kBM) {
  const QJob& jb = ja.job[j];
  const int64_t q_last = std::min(ja.sq, (qt + 1) * rows) - 1;
  int tiles = 0;
  for (int sg = 0; sg < jb.n_seg; ++sg) {
    int64_t nkeys = jb.seg[sg].sk;
    if (ja.causal) nkeys = std::max<int64_t>(0, std::min(nkeys, jb.q_pos0 + q_last - jb.seg[sg].k_pos0 + 1));
    tiles += static_cast<int>((nkeys + kBN - 1) / kBN);
  }
  return tiles;
}

// Should a two-job launch pair query tile p of job 0 with tile n-1-p of job 1
// in one workgroup?
//  * Grids of at most one workgroup per CU slot: when the pairs' cost beats
//    the plain grid's in a cost model in tiles at a full CU (an 8-wave
//    workgroup, fewer than two per CU, owns its CU; a 4-wave one shares it);
//    the paired grid runs as 8-wave key-split workgroups.
//  * Large grids (256-row workgroups, at least two per CU once paired): when
//    pairing evens out workgroups whose single loads differ by more than 2x
//    (every pair within 1/16 of the largest).  The head-tail diagonal step
//    is such a launch; with equal workgroups the ones an XCD runs together
//    stay in step and keep sharing its L2.
bool pairing_pays(const JobArgs& ja, int64_t batch, int d_qk) {
  if (ja.n_jobs != 2 || d_qk > 128) return false;
  const int64_t cus = device_cus();
  const int64_t nw = (ja.sq + 2 * kBM - 1) / (2 * kBM);
  if (nw * ja.hq * batch >= 2 * cus) {
    int max_single = 0, min_single = 1 << 30, max_pair = 0, min_pair = 1 << 30;
    for (int64_t p = 0; p < nw; ++p) {
      const int a0 = job_tiles(ja, 0, p, 2 * kBM), a1 = job_tiles(ja, 1, p, 2 * kBM);
      const int pr = a0 + job_tiles(ja, 1, nw - 1 - p, 2 * kBM);
      max_single = std::max(max_single, std::max(a0, a1));
      min_single = std::min(min_single, std::min(a0, a1));
      max_pair = std::max(max_pair, pr);
      min_pair = std::min(min_pair, pr);
    }
    return max_single > 2 * min_single && 16 * (max_pair - min_pair) <= max_pair;
  }
  const int64_t n = (ja.sq + kBM - 1) / kBM;
  const int64_t plain_wgs = 2 * n * ja.hq * batch, paired_wgs = n * ja.hq * batch;
  if (plain_wgs > 2 * cus) return false;
  int max_single = 0, max_pair = 0;
  for (int64_t p = 0; p < n; ++p) {
    const int a0 = job_tiles(ja, 0, p), a1 = job_tiles(ja, 1, p), b1 = job_tiles(ja, 1, n - 1 - p);
    max_single = std::max(max_single, std::max(a0, a1));
    max_pair = std::max(max_pair, a0 + b1);
  }
  if (paired_wgs >= 2 * cus) return false;
  const int plain_cost = plain_wgs < 2 * cus ? max_single : 2 * max_single;
  return 20 * max_pair < 17 * plain_cost;
}

// Do the byte ranges [x, x + nx) and [y, y + ny) share a byte?
inline bool overlaps(const void* x, int64_t nx, const void* y, int64_t ny) {
  if (x == nullptr || y == nullptr || nx <= 0 || ny <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(x), b0 = reinterpret_cast<uintptr_t>(y);
  return a0 < b0 + static_cast<uintptr_t>(ny) && b0 < a0 + static_cast<uintptr_t>(nx);
}

}  // namespace
}  // namespace ringattn

using namespace ringattn;

extern "C" int32_t ring_attn_step(const void* q, const void* k, const void* v, int32_t dtype,
                                  int32_t batch, int64_t sq, int64_t sk, int32_t hq, int32_t hkv,
                                  int32_t d_qk, int32_t d_v, int64_t q_pos0, int64_t k_pos0,
                                  int32_t mask, float scale, int32_t accumulate, float* o,
                                  float* lse, int32_t* class_out, void* stream) {
  RA_CHECK(dtype == CP_BF16 || dtype == CP_F32, CP_EDTYPE, "ring_attn_step: dtype=%d", dtype);
  RA_CHECK(batch >= 0 && sq >= 0 && sk >= 0, CP_EINVAL,
           "ring_attn_step: negative size (batch=%d sq=%lld sk=%lld)", batch,
           static_cast<long long>(sq), static_cast<long long>(sk));
  RA_CHECK(hq > 0 && hkv > 0 && hq % hkv == 0, CP_EINVAL,
           "ring_attn_step: hq=%d must be a positive multiple of hkv=%d", hq, hkv);
  RA_CHECK(mask == CP_MASK_NONE || mask == CP_MASK_CAUSAL, CP_EINVAL, "ring_attn_step: mask=%d",
           mask);
  RA_CHECK(accumulate == 0 || accumulate == 1, CP_EINVAL, "ring_attn_step: accumulate=%d",
           accumulate);
  RA_CHECK(scale > 0.f && scale < __builtin_huge_valf(), CP_EINVAL,
           "ring_attn_step: scale must be positive and finite");
  RA_CHECK(head_dims_ok(d_qk, d_v), CP_EUNSUPPORTED, "ring_attn_step: (d_qk, d_v) = (%d, %d) not supported", d_qk,
           d_v);
  const int64_t rows = static_cast<int64_t>(batch) * sq * hq;
  const bool work = rows > 0;
  if (work) {
    RA_CHECK(q && o && lse, CP_EINVAL, "ring_attn_step: NULL q/o/lse");
    RA_CHECK(sk == 0 || (k && v), CP_EINVAL, "ring_attn_step: NULL k/v");
    RA_CHECK(aligned16(q) && aligned16(o) && (sk == 0 || (aligned16(k) && aligned16(v))),
             CP_EINVAL, "ring_attn_step: device pointers must be 16-byte aligned");
  }
  const int32_t cls = classify_pair(q_pos0, sq, k_pos0, sk, mask);
  hipStream_t st = static_cast<hipStream_t>(stream);

  if (work) {
    if (cls == CP_CLASS_SKIP) {
      if (!accumulate) {
        hipLaunchKernelGGL(fill_empty_kernel, dim3(1024), dim3(256), 0, st, o, lse, rows, d_v);
        const hipError_t err = hipGetLastError();
        RA_CHECK(err == hipSuccess, CP_EHIP, "ring_attn_step: launch failed: %s",
                 hipGetErrorString(err));
      }
    } else {
      StepArgs args{};
      args.q = q; args.k = k; args.v = v; args.o = o; args.lse = lse;
      args.sq = sq; args.sk = sk; args.q_pos0 = q_pos0; args.k_pos0 = k_pos0;
      args.hq = hq; args.hkv = hkv; args.group = hq / hkv;
      args.causal = mask == CP_MASK_CAUSAL;
      args.accumulate = accumulate;
      args.reverse_q = cls == CP_CLASS_DIAG;  // heaviest query tiles first
      args.scale = scale;
      args.scale_log2 = scale * kLog2e;
      int32_t rc;
      if (dtype == CP_BF16) {
        JobArgs ja{};
        ja.job[0].q = q; ja.job[0].o = o; ja.job[0].lse = lse;
        ja.job[0].q_pos0 = q_pos0; ja.job[0].accumulate = accumulate; ja.job[0].n_seg = 1;
        ja.job[0].seg[0] = KvSeg{k, v, sk, k_pos0};
        ja.sq = sq; ja.n_jobs = 1; ja.hq = hq; ja.hkv = hkv; ja.group = hq / hkv;
        ja.causal = args.causal; ja.reverse_q = args.reverse_q;
        ja.scale = scale; ja.scale_log2 = args.scale_log2;
        rc = launch_bf16_any(d_qk, ja, batch, st);
      } else {
        if (d_qk == 64)
          rc = launch(attn_step_f32_kernel<64, 64>, kF32Rows, kF32Rows * kF32Waves, args, batch, st);
        else if (d_qk == 128)
          rc = launch(attn_step_f32_kernel<128, 128>, kF32Rows, kF32Rows * kF32Waves, args, batch, st);
        else
          rc = launch(attn_step_f32_kernel<192, 128>, kF32Rows, kF32Rows * kF32Waves, args, batch, st);
      }
      if (rc != CP_OK) return rc;
    }
  }
  if (class_out) *class_out = cls;
  return ok();
}

extern "C" int32_t ring_attn_step_jobs(const cp_attn_job_t* jobs, int32_t n_jobs,
                                       const cp_copy_t* forward, int32_t n_forward, int32_t dtype,
                                       int32_t batch, int64_t sq, int32_t hq, int32_t hkv,
                                       int32_t d_qk, int32_t d_v, int32_t mask, float scale,
                                       void* stream) {
  RA_CHECK(dtype == CP_BF16 || dtype == CP_F32, CP_EDTYPE, "ring_attn_step_jobs: dtype=%d", dtype);
  RA_CHECK(dtype == CP_BF16, CP_EUNSUPPORTED, "ring_attn_step_jobs: only bf16 inputs");
  RA_CHECK(jobs != nullptr && n_jobs >= 1 && n_jobs <= kMaxJobs, CP_EINVAL,
           "ring_attn_step_jobs: n_jobs=%d outside [1, %d]", n_jobs, kMaxJobs);
  RA_CHECK(batch >= 0 && sq >= 0, CP_EINVAL, "ring_attn_step_jobs: negative size");
  RA_CHECK(hq > 0 && hkv > 0 && hq % hkv == 0, CP_EINVAL,
           "ring_attn_step_jobs: hq=%d must be a positive multiple of hkv=%d", hq, hkv);
  RA_CHECK(mask == CP_MASK_NONE || mask == CP_MASK_CAUSAL, CP_EINVAL,
           "ring_attn_step_jobs: mask=%d", mask);
  RA_CHECK(scale > 0.f && scale < __builtin_huge_valf(), CP_EINVAL,
           "ring_attn_step_jobs: scale must be positive and finite");
  RA_CHECK(head_dims_ok(d_qk, d_v), CP_EUNSUPPORTED,
           "ring_attn_step_jobs: (d_qk, d_v) = (%d, %d) not supported", d_qk, d_v);
  const int64_t rows = static_cast<int64_t>(batch) * sq * hq;
  const int64_t o_bytes = rows * d_v * 4, lse_bytes = rows * 4;
  for (int j = 0; j < n_jobs; ++j) {
    const cp_attn_job_t& jb = jobs[j];
    RA_CHECK(jb.accumulate == 0 || jb.accumulate == 1, CP_EINVAL,
             "ring_attn_step_jobs: job %d accumulate=%d", j, jb.accumulate);
    RA_CHECK(jb.n_segments >= 0 && jb.n_segments <= kMaxSegs, CP_EINVAL,
             "ring_attn_step_jobs: job %d has %d segments (at most %d)", j, jb.n_segments, kMaxSegs);
    if (rows == 0) continue;
    RA_CHECK(jb.q && jb.o && jb.lse && aligned16(jb.q) && aligned16(jb.o), CP_EINVAL,
             "ring_attn_step_jobs: job %d needs 16-byte aligned q/o and a lse pointer", j);
    for (int sg = 0; sg < jb.n_segments; ++sg) {
      const cp_kv_segment_t& sgm = jb.segments[sg];
      RA_CHECK(sgm.sk >= 0, CP_EINVAL, "ring_attn_step_jobs: job %d segment %d sk < 0", j, sg);
      RA_CHECK(sgm.sk == 0 || (sgm.k && sgm.v && aligned16(sgm.k) && aligned16(sgm.v)), CP_EINVAL,
               "ring_attn_step_jobs: job %d segment %d needs 16-byte aligned k/v", j, sg);
    }
    // concurrent jobs must not write the same output rows
    for (int i = 0; i < j; ++i)
      RA_CHECK(!overlaps(jobs[i].o, o_bytes, jb.o, o_bytes) &&
                   !overlaps(jobs[i].lse, lse_bytes, jb.lse, lse_bytes),
               CP_EINVAL, "ring_attn_step_jobs: jobs %d and %d write overlapping outputs", i, j);
  }
  // Forwarded ranges: aligned, every destination disjoint from all else the
  // launch reads or writes, and every source disjoint from what it writes.
  RA_CHECK(n_forward >= 0 && n_forward <= kMaxFwd && (n_forward == 0 || forward != nullptr),
           CP_EINVAL, "ring_attn_step_jobs: n_forward=%d outside [0, %d]", n_forward, kMaxFwd);
  for (int f = 0; f < n_forward; ++f) {
    const cp_copy_t& c = forward[f];
    RA_CHECK(c.bytes >= 0 && c.bytes % 16 == 0, CP_EINVAL,
             "ring_attn_step_jobs: forward %d has %lld bytes (a non-negative multiple of 16)", f,
             static_cast<long long>(c.bytes));
    if (c.bytes == 0) continue;
    RA_CHECK(c.dst && c.src && aligned16(c.dst) && aligned16(c.src), CP_EINVAL,
             "ring_attn_step_jobs: forward %d needs 16-byte aligned device pointers", f);
    for (int g = 0; g < n_forward; ++g) {
      RA_CHECK(!overlaps(c.dst, c.bytes, forward[g].src, forward[g].bytes) &&
                   (g == f || !overlaps(c.dst, c.bytes, forward[g].dst, forward[g].bytes)),
               CP_EINVAL, "ring_attn_step_jobs: forward %d overlaps forward %d", f, g);
    }
    if (rows == 0) continue;
    for (int j = 0; j < n_jobs; ++j) {
      const cp_attn_job_t& jb = jobs[j];
      // (a source may not be an output either: the outputs are written
      // while the slices are copied)
      bool hit = overlaps(c.dst, c.bytes, jb.q, rows * d_qk * 2) ||
                 overlaps(c.dst, c.bytes, jb.o, o_bytes) || overlaps(c.dst, c.bytes, jb.lse, lse_bytes) ||
                 overlaps(c.src, c.bytes, jb.o, o_bytes) || overlaps(c.src, c.bytes, jb.lse, lse_bytes);
      for (int sg = 0; sg < jb.n_segments; ++sg) {
        const cp_kv_segment_t& sgm = jb.segments[sg];
        const int64_t kv_rows = static_cast<int64_t>(batch) * sgm.sk * hkv;
        hit = hit || overlaps(c.dst, c.bytes, sgm.k, kv_rows * d_qk * 2) ||
              overlaps(c.dst, c.bytes, sgm.v, kv_rows * d_v * 2);
      }
      RA_CHECK(!hit, CP_EINVAL, "ring_attn_step_jobs: forward %d overlaps a buffer of job %d", f, j);
    }
  }
  // Without attention work the forwarded ranges still move, as a plain copy.
  const auto forward_alone = [&]() -> int32_t {
    if (n_forward == 0) return ok();
    void* dsts[kMaxFwd];
    const void* srcs[kMaxFwd];
    int64_t bytes[kMaxFwd];
    for (int f = 0; f < n_forward; ++f) {
      dsts[f] = forward[f].dst; srcs[f] = forward[f].src; bytes[f] = forward[f].bytes;
    }
    return ring_stage_copy(dsts, srcs, bytes, n_forward, stream);
  };
  if (rows == 0) return forward_alone();

  JobArgs ja{};
  bool any_diag = false, any_work = false;
  for (int j = 0; j < n_jobs; ++j) {
    const cp_attn_job_t& jb = jobs[j];
    QJob& qj = ja.job[j];
    qj.q = jb.q; qj.o = jb.o; qj.lse = jb.lse; qj.q_pos0 = jb.q_pos0;
    qj.accumulate = jb.accumulate;
    int n = 0;
    for (int sg = 0; sg < jb.n_segments; ++sg) {   // SKIP segments add nothing
      const cp_kv_segment_t& sgm = jb.segments[sg];
      const int32_t cls = classify_pair(jb.q_pos0, sq, sgm.k_pos0, sgm.sk, mask);
      if (cls == CP_CLASS_SKIP) continue;
      any_diag |= cls == CP_CLASS_DIAG;
      qj.seg[n++] = KvSeg{sgm.k, sgm.v, sgm.sk, sgm.k_pos0};
    }
    qj.n_seg = n;
    any_work |= n > 0 || !jb.accumulate;   // a job without keys still writes its empty partial
  }
  if (!any_work) return forward_alone();
  int64_t units = 0;
  for (int f = 0; f < kMaxFwd; ++f) {
    if (f < n_forward) {
      ja.fwd[f] = FwdCopy{static_cast<u32x4*>(forward[f].dst), static_cast<const u32x4*>(forward[f].src)};
      units += forward[f].bytes / 16;
    }
    ja.fwd_end[f] = units;
  }
  ja.n_fwd = units > 0 ? n_forward : 0;
  ja.sq = sq; ja.n_jobs = n_jobs; ja.hq = hq; ja.hkv = hkv; ja.group = hq / hkv;
  ja.causal = mask == CP_MASK_CAUSAL;
  ja.reverse_q = any_diag;   // heaviest query tiles first
  ja.paired = pairing_pays(ja, batch, d_qk) ? 1 : 0;
  ja.scale = scale; ja.scale_log2 = scale * kLog2e;
  const int32_t rc = launch_bf16_any(d_qk, ja, batch, static_cast<hipStream_t>(stream));
  return rc == CP_OK ? ok() : rc;
}

extern "C" int32_t ring_attn_step_varlen(const void* q, const void* k, const void* v, int32_t dtype,
                                         int32_t n_req, const int64_t* cu_seqlens_q,
                                         const int64_t* cu_seqlens_k, const int64_t* q_pos0,
                                         const int64_t* k_pos0, int32_t hq, int32_t hkv, int32_t d_qk,
                                         int32_t d_v, int32_t mask, float scale, int32_t accumulate,
                                         float* o, float* lse, void* stream) {
  using namespace ringattn;
  RA_CHECK(dtype == CP_BF16 || dtype == CP_F32, CP_EDTYPE, "ring_attn_step_varlen: dtype=%d", dtype);
  RA_CHECK(dtype == CP_BF16, CP_EUNSUPPORTED, "ring_attn_step_varlen: only bf16 inputs");
  RA_CHECK(n_req >= 0, CP_EINVAL, "ring_attn_step_varlen: n_req=%d < 0", n_req);
  RA_CHECK(hq > 0 && hkv > 0 && hq % hkv == 0, CP_EINVAL,
           "ring_attn_step_varlen: hq=%d must be a positive multiple of hkv=%d", hq, hkv);
  RA_CHECK(mask == CP_MASK_NONE || mask == CP_MASK_CAUSAL, CP_EINVAL, "ring_attn_step_varlen: mask=%d", mask);
  RA_CHECK(scale > 0.f && scale < __builtin_huge_valf(), CP_EINVAL,
           "ring_attn_step_varlen: scale must be positive and finite");
  RA_CHECK(accumulate == 0 || accumulate == 1, CP_EINVAL, "ring_attn_step_varlen: accumulate=%d", accumulate);
  RA_CHECK(head_dims_ok(d_qk, d_v), CP_EUNSUPPORTED,
           "ring_attn_step_varlen: (d_qk, d_v) = (%d, %d) not supported", d_qk, d_v);
  if (n_req == 0) return ok();
  RA_CHECK(cu_seqlens_q && cu_seqlens_k && q_pos0 && k_pos0, CP_EINVAL,
           "ring_attn_step_varlen: NULL host array");
  int64_t max_q = 0;
  for (int32_t r = 0; r < n_req; ++r) {
    const int64_t lq = cu_seqlens_q[r + 1] - cu_seqlens_q[r], lk = cu_seqlens_k[r + 1] - cu_seqlens_k[r];
    RA_CHECK(cu_seqlens_q[r] >= 0 && cu_seqlens_k[r] >= 0 && lq >= 0 && lk >= 0, CP_EINVAL,
             "ring_attn_step_varlen: cu_seqlens must start >= 0 and not decrease (request %d)", r);
    max_q = std::max(max_q, lq);
  }
  const int64_t total_q = cu_seqlens_q[n_req], total_k = cu_seqlens_k[n_req];
  RA_CHECK(total_q < (int64_t{1} << 31) && total_k < (int64_t{1} << 31), CP_EUNSUPPORTED,
           "ring_attn_step_varlen: packed lengths must stay below 2^31 tokens");
  if (total_q == 0) return ok();
  RA_CHECK(q && o && lse && aligned16(q) && aligned16(o) && (total_k == 0 || (k && v && aligned16(k) && aligned16(v))),
           CP_EINVAL, "ring_attn_step_varlen: NULL or misaligned device pointer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  // Requests go kMaxReq per launch.
  for (int32_t r0 = 0; r0 < n_req; r0 += kMaxReq) {
    VarlenArgs va{};
    JobArgs& ja = va.base;
    ja.job[0].q = q; ja.job[0].o = o; ja.job[0].lse = lse; ja.job[0].accumulate = accumulate;
    ja.job[0].n_seg = 1;
    ja.job[0].seg[0] = KvSeg{k, v, 0, 0};
    ja.n_jobs = 1; ja.sq = 0; ja.hq = hq; ja.hkv = hkv; ja.group = hq / hkv;
    ja.causal = mask == CP_MASK_CAUSAL;
    ja.reverse_q = ja.causal;   // the longest query tiles of causal requests first
    ja.scale = scale; ja.scale_log2 = scale * kLog2e;
    int64_t group_max_q = 0;
    const int32_t n = std::min(kMaxReq, n_req - r0);
    // causal launches take the longest requests first
    int32_t order[kMaxReq];
    for (int32_t i = 0; i < n; ++i) order[i] = r0 + i;
    if (ja.causal)
      std::stable_sort(order, order + n, [&](int32_t x, int32_t y) {
        return cu_seqlens_q[x + 1] - cu_seqlens_q[x] > cu_seqlens_q[y + 1] - cu_seqlens_q[y];
      });
    for (int32_t i = 0; i < n; ++i) {
      const int32_t r = order[i];
      ReqDesc& d = va.req[i];
      d.q_start = static_cast<int32_t>(cu_seqlens_q[r]);
      d.q_len = static_cast<int32_t>(cu_seqlens_q[r + 1] - cu_seqlens_q[r]);
      d.k_start = static_cast<int32_t>(cu_seqlens_k[r]);
      d.k_len = static_cast<int32_t>(cu_seqlens_k[r + 1] - cu_seqlens_k[r]);
      d.q_pos0 = q_pos0[r];
      d.k_pos0 = k_pos0[r];
      group_max_q = std::max<int64_t>(group_max_q, d.q_len);
    }
    va.n_req = n;
    int32_t rc;
    if (d_qk == 64) rc = launch_bf16_varlen<64, 64>(va, group_max_q, st);
    else if (d_qk == 128) rc = launch_bf16_varlen<128, 128>(va, group_max_q, st);
    else rc = launch_bf16_varlen<192, 128>(va, group_max_q, st);
    if (rc != CP_OK) return rc;
  }
  return ok();
}
