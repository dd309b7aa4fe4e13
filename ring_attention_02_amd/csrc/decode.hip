// Grouped-query decode over a KV cache sharded along the sequence.
//
// vLLM-Ascend developer guide "Context Parallel (CP)", sections "Decode
// context parallel (DCP)" and the PCP decode paragraph: every device keeps a
// slice of each request's KV cache (placed by the interleaved block-table
// rule), attends the new query to its slice, and the partial outputs with
// their LSEs are combined.  Here all shards live on one GPU; this kernel
// produces the per-shard partials, lse_merge combines them.
//
// gfx950 design: one workgroup (4 waves) per (shard, request, kv head, key
// split).  The hq/hkv query heads of a kv head are packed into the 16
// columns of v_mfma_f32_16x16x32_bf16, so K and V are streamed once per kv
// head.  K and V are both read from HBM in whole 128-byte lines (16 lanes per
// 256-byte row piece of a kv head), non-temporally, and go through per-wave
// LDS slots: K is read back as the A operand with ds_read_b128, V transposed
// with ds_read_b64_tr_b16.  (Loading K straight in the A operand's layout
// reads half lines per instruction: a probe of this access pattern measured
// 5.9 TB/s that way against 6.6 TB/s in whole non-temporal lines.)  Waves
// interleave on 32-key tiles, prefetch one tile ahead, and their softmax
// states are merged through LDS at the end; KV splits (only when there are
// too few work items to fill the GPU) are merged by the LSE merge kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels_common.h"
#include "status.h"

// Key-split workspace of split_kv_decode_noalloc: a static device array
// instead of caller memory.  Every supported shape fits (d_v = 128, at most
// 16 query heads per kv head, splits only below 2,048 work items: at most
// 4,094 x 16 rows x 129 floats = 33.8 MB).  Each GPU the library runs on
// holds its own copy until the process ends.
static constexpr size_t kScratchBytes = size_t{40} << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace ringattn {

int32_t launch_lse_merge(const float* o_parts, const float* lse_parts, int32_t n_parts,
                         int64_t rows, int32_t d_v, void* o_out, int32_t out_dtype,
                         float* lse_out, hipStream_t stream);

namespace {

constexpr int kD = 128;            // head dim (q/k and v)
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;          // keys per wave per round
constexpr int kRound = kTile * kWaves;
constexpr int kVPitch = kD + 32;   // bf16 per V row in LDS (+64 B: conflict-free transposed reads)
constexpr int kKPitch = kD + 8;    // bf16 per K row in LDS (+16 B: conflict-free b128 reads)
constexpr int kMaxGroup = 16;      // query heads per kv head that fit the MFMA columns
constexpr int kTargetWgs = 2048;   // enough workgroups to fill 256 CUs several times

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;   // contiguous shards [n_shards, B, t_shard, Hkv, 128], or block pools
  const uint16_t* v;   // [n_shards, num_blocks, block_size, Hkv, 128] when paged
  const int64_t* shard_lens;
  const int32_t* block_table;   // paged: [n_shards, B, max_blocks] physical block ids
  int32_t block_size, max_blocks, num_blocks;
  float* o;    // [rows_out, 128] destination (o_parts, or split-major workspace)
  float* lse;  // [rows_out]
  int64_t t_shard;
  int32_t n_shards, batch, hq, hkv, group, n_splits;
  float scale, scale_log2;
};

// PAGED: token i of (shard, request) lives in block block_table[i / block_size]
// of the shard's pool, at row i % block_size ([CP] "Block table": the
// table maps a request's logical blocks to physical blocks).  block_size is a
// multiple of the 32-key wave tile, so one table entry serves a whole tile.
template <bool PAGED>
__global__ void __launch_bounds__(kThreads, 2) decode_bf16_kernel(DecodeArgs a) {
  // Per-wave V tile during the sweep; reused for the cross-wave merge.
  __shared__ __attribute__((aligned(16))) uint16_t smem[kWaves * kTile * kVPitch];
  // Per-wave K tile during the sweep.
  __shared__ __attribute__((aligned(16))) uint16_t ksmem[kWaves * kTile * kKPitch];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n16 = lane & 15;  // key row (A) / query column (B, C)
  const int g = lane >> 4;    // 16-lane group

  const int items = a.n_shards * a.batch * a.hkv * a.n_splits;
  const int logical = xcd_contiguous_id(blockIdx.x, items);
  const int sp = logical % a.n_splits;
  int rest = logical / a.n_splits;
  const int kvh = rest % a.hkv;
  rest /= a.hkv;
  const int b = rest % a.batch;
  const int s = rest / a.batch;

  int64_t len = a.shard_lens ? a.shard_lens[static_cast<int64_t>(s) * a.batch + b] : a.t_shard;
  len = len < 0 ? 0 : (len > a.t_shard ? a.t_shard : len);
  const int64_t per_split = (len + a.n_splits - 1) / a.n_splits;
  const int64_t chunk = (per_split + kRound - 1) / kRound * kRound;
  const int64_t k_begin = min(len, static_cast<int64_t>(sp) * chunk);
  const int64_t k_end = min(len, k_begin + chunk);
  const int rounds = static_cast<int>((k_end - k_begin + kRound - 1) / kRound);

  // Q^T operand: lane (column n16 = query head in group, g) holds
  // Q[head][32c + 8g .. +7] for MFMA step c.
  bf16x8 qf[4];
  {
    const int head = kvh * a.group + n16;
    const bool valid = n16 < a.group;
    const uint16_t* qp = a.q + (static_cast<int64_t>(b) * a.hq + head) * kD;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (valid) raw = *reinterpret_cast<const u32x4*>(qp + 32 * c + 8 * g);
      qf[c] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  const int64_t row_stride = static_cast<int64_t>(a.hkv) * kD;  // elements between keys
  uint16_t* vslot = smem + wave * kTile * kVPitch;
  uint16_t* kslot = ksmem + wave * kTile * kKPitch;

  // The wave's 32-key tile of round r: element offset of its first key (from
  // the K/V base) and how many of its keys exist (0 for a tile past the end
  // or, paged, in a block whose table entry is outside the pool).
  struct Tile {
    int64_t off;
    int valid;
  };
  // Paged: the table entry of a round's tile is fetched one round ahead
  // with a vector load (it completes in order with the K/V loads issued
  // after it, so using it never waits on anything the round needs).
  const int32_t* trow = PAGED ? a.block_table + (static_cast<int64_t>(s) * a.batch + b) * a.max_blocks
                              : nullptr;
  const auto trsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(trow), static_cast<short>(0),
                                                       PAGED ? a.max_blocks * 4 : 0, 0x00020000);
  auto fetch_entry = [&](int r) -> int32_t {
    const int64_t t0 = k_begin + static_cast<int64_t>(r) * kRound + wave * kTile;
    if (!PAGED || t0 >= k_end) return -1;
    return __builtin_amdgcn_raw_buffer_load_b32(trsrc, static_cast<int>(t0 / a.block_size) * 4, 0, 0);
  };
  auto tile_of = [&](int r, int32_t entry) -> Tile {
    const int64_t t0 = k_begin + static_cast<int64_t>(r) * kRound + wave * kTile;
    Tile t{0, 0};
    if (t0 >= k_end) return t;
    t.valid = static_cast<int>(min(static_cast<int64_t>(kTile), k_end - t0));
    if constexpr (PAGED) {
      const int32_t blk = __builtin_amdgcn_readfirstlane(entry);
      if (blk < 0 || blk >= a.num_blocks) {
        t.valid = 0;
        return t;
      }
      t.off = ((static_cast<int64_t>(s) * a.num_blocks + blk) * a.block_size + t0 % a.block_size) * row_stride;
    } else {
      t.off = ((static_cast<int64_t>(s) * a.batch + b) * a.t_shard + t0) * row_stride;
    }
    t.off += static_cast<int64_t>(kvh) * kD;
    return t;
  };

  // K and V alike: lane loads rows 4i + g of the tile, 16 bytes at column
  // 8 * (lane % 16): reg[i] = X[tile + 4i + lane/16][8*(lane%16) .. +7], so
  // each instruction reads four whole 256-byte row pieces.  Rows past the
  // tile's valid keys read as zero.
  u32x4 knext[8], vnext[8];
  auto load_rows = [&](const uint16_t* base, const Tile& t, u32x4* dst) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = 4 * i + g;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (key < t.valid)
        raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + t.off + key * row_stride + 8 * n16));
      dst[i] = raw;
    }
  };
  auto load_k = [&](const Tile& t) { load_rows(a.k, t, knext); };
  auto load_v = [&](const Tile& t) { load_rows(a.v, t, vnext); };

  f32x4 oacc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  int32_t entry_cur = fetch_entry(0), entry_next = fetch_entry(1);
  int32_t entry_now = entry_cur;     // entry of the round being computed
  if (rounds > 0) {
    const Tile t = tile_of(0, entry_cur);
    load_k(t);
    load_v(t);
  }
  for (int r = 0; r < rounds; ++r) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      *reinterpret_cast<u32x4*>(&vslot[(4 * i + g) * kVPitch + 8 * n16]) = vnext[i];
      *reinterpret_cast<u32x4*>(&kslot[(4 * i + g) * kKPitch + 8 * n16]) = knext[i];
    }
    __syncthreads();
    // A operand of step c for 16-key block kb: lane (key n16, g) holds
    // K[kb*16 + n16][32c + 8g .. +7].
    u32x4 kcur[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        kcur[kb * 4 + c] = *reinterpret_cast<const u32x4*>(&kslot[(kb * 16 + n16) * kKPitch + 32 * c + 8 * g]);
    if (r + 1 < rounds) {
      const Tile t = tile_of(r + 1, entry_next);
      load_k(t);
      load_v(t);
    }
    const int valid = tile_of(r, entry_now).valid;
    entry_now = entry_next;
    if (r + 2 < rounds) entry_next = fetch_entry(r + 2);
    if (valid > 0) {
      // S^T = K Q^T for two 16-key blocks; acc[kb][j] = score of key
      // t0 + kb*16 + 4g + j for query column n16.
      f32x4 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < 4; ++c)
          sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kcur[kb * 4 + c]),
                                                           qf[c], sc[kb], 0, 0, 0);
      }
      if (valid < kTile) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (kb * 16 + 4 * g + j >= valid) sc[kb][j] = kNegInf;
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sc[kb][j]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float neg_mc = -m_use * a.scale_log2;
      const float alpha = fast_exp2(m_run * a.scale_log2 + neg_mc);
      m_run = m_new;
      float psum = 0.f;
      bf16x8 pb;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = fast_exp2(fmaf(sc[kb][j], a.scale_log2, neg_mc));
          psum += p;
          pb[kb * 4 + j] = static_cast<__bf16>(p);
        }
      l_run = fmaf(l_run, alpha, psum);
      // O^T += V^T P^T: eight 16-wide d_v blocks, contraction over the 32 keys
      // in the order (4g + e) for e < 4, (16 + 4g + e - 4) for e >= 4.
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint16_t* pa = &vslot[(4 * g + (n16 >> 2)) * kVPitch + d * 16 + 4 * (n16 & 3)];
        const s16x4 lo = lds_read_tr16(pa);
        const s16x4 hi = lds_read_tr16(pa + 16 * kVPitch);
        oacc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(join_bf16x4(lo, hi), pb, oacc[d] * alpha,
                                                          0, 0, 0);
      }
    }
  }

  // ---- merge the four waves' states through LDS
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();  // every wave is done with its V slot
  float* om = reinterpret_cast<float*>(smem);           // [wave][16 q][128 dv]
  float* mm = om + kWaves * 16 * kD;                     // [wave][16]
  float* ll = mm + kWaves * 16;                          // [wave][16]
#pragma unroll
  for (int d = 0; d < 8; ++d)
    *reinterpret_cast<f32x4*>(&om[(wave * 16 + n16) * kD + d * 16 + 4 * g]) = oacc[d];
  if (g == 0) {
    mm[wave * 16 + n16] = m_run;
    ll[wave * 16 + n16] = l_run;
  }
  __syncthreads();
  const int qh = tid >> 4;        // query head in the group
  const int dv0 = (tid & 15) * 8;  // 8 consecutive d_v values
  if (qh >= a.group) return;
  float mw[kWaves];
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    mw[w] = mm[w * 16 + qh];
    M = fmaxf(M, mw[w]);
  }
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != kNegInf) {
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = fast_exp2((mw[w] - M) * a.scale_log2);
      L += e * ll[w * 16 + qh];
      acc0 += *reinterpret_cast<const f32x4*>(&om[(w * 16 + qh) * kD + dv0]) * e;
      acc1 += *reinterpret_cast<const f32x4*>(&om[(w * 16 + qh) * kD + dv0 + 4]) * e;
    }
  }
  const bool has = M != kNegInf && L > 0.f;
  const float inv = has ? 1.f / L : 0.f;
  const int64_t rows_out = static_cast<int64_t>(a.n_shards) * a.batch * a.hq;
  const int64_t row = (static_cast<int64_t>(s) * a.batch + b) * a.hq + kvh * a.group + qh;
  const int64_t orow = static_cast<int64_t>(sp) * rows_out + row;
  *reinterpret_cast<f32x4*>(a.o + orow * kD + dv0) = acc0 * inv;
  *reinterpret_cast<f32x4*>(a.o + orow * kD + dv0 + 4) = acc1 * inv;
  if ((tid & 15) == 0) a.lse[orow] = has ? M * a.scale + fast_log2(L) * kLn2 : kNegInf;
}

int32_t choose_splits(int32_t n_shards, int32_t batch, int32_t hkv, int64_t t_shard) {
  const int64_t items = static_cast<int64_t>(n_shards) * batch * hkv;
  if (items <= 0 || items >= kTargetWgs) return 1;
  int64_t splits = (kTargetWgs + items - 1) / items;
  const int64_t max_by_len = t_shard / (2 * kRound);  // keep at least two rounds per split
  if (splits > max_by_len) splits = max_by_len;
  return static_cast<int32_t>(splits < 1 ? 1 : splits);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace
}  // namespace ringattn

using namespace ringattn;

extern "C" size_t split_kv_decode_workspace(int32_t n_shards, int32_t batch, int32_t hq,
                                            int32_t hkv, int32_t d_v, int64_t t_shard) {
  if (n_shards <= 0 || batch <= 0 || hq <= 0 || hkv <= 0 || d_v <= 0 || t_shard < 0) return 0;
  const int32_t splits = choose_splits(n_shards, batch, hkv, t_shard);
  if (splits <= 1) return 0;
  const size_t rows = static_cast<size_t>(n_shards) * batch * hq;
  return static_cast<size_t>(splits) * rows * (static_cast<size_t>(d_v) + 1) * sizeof(float);
}

namespace ringattn {
namespace {

// Checks shared by both decode entry points, then the launch (and the merge
// of the key splits).  t_shard is the longest local context of a (shard,
// request): the contiguous shard length, or max_blocks * block_size.
int32_t run_decode(const char* who, bool paged, DecodeArgs args, int32_t dtype, int32_t d_qk,
                   int32_t d_v, float* o_parts, float* lse_parts, void* workspace, size_t ws_bytes,
                   hipStream_t st) {
  RA_CHECK(dtype == CP_BF16 || dtype == CP_F32, CP_EDTYPE, "%s: dtype=%d", who, dtype);
  RA_CHECK(dtype == CP_BF16, CP_EUNSUPPORTED, "%s: only bf16 inputs are supported", who);
  RA_CHECK(args.n_shards > 0 && args.batch >= 0 && args.t_shard >= 0, CP_EINVAL,
           "%s: bad sizes (n_shards=%d batch=%d tokens=%lld)", who, args.n_shards, args.batch,
           static_cast<long long>(args.t_shard));
  RA_CHECK(args.hq > 0 && args.hkv > 0 && args.hq % args.hkv == 0, CP_EINVAL,
           "%s: hq=%d must be a positive multiple of hkv=%d", who, args.hq, args.hkv);
  RA_CHECK(d_qk == kD && d_v == kD, CP_EUNSUPPORTED,
           "%s: only d_qk = d_v = 128 is supported (got %d, %d)", who, d_qk, d_v);
  RA_CHECK(args.hq / args.hkv <= kMaxGroup, CP_EUNSUPPORTED,
           "%s: hq/hkv=%d exceeds %d query heads per kv head", who, args.hq / args.hkv, kMaxGroup);
  RA_CHECK(args.scale > 0.f && args.scale < __builtin_huge_valf(), CP_EINVAL,
           "%s: scale must be positive and finite", who);
  if (args.batch == 0) return ok();
  RA_CHECK(args.q && o_parts && lse_parts && (args.t_shard == 0 || (args.k && args.v)), CP_EINVAL,
           "%s: NULL pointer", who);
  RA_CHECK(aligned16(args.q) && aligned16(o_parts) &&
               (args.t_shard == 0 || (aligned16(args.k) && aligned16(args.v))),
           CP_EINVAL, "%s: device pointers must be 16-byte aligned", who);
  const int32_t splits = choose_splits(args.n_shards, args.batch, args.hkv, args.t_shard);
  const size_t need =
      split_kv_decode_workspace(args.n_shards, args.batch, args.hq, args.hkv, d_v, args.t_shard);
  RA_CHECK(ws_bytes >= need && (need == 0 || (workspace && aligned16(workspace))), CP_EINVAL,
           "%s: workspace of %zu bytes (16-byte aligned) needed, got %zu", who, need, ws_bytes);
  const int64_t items = static_cast<int64_t>(args.n_shards) * args.batch * args.hkv * splits;
  RA_CHECK(items < (int64_t{1} << 31), CP_EUNSUPPORTED, "%s: too many work items", who);

  const int64_t rows = static_cast<int64_t>(args.n_shards) * args.batch * args.hq;
  args.group = args.hq / args.hkv;
  args.n_splits = splits;
  args.scale_log2 = args.scale * kLog2e;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_lse = ws_o ? ws_o + static_cast<size_t>(splits) * rows * kD : nullptr;
  args.o = splits > 1 ? ws_o : o_parts;
  args.lse = splits > 1 ? ws_lse : lse_parts;
  if (paged)
    hipLaunchKernelGGL(decode_bf16_kernel<true>, dim3(static_cast<unsigned>(items)), dim3(kThreads), 0,
                       st, args);
  else
    hipLaunchKernelGGL(decode_bf16_kernel<false>, dim3(static_cast<unsigned>(items)), dim3(kThreads), 0,
                       st, args);
  hipError_t err = hipGetLastError();
  RA_CHECK(err == hipSuccess, CP_EHIP, "%s: launch failed: %s", who, hipGetErrorString(err));
  if (splits > 1) {
    const int32_t rc = launch_lse_merge(ws_o, ws_lse, splits, rows, kD, o_parts, CP_F32, lse_parts, st);
    if (rc != CP_OK) return rc;
  }
  return ok();
}

}  // namespace
}  // namespace ringattn

extern "C" int32_t split_kv_decode(const void* q, const void* k_shards, const void* v_shards,
                                   int32_t dtype, int32_t n_shards, int32_t batch, int64_t t_shard,
                                   const int64_t* shard_lens, int32_t hq, int32_t hkv, int32_t d_qk,
                                   int32_t d_v, float scale, float* o_parts, float* lse_parts,
                                   void* workspace, size_t ws_bytes, void* stream) {
  DecodeArgs args{};
  args.q = static_cast<const uint16_t*>(q);
  args.k = static_cast<const uint16_t*>(k_shards);
  args.v = static_cast<const uint16_t*>(v_shards);
  args.shard_lens = shard_lens;
  args.t_shard = t_shard;
  args.n_shards = n_shards; args.batch = batch; args.hq = hq; args.hkv = hkv;
  args.scale = scale;
  return run_decode("split_kv_decode", false, args, dtype, d_qk, d_v, o_parts, lse_parts, workspace,
                    ws_bytes, static_cast<hipStream_t>(stream));
}

namespace {
// Device address of this GPU's scratch array, looked up once per device with
// that device current (the array's name in host code is only a stand-in).
int32_t scratch_address(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  RA_CHECK(err == hipSuccess && dev >= 0 && dev < kMaxDevices, CP_EHIP,
           "split_kv_decode_noalloc: no current device (%s)", hipGetErrorString(err));
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    RA_CHECK(err == hipSuccess && p != nullptr, CP_EHIP,
             "split_kv_decode_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
             hipGetErrorString(err));
    addr[dev] = p;
  }
  *out = addr[dev];
  return CP_OK;
}
}  // namespace

extern "C" int32_t split_kv_decode_noalloc(const void* q, const void* k_shards, const void* v_shards,
                                           int32_t dtype, int32_t n_shards, int32_t batch,
                                           int64_t t_shard, const int64_t* shard_lens, int32_t hq,
                                           int32_t hkv, int32_t d_qk, int32_t d_v, float scale,
                                           float* o_parts, float* lse_parts, void* stream) {
  // Every split's partial is written in full before the merge reads it, so
  // nothing left in the array by an earlier call is ever read.
  const size_t need = split_kv_decode_workspace(n_shards, batch, hq, hkv, d_v, t_shard);
  RA_CHECK(need <= kScratchBytes, CP_EUNSUPPORTED,
           "split_kv_decode_noalloc: %zu bytes of key-split scratch needed, the static array holds %zu",
           need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const int32_t rc = scratch_address(&ws);
    if (rc != CP_OK) return rc;
  }
  return split_kv_decode(q, k_shards, v_shards, dtype, n_shards, batch, t_shard, shard_lens, hq, hkv,
                         d_qk, d_v, scale, o_parts, lse_parts, ws, need > 0 ? kScratchBytes : 0, stream);
}

extern "C" int32_t split_kv_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                                         int32_t dtype, int32_t n_shards, int32_t batch,
                                         int32_t num_blocks, int32_t block_size,
                                         const int32_t* block_tables, int32_t max_blocks,
                                         const int64_t* shard_lens, int32_t hq, int32_t hkv,
                                         int32_t d_qk, int32_t d_v, float scale, float* o_parts,
                                         float* lse_parts, void* workspace, size_t ws_bytes,
                                         void* stream) {
  RA_CHECK(block_size > 0 && block_size % kTile == 0, CP_EINVAL,
           "split_kv_decode_paged: block_size=%d must be a positive multiple of %d", block_size, kTile);
  RA_CHECK(num_blocks > 0 && max_blocks >= 0, CP_EINVAL,
           "split_kv_decode_paged: num_blocks=%d must be positive, max_blocks=%d non-negative",
           num_blocks, max_blocks);
  RA_CHECK(batch == 0 || max_blocks == 0 || (block_tables && shard_lens), CP_EINVAL,
           "split_kv_decode_paged: block_tables and shard_lens are required");
  DecodeArgs args{};
  args.q = static_cast<const uint16_t*>(q);
  args.k = static_cast<const uint16_t*>(k_pool);
  args.v = static_cast<const uint16_t*>(v_pool);
  args.shard_lens = shard_lens;
  args.block_table = block_tables;
  args.block_size = block_size; args.max_blocks = max_blocks; args.num_blocks = num_blocks;
  args.t_shard = static_cast<int64_t>(max_blocks) * block_size;
  args.n_shards = n_shards; args.batch = batch; args.hq = hq; args.hkv = hkv;
  args.scale = scale;
  return run_decode("split_kv_decode_paged", true, args, dtype, d_qk, d_v, o_parts, lse_parts,
                    workspace, ws_bytes, static_cast<hipStream_t>(stream));
}
