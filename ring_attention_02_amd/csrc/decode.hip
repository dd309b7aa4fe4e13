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
// head.  K goes from HBM straight into the A operand registers (each lane's
// 64 contiguous bytes are exactly its operand), V goes through a per-wave LDS
// slot and is read transposed with ds_read_b64_tr_b16.  Waves interleave on
// 32-key tiles, prefetch one tile ahead, and their softmax states are merged
// through LDS at the end; KV splits (only when there are too few work items
// to fill the GPU) are merged by the LSE merge kernel.
#include <hip/hip_runtime.h>

#include "kernels_common.h"
#include "status.h"

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
constexpr int kMaxGroup = 16;      // query heads per kv head that fit the MFMA columns
constexpr int kTargetWgs = 2048;   // enough workgroups to fill 256 CUs several times

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int64_t* shard_lens;
  float* o;    // [rows_out, 128] destination (o_parts, or split-major workspace)
  float* lse;  // [rows_out]
  int64_t t_shard;
  int32_t n_shards, batch, hq, hkv, group, n_splits;
  float scale, scale_log2;
};

__global__ void __launch_bounds__(kThreads, 2) decode_bf16_kernel(DecodeArgs a) {
  // Per-wave V tile during the sweep; reused for the cross-wave merge.
  __shared__ __attribute__((aligned(16))) uint16_t smem[kWaves * kTile * kVPitch];

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
  const int64_t shard_base =
      ((static_cast<int64_t>(s) * a.batch + b) * a.t_shard) * row_stride + static_cast<int64_t>(kvh) * kD;
  const uint16_t* kbase = a.k + shard_base;
  const uint16_t* vbase = a.v + shard_base;
  uint16_t* vslot = smem + wave * kTile * kVPitch;

  // K: lane (key n16 of block kb, g) loads 64 contiguous bytes per block:
  // kreg[kb*4 + c] = K[key][32c + 8g .. +7]  (the A operand of step c).
  // V: lane loads rows 4i + g/... : vreg[i] = V[tile + 4i + lane/16][8*(lane%16) .. +7].
  u32x4 kcur[8], knext[8], vnext[8];
  auto load_k = [&](int r, u32x4* dst) {
    const int64_t t0 = k_begin + static_cast<int64_t>(r) * kRound + wave * kTile;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int64_t key = t0 + kb * 16 + n16;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (key < k_end) raw = *reinterpret_cast<const u32x4*>(kbase + key * row_stride + 32 * c + 8 * g);
        dst[kb * 4 + c] = raw;
      }
    }
  };
  auto load_v = [&](int r) {
    const int64_t t0 = k_begin + static_cast<int64_t>(r) * kRound + wave * kTile;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t key = t0 + 4 * i + g;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (key < k_end) raw = *reinterpret_cast<const u32x4*>(vbase + key * row_stride + 8 * n16);
      vnext[i] = raw;
    }
  };

  f32x4 oacc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) oacc[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  if (rounds > 0) {
    load_k(0, kcur);
    load_v(0);
  }
  for (int r = 0; r < rounds; ++r) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(&vslot[(4 * i + g) * kVPitch + 8 * n16]) = vnext[i];
    __syncthreads();
    if (r + 1 < rounds) {
      load_k(r + 1, knext);
      load_v(r + 1);
    }
    const int64_t t0 = k_begin + static_cast<int64_t>(r) * kRound + wave * kTile;
    if (t0 < k_end) {
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
      if (t0 + kTile > k_end) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (t0 + kb * 16 + 4 * g + j >= k_end) sc[kb][j] = kNegInf;
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
#pragma unroll
    for (int i = 0; i < 8; ++i) kcur[i] = knext[i];
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

extern "C" int32_t split_kv_decode(const void* q, const void* k_shards, const void* v_shards,
                                   int32_t dtype, int32_t n_shards, int32_t batch, int64_t t_shard,
                                   const int64_t* shard_lens, int32_t hq, int32_t hkv, int32_t d_qk,
                                   int32_t d_v, float scale, float* o_parts, float* lse_parts,
                                   void* workspace, size_t ws_bytes, void* stream) {
  RA_CHECK(dtype == CP_BF16 || dtype == CP_F32, CP_EDTYPE, "split_kv_decode: dtype=%d", dtype);
  RA_CHECK(dtype == CP_BF16, CP_EUNSUPPORTED, "split_kv_decode: only bf16 inputs are supported");
  RA_CHECK(n_shards > 0 && batch >= 0 && t_shard >= 0, CP_EINVAL,
           "split_kv_decode: bad sizes (n_shards=%d batch=%d t_shard=%lld)", n_shards, batch,
           static_cast<long long>(t_shard));
  RA_CHECK(hq > 0 && hkv > 0 && hq % hkv == 0, CP_EINVAL,
           "split_kv_decode: hq=%d must be a positive multiple of hkv=%d", hq, hkv);
  RA_CHECK(d_qk == kD && d_v == kD, CP_EUNSUPPORTED,
           "split_kv_decode: only d_qk = d_v = 128 is supported (got %d, %d)", d_qk, d_v);
  RA_CHECK(hq / hkv <= kMaxGroup, CP_EUNSUPPORTED,
           "split_kv_decode: hq/hkv=%d exceeds %d query heads per kv head", hq / hkv, kMaxGroup);
  RA_CHECK(scale > 0.f && scale < __builtin_huge_valf(), CP_EINVAL,
           "split_kv_decode: scale must be positive and finite");
  if (batch == 0) return ok();
  RA_CHECK(q && o_parts && lse_parts && (t_shard == 0 || (k_shards && v_shards)), CP_EINVAL,
           "split_kv_decode: NULL pointer");
  RA_CHECK(aligned16(q) && aligned16(o_parts) && (t_shard == 0 || (aligned16(k_shards) && aligned16(v_shards))),
           CP_EINVAL, "split_kv_decode: device pointers must be 16-byte aligned");
  const int32_t splits = choose_splits(n_shards, batch, hkv, t_shard);
  const size_t need = split_kv_decode_workspace(n_shards, batch, hq, hkv, d_v, t_shard);
  RA_CHECK(ws_bytes >= need && (need == 0 || (workspace && aligned16(workspace))), CP_EINVAL,
           "split_kv_decode: workspace of %zu bytes (16-byte aligned) needed, got %zu", need,
           ws_bytes);
  const int64_t items = static_cast<int64_t>(n_shards) * batch * hkv * splits;
  RA_CHECK(items < (int64_t{1} << 31), CP_EUNSUPPORTED, "split_kv_decode: too many work items");

  const int64_t rows = static_cast<int64_t>(n_shards) * batch * hq;
  DecodeArgs args{};
  args.q = static_cast<const uint16_t*>(q);
  args.k = static_cast<const uint16_t*>(k_shards);
  args.v = static_cast<const uint16_t*>(v_shards);
  args.shard_lens = shard_lens;
  args.t_shard = t_shard;
  args.n_shards = n_shards; args.batch = batch; args.hq = hq; args.hkv = hkv;
  args.group = hq / hkv; args.n_splits = splits;
  args.scale = scale; args.scale_log2 = scale * kLog2e;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_lse = ws_o ? ws_o + static_cast<size_t>(splits) * rows * kD : nullptr;
  args.o = splits > 1 ? ws_o : o_parts;
  args.lse = splits > 1 ? ws_lse : lse_parts;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipLaunchKernelGGL(decode_bf16_kernel, dim3(static_cast<unsigned>(items)), dim3(kThreads), 0, st,
                     args);
  hipError_t err = hipGetLastError();
  RA_CHECK(err == hipSuccess, CP_EHIP, "split_kv_decode: launch failed: %s", hipGetErrorString(err));
  if (splits > 1) {
    const int32_t rc = launch_lse_merge(ws_o, ws_lse, splits, rows, kD, o_parts, CP_F32, lse_parts, st);
    if (rc != CP_OK) return rc;
  }
  return ok();
}
