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
//  * workgroup = 4 waves = 128 query rows of one (batch, query head); each
//    wave owns 32 rows whose Q fragment stays in registers for the sweep;
//  * K/V tiles of 64 keys go global -> registers (prefetched one tile ahead)
//    -> LDS; K rows padded by 16 B, V rows by 64 B (bank-conflict-free
//    b128 / transposed reads);
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand,
//    Q^T as B), so each lane holds 32 scores of ONE query row: the row max
//    and row sum are in-register plus one cross-half exchange;
//  * P^T stays in registers and is the B operand of O^T += V^T P^T; the
//    contraction order over keys is permuted to match the score layout, and
//    V^T is read with ds_read_b64_tr_b16 from row-major V in LDS;
//  * exp2-domain online softmax; fully visible tiles skip the mask.
#include <hip/hip_runtime.h>

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
constexpr int kBM = 128;  // query rows per workgroup
constexpr int kBN = 64;   // keys per tile
constexpr int kThreads = 256;

template <int DQK, int DV>
struct Bf16Cfg {
  static constexpr int KPITCH = DQK + 8;   // bf16 elements per K row in LDS (+16 B)
  static constexpr int VPITCH = DV + 32;   // bf16 elements per V row in LDS (+64 B)
  static constexpr int KCH = kBN * DQK / 8 / kThreads;  // 16-B chunks per thread, K tile
  static constexpr int VCH = kBN * DV / 8 / kThreads;   // 16-B chunks per thread, V tile
  static constexpr int QC = DQK / 16;  // 16-wide d chunks (MFMA K steps) for Q K^T
  static constexpr int DB = DV / 32;   // 32-wide d_v blocks of O^T
  static_assert(KCH * kThreads * 8 == kBN * DQK, "K tile must split evenly");
  static_assert(VCH * kThreads * 8 == kBN * DV, "V tile must split evenly");
};

template <int DQK, int DV>
__global__ void __launch_bounds__(kThreads, 2) attn_step_bf16_kernel(StepArgs a) {
  using C = Bf16Cfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBN * C::KPITCH];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[kBN * C::VPITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 31;  // query row within the wave (B / C column)
  const int hh = lane >> 5;   // which half of the contraction slice this lane holds

  const int logical = xcd_contiguous_id(blockIdx.x, a.total_wgs);
  int qt = logical % a.n_qtiles;
  const int rest = logical / a.n_qtiles;
  const int h = rest % a.hq;
  const int b = rest / a.hq;
  if (a.reverse_q) qt = a.n_qtiles - 1 - qt;
  const int kvh = h / a.group;

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);

  const int64_t q_first = static_cast<int64_t>(qt) * kBM;
  const int64_t q_last = min(a.sq, q_first + kBM) - 1;  // last valid local row of the WG
  const int64_t wq0 = q_first + wave * 32;              // first row of this wave
  const int64_t wq_last = min(wq0 + 31, a.sq - 1);
  const int64_t my_row = wq0 + col;
  const bool row_valid = my_row < a.sq;

  // Number of keys any row of this workgroup can see.
  int64_t nkeys = a.sk;
  if (a.causal) {
    const int64_t lim = a.q_pos0 + q_last - a.k_pos0 + 1;
    nkeys = lim < 0 ? 0 : (lim < a.sk ? lim : a.sk);
  }
  const int ntiles = static_cast<int>((nkeys + kBN - 1) / kBN);

  // Q fragment: for chunk c, lane holds Q[row][16c + 8hh .. +7] (B operand).
  bf16x8 qf[C::QC];
  {
    const uint16_t* qp = qg + ((static_cast<int64_t>(b) * a.sq + my_row) * a.hq + h) * DQK;
#pragma unroll
    for (int c = 0; c < C::QC; ++c) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (row_valid) raw = *reinterpret_cast<const u32x4*>(qp + 16 * c + 8 * hh);
      qf[c] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 oacc[C::DB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[d][i] = 0.f;
  float m_run = kNegInf;  // running max of raw scores of this lane's row
  float l_run = 0.f;      // running sum over this lane's half of the keys

  u32x4 kreg[C::KCH];
  u32x4 vreg[C::VCH];
  const int64_t kv_row_stride = static_cast<int64_t>(a.hkv);
  const int64_t kv_base_row = static_cast<int64_t>(b) * a.sk;

  auto load_tile = [&](int t) {
    const int64_t key0 = static_cast<int64_t>(t) * kBN;
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
      const int ci = tid + kThreads * i;
      const int row = ci / (DQK / 8);
      const int cc = ci % (DQK / 8);
      const int64_t key = key0 + row;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (key < a.sk)
        raw = *reinterpret_cast<const u32x4*>(
            kg + ((kv_base_row + key) * kv_row_stride + kvh) * DQK + cc * 8);
      kreg[i] = raw;
    }
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) {
      const int ci = tid + kThreads * i;
      const int row = ci / (DV / 8);
      const int cc = ci % (DV / 8);
      const int64_t key = key0 + row;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (key < a.sk)
        raw = *reinterpret_cast<const u32x4*>(
            vg + ((kv_base_row + key) * kv_row_stride + kvh) * DV + cc * 8);
      vreg[i] = raw;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < C::KCH; ++i) {
      const int ci = tid + kThreads * i;
      const int row = ci / (DQK / 8);
      const int cc = ci % (DQK / 8);
      *reinterpret_cast<u32x4*>(&Ks[row * C::KPITCH + cc * 8]) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < C::VCH; ++i) {
      const int ci = tid + kThreads * i;
      const int row = ci / (DV / 8);
      const int cc = ci % (DV / 8);
      *reinterpret_cast<u32x4*>(&Vs[row * C::VPITCH + cc * 8]) = vreg[i];
    }
  };

  if (ntiles > 0) load_tile(0);
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < ntiles) load_tile(t + 1);

    const int64_t key0 = static_cast<int64_t>(t) * kBN;
    // Rows of this wave that see no key of this tile skip the math.
    const bool wave_has_rows = wq0 < a.sq;
    const bool wave_sees_tile =
        wave_has_rows && (!a.causal || a.k_pos0 + key0 <= a.q_pos0 + wq_last);
    if (!wave_sees_tile) continue;
    const bool need_mask = (key0 + kBN > a.sk) ||
                           (a.causal && a.k_pos0 + key0 + kBN - 1 > a.q_pos0 + wq0);

    // ---- S^T = K Q^T: two 32-key blocks
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
      const uint16_t* krow = &Ks[(kb * 32 + col) * C::KPITCH + 8 * hh];
#pragma unroll
      for (int c = 0; c < C::QC; ++c) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(krow + 16 * c));
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kb], 0, 0, 0);
      }
    }
    // s[kb][i] is the score of key key0 + kb*32 + 8*(i/4) + 4*hh + i%4 for this lane's row.
    if (need_mask) {
      const int64_t qpos = a.q_pos0 + my_row;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t key = key0 + kb * 32 + 8 * (i / 4) + 4 * hh + (i % 4);
          const bool vis = key < a.sk && (!a.causal || a.k_pos0 + key <= qpos);
          if (!vis) s[kb][i] = kNegInf;
        }
    }

    // ---- online softmax (exp2 domain)
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = wave_max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float neg_mc = -m_use * a.scale_log2;
    const float alpha = fast_exp2(m_run * a.scale_log2 + neg_mc);  // 0 when m_run = -inf
    m_run = m_new;

    float psum = 0.f;
    bf16x8 pb[4];
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
    l_run = fmaf(l_run, alpha, psum);
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[d][i] *= alpha;

    // ---- O^T += V^T P^T over four 16-key chunks
    const int g = lane >> 4;   // 16-lane group
    const int i16 = lane & 15;
#pragma unroll
    for (int d = 0; d < C::DB; ++d) {
      const int dvb = d * 32 + 16 * (g & 1);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const int r0 = kc * 16 + 4 * (g >> 1) + (i16 >> 2);
        const uint16_t* pa = &Vs[r0 * C::VPITCH + dvb + 4 * (i16 & 3)];
        const s16x4 lo = lds_read_tr16(pa);
        const s16x4 hi = lds_read_tr16(pa + 8 * C::VPITCH);
        oacc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(join_bf16x4(lo, hi), pb[kc], oacc[d],
                                                          0, 0, 0);
      }
    }
  }

  // ---- epilogue: normalise, LSE, optional merge into the running result
  if (!row_valid) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const bool has = m_run != kNegInf && l_tot > 0.f;
  const float inv = has ? 1.f / l_tot : 0.f;
  const float lse_blk = has ? m_run * a.scale + fast_log2(l_tot) * kLn2 : kNegInf;
  const int64_t orow = (static_cast<int64_t>(b) * a.sq + my_row) * a.hq + h;
  float* op = a.o + orow * DV;
  float w_old = 0.f, w_blk = 1.f, lse_out = lse_blk;
  if (a.accumulate) lse_out = merge_weights(a.lse[orow], lse_blk, &w_old, &w_blk);
  const float wb = w_blk * inv;
#pragma unroll
  for (int d = 0; d < C::DB; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dv0 = d * 32 + 8 * j + 4 * hh;
      f32x4 val = {oacc[d][4 * j] * wb, oacc[d][4 * j + 1] * wb, oacc[d][4 * j + 2] * wb,
                   oacc[d][4 * j + 3] * wb};
      if (a.accumulate) {
        const f32x4 old = *reinterpret_cast<const f32x4*>(op + dv0);
        val += old * w_old;
      }
      *reinterpret_cast<f32x4*>(op + dv0) = val;
    }
  if (hh == 0) a.lse[orow] = lse_out;
}

// ---------------------------------------------------------------------------
// float32 vector kernel (correctness path for float32 inputs)
// ---------------------------------------------------------------------------
constexpr int kF32Rows = 64;  // one query row per lane, one wave per workgroup
constexpr int kF32Keys = 32;

template <int DQK, int DV>
__global__ void __launch_bounds__(kF32Rows) attn_step_f32_kernel(StepArgs a) {
  __shared__ float Ks[kF32Keys][DQK];
  __shared__ float Vs[kF32Keys][DV];
  const int lane = threadIdx.x;
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

  for (int64_t key0 = 0; key0 < nkeys; key0 += kF32Keys) {
    __syncthreads();
    for (int i = lane; i < kF32Keys * DQK; i += kF32Rows) {
      const int64_t key = key0 + i / DQK;
      Ks[i / DQK][i % DQK] =
          key < a.sk ? kg[((static_cast<int64_t>(b) * a.sk + key) * a.hkv + kvh) * DQK + i % DQK] : 0.f;
    }
    for (int i = lane; i < kF32Keys * DV; i += kF32Rows) {
      const int64_t key = key0 + i / DV;
      Vs[i / DV][i % DV] =
          key < a.sk ? vg[((static_cast<int64_t>(b) * a.sk + key) * a.hkv + kvh) * DV + i % DV] : 0.f;
    }
    __syncthreads();
    float s[kF32Keys];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < kF32Keys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < DQK; ++d) dot = fmaf(qr[d], Ks[j][d], dot);
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
      for (int j = 0; j < kF32Keys; ++j) x = fmaf(s[j], Vs[j][d], x);
      acc[d] = x;
    }
  }
  if (!row_valid) return;
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

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

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
  const bool pair_ok = (d_qk == 64 && d_v == 64) || (d_qk == 128 && d_v == 128) ||
                       (d_qk == 192 && d_v == 128);
  RA_CHECK(pair_ok, CP_EUNSUPPORTED, "ring_attn_step: (d_qk, d_v) = (%d, %d) not supported", d_qk,
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
        if (d_qk == 64)
          rc = launch(attn_step_bf16_kernel<64, 64>, kBM, kThreads, args, batch, st);
        else if (d_qk == 128)
          rc = launch(attn_step_bf16_kernel<128, 128>, kBM, kThreads, args, batch, st);
        else
          rc = launch(attn_step_bf16_kernel<192, 128>, kBM, kThreads, args, batch, st);
      } else {
        if (d_qk == 64)
          rc = launch(attn_step_f32_kernel<64, 64>, kF32Rows, kF32Rows, args, batch, st);
        else if (d_qk == 128)
          rc = launch(attn_step_f32_kernel<128, 128>, kF32Rows, kF32Rows, args, batch, st);
        else
          rc = launch(attn_step_f32_kernel<192, 128>, kF32Rows, kF32Rows, args, batch, st);
      }
      if (rc != CP_OK) return rc;
    }
  }
  if (class_out) *class_out = cls;
  return ok();
}
