// LSE-rescale merge of n partial attention results of the same rows.
//
// vLLM-Ascend developer guide "Context Parallel (CP)", DCP section: the
// partial outputs and LSEs computed against different slices of the keys are
// combined into the final output; guijiagi.com "Ring Attention", memory-wall
// excerpt: a running maximum and running sum make the combination exact.
//
// With M = max_k LSE_k:  LSE = M + ln sum_k exp(LSE_k - M),
//                        O   = sum_k exp(LSE_k - LSE) * O_k.
//
// HBM-bound: a row's threads are adjacent and each owns four 16-B pieces of
// it, tpr pieces apart (tpr = threads per row), so every load and store
// instruction of a wave covers whole 128-B lines; parts are read and the
// result written non-temporally (each byte is touched once).
#include <hip/hip_runtime.h>

#include "kernels_common.h"
#include "status.h"

namespace ringattn {
namespace {

constexpr int kMergeThreads = 256;

// One pass over the parts with a running maximum (the same online rule the
// attention kernels use): each thread owns UNROLL 16-B pieces of one row,
// columns 4c + 4 tpr u, so UNROLL independent 16-B loads per part are in
// flight and the tpr threads of a row write whole lines per instruction.
template <bool OUT_BF16, int UNROLL>
__global__ void __launch_bounds__(kMergeThreads)
lse_merge_kernel(const float* __restrict__ o_parts, const float* __restrict__ lse_parts,
                 int32_t n, int64_t rows, int32_t dv, void* __restrict__ o_out,
                 float* __restrict__ lse_out) {
  const int tpr = dv / (4 * UNROLL);  // threads per row
  const int rpb = kMergeThreads / tpr;
  const int local_row = threadIdx.x / tpr;
  const int c = threadIdx.x % tpr;
  if (local_row >= rpb) return;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * rpb + local_row;
  if (row >= rows) return;

  f32x4 acc[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, tot = 0.f;
  for (int k = 0; k < n; ++k) {
    const float l = lse_parts[k * rows + row];
    const float* src = o_parts + (k * rows + row) * dv + 4 * c;
    f32x4 x[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      x[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + 4 * tpr * u));
    if (l == kNegInf) continue;                 // an empty part changes nothing
    const float m_new = fmaxf(m, l);
    const float keep = fast_exp2((m - m_new) * kLog2e);   // 0 while m = -inf
    const float w = fast_exp2((l - m_new) * kLog2e);
    tot = tot * keep + w;
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) acc[u] = acc[u] * keep + x[u] * w;
    m = m_new;
  }
  const float inv = m == kNegInf ? 0.f : 1.f / tot;
  const float lse = m == kNegInf ? kNegInf : m + fast_log2(tot) * kLn2;
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const f32x4 r = acc[u] * inv;
    if (OUT_BF16) {
      bf16x4 b = {static_cast<__bf16>(r[0]), static_cast<__bf16>(r[1]), static_cast<__bf16>(r[2]),
                  static_cast<__bf16>(r[3])};
      *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(o_out) + row * dv + 4 * c + 4 * tpr * u) = b;
    } else {
      __builtin_nontemporal_store(r,
                                  reinterpret_cast<f32x4*>(static_cast<float*>(o_out) + row * dv + 4 * c + 4 * tpr * u));
    }
  }
  if (lse_out != nullptr && c == 0) lse_out[row] = lse;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

// Shared with the decode entry point, which merges its KV splits the same way.
int32_t launch_lse_merge(const float* o_parts, const float* lse_parts, int32_t n_parts,
                         int64_t rows, int32_t d_v, void* o_out, int32_t out_dtype,
                         float* lse_out, hipStream_t stream) {
  const bool wide = d_v % 16 == 0;
  const int tpr = d_v / (wide ? 16 : 4);
  const int rpb = kMergeThreads / tpr;
  const int64_t blocks = (rows + rpb - 1) / rpb;
  RA_CHECK(blocks < (int64_t{1} << 31), CP_EUNSUPPORTED, "lse_merge: %lld rows too many",
           static_cast<long long>(rows));
  const dim3 grid(static_cast<unsigned>(blocks)), block(kMergeThreads);
  if (out_dtype == CP_BF16) {
    if (wide)
      hipLaunchKernelGGL((lse_merge_kernel<true, 4>), grid, block, 0, stream, o_parts, lse_parts,
                         n_parts, rows, d_v, o_out, lse_out);
    else
      hipLaunchKernelGGL((lse_merge_kernel<true, 1>), grid, block, 0, stream, o_parts, lse_parts,
                         n_parts, rows, d_v, o_out, lse_out);
  } else {
    if (wide)
      hipLaunchKernelGGL((lse_merge_kernel<false, 4>), grid, block, 0, stream, o_parts, lse_parts,
                         n_parts, rows, d_v, o_out, lse_out);
    else
      hipLaunchKernelGGL((lse_merge_kernel<false, 1>), grid, block, 0, stream, o_parts, lse_parts,
                         n_parts, rows, d_v, o_out, lse_out);
  }
  const hipError_t err = hipGetLastError();
  RA_CHECK(err == hipSuccess, CP_EHIP, "lse_merge: launch failed: %s", hipGetErrorString(err));
  return CP_OK;
}

}  // namespace ringattn

extern "C" int32_t lse_merge(const float* o_parts, const float* lse_parts, int32_t n_parts,
                             int64_t rows, int32_t d_v, void* o_out, int32_t out_dtype,
                             float* lse_out, void* stream) {
  using namespace ringattn;
  RA_CHECK(out_dtype == CP_BF16 || out_dtype == CP_F32, CP_EDTYPE, "lse_merge: out_dtype=%d",
           out_dtype);
  RA_CHECK(n_parts > 0, CP_EINVAL, "lse_merge: n_parts=%d must be > 0", n_parts);
  RA_CHECK(rows >= 0, CP_EINVAL, "lse_merge: rows < 0");
  RA_CHECK(d_v > 0 && d_v % 4 == 0 && d_v <= 512, CP_EINVAL,
           "lse_merge: d_v=%d must be a positive multiple of 4, at most 512", d_v);
  if (rows == 0) return ok();
  RA_CHECK(o_parts && lse_parts && o_out, CP_EINVAL, "lse_merge: NULL pointer");
  RA_CHECK(aligned(o_parts, 16) && aligned(o_out, out_dtype == CP_BF16 ? 8 : 16) &&
               aligned(lse_parts, 4) && (lse_out == nullptr || aligned(lse_out, 4)),
           CP_EINVAL, "lse_merge: misaligned pointer");
  const int32_t rc = launch_lse_merge(o_parts, lse_parts, n_parts, rows, d_v, o_out, out_dtype,
                                      lse_out, static_cast<hipStream_t>(stream));
  return rc == CP_OK ? ok() : rc;
}
