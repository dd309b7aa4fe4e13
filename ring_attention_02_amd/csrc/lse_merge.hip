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
// HBM-bound: every thread owns 4 consecutive floats of one row; a row's
// threads are adjacent, so each part is read with fully coalesced 16-B loads.
#include <hip/hip_runtime.h>

#include "kernels_common.h"
#include "status.h"

namespace ringattn {
namespace {

constexpr int kMergeThreads = 256;

template <bool OUT_BF16>
__global__ void __launch_bounds__(kMergeThreads)
lse_merge_kernel(const float* __restrict__ o_parts, const float* __restrict__ lse_parts,
                 int32_t n, int64_t rows, int32_t dv, void* __restrict__ o_out,
                 float* __restrict__ lse_out) {
  const int tpr = dv / 4;  // threads per row
  const int rpb = kMergeThreads / tpr;
  const int local_row = threadIdx.x / tpr;
  const int c4 = threadIdx.x % tpr;
  if (local_row >= rpb) return;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * rpb + local_row;
  if (row >= rows) return;

  float m = kNegInf;
  for (int k = 0; k < n; ++k) m = fmaxf(m, lse_parts[k * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float lse = kNegInf;
  if (m != kNegInf) {
    float tot = 0.f;
    for (int k = 0; k < n; ++k) tot += fast_exp2((lse_parts[k * rows + row] - m) * kLog2e);
    const float inv = 1.f / tot;
    for (int k = 0; k < n; ++k) {
      const float w = fast_exp2((lse_parts[k * rows + row] - m) * kLog2e) * inv;
      if (w != 0.f) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(o_parts + (k * rows + row) * dv + 4 * c4);
        acc += x * w;
      }
    }
    lse = m + fast_log2(tot) * kLn2;
  }
  if (OUT_BF16) {
    bf16x4 b = {static_cast<__bf16>(acc[0]), static_cast<__bf16>(acc[1]),
                static_cast<__bf16>(acc[2]), static_cast<__bf16>(acc[3])};
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(o_out) + row * dv + 4 * c4) = b;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(o_out) + row * dv + 4 * c4) = acc;
  }
  if (lse_out != nullptr && c4 == 0) lse_out[row] = lse;
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

// Shared with the decode entry point, which merges its KV splits the same way.
int32_t launch_lse_merge(const float* o_parts, const float* lse_parts, int32_t n_parts,
                         int64_t rows, int32_t d_v, void* o_out, int32_t out_dtype,
                         float* lse_out, hipStream_t stream) {
  const int tpr = d_v / 4;
  const int rpb = kMergeThreads / tpr;
  const int64_t blocks = (rows + rpb - 1) / rpb;
  RA_CHECK(blocks < (int64_t{1} << 31), CP_EUNSUPPORTED, "lse_merge: %lld rows too many",
           static_cast<long long>(rows));
  if (out_dtype == CP_BF16)
    hipLaunchKernelGGL(lse_merge_kernel<true>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kMergeThreads), 0, stream, o_parts, lse_parts, n_parts, rows, d_v,
                       o_out, lse_out);
  else
    hipLaunchKernelGGL(lse_merge_kernel<false>, dim3(static_cast<unsigned>(blocks)),
                       dim3(kMergeThreads), 0, stream, o_parts, lse_parts, n_parts, rows, d_v,
                       o_out, lse_out);
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
