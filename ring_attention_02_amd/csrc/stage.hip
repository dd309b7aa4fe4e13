// Ring-step staging: "receiving" the next K/V block into a staging slot.
//
// In the ring (guijiagi.com "Ring Attention", ring-topology excerpt) every
// step hands the current K/V block to the next device while the local
// attention runs, and the video "How Context Parallelism Splits Long
// Sequences Across GPUs" (chapter on the wire budget) double-buffers that
// transfer.  On one GPU the transfer is a device-to-device copy of the
// block's pieces into the idle slot; this kernel moves all of them in one
// launch (16-byte vector loads and stores, grid-stride over the total).
//
// Also here: the row gather that applies an index on the device -- the
// restore index of the head-tail partition (vLLM-Ascend "Context Parallel
// (CP)", PCP head-tail paragraph) and the reorganisation of an all-gathered
// KV cache by request (same guide, MLA prefill note).
#include <hip/hip_runtime.h>

#include "kernels_common.h"
#include "status.h"

namespace ringattn {
namespace {

constexpr int kMaxPieces = 8;
constexpr int kStageThreads = 256;

struct StagePieces {
  u32x4* dst[kMaxPieces];
  const u32x4* src[kMaxPieces];
  int64_t end[kMaxPieces];   // exclusive prefix sums of the pieces' 16-B units
  int32_t n;
};

__global__ void __launch_bounds__(kStageThreads) stage_copy_kernel(StagePieces p) {
  const int64_t total = p.end[p.n - 1];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kStageThreads;
  int piece = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kStageThreads + threadIdx.x; i < total; i += stride) {
    while (i >= p.end[piece]) ++piece;                // indices only grow
    const int64_t local = i - (piece == 0 ? 0 : p.end[piece - 1]);
    p.dst[piece][local] = p.src[piece][local];
  }
}

}  // namespace
}  // namespace ringattn

extern "C" int32_t ring_stage_copy(void* const* dsts, const void* const* srcs,
                                   const int64_t* bytes, int32_t n, void* stream) {
  using namespace ringattn;
  RA_CHECK(n >= 1 && n <= kMaxPieces, CP_EINVAL, "ring_stage_copy: n=%d outside [1, %d]", n,
           kMaxPieces);
  RA_CHECK(dsts && srcs && bytes, CP_EINVAL, "ring_stage_copy: NULL array");
  StagePieces p{};
  p.n = n;
  int64_t units = 0;
  for (int i = 0; i < n; ++i) {
    RA_CHECK(bytes[i] >= 0 && bytes[i] % 16 == 0, CP_EINVAL,
             "ring_stage_copy: piece %d has %lld bytes (must be a non-negative multiple of 16)", i,
             static_cast<long long>(bytes[i]));
    RA_CHECK(bytes[i] == 0 || (dsts[i] && srcs[i]), CP_EINVAL, "ring_stage_copy: NULL piece %d", i);
    RA_CHECK((reinterpret_cast<uintptr_t>(dsts[i]) & 15u) == 0 &&
                 (reinterpret_cast<uintptr_t>(srcs[i]) & 15u) == 0,
             CP_EINVAL, "ring_stage_copy: piece %d is not 16-byte aligned", i);
    p.dst[i] = static_cast<u32x4*>(dsts[i]);
    p.src[i] = static_cast<const u32x4*>(srcs[i]);
    units += bytes[i] / 16;
    p.end[i] = units;
  }
  if (units == 0) return ok();
  const int64_t want = (units + kStageThreads * 4 - 1) / (kStageThreads * 4);
  const unsigned blocks = static_cast<unsigned>(want < 2048 ? want : 2048);
  hipLaunchKernelGGL(stage_copy_kernel, dim3(blocks), dim3(kStageThreads), 0,
                     static_cast<hipStream_t>(stream), p);
  const hipError_t err = hipGetLastError();
  RA_CHECK(err == hipSuccess, CP_EHIP, "ring_stage_copy: launch failed: %s", hipGetErrorString(err));
  return ok();
}

namespace ringattn {
namespace {

constexpr int kGatherInFlight = 48;  // 16-byte loads per lane before their stores (48 KiB per wave)

// One wave per row (rows grid-strided over all waves): the row's index is
// read once, then each lane moves 16-byte units lane, lane + 64, ... with
// kGatherInFlight loads in flight before their stores, so a row of up to
// 48 KiB is read as one burst and written as one.  Fewer waves with longer
// bursts beat more waves with short ones: on the 135,168-row reorganisation
// (rows of 48 and 32 KiB) 48 loads per lane at about two waves per SIMD
// moved 9 % more bytes per second than 8 loads at eight waves per SIMD.
// Every byte is moved once, so loads and stores are non-temporal
// (streaming): 2.5 % faster than cached ones.
__global__ void __launch_bounds__(kStageThreads) gather_rows_kernel(u32x4* __restrict__ dst,
                                                                   const u32x4* __restrict__ src,
                                                                   const int64_t* __restrict__ idx,
                                                                   int64_t n, int64_t n_src,
                                                                   int64_t units_per_row) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kStageThreads / 64);
  for (int64_t row = static_cast<int64_t>(blockIdx.x) * (kStageThreads / 64) + (threadIdx.x >> 6); row < n;
       row += waves) {
    const int64_t from = idx[row];
    const bool valid = from >= 0 && from < n_src;
    const u32x4* s = src + (valid ? from : 0) * units_per_row;
    u32x4* d = dst + row * units_per_row;
    for (int64_t u = lane; u < units_per_row; u += kGatherInFlight * 64) {
      u32x4 x[kGatherInFlight];
#pragma unroll
      for (int i = 0; i < kGatherInFlight; ++i) {
        const int64_t v = u + i * 64;
        x[i] = (valid && v < units_per_row) ? __builtin_nontemporal_load(s + v) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < kGatherInFlight; ++i)
        if (u + i * 64 < units_per_row) __builtin_nontemporal_store(x[i], d + u + i * 64);
    }
  }
}

}  // namespace
}  // namespace ringattn

extern "C" int32_t cp_gather_rows(void* dst, const void* src, const int64_t* idx, int64_t n,
                                  int64_t n_src, int64_t row_bytes, void* stream) {
  using namespace ringattn;
  RA_CHECK(n >= 0 && n_src >= 0, CP_EINVAL, "cp_gather_rows: negative row count");
  RA_CHECK(row_bytes > 0 && row_bytes % 16 == 0, CP_EINVAL,
           "cp_gather_rows: row_bytes=%lld must be a positive multiple of 16",
           static_cast<long long>(row_bytes));
  if (n == 0) return ok();
  RA_CHECK(dst && idx && (n_src == 0 || src), CP_EINVAL, "cp_gather_rows: NULL pointer");
  RA_CHECK((reinterpret_cast<uintptr_t>(dst) & 15u) == 0 && (reinterpret_cast<uintptr_t>(src) & 15u) == 0,
           CP_EINVAL, "cp_gather_rows: dst / src must be 16-byte aligned");
  const uintptr_t d0 = reinterpret_cast<uintptr_t>(dst), s0 = reinterpret_cast<uintptr_t>(src);
  RA_CHECK(n_src == 0 || d0 >= s0 + static_cast<uintptr_t>(n_src * row_bytes) ||
               s0 >= d0 + static_cast<uintptr_t>(n * row_bytes),
           CP_EINVAL, "cp_gather_rows: dst and src overlap");
  const int64_t units = row_bytes / 16;
  const int64_t rows_per_block = kStageThreads / 64;
  const int64_t want = (n + rows_per_block - 1) / rows_per_block;   // one row per wave
  const unsigned blocks = static_cast<unsigned>(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(kStageThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<u32x4*>(dst),
                     static_cast<const u32x4*>(src), idx, n, n_src, units);
  const hipError_t err = hipGetLastError();
  RA_CHECK(err == hipSuccess, CP_EHIP, "cp_gather_rows: launch failed: %s", hipGetErrorString(err));
  return ok();
}
