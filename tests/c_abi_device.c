/* The device entry points of the C ABI from plain C: device memory from the
 * HIP runtime, no framework.  Two ring steps of one query chunk, the second
 * LSE-merged into the first's result (accumulate), then the same queries'
 * result read back.
 *
 * usage: c_abi_device <input file> <output file>
 * input  (little endian): int64 sq, ska, skb, hq, hkv, d, q_pos0, ka_pos0,
 *        kb_pos0, causal; then bf16 bits of q [sq, hq, d], ka and va
 *        [ska, hkv, d], kb and vb [skb, hkv, d].
 * output: float32 o [sq, hq, d], float32 lse [sq, hq], int32 class of each
 *        step.
 * Exit status 0 on success; a failing call is named on stderr. */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "ringattn.h"

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static int read_all(FILE* f, void* dst, size_t bytes) { return fread(dst, 1, bytes, f) == bytes; }

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  if (!hip_ok(hipMalloc(&d, bytes > 0 ? bytes : 16), "hipMalloc")) return NULL;
  if (bytes > 0 && !hip_ok(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice), "hipMemcpy to device")) return NULL;
  return d;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <input> <output>\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  int64_t h[10];
  if (!in || !read_all(in, h, sizeof h)) {
    fprintf(stderr, "cannot read %s\n", argv[1]);
    return 1;
  }
  const int64_t sq = h[0], ska = h[1], skb = h[2], hq = h[3], hkv = h[4], d = h[5];
  const int64_t q_pos0 = h[6], ka_pos0 = h[7], kb_pos0 = h[8];
  const int32_t mask = h[9] ? CP_MASK_CAUSAL : CP_MASK_NONE;
  const size_t nq = (size_t)(sq * hq * d), nka = (size_t)(ska * hkv * d), nkb = (size_t)(skb * hkv * d);
  uint16_t* hq_ = malloc(2 * nq + 2);
  uint16_t* hka = malloc(2 * nka + 2);
  uint16_t* hva = malloc(2 * nka + 2);
  uint16_t* hkb = malloc(2 * nkb + 2);
  uint16_t* hvb = malloc(2 * nkb + 2);
  float* ho = malloc(4 * nq + 4);
  float* hl = malloc(4 * (size_t)(sq * hq) + 4);
  if (!hq_ || !hka || !hva || !hkb || !hvb || !ho || !hl) return 1;
  if (!read_all(in, hq_, 2 * nq) || !read_all(in, hka, 2 * nka) || !read_all(in, hva, 2 * nka) ||
      !read_all(in, hkb, 2 * nkb) || !read_all(in, hvb, 2 * nkb)) {
    fprintf(stderr, "short input\n");
    return 1;
  }
  fclose(in);

  void* dq = to_device(hq_, 2 * nq);
  void* dka = to_device(hka, 2 * nka);
  void* dva = to_device(hva, 2 * nka);
  void* dkb = to_device(hkb, 2 * nkb);
  void* dvb = to_device(hvb, 2 * nkb);
  float* dout = NULL;
  float* dlse = NULL;
  if (!dq || !dka || !dva || !dkb || !dvb) return 1;
  if (!hip_ok(hipMalloc((void**)&dout, 4 * nq + 4), "hipMalloc o") ||
      !hip_ok(hipMalloc((void**)&dlse, 4 * (size_t)(sq * hq) + 4), "hipMalloc lse"))
    return 1;

  const float scale = 1.0f / sqrtf((float)d);
  int32_t cls[2] = {-1, -1};
  int32_t st = ring_attn_step(dq, dka, dva, CP_BF16, 1, sq, ska, (int32_t)hq, (int32_t)hkv, (int32_t)d,
                              (int32_t)d, q_pos0, ka_pos0, mask, scale, 0, dout, dlse, &cls[0], NULL);
  if (st != CP_OK) {
    fprintf(stderr, "ring_attn_step (first block): %s: %s\n", cp_status_string(st), cp_last_error());
    return 1;
  }
  st = ring_attn_step(dq, dkb, dvb, CP_BF16, 1, sq, skb, (int32_t)hq, (int32_t)hkv, (int32_t)d, (int32_t)d,
                      q_pos0, kb_pos0, mask, scale, 1, dout, dlse, &cls[1], NULL);
  if (st != CP_OK) {
    fprintf(stderr, "ring_attn_step (second block, accumulate): %s: %s\n", cp_status_string(st),
            cp_last_error());
    return 1;
  }
  if (!hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize") ||
      !hip_ok(hipMemcpy(ho, dout, 4 * nq, hipMemcpyDeviceToHost), "hipMemcpy o") ||
      !hip_ok(hipMemcpy(hl, dlse, 4 * (size_t)(sq * hq), hipMemcpyDeviceToHost), "hipMemcpy lse"))
    return 1;

  FILE* out = fopen(argv[2], "wb");
  if (!out || fwrite(ho, 4, nq, out) != nq || fwrite(hl, 4, (size_t)(sq * hq), out) != (size_t)(sq * hq) ||
      fwrite(cls, 4, 2, out) != 2) {
    fprintf(stderr, "cannot write %s\n", argv[2]);
    return 1;
  }
  fclose(out);
  (void)hipFree(dq);
  (void)hipFree(dka);
  (void)hipFree(dva);
  (void)hipFree(dkb);
  (void)hipFree(dvb);
  (void)hipFree(dout);
  (void)hipFree(dlse);
  free(hq_);
  free(hka);
  free(hva);
  free(hkb);
  free(hvb);
  free(ho);
  free(hl);
  return 0;
}
