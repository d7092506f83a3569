// Diagnostic microbenchmark: the bf16 MFMA rate this device sustains, as the
// measured denominator beside the nominal peak in performance reports.
#include "common.h"
#include "internal.h"

namespace hstu {

namespace {

// Four independent accumulator chains of 32x32x16 bf16 MFMAs per wave, so
// every issue slot of the matrix core can be filled without waiting on a
// previous result; operands come from the lane index so nothing folds away.
__global__ __launch_bounds__(256, 2) void k_mfma_loop(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)(0.001f * (lane + e));
    b[e] = (bf16)(0.002f * (lane - e));
  }
  f32x16 acc[4] = {};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = mfma32(a, b, acc[j]);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  s = wave_sum(s);
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

}  // namespace

}  // namespace hstu

using namespace hstu;

extern "C" hstu_status hstu_diag_mfma_loop(int32_t iters, int32_t workgroups, float* out,
                                           void* stream) {
  if (iters < 1 || workgroups < 1 || !out) return HSTU_ERR_INVALID_ARG;
  (void)hipGetLastError();
  k_mfma_loop<<<workgroups, 256, 0, (hipStream_t)stream>>>(iters, out);
  return hipGetLastError() == hipSuccess ? HSTU_OK : HSTU_ERR_HIP;
}
