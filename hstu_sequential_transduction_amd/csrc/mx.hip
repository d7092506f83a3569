// MXFP8 quantization ("Bending the Scaling Law Curve in Large-Scale
// Recommendation Systems", Mixed precision: BF16 for most operations, FP8
// for the matrix products; element and scale formats of the OCP
// Microscaling (MX) specification).
//
// Every 32 consecutive values along the contraction index form a block with
// one E8M0 scale byte e (value 2^(e-127)): the block's shared exponent is
// floor(log2(amax)) - 8 (8 = the exponent of E4M3's largest power of two),
// so value / 2^shared lies in [0, 512) and is rounded to E4M3 (see mx.h).
// Division by the power of two is exact, so the codes depend on the inputs
// alone.  An all-zero block gets e = 0 and zero codes.
//
// Outputs are k-contiguous: codes [rows][K] bytes, scales [rows][K/32]
// bytes, the layout the MX GEMM streams into LDS.
#include "common.h"
#include "internal.h"
#include "mx.h"

namespace hstu {
namespace {

// one block of 32 values: shared exponent and the 32 codes (8 dwords)
HSTU_DEV int mx_block(const float (&v)[32], uint32_t (&out)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
  const int shared = mx_shared_exp(amax);
#pragma unroll
  for (int q = 0; q < 8; ++q)
    out[q] = mx_cvt4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3], shared);
  return shared + 127;
}

// rows x K values (element (r, k) at in[r * ld_r + k * ld_k], bf16) -> codes
// [rows][K] and scales [rows][K/32]; one lane per block
template <bool KCONT>
__global__ __launch_bounds__(256) void k_mx_quant(const bf16* __restrict__ in, int64_t ld_r,
                                                  int64_t ld_k, int64_t rows, int64_t K,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  const int64_t nb = K / 32;
  const int64_t total = rows * nb;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / nb, kb = i - r * nb;
    float v[32];
    if (KCONT) {
      const bf16* p = in + r * ld_r + kb * 32;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(p + 8 * q);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * q + e] = bf2f(x[e]);
      }
    } else {
      const bf16* p = in + r * ld_r + kb * 32 * ld_k;
#pragma unroll
      for (int e = 0; e < 32; ++e) v[e] = bf2f(p[e * ld_k]);
    }
    uint32_t out[8];
    const int s = mx_block(v, out);
    u32x4* dst = reinterpret_cast<u32x4*>(codes + r * K + kb * 32);
    dst[0] = u32x4{out[0], out[1], out[2], out[3]};
    dst[1] = u32x4{out[4], out[5], out[6], out[7]};
    scales[r * nb + kb] = (uint8_t)s;
  }
}

int quant_grid(int64_t blocks) {
  const int64_t g = (blocks + 255) / 256;
  return (int)std::min<int64_t>(std::max<int64_t>(g, 1), 8192);
}

}  // namespace

hipError_t launch_mx_quant_rows(const void* x, int64_t ld, int64_t rows, int64_t K,
                                uint8_t* codes, uint8_t* scales, hipStream_t st) {
  if (rows <= 0 || K <= 0) return hipSuccess;
  k_mx_quant<true><<<quant_grid(rows * K / 32), 256, 0, st>>>(
      static_cast<const bf16*>(x), ld, 1, rows, K, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_quant_cols(const void* w, int64_t K, int64_t N, uint8_t* codes,
                                uint8_t* scales, hipStream_t st) {
  if (N <= 0 || K <= 0) return hipSuccess;
  // output row n = column n of W [K, N]; its k-th value sits at W[k * N + n]
  k_mx_quant<false><<<quant_grid(N * K / 32), 256, 0, st>>>(
      static_cast<const bf16*>(w), 1, N, N, K, codes, scales);
  return hipGetLastError();
}

}  // namespace hstu
