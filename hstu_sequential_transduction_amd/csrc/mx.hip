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

// Transposed quantization for products contracted over the rows of a
// row-major matrix (the weight gradients, contracted over the tokens):
// in [T][C] (row stride ld) -> codes [C][Tp], blocks of 32 rows of one
// column, rows T..Tp-1 read as zeros (Tp a multiple of 128), and the scales
// k-step-major, [Tp/128][C][4]: the MX GEMM's k-step covers 128 codes, so a
// row's four scales of one step are one word and a wave's rows read
// adjacent words (with [C][Tp/32] every row's word would sit on its own
// cache line).  A workgroup stages a 128-row x 64-column tile in LDS with
// 16-byte row loads, then each thread encodes one column's block of 32 rows.
// With rcodes (ROWS): the same tile also encoded along its rows, codes
// [T][C] and scales [T][C/32] (the layout of k_mx_quant), so that a matrix
// needed in both orientations is read once.
template <bool ROWS>
__global__ __launch_bounds__(256) void k_mx_quant_t(const bf16* __restrict__ in, int64_t ld,
                                                    int64_t T, int64_t C, int64_t Tp,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales,
                                                    uint8_t* __restrict__ rcodes,
                                                    uint8_t* __restrict__ rscales) {
  __shared__ bf16 tile[128][64 + 8];  // padded rows: column reads stay off one bank
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * 128, c0 = (int64_t)blockIdx.y * 64;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = tid / 8 + 32 * k, ch = tid % 8;
    bf16x8 v{};
    if (t0 + r < T) v = *reinterpret_cast<const bf16x8*>(in + (t0 + r) * ld + c0 + 8 * ch);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[r][8 * ch + e] = v[e];
  }
  __syncthreads();
  if constexpr (ROWS) {
    // one block of 32 columns of one row per thread
    const int r = tid / 2, hb = tid % 2;
    if (t0 + r < T) {
      float v[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) v[e] = bf2f(tile[r][32 * hb + e]);
      uint32_t out[8];
      const int sc = mx_block(v, out);
      u32x4* dst = reinterpret_cast<u32x4*>(rcodes + (t0 + r) * C + c0 + 32 * hb);
      dst[0] = u32x4{out[0], out[1], out[2], out[3]};
      dst[1] = u32x4{out[4], out[5], out[6], out[7]};
      rscales[(t0 + r) * (C / 32) + c0 / 32 + hb] = (uint8_t)sc;
    }
  }
  const int c = tid % 64, b = tid / 64;  // a wave: the 64 columns of one block of rows
  float v[32];
#pragma unroll
  for (int e = 0; e < 32; ++e) v[e] = bf2f(tile[32 * b + e][c]);
  uint32_t out[8];
  const int sc = mx_block(v, out);
  u32x4* dst = reinterpret_cast<u32x4*>(codes + (c0 + c) * Tp + t0 + 32 * b);
  dst[0] = u32x4{out[0], out[1], out[2], out[3]};
  dst[1] = u32x4{out[4], out[5], out[6], out[7]};
  scales[((t0 / 128) * C + c0 + c) * 4 + b] = (uint8_t)sc;
}

int quant_grid(int64_t blocks) {
  const int64_t g = (blocks + 255) / 256;
  return (int)std::min<int64_t>(std::max<int64_t>(g, 1), 8192);
}

// Attention operands (q or k, [T][H*d] bf16, row stride ld): blocks of 32
// along each head's d channels; codes [T][ld_codes] bytes (head h at byte
// h*d) and one scale word per (head, row), head-major: scales[h*T + t],
// byte b = the E8M0 scale of channels 32b..32b+31 (d <= 128; unused bytes
// zero), so that a key tile's words are one contiguous run.  A workgroup
// takes 16 rows: thread i encodes block i of them (blocks numbered along
// each row, so consecutive threads read and write consecutive 64- and
// 32-byte pieces), the scale bytes meet in LDS, and the 16 words of each
// head go out as one contiguous 64-byte run.
constexpr int MXH_ROWS = 16;
__global__ __launch_bounds__(256) void k_mx_quant_heads(const bf16* __restrict__ in, int64_t ld,
                                                        int64_t T, int H, int d,
                                                        uint8_t* __restrict__ codes,
                                                        int64_t ld_codes,
                                                        uint32_t* __restrict__ scales) {
  __shared__ uint32_t wsc[MXH_ROWS * 64];  // [row][head] words, H <= 64
  const int nb = d / 32;
  const int bpr = H * nb;  // blocks per row
  const int64_t ngroups = (T + MXH_ROWS - 1) / MXH_ROWS;
  for (int64_t grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int64_t t0 = grp * MXH_ROWS;
    const int rows = (int)min<int64_t>(MXH_ROWS, T - t0);
    for (int i = threadIdx.x; i < MXH_ROWS * 64; i += 256) wsc[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < rows * bpr; i += 256) {
      const int r = i / bpr, c = i - r * bpr;  // c = h * nb + kb
      const bf16* p = in + (t0 + r) * ld + 32 * c;
      float v[32];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8 x = *reinterpret_cast<const bf16x8*>(p + 8 * q);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * q + e] = bf2f(x[e]);
      }
      uint32_t out[8];
      const uint32_t sb = (uint32_t)mx_block(v, out);
      u32x4* dst = reinterpret_cast<u32x4*>(codes + (t0 + r) * ld_codes + 32 * c);
      dst[0] = u32x4{out[0], out[1], out[2], out[3]};
      dst[1] = u32x4{out[4], out[5], out[6], out[7]};
      const int h = c / nb, kb = c - h * nb;
      atomicOr(&wsc[r * 64 + h], sb << (8 * kb));
    }
    __syncthreads();
    for (int i = threadIdx.x; i < H * MXH_ROWS; i += 256) {
      const int h = i / MXH_ROWS, r = i - h * MXH_ROWS;
      if (r < rows) scales[h * T + t0 + r] = wsc[r * 64 + h];
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_mx_quant_rows(const void* x, int64_t ld, int64_t rows, int64_t K,
                                uint8_t* codes, uint8_t* scales, hipStream_t st) {
  if (rows <= 0 || K <= 0) return hipSuccess;
  k_mx_quant<true><<<quant_grid(rows * K / 32), 256, 0, st>>>(
      static_cast<const bf16*>(x), ld, 1, rows, K, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_quant_heads(const void* x, int64_t ld, int64_t T, int H, int d,
                                 uint8_t* codes, int64_t ld_codes, uint32_t* scales,
                                 hipStream_t st) {
  if (T <= 0 || H <= 0) return hipSuccess;
  if (d % 32 || d > 128 || H > 64 || ld < (int64_t)H * d || (ld % 8) ||
      ld_codes < (int64_t)H * d ||
      (ld_codes % 16) || (reinterpret_cast<uintptr_t>(x) & 15) ||
      (reinterpret_cast<uintptr_t>(codes) & 15) || (reinterpret_cast<uintptr_t>(scales) & 3))
    return hipErrorInvalidValue;
  const int64_t groups = (T + MXH_ROWS - 1) / MXH_ROWS;
  k_mx_quant_heads<<<(unsigned)std::min<int64_t>(groups, 8192), 256, 0, st>>>(
      static_cast<const bf16*>(x), ld, T, H, d, codes, ld_codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_quant_rows_t(const void* x, int64_t ld, int64_t T, int64_t C, int64_t Tp,
                                  uint8_t* codes, uint8_t* scales, hipStream_t st) {
  if (C <= 0 || Tp <= 0) return hipSuccess;
  if (C % 64 || Tp % 128 || Tp < T || ld < C || (ld % 8) ||
      (reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(codes) & 15))
    return hipErrorInvalidValue;
  k_mx_quant_t<false><<<dim3((unsigned)(Tp / 128), (unsigned)(C / 64)), 256, 0, st>>>(
      static_cast<const bf16*>(x), ld, T, C, Tp, codes, scales, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_mx_quant_both(const void* x, int64_t ld, int64_t T, int64_t C, int64_t Tp,
                                uint8_t* codes, uint8_t* scales, uint8_t* rcodes,
                                uint8_t* rscales, hipStream_t st) {
  if (C <= 0 || Tp <= 0) return hipSuccess;
  if (C % 64 || Tp % 128 || Tp < T || ld < C || (ld % 8) ||
      (reinterpret_cast<uintptr_t>(x) & 15) || (reinterpret_cast<uintptr_t>(codes) & 15) ||
      (reinterpret_cast<uintptr_t>(rcodes) & 15))
    return hipErrorInvalidValue;
  k_mx_quant_t<true><<<dim3((unsigned)(Tp / 128), (unsigned)(C / 64)), 256, 0, st>>>(
      static_cast<const bf16*>(x), ld, T, C, Tp, codes, scales, rcodes, rscales);
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
