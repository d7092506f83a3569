// LayerNorm + U-gating epilogue of the HSTU layer, forward and backward.
//
// G = LayerNorm(O) * U over each token's H*d_v vector (elementwise gating
// before the output projection: NVIDIA generative-recommenders summary,
// "HSTU Architecture: Efficient Attention for User History"; the gated
// transformation of "DLRMv4 Brings Sequence-Based Recommendation Training to
// MLPerf", "Model Architecture").  Biased variance, eps, optional gamma/beta.
//
// Bandwidth-bound: one wave per token row, each lane holding EPL consecutive
// elements (16-byte loads at EPL = 8 in bf16), wave-wide shuffles for the two
// reductions, and a grid-stride loop over rows.  The backward also writes
// dU (optionally times SiLU'(Z_U), the projection's activation derivative)
// and per-workgroup partial column sums for dgamma/dbeta.
#include "common.h"
#include "internal.h"

namespace hstu {

namespace {

template <typename T>
HSTU_DEV float ldf(const T* p) { return (float)(*p); }

template <int EPL, typename T>
HSTU_DEV void load_row(const T* row, int c0, int W, float* x) {
#pragma unroll
  for (int e = 0; e < EPL; ++e) x[e] = (c0 + e < W) ? (float)row[c0 + e] : 0.0f;
}

template <int EPL, typename T>
HSTU_DEV void store_row(T* row, int c0, int W, const float* x) {
#pragma unroll
  for (int e = 0; e < EPL; ++e)
    if (c0 + e < W) row[c0 + e] = (T)x[e];
}

template <int EPL, typename T, typename TO>
__global__ __launch_bounds__(256) void k_ln_gate_fwd(LnArgs a) {
  const int lane = threadIdx.x & 63;
  const int W = a.W;
  const int c0 = lane * EPL;
  const TO* O = reinterpret_cast<const TO*>(a.O);
  const T* U = reinterpret_cast<const T*>(a.U);
  T* G = reinterpret_cast<T*>(a.G);
  const float invW = 1.0f / (float)W;
  float gam[EPL], bet[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    gam[e] = (a.gamma && c0 + e < W) ? a.gamma[c0 + e] : 1.0f;
    bet[e] = (a.beta && c0 + e < W) ? a.beta[c0 + e] : 0.0f;
  }
  for (int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); r < a.T;
       r += (int64_t)gridDim.x * 4) {
    float x[EPL], u[EPL];
    load_row<EPL>(O + r * a.ld_o, c0, W, x);
    load_row<EPL>(U + r * a.ld_u, c0, W, u);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) s += x[e];
    const float mean = wave_sum(s) * invW;
    float v = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const float d = (c0 + e < W) ? x[e] - mean : 0.0f;
      v = fmaf(d, d, v);
    }
    const float var = wave_sum(v) * invW;
    const float rstd = 1.0f / sqrtf(var + a.eps);
    float gv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) gv[e] = fmaf((x[e] - mean) * rstd, gam[e], bet[e]) * u[e];
    store_row<EPL>(G + r * a.ld_g, c0, W, gv);
    if (lane == 0) {
      if (a.mu) a.mu[r] = mean;
      if (a.rstd) a.rstd[r] = rstd;
    }
  }
}

template <int EPL, typename T, typename TO>
__global__ __launch_bounds__(256) void k_ln_gate_bwd(LnArgs a) {
  __shared__ float sg[4][64 * EPL], sb[4][64 * EPL];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int W = a.W;
  const int c0 = lane * EPL;
  const TO* O = reinterpret_cast<const TO*>(a.O);
  const T* U = reinterpret_cast<const T*>(a.U);
  const T* dG = reinterpret_cast<const T*>(a.dG);
  const T* zu = reinterpret_cast<const T*>(a.zu);
  T* dU = reinterpret_cast<T*>(a.dU);
  T* dO = reinterpret_cast<T*>(a.dO);
  const float invW = 1.0f / (float)W;
  float gam[EPL], bet[EPL], pg[EPL], pb[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    gam[e] = (a.gamma && c0 + e < W) ? a.gamma[c0 + e] : 1.0f;
    bet[e] = (a.beta && c0 + e < W) ? a.beta[c0 + e] : 0.0f;
    pg[e] = 0.0f;
    pb[e] = 0.0f;
  }
  for (int64_t r = (int64_t)blockIdx.x * 4 + wave; r < a.T; r += (int64_t)gridDim.x * 4) {
    float x[EPL], u[EPL], dg[EPL];
    load_row<EPL>(O + r * a.ld_o, c0, W, x);
    load_row<EPL>(U + r * a.ld_u, c0, W, u);
    load_row<EPL>(dG + r * a.ld_dg, c0, W, dg);
    const float mean = a.mu[r], rstd = a.rstd[r];
    float xh[EPL], dxh[EPL], du[EPL];
    float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      xh[e] = (c0 + e < W) ? (x[e] - mean) * rstd : 0.0f;
      const float y = fmaf(xh[e], gam[e], bet[e]);
      du[e] = dg[e] * y;
      const float dy = dg[e] * u[e];
      pg[e] = fmaf(dy, xh[e], pg[e]);
      pb[e] += dy;
      dxh[e] = dy * gam[e];
      s1 += dxh[e];
      s2 = fmaf(dxh[e], xh[e], s2);
    }
    const float m1 = wave_sum(s1) * invW, m2 = wave_sum(s2) * invW;
    float dx[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) dx[e] = rstd * (dxh[e] - m1 - xh[e] * m2);
    if (zu) {
      float z[EPL];
      load_row<EPL>(zu + r * a.ld_zu, c0, W, z);
#pragma unroll
      for (int e = 0; e < EPL; ++e) du[e] *= silu_grad_f(z[e]);
    }
    store_row<EPL>(dU + r * a.ld_du, c0, W, du);
    store_row<EPL>(dO + r * a.ld_do, c0, W, dx);
  }
  if (a.dgamma_part || a.dbeta_part) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      sg[wave][c0 + e] = pg[e];
      sb[wave][c0 + e] = pb[e];
    }
    __syncthreads();
    for (int col = threadIdx.x; col < W; col += 256) {
      const float tg = sg[0][col] + sg[1][col] + sg[2][col] + sg[3][col];
      const float tb = sb[0][col] + sb[1][col] + sb[2][col] + sb[3][col];
      if (a.dgamma_part) a.dgamma_part[(int64_t)blockIdx.x * W + col] = tg;
      if (a.dbeta_part) a.dbeta_part[(int64_t)blockIdx.x * W + col] = tb;
    }
  }
}

int epl_for(int W) {
  int e = 1;
  while (64 * e < W) e <<= 1;
  return e;
}

template <typename T, typename TO>
hipError_t fwd_t(const LnArgs& a, hipStream_t st) {
  int64_t blocks = (a.T + 3) / 4;
  if (blocks > 8192) blocks = 8192;
  if (blocks <= 0) return hipSuccess;
  switch (epl_for(a.W)) {
    case 1: k_ln_gate_fwd<1, T, TO><<<(unsigned)blocks, 256, 0, st>>>(a); break;
    case 2: k_ln_gate_fwd<2, T, TO><<<(unsigned)blocks, 256, 0, st>>>(a); break;
    case 4: k_ln_gate_fwd<4, T, TO><<<(unsigned)blocks, 256, 0, st>>>(a); break;
    case 8: k_ln_gate_fwd<8, T, TO><<<(unsigned)blocks, 256, 0, st>>>(a); break;
    case 16: k_ln_gate_fwd<16, T, TO><<<(unsigned)blocks, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, typename TO>
hipError_t bwd_t(const LnArgs& a, hipStream_t st) {
  const int64_t blocks = a.n_part_blocks;
  if (blocks <= 0) return hipSuccess;
  switch (epl_for(a.W)) {
    case 1: k_ln_gate_bwd<1, T, TO><<<(unsigned)blocks, 256, 0, st>>>(a); break;
    case 2: k_ln_gate_bwd<2, T, TO><<<(unsigned)blocks, 256, 0, st>>>(a); break;
    case 4: k_ln_gate_bwd<4, T, TO><<<(unsigned)blocks, 256, 0, st>>>(a); break;
    case 8: k_ln_gate_bwd<8, T, TO><<<(unsigned)blocks, 256, 0, st>>>(a); break;
    case 16: k_ln_gate_bwd<16, T, TO><<<(unsigned)blocks, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int64_t ln_bwd_part_blocks(int64_t T) {
  int64_t b = (T + 3) / 4;
  if (b > 1024) b = 1024;
  return b < 1 ? 1 : b;
}

hipError_t launch_ln_gate_fwd(const LnArgs& a, int dtype, hipStream_t st) {
  if (dtype != HSTU_BF16) return fwd_t<float, float>(a, st);
  return a.o_f32 ? fwd_t<bf16, float>(a, st) : fwd_t<bf16, bf16>(a, st);
}
hipError_t launch_ln_gate_bwd(const LnArgs& a, int dtype, hipStream_t st) {
  if (dtype != HSTU_BF16) return bwd_t<float, float>(a, st);
  return a.o_f32 ? bwd_t<bf16, float>(a, st) : bwd_t<bf16, bf16>(a, st);
}

}  // namespace hstu
