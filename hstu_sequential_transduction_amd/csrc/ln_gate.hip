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
#include "mx.h"

#include <type_traits>

namespace hstu {

namespace {

template <typename T>
HSTU_DEV float ldf(const T* p) { return (float)(*p); }

// Row chunk loads/stores.  With VEC (every lane's EPL elements inside the
// row and 16-byte aligned rows; checked on the host) a lane moves its chunk
// with 16- or 8-byte accesses; otherwise element by element with bounds checks.
HSTU_DEV void unpack4(const uint32_t* w, float* x, int nw, bool bf) {
  for (int i = 0; i < nw; ++i) {
    if (bf) {
      x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    } else {
      x[i] = __builtin_bit_cast(float, w[i]);
    }
  }
}

template <int EPL, bool VEC, typename T>
HSTU_DEV void load_row(const T* row, int c0, int W, float* x) {
  constexpr int BYTES = EPL * (int)sizeof(T);
  constexpr bool BF = sizeof(T) == 2;
  if constexpr (VEC && BYTES % 16 == 0) {
#pragma unroll
    for (int q = 0; q < BYTES / 16; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(row + c0) + 16 * q);
      const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
      unpack4(w, x + q * (BF ? 8 : 4), 4, BF);
    }
  } else if constexpr (VEC && BYTES == 8) {
    const uint2 v = *reinterpret_cast<const uint2*>(row + c0);
    const uint32_t w[2] = {v.x, v.y};
    unpack4(w, x, 2, BF);
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = (c0 + e < W) ? (float)row[c0 + e] : 0.0f;
  }
}

HSTU_DEV uint32_t packw(const float* x, int i, bool bf) {
  return bf ? pack_bf16x2(x[2 * i], x[2 * i + 1]) : __builtin_bit_cast(uint32_t, x[i]);
}

template <int EPL, bool VEC, typename T>
HSTU_DEV void store_row(T* row, int c0, int W, const float* x) {
  constexpr int BYTES = EPL * (int)sizeof(T);
  constexpr bool BF = sizeof(T) == 2;
  if constexpr (VEC && BYTES % 16 == 0) {
#pragma unroll
    for (int q = 0; q < BYTES / 16; ++q) {
      const float* xq = x + q * (BF ? 8 : 4);
      const u32x4 v = {packw(xq, 0, BF), packw(xq, 1, BF), packw(xq, 2, BF), packw(xq, 3, BF)};
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint8_t*>(row + c0) + 16 * q) = v;
    }
  } else if constexpr (VEC && BYTES == 8) {
    uint2 v;
    v.x = packw(x, 0, BF);
    v.y = packw(x, 1, BF);
    *reinterpret_cast<uint2*>(row + c0) = v;
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      if (c0 + e < W) row[c0 + e] = (T)x[e];
  }
}

// A lane's chunk of a row kept as loaded (16-byte words), for loads issued
// ahead of their use: unpacking to fp32 would make the load complete first.
template <int EPL, typename T>
struct RawChunk {
  static constexpr int NQ = EPL * (int)sizeof(T) / 16;
  u32x4 w[NQ];
};
template <int EPL, typename T>
HSTU_DEV void load_raw(const T* row, int c0, RawChunk<EPL, T>& r) {
#pragma unroll
  for (int q = 0; q < RawChunk<EPL, T>::NQ; ++q)
    r.w[q] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(row + c0) + 16 * q);
}
template <int EPL, typename T>
HSTU_DEV void unpack_raw(const RawChunk<EPL, T>& r, float* x) {
  constexpr bool BF = sizeof(T) == 2;
#pragma unroll
  for (int q = 0; q < RawChunk<EPL, T>::NQ; ++q) {
    const uint32_t w[4] = {r.w[q][0], r.w[q][1], r.w[q][2], r.w[q][3]};
    unpack4(w, x + q * (BF ? 8 : 4), 4, BF);
  }
}

template <int EPL, bool VEC, typename T, typename TO, bool MXO = false>
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
  // two adjacent rows per wave and iteration: both rows' loads are in flight
  // together, and the whole grid sweeps one contiguous stretch of rows
  const int64_t step = (int64_t)gridDim.x * 4;
  for (int64_t r0 = 2 * ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)); r0 < a.T; r0 += 2 * step) {
    const int64_t rr[2] = {r0, r0 + 1};
    float x[2][EPL], u[2][EPL];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (rr[k] < a.T) {
        load_row<EPL, VEC>(O + rr[k] * a.ld_o, c0, W, x[k]);
        load_row<EPL, VEC>(U + rr[k] * a.ld_u, c0, W, u[k]);
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (rr[k] >= a.T) break;
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s += x[k][e];
      const float mean = wave_sum(s) * invW;
      float v = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float d = (c0 + e < W) ? x[k][e] - mean : 0.0f;
        v = fmaf(d, d, v);
      }
      const float var = wave_sum(v) * invW;
      const float rstd = 1.0f / sqrtf(var + a.eps);
      float gv[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e)
        gv[e] = fmaf((x[k][e] - mean) * rstd, gam[e], bet[e]) * u[k][e];
      if constexpr (MXO) {
        // MXFP8 of the bf16-rounded G: a 32-value block spans 32 / EPL lanes
        constexpr int LPB = 32 / EPL;
        float am = 0.0f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          gv[e] = (float)(bf16)gv[e];
          am = fmaxf(am, fabsf(gv[e]));
        }
#pragma unroll
        for (int o = 1; o < LPB; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
        const int sh = mx_shared_exp(am);
        uint32_t cw[EPL / 4];
#pragma unroll
        for (int q = 0; q < EPL / 4; ++q)
          cw[q] = mx_cvt4(gv[4 * q], gv[4 * q + 1], gv[4 * q + 2], gv[4 * q + 3], sh);
        uint8_t* dst = a.g_codes + rr[k] * W + c0;
        if constexpr (EPL == 4) {
          *reinterpret_cast<uint32_t*>(dst) = cw[0];
        } else if constexpr (EPL == 8) {
          *reinterpret_cast<uint2*>(dst) = uint2{cw[0], cw[1]};
        } else {
#pragma unroll
          for (int q = 0; q < EPL / 16; ++q)
            reinterpret_cast<u32x4*>(dst)[q] = u32x4{cw[4 * q], cw[4 * q + 1], cw[4 * q + 2], cw[4 * q + 3]};
        }
        if (lane % LPB == 0) a.g_scales[rr[k] * (W / 32) + c0 / 32] = (uint8_t)(sh + 127);
        // training keeps the bf16 G as well (the backward's dW2 = G^T dY)
        if (G) store_row<EPL, VEC>(G + rr[k] * a.ld_g, c0, W, gv);
      } else {
        store_row<EPL, VEC>(G + rr[k] * a.ld_g, c0, W, gv);
      }
      if (lane == 0) {
        if (a.mu) a.mu[rr[k]] = mean;
        if (a.rstd) a.rstd[rr[k]] = rstd;
      }
    }
  }
}

template <int EPL, bool VEC, typename T, typename TO>
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
  // Two adjacent rows per wave and iteration (as in the forward).
  const int64_t step = (int64_t)gridDim.x * 4;
  auto process = [&](const float (&x)[2][EPL], const float (&u)[2][EPL], const float (&dg)[2][EPL],
                     const float (&z)[2][EPL], const float (&mean)[2], const float (&rstd)[2],
                     int64_t r0) HSTU_INLINE_LAMBDA {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int64_t r = r0 + k;
      if (r >= a.T) break;
      float xh[EPL], dxh[EPL], du[EPL];
      float s1 = 0.0f, s2 = 0.0f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        xh[e] = (c0 + e < W) ? (x[k][e] - mean[k]) * rstd[k] : 0.0f;
        const float y = fmaf(xh[e], gam[e], bet[e]);
        du[e] = dg[k][e] * y;
        const float dy = dg[k][e] * u[k][e];
        pg[e] = fmaf(dy, xh[e], pg[e]);
        pb[e] += dy;
        dxh[e] = dy * gam[e];
        s1 += dxh[e];
        s2 = fmaf(dxh[e], xh[e], s2);
      }
      const float m1 = wave_sum(s1) * invW, m2 = wave_sum(s2) * invW;
      float dx[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) dx[e] = rstd[k] * (dxh[e] - m1 - xh[e] * m2);
      if (zu) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) du[e] *= silu_grad_f(z[k][e]);
      }
      store_row<EPL, VEC>(dU + r * a.ld_du, c0, W, du);
      store_row<EPL, VEC>(dO + r * a.ld_do, c0, W, dx);
    }
  };
  int64_t r0 = 2 * ((int64_t)blockIdx.x * 4 + wave);
  constexpr bool RAW = VEC && EPL <= 8 && (EPL * sizeof(T)) % 16 == 0 &&
                       (EPL * sizeof(TO)) % 16 == 0;
  if constexpr (RAW) {
    // The next iteration's rows are loaded, as raw 16-byte words, before the
    // current ones are computed (register sets A and B in turn), so a wave
    // always has loads in flight while it computes and stores.
    struct Raw {
      RawChunk<EPL, TO> x[2];
      RawChunk<EPL, T> u[2], dg[2], z[2];
      float mean[2], rstd[2];
    };
    auto load = [&](Raw& R, int64_t rb) HSTU_INLINE_LAMBDA {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        // rows past the end repeat the last row (loaded, never used)
        const int64_t r = rb + k < a.T ? rb + k : a.T - 1;
        load_raw<EPL, TO>(O + r * a.ld_o, c0, R.x[k]);
        load_raw<EPL, T>(U + r * a.ld_u, c0, R.u[k]);
        load_raw<EPL, T>(dG + r * a.ld_dg, c0, R.dg[k]);
        if (zu) load_raw<EPL, T>(zu + r * a.ld_zu, c0, R.z[k]);
        R.mean[k] = a.mu[r];
        R.rstd[k] = a.rstd[r];
      }
    };
    auto run = [&](const Raw& R, int64_t rb) HSTU_INLINE_LAMBDA {
      float x[2][EPL], u[2][EPL], dg[2][EPL], z[2][EPL];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        unpack_raw<EPL, TO>(R.x[k], x[k]);
        unpack_raw<EPL, T>(R.u[k], u[k]);
        unpack_raw<EPL, T>(R.dg[k], dg[k]);
        if (zu) unpack_raw<EPL, T>(R.z[k], z[k]);
      }
      process(x, u, dg, z, R.mean, R.rstd, rb);
    };
    Raw A, B;
    if (r0 < a.T) load(A, r0);
    while (r0 < a.T) {
      if (r0 + 2 * step < a.T) load(B, r0 + 2 * step);
      run(A, r0);
      r0 += 2 * step;
      if (r0 >= a.T) break;
      if (r0 + 2 * step < a.T) load(A, r0 + 2 * step);
      run(B, r0);
      r0 += 2 * step;
    }
  } else {
    for (; r0 < a.T; r0 += 2 * step) {
      float x[2][EPL], u[2][EPL], dg[2][EPL], z[2][EPL];
      float mean[2] = {0.f, 0.f}, rstd[2] = {0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        if (r0 + k < a.T) {
          load_row<EPL, VEC>(O + (r0 + k) * a.ld_o, c0, W, x[k]);
          load_row<EPL, VEC>(U + (r0 + k) * a.ld_u, c0, W, u[k]);
          load_row<EPL, VEC>(dG + (r0 + k) * a.ld_dg, c0, W, dg[k]);
          if (zu) load_row<EPL, VEC>(zu + (r0 + k) * a.ld_zu, c0, W, z[k]);
          mean[k] = a.mu[r0 + k];
          rstd[k] = a.rstd[r0 + k];
        }
      }
      process(x, u, dg, z, mean, rstd, r0);
    }
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

// The vector path needs every lane's chunk inside the row (W = 64 * EPL),
// 8- or 16-byte chunks, and 16-byte aligned rows of every tensor.
template <typename T, typename TO>
bool vec_ok(const LnArgs& a, int epl) {
  if (a.W != 64 * epl) return false;
  const int bt = epl * (int)sizeof(T), bo = epl * (int)sizeof(TO);
  if (!(bt == 8 || bt % 16 == 0) || !(bo == 8 || bo % 16 == 0)) return false;
  auto ok = [](const void* p, int64_t ld, size_t es) {
    return !p || ((reinterpret_cast<uintptr_t>(p) & 15) == 0 && ((uint64_t)ld * es) % 16 == 0);
  };
  return ok(a.O, a.ld_o, sizeof(TO)) && ok(a.U, a.ld_u, sizeof(T)) && ok(a.G, a.ld_g, sizeof(T)) &&
         ok(a.dG, a.ld_dg, sizeof(T)) && ok(a.zu, a.ld_zu, sizeof(T)) &&
         ok(a.dU, a.ld_du, sizeof(T)) && ok(a.dO, a.ld_do, sizeof(T));
}

#define HSTU_LN_CASES(K, T, TO, VEC, grid)                                    \
  switch (epl_for(a.W)) {                                                    \
    case 1: K<1, VEC, T, TO><<<grid, 256, 0, st>>>(a); break;                \
    case 2: K<2, VEC, T, TO><<<grid, 256, 0, st>>>(a); break;                \
    case 4: K<4, VEC, T, TO><<<grid, 256, 0, st>>>(a); break;                \
    case 8: K<8, VEC, T, TO><<<grid, 256, 0, st>>>(a); break;                \
    case 16: K<16, VEC, T, TO><<<grid, 256, 0, st>>>(a); break;              \
    default: return hipErrorInvalidValue;                                    \
  }

template <typename T, typename TO>
hipError_t fwd_t(const LnArgs& a, hipStream_t st) {
  int64_t blocks = (a.T + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  if (blocks <= 0) return hipSuccess;
  const unsigned grid = (unsigned)blocks;
  if (a.g_codes) {
    // MXFP8 output: bf16, whole rows of 4, 8 or 16 values per lane
    if (!std::is_same<T, bf16>::value || !vec_ok<T, TO>(a, epl_for(a.W)) || !a.g_scales)
      return hipErrorInvalidValue;
    switch (epl_for(a.W)) {
      case 4: k_ln_gate_fwd<4, true, T, TO, true><<<grid, 256, 0, st>>>(a); break;
      case 8: k_ln_gate_fwd<8, true, T, TO, true><<<grid, 256, 0, st>>>(a); break;
      case 16: k_ln_gate_fwd<16, true, T, TO, true><<<grid, 256, 0, st>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  } else if (vec_ok<T, TO>(a, epl_for(a.W))) {
    HSTU_LN_CASES(k_ln_gate_fwd, T, TO, true, grid)
  } else {
    HSTU_LN_CASES(k_ln_gate_fwd, T, TO, false, grid)
  }
  return hipGetLastError();
}

template <typename T, typename TO>
hipError_t bwd_t(const LnArgs& a, hipStream_t st) {
  const int64_t blocks = a.n_part_blocks;
  if (blocks <= 0) return hipSuccess;
  const unsigned grid = (unsigned)blocks;
  if (vec_ok<T, TO>(a, epl_for(a.W))) {
    HSTU_LN_CASES(k_ln_gate_bwd, T, TO, true, grid)
  } else {
    HSTU_LN_CASES(k_ln_gate_bwd, T, TO, false, grid)
  }
  return hipGetLastError();
}

}  // namespace

// Workgroups of the backward (each writes one row of dgamma/dbeta partials):
// 512, two per CU, measured faster than 1024 or 2048 on 49K rows of 512.
int64_t ln_bwd_part_blocks(int64_t T) {
  int64_t b = (T + 3) / 4;
  if (b > 512) b = 512;
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
