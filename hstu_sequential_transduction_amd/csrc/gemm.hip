// Dense GEMMs of the HSTU layer: the U|V|Q|K projection (with the SiLU in the
// epilogue), the output projection (bias + residual in the epilogue) and the
// weight/input gradients of both ("DLRMv4 Brings Sequence-Based
// Recommendation Training to MLPerf", Table 7: the UVQK and output-projection
// GEMM rows, three GEMMs each for forward plus backward).
//
// bf16 kernel: 128x128 output tile, k-step 64, four waves each owning a
// 64x64 quadrant as 2x2 blocks of 32x32x16 MFMA.  Operands are staged in LDS
// as [row][k] tiles; an operand whose k index is not the contiguous one is
// transposed while it is staged (pairs of k rows packed into dwords, rows
// XOR-swizzled to spread the banks), so one kernel covers X W, G W^T-style
// and X^T dZ-style products without separate transpose passes.  Global loads
// of the next k-step are issued before the MFMAs of the current one.
#include "common.h"
#include "internal.h"

namespace hstu {

namespace {

constexpr int GBM = 128, GBN = 128, GBK = 64;
using GT = LdsTile<GBK>;

struct GemmSmem {
  uint32_t a[GT::S_DW * GBM];
  uint32_t b[GT::S_DW * GBN];
};

// Register staging of one operand tile: R rows (m or n) x 64 k.
template <bool KCONT, int R>
struct Stage {
  // k-contiguous: R*8 chunks of 16 B; transposed: 32 k-pairs x R/8 chunks, two loads each
  static constexpr int NLD = KCONT ? (R * 8) / 256 : (32 * (R / 8) * 2) / 256;
  u32x4 v[NLD];

  HSTU_DEV void load(const bf16* base, int64_t ld, int64_t r0, int64_t k0, int64_t Rmax,
                     int64_t Kmax, int tid) {
    if (KCONT) {
#pragma unroll
      for (int s = 0; s < NLD; ++s) {
        const int idx = tid + 256 * s;
        const int row = idx >> 3, ch = idx & 7;
        const int64_t rr = r0 + row, kk = k0 + ch * 8;
        v[s] = (rr < Rmax && kk < Kmax) ? ld16(base + rr * ld + kk) : u32x4{0, 0, 0, 0};
      }
    } else {
#pragma unroll
      for (int s = 0; s < NLD / 2; ++s) {
        const int idx = tid + 256 * s;
        const int rest = idx >> 6;
        const int kp = (rest & 3) * 8 + ((idx >> 3) & 7);
        const int cc = (rest >> 2) * 8 + (idx & 7);
        const int64_t kk = k0 + 2 * kp, rr = r0 + cc * 8;
        v[2 * s] = (kk < Kmax && rr < Rmax) ? ld16(base + kk * ld + rr) : u32x4{0, 0, 0, 0};
        v[2 * s + 1] =
            (kk + 1 < Kmax && rr < Rmax) ? ld16(base + (kk + 1) * ld + rr) : u32x4{0, 0, 0, 0};
      }
    }
  }
  HSTU_DEV void store(uint32_t* lds, int tid) const {
    if (KCONT) {
#pragma unroll
      for (int s = 0; s < NLD; ++s) {
        const int idx = tid + 256 * s;
        const int row = idx >> 3, ch = idx & 7;
        *reinterpret_cast<u32x4*>(&lds[GT::off(row, ch * 4)]) = v[s];
      }
    } else {
#pragma unroll
      for (int s = 0; s < NLD / 2; ++s) {
        const int idx = tid + 256 * s;
        const int rest = idx >> 6;
        const int kp = (rest & 3) * 8 + ((idx >> 3) & 7);
        const int cc = (rest >> 2) * 8 + (idx & 7);
        const u32x4 va = v[2 * s], vb = v[2 * s + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lds[GT::off(cc * 8 + 2 * e, kp)] = (va[e] & 0xFFFFu) | (vb[e] << 16);
          lds[GT::off(cc * 8 + 2 * e + 1, kp)] = (va[e] >> 16) | (vb[e] & 0xFFFF0000u);
        }
      }
    }
  }
};

template <bool AK, bool BK, int EPI, bool OUTF32>
__global__ __launch_bounds__(256, 2) void k_gemm_bf16(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) GemmSmem sm;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, gq = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * GBM, n0 = (int64_t)blockIdx.x * GBN;
  const bf16* A = reinterpret_cast<const bf16*>(g.A);
  const bf16* B = reinterpret_cast<const bf16*>(g.B);

  int64_t kbeg = 0, kend = g.K;
  if (EPI == EPI_PARTIAL) {
    const int64_t per = ((g.K + g.split_k - 1) / g.split_k + GBK - 1) / GBK * GBK;
    kbeg = (int64_t)blockIdx.z * per;
    kend = kbeg + per < g.K ? kbeg + per : g.K;
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  Stage<AK, GBM> sa;
  Stage<BK, GBN> sb;
  if (kbeg < kend) {
    sa.load(A, g.lda, m0, kbeg, g.M, kend, tid);
    sb.load(B, g.ldb, n0, kbeg, g.N, kend, tid);
  }
  for (int64_t k0 = kbeg; k0 < kend; k0 += GBK) {
    __syncthreads();
    sa.store(sm.a, tid);
    sb.store(sm.b, tid);
    __syncthreads();
    if (k0 + GBK < kend) {
      sa.load(A, g.lda, m0, k0 + GBK, g.M, kend, tid);
      sb.load(B, g.ldb, n0, k0 + GBK, g.N, kend, tid);
    }
#pragma unroll
    for (int kc = 0; kc < GBK / 16; ++kc) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(
            &sm.a[GT::off(wm * 64 + i * 32 + ql, kc * 8 + 4 * gq)]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(
            &sm.b[GT::off(wn * 64 + j * 32 + ql, kc * 8 + 4 * gq)]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
  }

  // epilogue: lane holds rows m0 + wm*64 + i*32 + 8*(r/4) + 4*gq + r%4, column n0 + wn*64 + j*32 + ql
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t n = n0 + wn * 64 + j * 32 + ql;
    if (n >= g.N) continue;
    const float bias = (g.bias && (EPI == EPI_SILU || EPI == EPI_RESID)) ? g.bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * gq + (r & 3);
        if (m >= g.M) continue;
        float v = acc[i][j][r];
        if (EPI == EPI_PARTIAL) {
          g.partial[((int64_t)blockIdx.z * g.M + m) * g.N + n] = v;
        } else if (EPI == EPI_SILU) {
          v += bias;
          if (g.C2) reinterpret_cast<bf16*>(g.C2)[m * g.ldc + n] = (bf16)v;
          reinterpret_cast<bf16*>(g.C)[m * g.ldc + n] = (bf16)silu_f(v);
        } else {
          if (EPI == EPI_RESID) {
            v += bias;
            if (g.R) v += (float)reinterpret_cast<const bf16*>(g.R)[m * g.ldr + n];
          }
          if (OUTF32) reinterpret_cast<float*>(g.C)[m * g.ldc + n] = v;
          else reinterpret_cast<bf16*>(g.C)[m * g.ldc + n] = (bf16)v;
        }
      }
    }
  }
}

// fp32 GEMM on the VALU: 64x64 tile, 4x4 outputs per thread, k-step 16.
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmArgs g) {
  __shared__ float as[16][64 + 1], bs[16][64 + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = (int64_t)blockIdx.y * 64, n0 = (int64_t)blockIdx.x * 64;
  const float* A = reinterpret_cast<const float*>(g.A);
  const float* B = reinterpret_cast<const float*>(g.B);
  int64_t kbeg = 0, kend = g.K;
  if (EPI == EPI_PARTIAL) {
    const int64_t per = ((g.K + g.split_k - 1) / g.split_k + 15) / 16 * 16;
    kbeg = (int64_t)blockIdx.z * per;
    kend = kbeg + per < g.K ? kbeg + per : g.K;
  }
  float acc[4][4] = {};
  for (int64_t k0 = kbeg; k0 < kend; k0 += 16) {
    __syncthreads();
    for (int idx = tid; idx < 16 * 64; idx += 256) {
      const int kk = idx / 64, rr = idx % 64;
      const int64_t k = k0 + kk, m = m0 + rr, n = n0 + rr;
      as[kk][rr] = (k < kend && m < g.M) ? (g.a_kcont ? A[m * g.lda + k] : A[k * g.lda + m]) : 0.f;
      bs[kk][rr] = (k < kend && n < g.N) ? (g.b_kcont ? B[n * g.ldb + k] : B[k * g.ldb + n]) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = as[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
  }
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= g.M) continue;
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n >= g.N) continue;
      float v = acc[i][j];
      float* C = reinterpret_cast<float*>(g.C);
      if (EPI == EPI_PARTIAL) {
        g.partial[((int64_t)blockIdx.z * g.M + m) * g.N + n] = v;
      } else if (EPI == EPI_SILU) {
        if (g.bias) v += g.bias[n];
        if (g.C2) reinterpret_cast<float*>(g.C2)[m * g.ldc + n] = v;
        C[m * g.ldc + n] = v / (1.0f + __expf(-v));
      } else {
        if (EPI == EPI_RESID) {
          if (g.bias) v += g.bias[n];
          if (g.R) v += reinterpret_cast<const float*>(g.R)[m * g.ldr + n];
        }
        C[m * g.ldc + n] = v;
      }
    }
  }
}

template <bool AK, bool BK>
hipError_t gemm_bf16_ab(const GemmArgs& g, hipStream_t st) {
  dim3 grid((unsigned)((g.N + GBN - 1) / GBN), (unsigned)((g.M + GBM - 1) / GBM),
            (unsigned)(g.epi == EPI_PARTIAL ? g.split_k : 1));
  switch (g.epi) {
    case EPI_STORE:
      if (g.c_f32) k_gemm_bf16<AK, BK, EPI_STORE, true><<<grid, 256, 0, st>>>(g);
      else k_gemm_bf16<AK, BK, EPI_STORE, false><<<grid, 256, 0, st>>>(g);
      break;
    case EPI_SILU: k_gemm_bf16<AK, BK, EPI_SILU, false><<<grid, 256, 0, st>>>(g); break;
    case EPI_RESID:
      if (g.c_f32) k_gemm_bf16<AK, BK, EPI_RESID, true><<<grid, 256, 0, st>>>(g);
      else k_gemm_bf16<AK, BK, EPI_RESID, false><<<grid, 256, 0, st>>>(g);
      break;
    case EPI_PARTIAL: k_gemm_bf16<AK, BK, EPI_PARTIAL, true><<<grid, 256, 0, st>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

__global__ void k_splitk_reduce(const float* __restrict__ part, int split, int64_t M, int64_t N,
                                float* __restrict__ out, int64_t ldo) {
  const int64_t total = M * N;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.0f;
    for (int z = 0; z < split; ++z) s += part[z * total + i];
    const int64_t m = i / N, n = i % N;
    out[m * ldo + n] = s;
  }
}

// Column sums: stage 1 writes per-block partials [blocks][cols], stage 2 sums them.
template <typename T>
__global__ void k_colsum_part(const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
                              int64_t rows_per_block, float* __restrict__ part) {
  const int64_t r0 = blockIdx.y * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < cols;
       c += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.0f;
    for (int64_t r = r0; r < r1; ++r) s += (float)x[r * ld + c];
    part[blockIdx.y * cols + c] = s;
  }
}
__global__ void k_colsum_final(const float* __restrict__ part, int nb, int64_t cols,
                               float* __restrict__ out) {
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < cols;
       c += (int64_t)gridDim.x * blockDim.x) {
    float s = 0.0f;
    for (int z = 0; z < nb; ++z) s += part[z * cols + c];
    out[c] = s;
  }
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, int dtype, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (dtype == HSTU_BF16) {
    if (g.a_kcont && g.b_kcont) return gemm_bf16_ab<true, true>(g, st);
    if (g.a_kcont && !g.b_kcont) return gemm_bf16_ab<true, false>(g, st);
    if (!g.a_kcont && g.b_kcont) return gemm_bf16_ab<false, true>(g, st);
    return gemm_bf16_ab<false, false>(g, st);
  }
  dim3 grid((unsigned)((g.N + 63) / 64), (unsigned)((g.M + 63) / 64),
            (unsigned)(g.epi == EPI_PARTIAL ? g.split_k : 1));
  switch (g.epi) {
    case EPI_STORE: k_gemm_f32<EPI_STORE><<<grid, 256, 0, st>>>(g); break;
    case EPI_SILU: k_gemm_f32<EPI_SILU><<<grid, 256, 0, st>>>(g); break;
    case EPI_RESID: k_gemm_f32<EPI_RESID><<<grid, 256, 0, st>>>(g); break;
    case EPI_PARTIAL: k_gemm_f32<EPI_PARTIAL><<<grid, 256, 0, st>>>(g); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float* partial, int split, int64_t M, int64_t N,
                                float* out, int64_t ldo, hipStream_t st) {
  const int64_t total = M * N;
  if (total <= 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  k_splitk_reduce<<<(unsigned)blocks, 256, 0, st>>>(partial, split, M, N, out, ldo);
  return hipGetLastError();
}

hipError_t launch_colsum(const void* x, int64_t rows, int64_t cols, int64_t ld, int dtype,
                         float* out, float* ws, hipStream_t st) {
  if (cols <= 0) return hipSuccess;
  const int64_t nb = 64;
  const int64_t rpb = (rows + nb - 1) / nb;
  dim3 g1((unsigned)((cols + 255) / 256), (unsigned)nb);
  if (dtype == HSTU_BF16)
    k_colsum_part<bf16><<<g1, 256, 0, st>>>(reinterpret_cast<const bf16*>(x), rows, cols, ld,
                                            rpb > 0 ? rpb : 1, ws);
  else
    k_colsum_part<float><<<g1, 256, 0, st>>>(reinterpret_cast<const float*>(x), rows, cols, ld,
                                             rpb > 0 ? rpb : 1, ws);
  k_colsum_final<<<(unsigned)((cols + 255) / 256), 256, 0, st>>>(ws, (int)nb, cols, out);
  return hipGetLastError();
}

}  // namespace hstu
