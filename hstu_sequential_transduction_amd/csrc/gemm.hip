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
#include "lds.h"
#include "mx.h"

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

// ---------------------------------------------------------------------------
// DMA-staged bf16 GEMM, BM x BN output tile per workgroup of four waves
// (2 x 2), each wave a (BM/2) x (BN/2) block of 32x32x16 MFMAs, k-step 64.
// The layer uses 128x128 tiles with one operand stage (four workgroups per
// CU, so the DMA waits and epilogues of some overlap the main loops of the
// others), or two stages for split-K; 256x256 (one workgroup per CU, eight
// 16-byte LDS operand reads per sixteen MFMAs) is available to the template.
// Operand tiles arrive by buffer->LDS DMA into static LDS stages.  A
// k-contiguous operand is stored [rows][64 k] and read along rows; a k-major
// operand ([k][rows] in memory) is stored as [64 k][128]-column tiles and read
// down columns with transpose reads, so no operand is ever transposed in
// memory.  Workgroups are ordered so that the tiles sharing one row block of
// A run on the same XCD (workgroup w runs on XCD w % 8) and share its L2.
// ---------------------------------------------------------------------------
constexpr int G2_BK = 64;
constexpr int G2_NW = 4;  // waves: 2 (m) x 2 (n)

// DMA of one operand tile: R rows r0.. (the m or n index) x k0..k0+63
template <bool KCONT, int R>
HSTU_DEV void g2_issue(uint8_t* t, const bf16* X, int64_t ld, int64_t r0, int64_t Rmax,
                       int64_t k0, int64_t kend, int wave, int lane) {
  if (KCONT) {
    // [rows][k]: rows beyond Rmax arrive as zeros; k0 + 64 <= K (checked on the host)
    dma_tile<64, R, G2_NW>(t, X + k0, ld, (int)r0, (int)Rmax, wave, lane);
  } else {
    // [k][rows]: 128-column pieces; k rows beyond kend arrive as zeros and the
    // last k row is cut at the matrix's right edge
#pragma unroll
    for (int hf = 0; hf < R / 128; ++hf) {
      const int64_t c0 = r0 + 128 * hf;
      const int cols = (int)max<int64_t>(0, min<int64_t>(128, Rmax - c0));
      dma_tile<128, 64, G2_NW>(t + hf * (64 * 256), X + c0, ld, (int)k0, (int)kend, wave, lane,
                               cols);
    }
  }
}

// Per-lane byte offsets of a wave's MFMA operand reads within a staged tile,
// for the wave's NF x 32 rows starting at r0.  The swizzle makes the
// lane-dependent part of every address one of a few values; the rest (row
// block, k-chunk, stage) is a constant that rides in the instruction's
// immediate offset, so the whole main loop needs only these registers.
template <bool KCONT, int NF>
struct G2Off {
  int o[KCONT ? 4 : 2 * NF];
  HSTU_DEV void init(int r0, int lane) {
    const int ql = lane & 31, g = lane >> 5;
    if (KCONT) {
      // SwzTile<64>: row r0 + 32 i + ql, logical chunk 2 kc + g; the swizzle of
      // these rows depends on ql only
      const int s = SwzTile<64>::swz(ql);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) o[kc] = (r0 + ql) * 128 + (((2 * kc + g) ^ s) << 4);
    } else {
      // SwzTile<128> pieces [64 k][128]; fragment i covers columns r0 + 32 i ..,
      // k rows 16 kc + 8 g + j/4 (+4 for the upper read)
      const int j = lane & 15;
      const int cl = 2 * ((lane >> 4) & 1) + ((j & 3) >> 1);
      const int cb = (j & 1) * 8;
#pragma unroll
      for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int col = r0 + 32 * i;
          const int r = 8 * g + (j >> 2) + 4 * h;
          const int c = (col & 127) / 8 + cl;  // logical chunk (column / 8)
          o[2 * i + h] =
              (col >> 7) * (64 * 256) + r * 256 + ((c ^ SwzTile<128>::swz(r)) << 4) + cb;
        }
    }
  }
  // operand of row block i (32 rows), k-chunk kc
  HSTU_DEV bf16x8 frag(const uint8_t* t, int i, int kc) const {
    if (KCONT) {
      return *reinterpret_cast<const bf16x8*>(t + o[kc] + i * 32 * 128);
    } else {
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (HSTU_LDS bf16x4*)(t + o[2 * i] + kc * 16 * 256));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (HSTU_LDS bf16x4*)(t + o[2 * i + 1] + kc * 16 * 256));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
};

// MXFP8 operand reads from the same k-contiguous tiles (128-byte rows of E4M3
// codes).  The scaled 32x32x64 FP8 MFMA (established with an in-bounds probe)
// takes from lane half g bytes 0-15 as k = 16 g + e and bytes 16-31 as
// k = 32 + 16 g + e, and the scale of its k-block b (k in [32 b, 32 b + 32))
// from lane half b.  So for MFMA half kh (MX blocks 2 kh and 2 kh + 1 of the
// k-step) a lane reads logical chunks 4 kh + g and 4 kh + 2 + g, and its
// scale byte is that of block 2 kh + g.
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
struct G2OffMX {
  int o[4];
  HSTU_DEV void init(int r0, int lane) {
    const int ql = lane & 31, g = lane >> 5;
    const int s = SwzTile<64>::swz(ql);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      o[c] = (r0 + ql) * 128 + (((4 * (c >> 1) + 2 * (c & 1) + g) ^ s) << 4);
  }
  HSTU_DEV i32x8 frag(const uint8_t* t, int i, int kh) const {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(t + o[2 * kh] + i * 32 * 128);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(t + o[2 * kh + 1] + i * 32 * 128);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// NST operand stages: 2 = double buffer (the DMA of step k+1 runs under the
// MFMAs of step k); 1 = a single stage, which halves the LDS of a workgroup so
// that twice as many are resident and hide each other's DMA and epilogue.
template <int BM, int BN, int NST>
struct G2Shape {
  static constexpr int FM = BM / 64, FN = BN / 64;  // 32-row fragments per wave
  static constexpr int TA = BM * G2_BK * 2, TB = BN * G2_BK * 2;  // tile bytes
  static constexpr int WPC = (BM * BN >= 256 * 256 ? 1 : 2) * (NST == 1 ? 2 : 1);  // WGs per CU
};

// GEMM epilogue of one wave's (32 FM) x (32 FN) accumulator block at rows
// m0 + wm 32 FM.., columns n0 + wn 32 FN..: the accumulator layout gives each
// lane one column and rows 8*(r/4) + 4*gq + r%4, so writing it straight to
// memory would take one 2-byte store per element.  Instead the wave stages SR
// rows of its fp32 results at a time in its own LDS region `stg` (row stride
// ES floats: rows 4 apart fall on different banks), then reads rows back as
// four consecutive columns per lane and applies the epilogue in fp32 with 8-
// or 16-byte vector accesses.  The caller has every wave past its last read
// of the region's memory.  z: the split of EPI_PARTIAL.
template <int FM, int FN, int EPI, bool OUTF32, bool MX, int SR>
HSTU_DEV void g2_epilogue(const GemmArgs& g, f32x16 (&acc)[FM][FN], float* stg, int64_t m0,
                          int64_t n0, int wm, int wn, int lane, int z) {
  constexpr int WN = 32 * FN;        // columns of the wave's block
  constexpr int ES = WN + 8;         // staging row stride (floats)
  constexpr int LPR = WN / 4;        // lanes per staged row
  constexpr int RPI = 64 / LPR;      // rows per read instruction
  constexpr int GPR = SR / 8;  // accumulator register groups (of four) per round
  const int ql = lane & 31, gq = lane >> 5;
  const int lr = lane / LPR, lc = lane % LPR;
  const int64_t ncol = n0 + wn * WN + 4 * lc;  // this lane's four output columns
  float bias4[4] = {0.f, 0.f, 0.f, 0.f};
  if (g.bias && (EPI == EPI_SILU || EPI == EPI_RESID)) {
#pragma unroll
    for (int e = 0; e < 4; ++e) bias4[e] = ncol + e < g.N ? g.bias[ncol + e] : 0.0f;
  }
  const bool vec = ncol + 3 < g.N;
  // Residual (EPI_RESID): every load of the wave's block is issued here, ahead
  // of the staging rounds, so one memory latency is paid per workgroup
  // instead of one per round (the accumulators' operand registers are free)
  constexpr int NRND = FM * (32 / SR), NRR = SR / RPI;
  uint2 rres[EPI == EPI_RESID ? NRND : 1][EPI == EPI_RESID ? NRR : 1];
  if constexpr (EPI == EPI_RESID) {
    if (g.R && vec) {
#pragma unroll
      for (int ih = 0; ih < NRND; ++ih)
#pragma unroll
        for (int rr = 0; rr < NRR; ++rr) {
          const int64_t m = m0 + wm * 32 * FM + (ih / (32 / SR)) * 32 + (ih % (32 / SR)) * SR +
                            RPI * rr + lr;
          rres[ih][rr] = m < g.M ? *reinterpret_cast<const uint2*>(
                                       reinterpret_cast<const bf16*>(g.R) + m * g.ldr + ncol)
                                 : uint2{0u, 0u};
        }
    }
  }
#pragma unroll
  for (int ih = 0; ih < NRND; ++ih) {
    const int i = ih / (32 / SR), hh = ih % (32 / SR);
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < GPR; ++q)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          stg[(8 * q + 4 * gq + rr) * ES + j * 32 + ql] = acc[i][j][4 * (hh * GPR + q) + rr];
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int rr = 0; rr < SR / RPI; ++rr) {
      const int rho = RPI * rr + lr;
      const int64_t m = m0 + wm * 32 * FM + i * 32 + hh * SR + rho;
      const f32x4 v4 = *reinterpret_cast<const f32x4*>(&stg[rho * ES + 4 * lc]);
      if (m >= g.M) continue;
      float v[4] = {v4[0], v4[1], v4[2], v4[3]};
      if (EPI == EPI_PARTIAL) {
        float* dst = g.partial + ((int64_t)z * g.M + m) * g.N + ncol;
        if (vec) {
          *reinterpret_cast<f32x4*>(dst) = v4;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ncol + e < g.N) dst[e] = v[e];
        }
        continue;
      }
      if (EPI == EPI_SILU || EPI == EPI_RESID) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += bias4[e];
      }
      if (EPI == EPI_RESID && g.R) {
        const bf16* rp = reinterpret_cast<const bf16*>(g.R) + m * g.ldr + ncol;
        if (vec) {
          const uint2 rv = rres[EPI == EPI_RESID ? ih : 0][EPI == EPI_RESID ? rr : 0];
          v[0] += __builtin_bit_cast(float, rv.x << 16);
          v[1] += __builtin_bit_cast(float, rv.x & 0xFFFF0000u);
          v[2] += __builtin_bit_cast(float, rv.y << 16);
          v[3] += __builtin_bit_cast(float, rv.y & 0xFFFF0000u);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (ncol + e < g.N) v[e] += (float)rp[e];
        }
      }
      auto put = [&](void* base, const float (&x)[4], bool f32) HSTU_INLINE_LAMBDA {
        if (f32) {
          float* dst = reinterpret_cast<float*>(base) + m * g.ldc + ncol;
          if (vec) {
            *reinterpret_cast<f32x4*>(dst) = f32x4{x[0], x[1], x[2], x[3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (ncol + e < g.N) dst[e] = x[e];
          }
        } else {
          bf16* dst = reinterpret_cast<bf16*>(base) + m * g.ldc + ncol;
          if (vec) {
            uint2 o;
            o.x = pack_bf16x2(x[0], x[1]);
            o.y = pack_bf16x2(x[2], x[3]);
            *reinterpret_cast<uint2*>(dst) = o;
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (ncol + e < g.N) dst[e] = (bf16)x[e];
          }
        }
      };
      if (EPI == EPI_SILU) {
        if (g.C2) put(g.C2, v, false);
        float sv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[e] = silu_f(v[e]);
        put(g.C, sv, false);
        if constexpr (MX) {
          // the attention's q|k columns also as MXFP8 along each head's
          // channels (the 32-column blocks and the range are aligned, so the
          // eight lanes of a block take this branch together)
          const int64_t cq = ncol - g.qk_col0;
          if (g.qk_codes && cq >= 0 && cq < g.qk_cols) {
            float q[4], am = 0.0f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              q[e] = (float)(bf16)sv[e];
              am = fmaxf(am, fabsf(q[e]));
            }
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
            const int sh = mx_shared_exp(am);
            const uint32_t w4 = mx_cvt4(q[0], q[1], q[2], q[3], sh);
            *reinterpret_cast<uint32_t*>(g.qk_codes + m * g.qk_cols + cq) = w4;
            if (g.qk_dequant) {
              // the stored q|k become their MXFP8 values (exact in bf16),
              // over the bf16 values the same lane stored above
              float dq[4];
              dq[0] = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)w4, 0), sh);
              dq[1] = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)w4, 1), sh);
              dq[2] = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)w4, 2), sh);
              dq[3] = ldexpf(__builtin_amdgcn_cvt_f32_fp8((int)w4, 3), sh);
              put(g.C, dq, false);
            }
            if ((lc & 7) == 0) {
              const int64_t hq = cq / g.qk_d, kb = (cq - hq * g.qk_d) / 32;
              g.qk_scales[(hq * g.M + m) * 4 + kb] = (uint8_t)(sh + 127);
            }
          }
        }
      } else {
        put(g.C, v, OUTF32);
      }
      if constexpr (MX && EPI == EPI_RESID && !OUTF32) {
        if (g.c_codes) {
          // MXFP8 copy of the stored (bf16-rounded) row values: the eight
          // lanes of a 32-column block share the row, so their amax is a
          // three-step shuffle (all eight skip rows past M together)
          float q[4], am = 0.0f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            q[e] = (float)(bf16)v[e];
            am = fmaxf(am, fabsf(q[e]));
          }
#pragma unroll
          for (int o = 1; o < 8; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
          const int sh = mx_shared_exp(am);
          *reinterpret_cast<uint32_t*>(g.c_codes + m * g.N + ncol) =
              mx_cvt4(q[0], q[1], q[2], q[3], sh);
          if ((lc & 7) == 0) g.c_scales[m * (g.N / 32) + ncol / 32] = (uint8_t)(sh + 127);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

template <int BM, int BN, bool AK, bool BK, int EPI, bool OUTF32, int NST, bool MX = false>
__global__ __launch_bounds__(64 * G2_NW, (G2Shape<BM, BN, NST>::WPC)) void k_gemm2_bf16(
    GemmArgs g, int mt, int nt, int slots) {
  using SH = G2Shape<BM, BN, NST>;
  constexpr int FM = SH::FM, FN = SH::FN;
  // the tiles as separate LDS objects: the DMA into one stage then provably
  // does not touch the stage being read
  __shared__ __attribute__((aligned(1024))) uint8_t a0[SH::TA];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[SH::TB];
  __shared__ __attribute__((aligned(1024))) uint8_t a1[NST == 2 ? SH::TA : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t b1[NST == 2 ? SH::TB : 16];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, ql = lane & 31, gq = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int w = blockIdx.x;
  int t, z = 0;
  if (EPI == EPI_PARTIAL && g.split_k % 8 == 0) {
    // one-dimensional grid, split z on XCD z % 8 with every tile of it: the
    // XCD's workgroups walk the same k-slice of both operands together, so
    // each operand byte comes from HBM once and is shared through that L2
    // (tile-major order instead reads A once per column block)
    const int r = w >> 3, tiles = mt * nt;
    z = (w & 7) + 8 * (r / tiles);
    t = r - (r / tiles) * tiles;
  } else {
    t = (w & 7) * slots + (w >> 3);
    z = blockIdx.y;
  }
  if (t >= mt * nt) return;
  const int mb = t / nt, nb = t - mb * nt;
  const int64_t m0 = (int64_t)mb * BM, n0 = (int64_t)nb * BN;
  const bf16* A = reinterpret_cast<const bf16*>(g.A);
  const bf16* B = reinterpret_cast<const bf16*>(g.B);

  int64_t kbeg = 0, kend = g.K;
  if (EPI == EPI_PARTIAL) {
    const int64_t per = ((g.K + g.split_k - 1) / g.split_k + G2_BK - 1) / G2_BK * G2_BK;
    kbeg = (int64_t)z * per;
    kend = kbeg + per < g.K ? kbeg + per : g.K;
  }

  G2Off<AK, FM> ao;
  G2Off<BK, FN> bo;
  ao.init(wm * 32 * FM, lane);
  bo.init(wn * 32 * FN, lane);

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};

  auto issue = [&](uint8_t* ta, uint8_t* tb, int64_t k0) HSTU_INLINE_LAMBDA {
    g2_issue<AK, BM>(ta, A, g.lda, m0, g.M, k0, kend, wave, lane);
    g2_issue<BK, BN>(tb, B, g.ldb, n0, g.N, k0, kend, wave, lane);
  };
  // fragments of k-chunk kc+1 are read while the MFMAs of chunk kc run
  auto compute = [&](const uint8_t* ta, const uint8_t* tb) HSTU_INLINE_LAMBDA {
    bf16x8 af[2][FM], bfr[2][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) af[0][i] = ao.frag(ta, i, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[0][j] = bo.frag(tb, j, 0);
#pragma unroll
    for (int kc = 0; kc < G2_BK / 16; ++kc) {
      const int cu = kc & 1;
      if (kc + 1 < G2_BK / 16) {
#pragma unroll
        for (int i = 0; i < FM; ++i) af[cu ^ 1][i] = ao.frag(ta, i, kc + 1);
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[cu ^ 1][j] = bo.frag(tb, j, kc + 1);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32(af[cu][i], bfr[cu][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // MXFP8: per k-step (128 codes = four MX blocks) each lane needs the scales
  // of its rows' blocks g and 2 + g: one 32-bit word of four scale bytes per
  // row, kept as loaded and shifted at use so that bytes 0 and 2 are the two
  // blocks (MFMA op_sel); the shift at use also lets the loads of the next
  // k-step's words stay in flight under the current step's MFMAs.
  G2OffMX amx, bmx;
  const int64_t kblk = g.K / 16;  // MX blocks per row (K counts pairs of codes)
  if constexpr (MX) {
    amx.init(wm * 32 * FM, lane);
    bmx.init(wn * 32 * FN, lane);
  }
  // word of row r at k-step k0: [rows][K/32] (four adjacent bytes of the
  // row) or k-step-major [K/128][rows][4]
  auto scale_word = [&](const uint8_t* sc, int64_t rows, int64_t r, int64_t k0) HSTU_INLINE_LAMBDA {
    const int64_t off = g.scale_kstep_major ? ((k0 / G2_BK) * rows + r) * 4 : r * kblk + k0 / 16;
    return *reinterpret_cast<const uint32_t*>(sc + off);
  };
  auto load_scales = [&](int64_t k0, uint32_t (&wa)[FM], uint32_t (&wb)[FN]) HSTU_INLINE_LAMBDA {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t r = m0 + wm * 32 * FM + 32 * i + ql;
      wa[i] = r < g.M ? scale_word(g.scale_a, g.M, r, k0) : 0x7F7F7F7Fu;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t r = n0 + wn * 32 * FN + 32 * j + ql;
      wb[j] = r < g.N ? scale_word(g.scale_b, g.N, r, k0) : 0x7F7F7F7Fu;
    }
  };
  auto compute_mx = [&](const uint8_t* ta, const uint8_t* tb, const uint32_t (&wa)[FM],
                        const uint32_t (&wb)[FN]) HSTU_INLINE_LAMBDA {
    int sa[FM], sb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) sa[i] = (int)(wa[i] >> (8 * gq));
#pragma unroll
    for (int j = 0; j < FN; ++j) sb[j] = (int)(wb[j] >> (8 * gq));
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      i32x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = amx.frag(ta, i, kh);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = bmx.frag(tb, j, kh);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if (kh == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i], bfr[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                af[i], bfr[j], acc[i][j], 0, 0, 2, sa[i], 2, sb[j]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // double buffer, two stages per iteration so that every access names its
  // stage statically (and no exit in the middle of the iteration, which would
  // make the register allocator shuffle the accumulators)
  // k-steps of this split (an empty last split has kend < kbeg)
  const int nks = kend > kbeg ? (int)((kend - kbeg + G2_BK - 1) / G2_BK) : 0;
  uint32_t wa0[FM] = {}, wb0[FN] = {}, wa1[FM] = {}, wb1[FN] = {};
  auto step = [&](const uint8_t* ta, const uint8_t* tb, const uint32_t (&wa)[FM],
                  const uint32_t (&wb)[FN]) HSTU_INLINE_LAMBDA {
    if constexpr (MX) compute_mx(ta, tb, wa, wb);
    else compute(ta, tb);
  };
  auto issue_s = [&](uint8_t* ta, uint8_t* tb, int64_t k0, uint32_t (&wa)[FM],
                     uint32_t (&wb)[FN]) HSTU_INLINE_LAMBDA {
    issue(ta, tb, k0);
    if constexpr (MX) load_scales(k0, wa, wb);
  };
  if constexpr (NST == 2) {
    if (nks > 0) issue_s(a0, b0, kbeg, wa0, wb0);
    dma_wait();
    __syncthreads();
    for (int ks = 0; ks + 1 < nks; ks += 2) {
      issue_s(a1, b1, kbeg + (int64_t)(ks + 1) * G2_BK, wa1, wb1);
      step(a0, b0, wa0, wb0);
      dma_wait();
      __syncthreads();
      if (ks + 2 < nks) issue_s(a0, b0, kbeg + (int64_t)(ks + 2) * G2_BK, wa0, wb0);
      step(a1, b1, wa1, wb1);
      dma_wait();
      __syncthreads();
    }
    if (nks & 1) step(a0, b0, wa0, wb0);
  } else {
    for (int ks = 0; ks < nks; ++ks) {
      issue_s(a0, b0, kbeg + (int64_t)ks * G2_BK, wa0, wb0);
      dma_wait();
      __syncthreads();
      step(a0, b0, wa0, wb0);
      __syncthreads();
    }
  }

  // Epilogue.  The accumulator layout gives each lane one column and rows
  // 8*(r/4) + 4*gq + r%4, so writing it straight to memory takes one 2-byte
  // store per element.  Instead each wave stages one 32-row block of its fp32
  // results at a time in its own LDS region (row stride ES floats: rows 4
  // apart fall on different banks), then reads rows back as four consecutive
  // columns per lane and applies the epilogue in fp32 with 8- or 16-byte
  // vector accesses.  Every wave is past the main loop (and its last LDS
  // read) before any staging write.
  __syncthreads();
  constexpr int SR = NST == 2 ? 32 : 16;  // rows staged per round (region: a tile, or half of one)
  static_assert(SR * (32 * FN + 8) * 4 <= (NST == 2 ? SH::TA : SH::TA / 2) &&
                    SR * (32 * FN + 8) * 4 <= (NST == 2 ? SH::TB : SH::TB / 2),
                "staging region");
  uint8_t* const region = NST == 2 ? (wave == 0 ? a0 : wave == 1 ? b0 : wave == 2 ? a1 : b1)
                                   : (wave < 2 ? a0 + (wave & 1) * (SH::TA / 2)
                                               : b0 + (wave & 1) * (SH::TB / 2));
  g2_epilogue<FM, FN, EPI, OUTF32, MX, SR>(g, acc, reinterpret_cast<float*>(region), m0, n0, wm,
                                           wn, lane, z);
}

// Whether the DMA-staged kernel's layout assumptions hold for g: 16-byte
// aligned operands and rows, k-contiguous operands with K a multiple of 64,
// k-major operands with a row count (m or n) that is a multiple of 8, and
// 8-byte aligned output rows for the vector epilogue.
bool gemm2_ok(const GemmArgs& g) {
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  if (!al(g.A) || !al(g.B) || (g.lda & 7) || (g.ldb & 7)) return false;
  if ((g.a_kcont || g.b_kcont) && (g.K % G2_BK)) return false;
  if (!g.a_kcont && (g.M & 7)) return false;
  if (!g.b_kcont && (g.N & 7)) return false;
  if (g.epi != EPI_PARTIAL) {
    if (!al(g.C) || (g.ldc & 3)) return false;
    if (g.C2 && !al(g.C2)) return false;
    if (g.R && (!al(g.R) || (g.ldr & 3))) return false;
  } else if (!al(g.partial) || (g.N & 3)) {
    return false;
  }
  // 32-bit DMA offsets: a staged tile spans at most 256 rows of the stride
  if (g.lda > (1 << 22) || g.ldb > (1 << 22)) return false;
  if (g.M > INT32_MAX || g.N > INT32_MAX || g.K > INT32_MAX) return false;
  return true;
}

// Operand stages: one (four workgroups per CU) for the output-heavy shapes,
// measured 16-25% faster on the layer's forward and dX GEMMs; two for the
// split-K weight gradients, whose long k loops gain from the DMA overlap.
template <int BM, int BN, bool AK, bool BK>
hipError_t gemm2_launch(const GemmArgs& g, hipStream_t st) {
  constexpr int NST = 1;
  const int mt = (int)((g.M + BM - 1) / BM), nt = (int)((g.N + BN - 1) / BN);
  const int slots = (mt * nt + 7) / 8;
  dim3 grid((unsigned)(8 * slots), (unsigned)(g.epi == EPI_PARTIAL ? g.split_k : 1));
  if (g.epi == EPI_PARTIAL && g.split_k % 8 == 0) grid = dim3((unsigned)(g.split_k * mt * nt), 1);
  constexpr int NT = 64 * G2_NW;
  switch (g.epi) {
    case EPI_STORE:
      if (g.c_f32) k_gemm2_bf16<BM, BN, AK, BK, EPI_STORE, true, NST><<<grid, NT, 0, st>>>(g, mt, nt, slots);
      else k_gemm2_bf16<BM, BN, AK, BK, EPI_STORE, false, NST><<<grid, NT, 0, st>>>(g, mt, nt, slots);
      break;
    case EPI_SILU:
      k_gemm2_bf16<BM, BN, AK, BK, EPI_SILU, false, NST><<<grid, NT, 0, st>>>(g, mt, nt, slots);
      break;
    case EPI_RESID:
      if (g.c_f32) k_gemm2_bf16<BM, BN, AK, BK, EPI_RESID, true, NST><<<grid, NT, 0, st>>>(g, mt, nt, slots);
      else k_gemm2_bf16<BM, BN, AK, BK, EPI_RESID, false, NST><<<grid, NT, 0, st>>>(g, mt, nt, slots);
      break;
    case EPI_PARTIAL:
      k_gemm2_bf16<BM, BN, AK, BK, EPI_PARTIAL, true, 2><<<grid, NT, 0, st>>>(g, mt, nt, slots);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Tile shape.  Measured on the layer's six GEMMs (M = 34K..57K tokens,
// N, K in 512..2048): 128x128 tiles with two workgroups per CU beat 256x256
// tiles with one in every case (UVQK 0.28 vs 0.31 ms, output projection 0.11
// vs 0.15 ms, 8-layer UVQK 0.98 vs 1.34 ms): the second workgroup hides the
// other's epilogue and DMA latency, which outweighs the larger tile's halved
// LDS reads per MFMA.  The template still accepts 256x256 (one workgroup
// per CU) for shapes where that measures faster.  A persistent variant (one
// workgroup per CU walking its tiles through a four-stage LDS ring, the DMA
// running three k-steps ahead across tiles and under the epilogue) measured
// 1.3-1.8x slower than four resident one-stage workgroups (training-workload
// UVQK 0.36 vs 0.23 ms, dX 0.23 vs 0.17 ms): with one wave per SIMD nothing
// hides the LDS-read and MFMA dependency latencies inside a k-step.
template <bool AK, bool BK>
hipError_t gemm2_ab(const GemmArgs& g, hipStream_t st) {
  return gemm2_launch<128, 128, AK, BK>(g, st);
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

// The same with four consecutive columns per thread (N, ldo and both base
// addresses multiples of four floats) and the loads of eight splits in
// flight at once: the partials are read once, at memory rate, instead of one
// latency per split.
__global__ __launch_bounds__(256) void k_splitk_reduce4(const float4* __restrict__ part, int split,
                                                         int64_t M, int64_t N4,
                                                         float* __restrict__ out, int64_t ldo) {
  const int64_t total = M * N4;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    float4 s = {0.0f, 0.0f, 0.0f, 0.0f};
    int z = 0;
    for (; z + 8 <= split; z += 8) {
      float4 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = part[(z + u) * total + i];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s.x += x[u].x;
        s.y += x[u].y;
        s.z += x[u].z;
        s.w += x[u].w;
      }
    }
    for (; z < split; ++z) {
      const float4 x = part[z * total + i];
      s.x += x.x;
      s.y += x.y;
      s.z += x.z;
      s.w += x.w;
    }
    const int64_t m = i / N4, n = 4 * (i % N4);
    *reinterpret_cast<float4*>(out + m * ldo + n) = s;
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

// MXFP8 GEMM: both operands k-contiguous E4M3 codes (k-steps of 128 codes),
// the DMA-staged kernel with the scaled MFMA; one operand stage.
hipError_t gemm2_mx(const GemmArgs& g, hipStream_t st) {
  if (!g.a_kcont || !g.b_kcont || !g.scale_a || !g.scale_b || !gemm2_ok(g))
    return hipErrorInvalidValue;
  if ((reinterpret_cast<uintptr_t>(g.scale_a) & 3) || (reinterpret_cast<uintptr_t>(g.scale_b) & 3))
    return hipErrorInvalidValue;
  if (g.c_codes && (g.epi != EPI_RESID || g.c_f32 || (g.N % 32) || !g.c_scales ||
                    (reinterpret_cast<uintptr_t>(g.c_codes) & 3)))
    return hipErrorInvalidValue;
  if (g.qk_codes && (g.epi != EPI_SILU || !g.qk_scales || g.qk_d <= 0 || g.qk_d % 32 ||
                     g.qk_d > 128 || g.qk_col0 % 32 || g.qk_cols % g.qk_d ||
                     g.qk_col0 < 0 || g.qk_col0 + g.qk_cols > g.N ||
                     (reinterpret_cast<uintptr_t>(g.qk_codes) & 3) ||
                     (reinterpret_cast<uintptr_t>(g.qk_scales) & 3)))
    return hipErrorInvalidValue;
  constexpr int BM = 128, BN = 128, NT = 64 * G2_NW;
  const int mt = (int)((g.M + BM - 1) / BM), nt = (int)((g.N + BN - 1) / BN);
  const int slots = (mt * nt + 7) / 8;
  dim3 grid((unsigned)(8 * slots), 1);
  if (g.epi == EPI_PARTIAL) {
    // split-K (the weight gradients, contracted over the tokens): the same
    // grid as the bf16 split-K products
    if (g.split_k < 1) return hipErrorInvalidValue;
    grid = g.split_k % 8 == 0 ? dim3((unsigned)(g.split_k * mt * nt), 1)
                              : dim3((unsigned)(8 * slots), (unsigned)g.split_k);
  }
  switch (g.epi) {
    case EPI_PARTIAL:  // long k: two stages, as the bf16 split-K products
      k_gemm2_bf16<BM, BN, true, true, EPI_PARTIAL, true, 2, true><<<grid, NT, 0, st>>>(g, mt, nt, slots);
      break;
    case EPI_STORE:
      if (g.c_f32)
        k_gemm2_bf16<BM, BN, true, true, EPI_STORE, true, 1, true><<<grid, NT, 0, st>>>(g, mt, nt, slots);
      else
        k_gemm2_bf16<BM, BN, true, true, EPI_STORE, false, 1, true><<<grid, NT, 0, st>>>(g, mt, nt, slots);
      break;
    case EPI_SILU:
      k_gemm2_bf16<BM, BN, true, true, EPI_SILU, false, 1, true><<<grid, NT, 0, st>>>(g, mt, nt, slots);
      break;
    case EPI_RESID:
      k_gemm2_bf16<BM, BN, true, true, EPI_RESID, false, 1, true><<<grid, NT, 0, st>>>(g, mt, nt, slots);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& g, int dtype, hipStream_t st) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.mx) return gemm2_mx(g, st);
  if (dtype == HSTU_BF16) {
    if (gemm2_ok(g)) {
      if (g.a_kcont && g.b_kcont) return gemm2_ab<true, true>(g, st);
      if (g.a_kcont && !g.b_kcont) return gemm2_ab<true, false>(g, st);
      if (!g.a_kcont && g.b_kcont) return gemm2_ab<false, true>(g, st);
      return gemm2_ab<false, false>(g, st);
    }
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
  const bool v4 = (N & 3) == 0 && (ldo & 3) == 0 &&
                  ((reinterpret_cast<uintptr_t>(partial) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
  int64_t blocks = ((v4 ? total / 4 : total) + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (v4)
    k_splitk_reduce4<<<(unsigned)blocks, 256, 0, st>>>(reinterpret_cast<const float4*>(partial),
                                                        split, M, N / 4, out, ldo);
  else
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
