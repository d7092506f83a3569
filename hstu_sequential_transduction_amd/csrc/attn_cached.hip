// Ranking against a cached history.
//
// Candidates are appended to a user's history and compared with it in one
// pass ("DLRMv4 Brings Sequence-Based Recommendation Training to MLPerf",
// "Model Architecture"); a history row never attends to a candidate, so the
// history's keys and values at every layer can be computed once and kept.
// For a batch of candidates of user b (rows cand_offsets[b] ..), each at
// position n_h (the history length):
//   O_r = (1/N) * ( sum_{j < n_h, allowed} SiLU(q_r . k_j + bias(n_h - j, t_r - t_j)) v_j
//                   + SiLU(q_r . k_r + bias(0, 0)) v_r )
// with allowed = every history key, or under semi-local windows (Semi-Local
// Attention of "Bending the Scaling Law Curve in Large-Scale Recommendation
// Systems") n_h - j < W_l or j < W_g.
//
// This is a rectangular block per user with no causal mask.  bf16 kernel:
// one workgroup = (user, candidate block, head, key split); four waves of
// 32 (d = 128) or 64 (d <= 64) candidate rows keep Q in registers as the B
// operand of S^T = K Q^T; history key tiles of 64 arrive by buffer->LDS DMA,
// double-buffered; P is the A operand of O += P V with V read down its
// columns (the same tile scheme as the causal forward).  The user's key
// range is split over `splits` workgroups so that small candidate batches
// still fill the chip; without a softmax the partial sums simply add (fp32
// partial buffers, one reduction launch).  The candidate's own key (distance
// 0 in position and time) is added by split 0 after its key loop.
#include "bias.h"
#include "common.h"
#include "internal.h"
#include "lds.h"

#include <type_traits>

namespace hstu {

namespace {

constexpr int CBN = 64;  // history keys per tile

// One 32-row candidate group per wave; as in the forward kernel, waves per
// SIMD decide the speed (latency inside each wave), so d <= 64 runs three
// workgroups per compute unit.
template <int DQK, int DV>
struct CShape {
  static constexpr int QG = 1;
  static constexpr int BM = 4 * 32 * QG;
  static constexpr int OCC = (DQK <= 64 && DV <= 64) ? 3 : 2;  // workgroups per CU
};

template <int DQK, int DV>
struct CBuf {
  uint8_t k[SwzTile<DQK>::bytes(CBN)];
  uint8_t v[SwzTile<DV>::bytes(CBN)];
  int32_t t[CBN];    // key times relative to the user's minimum (narrow)
  int64_t t64[CBN];  // key times (wide users)
};

struct CTables {
  float tfar[32];    // (rab_pos[nP-1] + rab_time[bucket(c)]) * -log2 e, by clz index c
  float ttime[32];   // rab_time[bucket(c)] * -log2 e
  float tpos[1024];  // rab_pos * -log2 e
};

template <bool V>
using bconst = std::integral_constant<bool, V>;

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
template <int DQK, int DV, bool WIN>
__global__ __launch_bounds__(256, (CShape<DQK, DV>::OCC)) void k_attn_cached_bf16(CachedArgs a) {
  constexpr int QG = CShape<DQK, DV>::QG;
  constexpr int BM = CShape<DQK, DV>::BM;
  __shared__ __attribute__((aligned(1024))) CBuf<DQK, DV> cb0;
  __shared__ __attribute__((aligned(1024))) CBuf<DQK, DV> cb1;
  __shared__ CTables sm;

  const int S = a.splits;
  const int per_item = a.H * S;
  const int w = blockIdx.x;
  const int n_items = a.counters[0];
  if (w >= n_items * per_item) return;
  const int it = w / per_item;
  const int rem = w - it * per_item;
  const int h = rem / S, sp = rem - h * S;
  const int b = __builtin_amdgcn_readfirstlane(a.items[2 * it]);
  const int m = __builtin_amdgcn_readfirstlane(a.items[2 * it + 1]);
  if (b < 0 || b >= a.B || m < 0) return;  // not an item of this batch
  const int c0 = __builtin_amdgcn_readfirstlane(a.cand_offsets[b]);
  const int nc = __builtin_amdgcn_readfirstlane(a.cand_offsets[b + 1]) - c0;
  const int h0 = __builtin_amdgcn_readfirstlane(a.hist_offsets[b]);
  const int nh = __builtin_amdgcn_readfirstlane(a.hist_offsets[b + 1]) - h0;
  const int flags = __builtin_amdgcn_readfirstlane(a.flags[b]);
  const bool wide = flags & 1;
  const bool sorted = flags & 2;
  const int nP = a.nP, nT = a.nT;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int ql = lane & 31, g = lane >> 5;

  {
    const float* rp = a.rab_pos + h * a.rab_stride;
    const float* rtb = a.rab_time + h * a.rab_stride;
    for (int i = tid; i < nP; i += 256) sm.tpos[i] = rp[i] * HSTU_NEG_LOG2E;
    if (tid < 32) {
      const float tv = rtb[tbucket_from_clz(tid, nT)];
      sm.ttime[tid] = tv * HSTU_NEG_LOG2E;
      sm.tfar[tid] = (rp[nP - 1] + tv) * HSTU_NEG_LOG2E;
    }
  }

  const int r0 = m * BM + wave * 32 * QG;
  const int rw1 = min(r0 + 32 * QG, nc);

  const bf16* qbase = reinterpret_cast<const bf16*>(a.q) + (int64_t)c0 * a.ld_qk + h * DQK;
  const bf16* kh = reinterpret_cast<const bf16*>(a.kh) + (int64_t)h0 * a.ld_kh + h * DQK;
  const bf16* vh = reinterpret_cast<const bf16*>(a.vh) + (int64_t)h0 * a.ld_vh + h * DV;

  int iq[QG];
  int32_t ti1[QG];
  int64_t tq64[QG];
  bf16x8 qr[QG][DQK / 16];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    iq[qg] = r0 + 32 * qg + ql;
    const bool qv = iq[qg] < nc;
    ti1[qg] = (qv && !wide) ? a.rel_c[c0 + iq[qg]] + 1 : 0;
    tq64[qg] = (qv && wide) ? a.cand_ts[c0 + iq[qg]] : 0;
#pragma unroll
    for (int ch = 0; ch < DQK / 16; ++ch)
      qr[qg][ch] = qv ? *reinterpret_cast<const bf16x8*>(qbase + (int64_t)iq[qg] * a.ld_qk +
                                                         ch * 16 + 8 * g)
                      : bf16x8{};
  }

  f32x16 oacc[QG][DV / 32];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) oacc[qg][d] = f32x16{};

  // this split's key tiles [kt_lo, kt_hi); under windows, tiles wholly
  // between the global window [0, W_g) and the local band [band, n_h) are skipped
  const int KT = (nh + CBN - 1) / CBN;
  const int kt_lo = (int)((int64_t)sp * KT / S);
  const int kt_hi = (int)((int64_t)(sp + 1) * KT / S);
  const int wl = WIN ? a.win_local : 0, wg = WIN ? a.win_global : 0;
  const int band = wl > 0 ? max(nh - wl + 1, 0) : 0;
  const int gtiles = (wg + CBN - 1) / CBN;
  const int btile = band / CBN;
  auto skip_window = [&](int kt) HSTU_INLINE_LAMBDA {
    return (wl > 0 && kt >= gtiles && kt < btile) ? btile : kt;
  };

  auto issue = [&](CBuf<DQK, DV>& Bf, int kt) HSTU_INLINE_LAMBDA {
    const int j0 = kt * CBN;
    dma_tile<DQK, CBN, 4>(Bf.k, kh, a.ld_kh, j0, nh, wave, lane);
    dma_tile<DV, CBN, 4>(Bf.v, vh, a.ld_vh, j0, nh, wave, lane);
    if (wave == 0) {
      if (!wide) dma_words64(Bf.t, a.rel_h + h0, j0, nh, lane);
      else dma_dwords64(Bf.t64, a.hist_ts + h0, j0, nh, lane);
    }
  };

  auto body = [&](const CBuf<DQK, DV>& B, int kt) HSTU_INLINE_LAMBDA {
    const int j0 = kt * CBN;
    const int j1 = min(j0 + CBN, nh);
    if (r0 < rw1) {
      // keys past n_h arrive as zero rows of K and V and add nothing; only
      // keys outside both windows need a mask
      const bool win_mask = wl > 0 && max(j0, wg) < min(j1, band);
      const bool far = !win_mask && !wide && (nh - (j1 - 1) >= nP - 1);

      int mode = 3;  // 0: constant per row, 1: one threshold per row, 2: gather, 3: general
      int cF[QG], cL[QG];
      if (far) {
        const int32_t tfirst = B.t[0], tlast = B.t[j1 - 1 - j0];
        bool one = sorted, cst = sorted;
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          cF[qg] = tclz_narrow(ti1[qg], tfirst);
          cL[qg] = tclz_narrow(ti1[qg], tlast);
          one = one && (cL[qg] - cF[qg] <= 1);
          cst = cst && (cL[qg] == cF[qg]);
        }
        mode = __all(cst) ? 0 : (__all(one) ? 1 : 2);
      }
      float ba[QG], bb[QG];
      int32_t thr[QG];
      if (mode <= 1) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          ba[qg] = sm.tfar[cF[qg]];
          bb[qg] = sm.tfar[min(cF[qg] + 1, 31)];
          thr[qg] = (cL[qg] == cF[qg]) ? INT32_MAX : ti1[qg] - (1 << (31 - cF[qg]));
        }
      }
      // key index in the tile: kk = kc + 4g (kc a compile-time constant)
      const int dJ = nh - j0 - 4 * g;    // n_h - (j0 + 4g): position distance at kc = 0
      const int wlo = band - j0 - 4 * g;  // keys kc >= wlo are in the local band
      const int wgl = wg - j0 - 4 * g;    // keys kc < wgl are in the global window

#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        f32x16 sacc[QG];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) sacc[qg] = f32x16{};
        {
          bf16x8 ka[DQK / 16];
#pragma unroll
          for (int ch = 0; ch < DQK / 16; ++ch) ka[ch] = lds_row8<DQK>(B.k, hf * 32 + ql, ch, g);
#pragma unroll
          for (int ch = 0; ch < DQK / 16; ++ch)
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) sacc[qg] = mfma32(ka[ch], qr[qg][ch], sacc[qg]);
        }

        bf16x8 pk[QG][2];
        auto silu_half = [&](auto bias_of, auto masked) HSTU_INLINE_LAMBDA {
#pragma unroll
          for (int qg = 0; qg < QG; ++qg)
#pragma unroll
            for (int aa = 0; aa < 4; ++aa) {
              const int kk0 = hf * 32 + 8 * aa + 4 * g;
              const i32x4 tj = *reinterpret_cast<const i32x4*>(&B.t[kk0]);
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int kc = hf * 32 + 8 * aa + r;
                const float sb =
                    fmaf(sacc[qg][4 * aa + r], HSTU_NEG_LOG2E, bias_of(qg, kc, tj[r]));
                float p = sb * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sb));
                if constexpr (decltype(masked)::value) p = (kc >= wlo || kc < wgl) ? p : 0.0f;
                pk[qg][aa >> 1][(aa & 1) * 4 + r] = (bf16)p;
              }
            }
        };
        if (mode == 0) {
          silu_half([&](int qg, int, int32_t) { return ba[qg]; }, bconst<false>{});
        } else if (mode == 1) {
          silu_half([&](int qg, int, int32_t tj) { return tj <= thr[qg] ? ba[qg] : bb[qg]; },
                    bconst<false>{});
        } else if (mode == 2) {
          silu_half([&](int qg, int, int32_t tj) { return sm.tfar[tclz_narrow(ti1[qg], tj)]; },
                    bconst<false>{});
        } else if (!wide) {
          auto bias = [&](int qg, int kc, int32_t tj) HSTU_INLINE_LAMBDA {
            const int bp = min(max(dJ - kc, 0), nP - 1);
            return sm.tpos[bp] + sm.ttime[tclz_narrow(ti1[qg], tj)];
          };
          if (win_mask) silu_half(bias, bconst<true>{});
          else silu_half(bias, bconst<false>{});
        } else {
          auto bias = [&](int qg, int kc, int32_t) HSTU_INLINE_LAMBDA {
            const int bp = min(max(dJ - kc, 0), nP - 1);
            return sm.tpos[bp] + sm.ttime[tclz_wide(tq64[qg], B.t64[kc + 4 * g])];
          };
          if (win_mask) silu_half(bias, bconst<true>{});
          else silu_half(bias, bconst<false>{});
        }

#pragma unroll
        for (int u = 0; u < 2; ++u) {
          bf16x8 vb[DV / 32];
#pragma unroll
          for (int d = 0; d < DV / 32; ++d) vb[d] = lds_col8<DV>(B.v, hf * 32 + 16 * u, d * 32, lane);
#pragma unroll
          for (int d = 0; d < DV / 32; ++d)
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) oacc[qg][d] = mfma32(pk[qg][u], vb[d], oacc[qg][d]);
        }
      }
    }
  };

  int kt = skip_window(kt_lo);
  if (kt < kt_hi) issue(cb0, kt);
  dma_wait();
  __syncthreads();
  while (kt < kt_hi) {
    int nk = skip_window(kt + 1);
    if (nk < kt_hi) issue(cb1, nk);
    body(cb0, kt);
    dma_wait();
    __syncthreads();
    kt = nk;
    if (kt >= kt_hi) break;
    nk = skip_window(kt + 1);
    if (nk < kt_hi) issue(cb0, nk);
    body(cb1, kt);
    dma_wait();
    __syncthreads();
    kt = nk;
  }

  if (r0 >= rw1) return;
  // the candidate's own key: position and time distance 0 (clz index 31)
  if (sp == 0) {
    const float bias0 = sm.tpos[0] + sm.ttime[31];
    const bf16* kc_ = reinterpret_cast<const bf16*>(a.k) + (int64_t)c0 * a.ld_qk + h * DQK;
    const bf16* vc_ = reinterpret_cast<const bf16*>(a.v) + (int64_t)c0 * a.ld_v + h * DV;
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      float dot = 0.0f;
      if (iq[qg] < nc) {
#pragma unroll
        for (int ch = 0; ch < DQK / 16; ++ch) {
          const bf16x8 kv =
              *reinterpret_cast<const bf16x8*>(kc_ + (int64_t)iq[qg] * a.ld_qk + ch * 16 + 8 * g);
#pragma unroll
          for (int e = 0; e < 8; ++e) dot = fmaf(bf2f(qr[qg][ch][e]), bf2f(kv[e]), dot);
        }
      }
      dot += __shfl_xor(dot, 32, 64);
      const float sb = fmaf(dot, HSTU_NEG_LOG2E, bias0);
      const float pself = sb * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sb));
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int R = 8 * (r >> 2) + 4 * g + (r & 3);  // accumulator row of register r
        const float pR = __shfl(pself, R, 64);
        const int i = r0 + 32 * qg + R;
        if (i < nc) {
#pragma unroll
          for (int d = 0; d < DV / 32; ++d)
            oacc[qg][d][r] =
                fmaf(pR, bf2f(vc_[(int64_t)i * a.ld_v + d * 32 + ql]), oacc[qg][d][r]);
        }
      }
    }
  }

  const float scale = -HSTU_LN2 / (float)a.norm_len;
  const int64_t W = (int64_t)a.H * DV;
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = r0 + 32 * qg + 8 * (r >> 2) + 4 * g + (r & 3);
        if (i < nc) {
          const float o = oacc[qg][d][r] * scale;
          const int col = h * DV + d * 32 + ql;
          if (S > 1) a.part[((int64_t)sp * a.Tc + c0 + i) * W + col] = o;
          else if (a.out_f32) reinterpret_cast<float*>(a.out)[(int64_t)(c0 + i) * a.ld_out + col] = o;
          else reinterpret_cast<bf16*>(a.out)[(int64_t)(c0 + i) * a.ld_out + col] = (bf16)o;
        }
      }
}

// ---------------------------------------------------------------------------
// fp32 kernel: 64 candidate rows per workgroup, four lanes per row, VALU.
// ---------------------------------------------------------------------------
constexpr int CF_BN = 32;

template <int DQK, int DV>
__global__ __launch_bounds__(256) void k_attn_cached_f32(CachedArgs a) {
  __shared__ float sk[CF_BN][DQK + 1];
  __shared__ float sv[CF_BN][DV + 1];
  __shared__ int32_t st[CF_BN];
  __shared__ int64_t st64[CF_BN];
  __shared__ float spos[1024];
  __shared__ float stime[32];

  const int S = a.splits;
  const int per_item = a.H * S;
  const int w = blockIdx.x;
  const int n_items = a.counters[0];
  if (w >= n_items * per_item) return;
  const int it = w / per_item;
  const int rem = w - it * per_item;
  const int h = rem / S, sp = rem - h * S;
  const int b = a.items[2 * it], m = a.items[2 * it + 1];
  if (b < 0 || b >= a.B || m < 0) return;  // not an item of this batch
  const int c0 = a.cand_offsets[b];
  const int nc = a.cand_offsets[b + 1] - c0;
  const int h0 = a.hist_offsets[b];
  const int nh = a.hist_offsets[b + 1] - h0;
  const bool wide = a.flags[b] & 1;
  const int tid = threadIdx.x;
  const float* rp = a.rab_pos + h * a.rab_stride;
  const float* rt = a.rab_time + h * a.rab_stride;
  for (int i = tid; i < a.nP; i += 256) spos[i] = rp[i];
  if (tid < 32) stime[tid] = rt[tbucket_from_clz(tid, a.nT)];

  const int row = tid >> 2, part = tid & 3;
  const int iq = m * ATTN_FWD_BM_F32 + row;
  const bool qvalid = iq < nc;
  constexpr int QC = DQK / 4, VC = DV / 4;
  const float* qp = reinterpret_cast<const float*>(a.q);
  const float* kcp = reinterpret_cast<const float*>(a.k);
  const float* vcp = reinterpret_cast<const float*>(a.v);
  const float* khp = reinterpret_cast<const float*>(a.kh);
  const float* vhp = reinterpret_cast<const float*>(a.vh);
  float q[QC], o[VC];
#pragma unroll
  for (int cc = 0; cc < QC; ++cc)
    q[cc] = qvalid ? qp[(int64_t)(c0 + iq) * a.ld_qk + h * DQK + part * QC + cc] : 0.0f;
#pragma unroll
  for (int cc = 0; cc < VC; ++cc) o[cc] = 0.0f;
  int32_t ti1 = 0;
  int64_t ti64 = 0;
  if (qvalid) {
    if (wide) ti64 = a.cand_ts[c0 + iq];
    else ti1 = a.rel_c[c0 + iq] + 1;
  }
  const int wl = a.win_local, wg = a.win_global;

  const int KT = (nh + CF_BN - 1) / CF_BN;
  const int kt_lo = (int)((int64_t)sp * KT / S), kt_hi = (int)((int64_t)(sp + 1) * KT / S);
  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    const int j0 = kt * CF_BN;
    __syncthreads();
    for (int idx = tid; idx < CF_BN * DQK; idx += 256) {
      const int r = idx / DQK, cc = idx % DQK;
      const int j = j0 + r;
      sk[r][cc] = j < nh ? khp[(int64_t)(h0 + j) * a.ld_kh + h * DQK + cc] : 0.0f;
    }
    for (int idx = tid; idx < CF_BN * DV; idx += 256) {
      const int r = idx / DV, cc = idx % DV;
      const int j = j0 + r;
      sv[r][cc] = j < nh ? vhp[(int64_t)(h0 + j) * a.ld_vh + h * DV + cc] : 0.0f;
    }
    if (tid < CF_BN) {
      const int j = j0 + tid;
      st[tid] = (j < nh && !wide) ? a.rel_h[h0 + j] : 0;
      st64[tid] = (j < nh && wide) ? a.hist_ts[h0 + j] : 0;
    }
    __syncthreads();
    for (int jj = 0; jj < CF_BN; ++jj) {
      const int j = j0 + jj;
      float dot = 0.0f;
#pragma unroll
      for (int cc = 0; cc < QC; ++cc) dot = fmaf(q[cc], sk[jj][part * QC + cc], dot);
      dot += __shfl_xor(dot, 1, 64);
      dot += __shfl_xor(dot, 2, 64);
      const bool ok = j < nh && (wl <= 0 || nh - j < wl || j < wg);
      const int bpv = pbucket(nh, j, a.nP);
      const int cl = wide ? tclz_wide(ti64, st64[jj]) : tclz_narrow(ti1, st[jj]);
      const float s = dot + spos[bpv] + stime[cl];
      float p = s / (1.0f + __expf(-s));
      p = ok ? p : 0.0f;
#pragma unroll
      for (int cc = 0; cc < VC; ++cc) o[cc] = fmaf(p, sv[jj][part * VC + cc], o[cc]);
    }
  }
  if (sp == 0) {
    float dot = 0.0f;
    if (qvalid) {
#pragma unroll
      for (int cc = 0; cc < QC; ++cc)
        dot = fmaf(q[cc], kcp[(int64_t)(c0 + iq) * a.ld_qk + h * DQK + part * QC + cc], dot);
    }
    dot += __shfl_xor(dot, 1, 64);
    dot += __shfl_xor(dot, 2, 64);
    const float s = dot + spos[0] + stime[31];
    const float p = s / (1.0f + __expf(-s));
    if (qvalid) {
#pragma unroll
      for (int cc = 0; cc < VC; ++cc)
        o[cc] = fmaf(p, vcp[(int64_t)(c0 + iq) * a.ld_v + h * DV + part * VC + cc], o[cc]);
    }
  }
  if (!qvalid) return;
  const float inv = 1.0f / (float)a.norm_len;
  const int64_t W = (int64_t)a.H * DV;
#pragma unroll
  for (int cc = 0; cc < VC; ++cc) {
    const int col = h * DV + part * VC + cc;
    if (S > 1) a.part[((int64_t)sp * a.Tc + c0 + iq) * W + col] = o[cc] * inv;
    else reinterpret_cast<float*>(a.out)[(int64_t)(c0 + iq) * a.ld_out + col] = o[cc] * inv;
  }
}

// out[r][c] = sum_s part[s][r][c] for the key splits (4 columns per thread)
__global__ __launch_bounds__(256) void k_cached_reduce(const float* __restrict__ part, int S,
                                                       int64_t Tc, int64_t W, void* out,
                                                       int64_t ld_out, int out_f32) {
  const int64_t n4 = Tc * W / 4;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4;
       i += (int64_t)gridDim.x * 256) {
    f32x4 acc = reinterpret_cast<const f32x4*>(part)[i];
    for (int s = 1; s < S; ++s) acc += reinterpret_cast<const f32x4*>(part + s * Tc * W)[i];
    const int64_t r = (i * 4) / W, c = (i * 4) - r * W;
    if (out_f32) {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + r * ld_out + c) = acc;
    } else {
      bf16* o = reinterpret_cast<bf16*>(out) + r * ld_out + c;
      o[0] = (bf16)acc[0];
      o[1] = (bf16)acc[1];
      o[2] = (bf16)acc[2];
      o[3] = (bf16)acc[3];
    }
  }
}

template <int DQK, int DV>
hipError_t launch_cached_t(const CachedArgs& a, int dtype, int64_t max_items, hipStream_t st) {
  const int64_t grid = max_items * a.H * a.splits;
  if (grid <= 0) return hipSuccess;
  if (dtype == HSTU_BF16) {
    if (a.win_local > 0) k_attn_cached_bf16<DQK, DV, true><<<(unsigned)grid, 256, 0, st>>>(a);
    else k_attn_cached_bf16<DQK, DV, false><<<(unsigned)grid, 256, 0, st>>>(a);
  } else {
    k_attn_cached_f32<DQK, DV><<<(unsigned)grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <int DQK>
hipError_t launch_cached_dv(const CachedArgs& a, int dtype, int d_v, int64_t mi, hipStream_t st) {
  switch (d_v) {
    case 32: return launch_cached_t<DQK, 32>(a, dtype, mi, st);
    case 64: return launch_cached_t<DQK, 64>(a, dtype, mi, st);
    case 128: return launch_cached_t<DQK, 128>(a, dtype, mi, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int attn_cached_block_rows(int dtype, int d_qk, int d_v) {
  if (dtype != HSTU_BF16) return ATTN_FWD_BM_F32;
  return (d_qk <= 64 && d_v <= 64) ? CShape<64, 64>::BM : CShape<128, 128>::BM;
}

int attn_cached_occupancy(int dtype, int d_qk, int d_v) {
  if (dtype != HSTU_BF16) return 2;
  return (d_qk <= 64 && d_v <= 64) ? CShape<64, 64>::OCC : CShape<128, 128>::OCC;
}

hipError_t launch_attn_cached(const CachedArgs& a, int dtype, int d_qk, int d_v,
                              int64_t max_items, hipStream_t st) {
  hipError_t e = hipErrorInvalidValue;
  switch (d_qk) {
    case 32: e = launch_cached_dv<32>(a, dtype, d_v, max_items, st); break;
    case 64: e = launch_cached_dv<64>(a, dtype, d_v, max_items, st); break;
    case 128: e = launch_cached_dv<128>(a, dtype, d_v, max_items, st); break;
  }
  if (e != hipSuccess || a.splits <= 1 || a.Tc <= 0) return e;
  const int64_t W = (int64_t)a.H * d_v;
  const int64_t n4 = a.Tc * W / 4;
  const int grid = (int)std::min<int64_t>((n4 + 255) / 256, 4096);
  k_cached_reduce<<<grid, 256, 0, st>>>(a.part, a.splits, a.Tc, W, a.out, a.ld_out,
                                        a.out_f32 || dtype != HSTU_BF16 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace hstu
