// Fused HSTU pointwise attention, forward.
//
// O_i = (1/N) * sum_j allowed(i,j) * SiLU(q_i . k_j + rab_pos[bp] + rab_time[bt]) * v_j
// (SiLU weighting instead of softmax and a relative bias: NVIDIA
// generative-recommenders summary, "HSTU Architecture: Efficient Attention for
// User History"; positional/temporal-distance bias and the appended candidate:
// "DLRMv4 Brings Sequence-Based Recommendation Training to MLPerf", "Model
// Architecture"; lower triangle only: its Table 7 note).
//
// bf16 kernel (gfx950 MFMA): one workgroup = one (sequence, query block,
// head) work item, four waves of 32 query rows.  Q
// stays in registers as the B operand of S^T = K Q^T (32x32x16 MFMA).  Tiles
// of 64 keys of K and V arrive row-major by buffer->LDS DMA, double-buffered;
// K is read along rows (A operand of S^T) and V down its columns with
// transpose reads, in the key order the S^T accumulator leaves in each lane,
// so the accumulator is consumed directly as the A operand of O += P V.  Per
// score element the VALU adds the bias (LDS table gathers indexed by the
// position distance and by clz of the time distance), evaluates
// SiLU(s) = s / (1 + 2^(-s log2 e)) with one v_exp and one v_rcp, applies the
// mask only on tiles that need it, and rounds to bf16.  Work is scaled by
// -log2(e) throughout (folded into the bias tables and one FMA) and the
// factor -ln(2)/N is applied once to the output accumulator.
#include "bias.h"
#include "common.h"
#include "internal.h"
#include "lds.h"

#include <type_traits>

namespace hstu {

namespace {

constexpr int FWD_BN = 64;  // keys per tile

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// One 32-row query group per wave.  The kernel is bound by latency inside
// each wave (LDS reads -> S MFMAs -> VALU -> P V MFMAs), so what pays is
// waves per SIMD: at d <= 64 a wave fits in 159 VGPRs and three workgroups
// share a compute unit (three waves per SIMD); at d = 128 registers allow
// two.  (Two 32-row groups per wave at d <= 64, which let every K/V fragment
// read from LDS feed two MFMAs, needed 240 VGPRs and two workgroups per
// compute unit, and was 1.26x slower on the 8-layer Zipf workload.)
template <int DQK, int DV>
struct FwdShape {
  static constexpr int QG = 1;
  static constexpr int BM = 4 * 32 * QG;  // query rows per workgroup (four waves)
  static constexpr int OCC = (DQK <= 64 && DV <= 64) ? 3 : 2;  // workgroups per CU
};

// One staged key tile: row-major K and V and the key times.  MX: K as E4M3
// codes (DQK bytes per row, staged like DQK/2 bf16) and the keys' scale words.
template <int DQK, bool MX>
constexpr int fwd_k_bytes() {
  if constexpr (MX) return SwzTile<DQK / 2>::bytes(FWD_BN);
  else return SwzTile<DQK>::bytes(FWD_BN);
}
template <int DQK, int DV, bool MX = false>
struct FwdBuf {
  uint8_t k[fwd_k_bytes<DQK, MX>()];
  uint8_t v[SwzTile<DV>::bytes(FWD_BN)];
  int32_t t[FWD_BN];    // key times relative to the sequence minimum (narrow)
  int64_t t64[FWD_BN];  // key times (wide sequences)
  uint32_t ks[MX ? FWD_BN : 1];  // MX: scale word of each key (byte b: channels 32b..)
};

// Bias tables, a separate LDS object from the tile buffers.
// Position table with saturated margins: tposx[TPOS_PADL + x] holds
// rab_pos[clamp(x, 0, nP-1)] for x in [-TPOS_PADL, nP + TPOS_PADH).  Tiles of
// history keys near the diagonal see position distances in [-126, nP + 125]
// (a 64-row wave against a 64-key tile that is active and not far), so their
// gathers need no clamp and no per-element address arithmetic.
constexpr int TPOS_PADL = 192, TPOS_PADH = 128;

struct FwdTables {
  float tfar[32];    // (rab_pos[nP-1] + rab_time[bucket(c)]) * -log2 e, by clz index c
  float ttime[32];   // rab_time[bucket(c)] * -log2 e
  float tposx[TPOS_PADL + 1024 + TPOS_PADH];  // rab_pos * -log2 e, saturated margins
};

// mask kinds: 0 none, 1 causal only (tiles of history keys), 2 causal,
// candidate and window terms
template <int V>
using mconst = std::integral_constant<int, V>;

// SPLIT: workgroup w takes part w / I of work item w % I (S = a.splits parts
// of I = gridDim.x / S items): the
// item's visited key tiles are cut into np <= S contiguous runs of at least
// four tiles.  With np = 1 the one part writes O; otherwise each part writes
// its scaled partial sum of O to a.part and k_attn_fwd_combine adds them.
// KH (key halves): 64-row work items; waves 2r and 2r+1 share the rows of
// group r and each takes one 32-key half of every tile (half the work per
// tile, so the longest item's chain of tiles takes about half as long),
// adding their partial sums of O through LDS at the end.  For batches whose
// 128-row items do not fill the GPU.
// MX: the score product in MXFP8 (E4M3 codes of q and k with E8M0 block
// scales along d_qk, the scaled 32x32x64 FP8 MFMA; one per 64 channels);
// P V stays bf16.
template <int DQK, int DV, bool WIN, bool SPLIT, bool KH = false, bool MX = false>
__global__ __launch_bounds__(256, (FwdShape<DQK, DV>::OCC)) void k_attn_fwd_bf16(AttnArgs a) {
  static_assert(!(KH && (SPLIT || WIN)), "key halves: no split, no windows");
  static_assert(!MX || (!SPLIT && !WIN && (DQK == 64 || DQK == 128)),
                "MX scores: no split, no windows, d_qk 64 or 128");
  constexpr int QG = FwdShape<DQK, DV>::QG;
  constexpr int BM = KH ? 64 : FwdShape<DQK, DV>::BM;
  using Buf = FwdBuf<DQK, DV, MX>;
  __shared__ __attribute__((aligned(1024))) Buf fwb0;
  __shared__ __attribute__((aligned(1024))) Buf fwb1;
  __shared__ FwdTables sm;

  // part-major numbering (parts 0 of every item first): consecutive workgroups
  // go to different XCDs, and with item-major numbering and S a power of two
  // the parts 0 of all items (all of the unsplit items' work) would share
  // S-th of the XCDs
  const int S = SPLIT ? a.splits : 1;
  const int nwi = SPLIT ? (int)(gridDim.x / (unsigned)S) : 0;
  const int part = SPLIT ? (int)(blockIdx.x / (unsigned)max(nwi, 1)) : 0;
  const int wi = SPLIT ? (int)blockIdx.x - part * nwi : (int)blockIdx.x;
  const int n_items = a.counters[0];
  if (wi >= n_items * a.H) return;
  const int it = wi / a.H, h = wi - it * a.H;
  const int b = __builtin_amdgcn_readfirstlane(a.items[2 * it]);
  const int m = __builtin_amdgcn_readfirstlane(a.items[2 * it + 1]);
  if (b < 0 || b >= a.B || m < 0) return;  // not an item of this batch
  const int o0 = __builtin_amdgcn_readfirstlane(a.seq_offsets[b]);
  const int n = __builtin_amdgcn_readfirstlane(a.seq_offsets[b + 1]) - o0;
  if (m >= (n + BM - 1) / BM) return;
  const int c = a.num_cand ? __builtin_amdgcn_readfirstlane(a.num_cand[b]) : 0;
  const int nh = n - c;
  // SPLIT: this part's run of visited key tiles, [kt_a, kt_b), decided before
  // anything else is loaded so that parts with no run leave at once.  Visited
  // tiles: [0, ceil(rb1 / BN)) minus the tiles of candidate keys that end
  // before the block, [ceil(nh / BN), rb0 / BN) (the order next_tile walks).
  int np = 1, kt_a = 0, kt_b = 0;
  if constexpr (SPLIT) {
    const int b0 = m * BM, kt_all = (min(b0 + BM, n) + FWD_BN - 1) / FWD_BN;
    const int s0 = (nh + FWD_BN - 1) / FWD_BN, nskip = max(0, b0 / FWD_BN - s0);
    const int nv = kt_all - nskip;
    np = min(S, max(1, nv / 4));
    if (part >= np) return;
    const int lo = nv * part / np, hi = nv * (part + 1) / np;
    auto tile_of = [&](int v) HSTU_INLINE_LAMBDA { return v < s0 ? v : v + nskip; };
    kt_a = tile_of(lo);
    kt_b = hi < nv ? tile_of(hi) : kt_all;
  }
  const int flags = __builtin_amdgcn_readfirstlane(a.seq_flags[b]);
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
    for (int i = tid; i < nP + TPOS_PADL + TPOS_PADH; i += 256)
      sm.tposx[i] = rp[min(max(i - TPOS_PADL, 0), nP - 1)] * HSTU_NEG_LOG2E;
    if (tid < 32) {
      const float tv = rtb[tbucket_from_clz(tid, nT)];
      sm.ttime[tid] = tv * HSTU_NEG_LOG2E;
      sm.tfar[tid] = (rp[nP - 1] + tv) * HSTU_NEG_LOG2E;
    }
  }

  const int rb0 = m * BM;
  const int rb1 = min(rb0 + BM, n);
  const int rg = KH ? (wave >> 1) : wave;  // row group of this wave
  const int khalf = KH ? (wave & 1) : 0;   // its key half of every tile (KH)
  const int r0 = rb0 + rg * 32 * QG;
  const int rw1 = min(r0 + 32 * QG, n);

  const bf16* qbase = reinterpret_cast<const bf16*>(a.q) + (int64_t)o0 * a.ld_qk + h * DQK;
  const bf16* kh = reinterpret_cast<const bf16*>(a.k) + (int64_t)o0 * a.ld_qk + h * DQK;
  const bf16* vh = reinterpret_cast<const bf16*>(a.v) + (int64_t)o0 * a.ld_v + h * DV;
  const int64_t* tsq = a.ts + o0;

  int iq[QG], pI[QG];
  int32_t ti1[QG];
  int64_t tq64[QG];
  bf16x8 qr[QG][MX ? 1 : DQK / 16];
  // MX: lane half g holds channels 64 c + 16 g + {0..15} and 64 c + 32 + 16 g
  // + {0..15} of its row (c = 0 .. DQK/64 - 1) (the scaled MFMA's k order) and the row's scale word
  // shifted so that bytes 0 and 2 are blocks g and 2 + g
  i32x8 qm[QG][MX ? DQK / 64 : 1];
  int qsc[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    iq[qg] = r0 + 32 * qg + ql;
    const bool qv = iq[qg] < n;
    pI[qg] = min(iq[qg], nh);
    ti1[qg] = (qv && !wide) ? a.rel_t[o0 + iq[qg]] + 1 : 0;
    tq64[qg] = (qv && wide) ? tsq[iq[qg]] : 0;
    if constexpr (MX) {
      const uint8_t* qp = a.q_mx + (int64_t)(o0 + iq[qg]) * a.ld_mx + h * DQK + 16 * g;
#pragma unroll
      for (int c64 = 0; c64 < DQK / 64; ++c64) {
        const i32x4 lo = qv ? *reinterpret_cast<const i32x4*>(qp + 64 * c64) : i32x4{};
        const i32x4 hi = qv ? *reinterpret_cast<const i32x4*>(qp + 64 * c64 + 32) : i32x4{};
        qm[qg][c64] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      qsc[qg] = qv ? (int)(a.q_mxs[h * a.T_rows + o0 + iq[qg]] >> (8 * g)) : 0;
    } else {
#pragma unroll
      for (int ch = 0; ch < DQK / 16; ++ch)
        qr[qg][ch] = qv ? *reinterpret_cast<const bf16x8*>(qbase + (int64_t)iq[qg] * a.ld_qk +
                                                           ch * 16 + 8 * g)
                        : bf16x8{};
    }
  }

  f32x16 oacc[QG][DV / 32];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) oacc[qg][d] = f32x16{};

  // Semi-local windows: history key j is allowed for row i only if
  // j >= p(i) - W_l + 1 or j < W_g.  Key tiles past the global window and
  // below the band of every row of the workgroup hold no allowed pair.
  // WIN: semi-local windows compiled in (otherwise every window term folds away)
  const int wl = WIN ? a.win_local : 0, wg = WIN ? a.win_global : 0;
  const int band_wg = wl > 0 ? max(min(rb0, nh) - wl + 1, 0) : 0;  // lowest band key of the WG
  const int gtiles = (wg + FWD_BN - 1) / FWD_BN;                     // tiles touching [0, W_g)
  const int btile = band_wg / FWD_BN;
  auto skip_window = [&](int kt) HSTU_INLINE_LAMBDA {
    return (wl > 0 && kt >= gtiles && kt < btile) ? btile : kt;
  };

  // key tiles: 0 .. ktiles-1, skipping tiles that hold only other candidates' keys
  const int ktiles = (rb1 + FWD_BN - 1) / FWD_BN;
  auto next_tile = [&](int kt) HSTU_INLINE_LAMBDA {
    const int nk = skip_window(kt + 1);
    const int j0 = nk * FWD_BN;
    if (j0 >= nh && j0 + FWD_BN <= rb0) return rb0 / FWD_BN;
    return nk;
  };

  // DMA of key tile kt; keys >= n arrive as zeros
  // MX: rows of DQK code bytes staged as DQK/2 bf16; the keys' scale words
  const bf16* kmx = MX ? reinterpret_cast<const bf16*>(a.k_mx + (int64_t)o0 * a.ld_mx + h * DQK)
                       : nullptr;
  auto issue = [&](Buf& Bf, int kt) HSTU_INLINE_LAMBDA {
    const int j0 = kt * FWD_BN;
    if constexpr (MX) {
      dma_tile<DQK / 2, FWD_BN, 4>(Bf.k, kmx, a.ld_mx / 2, j0, n, wave, lane);
      if (wave == 1) dma_words64(Bf.ks, a.k_mxs + h * a.T_rows + o0, j0, n, lane);
    } else {
      dma_tile<DQK, FWD_BN, 4>(Bf.k, kh, a.ld_qk, j0, n, wave, lane);
    }
    dma_tile<DV, FWD_BN, 4>(Bf.v, vh, a.ld_v, j0, n, wave, lane);
    if (wave == 0) {
      if (!wide) dma_words64(Bf.t, a.rel_t + o0, j0, n, lane);
      else dma_dwords64(Bf.t64, tsq, j0, n, lane);
    }
  };

  auto body = [&](const Buf& B, int kt) HSTU_INLINE_LAMBDA {
    const int j0 = kt * FWD_BN;
    const int j1 = min(j0 + FWD_BN, n);
    const bool hist_rows = r0 < nh;
    const bool cand_rows = rw1 > nh;
    // window: lowest band key of the wave's first and last rows
    const int band_lo = wl > 0 ? min(r0, nh) - wl + 1 : 0;
    const int band_hi = wl > 0 ? min(rw1 - 1, nh) - wl + 1 : 0;
    const bool win_out = wl > 0 && j0 >= wg && j1 - 1 < band_lo && j1 <= nh;
    const bool active = (r0 < rw1) && !win_out &&
                        ((hist_rows && j0 <= min(rw1, nh) - 1) ||
                         (cand_rows && (j0 < nh || (j0 < rw1 && j1 > max(r0, nh)))));
    if (active) {
      const bool win_mask = wl > 0 && j1 > wg && j0 < band_hi;
      const bool need_mask = (hist_rows && j1 - 1 > r0) || (j1 > nh) || win_mask;
      const bool far = !need_mask && !wide && (min(r0, nh) - min(j1 - 1, nh) >= nP - 1);

      // tile class (wave-uniform): far tiles have position bucket nP-1 everywhere; with
      // sorted timestamps a row's time bucket usually changes at most once per tile
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

      // per-lane constants of the general path, shifted by 4g (see silu_half)
      int dI[QG], pmin[QG], lim[QG], slf[QG], wlo[QG], wgl[QG];
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        const int i = iq[qg];
        dI[qg] = pI[qg] - j0 - 4 * g;             // p(i) - (j0 + 4g)
        pmin[qg] = pI[qg] - nh;                   // p(i) - n_h (candidate keys)
        lim[qg] = (i < nh ? i : nh - 1) - j0 - 4 * g;  // last allowed key of the causal part
        slf[qg] = i - j0 - 4 * g;                 // the row's own key (candidates)
        // window: keys >= wlo (local band) or < wgl (global window) pass
        wlo[qg] = (wl > 0 ? pI[qg] - wl + 1 : INT32_MIN / 2) - j0 - 4 * g;
        wgl[qg] = wg - j0 - 4 * g;
      }

#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if (KH && hf != khalf) continue;
        f32x16 sacc[QG];
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) sacc[qg] = f32x16{};
        if constexpr (MX) {
          // S^T = K Q^T with E8M0 block scales: key row hf*32 + ql of the
          // tile, channels in the order of the Q registers above
          const int ksc = (int)(B.ks[hf * 32 + ql] >> (8 * g));
          i32x8 ka[DQK / 64];
#pragma unroll
          for (int c64 = 0; c64 < DQK / 64; ++c64) {
            const i32x4 lo =
                __builtin_bit_cast(i32x4, lds_row8<DQK / 2>(B.k, hf * 32 + ql, 2 * c64, g));
            const i32x4 hi =
                __builtin_bit_cast(i32x4, lds_row8<DQK / 2>(B.k, hf * 32 + ql, 2 * c64 + 1, g));
            ka[c64] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) {
            sacc[qg] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                ka[0], qm[qg][0], sacc[qg], 0, 0, 0, ksc, 0, qsc[qg]);
            if constexpr (DQK == 128)
              sacc[qg] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  ka[1], qm[qg][1], sacc[qg], 0, 0, 2, ksc, 2, qsc[qg]);
          }
        } else {
          bf16x8 ka[DQK / 16];
#pragma unroll
          for (int ch = 0; ch < DQK / 16; ++ch) ka[ch] = lds_row8<DQK>(B.k, hf * 32 + ql, ch, g);
#pragma unroll
          for (int ch = 0; ch < DQK / 16; ++ch)
#pragma unroll
            for (int qg = 0; qg < QG; ++qg) sacc[qg] = mfma32(ka[ch], qr[qg][ch], sacc[qg]);
        }

        bf16x8 pk[QG][2];
        // P' = s' / (1 + 2^s') with s' = -log2(e) * (q.k + bias).  Key index in the
        // tile: kk = kc + 4g with kc = hf*32 + 8*aa + r a compile-time constant, so
        // per-lane limits are pre-shifted by 4g and compared with immediates.
        // bias_of(qg, kc, key time) returns the pre-scaled bias.
        auto silu_half = [&](auto bias_of, auto masked) HSTU_INLINE_LAMBDA {
#pragma unroll
          for (int qg = 0; qg < QG; ++qg)
#pragma unroll
            for (int aa = 0; aa < 4; ++aa) {
              const int kk0 = hf * 32 + 8 * aa + 4 * g;
              const i32x4 tj = *reinterpret_cast<const i32x4*>(&B.t[kk0]);
              float pv[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int kc = hf * 32 + 8 * aa + r;
                const float sb =
                    fmaf(sacc[qg][4 * aa + r], HSTU_NEG_LOG2E, bias_of(qg, kc, tj[r]));
                float p = sb * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sb));
                if constexpr (decltype(masked)::value != 0) {
                  bool ok = kc <= lim[qg];
                  if constexpr (decltype(masked)::value == 2) {
                    ok = ok || kc == slf[qg];
                    if constexpr (WIN) ok = ok && (kc >= wlo[qg] || kc < wgl[qg]);
                  }
                  p = ok ? p : 0.0f;
                }
                pv[r] = p;
              }
              // round pairs to bf16 (one v_cvt_pk_bf16_f32 per two scores)
#pragma unroll
              for (int r = 0; r < 4; r += 2) {
                const bf16x2 two = __builtin_convertvector(f32x2{pv[r], pv[r + 1]}, bf16x2);
                pk[qg][aa >> 1][(aa & 1) * 4 + r] = two[0];
                pk[qg][aa >> 1][(aa & 1) * 4 + r + 1] = two[1];
              }
            }
        };
        if (mode == 0) {
          silu_half([&](int qg, int, int32_t) { return ba[qg]; }, mconst<0>{});
        } else if (mode == 1) {
          silu_half([&](int qg, int, int32_t tj) { return tj <= thr[qg] ? ba[qg] : bb[qg]; },
                    mconst<0>{});
        } else if (mode == 2) {
          silu_half([&](int qg, int, int32_t tj) { return sm.tfar[tclz_narrow(ti1[qg], tj)]; },
                    mconst<0>{});
        } else if (!wide && j1 <= nh && wl == 0) {
          // history keys only, no windows: p(i) - j = dI - kc stays inside the
          // padded table, read at a per-lane base plus an immediate offset;
          // the only mask term is causality (no key of the tile is a candidate)
          const float* pb[QG];
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) pb[qg] = &sm.tposx[TPOS_PADL + dI[qg] - (FWD_BN - 1)];
          auto bias = [&](int qg, int kc, int32_t tj) HSTU_INLINE_LAMBDA {
            return pb[qg][(FWD_BN - 1) - kc] + sm.ttime[tclz_narrow(ti1[qg], tj)];
          };
          if (need_mask) silu_half(bias, mconst<1>{});
          else silu_half(bias, mconst<0>{});
        } else if (!wide) {
          // position bucket: clamp(p(i) - min(j, n_h), 0, nP-1) = med3(max(dI - kc, pI - nh), 0, nP-1)
          auto bias = [&](int qg, int kc, int32_t tj) HSTU_INLINE_LAMBDA {
            const int bp = min(max(max(dI[qg] - kc, pmin[qg]), 0), nP - 1);
            return sm.tposx[TPOS_PADL + bp] + sm.ttime[tclz_narrow(ti1[qg], tj)];
          };
          if (need_mask) silu_half(bias, mconst<2>{});
          else silu_half(bias, mconst<0>{});
        } else {
          auto bias = [&](int qg, int kc, int32_t) HSTU_INLINE_LAMBDA {
            const int bp = min(max(max(dI[qg] - kc, pmin[qg]), 0), nP - 1);
            return sm.tposx[TPOS_PADL + bp] + sm.ttime[tclz_wide(tq64[qg], B.t64[kc + 4 * g])];
          };
          silu_half(bias, mconst<2>{});
        }

        // O += P V: V read down its columns (keys are the k index)
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

  // double-buffered key-tile pipeline, unrolled by two so that every access
  // names its buffer statically (the DMA into one buffer then needs no wait
  // before reads of the other)
  int kt = skip_window(0);
  if (kt < ktiles && kt * FWD_BN >= nh && kt * FWD_BN + FWD_BN <= rb0) kt = rb0 / FWD_BN;
  // kend: the first visited tile past this workgroup's run (any value >= ktiles
  // when the run goes to the end)
  int kend = ktiles;
  if constexpr (SPLIT) {
    kt = kt_a;
    kend = kt_b;
  }
  if (kt < kend) issue(fwb0, kt);
  dma_wait();
  __syncthreads();
  while (kt < kend) {
    int nk = next_tile(kt);
    if (nk < kend) issue(fwb1, nk);
    body(fwb0, kt);
    dma_wait();
    __syncthreads();
    kt = nk;
    if (kt >= kend) break;
    nk = next_tile(kt);
    if (nk < kend) issue(fwb0, nk);
    body(fwb1, kt);
    dma_wait();
    __syncthreads();
    kt = nk;
  }

  const float scale = -HSTU_LN2 / (float)(a.norm_mode == 0 ? a.norm_len : n);
  if constexpr (SPLIT) {
    static_assert(QG == 1, "split partials assume one query group per wave");
    if (part == 0 && tid == 0) a.part_cnt[wi] = np;  // read by k_attn_fwd_combine
    if (np > 1) {
      // scaled partial sums of rows rb0 .. rb1-1, [BM][DV] per part; the
      // combine kernel that runs next adds them (no fence or counter here:
      // on this GPU a device-scope fence writes back the whole L2)
      float* pw = a.part + ((int64_t)wi * S + part) * (BM * DV);
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = r0 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (i < n) pw[(i - rb0) * DV + d * 32 + ql] = oacc[0][d][r] * scale;
        }
      return;
    }
  }

  if constexpr (KH) {
    // the key-half-1 wave of each row group hands its partial sum of O to the
    // key-half-0 wave (the tile buffers are free after the loop's last barrier)
    static_assert((DV / 32) * 16 * 64 * 4 <= (int)sizeof(Buf), "exchange fits a tile buffer");
    float* xo = reinterpret_cast<float*>(rg == 0 ? reinterpret_cast<uint8_t*>(&fwb0)
                                                 : reinterpret_cast<uint8_t*>(&fwb1));
    if (khalf == 1) {
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(d * 16 + r) * 64 + lane] = oacc[0][d][r];
    }
    __syncthreads();
    if (khalf == 1) return;
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[0][d][r] += xo[(d * 16 + r) * 64 + lane];
  }

  // ---- write O * (-ln2 / N) ----
  if (r0 >= rw1) return;
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int d = 0; d < DV / 32; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = r0 + 32 * qg + 8 * (r >> 2) + 4 * g + (r & 3);
        if (i < n) {
          const int64_t off = (int64_t)(o0 + i) * a.ld_out + h * DV + d * 32 + ql;
          if (a.out_f32) reinterpret_cast<float*>(a.out)[off] = oacc[qg][d][r] * scale;
          else reinterpret_cast<bf16*>(a.out)[off] = (bf16)(oacc[qg][d][r] * scale);
        }
      }
}

// Sum of the np partial sums of each split work item (np = part_cnt[item],
// written by the item's part 0; items with np = 1 wrote O themselves).  One
// wave per 16 rows of a work item, every load of a part in flight at once.
constexpr int CMB_ROWS = 16;

template <int BM, int DV>
__global__ __launch_bounds__(64) void k_attn_fwd_combine(AttnArgs a) {
  constexpr int CPI = BM / CMB_ROWS;        // waves per work item
  constexpr int PER = CMB_ROWS * DV / 4 / 64;  // float4s per lane and part
  const int wi = blockIdx.x / CPI;
  const int rg = blockIdx.x - wi * CPI;
  if (wi >= a.counters[0] * a.H) return;
  const int np = a.part_cnt[wi];
  if (np <= 1) return;
  const int it = wi / a.H, h = wi - it * a.H;
  const int b = a.items[2 * it], m = a.items[2 * it + 1];
  if (b < 0 || b >= a.B || m < 0) return;
  const int o0 = a.seq_offsets[b];
  const int n = a.seq_offsets[b + 1] - o0;
  const int lr0 = rg * CMB_ROWS;  // first row of this wave within the block
  const int rows = min(CMB_ROWS, n - m * BM - lr0);
  if (rows <= 0) return;
  constexpr int P4 = BM * DV / 4;  // float4s per part
  const float4* pr = reinterpret_cast<const float4*>(a.part + (int64_t)wi * a.splits * (BM * DV)) +
                     lr0 * (DV / 4);
  const int ne = rows * (DV / 4);
  float4 acc[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = threadIdx.x + 64 * k;
    acc[k] = e < ne ? pr[e] : float4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  for (int p = 1; p < np; ++p) {
    float4 x[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int e = threadIdx.x + 64 * k;
      x[k] = e < ne ? pr[p * P4 + e] : float4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      acc[k].x += x[k].x;
      acc[k].y += x[k].y;
      acc[k].z += x[k].z;
      acc[k].w += x[k].w;
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int e = threadIdx.x + 64 * k;
    if (e >= ne) continue;
    const int i = m * BM + lr0 + e / (DV / 4), col = 4 * (e % (DV / 4));
    const int64_t off = (int64_t)(o0 + i) * a.ld_out + h * DV + col;
    if (a.out_f32) {  // (ld_out need not keep rows 16-byte aligned)
      float* o = reinterpret_cast<float*>(a.out) + off;
      o[0] = acc[k].x;
      o[1] = acc[k].y;
      o[2] = acc[k].z;
      o[3] = acc[k].w;
    } else {
      bf16* o = reinterpret_cast<bf16*>(a.out) + off;
      o[0] = (bf16)acc[k].x;
      o[1] = (bf16)acc[k].y;
      o[2] = (bf16)acc[k].z;
      o[3] = (bf16)acc[k].w;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: 64 query rows per workgroup, four lanes per row, VALU math.
// ---------------------------------------------------------------------------
constexpr int F32_BN = 32;

template <int DQK, int DV>
__global__ __launch_bounds__(256) void k_attn_fwd_f32(AttnArgs a) {
  __shared__ float sk[F32_BN][DQK + 1];
  __shared__ float sv[F32_BN][DV + 1];
  __shared__ int32_t st[F32_BN];
  __shared__ int64_t st64[F32_BN];
  __shared__ float spos[1024];
  __shared__ float stime[32];

  const int w = blockIdx.x;
  const int n_items = a.counters[0];
  if (w >= n_items * a.H) return;
  const int it = w / a.H, h = w - it * a.H;
  const int b = a.items[2 * it], m = a.items[2 * it + 1];
  if (b < 0 || b >= a.B || m < 0) return;  // not an item of this batch
  const int o0 = a.seq_offsets[b];
  const int n = a.seq_offsets[b + 1] - o0;
  if (m * 64 >= n) return;
  const int c = a.num_cand ? a.num_cand[b] : 0;
  const int nh = n - c;
  const bool wide = a.seq_flags[b] & 1;
  const int tid = threadIdx.x;
  const float* rp = a.rab_pos + h * a.rab_stride;
  const float* rt = a.rab_time + h * a.rab_stride;
  for (int i = tid; i < a.nP; i += 256) spos[i] = rp[i];
  if (tid < 32) stime[tid] = rt[tbucket_from_clz(tid, a.nT)];

  const int row = tid >> 2, part = tid & 3;
  const int rb0 = m * 64, rb1 = min(rb0 + 64, n);
  const int iq = rb0 + row;
  const bool qvalid = iq < n;
  const int pI = min(iq, nh);
  constexpr int QC = DQK / 4, VC = DV / 4;
  const float* qp = reinterpret_cast<const float*>(a.q);
  const float* kp = reinterpret_cast<const float*>(a.k);
  const float* vp = reinterpret_cast<const float*>(a.v);
  float q[QC], o[VC];
#pragma unroll
  for (int cc = 0; cc < QC; ++cc)
    q[cc] = qvalid ? qp[(int64_t)(o0 + iq) * a.ld_qk + h * DQK + part * QC + cc] : 0.0f;
#pragma unroll
  for (int cc = 0; cc < VC; ++cc) o[cc] = 0.0f;
  int32_t ti1 = 0;
  int64_t ti64 = 0;
  if (qvalid) {
    if (wide) ti64 = a.ts[o0 + iq];
    else ti1 = a.rel_t[o0 + iq] + 1;
  }

  const int ktiles = (rb1 + F32_BN - 1) / F32_BN;
  for (int kt = 0; kt < ktiles; ++kt) {
    const int j0 = kt * F32_BN;
    const int j1 = min(j0 + F32_BN, n);
    if (j0 >= nh && (j1 <= rb0 || j0 >= rb1)) continue;
    __syncthreads();
    for (int idx = tid; idx < F32_BN * DQK; idx += 256) {
      const int r = idx / DQK, cc = idx % DQK;
      const int j = j0 + r;
      sk[r][cc] = j < n ? kp[(int64_t)(o0 + j) * a.ld_qk + h * DQK + cc] : 0.0f;
    }
    for (int idx = tid; idx < F32_BN * DV; idx += 256) {
      const int r = idx / DV, cc = idx % DV;
      const int j = j0 + r;
      sv[r][cc] = j < n ? vp[(int64_t)(o0 + j) * a.ld_v + h * DV + cc] : 0.0f;
    }
    if (tid < F32_BN) {
      const int j = j0 + tid;
      st[tid] = (j < n && !wide) ? a.rel_t[o0 + j] : 0;
      st64[tid] = (j < n && wide) ? a.ts[o0 + j] : 0;
    }
    __syncthreads();
    for (int jj = 0; jj < F32_BN; ++jj) {
      const int j = j0 + jj;
      float dot = 0.0f;
#pragma unroll
      for (int cc = 0; cc < QC; ++cc) dot = fmaf(q[cc], sk[jj][part * QC + cc], dot);
      dot += __shfl_xor(dot, 1, 64);
      dot += __shfl_xor(dot, 2, 64);
      const bool ok = (j < n) && ((iq < nh) ? (j <= iq) : (j < nh || j == iq)) &&
                      (a.win_local <= 0 || j >= nh || pI - j < a.win_local || j < a.win_global);
      const int bpv = pbucket(pI, min(j, nh), a.nP);
      const int cl = wide ? tclz_wide(ti64, st64[jj]) : tclz_narrow(ti1, st[jj]);
      const float s = dot + spos[bpv] + stime[cl];
      float p = s / (1.0f + __expf(-s));
      p = ok ? p : 0.0f;
#pragma unroll
      for (int cc = 0; cc < VC; ++cc) o[cc] = fmaf(p, sv[jj][part * VC + cc], o[cc]);
    }
  }
  if (!qvalid) return;
  const float inv = 1.0f / (float)(a.norm_mode == 0 ? a.norm_len : n);
  float* op = reinterpret_cast<float*>(a.out);
#pragma unroll
  for (int cc = 0; cc < VC; ++cc)
    op[(int64_t)(o0 + iq) * a.ld_out + h * DV + part * VC + cc] = o[cc] * inv;
}

template <int DQK, int DV>
hipError_t launch_fwd_t(const AttnArgs& a, int dtype, int64_t max_items, hipStream_t st) {
  const int64_t grid = max_items * a.H;
  if (grid <= 0) return hipSuccess;
  if (dtype == HSTU_BF16) {
    if (a.splits > 1 && (a.win_local > 0 || !a.part || !a.part_cnt)) return hipErrorInvalidValue;
    if (a.key_halves && (a.win_local > 0 || a.splits > 1)) return hipErrorInvalidValue;
    if (a.q_mx) {
      // MX scores: d_qk = d_v in {64, 128}, no windows, no key split
      if constexpr (DQK == DV && (DQK == 64 || DQK == 128)) {
        if (a.win_local > 0 || a.splits > 1 || !a.k_mx || !a.q_mxs || !a.k_mxs)
          return hipErrorInvalidValue;
        if (a.key_halves)
          k_attn_fwd_bf16<DQK, DV, false, false, true, true><<<(unsigned)grid, 256, 0, st>>>(a);
        else
          k_attn_fwd_bf16<DQK, DV, false, false, false, true><<<(unsigned)grid, 256, 0, st>>>(a);
        return hipGetLastError();
      } else {
        return hipErrorInvalidValue;
      }
    }
    if (a.win_local > 0)
      k_attn_fwd_bf16<DQK, DV, true, false><<<(unsigned)grid, 256, 0, st>>>(a);
    else if (a.key_halves)
      k_attn_fwd_bf16<DQK, DV, false, false, true><<<(unsigned)grid, 256, 0, st>>>(a);
    else if (a.splits > 1) {
      k_attn_fwd_bf16<DQK, DV, false, true><<<(unsigned)(grid * a.splits), 256, 0, st>>>(a);
      constexpr int BM = FwdShape<DQK, DV>::BM;
      k_attn_fwd_combine<BM, DV><<<(unsigned)(grid * (BM / CMB_ROWS)), 64, 0, st>>>(a);
    } else
      k_attn_fwd_bf16<DQK, DV, false, false><<<(unsigned)grid, 256, 0, st>>>(a);
  } else {
    k_attn_fwd_f32<DQK, DV><<<(unsigned)grid, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <int DQK>
hipError_t launch_fwd_dv(const AttnArgs& a, int dtype, int d_v, int64_t mi, hipStream_t st) {
  switch (d_v) {
    case 32: return launch_fwd_t<DQK, 32>(a, dtype, mi, st);
    case 64: return launch_fwd_t<DQK, 64>(a, dtype, mi, st);
    case 128: return launch_fwd_t<DQK, 128>(a, dtype, mi, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int attn_fwd_block_rows(int dtype, int d_qk, int d_v, bool key_halves) {
  if (dtype != HSTU_BF16) return ATTN_FWD_BM_F32;
  (void)d_qk;
  (void)d_v;
  return key_halves ? 64 : FwdShape<64, 64>::BM;  // the same for every head size
}

int attn_fwd_occupancy(int d_qk, int d_v) {
  return (d_qk <= 64 && d_v <= 64) ? FwdShape<64, 64>::OCC : FwdShape<128, 128>::OCC;
}

hipError_t launch_attn_fwd(const AttnArgs& a, int dtype, int d_qk, int d_v, int64_t max_items,
                           hipStream_t st) {
  switch (d_qk) {
    case 32: return launch_fwd_dv<32>(a, dtype, d_v, max_items, st);
    case 64: return launch_fwd_dv<64>(a, dtype, d_v, max_items, st);
    case 128: return launch_fwd_dv<128>(a, dtype, d_v, max_items, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace hstu
