// Fused HSTU pointwise attention, backward (bf16, gfx950 MFMA).
//
// With s = q_i . k_j + bias, a = SiLU(s)/N and dA = dO_i . v_j for allowed
// pairs, the gradients are dV_j = sum_i a dO_i, dS = dA SiLU'(s) / N,
// dQ_i = sum_j dS k_j, dK_j = sum_i dS q_i and both bias tables receive dS at
// the pair's buckets.  The backward costs about five GEMM-shaped products per
// pair against two in the forward ("DLRMv4 Brings Sequence-Based
// Recommendation Training to MLPerf", Table 7 note).
//
// Two kernels, neither materialising S:
//  * k_attn_bwd_dkdv: one workgroup per (sequence, 128-key block, head), four
//    waves of 32 keys keeping K and V in registers (B operands) and dK, dV in
//    accumulators; it walks the 64-row query tiles that can see its keys
//    (history keys: all later rows including every candidate; candidate keys:
//    only themselves).  Q and dO tiles arrive row-major by buffer->LDS DMA,
//    double-buffered; they are read along rows as A operands of S = Q K^T and
//    dA = dO V^T and down columns (transpose reads) as B operands of
//    dK += dS^T Q and dV += P^T dO.  The rab-table gradients go to LDS
//    histograms: tiles far enough from the keys (position bucket saturated,
//    no mask) keep per-lane running sums flushed when a lane's time bucket
//    changes; the other tiles use LDS atomics.
//  * k_attn_bwd_dq: one workgroup per (sequence, 128-row query block, head),
//    structured like the forward kernel: S^T = K Q^T and dA^T = V dO^T, then
//    dQ += dS K with K read down its columns from the same row-major tile.
//    No atomics on dQ.
// SiLU is evaluated as in the forward kernel, s' = -log2(e) s, sigma =
// 1/(1 + 2^s'), P' = s' sigma = -log2(e) SiLU(s), SiLU'(s) = sigma +
// P' ln2 (sigma - 1); the -ln2 of P' is applied once to dV.
// Optional epilogue (layer backward): each gradient is multiplied by
// SiLU'(Z) of the projection's pre-activation before it is stored.
#include <type_traits>

#include "bias.h"
#include "common.h"
#include "internal.h"
#include "lds.h"

namespace hstu {

namespace {

constexpr int KV_QT = 64;   // query rows per tile in the dK/dV kernel (halves of 32 rows)
constexpr int KV_NH = KV_QT / 32;
constexpr int DQ_BN = 64;   // keys per tile in the dQ kernel

template <bool V>
using bconst = std::integral_constant<bool, V>;

// f(integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time
template <int I, int N, typename F>
HSTU_DEV void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// The value held by the next lane (lane + 1) of each 16-lane row; 0 in the
// last lane of a row (DPP row shift with out-of-row reads bound to zero).
HSTU_DEV float dpp_row_next(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x101, 0xF, 0xF, true));
}

// sigma and P' from the pre-scaled score s' = -log2(e) * (q.k + bias)
HSTU_DEV void silu_parts(float sb, float& sig, float& pp) {
  sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sb));
  pp = sb * sig;
}
// SiLU'(s) from sigma and P'
HSTU_DEV float silu_deriv(float sig, float pp) {
  return fmaf(pp, fmaf(sig, HSTU_LN2, -HSTU_LN2), sig);
}

// Store a 32-row x (32*NB)-column accumulator block (rows 8*(r/4)+4g+r%4,
// column lane%32 of each 32-column block) as bf16, optionally times SiLU'(Z).
// The Z loads use clamped rows so that they issue back to back without
// per-element branches; only the stores are predicated.
template <int NB>
HSTU_DEV void store_grad(const f32x16* acc, float scale, bf16* dst, int64_t ld, int o0,
                         int row0, int n, int col0, const bf16* z, int64_t ldz, int64_t zcol,
                         int ql, int g) {
  float f[NB][16];
#pragma unroll
  for (int d = 0; d < NB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) f[d][r] = scale;
  if (z) {
    bf16 zv[NB][16];
#pragma unroll
    for (int d = 0; d < NB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = min(row0 + 8 * (r >> 2) + 4 * g + (r & 3), n - 1);
        zv[d][r] = z[(int64_t)(o0 + i) * ldz + zcol + d * 32 + ql];
      }
#pragma unroll
    for (int d = 0; d < NB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) f[d][r] *= silu_grad_f((float)zv[d][r]);
  }
#pragma unroll
  for (int d = 0; d < NB; ++d) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = row0 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (i < n) dst[(int64_t)(o0 + i) * ld + col0 + d * 32 + ql] = (bf16)(acc[d][r] * f[d][r]);
    }
  }
}

// ===========================================================================
// dK / dV (key-block major)
// ===========================================================================
// d <= 64: four waves, each a 32-key group holding K, V, dK and dV in
// registers and walking both 32-row halves of every query tile.
// d_qk = d_v = 128 (WIDE): those registers would leave one wave per SIMD, so the
// workgroup has eight waves (two per SIMD): K and V of the 128-key block sit
// in LDS, wave w owns key group w % 4 and row half w / 4 of every tile, and
// the two waves of a key group add their dK, dV partials at the end.
template <int DQK, int DV>
struct KvShape {
  static constexpr bool WIDE = (DQK == 128 && DV == 128);
  static constexpr int NW = WIDE ? 8 : 4;   // waves per workgroup
  static constexpr int NT = 64 * NW;        // threads
  // workgroups per CU the registers allow (mixed widths with a 128 side: one)
  static constexpr int OCC = (WIDE || DQK >= 128 || DV >= 128) ? 1 : 2;
};

// K and V of the workgroup's keys (WIDE shape only; read along rows)
template <int DQK, int DV, bool USED>
struct KvKeys {
  uint8_t k[USED ? PadTile<DQK, false>::bytes(ATTN_BWD_BN) : 16];
  uint8_t v[USED ? PadTile<DV, false>::bytes(ATTN_BWD_BN) : 16];
};

// One staged query tile: row-major Q and dO (filled by DMA, read along rows for
// S and dA and down columns for the dK and dV products) and the row times.
template <int DQK, int DV>
struct KvBuf {
  uint8_t q[PadTile<DQK, true>::bytes(KV_QT)];
  uint8_t o[PadTile<DV, true>::bytes(KV_QT)];
  int32_t t[KV_QT];    // query times relative to the sequence minimum (narrow)
  int64_t t64[KV_QT];  // query times (wide sequences)
};

// Bias tables and gradient histograms (a separate LDS object from the two tile
// buffers, so that the compiler can see that DMA into one buffer never touches
// them or the other buffer and needs no wait before their accesses).
struct KvTables {
  float tpos[1024];   // rab_pos * -log2 e
  float ttime[32];    // rab_time[bucket(c)] * -log2 e, by clz index
  float tfar[32];     // (rab_pos[nP-1] + rab_time[bucket(c)]) * -log2 e
  float gpos[1024];   // d rab_pos histogram (by bucket)
  float gtime[32];    // d rab_time histogram (by clz index)
};

template <int DQK, int DV, bool WIN, bool KEEP_DS = false>
__global__ __launch_bounds__((KvShape<DQK, DV>::NT), (KvShape<DQK, DV>::OCC)) void k_attn_bwd_dkdv(AttnArgs a) {
  constexpr bool WIDE = KvShape<DQK, DV>::WIDE;
  constexpr int NW = KvShape<DQK, DV>::NW, NT = KvShape<DQK, DV>::NT;
  __shared__ __attribute__((aligned(1024))) KvBuf<DQK, DV> kvb0;
  __shared__ __attribute__((aligned(1024))) KvBuf<DQK, DV> kvb1;
  __shared__ __attribute__((aligned(1024))) KvKeys<DQK, DV, WIDE> keys;
  __shared__ KvTables sm;

  const int w = blockIdx.x;
  const int n_items = a.counters[0];
  if (w >= n_items * a.H) return;
  // work-item fields are wave-uniform: keep them in scalar registers so that
  // buffer descriptors built from them need no per-lane handling
  const int it = w / a.H, h = w - it * a.H;
  const int b = __builtin_amdgcn_readfirstlane(a.items[2 * it]);
  const int kb = __builtin_amdgcn_readfirstlane(a.items[2 * it + 1]);
  if (b < 0 || b >= a.B || kb < 0) return;  // not an item of this batch
  const int o0 = __builtin_amdgcn_readfirstlane(a.seq_offsets[b]);
  const int n = __builtin_amdgcn_readfirstlane(a.seq_offsets[b + 1]) - o0;
  const int c = a.num_cand ? __builtin_amdgcn_readfirstlane(a.num_cand[b]) : 0;
  const int nh = n - c;
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
    for (int i = tid; i < nP; i += NT) {
      sm.tpos[i] = rp[i] * HSTU_NEG_LOG2E;
      sm.gpos[i] = 0.0f;
    }
    if (tid < 32) {
      const float tv = rtb[tbucket_from_clz(tid, nT)];
      sm.ttime[tid] = tv * HSTU_NEG_LOG2E;
      sm.tfar[tid] = (rp[nP - 1] + tv) * HSTU_NEG_LOG2E;
      sm.gtime[tid] = 0.0f;
    }
  }

  const int k0 = kb * ATTN_BWD_BN;
  const int k1 = min(k0 + ATTN_BWD_BN, n);
  const int kg = WIDE ? (wave & 3) : wave;  // key group
  const int rh = WIDE ? (wave >> 2) : 0;    // row half of each tile (WIDE)
  const int kw0 = k0 + kg * 32;
  const int kw1 = min(kw0 + 32, n);
  const int jk = kw0 + ql;  // this lane's key
  const bool kvalid = jk < n;
  const int pJ = min(jk, nh);
  const int64_t* tsq = a.ts + o0;
  // key time minus one: tclz_narrow(t_i - tjm) is the bucket of t_i - t_j
  const int32_t tjm = ((kvalid && !wide) ? a.rel_t[o0 + jk] : 0) - 1;
  const int64_t tj64 = (kvalid && wide) ? tsq[jk] : 0;

  const bf16* qh_ = reinterpret_cast<const bf16*>(a.q) + (int64_t)o0 * a.ld_qk + h * DQK;
  const bf16* kh_ = reinterpret_cast<const bf16*>(a.k) + (int64_t)o0 * a.ld_qk + h * DQK;
  const bf16* vh_ = reinterpret_cast<const bf16*>(a.v) + (int64_t)o0 * a.ld_v + h * DV;
  const bf16* doh = reinterpret_cast<const bf16*>(a.dout) + (int64_t)o0 * a.ld_dout + h * DV;

  // kept dS (WIDE shape): the 128 x 128 blocks (key-major) of this key block
  // kb, one per 128-row block rb >= kb (a wave-uniform base; each lane adds
  // its key's row when it stores)
  bf16* ds_kb = nullptr;
  if constexpr (WIDE && KEEP_DS) {
    if (a.ds && __builtin_amdgcn_readfirstlane(*a.ds_flag) == 0) {
      const int64_t nrb = (n + 127) / 128;
      const int64_t blk = __builtin_amdgcn_readfirstlane(a.ds_base[b]) + h * (nrb * (nrb + 1) / 2) +
                          kb * nrb - (int64_t)kb * (kb - 1) / 2 - kb;
      ds_kb = reinterpret_cast<bf16*>(a.ds) + blk * (128 * 128);
    }
  }

  // per-lane byte offsets of the S/dA row operands (row ql of a 32-row block,
  // chunk g; k-chunk ch adds 32 ch bytes): tile rows and (WIDE) key rows
  constexpr int SQ = PadTile<DQK, true>::STRIDE, SO = PadTile<DV, true>::STRIDE;
  constexpr int SK = PadTile<DQK, false>::STRIDE;
  const int roff = ql * SQ + 16 * g;
  const int koff = (kg * 32 + ql) * SK + 16 * g;
  bf16x8 kr[WIDE ? 1 : DQK / 16], vr[WIDE ? 1 : DV / 16];
  if constexpr (WIDE) {
    // the block's K and V rows go to LDS (keys >= n arrive as zeros); complete
    // before the first tile's barrier
    dma_pad_tile<DQK, false, ATTN_BWD_BN, NW>(keys.k, kh_, a.ld_qk, k0, n, wave, lane);
    dma_pad_tile<DV, false, ATTN_BWD_BN, NW>(keys.v, vh_, a.ld_v, k0, n, wave, lane);
  } else {
#pragma unroll
    for (int ch = 0; ch < DQK / 16; ++ch)
      kr[ch] = kvalid ? *reinterpret_cast<const bf16x8*>(kh_ + (int64_t)jk * a.ld_qk + ch * 16 +
                                                         8 * g)
                      : bf16x8{};
#pragma unroll
    for (int ch = 0; ch < DV / 16; ++ch)
      vr[ch] = kvalid ? *reinterpret_cast<const bf16x8*>(vh_ + (int64_t)jk * a.ld_v + ch * 16 +
                                                         8 * g)
                      : bf16x8{};
  }

  f32x16 dk[DQK / 32], dv[DV / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) dk[d] = f32x16{};
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) dv[d] = f32x16{};

  // query tiles: [k0, qend); candidate keys are seen by themselves only
  const int qend = (k0 >= nh) ? k1 : n;
  // DMA of query tile i0 into Bf; rows >= qend arrive as zeros (times: rows >= n)
  auto issue = [&](KvBuf<DQK, DV>& Bf, int i0) HSTU_INLINE_LAMBDA {
    dma_pad_tile<DQK, true, KV_QT, NW>(Bf.q, qh_, a.ld_qk, i0, qend, wave, lane);
    dma_pad_tile<DV, true, KV_QT, NW>(Bf.o, doh, a.ld_dout, i0, qend, wave, lane);
    if (wave < KV_QT / 64) {
      const int r = i0 + 64 * wave;
      if (!wide) dma_words64(Bf.t + 64 * wave, a.rel_t + o0, r, n, lane);
      else dma_dwords64(Bf.t64 + 64 * wave, tsq, r, n, lane);
    }
  };

  // Query tiles split into a near phase (tiles that may need masks or per-element
  // buckets) and a far phase: every row of the tile is at least nP-1 positions
  // after every key of the workgroup and no candidate key is involved, so the
  // position bucket is nP-1 and no mask applies (rows past qend and keys past n
  // are zero-filled and contribute nothing).
  int far_start = qend;
  if (!wide && k1 <= nh) {
    const int need = k1 - 1 + nP - 1;  // first row with p(i) - p(k1-1) >= nP-1
    if (need <= nh) far_start = min(qend, k0 + ((max(need - k0, 0) + KV_QT - 1) / KV_QT) * KV_QT);
  }
  // Semi-local windows (history key j is seen by row i only if p(i) - j < W_l
  // or j < W_g): rows past the window of every key of the block see none of
  // it (unless some key is global or within W_l of the candidates' position),
  // and the far phase keeps only whole tiles whose rows see every key of the
  // block; the rows after it up to qend_w run the masked near body again.
  // WIN: semi-local windows compiled in (otherwise every window term folds away)
  const int wl = WIN ? a.win_local : 0, wg = WIN ? a.win_global : 0;
  int qend_w = qend, fw_end = qend;
  if (wl > 0 && k1 > wg && k1 <= nh) {
    if (k0 >= wg && nh - (k1 - 1) >= wl) qend_w = min(qend, k1 - 1 + wl);
    const int jng = max(k0, wg);  // smallest key subject to the local window
    fw_end = far_start + max((jng + wl - far_start) / KV_QT, 0) * KV_QT;
    fw_end = min(max(fw_end, far_start), qend_w);
  }
  // last row that sees this lane's key: past its local window, unless the key
  // is global or within W_l of the candidates' position
  const int wrow = (wl > 0 && jk >= wg && jk < nh && nh - jk >= wl) ? jk + wl - 1 : (1 << 30);

  // per-lane running sums of the far phase (position bucket nP-1): run_u holds
  // rows of time bucket curB from halves where no lane changes bucket; run_tot
  // and run_a the rows of halves with one change (run_a: those in bucket curB,
  // the rest in curB + 1)
  int curB = -1;
  float run_u = 0.0f, run_tot = 0.0f, run_a = 0.0f, ptot = 0.0f;
  auto flush_time = [&]() HSTU_INLINE_LAMBDA {
    if (curB >= 0) {
      if (run_a + run_u != 0.0f) atomicAdd(&sm.gtime[curB], run_a + run_u);
      if (run_tot - run_a != 0.0f) atomicAdd(&sm.gtime[curB + 1], run_tot - run_a);
    }
    ptot += run_tot + run_u;
    run_u = 0.0f;
    run_tot = 0.0f;
    run_a = 0.0f;
  };

  // S = Q K^T and dA = dO V^T for the 32-row half qh of the staged tile
  auto mm_sd = [&](const KvBuf<DQK, DV>& B, int qh, f32x16& sacc, f32x16& dacc) HSTU_INLINE_LAMBDA {
    sacc = f32x16{};
    dacc = f32x16{};
    if constexpr (WIDE) {
      // both operands from LDS; reads run at most two k-chunks ahead (the
      // other wave on the SIMD covers the latency) to stay within 256 registers.
      // Addresses: the per-lane offsets roff/koff plus constants (tile, row
      // block) that the compiler folds into the instructions' immediates.
      static_assert(DQK == DV, "wide shape");
#pragma unroll
      for (int c2 = 0; c2 < DQK / 16; c2 += 2) {
#pragma unroll
        for (int ch = c2; ch < c2 + 2; ++ch) {
          const bf16x8 qa = *reinterpret_cast<const bf16x8*>(B.q + qh * 32 * SQ + roff + 32 * ch);
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(keys.k + koff + 32 * ch);
          const bf16x8 oa = *reinterpret_cast<const bf16x8*>(B.o + qh * 32 * SO + roff + 32 * ch);
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(keys.v + koff + 32 * ch);
          sacc = mfma32(qa, ka, sacc);
          dacc = mfma32(oa, va, dacc);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      bf16x8 qa[DQK / 16], oa[DV / 16];
#pragma unroll
      for (int ch = 0; ch < DQK / 16; ++ch)
        qa[ch] = *reinterpret_cast<const bf16x8*>(B.q + qh * 32 * SQ + roff + 32 * ch);
#pragma unroll
      for (int ch = 0; ch < DV / 16; ++ch)
        oa[ch] = *reinterpret_cast<const bf16x8*>(B.o + qh * 32 * SO + ql * SO + 16 * g + 32 * ch);
#pragma unroll
      for (int ch = 0; ch < DQK / 16; ++ch) sacc = mfma32(qa[ch], kr[ch], sacc);
#pragma unroll
      for (int ch = 0; ch < DV / 16; ++ch) dacc = mfma32(oa[ch], vr[ch], dacc);
    }
  };
  // dV += P'^T dO ; dK += dS^T Q   (k = the 32 rows of half qh)
  auto mm_grad = [&](const KvBuf<DQK, DV>& B, int qh, const bf16x8 (&pp)[2],
                     const bf16x8 (&dd)[2]) HSTU_INLINE_LAMBDA {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bf16x8 ob[DV / 32], qb[DQK / 32];
#pragma unroll
      for (int d = 0; d < DV / 32; ++d) ob[d] = pad_col8<DV>(B.o, qh * 32 + 16 * u, d * 32, lane);
#pragma unroll
      for (int d = 0; d < DQK / 32; ++d)
        qb[d] = pad_col8<DQK>(B.q, qh * 32 + 16 * u, d * 32, lane);
#pragma unroll
      for (int d = 0; d < DV / 32; ++d) dv[d] = mfma32(pp[u], ob[d], dv[d]);
#pragma unroll
      for (int d = 0; d < DQK / 32; ++d) dk[d] = mfma32(dd[u], qb[d], dk[d]);
    }
  };

  // Element loop of one half: lane = key jk, element r is row ib + kc with
  // kc = 8*(r/4) + r%4; bias_of(kc, t) is pre-scaled, grad_of(kc, t, ds).
  // grad4(aa, x) receives the dS of the four consecutive rows 8 aa + {0..3}.
  auto elems = [&](const KvBuf<DQK, DV>& B, int qh, const f32x16& sacc, const f32x16& dacc,
                   bf16x8 (&pp)[2], bf16x8 (&dd)[2], auto bias_of, auto grad_of, auto masked,
                   int lo, int hi, auto grad4) HSTU_INLINE_LAMBDA {
#pragma unroll
    for (int aa = 0; aa < 4; ++aa) {
      const i32x4 t4 = *reinterpret_cast<const i32x4*>(&B.t[qh * 32 + 8 * aa + 4 * g]);
      float x4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kc = 8 * aa + r;
        const int e = 4 * aa + r;
        const float sb = fmaf(sacc[e], HSTU_NEG_LOG2E, bias_of(kc, t4[r]));
        float sig, p;
        silu_parts(sb, sig, p);
        float ds = dacc[e] * silu_deriv(sig, p);
        if constexpr (decltype(masked)::value) {
          const bool ok = kc >= lo && kc <= hi;
          p = ok ? p : 0.0f;
          ds = ok ? ds : 0.0f;
        }
        grad_of(kc, t4[r], ds);
        x4[r] = ds;
        pp[aa >> 1][(aa & 1) * 4 + r] = (bf16)p;
        dd[aa >> 1][(aa & 1) * 4 + r] = (bf16)ds;
      }
      grad4(aa, x4);
      // masked tiles: keep the table reads of later groups from being hoisted
      // (their addresses and results would all be live at once)
      if constexpr (decltype(masked)::value) __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto no4 = [&](int, const float (&)[4]) HSTU_INLINE_LAMBDA {};

  // The 32-row halves of a staged tile this wave computes: both (d <= 64), or
  // its own (WIDE; one copy of the code with the half index in a register).
  auto for_halves = [&](auto f) HSTU_INLINE_LAMBDA {
    if constexpr (WIDE) {
      f(rh);
    } else {
      static_for<0, KV_NH>([&](auto qhc) HSTU_INLINE_LAMBDA { f(decltype(qhc)::value); });
    }
  };

  // Near-phase rab gradients.  Position buckets below nP-1 differ across the
  // lanes of one element (one key per lane), so their LDS atomics do not
  // collide; saturated elements go to the per-lane sum ptot and masked ones
  // (dS = 0) are skipped.  Time buckets are shared by neighbouring keys, so
  // each lane run-length encodes them instead: along a lane the rows come in
  // order, and the running sum is flushed to the histogram only when the
  // lane's bucket changes (for sorted timestamps a handful of times per tile).
  int nb_cur = 0;
  float nb_acc = 0.0f;
  auto near_pos_grad = [&](int bp, float ds) HSTU_INLINE_LAMBDA {
    if (bp < nP - 1 && ds != 0.0f) atomicAdd(&sm.gpos[bp], ds);
    ptot += (bp >= nP - 1) ? ds : 0.0f;
  };
  auto near_time_grad = [&](int ct, float ds) HSTU_INLINE_LAMBDA {
    if (ct != nb_cur) {
      if (nb_acc != 0.0f) atomicAdd(&sm.gtime[nb_cur], nb_acc);
      nb_acc = 0.0f;
      nb_cur = ct;
    }
    nb_acc += ds;
  };
  // Position gradient of four consecutive rows 8 aa + {0..3} when the bucket is
  // a function of i - j alone (history rows and keys): element (row r, lane l)
  // shares its bucket with (row r + 1, lane l + 1), so the four rows are summed
  // along diagonals within each 16-lane row first (three DPP shifts) and the
  // LDS float atomics, which cost a few clocks per active lane, drop from four
  // full-wave instructions to one plus three at the first lane of each row
  // (whose diagonals leave the row).
  auto near_pos4 = [&](int aa, const float (&x)[4], auto bidx) HSTU_INLINE_LAMBDA {
    const float p3 = x[3];
    const float p2 = x[2] + dpp_row_next(p3);
    const float p1 = x[1] + dpp_row_next(p2);
    const float y = x[0] + dpp_row_next(p1);
    near_pos_grad(bidx(8 * aa), y);
    if ((lane & 15) == 0) {
      near_pos_grad(bidx(8 * aa + 1), p1);
      near_pos_grad(bidx(8 * aa + 2), p2);
      near_pos_grad(bidx(8 * aa + 3), p3);
    }
  };

  // near-phase tile: per-half masks and per-element buckets
  // kept dS of one 32-row half (rows i0 + 32 qh .. of the tile starting at
  // row i0).  Lane (key ql, half g) holds rows 8 aa + 4 g + {0..3}; one swap
  // between the wave's halves (v_permlane32_swap) of the aa = 1 pieces of
  // half 0 and the aa = 0 pieces of half 1 (likewise aa = 3 and 2) leaves
  // each lane eight consecutive rows twice, so a half is two 16-byte stores
  // per lane.  ds_stores counts them for the tile's DMA wait (see run_phase).
  int ds_stores = 0;
  auto store_ds = [&](int i0, int qh, const bf16x8 (&dd)[2]) HSTU_INLINE_LAMBDA {
    if constexpr (WIDE && KEEP_DS) {
      if (ds_kb) {
        ds_stores = 2;
        bf16* dst = ds_kb + (int64_t)(i0 >> 7) * (128 * 128) +
                    (((kg * 32 + (lane & 31)) * 128) + (i0 & 127) + qh * 32 + 8 * (lane >> 5));
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          // dwords 0, 1: rows 16 hh + 4 g + {0..3}; dwords 2, 3: rows 16 hh + 8 + 4 g + {0..3}
          const u32x4 d = __builtin_bit_cast(u32x4, dd[hh]);
          const auto s0 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
          *reinterpret_cast<u32x4*>(dst + 16 * hh) = u32x4{s0[0], s1[0], s0[1], s1[1]};
        }
      }
    }
  };

  auto near_tile = [&](const KvBuf<DQK, DV>& B, int i0) HSTU_INLINE_LAMBDA {
    if (kw0 >= kw1) return;
    for_halves([&](const int qh) HSTU_INLINE_LAMBDA {
      const int ir0 = i0 + qh * 32;
      const int ir1 = min(ir0 + 32, qend);
      bool active;
      if (kw0 < nh) active = ir1 - 1 >= kw0;
      else active = ir0 < kw1 && ir1 > kw0;
      if constexpr (KEEP_DS) {
        if (!active && ir0 < ir1) {
          // every pair of the half is masked: the kept dS block holds zeros there
          const bf16x8 z[2] = {bf16x8{}, bf16x8{}};
          store_ds(i0, qh, z);
        }
      }
      if (!active || ir0 >= ir1) return;
      // window: every row of the half past the window of every key of the wave
      if (wl > 0 && kw0 >= wg && kw1 <= nh && nh - (kw1 - 1) >= wl && ir0 >= kw1 - 1 + wl) return;
      f32x16 sacc, dacc;
      // keep the element loop's address arithmetic out of the product block,
      // which needs the registers for operand read-ahead
      __builtin_amdgcn_sched_barrier(0);
      mm_sd(B, qh, sacc, dacc);
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 pp[2], dd[2];
      const int ib = ir0 + 4 * g;
      // p(i) - p(j) = min(ib + kc, nh) - pJ ; allowed rows: history key -> i >= j,
      // candidate key -> i == j; rows >= qend and keys >= n never.
      const int pd0 = ib - pJ, pdmax = nh - pJ;
      const int d0 = jk - ib;
      const int lo = kvalid ? d0 : 1 << 20;
      // window: rows past the key's local window, unless the key is global or
      // within W_l of the candidates' position (then every row may see it)
      const int hi = min(min(jk < nh ? (1 << 20) : d0, qend - 1 - ib), wrow - ib);
      auto bidx = [&](int kc) HSTU_INLINE_LAMBDA { return min(max(min(pd0 + kc, pdmax), 0), nP - 1); };
      // history keys and rows (or masked rows): the bucket depends on i - j only
      const bool diag = k1 <= nh && min(ir0 + 32, qend) <= nh;
      if (!wide) {
        elems(B, qh, sacc, dacc, pp, dd,
              [&](int kc, int32_t t) { return sm.tpos[bidx(kc)] + sm.ttime[tclz_narrow(t, tjm)]; },
              [&](int, int32_t t, float ds) { near_time_grad(tclz_narrow(t, tjm), ds); },
              bconst<true>{}, lo, hi, [&](int aa, const float (&x)[4]) {
                if (diag) {
                  near_pos4(aa, x, bidx);
                } else {
#pragma unroll
                  for (int r = 0; r < 4; ++r) near_pos_grad(bidx(8 * aa + r), x[r]);
                }
              });
      } else {
        elems(B, qh, sacc, dacc, pp, dd,
              [&](int kc, int32_t) {
                return sm.tpos[bidx(kc)] +
                       sm.ttime[tclz_wide(B.t64[qh * 32 + 4 * g + kc], tj64)];
              },
              [&](int kc, int32_t, float ds) {
                near_pos_grad(bidx(kc), ds);
                near_time_grad(tclz_wide(B.t64[qh * 32 + 4 * g + kc], tj64), ds);
              },
              bconst<true>{}, lo, hi, no4);
      }
      store_ds(i0, qh, dd);
      mm_grad(B, qh, pp, dd);
    });
  };

  // far-phase tile: no masks, position bucket nP-1; with sorted timestamps a
  // lane's time bucket changes at most once inside a half in the common case
  auto far_tile = [&](const KvBuf<DQK, DV>& B, int i0) HSTU_INLINE_LAMBDA {
    if (kw0 >= kw1) return;
    for_halves([&](const int qh) HSTU_INLINE_LAMBDA {
      const int ir0 = i0 + qh * 32;
      if (ir0 >= qend) return;
      const int last = min(31, qend - 1 - ir0);
      const int cF = tclz_narrow(B.t[qh * 32 + last], tjm);
      const int cL = tclz_narrow(B.t[qh * 32], tjm);
      const bool uni = __all(!kvalid || (sorted && cL == cF));
      const bool one = __all(!kvalid || (sorted && cL - cF <= 1));
      f32x16 sacc, dacc;
      mm_sd(B, qh, sacc, dacc);
      bf16x8 pp[2], dd[2];
      if (uni) {
        // every lane sees one time bucket on this half: constant bias, one sum
        if (kvalid && cF != curB) {
          flush_time();
          curB = cF;
        }
        const float ba = sm.tfar[cF];
        elems(B, qh, sacc, dacc, pp, dd, [&](int, int32_t) { return ba; },
              [&](int, int32_t, float ds) { run_u += ds; }, bconst<false>{}, 0, 0, no4);
      } else if (one) {
        if (kvalid && cF != curB) {
          flush_time();
          curB = cF;
        }
        const float ba = sm.tfar[cF], bb = sm.tfar[min(cF + 1, 31)];
        // rows with t >= thr are in bucket cF, the others in cF + 1
        const int32_t thr = (cL == cF) ? INT32_MIN : tjm + (1 << (31 - cF));
        elems(B, qh, sacc, dacc, pp, dd, [&](int, int32_t t) { return t >= thr ? ba : bb; },
              [&](int, int32_t t, float ds) {
                run_tot += ds;
                run_a += t >= thr ? ds : 0.0f;
              },
              bconst<false>{}, 0, 0, no4);
      } else {
        elems(B, qh, sacc, dacc, pp, dd,
              [&](int, int32_t t) { return sm.tfar[tclz_narrow(t, tjm)]; },
              [&](int, int32_t t, float ds) {
                ptot += ds;
                atomicAdd(&sm.gtime[tclz_narrow(t, tjm)], ds);
              },
              bconst<false>{}, 0, 0, no4);
      }
      store_ds(i0, qh, dd);
      mm_grad(B, qh, pp, dd);
    });
  };

  // double-buffered tile pipeline over [ibeg, iend) in steps of KV_QT, jumping
  // from tile sk0 to tile sk1: the DMA of tile t+1 runs while tile t is
  // computed (unrolled by two so that every access names its buffer statically)
  auto run_phase = [&](int ibeg, int iend, auto body, int sk0, int sk1) HSTU_INLINE_LAMBDA {
    if (ibeg >= iend) return;
    auto next_row = [&](int i) HSTU_INLINE_LAMBDA {
      i += KV_QT;
      return (i >= sk0 && i < sk1) ? sk1 : i;
    };
    // The next tile's DMA is issued before the body, whose only vector-memory
    // operations are the two kept-dS stores (when a half stored them).  The
    // vector-memory counter retires in issue order, so vmcnt(2) means the DMA
    // has landed while the stores may still be in flight.
    auto tile_wait = [&]() HSTU_INLINE_LAMBDA {
      if constexpr (KEEP_DS) {
        if (ds_stores == 2) __builtin_amdgcn_s_waitcnt(0x0F72);  // vmcnt(2)
        else dma_wait();
        ds_stores = 0;
      } else {
        dma_wait();
      }
    };
    issue(kvb0, ibeg);
    dma_wait();
    __syncthreads();
    for (int i0 = ibeg; i0 < iend;) {
      const int i1 = next_row(i0);
      if (i1 < iend) issue(kvb1, i1);
      body(kvb0, i0);
      tile_wait();
      __syncthreads();
      if (i1 >= iend) break;
      const int i2 = next_row(i1);
      if (i2 < iend) issue(kvb0, i2);
      body(kvb1, i1);
      tile_wait();
      __syncthreads();
      i0 = i2;
    }
  };
  run_phase(k0, qend_w, near_tile, far_start, fw_end);
  if (nb_acc != 0.0f) atomicAdd(&sm.gtime[nb_cur], nb_acc);
  run_phase(far_start, fw_end, far_tile, 0, 0);
  flush_time();
  if (ptot != 0.0f) atomicAdd(&sm.gpos[nP - 1], ptot);

  if constexpr (WIDE) {
    // the row-half-1 waves hand their dK, dV partials to the row-half-0 waves
    // of the same key group through LDS (tile buffers and key block are free
    // after the last barrier of the tile loop)
    dma_wait();  // the key-block DMA, if no tile ran
    __syncthreads();
    float* xk = reinterpret_cast<float*>(kg < 2 ? (uint8_t*)keys.k : (uint8_t*)keys.v) +
                (kg & 1) * (DQK / 32) * 16 * 64;
    float* xv = reinterpret_cast<float*>(kg < 2 ? (uint8_t*)&kvb0 : (uint8_t*)&kvb1) +
                (kg & 1) * (DV / 32) * 16 * 64;
    static_assert((DQK / 32) * 16 * 64 * 4 * 2 <= (int)sizeof(KvKeys<DQK, DV, WIDE>) / 2 || !WIDE,
                  "dK exchange fits the key block");
    static_assert((DV / 32) * 16 * 64 * 4 * 2 <= (int)sizeof(kvb0.q) + (int)sizeof(kvb0.o) || !WIDE,
                  "dV exchange fits a tile buffer");
    if (rh == 1) {
#pragma unroll
      for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) xk[(d * 16 + r) * 64 + lane] = dk[d][r];
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) xv[(d * 16 + r) * 64 + lane] = dv[d][r];
    }
    __syncthreads();
    if (rh == 0) {
#pragma unroll
      for (int d = 0; d < DQK / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) dk[d][r] += xk[(d * 16 + r) * 64 + lane];
#pragma unroll
      for (int d = 0; d < DV / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) dv[d][r] += xv[(d * 16 + r) * 64 + lane];
    }
  }
  const float invN = 1.0f / (float)(a.norm_mode == 0 ? a.norm_len : n);
  if (kw0 < kw1 && rh == 0) {
    store_grad<DQK / 32>(dk, invN, reinterpret_cast<bf16*>(a.dk), a.ld_qk, o0, kw0, n, h * DQK,
                         reinterpret_cast<const bf16*>(a.zpre), a.ld_z, a.zk_col + h * DQK, ql,
                         g);
    store_grad<DV / 32>(dv, -HSTU_LN2 * invN, reinterpret_cast<bf16*>(a.dv), a.ld_v, o0, kw0, n,
                        h * DV, reinterpret_cast<const bf16*>(a.zpre), a.ld_z,
                        a.zv_col + h * DV, ql, g);
  }
  __syncthreads();
  float* gp = a.drab_pos + h * a.rab_stride;
  float* gt = a.drab_time + h * a.rab_stride;
  for (int i = tid; i < nP; i += NT)
    if (sm.gpos[i] != 0.0f) atomicAdd(&gp[i], sm.gpos[i] * invN);
  if (tid < 32 && sm.gtime[tid] != 0.0f)
    atomicAdd(&gt[tbucket_from_clz(tid, nT)], sm.gtime[tid] * invN);
}

// ===========================================================================
// dQ (query-block major)
// ===========================================================================
// One staged key tile: row-major K (A of S^T = K Q^T along rows, B of
// dQ += dS K down columns) and V (A of dA^T = V dO^T), and the key times.
// Padded rows (PadTile): K is read both ways, V along rows only.
template <int DQK, int DV>
struct DqBuf {
  uint8_t k[PadTile<DQK, true>::bytes(DQ_BN)];
  uint8_t v[PadTile<DV, false>::bytes(DQ_BN)];
  int32_t t[DQ_BN];    // key times relative to the sequence minimum (narrow)
  int64_t t64[DQ_BN];  // key times (wide sequences)
};

struct DqTables {
  float tpos[1024];
  float ttime[32];
  float tfar[32];
};

template <int DQK, int DV, bool WIN>
__global__ __launch_bounds__(256, 2) void k_attn_bwd_dq(AttnArgs a) {
  // dS kept by the dK/dV kernel: dQ comes from k_attn_bwd_dq_ds instead
  if (a.ds_flag && __builtin_amdgcn_readfirstlane(*a.ds_flag) == 0) return;
  __shared__ __attribute__((aligned(1024))) DqBuf<DQK, DV> dqb0;
  __shared__ __attribute__((aligned(1024))) DqBuf<DQK, DV> dqb1;
  __shared__ DqTables sm;

  const int w = blockIdx.x;
  const int n_items = a.counters[0];
  if (w >= n_items * a.H) return;
  const int it = w / a.H, h = w - it * a.H;
  const int b = __builtin_amdgcn_readfirstlane(a.items[2 * it]);
  const int m = __builtin_amdgcn_readfirstlane(a.items[2 * it + 1]);
  if (b < 0 || b >= a.B || m < 0) return;  // not an item of this batch
  const int o0 = __builtin_amdgcn_readfirstlane(a.seq_offsets[b]);
  const int n = __builtin_amdgcn_readfirstlane(a.seq_offsets[b + 1]) - o0;
  const int c = a.num_cand ? __builtin_amdgcn_readfirstlane(a.num_cand[b]) : 0;
  const int nh = n - c;
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
    for (int i = tid; i < nP; i += 256) sm.tpos[i] = rp[i] * HSTU_NEG_LOG2E;
    if (tid < 32) {
      const float tv = rtb[tbucket_from_clz(tid, nT)];
      sm.ttime[tid] = tv * HSTU_NEG_LOG2E;
      sm.tfar[tid] = (rp[nP - 1] + tv) * HSTU_NEG_LOG2E;
    }
  }
  const int rb0 = m * ATTN_BWD_BM;
  const int rb1 = min(rb0 + ATTN_BWD_BM, n);
  const int r0 = rb0 + wave * 32;
  const int rw1 = min(r0 + 32, n);
  const int iq = r0 + ql;
  const bool qvalid = iq < n;
  const int pI = min(iq, nh);
  const int64_t* tsq = a.ts + o0;
  const int32_t ti1 = (qvalid && !wide) ? a.rel_t[o0 + iq] + 1 : 0;
  const int64_t tq64 = (qvalid && wide) ? tsq[iq] : 0;

  const bf16* qb = reinterpret_cast<const bf16*>(a.q) + (int64_t)o0 * a.ld_qk + h * DQK;
  const bf16* kh_ = reinterpret_cast<const bf16*>(a.k) + (int64_t)o0 * a.ld_qk + h * DQK;
  const bf16* vh_ = reinterpret_cast<const bf16*>(a.v) + (int64_t)o0 * a.ld_v + h * DV;
  const bf16* dob = reinterpret_cast<const bf16*>(a.dout) + (int64_t)o0 * a.ld_dout + h * DV;
  bf16x8 qr[DQK / 16], orr[DV / 16];
#pragma unroll
  for (int ch = 0; ch < DQK / 16; ++ch)
    qr[ch] = qvalid ? *reinterpret_cast<const bf16x8*>(qb + (int64_t)iq * a.ld_qk + ch * 16 + 8 * g)
                    : bf16x8{};
#pragma unroll
  for (int ch = 0; ch < DV / 16; ++ch)
    orr[ch] = qvalid ? *reinterpret_cast<const bf16x8*>(dob + (int64_t)iq * a.ld_dout + ch * 16 +
                                                        8 * g)
                     : bf16x8{};
  f32x16 dq[DQK / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) dq[d] = f32x16{};

  const int ktiles = (rb1 + DQ_BN - 1) / DQ_BN;
  // semi-local windows: history key j is allowed for row i only if
  // j >= p(i) - W_l + 1 or j < W_g; tiles past the global window and below
  // the band of every row of the workgroup hold no allowed pair
  // WIN: semi-local windows compiled in (otherwise every window term folds away)
  const int wl = WIN ? a.win_local : 0, wg = WIN ? a.win_global : 0;
  const int gtiles = (wg + DQ_BN - 1) / DQ_BN;
  const int btile = (wl > 0 ? max(min(rb0, nh) - wl + 1, 0) : 0) / DQ_BN;
  auto first_from = [&](int kt) HSTU_INLINE_LAMBDA {
    if (wl > 0 && kt >= gtiles && kt < btile) kt = btile;
    const int j0 = kt * DQ_BN;
    if (j0 >= nh && j0 + DQ_BN <= rb0) kt = rb0 / DQ_BN;  // only other candidates' keys
    return kt;
  };
  auto next_tile = [&](int kt) HSTU_INLINE_LAMBDA { return first_from(kt + 1); };

  // DMA of key tile kt; keys >= n arrive as zeros
  auto issue = [&](DqBuf<DQK, DV>& Bf, int kt) HSTU_INLINE_LAMBDA {
    const int j0 = kt * DQ_BN;
    dma_pad_tile<DQK, true, DQ_BN, 4>(Bf.k, kh_, a.ld_qk, j0, n, wave, lane);
    dma_pad_tile<DV, false, DQ_BN, 4>(Bf.v, vh_, a.ld_v, j0, n, wave, lane);
    if (wave == 0) {
      if (!wide) dma_words64(Bf.t, a.rel_t + o0, j0, n, lane);
      else dma_dwords64(Bf.t64, tsq, j0, n, lane);
    }
  };

  auto body = [&](const DqBuf<DQK, DV>& B, int kt) HSTU_INLINE_LAMBDA {
    const int j0 = kt * DQ_BN;
    const int j1 = min(j0 + DQ_BN, n);
    const bool hist_rows = r0 < nh;
    const bool cand_rows = rw1 > nh;
    const int band_lo = wl > 0 ? min(r0, nh) - wl + 1 : 0;
    const int band_hi = wl > 0 ? min(rw1 - 1, nh) - wl + 1 : 0;
    const bool win_out = wl > 0 && j0 >= wg && j1 - 1 < band_lo && j1 <= nh;
    const bool active = (r0 < rw1) && !win_out &&
                        ((hist_rows && j0 <= min(rw1, nh) - 1) ||
                         (cand_rows && (j0 < nh || (j0 < rw1 && j1 > max(r0, nh)))));
    if (!active) return;
    const bool win_mask = wl > 0 && j1 > wg && j0 < band_hi;
    const bool need_mask = (hist_rows && j1 - 1 > r0) || (j1 > nh) || win_mask;
    const bool far = !need_mask && !wide && (min(r0, nh) - min(j1 - 1, nh) >= nP - 1);
    int mode = 3;  // 0 constant per row, 1 one threshold, 2 gather, 3 general
    int cF = 0, cL = 0;
    if (far) {
      cF = tclz_narrow(ti1, B.t[0]);
      cL = tclz_narrow(ti1, B.t[j1 - 1 - j0]);
      mode = __all(sorted && cL == cF) ? 0 : (__all(sorted && cL - cF <= 1) ? 1 : 2);
    }
    const float ba = sm.tfar[cF], bb = sm.tfar[min(cF + 1, 31)];
    const int32_t thr = (cL == cF) ? INT32_MAX : ti1 - (1 << (31 - cF));
    const int dI = pI - j0 - 4 * g, pmin = pI - nh;
    const int lim = (iq < nh ? iq : nh - 1) - j0 - 4 * g, slf = iq - j0 - 4 * g;
    // window: keys >= wlo (local band) or < wgl (global window) pass
    const int wlo = (wl > 0 ? pI - wl + 1 : INT32_MIN / 2) - j0 - 4 * g;
    const int wgl = wg - j0 - 4 * g;

#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x16 sacc = f32x16{}, dacc = f32x16{};
      {
        bf16x8 ka[DQK / 16], va[DV / 16];
#pragma unroll
        for (int ch = 0; ch < DQK / 16; ++ch) ka[ch] = pad_row8<DQK, true>(B.k, hf * 32 + ql, ch, g);
#pragma unroll
        for (int ch = 0; ch < DV / 16; ++ch) va[ch] = pad_row8<DV, false>(B.v, hf * 32 + ql, ch, g);
#pragma unroll
        for (int ch = 0; ch < DQK / 16; ++ch) sacc = mfma32(ka[ch], qr[ch], sacc);
#pragma unroll
        for (int ch = 0; ch < DV / 16; ++ch) dacc = mfma32(va[ch], orr[ch], dacc);
      }
      bf16x8 dsk[2];
      auto elems = [&](auto bias_of, auto masked) HSTU_INLINE_LAMBDA {
#pragma unroll
        for (int aa = 0; aa < 4; ++aa) {
          const int kk0 = hf * 32 + 8 * aa + 4 * g;
          const i32x4 tj = *reinterpret_cast<const i32x4*>(&B.t[kk0]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int kc = hf * 32 + 8 * aa + r;
            const float sb = fmaf(sacc[4 * aa + r], HSTU_NEG_LOG2E, bias_of(kc, tj[r]));
            float sig, p;
            silu_parts(sb, sig, p);
            float ds = dacc[4 * aa + r] * silu_deriv(sig, p);
            if constexpr (decltype(masked)::value) {
              bool ok = kc <= lim || kc == slf;
              if constexpr (WIN) ok = ok && (kc >= wlo || kc < wgl);
              ds = ok ? ds : 0.0f;
            }
            dsk[aa >> 1][(aa & 1) * 4 + r] = (bf16)ds;
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      auto bgen = [&](int kc) HSTU_INLINE_LAMBDA { return min(max(max(dI - kc, pmin), 0), nP - 1); };
      if (mode == 0) {
        elems([&](int, int32_t) { return ba; }, bconst<false>{});
      } else if (mode == 1) {
        elems([&](int, int32_t t) { return t <= thr ? ba : bb; }, bconst<false>{});
      } else if (mode == 2) {
        elems([&](int, int32_t t) { return sm.tfar[tclz_narrow(ti1, t)]; }, bconst<false>{});
      } else if (!wide) {
        auto bias = [&](int kc, int32_t t) HSTU_INLINE_LAMBDA {
          return sm.tpos[bgen(kc)] + sm.ttime[tclz_narrow(ti1, t)];
        };
        if (need_mask) elems(bias, bconst<true>{});
        else elems(bias, bconst<false>{});
      } else {
        elems([&](int kc, int32_t) {
                return sm.tpos[bgen(kc)] + sm.ttime[tclz_wide(tq64, B.t64[kc + 4 * g])];
              },
              bconst<true>{});
      }
      // dQ += dS K: K read down its columns (keys are the k index)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 kb[DQK / 32];
#pragma unroll
        for (int d = 0; d < DQK / 32; ++d) kb[d] = pad_col8<DQK>(B.k, hf * 32 + 16 * u, d * 32, lane);
#pragma unroll
        for (int d = 0; d < DQK / 32; ++d) dq[d] = mfma32(dsk[u], kb[d], dq[d]);
      }
    }
  };

  // double-buffered key-tile pipeline, unrolled by two so that every access
  // names its buffer statically
  int kt = first_from(0);
  if (kt < ktiles) issue(dqb0, kt);
  dma_wait();
  __syncthreads();
  while (kt < ktiles) {
    int nk = next_tile(kt);
    if (nk < ktiles) issue(dqb1, nk);
    body(dqb0, kt);
    dma_wait();
    __syncthreads();
    kt = nk;
    if (kt >= ktiles) break;
    nk = next_tile(kt);
    if (nk < ktiles) issue(dqb0, nk);
    body(dqb1, kt);
    dma_wait();
    __syncthreads();
    kt = nk;
  }
  if (r0 >= rw1) return;
  const float invN = 1.0f / (float)(a.norm_mode == 0 ? a.norm_len : n);
  store_grad<DQK / 32>(dq, invN, reinterpret_cast<bf16*>(a.dq), a.ld_qk, o0, r0, n, h * DQK,
                       reinterpret_cast<const bf16*>(a.zpre), a.ld_z, a.zq_col + h * DQK, ql, g);
}

// ===========================================================================
// dQ from the kept dS (d_qk = 128): dQ_i = (1/N) sum_j dS_ij k_j as a tiled
// product over the causal 128 x 128 blocks, with no recomputation of S, dA
// or the SiLU terms.  Workgroup = (sequence, 128-row block rb, head), four
// waves of 64 rows x 64 columns.  Per 64-key step the dS block rows (keys)
// and the K rows arrive by DMA (rows past the sequence as zeros) and both are
// read down their columns (transpose reads, the same k order for both).
// Key blocks that hold only candidates are skipped except the diagonal one
// (a candidate key is seen by its own row only).
// ===========================================================================
__global__ __launch_bounds__(256, 2) void k_attn_bwd_dq_ds(AttnArgs a) {
  constexpr int D = 128;
  constexpr int TB = SwzTile<128>::bytes(64);  // one 64-key stage of dS or K
  __shared__ __attribute__((aligned(1024))) uint8_t ta0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t tb0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t ta1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t tb1[TB];
  if (__builtin_amdgcn_readfirstlane(*a.ds_flag) != 0) return;
  const int w = blockIdx.x;
  const int n_items = a.counters[0];
  if (w >= n_items * a.H) return;
  const int it = w / a.H, h = w - it * a.H;
  const int b = __builtin_amdgcn_readfirstlane(a.items[2 * it]);
  const int rb = __builtin_amdgcn_readfirstlane(a.items[2 * it + 1]);
  if (b < 0 || b >= a.B || rb < 0) return;  // not an item of this batch
  const int o0 = __builtin_amdgcn_readfirstlane(a.seq_offsets[b]);
  const int n = __builtin_amdgcn_readfirstlane(a.seq_offsets[b + 1]) - o0;
  const int c = a.num_cand ? __builtin_amdgcn_readfirstlane(a.num_cand[b]) : 0;
  const int nh = n - c;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, ql = lane & 31, g = lane >> 5;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t nrb = (n + 127) / 128;
  const bf16* base = reinterpret_cast<const bf16*>(a.ds) +
                     (__builtin_amdgcn_readfirstlane(a.ds_base[b]) + h * (nrb * (nrb + 1) / 2)) *
                         (128 * 128);
  const bf16* kh_ = reinterpret_cast<const bf16*>(a.k) + (int64_t)o0 * a.ld_qk + h * D;
  // key blocks: the history blocks below rb, then rb itself (blocks holding
  // only candidates are seen by their own rows only); a step is one 64-key
  // half of a block, step index q -> block kb(q), half q & 1
  const int kh_end = min(rb, (nh + 127) / 128);
  const int nsteps = 2 * (kh_end + 1);
  auto step_kb = [&](int q) HSTU_INLINE_LAMBDA { return (q >> 1) < kh_end ? (q >> 1) : rb; };
  auto step_rows = [&](int q) HSTU_INLINE_LAMBDA {
    return min(64, n - (step_kb(q) * 128 + 64 * (q & 1)));
  };
  auto issue = [&](uint8_t* ta, uint8_t* tb, int q) HSTU_INLINE_LAMBDA {
    const int kb = step_kb(q);
    const int krow = kb * 128 + 64 * (q & 1);
    const int rlim = step_rows(q);
    const bf16* blk = base + (kb * nrb - (int64_t)kb * (kb - 1) / 2 + rb - kb) * (128 * 128);
    // dS is read once: non-temporal, so that the K tiles the other row
    // blocks of the sequence re-read stay in the L2
    dma_tile<128, 64, 4, 2>(ta, blk + 64 * (q & 1) * 128, 128, 0, rlim, wave, lane);
    dma_tile<128, 64, 4>(tb, kh_ + (int64_t)krow * a.ld_qk, a.ld_qk, 0, rlim, wave, lane, D);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  auto compute = [&](const uint8_t* ta, const uint8_t* tb) HSTU_INLINE_LAMBDA {
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = lds_col8<128>(ta, 16 * kc, wm * 64 + 32 * i, lane);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = lds_col8<128>(tb, 16 * kc, wn * 64 + 32 * j, lane);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
  };

  // double buffer over the steps (a second half past the sequence's end has
  // no rows and is skipped), unrolled by two so that every access names its
  // stage statically
  auto next_step = [&](int q) HSTU_INLINE_LAMBDA {
    ++q;
    while (q < nsteps && step_rows(q) <= 0) ++q;
    return q;
  };
  int q = next_step(-1);
  if (q < nsteps) issue(ta0, tb0, q);
  dma_wait();
  __syncthreads();
  while (q < nsteps) {
    int nq = next_step(q);
    if (nq < nsteps) issue(ta1, tb1, nq);
    compute(ta0, tb0);
    dma_wait();
    __syncthreads();
    q = nq;
    if (q >= nsteps) break;
    nq = next_step(q);
    if (nq < nsteps) issue(ta0, tb0, nq);
    compute(ta1, tb1);
    dma_wait();
    __syncthreads();
    q = nq;
  }
  const float invN = 1.0f / (float)(a.norm_mode == 0 ? a.norm_len : n);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row0 = rb * 128 + wm * 64 + 32 * i;
    if (row0 >= n) continue;
    store_grad<2>(acc[i], invN, reinterpret_cast<bf16*>(a.dq), a.ld_qk, o0, row0, n,
                  h * D + wn * 64, reinterpret_cast<const bf16*>(a.zpre), a.ld_z,
                  a.zq_col + h * D + wn * 64, ql, g);
  }
}

template <int DQK, int DV>
hipError_t launch_kv_t(const AttnArgs& a, int64_t mi, hipStream_t st) {
  const int64_t grid = mi * a.H;
  if (grid <= 0) return hipSuccess;
  if (a.win_local > 0) k_attn_bwd_dkdv<DQK, DV, true><<<(unsigned)grid, KvShape<DQK, DV>::NT, 0, st>>>(a);
  else if (a.ds && DQK == 128 && DV == 128)
    k_attn_bwd_dkdv<DQK, DV, false, true><<<(unsigned)grid, KvShape<DQK, DV>::NT, 0, st>>>(a);
  else k_attn_bwd_dkdv<DQK, DV, false><<<(unsigned)grid, KvShape<DQK, DV>::NT, 0, st>>>(a);
  return hipGetLastError();
}
template <int DQK, int DV>
hipError_t launch_dq_t(const AttnArgs& a, int64_t mi, hipStream_t st) {
  const int64_t grid = mi * a.H;
  if (grid <= 0) return hipSuccess;
  if (a.win_local > 0) k_attn_bwd_dq<DQK, DV, true><<<(unsigned)grid, 256, 0, st>>>(a);
  else k_attn_bwd_dq<DQK, DV, false><<<(unsigned)grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

#define HSTU_DISPATCH_D(FN, DQK_, DV_, ...)                         \
  switch (DQK_ * 1000 + DV_) {                                     \
    case 32032: return FN<32, 32>(__VA_ARGS__);                    \
    case 32064: return FN<32, 64>(__VA_ARGS__);                    \
    case 32128: return FN<32, 128>(__VA_ARGS__);                   \
    case 64032: return FN<64, 32>(__VA_ARGS__);                    \
    case 64064: return FN<64, 64>(__VA_ARGS__);                    \
    case 64128: return FN<64, 128>(__VA_ARGS__);                   \
    case 128032: return FN<128, 32>(__VA_ARGS__);                  \
    case 128064: return FN<128, 64>(__VA_ARGS__);                  \
    case 128128: return FN<128, 128>(__VA_ARGS__);                 \
  }                                                                \
  return hipErrorInvalidValue;

}  // namespace

hipError_t launch_attn_bwd_dkdv(const AttnArgs& a, int d_qk, int d_v, int64_t mi,
                                hipStream_t st) {
  HSTU_DISPATCH_D(launch_kv_t, d_qk, d_v, a, mi, st)
}
hipError_t launch_attn_bwd_dq(const AttnArgs& a, int d_qk, int d_v, int64_t mi, hipStream_t st) {
  if (a.ds) {
    // from the kept dS when it fit (the recomputing kernel then exits at once)
    if (d_qk != 128 || d_v != 128) return hipErrorInvalidValue;
    if (mi * a.H > 0) k_attn_bwd_dq_ds<<<(unsigned)(mi * a.H), 256, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  HSTU_DISPATCH_D(launch_dq_t, d_qk, d_v, a, mi, st)
}

}  // namespace hstu
