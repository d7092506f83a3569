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
//    waves of 32 keys keeping K and V in registers and dK, dV in accumulators;
//    it walks the 64-row query tiles that can see its keys (history keys: all
//    later rows including every candidate; candidate keys: only themselves),
//    recomputes S and dA on MFMA, and accumulates the rab-table gradients in
//    LDS histograms (tile sums where the position bucket is constant,
//    bucket-range reductions for the time buckets of far tiles, LDS atomics
//    near the diagonal).
//  * k_attn_bwd_dq: one workgroup per (sequence, 128-row query block, head),
//    structured like the forward kernel; it recomputes S^T and dA^T and
//    accumulates dQ = dS K with K^T staged in LDS.  No atomics on dQ.
// Optional epilogue (layer backward): each gradient is multiplied by
// SiLU'(Z) of the projection's pre-activation before it is stored.
#include "bias.h"
#include "common.h"
#include "internal.h"

namespace hstu {

namespace {

constexpr int KV_QT = 64;   // query rows per tile in the dK/dV kernel
constexpr int DQ_BN = 64;   // keys per tile in the dQ kernel

HSTU_DEV float silu_from_parts(float s, float& sig) {
  sig = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(s * HSTU_NEG_LOG2E));
  return s * sig;
}

template <int DQK, int DV>
struct KvSmem {
  using QT = LdsTile<DQK>;
  using OT = LdsTile<DV>;
  using TT = LdsTile<KV_QT>;
  uint32_t q[QT::S_DW * KV_QT];    // Q tile row-major  (A operand of S = Q K^T)
  uint32_t qt[TT::S_DW * DQK];     // Q tile transposed (B operand of dK += dS^T Q)
  uint32_t o[OT::S_DW * KV_QT];    // dO tile row-major (A operand of dA = dO V^T)
  uint32_t ot[TT::S_DW * DV];      // dO tile transposed (B operand of dV += P^T dO)
  int32_t t1[KV_QT];               // query times + 1 (narrow path)
  float tpos[1024];
  float ttime[32];
  float gpos[1024];                // d rab_pos histogram (by bucket)
  float gtime[32];                 // d rab_time histogram (by clz index)
};

// Stage rows [i0, i0+RT) of a [*, ld] bf16 matrix (columns col0..col0+D) into
// a row-major tile and a transposed tile (rows = channels, columns = kperm(row)).
template <int D, int RT>
HSTU_DEV void stage_both(const bf16* base, int64_t ld, int o0, int i0, int n, int col0,
                         uint32_t* rm, uint32_t* tr, int tid) {
  using RM = LdsTile<D>;
  using TR = LdsTile<RT>;
  // row-major copy
  constexpr int CPR = D / 8;
#pragma unroll
  for (int s = 0; s < (RT * CPR + 255) / 256; ++s) {
    const int idx = tid + 256 * s;
    if (idx < RT * CPR) {
      const int row = idx / CPR, ch = idx % CPR;
      const int i = i0 + row;
      u32x4 val = {0, 0, 0, 0};
      if (i < n) val = ld16(base + (int64_t)(o0 + i) * ld + col0 + ch * 8);
      *reinterpret_cast<u32x4*>(&rm[RM::off(row, ch * 4)]) = val;
    }
  }
  // transposed copy
  constexpr int NCH = D / 8;
  constexpr int NITEM = (RT / 2) * NCH;
#pragma unroll
  for (int s = 0; s < (NITEM + 255) / 256; ++s) {
    const int idx = tid + 256 * s;
    if (idx < NITEM) {
      int kp, cc;
      if (NCH >= 8) {
        const int rest = idx >> 6;
        kp = (rest & 3) * 8 + ((idx >> 3) & 7);
        cc = (rest >> 2) * 8 + (idx & 7);
      } else {
        cc = idx % NCH;
        kp = idx / NCH;
      }
      const int i = i0 + 2 * kp;
      u32x4 va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
      if (i < n) va = ld16(base + (int64_t)(o0 + i) * ld + col0 + cc * 8);
      if (i + 1 < n) vb = ld16(base + (int64_t)(o0 + i + 1) * ld + col0 + cc * 8);
      const int col = kperm(2 * kp) >> 1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tr[TR::off(cc * 8 + 2 * e, col)] = (va[e] & 0xFFFFu) | (vb[e] << 16);
        tr[TR::off(cc * 8 + 2 * e + 1, col)] = (va[e] >> 16) | (vb[e] & 0xFFFF0000u);
      }
    }
  }
}

// Store a 32-row x (32*NB)-column accumulator block (rows 8*(r/4)+4g+r%4,
// column lane%32 of each 32-column block) as bf16, optionally times SiLU'(Z).
template <int NB>
HSTU_DEV void store_grad(const f32x16* acc, float scale, bf16* dst, int64_t ld, int o0,
                         int row0, int n, int col0, const bf16* z, int64_t ldz, int64_t zcol,
                         int ql, int g) {
#pragma unroll
  for (int d = 0; d < NB; ++d) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = row0 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (i < n) {
        float v = acc[d][r] * scale;
        if (z) v *= silu_grad_f((float)z[(int64_t)(o0 + i) * ldz + zcol + d * 32 + ql]);
        dst[(int64_t)(o0 + i) * ld + col0 + d * 32 + ql] = (bf16)v;
      }
    }
  }
}

template <int DQK, int DV>
__global__ __launch_bounds__(256, (DQK >= 128 || DV >= 128) ? 1 : 2) void k_attn_bwd_dkdv(AttnArgs a) {
  using QT = LdsTile<DQK>;
  using OT = LdsTile<DV>;
  using TT = LdsTile<KV_QT>;
  __shared__ __attribute__((aligned(16))) KvSmem<DQK, DV> sm;

  const int w = blockIdx.x;
  const int n_items = a.counters[0];
  if (w >= n_items * a.H) return;
  const int it = w / a.H, h = w - it * a.H;
  const int b = a.items[2 * it], kb = a.items[2 * it + 1];
  const int o0 = a.seq_offsets[b];
  const int n = a.seq_offsets[b + 1] - o0;
  const int c = a.num_cand ? a.num_cand[b] : 0;
  const int nh = n - c;
  const bool wide = a.seq_flags[b] & 1;
  const int nP = a.nP, nT = a.nT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, g = lane >> 5;

  {
    const float* rp = a.rab_pos + h * a.rab_stride;
    const float* rt = a.rab_time + h * a.rab_stride;
    for (int i = tid; i < nP; i += 256) {
      sm.tpos[i] = rp[i];
      sm.gpos[i] = 0.0f;
    }
    if (tid < 32) {
      sm.ttime[tid] = rt[tbucket_from_clz(tid, nT)];
      sm.gtime[tid] = 0.0f;
    }
  }

  const int k0 = kb * ATTN_BWD_BN;
  const int k1 = min(k0 + ATTN_BWD_BN, n);
  const int kw0 = k0 + wave * 32;
  const int kw1 = min(kw0 + 32, n);
  const int jk = kw0 + ql;  // this lane's key
  const bool kvalid = jk < n;
  const int pJ = min(jk, nh);
  int32_t tj = 0;
  int64_t tj64 = 0;
  if (kvalid) {
    if (wide) tj64 = a.ts[o0 + jk];
    else tj = a.rel_t[o0 + jk];
  }

  const bf16* qb = reinterpret_cast<const bf16*>(a.q);
  const bf16* kbp = reinterpret_cast<const bf16*>(a.k);
  const bf16* vbp = reinterpret_cast<const bf16*>(a.v);
  const bf16* dob = reinterpret_cast<const bf16*>(a.dout);

  bf16x8 kr[DQK / 16], vr[DV / 16];
#pragma unroll
  for (int ch = 0; ch < DQK / 16; ++ch)
    kr[ch] = kvalid ? *reinterpret_cast<const bf16x8*>(kbp + (int64_t)(o0 + jk) * a.ld_qk +
                                                       h * DQK + ch * 16 + 8 * g)
                    : bf16x8{};
#pragma unroll
  for (int ch = 0; ch < DV / 16; ++ch)
    vr[ch] = kvalid ? *reinterpret_cast<const bf16x8*>(vbp + (int64_t)(o0 + jk) * a.ld_v +
                                                       h * DV + ch * 16 + 8 * g)
                    : bf16x8{};

  f32x16 dk[DQK / 32], dv[DV / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) dk[d] = f32x16{};
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) dv[d] = f32x16{};

  const int qend = (k0 >= nh) ? k1 : n;  // candidate keys are seen by themselves only
  for (int i0 = k0; i0 < qend; i0 += KV_QT) {
    const int i1 = min(i0 + KV_QT, qend);
    __syncthreads();
    stage_both<DQK, KV_QT>(qb, a.ld_qk, o0, i0, i1, h * DQK, sm.q, sm.qt, tid);
    stage_both<DV, KV_QT>(dob, a.ld_dout, o0, i0, i1, h * DV, sm.o, sm.ot, tid);
    if (tid < KV_QT) sm.t1[tid] = (i0 + tid < n && !wide) ? a.rel_t[o0 + i0 + tid] + 1 : 0;
    __syncthreads();

    if (kw0 >= kw1) continue;
    // some allowed pair for this wave's keys?
    const bool hist_keys = kw0 < nh;
    bool active;
    if (hist_keys) active = (i1 - 1 >= kw0);
    else active = (i0 < kw1 && i1 > kw0);
    if (!active) continue;
    const bool need_mask = (i0 < kw1 - 1) || (kw1 > nh && i1 > nh);
    const bool far = !need_mask && !wide && (min(i0, nh) - min(kw1 - 1, nh) >= nP - 1);

    float dpos_far = 0.0f;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
      int cmin = 32, cmax = -1;
      float dsv[16];
      int clv[16];
      f32x16 sacc = f32x16{}, dacc = f32x16{};
#pragma unroll
      for (int ch = 0; ch < DQK / 16; ++ch) {
        const bf16x8 qa =
            *reinterpret_cast<const bf16x8*>(&sm.q[QT::off(qh * 32 + ql, ch * 8 + 4 * g)]);
        sacc = mfma32(qa, kr[ch], sacc);
      }
#pragma unroll
      for (int ch = 0; ch < DV / 16; ++ch) {
        const bf16x8 oa =
            *reinterpret_cast<const bf16x8*>(&sm.o[OT::off(qh * 32 + ql, ch * 8 + 4 * g)]);
        dacc = mfma32(oa, vr[ch], dacc);
      }
      bf16x8 pp[2], dd[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = qh * 32 + 8 * (r >> 2) + 4 * g + (r & 3);  // row inside the tile
        const int i = i0 + qi;
        bool ok = true;
        int cl;
        float bias;
        if (wide) cl = tclz_wide(i < n ? a.ts[o0 + i] : tj64, tj64);
        else cl = tclz_narrow(sm.t1[qi], tj);
        if (far) {
          bias = sm.tpos[nP - 1] + sm.ttime[cl];
        } else {
          ok = (i < n) && ((i < nh) ? (jk <= i) : (jk < nh || jk == i));
          bias = sm.tpos[pbucket(min(i, nh), pJ, nP)] + sm.ttime[cl];
        }
        const float s = sacc[r] + bias;
        float sig;
        float p = silu_from_parts(s, sig);
        float ds = dacc[r] * fmaf(p, 1.0f - sig, sig);
        if (need_mask && !ok) {
          p = 0.0f;
          ds = 0.0f;
        }
        pp[r >> 3][r & 7] = (bf16)p;
        dd[r >> 3][r & 7] = (bf16)ds;
        if (far) {
          dpos_far += ds;
          cmin = min(cmin, cl);
          cmax = max(cmax, cl);
          dsv[r] = ds;
          clv[r] = cl;
        } else if (ok && i < n && kvalid) {
          atomicAdd(&sm.gpos[pbucket(min(i, nh), pJ, nP)], ds);
          atomicAdd(&sm.gtime[cl], ds);
        }
      }
      // dV += P^T dO ; dK += dS^T Q   (k = 32 query rows of this half)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int d = 0; d < DV / 32; ++d) {
          const bf16x8 ob = *reinterpret_cast<const bf16x8*>(
              &sm.ot[TT::off(d * 32 + ql, 8 * (qh * 2 + u) + 4 * g)]);
          dv[d] = mfma32(pp[u], ob, dv[d]);
        }
#pragma unroll
        for (int d = 0; d < DQK / 32; ++d) {
          const bf16x8 qbv = *reinterpret_cast<const bf16x8*>(
              &sm.qt[TT::off(d * 32 + ql, 8 * (qh * 2 + u) + 4 * g)]);
          dk[d] = mfma32(dd[u], qbv, dk[d]);
        }
      }
      if (far) {
        // time buckets of a far tile: one wave reduction per bucket in its range
        const int lo = wave_min_i(cmin), hi = wave_max_i(cmax);
        for (int cv = lo; cv <= hi; ++cv) {
          float part = 0.0f;
#pragma unroll
          for (int r = 0; r < 16; ++r) part += (clv[r] == cv) ? dsv[r] : 0.0f;
          part = wave_sum(part);
          if (lane == 0) atomicAdd(&sm.gtime[cv], part);
        }
      }
    }
    if (far) {
      // the position bucket is constant on a far tile: one sum
      const float tot = wave_sum(dpos_far);
      if (lane == 0) atomicAdd(&sm.gpos[nP - 1], tot);
    }
  }

  const float invN = 1.0f / (float)(a.norm_mode == 0 ? a.norm_len : n);
  if (kw0 < kw1) {
    // dK/dV rows are keys: 8*(r/4)+4g+r%4 inside the wave's 32 keys, columns = channels
    f32x16 tk[DQK / 32], tv[DV / 32];
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d) tk[d] = dk[d];
#pragma unroll
    for (int d = 0; d < DV / 32; ++d) tv[d] = dv[d];
    store_grad<DQK / 32>(tk, invN, reinterpret_cast<bf16*>(a.dk), a.ld_qk, o0, kw0, n, h * DQK,
                         reinterpret_cast<const bf16*>(a.zpre), a.ld_z, a.zk_col + h * DQK, ql,
                         g);
    store_grad<DV / 32>(tv, invN, reinterpret_cast<bf16*>(a.dv), a.ld_v, o0, kw0, n, h * DV,
                        reinterpret_cast<const bf16*>(a.zpre), a.ld_z, a.zv_col + h * DV, ql, g);
  }
  __syncthreads();
  float* gp = a.drab_pos + h * a.rab_stride;
  float* gt = a.drab_time + h * a.rab_stride;
  for (int i = tid; i < nP; i += 256)
    if (sm.gpos[i] != 0.0f) atomicAdd(&gp[i], sm.gpos[i] * invN);
  if (tid < 32 && sm.gtime[tid] != 0.0f) atomicAdd(&gt[tbucket_from_clz(tid, nT)], sm.gtime[tid] * invN);
}

// ---------------------------------------------------------------------------
template <int DQK, int DV>
struct DqSmem {
  using KT = LdsTile<DQK>;
  using VR = LdsTile<DV>;
  using TT = LdsTile<DQ_BN>;
  uint32_t k[KT::S_DW * DQ_BN];    // K tile row-major (A operand of S^T = K Q^T)
  uint32_t kt[TT::S_DW * DQK];     // K tile transposed (B operand of dQ += dS K)
  uint32_t v[VR::S_DW * DQ_BN];    // V tile row-major (A operand of dA^T = V dO^T)
  int32_t t[DQ_BN];
  float tpos[1024];
  float ttime[32];
};

template <int DQK, int DV>
__global__ __launch_bounds__(256, (DQK >= 128 || DV >= 128) ? 1 : 2) void k_attn_bwd_dq(AttnArgs a) {
  using KT = LdsTile<DQK>;
  using VR = LdsTile<DV>;
  using TT = LdsTile<DQ_BN>;
  __shared__ __attribute__((aligned(16))) DqSmem<DQK, DV> sm;

  const int w = blockIdx.x;
  const int n_items = a.counters[0];
  if (w >= n_items * a.H) return;
  const int it = w / a.H, h = w - it * a.H;
  const int b = a.items[2 * it], m = a.items[2 * it + 1];
  const int o0 = a.seq_offsets[b];
  const int n = a.seq_offsets[b + 1] - o0;
  const int c = a.num_cand ? a.num_cand[b] : 0;
  const int nh = n - c;
  const bool wide = a.seq_flags[b] & 1;
  const int nP = a.nP, nT = a.nT;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ql = lane & 31, g = lane >> 5;
  {
    const float* rp = a.rab_pos + h * a.rab_stride;
    const float* rt = a.rab_time + h * a.rab_stride;
    for (int i = tid; i < nP; i += 256) sm.tpos[i] = rp[i];
    if (tid < 32) sm.ttime[tid] = rt[tbucket_from_clz(tid, nT)];
  }
  const int rb0 = m * ATTN_BWD_BM;
  const int rb1 = min(rb0 + ATTN_BWD_BM, n);
  const int r0 = rb0 + wave * 32;
  const int rw1 = min(r0 + 32, n);
  const int iq = r0 + ql;
  const bool qvalid = iq < n;
  const int pI = min(iq, nh);
  int32_t ti1 = 0;
  int64_t ti64 = 0;
  if (qvalid) {
    if (wide) ti64 = a.ts[o0 + iq];
    else ti1 = a.rel_t[o0 + iq] + 1;
  }
  const bf16* qb = reinterpret_cast<const bf16*>(a.q);
  const bf16* kbp = reinterpret_cast<const bf16*>(a.k);
  const bf16* vbp = reinterpret_cast<const bf16*>(a.v);
  const bf16* dob = reinterpret_cast<const bf16*>(a.dout);
  bf16x8 qr[DQK / 16], orr[DV / 16];
#pragma unroll
  for (int ch = 0; ch < DQK / 16; ++ch)
    qr[ch] = qvalid ? *reinterpret_cast<const bf16x8*>(qb + (int64_t)(o0 + iq) * a.ld_qk +
                                                       h * DQK + ch * 16 + 8 * g)
                    : bf16x8{};
#pragma unroll
  for (int ch = 0; ch < DV / 16; ++ch)
    orr[ch] = qvalid ? *reinterpret_cast<const bf16x8*>(dob + (int64_t)(o0 + iq) * a.ld_dout +
                                                        h * DV + ch * 16 + 8 * g)
                     : bf16x8{};
  f32x16 dq[DQK / 32];
#pragma unroll
  for (int d = 0; d < DQK / 32; ++d) dq[d] = f32x16{};

  const int ktiles = (rb1 + DQ_BN - 1) / DQ_BN;
  for (int kt = 0; kt < ktiles; ++kt) {
    const int j0 = kt * DQ_BN;
    const int j1 = min(j0 + DQ_BN, n);
    if (j0 >= nh && (j1 <= rb0 || j0 >= rb1)) continue;
    __syncthreads();
    stage_both<DQK, DQ_BN>(kbp, a.ld_qk, o0, j0, j1, h * DQK, sm.k, sm.kt, tid);
    {
      constexpr int CPR = DV / 8;
#pragma unroll
      for (int s = 0; s < (DQ_BN * CPR + 255) / 256; ++s) {
        const int idx = tid + 256 * s;
        if (idx < DQ_BN * CPR) {
          const int row = idx / CPR, ch = idx % CPR;
          const int j = j0 + row;
          u32x4 val = {0, 0, 0, 0};
          if (j < j1) val = ld16(vbp + (int64_t)(o0 + j) * a.ld_v + h * DV + ch * 8);
          *reinterpret_cast<u32x4*>(&sm.v[VR::off(row, ch * 4)]) = val;
        }
      }
    }
    if (tid < DQ_BN) sm.t[tid] = (j0 + tid < n && !wide) ? a.rel_t[o0 + j0 + tid] : 0;
    __syncthreads();

    if (r0 >= rw1) continue;
    const bool hist_rows = r0 < nh;
    const bool cand_rows = rw1 > nh;
    const bool active = (hist_rows && j0 <= min(rw1, nh) - 1) ||
                        (cand_rows && (j0 < nh || (j0 < rw1 && j1 > max(r0, nh))));
    if (!active) continue;
    const bool need_mask = (hist_rows && j1 - 1 > r0) || (j1 > nh);
    const bool far = !need_mask && !wide && (min(r0, nh) - min(j1 - 1, nh) >= nP - 1);

    bf16x8 dsk[4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      f32x16 sacc = f32x16{}, dacc = f32x16{};
#pragma unroll
      for (int ch = 0; ch < DQK / 16; ++ch) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(&sm.k[KT::off(hf * 32 + ql, ch * 8 + 4 * g)]);
        sacc = mfma32(ka, qr[ch], sacc);
      }
#pragma unroll
      for (int ch = 0; ch < DV / 16; ++ch) {
        const bf16x8 va =
            *reinterpret_cast<const bf16x8*>(&sm.v[VR::off(hf * 32 + ql, ch * 8 + 4 * g)]);
        dacc = mfma32(va, orr[ch], dacc);
      }
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const int kk0 = hf * 32 + 8 * aa + 4 * g;
        const i32x4 tj = *reinterpret_cast<const i32x4*>(&sm.t[kk0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = j0 + kk0 + r;
          int cl;
          if (wide) cl = tclz_wide(ti64, j < n ? a.ts[o0 + j] : ti64);
          else cl = tclz_narrow(ti1, tj[r]);
          bool ok = true;
          float bias;
          if (far) {
            bias = sm.tpos[nP - 1] + sm.ttime[cl];
          } else {
            ok = (iq < nh) ? (j <= iq) : (j < nh || j == iq);
            bias = sm.tpos[pbucket(pI, min(j, nh), nP)] + sm.ttime[cl];
          }
          const float s = sacc[4 * aa + r] + bias;
          float sig;
          const float p = silu_from_parts(s, sig);
          float ds = dacc[4 * aa + r] * fmaf(p, 1.0f - sig, sig);
          if (need_mask && !ok) ds = 0.0f;
          dsk[hf * 2 + (aa >> 1)][(aa & 1) * 4 + r] = (bf16)ds;
        }
      }
    }
#pragma unroll
    for (int d = 0; d < DQK / 32; ++d) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 kb =
            *reinterpret_cast<const bf16x8*>(&sm.kt[TT::off(d * 32 + ql, 8 * u + 4 * g)]);
        dq[d] = mfma32(dsk[u], kb, dq[d]);
      }
    }
  }
  if (r0 >= rw1) return;
  const float invN = 1.0f / (float)(a.norm_mode == 0 ? a.norm_len : n);
  store_grad<DQK / 32>(dq, invN, reinterpret_cast<bf16*>(a.dq), a.ld_qk, o0, r0, n, h * DQK,
                       reinterpret_cast<const bf16*>(a.zpre), a.ld_z, a.zq_col + h * DQK, ql, g);
}

template <int DQK, int DV>
hipError_t launch_kv_t(const AttnArgs& a, int64_t mi, hipStream_t st) {
  const int64_t grid = mi * a.H;
  if (grid <= 0) return hipSuccess;
  k_attn_bwd_dkdv<DQK, DV><<<(unsigned)grid, 256, 0, st>>>(a);
  return hipGetLastError();
}
template <int DQK, int DV>
hipError_t launch_dq_t(const AttnArgs& a, int64_t mi, hipStream_t st) {
  const int64_t grid = mi * a.H;
  if (grid <= 0) return hipSuccess;
  k_attn_bwd_dq<DQK, DV><<<(unsigned)grid, 256, 0, st>>>(a);
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
  HSTU_DISPATCH_D(launch_dq_t, d_qk, d_v, a, mi, st)
}

}  // namespace hstu
