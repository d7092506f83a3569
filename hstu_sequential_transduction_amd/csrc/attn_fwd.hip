// Fused HSTU pointwise attention, forward.
//
// O_i = (1/N) * sum_j allowed(i,j) * SiLU(q_i . k_j + rab_pos[bp] + rab_time[bt]) * v_j
// (SiLU weighting instead of softmax and a relative bias: NVIDIA
// generative-recommenders summary, "HSTU Architecture: Efficient Attention for
// User History"; positional/temporal-distance bias and the appended candidate:
// "DLRMv4 Brings Sequence-Based Recommendation Training to MLPerf", "Model
// Architecture"; lower triangle only: its Table 7 note).
//
// bf16 kernel (gfx950 MFMA): one workgroup = one (sequence, 128-row query
// block, head) work item, four waves of 32 query rows.  Q stays in registers
// as the B operand of S^T = K Q^T (32x32x16 MFMA), K tiles of 64 keys are
// staged row-major in LDS, V tiles transposed (channel-major, keys permuted
// so each lane group's eight keys are contiguous), so the S^T accumulator is
// consumed directly as the A operand of O += P V without any shuffle.  Per
// score element the VALU adds the bias (LDS table gathers indexed by the
// position distance and by clz of the time distance), evaluates
// SiLU(s) = s / (1 + 2^(-s log2 e)) with one v_exp and one v_rcp, applies the
// mask only on tiles that need it, and rounds to bf16.  Work is scaled by
// -log2(e) throughout (folded into the bias tables and one FMA) and the
// factor -ln(2)/N is applied once to the output accumulator.
#include "bias.h"
#include "common.h"
#include "internal.h"

namespace hstu {

namespace {

constexpr int FWD_BN = 64;  // keys per tile

template <int DQK, int DV>
struct FwdSmem {
  using KT = LdsTile<DQK>;
  using VT = LdsTile<FWD_BN>;
  uint32_t k[KT::S_DW * FWD_BN];
  uint32_t vt[VT::S_DW * DV];
  int32_t t[FWD_BN];
  float tfar[32];
  float ttime[32];
  float tpos[1024];
};

template <int DQK, int DV>
__global__ __launch_bounds__(256, 2) void k_attn_fwd_bf16(AttnArgs a) {
  using KT = LdsTile<DQK>;
  using VT = LdsTile<FWD_BN>;
  __shared__ __attribute__((aligned(16))) FwdSmem<DQK, DV> sm;

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

  // bias tables (pre-scaled by -log2 e)
  {
    const float* rp = a.rab_pos + h * a.rab_stride;
    const float* rt = a.rab_time + h * a.rab_stride;
    for (int i = tid; i < nP; i += 256) sm.tpos[i] = rp[i] * HSTU_NEG_LOG2E;
    if (tid < 32) {
      float tv = rt[tbucket_from_clz(tid, nT)];
      sm.ttime[tid] = tv * HSTU_NEG_LOG2E;
      sm.tfar[tid] = (rp[nP - 1] + tv) * HSTU_NEG_LOG2E;
    }
  }

  const int rb0 = m * 128;
  const int rb1 = min(rb0 + 128, n);
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

  const bf16* qbase = reinterpret_cast<const bf16*>(a.q);
  const bf16* kbase = reinterpret_cast<const bf16*>(a.k);
  const bf16* vbase = reinterpret_cast<const bf16*>(a.v);

  bf16x8 qr[DQK / 16];
#pragma unroll
  for (int ch = 0; ch < DQK / 16; ++ch) {
    if (qvalid)
      qr[ch] = *reinterpret_cast<const bf16x8*>(qbase + (int64_t)(o0 + iq) * a.ld_qk + h * DQK +
                                                ch * 16 + 8 * g);
    else
      qr[ch] = bf16x8{};
  }

  f32x16 oacc[DV / 32];
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) oacc[d] = f32x16{};

  const int ktiles = (rb1 + FWD_BN - 1) / FWD_BN;
  for (int kt = 0; kt < ktiles; ++kt) {
    const int j0 = kt * FWD_BN;
    const int j1 = min(j0 + FWD_BN, n);
    if (j0 >= nh && (j1 <= rb0 || j0 >= rb1)) continue;  // only other candidates' keys

    __syncthreads();
    // ---- stage K (row-major) ----
    {
      constexpr int CPR = DQK / 8;
#pragma unroll
      for (int s = 0; s < (FWD_BN * CPR + 255) / 256; ++s) {
        const int idx = tid + 256 * s;
        if (idx < FWD_BN * CPR) {
          const int row = idx / CPR, ch = idx % CPR;
          const int j = j0 + row;
          u32x4 val = {0, 0, 0, 0};
          if (j < n) val = ld16(kbase + (int64_t)(o0 + j) * a.ld_qk + h * DQK + ch * 8);
          *reinterpret_cast<u32x4*>(&sm.k[KT::off(row, ch * 4)]) = val;
        }
      }
    }
    // ---- stage V transposed: vt[channel][kperm(key)] ----
    {
      constexpr int NCH = DV / 8;          // 8-channel chunks
      constexpr int NITEM = (FWD_BN / 2) * NCH;
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
          const int j = j0 + 2 * kp;
          u32x4 va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
          if (j < n) va = ld16(vbase + (int64_t)(o0 + j) * a.ld_v + h * DV + cc * 8);
          if (j + 1 < n) vb = ld16(vbase + (int64_t)(o0 + j + 1) * a.ld_v + h * DV + cc * 8);
          const int col = kperm(2 * kp) >> 1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t lo = (va[e] & 0xFFFFu) | (vb[e] << 16);
            const uint32_t hi = (va[e] >> 16) | (vb[e] & 0xFFFF0000u);
            sm.vt[VT::off(cc * 8 + 2 * e, col)] = lo;
            sm.vt[VT::off(cc * 8 + 2 * e + 1, col)] = hi;
          }
        }
      }
    }
    if (tid < FWD_BN) sm.t[tid] = (j0 + tid < n && !wide) ? a.rel_t[o0 + j0 + tid] : 0;
    __syncthreads();

    // ---- per-wave work on this tile ----
    if (r0 >= rw1) continue;
    const bool hist_rows = r0 < nh;
    const bool cand_rows = rw1 > nh;
    const bool active = (hist_rows && j0 <= min(rw1, nh) - 1) ||
                        (cand_rows && (j0 < nh || (j0 < rw1 && j1 > max(r0, nh))));
    if (!active) continue;
    const bool need_mask = (hist_rows && j1 - 1 > r0) || (j1 > nh);
    const bool far = !need_mask && !wide && (min(r0, nh) - min(j1 - 1, nh) >= nP - 1);

    f32x16 sacc[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      sacc[hf] = f32x16{};
#pragma unroll
      for (int ch = 0; ch < DQK / 16; ++ch) {
        const bf16x8 ka =
            *reinterpret_cast<const bf16x8*>(&sm.k[KT::off(hf * 32 + ql, ch * 8 + 4 * g)]);
        sacc[hf] = mfma32(ka, qr[ch], sacc[hf]);
      }
    }

    bf16x8 pk[4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
      for (int aa = 0; aa < 4; ++aa) {
        const int kk0 = hf * 32 + 8 * aa + 4 * g;
        const i32x4 tj = *reinterpret_cast<const i32x4*>(&sm.t[kk0]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float s = sacc[hf][4 * aa + r];
          float sb;
          bool ok = true;
          if (far) {
            sb = fmaf(s, HSTU_NEG_LOG2E, sm.tfar[tclz_narrow(ti1, tj[r])]);
          } else {
            const int j = j0 + kk0 + r;
            ok = (iq < nh) ? (j <= iq) : (j < nh || j == iq);
            const int bpv = pbucket(pI, min(j, nh), nP);
            int cl;
            if (wide) cl = tclz_wide(ti64, j < n ? a.ts[o0 + j] : ti64);
            else cl = tclz_narrow(ti1, tj[r]);
            sb = fmaf(s, HSTU_NEG_LOG2E, sm.tpos[bpv] + sm.ttime[cl]);
          }
          float p = sb * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(sb));
          if (need_mask && !ok) p = 0.0f;
          pk[hf * 2 + (aa >> 1)][(aa & 1) * 4 + r] = (bf16)p;
        }
      }
    }

#pragma unroll
    for (int d = 0; d < DV / 32; ++d) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bf16x8 vb =
            *reinterpret_cast<const bf16x8*>(&sm.vt[VT::off(d * 32 + ql, 8 * u + 4 * g)]);
        oacc[d] = mfma32(pk[u], vb, oacc[d]);
      }
    }
  }

  // ---- write O * (-ln2 / N) ----
  if (r0 >= rw1) return;
  const float scale = -HSTU_LN2 / (float)(a.norm_mode == 0 ? a.norm_len : n);
#pragma unroll
  for (int d = 0; d < DV / 32; ++d) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = r0 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (i < n) {
        const int64_t off = (int64_t)(o0 + i) * a.ld_out + h * DV + d * 32 + ql;
        if (a.out_f32) reinterpret_cast<float*>(a.out)[off] = oacc[d][r] * scale;
        else reinterpret_cast<bf16*>(a.out)[off] = (bf16)(oacc[d][r] * scale);
      }
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
  const int o0 = a.seq_offsets[b];
  const int n = a.seq_offsets[b + 1] - o0;
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
      const bool ok = (j < n) && ((iq < nh) ? (j <= iq) : (j < nh || j == iq));
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
  if (dtype == HSTU_BF16)
    k_attn_fwd_bf16<DQK, DV><<<(unsigned)grid, 256, 0, st>>>(a);
  else
    k_attn_fwd_f32<DQK, DV><<<(unsigned)grid, 256, 0, st>>>(a);
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
