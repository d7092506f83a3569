// Host-side declarations shared by the C-ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/hstu.h"

namespace hstu {

// Bump allocator over the caller's workspace.  With base == nullptr it only
// measures, so the *_workspace_size functions and the entry points share one
// carving routine.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  template <class T>
  T* take(size_t n) {
    off = (off + 255) & ~size_t(255);
    T* p = base ? reinterpret_cast<T*>(base + off) : nullptr;
    off += n * sizeof(T);
    return p;
  }
};

// Jagged work list of (sequence, row block) items.
struct Sched {
  int32_t* items = nullptr;     // [2*cap]
  int32_t* counters = nullptr;  // [0] items, [1] max blocks per sequence
  int32_t* hist = nullptr;      // [cap+2] sequences per block count
  int32_t* cnt = nullptr;       // [cap+2] sequences with more than m blocks
  int32_t* levelstart = nullptr;// [cap+2]
  int32_t* tie = nullptr;       // [cap+2]
  int64_t cap = 0;
  int block_rows = 0;
};

inline int64_t sched_capacity(int64_t T, int64_t B, int block_rows) {
  return (T + B * (int64_t)(block_rows - 1)) / block_rows + 1;
}
Sched carve_sched(Carver& c, int64_t T, int64_t B, int block_rows);
hipError_t launch_sched(const Sched& s, int B, const int32_t* seq_offsets, int reverse,
                        hipStream_t st);

// Per-token relative timestamps and per-sequence flags.
struct TimeMeta {
  int32_t* rel_t = nullptr;      // [T] t - min_t of the sequence (valid when not wide)
  int32_t* seq_flags = nullptr;  // [B] bit0: span >= 2^31 ("wide"), bit1: non-decreasing
};
TimeMeta carve_time(Carver& c, int64_t T, int64_t B);
// Also clears z0[0..nz) and z1[0..nz) (the backward's rab-gradient sums) when given.
hipError_t launch_time_prepass(const TimeMeta& tm, int B, const int32_t* seq_offsets,
                               const int64_t* ts, hipStream_t st, float* z0 = nullptr,
                               float* z1 = nullptr, int64_t nz = 0);

// One schedule to build: its arrays, block rows and order.
struct SchedJob {
  int32_t* items = nullptr;
  int32_t* counters = nullptr;
  int32_t* hist = nullptr;
  int32_t* cnt = nullptr;
  int32_t* levelstart = nullptr;
  int32_t* tie = nullptr;
  int cap = 0, bm = 1, reverse = 0;
};

// A call's plan in one launch: the time pre-pass over npre sequences (mode
// 0: one timestamp array; mode 1: a user's history offs/ts and candidates
// coffs/cts) and up to two work lists over sched_offs.
struct PlanArgs {
  int npre = 0;
  int mode = 0;
  const int32_t* offs = nullptr;
  const int64_t* ts = nullptr;
  int32_t* rel_t = nullptr;
  int32_t* flags = nullptr;
  const int32_t* coffs = nullptr;
  const int64_t* cts = nullptr;
  int32_t* rel_c = nullptr;
  float* z0 = nullptr;
  float* z1 = nullptr;
  int64_t nz = 0;
  int B = 0;
  const int32_t* sched_offs = nullptr;
  int njobs = 0;
  int lds_sched = 0;
  SchedJob job[2];
  // kept dS of the backward: per-sequence first block (H * nrb (nrb + 1) / 2
  // blocks of 128 x 128 per sequence, nrb = ceil(n / 128)) and the overflow
  // flag against the capacity (one more workgroup when ds_base is given)
  int32_t* ds_base = nullptr;
  int32_t* ds_flag = nullptr;
  int64_t ds_cap = 0;
  int H = 0;
};
PlanArgs plan_prepass(const TimeMeta& tm, int B, const int32_t* seq_offsets,
                      const int64_t* ts, float* z0 = nullptr, float* z1 = nullptr,
                      int64_t nz = 0);
void plan_add_job(PlanArgs& p, const Sched& s, int reverse, const int32_t* sched_offs);
hipError_t launch_plan(PlanArgs p, hipStream_t st);

struct AttnArgs {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  int64_t ld_qk = 0, ld_v = 0;
  void* out = nullptr;
  int64_t ld_out = 0;
  bool out_f32 = false;   // bf16 kernels: store O in fp32 (the layer keeps O in fp32 for the LayerNorm)
  const int32_t* seq_offsets = nullptr;
  const int32_t* num_cand = nullptr;
  const int64_t* ts = nullptr;
  const int32_t* rel_t = nullptr;
  const int32_t* seq_flags = nullptr;
  const int32_t* items = nullptr;
  const int32_t* counters = nullptr;
  const float* rab_pos = nullptr;
  const float* rab_time = nullptr;
  int64_t rab_stride = 0;
  int B = 0;  // sequences: a work item naming another sequence is skipped
  int H = 0, nP = 0, nT = 0, norm_mode = 0, norm_len = 1;
  // semi-local windows (win_local 0: full causal)
  int win_local = 0, win_global = 0;
  // forward key splits: workgroup w = (item, head) * splits + part; the parts
  // of one block write fp32 partial sums to part[(item, head)][part][BM][d_v],
  // part 0 writes their number to part_cnt[(item, head)], and a combine
  // kernel adds them into out
  int splits = 1;
  float* part = nullptr;
  int32_t* part_cnt = nullptr;
  // forward: 64-row work items whose key tiles two waves share (1), or
  // 128-row items (0); the plan's block rows must match
  int key_halves = 0;
  // forward with the score product in MXFP8: E4M3 codes of q and k (rows of
  // ld_mx bytes, head h at byte h*d_qk) and head-major scale words
  // (q_mxs[h*T_rows + row], byte b = E8M0 scale of channels 32b..32b+31);
  // q_mx == nullptr: bf16 q and k
  const uint8_t* q_mx = nullptr;
  const uint8_t* k_mx = nullptr;
  int64_t ld_mx = 0;
  const uint32_t* q_mxs = nullptr;
  const uint32_t* k_mxs = nullptr;
  int64_t T_rows = 0;
  // backward with dS kept: 128 x 128 bf16 blocks (key-major) of the causal
  // part, per sequence and head; ds_base[b] = first block of sequence b;
  // *ds_flag != 0: the blocks did not fit, dQ is recomputed instead
  uint16_t* ds = nullptr;   // bf16 bits
  const int32_t* ds_base = nullptr;
  const int32_t* ds_flag = nullptr;
  // backward
  const void* dout = nullptr;
  int64_t ld_dout = 0;
  void* dq = nullptr;
  void* dk = nullptr;
  void* dv = nullptr;
  float* drab_pos = nullptr;
  float* drab_time = nullptr;
  // Optional pre-activation Z: gradients are multiplied by SiLU'(Z) before
  // they are stored (the layer backward's dZ = dZh * SiLU'(Z)).
  const void* zpre = nullptr;
  int64_t ld_z = 0;
  int64_t zq_col = 0, zk_col = 0, zv_col = 0;
};

// Row-block sizes of the kernels (rows of Q per forward work item, keys per
// backward key-block work item).
constexpr int ATTN_FWD_BM_F32 = 64;
constexpr int ATTN_BWD_BN = 128;   // keys per dK/dV work item
constexpr int ATTN_BWD_BM = 128;   // queries per dQ work item

// Query rows per forward work item for a head size (bf16 kernels use 32 or 64
// rows per wave; fp32 uses 64 rows per workgroup).
int attn_fwd_block_rows(int dtype, int d_qk, int d_v, bool key_halves = false);
// forward attention workgroups one compute unit holds (bf16)
int attn_fwd_occupancy(int d_qk, int d_v);
hipError_t launch_attn_fwd(const AttnArgs& a, int dtype, int d_qk, int d_v,
                           int64_t max_items, hipStream_t st);
hipError_t launch_attn_bwd_dkdv(const AttnArgs& a, int d_qk, int d_v, int64_t max_items,
                                hipStream_t st);
hipError_t launch_attn_bwd_dq(const AttnArgs& a, int d_qk, int d_v, int64_t max_items,
                              hipStream_t st);
hipError_t launch_bias_buckets(const AttnArgs& a, const int32_t* pair_seq,
                               const int32_t* pair_i, const int32_t* pair_j, int64_t n,
                               int32_t* bp, int32_t* bt, hipStream_t st);
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t st);
hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t st);

// GEMM: C[M,N] = sum_k A(m,k) B(k,n), epilogue below.
//  a_kcont: A(m,k) at A[m*lda + k] (else A[k*lda + m]);
//  b_kcont: B(k,n) at B[n*ldb + k] (else B[k*ldb + n]).
enum GemmEpi {
  EPI_STORE = 0,    // C = acc
  EPI_SILU = 1,     // Z = acc + bias; C2 = Z (optional); C = SiLU(Z)  (bf16)
  EPI_RESID = 2,    // C = acc + bias + R
  EPI_PARTIAL = 3,  // fp32 partial sums of a split-K slice -> ws[z][M][N]
};
struct GemmArgs {
  int64_t M = 0, N = 0, K = 0;
  const void* A = nullptr;
  int64_t lda = 0;
  bool a_kcont = true;
  const void* B = nullptr;
  int64_t ldb = 0;
  bool b_kcont = true;
  void* C = nullptr;
  int64_t ldc = 0;
  bool c_f32 = false;     // output fp32 (else dtype of inputs)
  void* C2 = nullptr;     // EPI_SILU: pre-activation output (may be null)
  const float* bias = nullptr;  // [N] or null
  const void* R = nullptr;      // EPI_RESID residual, same dtype as C, row stride ldr
  int64_t ldr = 0;
  int epi = EPI_STORE;
  int split_k = 1;
  float* partial = nullptr;     // EPI_PARTIAL workspace [split_k][M][N]
  // MXFP8 operands (both k-contiguous): A, B hold E4M3 codes, lda/ldb/K count
  // pairs of codes (2 bytes), scale_a [M][K/32] and scale_b [N][K/32] are the
  // E8M0 block scales (K here in codes)
  bool mx = false;
  const uint8_t* scale_a = nullptr;
  const uint8_t* scale_b = nullptr;
  // scales laid out k-step-major instead: [K/128 codes][rows][4], the four
  // blocks of one k-step of a row in one word and consecutive rows' words
  // adjacent (long contractions, e.g. over the tokens)
  bool scale_kstep_major = false;
  // MX kernels, EPI_RESID with bf16 C: also write C as MXFP8 along N
  // (codes [M][N], scales [M][N/32]; N a multiple of 32)
  uint8_t* c_codes = nullptr;
  uint8_t* c_scales = nullptr;
  // MX kernels, EPI_SILU: also write the (bf16-rounded) SiLU outputs of
  // columns [qk_col0, qk_col0 + qk_cols) as MXFP8 along each head's qk_d
  // channels, the attention's q|k operands: codes [M][qk_cols], head-major
  // scale words (qk_scales bytes, word h*M + m, byte = 32-channel block of the
  // head; bytes past qk_d/32 are not written)
  uint8_t* qk_codes = nullptr;
  uint8_t* qk_scales = nullptr;
  int64_t qk_col0 = 0, qk_cols = 0;
  int qk_d = 0;
  // also store those columns of C as their MXFP8 values (training: the
  // backward then differentiates the scores the forward computed)
  bool qk_dequant = false;
};
hipError_t launch_gemm(const GemmArgs& g, int dtype, hipStream_t st);
// Split-K reduction: out[m*ldo + n] = sum_z partial[z][m][n]  (fp32)
hipError_t launch_splitk_reduce(const float* partial, int split, int64_t M, int64_t N,
                                float* out, int64_t ldo, hipStream_t st);
// Column sums over rows of a [rows, cols] matrix (dtype) -> fp32 out[cols].
hipError_t launch_colsum(const void* x, int64_t rows, int64_t cols, int64_t ld, int dtype,
                         float* out, float* ws, hipStream_t st);

// LayerNorm + gating.
struct LnArgs {
  bool o_f32 = false;        // O (and its saved copy) is fp32 regardless of the layer dtype
  int64_t T = 0;
  int W = 0;                 // H*d_v
  const void* O = nullptr;   // [T, W] stride ld_o
  int64_t ld_o = 0;
  const void* U = nullptr;   // [T, W] stride ld_u
  int64_t ld_u = 0;
  const float* gamma = nullptr;
  const float* beta = nullptr;
  float eps = 1e-6f;
  void* G = nullptr;         // [T, W] stride ld_g
  int64_t ld_g = 0;
  float* mu = nullptr;       // [T] or null
  float* rstd = nullptr;     // [T] or null
  // forward, bf16: write G as MXFP8 (codes [T][W], scales [T][W/32]) instead
  // of G itself (the rounding of the bf16 value G would have been stored as)
  uint8_t* g_codes = nullptr;
  uint8_t* g_scales = nullptr;
  // backward
  const void* dG = nullptr;  int64_t ld_dg = 0;
  void* dU = nullptr;        int64_t ld_du = 0;   // written as dU * SiLU'(Zu) if zu != null
  const void* zu = nullptr;  int64_t ld_zu = 0;
  void* dO = nullptr;        int64_t ld_do = 0;
  float* dgamma_part = nullptr;  // [blocks][W] partial column sums (or null)
  float* dbeta_part = nullptr;
  int64_t n_part_blocks = 0;
};
hipError_t launch_ln_gate_fwd(const LnArgs& a, int dtype, hipStream_t st);
hipError_t launch_ln_gate_bwd(const LnArgs& a, int dtype, hipStream_t st);
int64_t ln_bwd_part_blocks(int64_t T);

hipError_t launch_validate(int B, const int32_t* seq_offsets, const int32_t* num_cand,
                           int64_t T, int32_t* flag, hipStream_t st);

// Ranking against a cached history: candidate rows (q, k, v: their own
// projections) against the user's cached history keys and values.
struct CachedArgs {
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  int64_t ld_qk = 0, ld_v = 0;
  const int32_t* cand_offsets = nullptr;
  const int64_t* cand_ts = nullptr;
  const void* kh = nullptr;
  const void* vh = nullptr;
  int64_t ld_kh = 0, ld_vh = 0;
  const int32_t* hist_offsets = nullptr;
  const int64_t* hist_ts = nullptr;
  const int32_t* rel_h = nullptr;   // history times relative to the user's minimum
  const int32_t* rel_c = nullptr;   // candidate times relative to the same minimum
  const int32_t* flags = nullptr;   // per user: bit0 wide, bit1 history sorted
  const int32_t* items = nullptr;   // work list over (user, candidate block)
  const int32_t* counters = nullptr;
  void* out = nullptr;
  int64_t ld_out = 0;
  bool out_f32 = false;
  float* part = nullptr;            // [splits, Tc, H*d_v] partial sums when splits > 1
  int64_t Tc = 0;
  int splits = 1;
  const float* rab_pos = nullptr;
  const float* rab_time = nullptr;
  int64_t rab_stride = 0;
  int B = 0;  // users: a work item naming another user is skipped
  int H = 0, nP = 0, nT = 0, norm_len = 1, win_local = 0, win_global = 0;
};
int attn_cached_block_rows(int dtype, int d_qk, int d_v);
// workgroups of the cached-attention kernel that share one compute unit
int attn_cached_occupancy(int dtype, int d_qk, int d_v);
hipError_t launch_attn_cached(const CachedArgs& a, int dtype, int d_qk, int d_v,
                              int64_t max_items, hipStream_t st);

// MXFP8 quantization (blocks of 32 along the contraction, k-contiguous output)
hipError_t launch_mx_quant_rows(const void* x, int64_t ld, int64_t rows, int64_t K,
                                uint8_t* codes, uint8_t* scales, hipStream_t st);
// MXFP8 of x^T: x [T][C] (row stride ld) -> codes [C][Tp] and k-step-major
// scales [Tp/128][C][4], blocks of 32 rows, rows T..Tp-1 as zeros
// (C % 64 == 0, Tp % 128 == 0)
hipError_t launch_mx_quant_rows_t(const void* x, int64_t ld, int64_t T, int64_t C, int64_t Tp,
                                  uint8_t* codes, uint8_t* scales, hipStream_t st);
// both at once from one read of x: the transposed codes and scales above and
// the row-wise ones of launch_mx_quant_rows (rcodes [T][C], rscales [T][C/32])
hipError_t launch_mx_quant_both(const void* x, int64_t ld, int64_t T, int64_t C, int64_t Tp,
                                uint8_t* codes, uint8_t* scales, uint8_t* rcodes,
                                uint8_t* rscales, hipStream_t st);
// MXFP8 of attention operands along each head's channels: codes [T][ld_codes]
// (head h at byte h*d), head-major scale words scales[h*T + t] (byte b: block b)
hipError_t launch_mx_quant_heads(const void* x, int64_t ld, int64_t T, int H, int d,
                                 uint8_t* codes, int64_t ld_codes, uint32_t* scales,
                                 hipStream_t st);
hipError_t launch_mx_quant_cols(const void* w, int64_t K, int64_t N, uint8_t* codes,
                                uint8_t* scales, hipStream_t st);

// Attention truncation: segment offsets, row gather, gradient scatter.
hipError_t launch_trunc_offsets(int B, const int32_t* seq_offsets, const int32_t* num_cand,
                                int keep, int32_t* seg_offsets, hipStream_t st);
hipError_t launch_trunc_gather(int B, int64_t T, int64_t T_seg, int64_t row_bytes,
                               const int32_t* seq_offsets, const int32_t* seg_offsets,
                               const void* x, void* x_seg, const int64_t* ts, int64_t* ts_seg,
                               hipStream_t st);
hipError_t launch_trunc_scatter(int B, int64_t T, int64_t T_seg, int64_t row_bytes,
                                const int32_t* seq_offsets, const int32_t* seg_offsets,
                                const void* dx_seg, void* dx, hipStream_t st);

}  // namespace hstu
