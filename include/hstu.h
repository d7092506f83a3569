/*
 * hstu.h -- C ABI of the HSTU layer library for MI355X (gfx950).
 *
 * The HSTU layer works on jagged, timestamp-ordered user-history sequences:
 * a projection into U, V, Q, K; pointwise attention SiLU(Q K^T + relative
 * bias) with no softmax; a gated output LayerNorm(A V) * U; and an output
 * projection.  Pages this interface follows:
 *   [GR]     NVIDIA generative-recommenders summary (quantumzeitgeist.com),
 *            section "HSTU Architecture: Efficient Attention for User History":
 *            SiLU weighting instead of softmax, relative attention bias,
 *            elementwise gating before the output projection.
 *   [DLRMv4] "DLRMv4 Brings Sequence-Based Recommendation Training to MLPerf"
 *            (xfinit.ro): "Model Architecture" (projection, pointwise
 *            attention with positional and temporal-distance bias, gated
 *            transformation; candidate appended to the history and processed
 *            in one causal pass), "HSTU Hyperparameters" (jagged attention,
 *            bf16), "Computation Cost Analysis" Table 7 (U|V|Q|K width
 *            h*(2*d_qk + 2*d_v); only the lower triangle is evaluated).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Packed jagged layout: sequence b owns rows seq_offsets[b] .. seq_offsets[b+1]-1
 *   of every [T, ...] tensor.  seq_offsets is int32 [B+1] in device memory,
 *   non-decreasing, seq_offsets[0] = 0, seq_offsets[B] = T.  Empty sequences
 *   are allowed.
 * - timestamps: int64 [T] seconds, device memory.  Within a sequence they are
 *   expected to be non-decreasing; a negative distance is treated as 0.
 * - num_candidates: int32 [B] device memory or NULL (no candidates).  The last
 *   num_candidates[b] rows of sequence b are candidates; 0 <= c_b <= n_b.
 *   A history row attends to itself and earlier history rows; a candidate row
 *   attends to the whole history and to itself only.
 * - Relative bias for a query row i and key row j of one sequence (n_h =
 *   history length, p(i) = min(i, n_h)):
 *     bp = min(p(i) - p(j), n_pos_buckets - 1)
 *     bt = min(floor(log2(dt + 1)), n_time_buckets - 1),
 *          dt = min(max(t_i - t_j, 0), 2^31 - 1)
 *     bias = rab_pos[h][bp] + rab_time[h][bt]
 *   rab_pos/rab_time are fp32, head h's table starts at h * rab_head_stride
 *   floats (rab_head_stride = 0: one table shared by all heads).
 * - Attention weight a_ij = SiLU(q_i . k_j + bias) / N for allowed pairs, with
 *   N = norm_len (norm_mode 0) or the sequence's own length n_b (norm_mode 1).
 * - Heads are contiguous inside a row: element (row r, head h, channel c) of
 *   Q is at q[r * ld_qk + h * d_qk + c].
 * - dtype HSTU_BF16: activations and weights bf16, fp32 accumulation, bf16
 *   results rounded to nearest even.  HSTU_F32: fp32 throughout.
 * - Every pointer is device memory owned by the caller.  The library never
 *   allocates or frees device memory; scratch space is the caller's workspace
 *   (16-byte aligned, size from the *_workspace_size functions).  All calls
 *   are asynchronous on `stream` (a hipStream_t passed as void*, NULL = the
 *   default stream) and never synchronise.  Outputs are fully overwritten.
 * - Errors: only host-visible arguments are validated (NULL required
 *   pointers, unsupported sizes, misaligned pointers or strides, workspace
 *   too small).  On such an error nothing is launched and nothing is written.
 *   Launch failures return HSTU_ERR_HIP.  Device-side contracts (offsets,
 *   candidate counts, timestamps) are the caller's; hstu_validate_inputs
 *   checks them synchronously.
 * - Supported sizes: d_qk, d_v in {32, 64, 128}; 1 <= H <= 64; T < 2^31;
 *   1 <= n_pos_buckets, n_time_buckets <= 1024; bf16 row strides multiples of
 *   8 elements (fp32: 4) and 16-byte aligned base pointers.
 */
#ifndef HSTU_H_
#define HSTU_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HSTU_OK = 0,
  HSTU_ERR_INVALID_ARG = -1,
  HSTU_ERR_UNSUPPORTED = -2,
  HSTU_ERR_WORKSPACE = -3,
  HSTU_ERR_HIP = -4,
  HSTU_ERR_VALIDATION = -5
} hstu_status;

typedef enum { HSTU_F32 = 0, HSTU_BF16 = 1 } hstu_dtype;

/* Shape and options of one pointwise-attention call. */
typedef struct {
  int32_t B;               /* sequences */
  int64_t T;               /* packed rows = seq_offsets[B] */
  int32_t H;               /* heads */
  int32_t d_qk;            /* query/key channels per head */
  int32_t d_v;             /* value channels per head */
  int32_t n_pos_buckets;   /* entries per position table (e.g. 128) */
  int32_t n_time_buckets;  /* entries per time table (e.g. 128) */
  int32_t norm_mode;       /* 0: divide by norm_len; 1: divide by n_b */
  int32_t norm_len;        /* N for norm_mode 0 (> 0) */
  int32_t dtype;           /* hstu_dtype */
  int64_t rab_head_stride; /* floats between heads' tables; 0 = shared */
  /* Semi-local attention ("Bending the Scaling Law Curve in Large-Scale
   * Recommendation Systems", Semi-Local Attention: a local and a global window
   * instead of the full causal mask).  win_local > 0 additionally requires of
   * every allowed pair p(i) - p(j) < win_local (the win_local most recent
   * positions, the token itself included) or j < win_global (the first
   * win_global tokens of the sequence).  win_local = 0: full causal /
   * target-aware attention (win_global is then ignored).  Both >= 0. */
  int32_t win_local;
  int32_t win_global;
  /* Longest sequence of the batch (rows), or 0 if not given.  With d_qk =
   * d_v = 128, bf16 and no windows, a positive max_len lets the backward keep
   * dS, the gradient of the scores, in its workspace (bf16, 128 x 128 blocks
   * of the causal part, about 2 T max_len H bytes) and form dQ from it instead
   * of recomputing S and dA.  If the batch's blocks do not fit (a sequence
   * longer than max_len), the backward recomputes; results agree either way.
   * A shape whose bound (max_len taken at most T) exceeds 2^27 blocks of
   * 32 KiB never keeps dS and asks for no such workspace. */
  int32_t max_len;
  /* Forward only (hstu_attn_fwd, hstu_attn_fwd_noalloc, hstu_layer_fwd,
   * hstu_layer_fwd_mx): 1 asks to skip the plan (time pre-pass and work
   * list) because the workspace already holds the plan an earlier forward
   * call on the same batch wrote, e.g. the previous layer of a stack run
   * with one workspace.  The plan depends on B, T, H, dtype, d_qk, d_v,
   * key_splits and win_local (which fix its work-item rows) and the
   * contents of seq_offsets and timestamps.  The library records, per device,
   * every plan a forward call writes (its bytes in the workspace, those
   * sizes and the offsets and timestamps pointers) and forgets the plans in
   * any workspace bytes a later call may write; a reuse_plan call whose
   * workspace bytes, sizes or pointers match no recorded plan returns
   * HSTU_ERR_INVALID_ARG before anything is launched.  The caller still
   * asserts that the contents of seq_offsets and timestamps are unchanged,
   * that nothing outside the library wrote the plan's bytes, and that the
   * planning call is ordered before this one (e.g. the same stream).
   * 0 (default): plan.  Other values: HSTU_ERR_INVALID_ARG.  Ignored by
   * backward and cached-history calls, which always plan. */
  int32_t reuse_plan;
  /* Forward (bf16, no semi-local windows): split the keys of long query
   * blocks so that partial sums add (no softmax, so the parts add exactly up
   * to rounding order), meant for batches too small to fill the GPU.
   * 0: library default: when even an upper bound on the work items of
   * 128 query rows (T/128 + B per head) fits the GPU's workgroup slots at
   * once, 64-row items whose 64-key tiles two waves share, each adding half
   * of every tile's keys (their partial sums meet in LDS); otherwise no
   * split.  1: never split.  2..8: split every query block into up to this
   * many runs of at least 4 key tiles of 64 over separate workgroups; the
   * parts write fp32 partial sums to the workspace and a second kernel adds
   * them (measured slower on every workload tried).  Other values:
   * HSTU_ERR_INVALID_ARG.  The workspace size depends on it. */
  int32_t key_splits;
} hstu_attn_desc;

/* One layer: attention options plus model width and layer flags. */
typedef struct {
  hstu_attn_desc attn;
  int32_t D;          /* model width (rows of W1, columns of W2) */
  int32_t proj_silu;  /* 1: U|V|Q|K = SiLU(X W1 + b1); 0: no nonlinearity */
  int32_t residual;   /* 1: Y = X + G W2 + b2; 0: Y = G W2 + b2 */
  float ln_eps;       /* LayerNorm epsilon (e.g. 1e-6) */
} hstu_layer_desc;

/* Weights of one layer (device memory, caller-owned). */
typedef struct {
  const void* W1;        /* [D, F1] row-major, dtype; F1 = H*(2*d_v + 2*d_qk), columns U|V|Q|K */
  const void* W2;        /* [H*d_v, D] row-major, dtype */
  const float* b1;       /* [F1] fp32 or NULL */
  const float* b2;       /* [D] fp32 or NULL */
  const float* ln_gamma; /* [H*d_v] fp32 or NULL (1) */
  const float* ln_beta;  /* [H*d_v] fp32 or NULL (0) */
  const float* rab_pos;  /* position tables, see conventions */
  const float* rab_time; /* time tables, see conventions */
} hstu_layer_weights;

/* Forward intermediates a training step keeps for the backward pass. */
typedef struct {
  void* Z;     /* [T, F1] dtype: X W1 + b1 before the SiLU */
  void* Zh;    /* [T, F1] dtype: U|V|Q|K after the SiLU */
  float* O;    /* [T, H*d_v] fp32: attention output (kept in fp32 for the LayerNorm, whose
                  mean subtraction would otherwise cancel the bits bf16 keeps) */
  void* G;     /* [T, H*d_v] dtype: LayerNorm(O) * U */
  float* mu;   /* [T] LayerNorm mean */
  float* rstd; /* [T] LayerNorm 1/sqrt(var + eps) */
} hstu_layer_saved;

/* Gradients of one layer's parameters (fp32, overwritten). */
typedef struct {
  float* dW1;       /* [D, F1] */
  float* dW2;       /* [H*d_v, D] */
  float* db1;       /* [F1], required iff b1 != NULL */
  float* db2;       /* [D], required iff b2 != NULL */
  float* dgamma;    /* [H*d_v], required iff ln_gamma != NULL */
  float* dbeta;     /* [H*d_v], required iff ln_beta != NULL */
  float* drab_pos;  /* same shape as rab_pos (H tables, or 1 if shared) */
  float* drab_time; /* same shape as rab_time */
} hstu_layer_grads;

const char* hstu_status_string(hstu_status s);
/* Text of the HIP error behind the calling thread's last HSTU_ERR_HIP. */
const char* hstu_last_hip_error(void);
/* The library step ("api.cpp:<line>: <call>") whose HIP call or launch
 * returned that error; "" if none did. */
const char* hstu_last_error_site(void);
/*
 * Check mode, for debugging: with it on, every entry point waits for the
 * device after each kernel launch and stream operation it makes and reads
 * the launch error, so that an asynchronous kernel failure is reported as
 * HSTU_ERR_HIP by the call that caused it, with hstu_last_error_site naming
 * the launching step.  Calls become synchronous and slow; not for use under
 * HIP graph capture (the wait is not allowed there).  Process-wide; off by
 * default, on at load when the environment variable HSTU_CHECK is set to a
 * value other than "0".  hstu_set_check_mode: on = 0 or 1, other values
 * HSTU_ERR_INVALID_ARG.  hstu_check_mode: the current setting.
 */
hstu_status hstu_set_check_mode(int32_t on);
int32_t hstu_check_mode(void);
/* Library version string. */
const char* hstu_version(void);

/* ---- pointwise attention ------------------------------------------------ */

size_t hstu_attn_fwd_workspace_size(const hstu_attn_desc* desc);
size_t hstu_attn_bwd_workspace_size(const hstu_attn_desc* desc);

/*
 * O = pointwise attention of Q, K, V ([GR] and [DLRMv4] "Model Architecture";
 * lower triangle only per [DLRMv4] Table 7's note).
 * q, k: rows of stride ld_qk; v: rows of stride ld_v (elements), so the three
 * may be column views into one U|V|Q|K projection buffer.
 * out: [T, H*d_v] rows of stride ld_out.
 */
hstu_status hstu_attn_fwd(const hstu_attn_desc* desc,
                          const void* q, const void* k, int64_t ld_qk,
                          const void* v, int64_t ld_v,
                          const int32_t* seq_offsets, const int64_t* timestamps,
                          const float* rab_pos, const float* rab_time,
                          const int32_t* num_candidates,
                          void* out, int64_t ld_out,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * hstu_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and kernels, with no workspace argument.  The plan
 * (time pre-pass and work list) goes to a library-owned scratch array of
 * HSTU_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends; the call
 * itself never allocates or frees.  Problems whose forward workspace
 * (hstu_attn_fwd_workspace_size) exceeds that size are rejected with
 * HSTU_ERR_WORKSPACE before anything is launched (8 MiB holds the plan of
 * about 1.9 million rows).  A key split (key_splits 2..8) counts its
 * partial sums against the same limit.  Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (other streams, other threads)
 * race and must be ordered by the caller.  reuse_plan = 1 refers to the
 * plan the previous no-allocation call on the device left there.  Other
 * arguments and errors as hstu_attn_fwd.
 */
#define HSTU_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
hstu_status hstu_attn_fwd_noalloc(const hstu_attn_desc* desc,
                                  const void* q, const void* k, int64_t ld_qk,
                                  const void* v, int64_t ld_v,
                                  const int32_t* seq_offsets, const int64_t* timestamps,
                                  const float* rab_pos, const float* rab_time,
                                  const int32_t* num_candidates,
                                  void* out, int64_t ld_out, void* stream);

/*
 * Gradients of hstu_attn_fwd for the output gradient d_out ([T, H*d_v],
 * stride ld_out).  dq, dk (stride ld_qk) and dv (stride ld_v) are written in
 * dtype; d_rab_pos / d_rab_time (fp32, same shape as the tables) are
 * overwritten.  bf16 only.
 */
hstu_status hstu_attn_bwd(const hstu_attn_desc* desc,
                          const void* q, const void* k, int64_t ld_qk,
                          const void* v, int64_t ld_v,
                          const int32_t* seq_offsets, const int64_t* timestamps,
                          const float* rab_pos, const float* rab_time,
                          const int32_t* num_candidates,
                          const void* d_out, int64_t ld_out,
                          void* dq, void* dk, void* dv,
                          float* d_rab_pos, float* d_rab_time,
                          void* workspace, size_t workspace_bytes, void* stream);

/* ---- whole layer ------------------------------------------------------------ */

/* training != 0: the forward keeps its intermediates in a caller `saved`. */
size_t hstu_layer_fwd_workspace_size(const hstu_layer_desc* desc, int training);
size_t hstu_layer_bwd_workspace_size(const hstu_layer_desc* desc);

/*
 * Y = HSTU layer(X) ([DLRMv4] "Model Architecture"; [GR]).  x, y: [T, D]
 * dtype, contiguous rows; y may not alias x.  saved == NULL: inference
 * (intermediates live in the workspace); saved with every buffer set: a
 * training forward, all written (workspace sized with training = 1);
 * saved with only Zh set: inference that keeps U|V|Q|K in Zh, e.g. the
 * keys and values of a history for hstu_layer_fwd_cached (workspace sized
 * with training = 0).
 */
hstu_status hstu_layer_fwd(const hstu_layer_desc* desc, const void* x,
                           const hstu_layer_weights* w,
                           const int32_t* seq_offsets, const int64_t* timestamps,
                           const int32_t* num_candidates,
                           void* y, const hstu_layer_saved* saved,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward of hstu_layer_fwd given dy ([T, D] dtype): dx ([T, D] dtype) and
 * every parameter gradient in g (fp32, overwritten).  `saved` must hold the
 * intermediates of the matching training forward.  bf16 only.
 * Part of the work (the attention work lists, dW1, dW2) runs on a side
 * stream that the library keeps per host thread and device (created on first
 * use, default priority, held until the process ends); it starts after all
 * work queued on `stream` before the call, and `stream` waits for all of it
 * before the call returns, so every output is ordered on `stream` as if the
 * whole call had run there.  A capture of `stream` into a graph includes the
 * side work.  If the side stream cannot be created, everything runs on
 * `stream`.
 */
hstu_status hstu_layer_bwd(const hstu_layer_desc* desc, const void* x,
                           const hstu_layer_weights* w,
                           const int32_t* seq_offsets, const int64_t* timestamps,
                           const int32_t* num_candidates,
                           const hstu_layer_saved* saved, const void* dy,
                           void* dx, const hstu_layer_grads* g,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---- MXFP8 matmuls ------------------------------------------------------- */
/*
 * "Bending the Scaling Law Curve in Large-Scale Recommendation Systems",
 * Mixed precision: most operations stay in BF16, the matrix products run in
 * FP8.  The scaling recipe is not given there; these entry points use the
 * OCP Microscaling (MX) format: every 32 consecutive values along the
 * contraction index share one E8M0 scale byte e (2^(e-127)), chosen as
 * 2^(floor(log2 amax) - 8), and are stored as E4M3 codes rounded to nearest
 * (ties to even) with saturation at 448; an all-zero block has e = 0.  The
 * matrix cores apply the block scales (scaled 32x32x64 FP8 MFMA), so a
 * product needs no separate rescaling.  Codes and scales are k-contiguous:
 * codes [rows][K] bytes, scales [rows][K/32] bytes.
 */

/* One layer's MXFP8 weights (device memory, caller-owned). */
typedef struct {
  const void* W1;         /* [F1][D] E4M3 codes: W1 transposed, blocks along D */
  const void* W1_scales;  /* [F1][D/32] E8M0 */
  const void* W2;         /* [D][H*d_v] codes: W2 transposed, blocks along H*d_v */
  const void* W2_scales;  /* [D][H*d_v/32] */
} hstu_mx_weights;

/* MXFP8 of rows x K bf16 values (row stride ld, blocks along each row;
 * K a multiple of 32, x and codes 16-byte aligned, ld a multiple of 8). */
hstu_status hstu_mx_quantize(int64_t rows, int64_t K, const void* x, int64_t ld, void* codes,
                             void* scales, void* stream);
/* MXFP8 of a [K][N] bf16 weight along K, written transposed: codes [N][K],
 * scales [N][K/32] (K a multiple of 32). */
hstu_status hstu_mx_quantize_weight(int64_t K, int64_t N, const void* w, void* codes,
                                    void* scales, void* stream);
/* C [M][ldc] fp32 = A B^T for MXFP8 A [M][K] and B [N][K] (K a multiple of
 * 128; codes and C 16-byte aligned, scale arrays 4-byte aligned). */
hstu_status hstu_mx_gemm(int64_t M, int64_t N, int64_t K, const void* a, const void* a_scales,
                         const void* b, const void* b_scales, float* c, int64_t ldc,
                         void* stream);
/*
 * The attention's score product in MXFP8 ("Bending the Scaling Law Curve in
 * Large-Scale Recommendation Systems", Mixed precision: the matrix products
 * in FP8; the scores q_i . k_j are one of the attention's two products).
 * q and k are rounded along their contraction, the d_qk channels of each
 * head, in blocks of 32 (the MX encoding above); the scaled FP8 matrix
 * cores multiply the codes, and the bias, SiLU, mask, normalisation and
 * the product with v run as in hstu_attn_fwd (P and v in bf16).
 *
 * hstu_mx_quantize_heads: MXFP8 of x [T][H*d] bf16 (row stride ld
 * elements, a multiple of 8; x 16-byte aligned) along each head's d
 * channels (d a multiple of 32, at most 128; H at most 64; q and k side by
 * side, as in the layer's U|V|Q|K rows, can be quantized in one call as 2H
 * heads): codes [T][ld_codes] bytes
 * (head h at byte h*d; ld_codes >= H*d, a multiple of 16; codes 16-byte
 * aligned) and one 32-bit scale word per head and row, head-major:
 * scales[h*T + t], byte b = the E8M0 scale of channels 32b..32b+31 of head
 * h (bytes past d/32 zero; scales 4-byte aligned).  A key tile's scale
 * words are then one contiguous run.  Invalid sizes or alignment:
 * HSTU_ERR_INVALID_ARG.
 */
hstu_status hstu_mx_quantize_heads(int64_t T, int32_t H, int32_t d, const void* x, int64_t ld,
                                   void* codes, int64_t ld_codes, uint32_t* scales,
                                   void* stream);

/* q and k of hstu_attn_fwd_mx as written by hstu_mx_quantize_heads (device
 * memory, caller-owned; both with the same ld_codes). */
typedef struct {
  const void* q_codes;
  const void* k_codes;
  int64_t ld_codes;
  const uint32_t* q_scales; /* [H][T] words */
  const uint32_t* k_scales; /* [H][T] words */
} hstu_attn_mx_qk;

/* hstu_attn_fwd with the score product in MXFP8: `qk` replaces q, k and
 * ld_qk; v, out (bf16), the tables, offsets, timestamps, candidates,
 * workspace (hstu_attn_fwd_workspace_size of the same descriptor) and
 * reuse_plan as for hstu_attn_fwd.  Supported: bf16, d_qk = d_v in
 * {64, 128}, no semi-local windows, key_splits 0 or 1; other descriptors
 * return HSTU_ERR_UNSUPPORTED before anything is launched. */
hstu_status hstu_attn_fwd_mx(const hstu_attn_desc* desc, const hstu_attn_mx_qk* qk,
                             const void* v, int64_t ld_v,
                             const int32_t* seq_offsets, const int64_t* timestamps,
                             const float* rab_pos, const float* rab_time,
                             const int32_t* num_candidates,
                             void* out, int64_t ld_out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forward of one layer with MXFP8 projection and output products
 * ("Bending the Scaling Law Curve in Large-Scale Recommendation Systems",
 * Mixed precision: the matrix products in FP8; X and the gated LayerNorm G
 * are quantized on the fly; attention, LayerNorm and gating in bf16 / fp32
 * as in hstu_layer_fwd).  `w` supplies the biases, LayerNorm affine and bias
 * tables (its W1, W2 are not read); `wm` the MXFP8 weights; `io` (may be
 * NULL) the optional MXFP8 inputs and outputs below; `saved` (may be NULL;
 * all six buffers, as for hstu_layer_fwd) keeps the intermediates for
 * hstu_layer_bwd_mx.  bf16 only, D and H*d_v multiples of 128.
 */
typedef struct {
  /* x already in MXFP8 ([T][D] codes, [T][D/32] scales): skips its
   * quantization, e.g. the y_codes/y_scales of the previous layer */
  const void* x_codes;
  const void* x_scales;
  /* also write y in MXFP8 (same layout), for the next layer */
  void* y_codes;
  void* y_scales;
  /* receive the quantized gated output G ([T][H*d_v], [T][H*d_v/32]) */
  void* g_codes;
  void* g_scales;
  /* 1: the attention's score product in MXFP8 too (as hstu_attn_fwd_mx: q
   * and k quantized along each head's channels inside the call, into the
   * workspace); d_qk = d_v in {64, 128}, no semi-local windows, key_splits
   * 0 or 1, else HSTU_ERR_UNSUPPORTED.  With `saved` (training; the layer
   * must have its projection SiLU) the stored U|V|Q|K holds q and k as their
   * MXFP8 values, so that hstu_layer_bwd_mx differentiates the scores the
   * forward computed (the quantizer taken as the identity).
   * 0: bf16 attention. */
  int32_t mx_scores;
} hstu_mx_io;  /* each pair NULL or both given; codes 16-, scales 4-byte aligned */
size_t hstu_layer_fwd_mx_workspace_size(const hstu_layer_desc* desc);
hstu_status hstu_layer_fwd_mx(const hstu_layer_desc* desc, const void* x,
                              const hstu_layer_weights* w, const hstu_mx_weights* wm,
                              const int32_t* seq_offsets, const int64_t* timestamps,
                              const int32_t* num_candidates, void* y, const hstu_mx_io* io,
                              const hstu_layer_saved* saved,
                              void* workspace, size_t workspace_bytes, void* stream);
/*
 * Training backward of hstu_layer_fwd_mx (same arguments as hstu_layer_bwd;
 * `saved` from hstu_layer_fwd_mx).  All four products of the backward are
 * MXFP8 products ("Bending the Scaling Law Curve in Large-Scale
 * Recommendation Systems", Mixed precision: the matrix products in FP8),
 * each operand quantized along its own contraction as in the forward:
 * dG = dY W2^T (dY and W2 in blocks of 32 along d_model), dX = dZ W1^T (+ dY)
 * (dZ and W1 in blocks along F1), and the weight gradients dW2 = G^T dY and
 * dW1 = X^T dZ (G, dY, X and dZ in blocks of 32 tokens, the last block of
 * a token count that is not a multiple of 32 padded with zeros); the
 * attention and LayerNorm backward stay bf16 / fp32; the forward's
 * quantizers count as the identity in the chain rule.  Every MXFP8 copy
 * (the weights' too) is made inside the call.  bf16 only; D, H*d_v and F1
 * multiples of 128, else HSTU_ERR_UNSUPPORTED.  The workspace holds the
 * copies: (1 + 1/32)(3 D + 2 F1 + H*d_v) bytes per token (tokens rounded up
 * to 128 for the transposed ones) and the weights' beyond hstu_layer_bwd's.
 */
size_t hstu_layer_bwd_mx_workspace_size(const hstu_layer_desc* desc);
hstu_status hstu_layer_bwd_mx(const hstu_layer_desc* desc, const void* x,
                              const hstu_layer_weights* w,
                              const int32_t* seq_offsets, const int64_t* timestamps,
                              const int32_t* num_candidates,
                              const hstu_layer_saved* saved, const void* dy, void* dx,
                              const hstu_layer_grads* grads,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ---- ranking against a cached history --------------------------------- */
/*
 * "DLRMv4 Brings Sequence-Based Recommendation Training to MLPerf", "Model
 * Architecture": candidates are appended to the history and compared with
 * it in one pass.  A history row never attends to a candidate, so each
 * layer's history keys and values (and the history's layer outputs) do not
 * depend on the candidates: computed once (hstu_layer_fwd over the history
 * alone, keeping Zh), they let later candidate batches run through the
 * layers alone.  Candidate r of user b sits at position n_h (the user's
 * history length) and attends to every cached history key of the user
 * (under semi-local windows: n_h - j < win_local or j < win_global) and to
 * its own key; this equals the candidate rows of the target-aware pass over
 * [history; candidates] when N is the fixed norm_len (norm_mode 0 only).
 */

/* One layer's cached history keys and values (device memory, caller-owned). */
typedef struct {
  const void* k;               /* [T, ld_k] dtype: H*d_qk key columns, head-major */
  const void* v;               /* [T, ld_v] dtype: H*d_v value columns */
  int64_t ld_k;                /* row strides in elements (bf16: multiples of 8) */
  int64_t ld_v;
  const int32_t* offsets;      /* [B+1] device int32: user b's history rows */
  const int64_t* timestamps;   /* [T] device int64 seconds */
  int64_t T;                   /* history rows = offsets[B] */
} hstu_history_kv;

/*
 * O [T, ld_out] dtype (desc->T = candidate rows, desc->B = users) of the
 * candidates against the cached history `hist` of the same users.  q, k, v:
 * the candidates' own projections ([T, ld] views as in hstu_attn_fwd);
 * cand_offsets [B+1], cand_timestamps [T] device arrays.  fp32 outputs must
 * be 16-byte aligned with ld_out a multiple of 4.  Errors as hstu_attn_fwd;
 * HSTU_ERR_UNSUPPORTED for norm_mode 1.
 */
size_t hstu_attn_cached_workspace_size(const hstu_attn_desc* desc, int64_t T_hist);
hstu_status hstu_attn_cached_fwd(const hstu_attn_desc* desc, const void* q, const void* k,
                                 int64_t ld_qk, const void* v, int64_t ld_v,
                                 const int32_t* cand_offsets, const int64_t* cand_timestamps,
                                 const hstu_history_kv* hist, const float* rab_pos,
                                 const float* rab_time, void* out, int64_t ld_out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Y = HSTU layer over candidate rows x ([T, D], desc->T = candidate rows)
 * with the attention against this layer's cached history (the K and V
 * column blocks of the Zh that hstu_layer_fwd kept for the history).
 * Inference only.  Errors as hstu_layer_fwd; HSTU_ERR_UNSUPPORTED for
 * norm_mode 1.
 */
size_t hstu_layer_cached_workspace_size(const hstu_layer_desc* desc, int64_t T_hist);
hstu_status hstu_layer_fwd_cached(const hstu_layer_desc* desc, const void* x,
                                  const hstu_layer_weights* w, const int32_t* cand_offsets,
                                  const int64_t* cand_timestamps, const hstu_history_kv* hist,
                                  void* y, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* ---- attention truncation ---------------------------------------------- */
/*
 * "Bending the Scaling Law Curve in Large-Scale Recommendation Systems",
 * Attention Truncation: after N layers over whole sequences, M further
 * layers run only on a segment of each history made of its most recent
 * events.  The segment of sequence b is its last min(n_b - c_b, keep)
 * history rows followed by its c_b candidate rows: a contiguous tail of the
 * sequence, attended as a sequence of its own (same num_candidates, its own
 * timestamps; relative position buckets are unchanged because they depend
 * on position differences only).  Segment row r of sequence b comes from
 * full row seq_offsets[b+1] - seg_offsets[b+1] + r.
 */

/*
 * seg_offsets[0..B] (device int32, written on `stream`) of the segments.
 * seq_offsets: [B+1] device int32; num_candidates: [B] device int32 or NULL
 * (no candidates; values are clamped to [0, n_b]); keep >= 0.  The segment
 * total T_seg = seg_offsets[B] is needed on the host to size the truncated
 * batch: the caller reads it back or knows it from the lengths.
 * Errors: HSTU_ERR_INVALID_ARG for B < 0, keep < 0 or a NULL pointer.
 */
hstu_status hstu_truncate_offsets(int32_t B, const int32_t* seq_offsets,
                                  const int32_t* num_candidates, int32_t keep,
                                  int32_t* seg_offsets, void* stream);

/*
 * Gather of the truncated batch: x_seg[r] = x[src(r)] for r < T_seg and,
 * when both are given, ts_seg[r] = timestamps[src(r)] (for T_seg > 0,
 * neither or both must be given).  x: [T, D] dtype,
 * x_seg: [T_seg, D] dtype, rows contiguous, both 16-byte aligned, D times
 * the element size a multiple of 16 bytes; T = seq_offsets[B],
 * T_seg = seg_offsets[B] (from hstu_truncate_offsets with the same
 * seq_offsets).  Rows whose source would fall outside [0, T) are written as
 * zeros.  x_seg may not overlap x.  Errors: HSTU_ERR_INVALID_ARG (sizes,
 * NULL pointers, alignment), HSTU_ERR_UNSUPPORTED (dtype).
 */
hstu_status hstu_truncate_gather(int32_t B, int64_t T, int64_t T_seg, int32_t D, int32_t dtype,
                                 const void* x, const int32_t* seq_offsets,
                                 const int32_t* seg_offsets, const int64_t* timestamps,
                                 void* x_seg, int64_t* ts_seg, void* stream);

/*
 * Backward of the gather: dx[i] = dx_seg[r] for the segment row r taken from
 * full row i, and dx[i] = 0 for every row outside the segments (all T rows
 * are written).  Shapes and alignment as for hstu_truncate_gather; dx may
 * not overlap dx_seg.
 */
hstu_status hstu_truncate_scatter(int32_t B, int64_t T, int64_t T_seg, int32_t D, int32_t dtype,
                                  const void* dx_seg, const int32_t* seq_offsets,
                                  const int32_t* seg_offsets, void* dx, void* stream);

/* ---- inspection entry points (tests, debugging) ------------------------- */

/*
 * Relative-bias buckets computed by the same device code the attention
 * kernels use: for each listed pair (sequence pair_seq[p], local query row
 * pair_i[p], local key row pair_j[p]) writes bp[p], bt[p] (int32).  The pair
 * must lie inside its sequence.  All arrays are device memory.
 */
hstu_status hstu_bias_buckets(const hstu_attn_desc* desc,
                              const int32_t* seq_offsets, const int64_t* timestamps,
                              const int32_t* num_candidates,
                              const int32_t* pair_seq, const int32_t* pair_i,
                              const int32_t* pair_j, int64_t n_pairs,
                              int32_t* bp, int32_t* bt,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * The jagged work list the forward attention uses for row blocks of
 * `block_rows` rows: items[2*w] = sequence, items[2*w+1] = block index, for
 * w < *n_items, ordered by decreasing block cost; *n_items (device int32)
 * receives the count.  items must hold hstu_schedule_capacity(...) pairs.
 * reverse != 0 orders blocks by increasing index instead (key-block-major
 * backward, where earlier blocks are the heavier ones).
 */
int64_t hstu_schedule_capacity(int64_t T, int32_t B, int32_t block_rows);
hstu_status hstu_schedule(int32_t B, int64_t T, const int32_t* seq_offsets,
                          int32_t block_rows, int32_t reverse,
                          int32_t* items, int32_t* n_items,
                          void* workspace, size_t workspace_bytes, void* stream);
size_t hstu_schedule_workspace_size(int32_t B, int64_t T, int32_t block_rows);

/*
 * Synchronous check of the device-side contracts (seq_offsets[0] = 0,
 * offsets non-decreasing, seq_offsets[B] = T, 0 <= c_b <= n_b).  flag_ws is
 * one device int32 of scratch.  Returns HSTU_OK or HSTU_ERR_VALIDATION.
 */
hstu_status hstu_validate_inputs(int32_t B, int64_t T, const int32_t* seq_offsets,
                                 const int32_t* num_candidates, int32_t* flag_ws, void* stream);

/*
 * MFMA-rate microbenchmark (a measured denominator for utilisation figures,
 * beside the nominal peak): `workgroups` workgroups of four waves each run
 * `iters` x 4 independent bf16 32x32x16 MFMAs (32768 flops each), so one
 * launch performs workgroups * 4 * iters * 4 * 32768 flops; out (device,
 * 4 * workgroups floats) receives a checksum per wave.  Time it with events
 * on `stream`.  HSTU_ERR_INVALID_ARG for iters or workgroups < 1 or out NULL.
 */
hstu_status hstu_diag_mfma_loop(int32_t iters, int32_t workgroups, float* out, void* stream);

/* ---- diagnostic kernel timer ------------------------------------------- */

/*
 * Per-kernel timing for benchmarking: while enabled, every kernel launch site
 * of the entry points above is bracketed by a pair of HIP events recorded on
 * the call's stream (at most max_launches pairs; later launches go untimed).
 * hstu_timer_enable(0) disables timing and releases the events; it creates or
 * destroys HIP events only (no device memory).  hstu_timer_reset forgets the
 * recorded launches.  hstu_timer_query waits for the recorded events of one
 * tag (0 <= tag < hstu_timer_tag_count()) and returns their count and summed
 * duration.  Not thread-safe: one benchmarking thread at a time.
 */
hstu_status hstu_timer_enable(int32_t max_launches);
hstu_status hstu_timer_reset(void);
int32_t hstu_timer_tag_count(void);
const char* hstu_timer_tag_name(int32_t tag);
hstu_status hstu_timer_query(int32_t tag, int64_t* launches, double* total_ms);

#ifdef __cplusplus
}
#endif

#endif /* HSTU_H_ */
