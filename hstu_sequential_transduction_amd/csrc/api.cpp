// C ABI of the HSTU layer library: argument checks, workspace carving and the
// launch sequence of each entry point.  Every step of the computation runs in
// the HIP kernels of this directory; this file only orders them on the
// caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <vector>

#include "internal.h"
#include "timer.h"

using namespace hstu;

namespace {

// HIP error behind the calling thread's last HSTU_ERR_HIP (hstu_last_hip_error)
// and the step that reported it (hstu_last_error_site)
thread_local hipError_t g_last_hip_error = hipSuccess;
thread_local const char* g_last_error_site = "";

// Check mode (hstu_set_check_mode, or HSTU_CHECK=1 in the environment when
// the library loads): after every launch or stream operation the library
// waits for the device and reads the launch error, so that a failing kernel
// is reported by the call and the step that launched it.
std::atomic<int> g_check_mode{0};
const int g_check_from_env = [] {
  const char* e = getenv("HSTU_CHECK");
  if (e && e[0] && strcmp(e, "0") != 0) g_check_mode.store(1);
  return 0;
}();

hipError_t check_step() {
  hipError_t e = hipDeviceSynchronize();
  const hipError_t l = hipGetLastError();
  return e != hipSuccess ? e : l;
}

#define HSTU_STR_(x) #x
#define HSTU_STR(x) HSTU_STR_(x)
#define HSTU_TRY(expr)                                                          \
  do {                                                                          \
    hipError_t e_ = (expr);                                                     \
    if (e_ == hipSuccess && g_check_mode.load(std::memory_order_relaxed))       \
      e_ = check_step();                                                        \
    if (e_ != hipSuccess) {                                                     \
      g_last_hip_error = e_;                                                    \
      g_last_error_site = "api.cpp:" HSTU_STR(__LINE__) ": " #expr;             \
      return HSTU_ERR_HIP;                                                      \
    }                                                                           \
  } while (0)

// Every entry point that launches work starts here: it clears an error that
// an earlier HIP call of another library may have left behind, so that a
// launch error the entry point reports is its own.
hipStream_t entry_stream(void* stream) {
  (void)hipGetLastError();
  return (hipStream_t)stream;
}

// Work inside one call that does not depend on the steps before it (the
// attention plan reads only offsets and timestamps; a weight gradient needs
// only its two operands) runs on a side stream: one per host thread and
// device, default priority, created on first use and kept until the process
// ends.  It is ordered after everything queued on the caller's stream before
// the call and joined back by an event before the call returns, so the caller
// sees the order of its own stream.  If the stream or its events cannot be
// created, that work stays on the caller's stream.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t ev[5] = {};
  int state = 0;  // 0 untried, 1 ready, -1 unavailable
};
SideStream* side_stream() {
  thread_local SideStream sides[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) {
    (void)hipGetLastError();
    return nullptr;
  }
  SideStream& sd = sides[dev];
  if (sd.state == 0) {
    bool ok = hipStreamCreateWithFlags(&sd.s, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; ok && i < 5; ++i)
      ok = hipEventCreateWithFlags(&sd.ev[i], hipEventDisableTiming) == hipSuccess;
    sd.state = ok ? 1 : -1;
    (void)hipGetLastError();
  }
  return sd.state == 1 ? &sd : nullptr;
}
// work queued on `to` from now on runs after all work queued on `from` so far
hipError_t order_after(hipStream_t to, hipStream_t from, hipEvent_t ev) {
  hipError_t e = hipEventRecord(ev, from);
  if (e == hipSuccess) e = hipStreamWaitEvent(to, ev, 0);
  return e;
}

// Once a call has forked work onto the side stream, the caller's stream waits
// for that work on every way out of the call, error returns included, so no
// side work runs unordered after the call has returned.
struct SideJoin {
  SideStream* sd = nullptr;
  hipStream_t st = nullptr;
  bool forked = false;
  hipError_t join() {
    if (!forked) return hipSuccess;
    forked = false;
    return order_after(st, sd->s, sd->ev[3]);
  }
  ~SideJoin() {
    if (forked && join() != hipSuccess) (void)hipGetLastError();
  }
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
size_t esize(int dtype) { return dtype == HSTU_BF16 ? 2 : 4; }

hstu_status check_attn_desc(const hstu_attn_desc* d) {
  if (!d) return HSTU_ERR_INVALID_ARG;
  if (d->B < 0 || d->T < 0 || d->T >= (int64_t(1) << 31)) return HSTU_ERR_INVALID_ARG;
  if (d->H < 1 || d->H > 64) return HSTU_ERR_UNSUPPORTED;
  auto okd = [](int x) { return x == 32 || x == 64 || x == 128; };
  if (!okd(d->d_qk) || !okd(d->d_v)) return HSTU_ERR_UNSUPPORTED;
  if (d->n_pos_buckets < 1 || d->n_pos_buckets > 1024) return HSTU_ERR_UNSUPPORTED;
  if (d->n_time_buckets < 1 || d->n_time_buckets > 1024) return HSTU_ERR_UNSUPPORTED;
  if (d->norm_mode != 0 && d->norm_mode != 1) return HSTU_ERR_INVALID_ARG;
  if (d->norm_mode == 0 && d->norm_len <= 0) return HSTU_ERR_INVALID_ARG;
  if (d->win_local < 0 || d->win_global < 0 || d->max_len < 0) return HSTU_ERR_INVALID_ARG;
  if (d->reuse_plan != 0 && d->reuse_plan != 1) return HSTU_ERR_INVALID_ARG;
  if (d->key_splits < 0 || d->key_splits > 8) return HSTU_ERR_INVALID_ARG;
  if (d->dtype != HSTU_F32 && d->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
  if (d->rab_head_stride < 0) return HSTU_ERR_INVALID_ARG;
  if (d->rab_head_stride != 0 &&
      d->rab_head_stride < std::max(d->n_pos_buckets, d->n_time_buckets))
    return HSTU_ERR_INVALID_ARG;
  return HSTU_OK;
}

// bf16 operands are read 16 bytes at a time.
bool stride_ok(int dtype, const void* p, int64_t ld, int64_t min_ld) {
  if (ld < min_ld) return false;
  if (dtype == HSTU_BF16) return aligned16(p) && (ld % 8) == 0;
  return (reinterpret_cast<uintptr_t>(p) & 3) == 0;
}


// Parts the forward splits long query blocks' keys into (1: none): bf16
// without windows, when the descriptor asks for it.  The default is not to
// split: on the 1-layer (32 sequences of U[64,1024]) and 8-layer Zipf
// workloads, whose work lists hold fewer items than the GPU holds
// workgroups or about twice as many, every split from 2 to 8 parts was
// slower (extra workgroups' start-up, the partial sums' round trip and the
// combine launch cost more than the shorter longest run saves).
int fwd_splits(const hstu_attn_desc* d) {
  if (d->dtype != HSTU_BF16 || d->win_local > 0) return 1;
  return d->key_splits >= 2 ? d->key_splits : 1;
}

// Whether the forward runs 64-row work items with the key tiles shared by two
// waves (bf16, no windows, key_splits 0): when even an upper bound on the
// 128-row items (T/128 + B per head) leaves compute units without work, the
// run is bound by the longest items' chains of key tiles, which this halves
// (1-layer workload: 32 sequences of U[64,1024], 4 heads of 64: at most 660
// items against 768 workgroup slots).  Decided from sizes alone, so a
// planning call and a reuse_plan call agree.
bool fwd_key_halves(const hstu_attn_desc* d) {
  if (d->dtype != HSTU_BF16 || d->win_local > 0 || d->key_splits != 0) return false;
  const int64_t items = (d->T + 127) / 128 + d->B;
  const int64_t slots = 256 * (int64_t)attn_fwd_occupancy(d->d_qk, d->d_v);
  return items * d->H <= slots;
}

struct FwdWs {
  TimeMeta tm;
  Sched sc;
  bool kh = false;
  int splits = 1;
  float* part = nullptr;       // [cap * H][splits][block rows][d_v]
  int32_t* part_cnt = nullptr; // [cap * H] parts per work item (written by the kernel)
};
FwdWs carve_fwd(Carver& c, const hstu_attn_desc* d) {
  FwdWs w;
  w.tm = carve_time(c, d->T, d->B);
  w.kh = fwd_key_halves(d);
  const int bm = attn_fwd_block_rows(d->dtype, d->d_qk, d->d_v, w.kh);
  w.sc = carve_sched(c, d->T, d->B, bm);
  w.splits = fwd_splits(d);
  if (w.splits > 1) {
    w.part = c.take<float>(w.sc.cap * d->H * w.splits * bm * d->d_v);
    w.part_cnt = c.take<int32_t>(w.sc.cap * d->H);
  }
  return w;
}

// ---- plans left in workspaces (reuse_plan) ---------------------------------
// A forward call that plans records what its plan depends on: the device, the
// plan's bytes in the workspace, B, T, the row-block size (dtype, head
// sizes and the key-half choice) and the seq_offsets / timestamps buffers.  A later forward that sets
// reuse_plan must name the same workspace bytes and the same inputs, else it
// is rejected before anything is launched.  Every other call that is handed
// a workspace forgets the plans recorded in the bytes it may write.  The
// registry cannot see writes made outside the library (e.g. the caller
// reusing the memory for another tensor), nor a change of the offsets' or
// timestamps' contents; kernels still skip work items that name rows outside
// the batch, so a stale plan gives wrong rows, never an out-of-bounds access.
struct PlanTag {
  int dev = -1;
  uintptr_t p0 = 0, p1 = 0;  // plan bytes [p0, p1)
  int32_t B = 0, H = 0, d_qk = 0, d_v = 0, dtype = 0, bm = 0;
  int64_t T = 0;
  const void* offs = nullptr;
  const void* ts = nullptr;
};
std::mutex g_plan_mu;
std::vector<PlanTag> g_plan_tags;
constexpr size_t kMaxPlanTags = 256;

int current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return -1;
  }
  return dev;
}

size_t fwd_plan_bytes(const hstu_attn_desc* d) {
  Carver c(nullptr);
  carve_fwd(c, d);
  return c.off;
}

// forget the plans recorded in [p, p + bytes) of the current device
void plans_forget(const void* p, size_t bytes) {
  if (!p || bytes == 0) return;
  const int dev = current_device();
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), a1 = a0 + bytes;
  std::lock_guard<std::mutex> lk(g_plan_mu);
  g_plan_tags.erase(std::remove_if(g_plan_tags.begin(), g_plan_tags.end(),
                                   [&](const PlanTag& t) {
                                     return t.dev == dev && t.p0 < a1 && a0 < t.p1;
                                   }),
                    g_plan_tags.end());
}

PlanTag plan_tag(const hstu_attn_desc* d, const void* ws, const int32_t* offs,
                 const int64_t* ts) {
  PlanTag t;
  t.dev = current_device();
  t.p0 = reinterpret_cast<uintptr_t>(ws);
  t.p1 = t.p0 + fwd_plan_bytes(d);
  t.B = d->B;
  t.H = d->H;
  t.d_qk = d->d_qk;
  t.d_v = d->d_v;
  t.dtype = d->dtype;
  t.bm = attn_fwd_block_rows(d->dtype, d->d_qk, d->d_v, fwd_key_halves(d));
  t.T = d->T;
  t.offs = offs;
  t.ts = ts;
  return t;
}

void plan_record(const hstu_attn_desc* d, const void* ws, const int32_t* offs,
                 const int64_t* ts) {
  const PlanTag t = plan_tag(d, ws, offs, ts);
  plans_forget(ws, t.p1 - t.p0);
  std::lock_guard<std::mutex> lk(g_plan_mu);
  if (g_plan_tags.size() >= kMaxPlanTags) g_plan_tags.erase(g_plan_tags.begin());
  g_plan_tags.push_back(t);
}

bool plan_recorded(const hstu_attn_desc* d, const void* ws, const int32_t* offs,
                   const int64_t* ts) {
  const PlanTag q = plan_tag(d, ws, offs, ts);
  std::lock_guard<std::mutex> lk(g_plan_mu);
  for (const PlanTag& t : g_plan_tags)
    if (t.dev == q.dev && t.p0 == q.p0 && t.p1 == q.p1 && t.B == q.B && t.T == q.T &&
        t.H == q.H && t.d_qk == q.d_qk && t.d_v == q.d_v && t.dtype == q.dtype &&
        t.bm == q.bm && t.offs == q.offs && t.ts == q.ts)
      return true;
  return false;
}

// The backward keeps dS (the scores' gradient) when max_len bounds the
// batch: 128 x 128 bf16 blocks of the causal part; with n_b <= max_len the
// blocks number at most H (R + 1) / 2 sum_b ceil(n_b / 128), R = ceil(max_len / 128).
// A batch whose bound exceeds kMaxDsBlocks (4 TiB of blocks, more than the
// device holds) never keeps dS; the bound is computed in 64 bits from
// max_len clamped to T, so no size arithmetic can overflow.
constexpr int64_t kMaxDsBlocks = int64_t(1) << 27;
int64_t ds_capacity_blocks(const hstu_attn_desc* d) {
  const int64_t R = (std::min<int64_t>(d->max_len, d->T) + 127) / 128;
  const int64_t rows = (d->T + 127) / 128 + d->B;
  const int64_t per_head = ((R + 1) * rows + 1) / 2;  // < 2^25 * 2^32
  if (per_head > kMaxDsBlocks) return 0;
  const int64_t blocks = (int64_t)d->H * per_head;
  return blocks > kMaxDsBlocks ? 0 : blocks;
}
bool keeps_ds(const hstu_attn_desc* d) {
  return d->max_len > 0 && d->dtype == HSTU_BF16 && d->d_qk == 128 && d->d_v == 128 &&
         d->win_local == 0 && ds_capacity_blocks(d) > 0;
}

struct BwdWs {
  TimeMeta tm;
  Sched kv, q;
  uint16_t* ds = nullptr;
  int32_t* ds_base = nullptr;
  int32_t* ds_flag = nullptr;
  int64_t ds_cap = 0;
};
BwdWs carve_bwd(Carver& c, const hstu_attn_desc* d) {
  BwdWs w;
  w.tm = carve_time(c, d->T, d->B);
  w.kv = carve_sched(c, d->T, d->B, ATTN_BWD_BN);
  w.q = carve_sched(c, d->T, d->B, ATTN_BWD_BM);
  if (keeps_ds(d)) {
    w.ds_cap = ds_capacity_blocks(d);
    w.ds_base = c.take<int32_t>(std::max<int64_t>(d->B, 1));
    w.ds_flag = c.take<int32_t>(1);
    w.ds = c.take<uint16_t>(w.ds_cap * 128 * 128);
  }
  return w;
}

AttnArgs base_args(const hstu_attn_desc* d, const void* q, const void* k, int64_t ld_qk,
                   const void* v, int64_t ld_v, const int32_t* offs, const int64_t* ts,
                   const float* rp, const float* rt, const int32_t* nc, const TimeMeta& tm) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.ld_qk = ld_qk;
  a.ld_v = ld_v;
  a.seq_offsets = offs;
  a.num_cand = nc;
  a.ts = ts;
  a.rel_t = tm.rel_t;
  a.seq_flags = tm.seq_flags;
  a.rab_pos = rp;
  a.rab_time = rt;
  a.rab_stride = d->rab_head_stride;
  a.B = d->B;
  a.H = d->H;
  a.nP = d->n_pos_buckets;
  a.nT = d->n_time_buckets;
  a.norm_mode = d->norm_mode;
  a.norm_len = d->norm_len;
  a.win_local = d->win_local;
  a.win_global = d->win_local > 0 ? d->win_global : 0;
  return a;
}

int64_t rab_floats(const hstu_attn_desc* d) {
  const int64_t per = std::max(d->n_pos_buckets, d->n_time_buckets);
  return d->rab_head_stride == 0 ? per : d->rab_head_stride * (d->H - 1) + per;
}

// ---- attention forward/backward bodies (shared with the layer) -------------

// The plan of a forward call (time pre-pass and work list, in the workspace)
hstu_status attn_fwd_plan(const hstu_attn_desc* d, const int32_t* offs, const int64_t* ts,
                          void* ws, hipStream_t st) {
  Carver c(ws);
  FwdWs w = carve_fwd(c, d);
  HSTU_TIMED(TT_PREPASS, st);
  PlanArgs p = plan_prepass(w.tm, d->B, offs, ts);
  plan_add_job(p, w.sc, 0, offs);
  HSTU_TRY(launch_plan(p, st));
  return HSTU_OK;
}

// The attention kernel of a forward call whose plan is already in `ws`
hstu_status attn_fwd_run(const hstu_attn_desc* d, const void* q, const void* k, int64_t ld_qk,
                         const void* v, int64_t ld_v, const int32_t* offs, const int64_t* ts,
                         const float* rp, const float* rt, const int32_t* nc, void* out,
                         int64_t ld_out, bool out_f32, void* ws, hipStream_t st,
                         const hstu_attn_mx_qk* mx = nullptr) {
  Carver c(ws);
  FwdWs w = carve_fwd(c, d);
  AttnArgs a = base_args(d, q, k, ld_qk, v, ld_v, offs, ts, rp, rt, nc, w.tm);
  if (mx) {
    a.q_mx = static_cast<const uint8_t*>(mx->q_codes);
    a.k_mx = static_cast<const uint8_t*>(mx->k_codes);
    a.ld_mx = mx->ld_codes;
    a.q_mxs = mx->q_scales;
    a.k_mxs = mx->k_scales;
    a.T_rows = d->T;
  }
  a.out = out;
  a.ld_out = ld_out;
  a.out_f32 = out_f32;
  a.items = w.sc.items;
  a.counters = w.sc.counters;
  a.splits = w.splits;
  a.part = w.part;
  a.part_cnt = w.part_cnt;
  a.key_halves = w.kh ? 1 : 0;
  { HSTU_TIMED(TT_ATTN_FWD, st); HSTU_TRY(launch_attn_fwd(a, d->dtype, d->d_qk, d->d_v, w.sc.cap, st)); }
  return HSTU_OK;
}

hstu_status attn_fwd_impl(const hstu_attn_desc* d, const void* q, const void* k, int64_t ld_qk,
                          const void* v, int64_t ld_v, const int32_t* offs, const int64_t* ts,
                          const float* rp, const float* rt, const int32_t* nc, void* out,
                          int64_t ld_out, bool out_f32, void* ws, hipStream_t st,
                          const hstu_attn_mx_qk* mx = nullptr) {
  if (!d->reuse_plan) {
    hstu_status s = attn_fwd_plan(d, offs, ts, ws, st);
    if (s != HSTU_OK) return s;
    plan_record(d, ws, offs, ts);
  }
  return attn_fwd_run(d, q, k, ld_qk, v, ld_v, offs, ts, rp, rt, nc, out, ld_out, out_f32, ws, st,
                      mx);
}

// Ranking against a cached history: key splits per (user, candidate block)
// chosen from the average history length so that the compute units are
// filled (256 times the workgroups one unit holds), with at least four key
// tiles per split.
int cached_splits(const hstu_attn_desc* d, int64_t T_hist) {
  const int bm = attn_cached_block_rows(d->dtype, d->d_qk, d->d_v);
  const int64_t B = std::max<int64_t>(d->B, 1);
  const int64_t items = std::max<int64_t>((d->T + bm - 1) / bm, B);  // work items (estimate)
  const int64_t tile = d->dtype == HSTU_BF16 ? 64 : 32;
  const int64_t tiles_per_user = (T_hist / B + tile - 1) / tile;
  const int64_t slots = 256 * (int64_t)attn_cached_occupancy(d->dtype, d->d_qk, d->d_v);
  int64_t S = (slots + items * d->H - 1) / (items * d->H);
  S = std::min<int64_t>(S, std::max<int64_t>(tiles_per_user / 4, 1));
  return (int)std::max<int64_t>(1, std::min<int64_t>(S, 16));
}

struct CachedWs {
  int32_t* rel_h = nullptr;
  int32_t* rel_c = nullptr;
  int32_t* flags = nullptr;
  Sched sc;
  float* part = nullptr;
  int splits = 1;
};
CachedWs carve_cached(Carver& c, const hstu_attn_desc* d, int64_t T_hist) {
  CachedWs w;
  w.rel_h = c.take<int32_t>(std::max<int64_t>(T_hist, 1));
  w.rel_c = c.take<int32_t>(std::max<int64_t>(d->T, 1));
  w.flags = c.take<int32_t>(std::max<int64_t>(d->B, 1));
  w.sc = carve_sched(c, d->T, d->B, attn_cached_block_rows(d->dtype, d->d_qk, d->d_v));
  w.splits = cached_splits(d, T_hist);
  if (w.splits > 1) w.part = c.take<float>(w.splits * std::max<int64_t>(d->T, 1) * d->H * d->d_v);
  return w;
}

hstu_status attn_cached_impl(const hstu_attn_desc* d, const void* q, const void* k,
                             int64_t ld_qk, const void* v, int64_t ld_v, const int32_t* coffs,
                             const int64_t* cts, const hstu_history_kv* hist, const float* rp,
                             const float* rt, void* out, int64_t ld_out, bool out_f32, void* ws,
                             hipStream_t st) {
  Carver c(ws);
  CachedWs w = carve_cached(c, d, hist->T);
  CachedArgs a;
  a.q = q; a.k = k; a.v = v; a.ld_qk = ld_qk; a.ld_v = ld_v;
  a.cand_offsets = coffs; a.cand_ts = cts;
  a.kh = hist->k; a.vh = hist->v; a.ld_kh = hist->ld_k; a.ld_vh = hist->ld_v;
  a.hist_offsets = hist->offsets; a.hist_ts = hist->timestamps;
  a.rel_h = w.rel_h; a.rel_c = w.rel_c; a.flags = w.flags;
  a.items = w.sc.items; a.counters = w.sc.counters;
  a.out = out; a.ld_out = ld_out; a.out_f32 = out_f32;
  a.part = w.part; a.Tc = d->T; a.splits = w.splits;
  a.rab_pos = rp; a.rab_time = rt; a.rab_stride = d->rab_head_stride;
  a.B = d->B;
  a.H = d->H; a.nP = d->n_pos_buckets; a.nT = d->n_time_buckets; a.norm_len = d->norm_len;
  a.win_local = d->win_local; a.win_global = d->win_global;
  {
    HSTU_TIMED(TT_PREPASS, st);
    PlanArgs p;
    p.npre = d->B;
    p.mode = 1;
    p.offs = hist->offsets;
    p.ts = hist->timestamps;
    p.rel_t = w.rel_h;
    p.flags = w.flags;
    p.coffs = coffs;
    p.cts = cts;
    p.rel_c = w.rel_c;
    p.B = d->B;
    plan_add_job(p, w.sc, 0, coffs);
    HSTU_TRY(launch_plan(p, st));
  }
  {
    HSTU_TIMED(TT_ATTN_CACHED, st);
    HSTU_TRY(launch_attn_cached(a, d->dtype, d->d_qk, d->d_v, w.sc.cap, st));
  }
  return HSTU_OK;
}

hstu_status check_history(const hstu_attn_desc* d, const hstu_history_kv* hist) {
  if (!hist || !hist->offsets || hist->T < 0 || hist->T >= (int64_t(1) << 31))
    return HSTU_ERR_INVALID_ARG;
  if (hist->T > 0 && (!hist->k || !hist->v || !hist->timestamps)) return HSTU_ERR_INVALID_ARG;
  const int64_t hq = (int64_t)d->H * d->d_qk, hv = (int64_t)d->H * d->d_v;
  if (hist->T > 0 && (!stride_ok(d->dtype, hist->k, hist->ld_k, hq) ||
                      !stride_ok(d->dtype, hist->v, hist->ld_v, hv)))
    return HSTU_ERR_INVALID_ARG;
  if (d->norm_mode != 0) return HSTU_ERR_UNSUPPORTED;
  return HSTU_OK;
}

// The plan of a backward call (time pre-pass, both work lists, kept-dS
// offsets; zeroes the rab gradients)
hstu_status attn_bwd_plan(const hstu_attn_desc* d, const int32_t* offs, const int64_t* ts,
                          float* drp, float* drt, void* ws, hipStream_t st) {
  Carver c(ws);
  BwdWs w = carve_bwd(c, d);
  HSTU_TIMED(TT_PREPASS, st);
  PlanArgs p = plan_prepass(w.tm, d->B, offs, ts, drp, drt, rab_floats(d));
  plan_add_job(p, w.kv, 1, offs);
  plan_add_job(p, w.q, 0, offs);
  if (w.ds) {
    p.ds_base = w.ds_base;
    p.ds_flag = w.ds_flag;
    p.ds_cap = w.ds_cap;
    p.H = d->H;
  }
  HSTU_TRY(launch_plan(p, st));
  return HSTU_OK;
}

// The attention kernels of a backward call whose plan is already in `ws`
hstu_status attn_bwd_run(const hstu_attn_desc* d, const void* q, const void* k, int64_t ld_qk,
                         const void* v, int64_t ld_v, const int32_t* offs, const int64_t* ts,
                         const float* rp, const float* rt, const int32_t* nc, const void* dout,
                         int64_t ld_dout, void* dq, void* dk, void* dv, float* drp, float* drt,
                         const void* zpre, int64_t ld_z, int64_t zq, int64_t zk, int64_t zv,
                         void* ws, hipStream_t st) {
  Carver c(ws);
  BwdWs w = carve_bwd(c, d);
  AttnArgs a = base_args(d, q, k, ld_qk, v, ld_v, offs, ts, rp, rt, nc, w.tm);
  a.dout = dout;
  a.ld_dout = ld_dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.drab_pos = drp;
  a.drab_time = drt;
  a.zpre = zpre;
  a.ld_z = ld_z;
  a.zq_col = zq;
  a.zk_col = zk;
  a.zv_col = zv;
  a.ds = w.ds;
  a.ds_base = w.ds_base;
  a.ds_flag = w.ds_flag;
  AttnArgs akv = a;
  akv.items = w.kv.items;
  akv.counters = w.kv.counters;
  { HSTU_TIMED(TT_ATTN_BWD_DKDV, st); HSTU_TRY(launch_attn_bwd_dkdv(akv, d->d_qk, d->d_v, w.kv.cap, st)); }
  AttnArgs aq = a;
  aq.items = w.q.items;
  aq.counters = w.q.counters;
  { HSTU_TIMED(TT_ATTN_BWD_DQ, st); HSTU_TRY(launch_attn_bwd_dq(aq, d->d_qk, d->d_v, w.q.cap, st)); }
  return HSTU_OK;
}

hstu_status attn_bwd_impl(const hstu_attn_desc* d, const void* q, const void* k, int64_t ld_qk,
                          const void* v, int64_t ld_v, const int32_t* offs, const int64_t* ts,
                          const float* rp, const float* rt, const int32_t* nc, const void* dout,
                          int64_t ld_dout, void* dq, void* dk, void* dv, float* drp, float* drt,
                          const void* zpre, int64_t ld_z, int64_t zq, int64_t zk, int64_t zv,
                          void* ws, hipStream_t st) {
  hstu_status s = attn_bwd_plan(d, offs, ts, drp, drt, ws, st);
  if (s != HSTU_OK) return s;
  return attn_bwd_run(d, q, k, ld_qk, v, ld_v, offs, ts, rp, rt, nc, dout, ld_dout, dq, dk, dv,
                      drp, drt, zpre, ld_z, zq, zk, zv, ws, st);
}

// ---- layer workspace layout --------------------------------------------------

int64_t f1_width(const hstu_layer_desc* L) {
  return (int64_t)L->attn.H * (2 * L->attn.d_v + 2 * L->attn.d_qk);
}

struct LayerFwdWs {
  void* Zh = nullptr;
  void* O = nullptr;
  void* G = nullptr;
  void* attn = nullptr;
};
LayerFwdWs carve_layer_fwd(Carver& c, const hstu_layer_desc* L, int training) {
  LayerFwdWs w;
  const hstu_attn_desc* d = &L->attn;
  const size_t es = esize(d->dtype);
  const int64_t T = std::max<int64_t>(d->T, 1);
  if (!training) {
    w.Zh = c.take<char>(T * f1_width(L) * es);
    w.O = c.take<float>(T * (int64_t)d->H * d->d_v);  // O stays fp32 up to the LayerNorm
    w.G = c.take<char>(T * (int64_t)d->H * d->d_v * es);
  }
  w.attn = c.take<char>(0);
  carve_fwd(c, d);
  return w;
}

// Candidate-only layer: Zh, O, G of the candidate rows, then the cached
// attention's own workspace.
LayerFwdWs carve_layer_cached(Carver& c, const hstu_layer_desc* L, int64_t T_hist) {
  LayerFwdWs w;
  const hstu_attn_desc* d = &L->attn;
  const size_t es = esize(d->dtype);
  const int64_t T = std::max<int64_t>(d->T, 1);
  w.Zh = c.take<char>(T * f1_width(L) * es);
  w.O = c.take<float>(T * (int64_t)d->H * d->d_v);
  w.G = c.take<char>(T * (int64_t)d->H * d->d_v * es);
  w.attn = c.take<char>(0);
  carve_cached(c, d, T_hist);
  return w;
}

// Splits of the weight-gradient GEMMs' k (token) range: enough workgroups to
// fill the GPU twice over, at least 512 tokens each, at most 32; a multiple
// of 8 from 8 up, so that every XCD takes whole splits (see the GEMM kernel).
int splitk_for(int64_t M, int64_t N, int64_t K) {
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int64_t s = (512 + tiles - 1) / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(1, K / 512));
  s = std::max<int64_t>(1, std::min<int64_t>(s, 32));
  return (int)(s >= 8 ? s / 8 * 8 : s);
}

struct LayerBwdWs {
  void* dG = nullptr;
  void* dO = nullptr;
  void* dZ = nullptr;
  float* part1 = nullptr;   // split-K partials of dW1
  float* part2 = nullptr;   // split-K partials of dW2
  float* colws = nullptr;   // column-sum scratch
  float* lnpg = nullptr;    // LayerNorm partial dgamma
  float* lnpb = nullptr;
  void* attn = nullptr;
  int s1 = 1, s2 = 1;
  int64_t ln_blocks = 1;
};
LayerBwdWs carve_layer_bwd(Carver& c, const hstu_layer_desc* L) {
  LayerBwdWs w;
  const hstu_attn_desc* d = &L->attn;
  const size_t es = esize(d->dtype);
  const int64_t T = std::max<int64_t>(d->T, 1);
  const int64_t W = (int64_t)d->H * d->d_v, F1 = f1_width(L), D = L->D;
  w.dG = c.take<char>(T * W * es);
  w.dO = c.take<char>(T * W * es);
  w.dZ = c.take<char>(T * F1 * es);
  w.s1 = splitk_for(D, F1, d->T);
  w.s2 = splitk_for(W, D, d->T);
  w.part1 = c.take<float>((int64_t)w.s1 * D * F1);
  w.part2 = c.take<float>((int64_t)w.s2 * W * D);
  w.colws = c.take<float>(64 * std::max<int64_t>(F1, std::max<int64_t>(D, W)));
  w.ln_blocks = ln_bwd_part_blocks(d->T);
  w.lnpg = c.take<float>(w.ln_blocks * W);
  w.lnpb = c.take<float>(w.ln_blocks * W);
  w.attn = c.take<char>(0);
  carve_bwd(c, d);
  return w;
}

hstu_status check_layer(const hstu_layer_desc* L) {
  if (!L) return HSTU_ERR_INVALID_ARG;
  hstu_status s = check_attn_desc(&L->attn);
  if (s != HSTU_OK) return s;
  if (L->D < 8 || L->D % 8 != 0) return HSTU_ERR_UNSUPPORTED;
  if ((int64_t)L->attn.H * L->attn.d_v > 1024) return HSTU_ERR_UNSUPPORTED;
  if (!(L->ln_eps >= 0.0f)) return HSTU_ERR_INVALID_ARG;
  return HSTU_OK;
}

hstu_status check_trunc_copy(int32_t B, int64_t T, int64_t T_seg, int32_t D, int32_t dtype,
                             const void* a, const void* b, const int32_t* offs,
                             const int32_t* seg) {
  if (dtype != HSTU_F32 && dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
  if (B < 0 || T < 0 || T_seg < 0 || D <= 0 || T >= (int64_t(1) << 31) ||
      T_seg >= (int64_t(1) << 31))
    return HSTU_ERR_INVALID_ARG;
  if ((int64_t(D) * esize(dtype)) % 16 != 0) return HSTU_ERR_INVALID_ARG;
  if (!offs || !seg) return HSTU_ERR_INVALID_ARG;
  if ((T > 0 && !a) || (T_seg > 0 && !b)) return HSTU_ERR_INVALID_ARG;
  if ((a && !aligned16(a)) || (b && !aligned16(b))) return HSTU_ERR_INVALID_ARG;
  return HSTU_OK;
}

// Steps 1-4 of one layer on T rows, with the attention step supplied by the
// caller (causal / target-aware over the rows' own sequences, or candidates
// against a cached history).  Zsave, mu, rstd: optional saved intermediates.
// MXFP8 projection and output products: the weights' codes and scales and
// workspace for the quantized activations (X and G).
struct MxPlan {
  const hstu_mx_weights* wm = nullptr;
  uint8_t* x8 = nullptr;
  uint8_t* xs = nullptr;
  bool x_ready = false;   // x8/xs already hold X (given by the caller)
  uint8_t* g8 = nullptr;
  uint8_t* gs = nullptr;
  uint8_t* y8 = nullptr;  // optional MXFP8 copy of Y (the next layer's X)
  uint8_t* ys = nullptr;
  // optional MXFP8 copy of the attention's Q|K columns ([T][2 H d_qk] codes,
  // [2H][T] scale words), written by the projection's epilogue
  uint8_t* qk8 = nullptr;
  uint32_t* qks = nullptr;
  bool qk_dequant = false;  // store Q|K as their MXFP8 values too (training)
};

template <typename Attn>
hstu_status layer_fwd_steps(const hstu_layer_desc* L, const void* x, const hstu_layer_weights* w,
                            void* y, void* Zsave, void* Zh, float* O, void* G, float* mu,
                            float* rstd, Attn attention, hipStream_t st,
                            const MxPlan* mx = nullptr) {
  const hstu_attn_desc* d = &L->attn;
  const int64_t T = d->T, D = L->D, F1 = f1_width(L);
  const int64_t W = (int64_t)d->H * d->d_v, HQ = (int64_t)d->H * d->d_qk;
  const size_t es = esize(d->dtype);
  char* zh = static_cast<char*>(Zh);

  // 1. Z = X W1 (+ b1); Zh = SiLU(Z)
  GemmArgs g1;
  g1.M = T;
  g1.N = F1;
  g1.K = D;
  g1.A = x;
  g1.lda = D;
  g1.a_kcont = true;
  g1.B = w->W1;
  g1.ldb = F1;
  g1.b_kcont = false;
  g1.C = Zh;
  g1.ldc = F1;
  g1.bias = w->b1;
  if (L->proj_silu) {
    g1.epi = EPI_SILU;
    g1.C2 = Zsave;
  } else {
    g1.epi = EPI_RESID;  // bias only
    g1.R = nullptr;
  }
  if (mx) {
    // X -> MXFP8 (blocks of 32 along d_model), W1 given as [F1][D] codes
    if (!mx->x_ready) {
      HSTU_TIMED(TT_MX_QUANT, st);
      HSTU_TRY(launch_mx_quant_rows(x, D, T, D, mx->x8, mx->xs, st));
    }
    g1.mx = true;
    g1.A = mx->x8;
    g1.lda = D / 2;
    g1.K = D / 2;
    g1.B = mx->wm->W1;
    g1.ldb = D / 2;
    g1.b_kcont = true;
    g1.scale_a = mx->xs;
    g1.scale_b = static_cast<const uint8_t*>(mx->wm->W1_scales);
    if (mx->qk8) {
      g1.qk_codes = mx->qk8;
      g1.qk_scales = reinterpret_cast<uint8_t*>(mx->qks);
      g1.qk_col0 = 2 * (int64_t)d->H * d->d_v;
      g1.qk_cols = 2 * (int64_t)d->H * d->d_qk;
      g1.qk_d = d->d_qk;
      g1.qk_dequant = mx->qk_dequant;
    }
  }
  { HSTU_TIMED(TT_GEMM_UVQK, st); HSTU_TRY(launch_gemm(g1, d->dtype, st)); }
  if (!L->proj_silu && Zsave) {
    // without the nonlinearity Z and Zh coincide
    GemmArgs gz = g1;
    gz.C = Zsave;
    HSTU_TRY(launch_gemm(gz, d->dtype, st));
  }
  // 2. attention on the V, Q, K column blocks (q, k, v, ld; O fp32)
  hstu_status s = attention(zh + 2 * W * es, zh + (2 * W + HQ) * es, zh + W * es, F1);
  if (s != HSTU_OK) return s;
  // 3. G = LN(O) * U
  LnArgs la;
  la.o_f32 = true;
  la.T = T;
  la.W = (int)W;
  la.O = O;
  la.ld_o = W;
  la.U = Zh;
  la.ld_u = F1;
  la.gamma = w->ln_gamma;
  la.beta = w->ln_beta;
  la.eps = L->ln_eps;
  la.G = G;
  la.ld_g = W;
  la.mu = mu;
  la.rstd = rstd;
  if (mx) {
    // G straight to MXFP8 for the output product; the bf16 G only when the
    // call keeps the intermediates for training
    la.g_codes = mx->g8;
    la.g_scales = mx->gs;
    if (!mu) la.G = nullptr;
  }
  { HSTU_TIMED(TT_LN_FWD, st); HSTU_TRY(launch_ln_gate_fwd(la, d->dtype, st)); }
  // 4. Y = G W2 (+ b2) (+ X)
  GemmArgs g2;
  g2.M = T;
  g2.N = D;
  g2.K = W;
  g2.A = G;
  g2.lda = W;
  g2.a_kcont = true;
  g2.B = w->W2;
  g2.ldb = D;
  g2.b_kcont = false;
  g2.C = y;
  g2.ldc = D;
  g2.epi = EPI_RESID;
  g2.bias = w->b2;
  g2.R = L->residual ? x : nullptr;
  g2.ldr = D;
  if (mx) {
    // G as MXFP8 (blocks of 32 along H d_v, written by the LayerNorm
    // kernel), W2 given as [D][H d_v] codes
    g2.mx = true;
    g2.A = mx->g8;
    g2.lda = W / 2;
    g2.K = W / 2;
    g2.B = mx->wm->W2;
    g2.ldb = W / 2;
    g2.b_kcont = true;
    g2.scale_a = mx->gs;
    g2.scale_b = static_cast<const uint8_t*>(mx->wm->W2_scales);
    g2.c_codes = mx->y8;
    g2.c_scales = mx->ys;
  }
  { HSTU_TIMED(TT_GEMM_OUT, st); HSTU_TRY(launch_gemm(g2, d->dtype, st)); }
  return HSTU_OK;
}

// ---- scratch of hstu_attn_fwd_noalloc ---------------------------------------
// The plan of the no-allocation forward lives in this array: one copy per GPU
// (each device holds its own, at its own address, until the process ends).
// In host code the name is only a stand-in for the symbol: device addresses
// come from hipGetSymbolAddress, taken once per device with that device
// current, and only those are handed to kernels.
__device__ __align__(256) unsigned char scratch[HSTU_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of the current device's scratch, resolved on first use
hipError_t scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char* hstu_status_string(hstu_status s) {
  switch (s) {
    case HSTU_OK: return "ok";
    case HSTU_ERR_INVALID_ARG: return "invalid argument";
    case HSTU_ERR_UNSUPPORTED: return "unsupported configuration";
    case HSTU_ERR_WORKSPACE: return "workspace too small";
    case HSTU_ERR_HIP: return "HIP launch error";
    case HSTU_ERR_VALIDATION: return "device-side input contract violated";
  }
  return "unknown status";
}

const char* hstu_last_hip_error(void) { return hipGetErrorString(g_last_hip_error); }

const char* hstu_last_error_site(void) { return g_last_error_site; }

hstu_status hstu_set_check_mode(int32_t on) {
  if (on != 0 && on != 1) return HSTU_ERR_INVALID_ARG;
  g_check_mode.store(on);
  return HSTU_OK;
}

int32_t hstu_check_mode(void) { return g_check_mode.load(); }

const char* hstu_version(void) { return "hstu-mi355x 0.1 (gfx950)"; }

size_t hstu_attn_fwd_workspace_size(const hstu_attn_desc* d) {
  if (check_attn_desc(d) != HSTU_OK) return 0;
  Carver c(nullptr);
  carve_fwd(c, d);
  return c.off + 256;
}

size_t hstu_attn_bwd_workspace_size(const hstu_attn_desc* d) {
  if (check_attn_desc(d) != HSTU_OK) return 0;
  Carver c(nullptr);
  carve_bwd(c, d);
  return c.off + 256;
}

hstu_status hstu_attn_fwd(const hstu_attn_desc* d, const void* q, const void* k, int64_t ld_qk,
                          const void* v, int64_t ld_v, const int32_t* offs, const int64_t* ts,
                          const float* rp, const float* rt, const int32_t* nc, void* out,
                          int64_t ld_out, void* ws, size_t ws_bytes, void* stream) {
  hstu_status s = check_attn_desc(d);
  if (s != HSTU_OK) return s;
  if (d->T > 0 && (!q || !k || !v || !out || !ts)) return HSTU_ERR_INVALID_ARG;
  if (!offs || !rp || !rt || !ws) return HSTU_ERR_INVALID_ARG;
  const int64_t hq = (int64_t)d->H * d->d_qk, hv = (int64_t)d->H * d->d_v;
  if (d->T > 0 && (!stride_ok(d->dtype, q, ld_qk, hq) || !stride_ok(d->dtype, k, ld_qk, hq) ||
                   !stride_ok(d->dtype, v, ld_v, hv) || ld_out < hv))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(ws)) return HSTU_ERR_INVALID_ARG;
  if (ws_bytes < hstu_attn_fwd_workspace_size(d)) return HSTU_ERR_WORKSPACE;
  if (d->reuse_plan && !plan_recorded(d, ws, offs, ts)) return HSTU_ERR_INVALID_ARG;
  return attn_fwd_impl(d, q, k, ld_qk, v, ld_v, offs, ts, rp, rt, nc, out, ld_out, false, ws,
                       entry_stream(stream));
}

hstu_status hstu_attn_fwd_mx(const hstu_attn_desc* d, const hstu_attn_mx_qk* qk, const void* v,
                             int64_t ld_v, const int32_t* offs, const int64_t* ts,
                             const float* rp, const float* rt, const int32_t* nc, void* out,
                             int64_t ld_out, void* ws, size_t ws_bytes, void* stream) {
  hstu_status s = check_attn_desc(d);
  if (s != HSTU_OK) return s;
  if (!qk) return HSTU_ERR_INVALID_ARG;
  if (d->dtype != HSTU_BF16 || d->d_qk != d->d_v || (d->d_qk != 64 && d->d_qk != 128) ||
      d->win_local > 0 || d->key_splits > 1)
    return HSTU_ERR_UNSUPPORTED;
  const int64_t hq = (int64_t)d->H * d->d_qk, hv = (int64_t)d->H * d->d_v;
  if (d->T > 0 && (!qk->q_codes || !qk->k_codes || !qk->q_scales || !qk->k_scales || !v ||
                   !out || !ts))
    return HSTU_ERR_INVALID_ARG;
  if (!offs || !rp || !rt || !ws) return HSTU_ERR_INVALID_ARG;
  if (d->T > 0 && (!aligned16(qk->q_codes) || !aligned16(qk->k_codes) || qk->ld_codes < hq ||
                   qk->ld_codes % 16 != 0 ||
                   (reinterpret_cast<uintptr_t>(qk->q_scales) & 3) ||
                   (reinterpret_cast<uintptr_t>(qk->k_scales) & 3) ||
                   !stride_ok(d->dtype, v, ld_v, hv) || ld_out < hv))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(ws)) return HSTU_ERR_INVALID_ARG;
  if (ws_bytes < hstu_attn_fwd_workspace_size(d)) return HSTU_ERR_WORKSPACE;
  if (d->reuse_plan && !plan_recorded(d, ws, offs, ts)) return HSTU_ERR_INVALID_ARG;
  return attn_fwd_impl(d, nullptr, nullptr, 0, v, ld_v, offs, ts, rp, rt, nc, out, ld_out, false,
                       ws, entry_stream(stream), qk);
}

hstu_status hstu_mx_quantize_heads(int64_t T, int32_t H, int32_t dh, const void* x, int64_t ld,
                                   void* codes, int64_t ld_codes, uint32_t* scales,
                                   void* stream) {
  if (T < 0 || H <= 0 || H > 64 || dh <= 0 || dh % 32 != 0 || dh > 128)
    return HSTU_ERR_INVALID_ARG;
  const int64_t w = (int64_t)H * dh;
  if (ld < w || ld_codes < w || ld % 8 != 0 || ld_codes % 16 != 0) return HSTU_ERR_INVALID_ARG;
  if (T > 0 && (!x || !codes || !scales || !aligned16(x) || !aligned16(codes) ||
                (reinterpret_cast<uintptr_t>(scales) & 3)))
    return HSTU_ERR_INVALID_ARG;
  hipStream_t st = entry_stream(stream);
  HSTU_TIMED(TT_MX_QUANT, st);
  HSTU_TRY(launch_mx_quant_heads(x, ld, T, H, dh, static_cast<uint8_t*>(codes), ld_codes,
                                 scales, st));
  return HSTU_OK;
}

hstu_status hstu_attn_fwd_noalloc(const hstu_attn_desc* d, const void* q, const void* k,
                                  int64_t ld_qk, const void* v, int64_t ld_v, const int32_t* offs,
                                  const int64_t* ts, const float* rp, const float* rt,
                                  const int32_t* nc, void* out, int64_t ld_out, void* stream) {
  hstu_status s = check_attn_desc(d);
  if (s != HSTU_OK) return s;
  if (d->T > 0 && (!q || !k || !v || !out || !ts)) return HSTU_ERR_INVALID_ARG;
  if (!offs || !rp || !rt) return HSTU_ERR_INVALID_ARG;
  const int64_t hq = (int64_t)d->H * d->d_qk, hv = (int64_t)d->H * d->d_v;
  if (d->T > 0 && (!stride_ok(d->dtype, q, ld_qk, hq) || !stride_ok(d->dtype, k, ld_qk, hq) ||
                   !stride_ok(d->dtype, v, ld_v, hv) || ld_out < hv))
    return HSTU_ERR_INVALID_ARG;
  if (hstu_attn_fwd_workspace_size(d) > HSTU_NOALLOC_SCRATCH_BYTES) return HSTU_ERR_WORKSPACE;
  void* ws = nullptr;
  HSTU_TRY(scratch_for_current_device(&ws));
  if (d->reuse_plan && !plan_recorded(d, ws, offs, ts)) return HSTU_ERR_INVALID_ARG;
  return attn_fwd_impl(d, q, k, ld_qk, v, ld_v, offs, ts, rp, rt, nc, out, ld_out, false, ws,
                       entry_stream(stream));
}

size_t hstu_attn_cached_workspace_size(const hstu_attn_desc* d, int64_t T_hist) {
  if (check_attn_desc(d) != HSTU_OK || T_hist < 0) return 0;
  Carver c(nullptr);
  carve_cached(c, d, T_hist);
  return c.off + 256;
}

hstu_status hstu_attn_cached_fwd(const hstu_attn_desc* d, const void* q, const void* k,
                                 int64_t ld_qk, const void* v, int64_t ld_v, const int32_t* coffs,
                                 const int64_t* cts, const hstu_history_kv* hist,
                                 const float* rp, const float* rt, void* out, int64_t ld_out,
                                 void* ws, size_t ws_bytes, void* stream) {
  hstu_status s = check_attn_desc(d);
  if (s != HSTU_OK) return s;
  s = check_history(d, hist);
  if (s != HSTU_OK) return s;
  if (d->T > 0 && (!q || !k || !v || !out || !cts)) return HSTU_ERR_INVALID_ARG;
  if (!coffs || !rp || !rt || !ws) return HSTU_ERR_INVALID_ARG;
  const int64_t hq = (int64_t)d->H * d->d_qk, hv = (int64_t)d->H * d->d_v;
  if (d->T > 0 && (!stride_ok(d->dtype, q, ld_qk, hq) || !stride_ok(d->dtype, k, ld_qk, hq) ||
                   !stride_ok(d->dtype, v, ld_v, hv) || ld_out < hv))
    return HSTU_ERR_INVALID_ARG;
  // fp32 outputs are written four at a time
  if (d->T > 0 && d->dtype == HSTU_F32 && (!aligned16(out) || ld_out % 4 != 0))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(ws)) return HSTU_ERR_INVALID_ARG;
  if (ws_bytes < hstu_attn_cached_workspace_size(d, hist->T)) return HSTU_ERR_WORKSPACE;
  plans_forget(ws, ws_bytes);
  return attn_cached_impl(d, q, k, ld_qk, v, ld_v, coffs, cts, hist, rp, rt, out, ld_out, false,
                          ws, entry_stream(stream));
}

hstu_status hstu_attn_bwd(const hstu_attn_desc* d, const void* q, const void* k, int64_t ld_qk,
                          const void* v, int64_t ld_v, const int32_t* offs, const int64_t* ts,
                          const float* rp, const float* rt, const int32_t* nc, const void* dout,
                          int64_t ld_dout, void* dq, void* dk, void* dv, float* drp, float* drt,
                          void* ws, size_t ws_bytes, void* stream) {
  hstu_status s = check_attn_desc(d);
  if (s != HSTU_OK) return s;
  if (d->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
  if (d->T > 0 && (!q || !k || !v || !dout || !dq || !dk || !dv || !ts))
    return HSTU_ERR_INVALID_ARG;
  if (!offs || !rp || !rt || !drp || !drt || !ws) return HSTU_ERR_INVALID_ARG;
  const int64_t hq = (int64_t)d->H * d->d_qk, hv = (int64_t)d->H * d->d_v;
  if (d->T > 0 && (!stride_ok(d->dtype, q, ld_qk, hq) || !stride_ok(d->dtype, k, ld_qk, hq) ||
                   !stride_ok(d->dtype, v, ld_v, hv) || !stride_ok(d->dtype, dout, ld_dout, hv)))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(ws)) return HSTU_ERR_INVALID_ARG;
  if (ws_bytes < hstu_attn_bwd_workspace_size(d)) return HSTU_ERR_WORKSPACE;
  plans_forget(ws, ws_bytes);
  return attn_bwd_impl(d, q, k, ld_qk, v, ld_v, offs, ts, rp, rt, nc, dout, ld_dout, dq, dk, dv,
                       drp, drt, nullptr, 0, 0, 0, 0, ws, entry_stream(stream));
}

size_t hstu_layer_fwd_workspace_size(const hstu_layer_desc* L, int training) {
  if (check_layer(L) != HSTU_OK) return 0;
  Carver c(nullptr);
  carve_layer_fwd(c, L, training);
  return c.off + 256;
}

size_t hstu_layer_bwd_workspace_size(const hstu_layer_desc* L) {
  if (check_layer(L) != HSTU_OK) return 0;
  Carver c(nullptr);
  carve_layer_bwd(c, L);
  return c.off + 256;
}

hstu_status hstu_layer_fwd(const hstu_layer_desc* L, const void* x, const hstu_layer_weights* w,
                           const int32_t* offs, const int64_t* ts, const int32_t* nc, void* y,
                           const hstu_layer_saved* saved, void* ws, size_t ws_bytes,
                           void* stream) {
  hstu_status s = check_layer(L);
  if (s != HSTU_OK) return s;
  const hstu_attn_desc* d = &L->attn;
  if (!w || !w->W1 || !w->W2 || !w->rab_pos || !w->rab_time || !offs || !ws)
    return HSTU_ERR_INVALID_ARG;
  if (d->T > 0 && (!x || !y || !ts)) return HSTU_ERR_INVALID_ARG;
  if (x == y && d->T > 0) return HSTU_ERR_INVALID_ARG;
  // saved: every buffer (training), or Zh alone (keeping U|V|Q|K, e.g. the
  // keys and values of a history for later cached ranking)
  const bool full = saved && saved->Z && saved->Zh && saved->O && saved->G && saved->mu &&
                    saved->rstd;
  const bool zh_only = saved && saved->Zh && !saved->Z && !saved->O && !saved->G &&
                       !saved->mu && !saved->rstd;
  if (saved && !full && !zh_only) return HSTU_ERR_INVALID_ARG;
  if (d->dtype == HSTU_BF16) {
    if (!aligned16(x) || !aligned16(y) || !aligned16(w->W1) || !aligned16(w->W2))
      return HSTU_ERR_INVALID_ARG;
    if (saved && (!aligned16(saved->Z) || !aligned16(saved->Zh) || !aligned16(saved->G)))
      return HSTU_ERR_INVALID_ARG;
  }
  if (!aligned16(ws)) return HSTU_ERR_INVALID_ARG;
  if (ws_bytes < hstu_layer_fwd_workspace_size(L, full)) return HSTU_ERR_WORKSPACE;
  hipStream_t st = entry_stream(stream);

  Carver c(ws);
  LayerFwdWs lw = carve_layer_fwd(c, L, full);
  if (d->reuse_plan) {
    if (!plan_recorded(d, lw.attn, offs, ts)) return HSTU_ERR_INVALID_ARG;
    plans_forget(ws, static_cast<char*>(lw.attn) - static_cast<char*>(ws));
  } else {
    plans_forget(ws, ws_bytes);
  }
  const int64_t W = (int64_t)d->H * d->d_v;
  void* Zh = saved ? saved->Zh : lw.Zh;
  float* O = full ? saved->O : static_cast<float*>(lw.O);
  void* G = full ? saved->G : lw.G;
  // (the plan stays on the caller's stream: moving it under the projection
  // GEMM on the side stream measured slower, the two events costing more
  // than the ~18 us plan)
  auto attention = [&](const void* q, const void* k, const void* v, int64_t ld) {
    return attn_fwd_impl(d, q, k, ld, v, ld, offs, ts, w->rab_pos, w->rab_time, nc, O, W,
                         /*out_f32=*/true, lw.attn, st);
  };
  return layer_fwd_steps(L, x, w, y, full ? saved->Z : nullptr, Zh, O, G,
                         full ? saved->mu : nullptr, full ? saved->rstd : nullptr, attention, st);
}

// descriptors whose attention can take its score product in MXFP8
bool mx_scores_ok(const hstu_attn_desc* d) {
  return d->dtype == HSTU_BF16 && d->d_qk == d->d_v && (d->d_qk == 64 || d->d_qk == 128) &&
         d->win_local == 0 && d->key_splits <= 1;
}

// MXFP8 layer: the inference workspace plus the quantized X and G, and (for
// descriptors that allow MXFP8 scores) the codes of Q|K, [T][2 H d_qk], and
// their head-major scale words, [2H][T]
struct MxWs {
  uint8_t *x8, *xs, *g8, *gs, *qk8 = nullptr;
  uint32_t* qks = nullptr;
};
MxWs carve_mx(Carver& c, const hstu_layer_desc* L) {
  const hstu_attn_desc* d = &L->attn;
  const int64_t T = std::max<int64_t>(d->T, 1), D = L->D, W = (int64_t)d->H * d->d_v;
  MxWs m;
  m.x8 = c.take<uint8_t>(T * D);
  m.xs = c.take<uint8_t>(T * D / 32);
  m.g8 = c.take<uint8_t>(T * W);
  m.gs = c.take<uint8_t>(T * W / 32);
  if (mx_scores_ok(d)) {
    m.qk8 = c.take<uint8_t>(T * 2 * d->H * d->d_qk);
    m.qks = c.take<uint32_t>(T * 2 * d->H);
  }
  return m;
}

hstu_status check_mx_layer(const hstu_layer_desc* L) {
  hstu_status s = check_layer(L);
  if (s != HSTU_OK) return s;
  const int64_t W = (int64_t)L->attn.H * L->attn.d_v;
  if (L->attn.dtype != HSTU_BF16 || L->D % 128 != 0 || W % 128 != 0) return HSTU_ERR_UNSUPPORTED;
  return HSTU_OK;
}

size_t hstu_layer_fwd_mx_workspace_size(const hstu_layer_desc* L) {
  if (check_mx_layer(L) != HSTU_OK) return 0;
  Carver c(nullptr);
  carve_mx(c, L);
  carve_layer_fwd(c, L, 0);
  return c.off + 256;
}

hstu_status hstu_layer_fwd_mx(const hstu_layer_desc* L, const void* x, const hstu_layer_weights* w,
                              const hstu_mx_weights* wm, const int32_t* offs, const int64_t* ts,
                              const int32_t* nc, void* y, const hstu_mx_io* io,
                              const hstu_layer_saved* saved, void* ws, size_t ws_bytes,
                              void* stream) {
  hstu_status s = check_mx_layer(L);
  if (s != HSTU_OK) return s;
  // saved (training): every buffer, as hstu_layer_fwd's
  if (saved && !(saved->Z && saved->Zh && saved->O && saved->G && saved->mu && saved->rstd &&
                 aligned16(saved->Z) && aligned16(saved->Zh) && aligned16(saved->G)))
    return HSTU_ERR_INVALID_ARG;
  const hstu_attn_desc* d = &L->attn;
  if (!w || !w->rab_pos || !w->rab_time || !offs || !ws || !wm || !wm->W1 || !wm->W1_scales ||
      !wm->W2 || !wm->W2_scales)
    return HSTU_ERR_INVALID_ARG;
  if (d->T > 0 && (!x || !y || !ts)) return HSTU_ERR_INVALID_ARG;
  if (x == y && d->T > 0) return HSTU_ERR_INVALID_ARG;
  if (io) {
    auto pair_ok = [](const void* c, const void* sc) {
      return (c == nullptr) == (sc == nullptr) && aligned16(c) &&
             (reinterpret_cast<uintptr_t>(sc) & 3) == 0;
    };
    if (!pair_ok(io->x_codes, io->x_scales) || !pair_ok(io->y_codes, io->y_scales) ||
        !pair_ok(io->g_codes, io->g_scales))
      return HSTU_ERR_INVALID_ARG;
    if (io->mx_scores != 0 && io->mx_scores != 1) return HSTU_ERR_INVALID_ARG;
    // training (saved) needs the projection's SiLU epilogue, which stores q
    // and k as their MXFP8 values for the backward
    if (io->mx_scores && (!mx_scores_ok(d) || (saved && !L->proj_silu)))
      return HSTU_ERR_UNSUPPORTED;
  }
  const bool mx_scores = io && io->mx_scores;
  if (!aligned16(x) || !aligned16(y) || !aligned16(wm->W1) || !aligned16(wm->W2) ||
      (reinterpret_cast<uintptr_t>(wm->W1_scales) & 3) ||
      (reinterpret_cast<uintptr_t>(wm->W2_scales) & 3))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(ws)) return HSTU_ERR_INVALID_ARG;
  if (ws_bytes < hstu_layer_fwd_mx_workspace_size(L)) return HSTU_ERR_WORKSPACE;
  hipStream_t st = entry_stream(stream);

  Carver c(ws);
  MxWs m = carve_mx(c, L);
  LayerFwdWs lw = carve_layer_fwd(c, L, 0);
  if (d->reuse_plan) {
    if (!plan_recorded(d, lw.attn, offs, ts)) return HSTU_ERR_INVALID_ARG;
    plans_forget(ws, static_cast<char*>(lw.attn) - static_cast<char*>(ws));
  } else {
    plans_forget(ws, ws_bytes);
  }
  const int64_t W = (int64_t)d->H * d->d_v;
  // O: the workspace's (inference) or saved->O (training)
  float* O = saved ? static_cast<float*>(saved->O) : static_cast<float*>(lw.O);
  auto attention = [&](const void* q, const void* k, const void* v, int64_t ld) {
    if (!mx_scores)
      return attn_fwd_impl(d, q, k, ld, v, ld, offs, ts, w->rab_pos, w->rab_time, nc, O, W,
                           /*out_f32=*/true, lw.attn, st);
    // Q|K as MXFP8 (codes [T][2 H d_qk], scale words of the 2H heads Q then
    // K): written by the projection's SiLU epilogue, or, without the SiLU,
    // by one pass over the adjacent Q and K column blocks
    const int64_t hq = (int64_t)d->H * d->d_qk;
    if (!L->proj_silu) {
      if (static_cast<const char*>(k) != static_cast<const char*>(q) + 2 * hq)
        return HSTU_ERR_INVALID_ARG;
      HSTU_TIMED(TT_MX_QUANT, st);
      HSTU_TRY(launch_mx_quant_heads(q, ld, d->T, 2 * d->H, d->d_qk, m.qk8, 2 * hq, m.qks, st));
    }
    hstu_attn_mx_qk qk;
    qk.q_codes = m.qk8;
    qk.k_codes = m.qk8 + hq;
    qk.ld_codes = 2 * hq;
    qk.q_scales = m.qks;
    qk.k_scales = m.qks + d->H * d->T;
    return attn_fwd_impl(d, nullptr, nullptr, 0, v, ld, offs, ts, w->rab_pos, w->rab_time, nc,
                         O, W, /*out_f32=*/true, lw.attn, st, &qk);
  };
  MxPlan plan;
  plan.wm = wm;
  plan.x8 = m.x8;
  plan.xs = m.xs;
  plan.g8 = m.g8;
  plan.gs = m.gs;
  if (io && io->x_codes) {
    plan.x8 = static_cast<uint8_t*>(const_cast<void*>(io->x_codes));
    plan.xs = static_cast<uint8_t*>(const_cast<void*>(io->x_scales));
    plan.x_ready = true;
  }
  if (io && io->g_codes) {
    plan.g8 = static_cast<uint8_t*>(io->g_codes);
    plan.gs = static_cast<uint8_t*>(io->g_scales);
  }
  if (io && io->y_codes) {
    plan.y8 = static_cast<uint8_t*>(io->y_codes);
    plan.ys = static_cast<uint8_t*>(io->y_scales);
  }
  if (mx_scores && L->proj_silu) {
    plan.qk8 = m.qk8;
    plan.qks = m.qks;
    plan.qk_dequant = saved != nullptr;
  }
  if (saved)
    return layer_fwd_steps(L, x, w, y, saved->Z, saved->Zh, O, saved->G, saved->mu,
                           saved->rstd, attention, st, &plan);
  return layer_fwd_steps(L, x, w, y, nullptr, lw.Zh, O, lw.G, nullptr, nullptr, attention, st,
                         &plan);
}

hstu_status hstu_mx_quantize(int64_t rows, int64_t K, const void* x, int64_t ld, void* codes,
                             void* scales, void* stream) {
  if (rows < 0 || K < 0 || K % 32 != 0 || ld < K) return HSTU_ERR_INVALID_ARG;
  if (rows > 0 && K > 0 && (!x || !codes || !scales)) return HSTU_ERR_INVALID_ARG;
  if (rows > 0 && K > 0 && (!aligned16(x) || ld % 8 != 0 || !aligned16(codes)))
    return HSTU_ERR_INVALID_ARG;
  hipStream_t st = entry_stream(stream);
  HSTU_TIMED(TT_MX_QUANT, st);
  HSTU_TRY(launch_mx_quant_rows(x, ld, rows, K, static_cast<uint8_t*>(codes),
                                static_cast<uint8_t*>(scales), st));
  return HSTU_OK;
}

hstu_status hstu_mx_quantize_weight(int64_t K, int64_t N, const void* w, void* codes,
                                    void* scales, void* stream) {
  if (K < 0 || N < 0 || K % 32 != 0) return HSTU_ERR_INVALID_ARG;
  if (K > 0 && N > 0 && (!w || !codes || !scales || !aligned16(codes)))
    return HSTU_ERR_INVALID_ARG;
  hipStream_t st = entry_stream(stream);
  HSTU_TIMED(TT_MX_QUANT, st);
  HSTU_TRY(launch_mx_quant_cols(w, K, N, static_cast<uint8_t*>(codes),
                                static_cast<uint8_t*>(scales), st));
  return HSTU_OK;
}

hstu_status hstu_mx_gemm(int64_t M, int64_t N, int64_t K, const void* a, const void* a_scales,
                         const void* b, const void* b_scales, float* c, int64_t ldc,
                         void* stream) {
  if (M < 0 || N < 0 || K < 0 || K % 128 != 0 || ldc < N) return HSTU_ERR_INVALID_ARG;
  if (M == 0 || N == 0) return HSTU_OK;
  if (!a || !b || !a_scales || !b_scales || !c || !aligned16(a) || !aligned16(b) ||
      !aligned16(c) || ldc % 4 != 0 || (reinterpret_cast<uintptr_t>(a_scales) & 3) ||
      (reinterpret_cast<uintptr_t>(b_scales) & 3))
    return HSTU_ERR_INVALID_ARG;
  if (K == 0) return HSTU_ERR_INVALID_ARG;
  hipStream_t st = entry_stream(stream);
  GemmArgs g;
  g.M = M; g.N = N; g.K = K / 2;
  g.A = a; g.lda = K / 2; g.a_kcont = true;
  g.B = b; g.ldb = K / 2; g.b_kcont = true;
  g.C = c; g.ldc = ldc; g.c_f32 = true;
  g.epi = EPI_STORE;
  g.mx = true;
  g.scale_a = static_cast<const uint8_t*>(a_scales);
  g.scale_b = static_cast<const uint8_t*>(b_scales);
  HSTU_TIMED(TT_GEMM_MX, st);
  HSTU_TRY(launch_gemm(g, HSTU_BF16, st));
  return HSTU_OK;
}

size_t hstu_layer_cached_workspace_size(const hstu_layer_desc* L, int64_t T_hist) {
  if (check_layer(L) != HSTU_OK || T_hist < 0) return 0;
  Carver c(nullptr);
  carve_layer_cached(c, L, T_hist);
  return c.off + 256;
}

hstu_status hstu_layer_fwd_cached(const hstu_layer_desc* L, const void* x,
                                  const hstu_layer_weights* w, const int32_t* coffs,
                                  const int64_t* cts, const hstu_history_kv* hist, void* y,
                                  void* ws, size_t ws_bytes, void* stream) {
  hstu_status s = check_layer(L);
  if (s != HSTU_OK) return s;
  const hstu_attn_desc* d = &L->attn;
  s = check_history(d, hist);
  if (s != HSTU_OK) return s;
  if (!w || !w->W1 || !w->W2 || !w->rab_pos || !w->rab_time || !coffs || !ws)
    return HSTU_ERR_INVALID_ARG;
  if (d->T > 0 && (!x || !y || !cts)) return HSTU_ERR_INVALID_ARG;
  if (x == y && d->T > 0) return HSTU_ERR_INVALID_ARG;
  if (d->dtype == HSTU_BF16 &&
      (!aligned16(x) || !aligned16(y) || !aligned16(w->W1) || !aligned16(w->W2)))
    return HSTU_ERR_INVALID_ARG;
  if (!aligned16(ws)) return HSTU_ERR_INVALID_ARG;
  if (ws_bytes < hstu_layer_cached_workspace_size(L, hist->T)) return HSTU_ERR_WORKSPACE;
  plans_forget(ws, ws_bytes);
  hipStream_t st = entry_stream(stream);

  Carver c(ws);
  LayerFwdWs lw = carve_layer_cached(c, L, hist->T);
  const int64_t W = (int64_t)d->H * d->d_v;
  float* O = static_cast<float*>(lw.O);
  auto attention = [&](const void* q, const void* k, const void* v, int64_t ld) {
    return attn_cached_impl(d, q, k, ld, v, ld, coffs, cts, hist, w->rab_pos, w->rab_time, O, W,
                            /*out_f32=*/true, lw.attn, st);
  };
  return layer_fwd_steps(L, x, w, y, nullptr, lw.Zh, O, lw.G, nullptr, nullptr, attention, st);
}

// MXFP8 operands of the training backward's two activation-gradient
// products: dY and W2 along d_model (dG = dY W2^T), dZ and W1 along F1
// (dX = dZ W1^T); codes [rows][K], scales [rows][K/32]
// MXFP8 operands of the training backward: dY, dZ and the weights along the
// activation products' contractions (d_model, F1), and G^T, dY^T, X^T, dZ^T
// along the tokens for the weight gradients (Tp = T rounded up to 128, the
// extra tokens zero).
struct MxBwdWs {
  uint8_t *dy8 = nullptr, *dys = nullptr, *dz8 = nullptr, *dzs = nullptr;
  uint8_t *w28 = nullptr, *w2s = nullptr, *w18 = nullptr, *w1s = nullptr;
  uint8_t *gt8 = nullptr, *gts = nullptr, *dyt8 = nullptr, *dyts = nullptr;
  uint8_t *xt8 = nullptr, *xts = nullptr, *dzt8 = nullptr, *dzts = nullptr;
  int64_t Tp = 0;
};
MxBwdWs carve_mx_bwd(Carver& c, const hstu_layer_desc* L) {
  const hstu_attn_desc* d = &L->attn;
  const int64_t T = std::max<int64_t>(d->T, 1), D = L->D, W = (int64_t)d->H * d->d_v;
  const int64_t F1 = f1_width(L);
  MxBwdWs m;
  m.dy8 = c.take<uint8_t>(T * D);
  m.dys = c.take<uint8_t>(T * D / 32);
  m.dz8 = c.take<uint8_t>(T * F1);
  m.dzs = c.take<uint8_t>(T * F1 / 32);
  m.w28 = c.take<uint8_t>(W * D);
  m.w2s = c.take<uint8_t>(W * D / 32);
  m.w18 = c.take<uint8_t>(D * F1);
  m.w1s = c.take<uint8_t>(D * F1 / 32);
  m.Tp = (T + 127) / 128 * 128;
  m.gt8 = c.take<uint8_t>(W * m.Tp);
  m.gts = c.take<uint8_t>(W * m.Tp / 32);
  m.dyt8 = c.take<uint8_t>(D * m.Tp);
  m.dyts = c.take<uint8_t>(D * m.Tp / 32);
  m.xt8 = c.take<uint8_t>(D * m.Tp);
  m.xts = c.take<uint8_t>(D * m.Tp / 32);
  m.dzt8 = c.take<uint8_t>(F1 * m.Tp);
  m.dzts = c.take<uint8_t>(F1 * m.Tp / 32);
  return m;
}

hstu_status check_mx_train(const hstu_layer_desc* L) {
  hstu_status s = check_layer(L);
  if (s != HSTU_OK) return s;
  const int64_t W = (int64_t)L->attn.H * L->attn.d_v;
  if (L->attn.dtype != HSTU_BF16 || L->D % 128 != 0 || W % 128 != 0 || f1_width(L) % 128 != 0)
    return HSTU_ERR_UNSUPPORTED;
  return HSTU_OK;
}

// The layer backward; mx: dG, dX, dW2 and dW1 as MXFP8 products (hstu_layer_bwd_mx)
hstu_status layer_bwd_impl(const hstu_layer_desc* L, const void* x, const hstu_layer_weights* w,
                           const int32_t* offs, const int64_t* ts, const int32_t* nc,
                           const hstu_layer_saved* saved, const void* dy, void* dx,
                           const hstu_layer_grads* g, void* ws, size_t ws_bytes, void* stream,
                           bool mx) {
  hstu_status s = mx ? check_mx_train(L) : check_layer(L);
  if (s != HSTU_OK) return s;
  const hstu_attn_desc* d = &L->attn;
  if (d->dtype != HSTU_BF16) return HSTU_ERR_UNSUPPORTED;
  if (!w || !w->W1 || !w->W2 || !w->rab_pos || !w->rab_time || !offs || !ws || !g || !saved)
    return HSTU_ERR_INVALID_ARG;
  if (!saved->Z || !saved->Zh || !saved->O || !saved->G || !saved->mu || !saved->rstd)
    return HSTU_ERR_INVALID_ARG;
  if (!g->dW1 || !g->dW2 || !g->drab_pos || !g->drab_time) return HSTU_ERR_INVALID_ARG;
  if ((w->b1 && !g->db1) || (w->b2 && !g->db2) || (w->ln_gamma && !g->dgamma) ||
      (w->ln_beta && !g->dbeta))
    return HSTU_ERR_INVALID_ARG;
  if (d->T > 0 && (!x || !dy || !dx || !ts)) return HSTU_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(dy) || !aligned16(dx) || !aligned16(w->W1) ||
      !aligned16(w->W2) || !aligned16(saved->Z) || !aligned16(saved->Zh) ||
      !aligned16(saved->O) || !aligned16(saved->G) || !aligned16(ws))
    return HSTU_ERR_INVALID_ARG;
  if (ws_bytes < (mx ? hstu_layer_bwd_mx_workspace_size(L) : hstu_layer_bwd_workspace_size(L)))
    return HSTU_ERR_WORKSPACE;
  plans_forget(ws, ws_bytes);
  hipStream_t st = entry_stream(stream);

  Carver c(ws);
  LayerBwdWs bw = carve_layer_bwd(c, L);
  MxBwdWs mb;
  if (mx) mb = carve_mx_bwd(c, L);
  const int64_t T = d->T, D = L->D, F1 = f1_width(L);
  const int64_t W = (int64_t)d->H * d->d_v, HQ = (int64_t)d->H * d->d_qk;
  const size_t es = esize(d->dtype);
  char* dz = static_cast<char*>(bw.dZ);
  const char* zh = static_cast<const char*>(saved->Zh);
  const void* zpre = L->proj_silu ? saved->Z : nullptr;

  // Side stream (when available): the attention plan and dW2 = G^T dY run
  // there from the start, dW1 once dZ is complete; the caller's stream waits
  // for the plan before the attention kernels and for everything before the
  // call returns.  The column sums (shared scratch) stay on the caller's
  // stream.
  SideStream* sd = side_stream();
  hipStream_t ss = sd ? sd->s : st;
  SideJoin side{sd, st};
  if (sd) {
    HSTU_TRY(order_after(ss, st, sd->ev[0]));
    side.forked = true;
  }
  s = attn_bwd_plan(d, offs, ts, g->drab_pos, g->drab_time, bw.attn, ss);
  if (s != HSTU_OK) return s;
  if (sd) HSTU_TRY(hipEventRecord(sd->ev[1], ss));

  // 1. dG = dY W2^T
  GemmArgs a1;
  a1.M = T; a1.N = W; a1.K = D;
  a1.A = dy; a1.lda = D; a1.a_kcont = true;
  a1.B = w->W2; a1.ldb = D; a1.b_kcont = true;
  a1.C = bw.dG; a1.ldc = W;
  a1.epi = EPI_STORE;
  if (mx) {
    {
      // dY along d_model for dG and along the tokens for dW2, one read
      HSTU_TIMED(TT_MX_QUANT, st);
      HSTU_TRY(launch_mx_quant_both(dy, D, T, D, mb.Tp, mb.dyt8, mb.dyts, mb.dy8, mb.dys, st));
      HSTU_TRY(launch_mx_quant_rows(w->W2, D, W, D, mb.w28, mb.w2s, st));
    }
    if (sd) HSTU_TRY(hipEventRecord(sd->ev[4], st));
    a1.mx = true;
    a1.A = mb.dy8; a1.lda = D / 2; a1.K = D / 2;
    a1.B = mb.w28; a1.ldb = D / 2;
    a1.scale_a = mb.dys; a1.scale_b = mb.w2s;
  }
  { HSTU_TIMED(TT_GEMM_DG, st); HSTU_TRY(launch_gemm(a1, d->dtype, st)); }
  // 2. dW2 = G^T dY (split over T)
  GemmArgs a2;
  a2.M = W; a2.N = D; a2.K = T;
  a2.A = saved->G; a2.lda = W; a2.a_kcont = false;
  a2.B = dy; a2.ldb = D; a2.b_kcont = false;
  a2.epi = EPI_PARTIAL; a2.split_k = bw.s2; a2.partial = bw.part2;
  if (mx) {
    // G^T along the tokens (X^T too: it is ready now); dY^T comes from the
    // caller's stream
    {
      HSTU_TIMED(TT_MX_QUANT, ss);
      HSTU_TRY(launch_mx_quant_rows_t(saved->G, W, T, W, mb.Tp, mb.gt8, mb.gts, ss));
      HSTU_TRY(launch_mx_quant_rows_t(x, D, T, D, mb.Tp, mb.xt8, mb.xts, ss));
    }
    if (sd) HSTU_TRY(hipStreamWaitEvent(ss, sd->ev[4], 0));
    a2.mx = true;
    a2.K = mb.Tp / 2;
    a2.A = mb.gt8; a2.lda = mb.Tp / 2; a2.a_kcont = true;
    a2.B = mb.dyt8; a2.ldb = mb.Tp / 2; a2.b_kcont = true;
    a2.scale_a = mb.gts; a2.scale_b = mb.dyts; a2.scale_kstep_major = true;
  }
  { HSTU_TIMED(TT_GEMM_DW2, ss); HSTU_TRY(launch_gemm(a2, d->dtype, ss)); }
  {
    HSTU_TIMED(TT_REDUCE, ss);
    HSTU_TRY(launch_splitk_reduce(bw.part2, bw.s2, W, D, g->dW2, D, ss));
  }
  if (w->b2) HSTU_TRY(launch_colsum(dy, T, D, D, d->dtype, g->db2, bw.colws, st));
  // 3. LayerNorm + gate backward: dU (into dZ's U block, times SiLU'(Z)), dO
  LnArgs la;
  la.o_f32 = true;
  la.T = T; la.W = (int)W;
  la.O = saved->O; la.ld_o = W;
  la.U = saved->Zh; la.ld_u = F1;
  la.gamma = w->ln_gamma; la.beta = w->ln_beta; la.eps = L->ln_eps;
  la.mu = saved->mu; la.rstd = saved->rstd;
  la.dG = bw.dG; la.ld_dg = W;
  la.dU = dz; la.ld_du = F1;
  la.zu = zpre; la.ld_zu = F1;
  la.dO = bw.dO; la.ld_do = W;
  la.dgamma_part = w->ln_gamma ? bw.lnpg : nullptr;
  la.dbeta_part = w->ln_beta ? bw.lnpb : nullptr;
  la.n_part_blocks = bw.ln_blocks;
  { HSTU_TIMED(TT_LN_BWD, st); HSTU_TRY(launch_ln_gate_bwd(la, d->dtype, st)); }
  if (w->ln_gamma)
    HSTU_TRY(launch_colsum(bw.lnpg, bw.ln_blocks, W, W, HSTU_F32, g->dgamma, bw.colws, st));
  if (w->ln_beta)
    HSTU_TRY(launch_colsum(bw.lnpb, bw.ln_blocks, W, W, HSTU_F32, g->dbeta, bw.colws, st));
  // 4. attention backward into dZ's V, Q, K blocks (times SiLU'(Z))
  if (sd) HSTU_TRY(hipStreamWaitEvent(st, sd->ev[1], 0));
  s = attn_bwd_run(d, zh + 2 * W * es, zh + (2 * W + HQ) * es, F1, zh + W * es, F1, offs, ts,
                    w->rab_pos, w->rab_time, nc, bw.dO, W, dz + 2 * W * es,
                    dz + (2 * W + HQ) * es, dz + W * es, g->drab_pos, g->drab_time, zpre, F1,
                    2 * W, 2 * W + HQ, W, bw.attn, st);
  if (s != HSTU_OK) return s;
  // 5. dW1 = X^T dZ (split over T), db1
  GemmArgs a3;
  a3.M = D; a3.N = F1; a3.K = T;
  a3.A = x; a3.lda = D; a3.a_kcont = false;
  a3.B = dz; a3.ldb = F1; a3.b_kcont = false;
  a3.epi = EPI_PARTIAL; a3.split_k = bw.s1; a3.partial = bw.part1;
  if (mx) {
    // dZ along F1 for dX and along the tokens for dW1, one read
    HSTU_TIMED(TT_MX_QUANT, st);
    HSTU_TRY(launch_mx_quant_both(dz, F1, T, F1, mb.Tp, mb.dzt8, mb.dzts, mb.dz8, mb.dzs, st));
    HSTU_TRY(launch_mx_quant_rows(w->W1, F1, D, F1, mb.w18, mb.w1s, st));
  }
  if (sd) HSTU_TRY(order_after(ss, st, sd->ev[2]));
  if (mx) {
    a3.mx = true;
    a3.K = mb.Tp / 2;
    a3.A = mb.xt8; a3.lda = mb.Tp / 2; a3.a_kcont = true;
    a3.B = mb.dzt8; a3.ldb = mb.Tp / 2; a3.b_kcont = true;
    a3.scale_a = mb.xts; a3.scale_b = mb.dzts; a3.scale_kstep_major = true;
  }
  { HSTU_TIMED(TT_GEMM_DW1, ss); HSTU_TRY(launch_gemm(a3, d->dtype, ss)); }
  {
    HSTU_TIMED(TT_REDUCE, ss);
    HSTU_TRY(launch_splitk_reduce(bw.part1, bw.s1, D, F1, g->dW1, F1, ss));
  }
  if (w->b1) HSTU_TRY(launch_colsum(dz, T, F1, F1, d->dtype, g->db1, bw.colws, st));
  // 6. dX = dZ W1^T (+ dY)
  GemmArgs a4;
  a4.M = T; a4.N = D; a4.K = F1;
  a4.A = dz; a4.lda = F1; a4.a_kcont = true;
  a4.B = w->W1; a4.ldb = F1; a4.b_kcont = true;
  a4.C = dx; a4.ldc = D;
  a4.epi = EPI_RESID;
  a4.R = L->residual ? dy : nullptr; a4.ldr = D;
  if (mx) {
    a4.mx = true;
    a4.A = mb.dz8; a4.lda = F1 / 2; a4.K = F1 / 2;
    a4.B = mb.w18; a4.ldb = F1 / 2;
    a4.scale_a = mb.dzs; a4.scale_b = mb.w1s;
  }
  { HSTU_TIMED(TT_GEMM_DX, st); HSTU_TRY(launch_gemm(a4, d->dtype, st)); }
  HSTU_TRY(side.join());
  return HSTU_OK;
}

hstu_status hstu_layer_bwd(const hstu_layer_desc* L, const void* x, const hstu_layer_weights* w,
                           const int32_t* offs, const int64_t* ts, const int32_t* nc,
                           const hstu_layer_saved* saved, const void* dy, void* dx,
                           const hstu_layer_grads* g, void* ws, size_t ws_bytes, void* stream) {
  return layer_bwd_impl(L, x, w, offs, ts, nc, saved, dy, dx, g, ws, ws_bytes, stream, false);
}

size_t hstu_layer_bwd_mx_workspace_size(const hstu_layer_desc* L) {
  if (check_mx_train(L) != HSTU_OK) return 0;
  Carver c(nullptr);
  carve_layer_bwd(c, L);
  carve_mx_bwd(c, L);
  return c.off + 256;
}

hstu_status hstu_layer_bwd_mx(const hstu_layer_desc* L, const void* x,
                              const hstu_layer_weights* w, const int32_t* offs, const int64_t* ts,
                              const int32_t* nc, const hstu_layer_saved* saved, const void* dy,
                              void* dx, const hstu_layer_grads* g, void* ws, size_t ws_bytes,
                              void* stream) {
  return layer_bwd_impl(L, x, w, offs, ts, nc, saved, dy, dx, g, ws, ws_bytes, stream, true);
}

size_t hstu_schedule_workspace_size(int32_t B, int64_t T, int32_t block_rows) {
  if (B < 0 || T < 0 || block_rows < 1) return 0;
  Carver c(nullptr);
  carve_sched(c, T, B, block_rows);
  return c.off + 256;
}

int64_t hstu_schedule_capacity(int64_t T, int32_t B, int32_t block_rows) {
  if (B < 0 || T < 0 || block_rows < 1) return 0;
  return sched_capacity(T, B, block_rows);
}

hstu_status hstu_schedule(int32_t B, int64_t T, const int32_t* offs, int32_t block_rows,
                          int32_t reverse, int32_t* items, int32_t* n_items, void* ws,
                          size_t ws_bytes, void* stream) {
  if (B < 0 || T < 0 || T >= (int64_t(1) << 31) || block_rows < 1 || !offs || !items ||
      !n_items || !ws)
    return HSTU_ERR_INVALID_ARG;
  if (ws_bytes < hstu_schedule_workspace_size(B, T, block_rows)) return HSTU_ERR_WORKSPACE;
  plans_forget(ws, ws_bytes);
  hipStream_t st = entry_stream(stream);
  Carver c(ws);
  Sched sc = carve_sched(c, T, B, block_rows);
  HSTU_TRY(launch_sched(sc, B, offs, reverse, st));
  HSTU_TRY(hipMemcpyAsync(items, sc.items, sizeof(int32_t) * 2 * sc.cap,
                          hipMemcpyDeviceToDevice, st));
  HSTU_TRY(hipMemcpyAsync(n_items, sc.counters, sizeof(int32_t), hipMemcpyDeviceToDevice, st));
  return HSTU_OK;
}

hstu_status hstu_bias_buckets(const hstu_attn_desc* d, const int32_t* offs, const int64_t* ts,
                              const int32_t* nc, const int32_t* ps, const int32_t* pi,
                              const int32_t* pj, int64_t n_pairs, int32_t* bp, int32_t* bt,
                              void* ws, size_t ws_bytes, void* stream) {
  hstu_status s = check_attn_desc(d);
  if (s != HSTU_OK) return s;
  if (!offs || !ws || n_pairs < 0) return HSTU_ERR_INVALID_ARG;
  if (n_pairs > 0 && (!ts || !ps || !pi || !pj || !bp || !bt)) return HSTU_ERR_INVALID_ARG;
  if (ws_bytes < hstu_attn_fwd_workspace_size(d)) return HSTU_ERR_WORKSPACE;
  plans_forget(ws, ws_bytes);
  hipStream_t st = entry_stream(stream);
  Carver c(ws);
  FwdWs w = carve_fwd(c, d);
  AttnArgs a = base_args(d, nullptr, nullptr, 0, nullptr, 0, offs, ts, nullptr, nullptr, nc, w.tm);
  HSTU_TRY(launch_time_prepass(w.tm, d->B, offs, ts, st));
  HSTU_TRY(launch_bias_buckets(a, ps, pi, pj, n_pairs, bp, bt, st));
  return HSTU_OK;
}

hstu_status hstu_truncate_offsets(int32_t B, const int32_t* offs, const int32_t* nc,
                                  int32_t keep, int32_t* seg, void* stream) {
  if (B < 0 || keep < 0 || !offs || !seg) return HSTU_ERR_INVALID_ARG;
  hipStream_t st = entry_stream(stream);
  { HSTU_TIMED(TT_TRUNCATE, st); HSTU_TRY(launch_trunc_offsets(B, offs, nc, keep, seg, st)); }
  return HSTU_OK;
}


hstu_status hstu_truncate_gather(int32_t B, int64_t T, int64_t T_seg, int32_t D, int32_t dtype,
                                 const void* x, const int32_t* offs, const int32_t* seg,
                                 const int64_t* ts, void* x_seg, int64_t* ts_seg,
                                 void* stream) {
  hstu_status s = check_trunc_copy(B, T, T_seg, D, dtype, x, x_seg, offs, seg);
  if (s != HSTU_OK) return s;
  if (T_seg > 0 && (ts == nullptr) != (ts_seg == nullptr)) return HSTU_ERR_INVALID_ARG;
  hipStream_t st = entry_stream(stream);
  HSTU_TIMED(TT_TRUNCATE, st);
  HSTU_TRY(launch_trunc_gather(B, T, T_seg, int64_t(D) * esize(dtype), offs, seg, x, x_seg, ts,
                               ts_seg, st));
  return HSTU_OK;
}

hstu_status hstu_truncate_scatter(int32_t B, int64_t T, int64_t T_seg, int32_t D, int32_t dtype,
                                  const void* dx_seg, const int32_t* offs, const int32_t* seg,
                                  void* dx, void* stream) {
  hstu_status s = check_trunc_copy(B, T, T_seg, D, dtype, dx, dx_seg, offs, seg);
  if (s != HSTU_OK) return s;
  hipStream_t st = entry_stream(stream);
  HSTU_TIMED(TT_TRUNCATE, st);
  HSTU_TRY(launch_trunc_scatter(B, T, T_seg, int64_t(D) * esize(dtype), offs, seg, dx_seg, dx,
                                st));
  return HSTU_OK;
}

hstu_status hstu_validate_inputs(int32_t B, int64_t T, const int32_t* offs, const int32_t* nc,
                                 int32_t* flag_ws, void* stream) {
  if (B < 0 || T < 0 || !offs || !flag_ws) return HSTU_ERR_INVALID_ARG;
  hipStream_t st = entry_stream(stream);
  HSTU_TRY(launch_zero_i32(flag_ws, 1, st));
  HSTU_TRY(launch_validate(B, offs, nc, T, flag_ws, st));
  int32_t h = 0;
  HSTU_TRY(hipMemcpyAsync(&h, flag_ws, sizeof(int32_t), hipMemcpyDeviceToHost, st));
  HSTU_TRY(hipStreamSynchronize(st));
  return h ? HSTU_ERR_VALIDATION : HSTU_OK;
}

}  // extern "C"
