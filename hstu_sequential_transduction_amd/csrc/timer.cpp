// Diagnostic per-kernel timer (see timer.h).  Not thread-safe: meant for one
// benchmarking thread.  Events come from a pool created by hstu_timer_enable.
#include "timer.h"

#include <vector>

#include "internal.h"

namespace hstu {

namespace {

struct Pool {
  std::vector<hipEvent_t> start, stop;
  std::vector<int> tag;
  int used = 0;
  bool on = false;
};
Pool g_pool;

const char* kNames[TT_COUNT] = {
    "plan", "sched", "attn_fwd", "attn_bwd_dkdv", "attn_bwd_dq", "gemm_uvqk", "gemm_out",
    "gemm_dG", "gemm_dW2", "gemm_dW1", "gemm_dX", "ln_gate_fwd", "ln_gate_bwd", "reduce",
    "truncate", "attn_cached", "mx_quant", "gemm_mx"};

void destroy() {
  for (auto e : g_pool.start) (void)hipEventDestroy(e);
  for (auto e : g_pool.stop) (void)hipEventDestroy(e);
  g_pool.start.clear();
  g_pool.stop.clear();
  g_pool.tag.clear();
  g_pool.used = 0;
  g_pool.on = false;
}

}  // namespace

const char* timer_tag_name(int tag) { return (tag >= 0 && tag < TT_COUNT) ? kNames[tag] : ""; }

int timer_start(int tag, hipStream_t st) {
  if (!g_pool.on || g_pool.used >= (int)g_pool.start.size()) return -1;
  const int s = g_pool.used++;
  g_pool.tag[s] = tag;
  if (hipEventRecord(g_pool.start[s], st) != hipSuccess) return -1;
  return s;
}

void timer_stop(int slot, hipStream_t st) {
  if (slot < 0) return;
  (void)hipEventRecord(g_pool.stop[slot], st);
}

}  // namespace hstu

using namespace hstu;

extern "C" {

hstu_status hstu_timer_enable(int32_t max_launches) {
  destroy();
  if (max_launches <= 0) return HSTU_OK;
  g_pool.start.resize(max_launches);
  g_pool.stop.resize(max_launches);
  g_pool.tag.assign(max_launches, -1);
  for (int i = 0; i < max_launches; ++i) {
    if (hipEventCreate(&g_pool.start[i]) != hipSuccess ||
        hipEventCreate(&g_pool.stop[i]) != hipSuccess) {
      g_pool.start.resize(i);
      g_pool.stop.resize(i);
      destroy();
      return HSTU_ERR_HIP;
    }
  }
  g_pool.on = true;
  return HSTU_OK;
}

hstu_status hstu_timer_reset(void) {
  g_pool.used = 0;
  return HSTU_OK;
}

int32_t hstu_timer_tag_count(void) { return TT_COUNT; }

const char* hstu_timer_tag_name(int32_t tag) { return timer_tag_name(tag); }

hstu_status hstu_timer_query(int32_t tag, int64_t* launches, double* total_ms) {
  if (!launches || !total_ms || tag < 0 || tag >= TT_COUNT) return HSTU_ERR_INVALID_ARG;
  int64_t n = 0;
  double tot = 0.0;
  for (int s = 0; s < g_pool.used; ++s) {
    if (g_pool.tag[s] != tag) continue;
    if (hipEventSynchronize(g_pool.stop[s]) != hipSuccess) return HSTU_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, g_pool.start[s], g_pool.stop[s]) != hipSuccess)
      return HSTU_ERR_HIP;
    tot += ms;
    ++n;
  }
  *launches = n;
  *total_ms = tot;
  return HSTU_OK;
}

}  // extern "C"
