// Diagnostic per-kernel timing: HIP event pairs recorded around each launch
// site while enabled (hstu_timer_enable), summed per kernel tag on query.
#pragma once

#include <hip/hip_runtime.h>

namespace hstu {

enum TimerTag {
  TT_PREPASS = 0,
  TT_SCHED,
  TT_ATTN_FWD,
  TT_ATTN_BWD_DKDV,
  TT_ATTN_BWD_DQ,
  TT_GEMM_UVQK,
  TT_GEMM_OUT,
  TT_GEMM_DG,
  TT_GEMM_DW2,
  TT_GEMM_DW1,
  TT_GEMM_DX,
  TT_LN_FWD,
  TT_LN_BWD,
  TT_REDUCE,
  TT_TRUNCATE,
  TT_ATTN_CACHED,
  TT_MX_QUANT,
  TT_GEMM_MX,
  TT_COUNT
};

const char* timer_tag_name(int tag);
// Returns the index of an event pair to close with timer_stop, or -1 when
// timing is off or the pool is exhausted.
int timer_start(int tag, hipStream_t st);
void timer_stop(int slot, hipStream_t st);

struct TimedScope {
  int slot;
  hipStream_t st;
  TimedScope(int tag, hipStream_t s) : slot(timer_start(tag, s)), st(s) {}
  ~TimedScope() { timer_stop(slot, st); }
};

}  // namespace hstu

// two-level paste so that __LINE__ expands: one distinct scope object per line
#define HSTU_CAT_(a, b) a##b
#define HSTU_CAT(a, b) HSTU_CAT_(a, b)
#define HSTU_TIMED(tag, st) ::hstu::TimedScope HSTU_CAT(hstu_timed_scope_, __LINE__)((tag), (st))
