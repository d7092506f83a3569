// Jagged-tile scheduler, timestamp pre-pass and small utility kernels.
//
// Work items are (sequence, row block) pairs.  A row block m of a causal
// sequence touches m+1 key blocks ("DLRMv4 Brings Sequence-Based
// Recommendation Training to MLPerf", Table 7 note: only the lower triangle
// is evaluated), so items are listed by decreasing m (longest first), which
// is a longest-processing-time order for the hardware's in-order dispatch.
// The list is built on the device (counting sort by block count), so no host
// synchronisation is needed; the launch grid uses the capacity bound
// sum_b ceil(n_b / BM) <= (T + B*(BM-1)) / BM and surplus workgroups exit.
#include "bias.h"
#include "common.h"
#include "internal.h"

namespace hstu {

__global__ void k_zero_i32(int32_t* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}
__global__ void k_zero_f32(float* p, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.0f;
}

static int grid_for(int64_t n, int per = 256) {
  int64_t g = (n + per - 1) / per;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (int)g;
}

hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  k_zero_i32<<<grid_for(n), 256, 0, st>>>(p, n);
  return hipGetLastError();
}
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  k_zero_f32<<<grid_for(n), 256, 0, st>>>(p, n);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Timestamp pre-pass: one workgroup per sequence.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_time_prepass(const int32_t* __restrict__ offs,
                                                      const int64_t* __restrict__ ts,
                                                      int32_t* __restrict__ rel_t,
                                                      int32_t* __restrict__ flags) {
  __shared__ int64_t smin[4], smax[4];
  __shared__ int sunsorted[4];
  const int b = blockIdx.x;
  const int64_t o0 = offs[b], o1 = offs[b + 1];
  int64_t mn = INT64_MAX, mx = INT64_MIN;
  int unsorted = 0;
  for (int64_t r = o0 + threadIdx.x; r < o1; r += 256) {
    int64_t t = ts[r];
    mn = t < mn ? t : mn;
    mx = t > mx ? t : mx;
    if (r > o0 && t < ts[r - 1]) unsorted = 1;
  }
  for (int o = 32; o > 0; o >>= 1) {
    int64_t a = __shfl_xor(mn, o, 64), c = __shfl_xor(mx, o, 64);
    mn = a < mn ? a : mn;
    mx = c > mx ? c : mx;
    unsorted |= __shfl_xor(unsorted, o, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    smin[w] = mn;
    smax[w] = mx;
    sunsorted[w] = unsorted;
  }
  __syncthreads();
  mn = smin[0];
  mx = smax[0];
  unsorted = sunsorted[0];
  for (int i = 1; i < 4; ++i) {
    mn = smin[i] < mn ? smin[i] : mn;
    mx = smax[i] > mx ? smax[i] : mx;
    unsorted |= sunsorted[i];
  }
  const bool wide = (o1 > o0) && (mx - mn > HSTU_NARROW_SPAN_MAX);
  for (int64_t r = o0 + threadIdx.x; r < o1; r += 256)
    rel_t[r] = wide ? 0 : (int32_t)(ts[r] - mn);
  if (threadIdx.x == 0) flags[b] = (wide ? 1 : 0) | (unsorted ? 0 : 2);
}

TimeMeta carve_time(Carver& c, int64_t T, int64_t B) {
  TimeMeta m;
  m.rel_t = c.take<int32_t>(T > 0 ? T : 1);
  m.seq_flags = c.take<int32_t>(B > 0 ? B : 1);
  return m;
}

hipError_t launch_time_prepass(const TimeMeta& tm, int B, const int32_t* offs,
                               const int64_t* ts, hipStream_t st) {
  if (B <= 0) return hipSuccess;
  k_time_prepass<<<B, 256, 0, st>>>(offs, ts, tm.rel_t, tm.seq_flags);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Work list.
// ---------------------------------------------------------------------------
__global__ void k_sched_count(int B, const int32_t* __restrict__ offs, int bm,
                              int32_t* __restrict__ hist, int32_t* __restrict__ counters) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int n = offs[b + 1] - offs[b];
  int nb = (n + bm - 1) / bm;
  atomicAdd(&hist[nb], 1);
  atomicMax(&counters[1], nb);
}

// Exclusive suffix sum of in[0..len) into out[0..len) by one workgroup of 1024.
__device__ void block_suffix_excl(const int32_t* in, int32_t* out, int len, int32_t* total) {
  __shared__ int32_t part[1024];
  const int t = threadIdx.x;
  const int chunk = (len + 1023) / 1024;
  const int lo = t * chunk, hi = min(len, lo + chunk);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += in[i];
  part[t] = s;
  __syncthreads();
  // inclusive suffix scan of part[] (Hillis-Steele)
  for (int o = 1; o < 1024; o <<= 1) {
    int v = (t + o < 1024) ? part[t + o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int acc = (t + 1 < 1024) ? part[t + 1] : 0;  // sum of later chunks
  for (int i = hi - 1; i >= lo; --i) {
    int v = in[i];
    out[i] = acc;
    acc += v;
  }
  if (t == 0 && total) *total = part[0];
  __syncthreads();
}

__global__ __launch_bounds__(1024) void k_sched_levels(int32_t* __restrict__ hist,
                                                       int32_t* __restrict__ cnt,
                                                       int32_t* __restrict__ levelstart,
                                                       int32_t* __restrict__ counters) {
  const int maxblk = counters[1];
  // cnt[m] = #sequences with more than m blocks, m in [0, maxblk]
  block_suffix_excl(hist, cnt, maxblk + 1, nullptr);
  __syncthreads();
  // levelstart[L] = sum of cnt[L'] for L' in (L, maxblk); n_items = sum over [0, maxblk)
  block_suffix_excl(cnt, levelstart, maxblk, &counters[0]);
  if (threadIdx.x == 0 && maxblk == 0) counters[0] = 0;
}

__global__ __launch_bounds__(256) void k_sched_items(const int32_t* __restrict__ offs, int bm,
                                                     int reverse,
                                                     const int32_t* __restrict__ cnt,
                                                     const int32_t* __restrict__ levelstart,
                                                     int32_t* __restrict__ tie,
                                                     int32_t* __restrict__ items) {
  __shared__ int spos;
  const int b = blockIdx.x;
  const int n = offs[b + 1] - offs[b];
  const int nb = (n + bm - 1) / bm;
  if (nb == 0) return;
  if (threadIdx.x == 0) spos = cnt[nb] + atomicAdd(&tie[nb], 1);
  __syncthreads();
  const int pos = spos;
  for (int m = threadIdx.x; m < nb; m += 256) {
    const int L = reverse ? (nb - 1 - m) : m;
    const int64_t w = (int64_t)levelstart[L] + pos;
    items[2 * w] = b;
    items[2 * w + 1] = m;
  }
}

Sched carve_sched(Carver& c, int64_t T, int64_t B, int block_rows) {
  Sched s;
  s.cap = sched_capacity(T, B, block_rows);
  s.block_rows = block_rows;
  s.items = c.take<int32_t>(2 * s.cap);
  s.counters = c.take<int32_t>(4);
  s.hist = c.take<int32_t>(s.cap + 2);
  s.cnt = c.take<int32_t>(s.cap + 2);
  s.levelstart = c.take<int32_t>(s.cap + 2);
  s.tie = c.take<int32_t>(s.cap + 2);
  return s;
}

hipError_t launch_sched(const Sched& s, int B, const int32_t* offs, int reverse, hipStream_t st) {
  hipError_t e;
  if ((e = launch_zero_i32(s.counters, 4, st)) != hipSuccess) return e;
  if ((e = launch_zero_i32(s.hist, s.cap + 2, st)) != hipSuccess) return e;
  if ((e = launch_zero_i32(s.tie, s.cap + 2, st)) != hipSuccess) return e;
  if (B <= 0) return hipSuccess;
  k_sched_count<<<(B + 255) / 256, 256, 0, st>>>(B, offs, s.block_rows, s.hist, s.counters);
  k_sched_levels<<<1, 1024, 0, st>>>(s.hist, s.cnt, s.levelstart, s.counters);
  k_sched_items<<<B, 256, 0, st>>>(offs, s.block_rows, reverse, s.cnt, s.levelstart, s.tie,
                                   s.items);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bucket inspection kernel (same device arithmetic as the attention kernels).
// ---------------------------------------------------------------------------
__global__ void k_bias_buckets(AttnArgs a, const int32_t* __restrict__ ps,
                               const int32_t* __restrict__ pi, const int32_t* __restrict__ pj,
                               int64_t n, int32_t* __restrict__ bp, int32_t* __restrict__ bt) {
  int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (p >= n) return;
  const int b = ps[p], i = pi[p], j = pj[p];
  const int o0 = a.seq_offsets[b];
  const int nn = a.seq_offsets[b + 1] - o0;
  const int c = a.num_cand ? a.num_cand[b] : 0;
  const int nh = nn - c;
  const int pI = min(i, nh), pJ = min(j, nh);
  bp[p] = pbucket(pI, pJ, a.nP);
  int cl;
  if (a.seq_flags[b] & 1)
    cl = tclz_wide(a.ts[o0 + i], a.ts[o0 + j]);
  else
    cl = tclz_narrow(a.rel_t[o0 + i] + 1, a.rel_t[o0 + j]);
  bt[p] = tbucket_from_clz(cl, a.nT);
}

hipError_t launch_bias_buckets(const AttnArgs& a, const int32_t* ps, const int32_t* pi,
                               const int32_t* pj, int64_t n, int32_t* bp, int32_t* bt,
                               hipStream_t st) {
  if (n <= 0) return hipSuccess;
  k_bias_buckets<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(a, ps, pi, pj, n, bp, bt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Device-contract validation.
// ---------------------------------------------------------------------------
__global__ void k_validate(int B, const int32_t* __restrict__ offs,
                           const int32_t* __restrict__ nc, int64_t T, int32_t* flag) {
  int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b > B) return;
  int bad = 0;
  if (b == 0 && offs[0] != 0) bad = 1;
  if (b == B && (int64_t)offs[B] != T) bad = 1;
  if (b < B) {
    int n = offs[b + 1] - offs[b];
    if (n < 0) bad = 1;
    if (nc && (nc[b] < 0 || nc[b] > n)) bad = 1;
  }
  if (bad) atomicOr(flag, 1);
}

hipError_t launch_validate(int B, const int32_t* offs, const int32_t* nc, int64_t T,
                           int32_t* flag, hipStream_t st) {
  k_validate<<<(B + 1 + 255) / 256, 256, 0, st>>>(B, offs, nc, T, flag);
  return hipGetLastError();
}

}  // namespace hstu
