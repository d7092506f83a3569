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
// Timestamp pre-pass: one workgroup per sequence (or per user of a cached
// history: its history and candidate times together).  Relative times
// t - min fit in int32 unless the span is "wide"; bit 1 of the flags says
// the (history) times are non-decreasing.
// ---------------------------------------------------------------------------
__device__ void minmax_reduce(int64_t& mn, int64_t& mx, int& unsorted) {
  __shared__ int64_t smin[16], smax[16];
  __shared__ int sunsorted[16];
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t a = __shfl_xor(mn, o, 64), c = __shfl_xor(mx, o, 64);
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
  for (int i = 1; i < 16; ++i) {
    mn = smin[i] < mn ? smin[i] : mn;
    mx = smax[i] > mx ? smax[i] : mx;
    unsorted |= sunsorted[i];
  }
}

__device__ void prepass_seq(int b, const PlanArgs& p) {
  const int64_t o0 = p.offs[b], o1 = p.offs[b + 1];
  int64_t mn = INT64_MAX, mx = INT64_MIN;
  int unsorted = 0;
  // 1024 threads, four strided loads in flight per thread: a few memory round
  // trips per sequence rather than one per 256 tokens
#pragma unroll 4
  for (int64_t r = o0 + threadIdx.x; r < o1; r += 1024) {
    const int64_t t = p.ts[r];
    mn = t < mn ? t : mn;
    mx = t > mx ? t : mx;
    if (r > o0 && t < p.ts[r - 1]) unsorted = 1;
  }
  minmax_reduce(mn, mx, unsorted);
  const bool wide = (o1 > o0) && (mx - mn > HSTU_NARROW_SPAN_MAX);
#pragma unroll 4
  for (int64_t r = o0 + threadIdx.x; r < o1; r += 1024)
    p.rel_t[r] = wide ? 0 : (int32_t)(p.ts[r] - mn);
  if (threadIdx.x == 0) p.flags[b] = (wide ? 1 : 0) | (unsorted ? 0 : 2);
}

__device__ void prepass_user(int b, const PlanArgs& p) {
  const int64_t h0 = p.offs[b], h1 = p.offs[b + 1], c0 = p.coffs[b], c1 = p.coffs[b + 1];
  int64_t mn = INT64_MAX, mx = INT64_MIN;
  int unsorted = 0;
#pragma unroll 4
  for (int64_t r = h0 + threadIdx.x; r < h1; r += 1024) {
    const int64_t t = p.ts[r];
    mn = t < mn ? t : mn;
    mx = t > mx ? t : mx;
    if (r > h0 && t < p.ts[r - 1]) unsorted = 1;
  }
  for (int64_t r = c0 + threadIdx.x; r < c1; r += 1024) {
    const int64_t t = p.cts[r];
    mn = t < mn ? t : mn;
    mx = t > mx ? t : mx;
  }
  minmax_reduce(mn, mx, unsorted);
  const bool wide = (h1 > h0 || c1 > c0) && (mx - mn > HSTU_NARROW_SPAN_MAX);
#pragma unroll 4
  for (int64_t r = h0 + threadIdx.x; r < h1; r += 1024)
    p.rel_t[r] = wide ? 0 : (int32_t)(p.ts[r] - mn);
  for (int64_t r = c0 + threadIdx.x; r < c1; r += 1024)
    p.rel_c[r] = wide ? 0 : (int32_t)(p.cts[r] - mn);
  if (threadIdx.x == 0) p.flags[b] = (wide ? 1 : 0) | (unsorted ? 0 : 2);
}

TimeMeta carve_time(Carver& c, int64_t T, int64_t B) {
  TimeMeta m;
  m.rel_t = c.take<int32_t>(T > 0 ? T : 1);
  m.seq_flags = c.take<int32_t>(B > 0 ? B : 1);
  return m;
}

// ---------------------------------------------------------------------------
// Work list.
// ---------------------------------------------------------------------------
// Exclusive suffix sum of in[0..len) into out[0..len) by one workgroup of
// 1024: contiguous chunks per thread, suffix scans inside each wave by
// shuffles, wave totals through LDS (two barriers).
__device__ void block_suffix_excl(const int32_t* in, int32_t* out, int len, int32_t* total) {
  __shared__ int32_t wsum[16];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int chunk = (len + 1023) / 1024;
  const int lo = min(t * chunk, len), hi = min(len, lo + chunk);
  int s = 0;
  for (int i = lo; i < hi; ++i) s += in[i];
  int x = s;  // inclusive suffix sum over the lanes >= this one
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_down(x, o, 64);
    if (lane + o < 64) x += y;
  }
  if (lane == 0) wsum[w] = x;
  __syncthreads();
  int later = 0;  // totals of the later waves
  for (int v = w + 1; v < 16; ++v) later += wsum[v];
  int acc = x - s + later;  // sum over the later threads' chunks
  for (int i = hi - 1; i >= lo; --i) {
    const int v = in[i];
    out[i] = acc;
    acc += v;
  }
  if (t == 0 && total) *total = x + later;
  __syncthreads();
}

// The steps communicate through memory inside the workgroup (LDS, or global
// memory for long lists), so each is separated by a barrier and an
// agent-scope acquire (the vector L1 then holds no stale line).
__device__ void sched_step_barrier() {
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// One workgroup builds one schedule: clear, count sequences per block count,
// the two suffix sums, then the items.  `lds` (4 (cap + 2) ints) replaces
// the job's global scratch arrays when given.
__device__ void build_schedule(int B, const int32_t* __restrict__ offs, const SchedJob& jg,
                               int32_t* lds) {
  SchedJob j = jg;
  if (lds) {
    const int E = j.cap + 2;
    j.hist = lds;
    j.cnt = lds + E;
    j.levelstart = lds + 2 * E;
    j.tie = lds + 3 * E;
  }
  __shared__ int32_t s_maxblk, s_items;
  const int t = threadIdx.x;
  for (int i = t; i < j.cap + 2; i += 1024) {
    j.hist[i] = 0;
    j.tie[i] = 0;
  }
  if (t == 0) s_maxblk = 0;
  sched_step_barrier();
  for (int b = t; b < B; b += 1024) {
    const int n = offs[b + 1] - offs[b];
    const int nb = (n + j.bm - 1) / j.bm;
    atomicAdd(&j.hist[nb], 1);
    atomicMax(&s_maxblk, nb);
  }
  sched_step_barrier();
  const int maxblk = s_maxblk;
  // cnt[m] = #sequences with more than m blocks, m in [0, maxblk]
  block_suffix_excl(j.hist, j.cnt, maxblk + 1, nullptr);
  sched_step_barrier();
  // levelstart[L] = sum of cnt[L'] for L' in (L, maxblk); n_items = sum over [0, maxblk)
  block_suffix_excl(j.cnt, j.levelstart, maxblk, &s_items);
  sched_step_barrier();
  if (t == 0) {
    j.counters[0] = maxblk == 0 ? 0 : s_items;
    j.counters[1] = maxblk;
  }
  for (int b = t; b < B; b += 1024) {
    const int n = offs[b + 1] - offs[b];
    const int nb = (n + j.bm - 1) / j.bm;
    if (nb == 0) continue;
    const int pos = j.cnt[nb] + atomicAdd(&j.tie[nb], 1);
    for (int m = 0; m < nb; ++m) {
      const int L = j.reverse ? (nb - 1 - m) : m;
      const int64_t w = (int64_t)j.levelstart[L] + pos;
      j.items[2 * w] = b;
      j.items[2 * w + 1] = m;
    }
  }
}

// First kept-dS block of every sequence (exclusive prefix sums of
// H nrb (nrb + 1) / 2) and the flag that says whether they fit ds_cap.  The
// total is summed in 64 bits, so the int32 bases are used only when it fits.
__device__ void ds_offsets(const PlanArgs& p) {
  __shared__ int64_t wtot[16];
  const int t = threadIdx.x;
  int64_t mine = 0;
  for (int b = t; b < p.B; b += 1024) {
    const int64_t nrb = (p.offs[b + 1] - p.offs[b] + 127) / 128;
    const int64_t cnt = (int64_t)p.H * nrb * (nrb + 1) / 2;
    mine += cnt;
    p.ds_base[b] = (int32_t)min<int64_t>(cnt, INT32_MAX / 2);
  }
  for (int o = 32; o > 0; o >>= 1) mine += __shfl_xor(mine, o, 64);
  if ((t & 63) == 0) wtot[t >> 6] = mine;
  sched_step_barrier();
  int64_t total = 0;
  for (int i = 0; i < 16; ++i) total += wtot[i];
  const bool fits = total <= p.ds_cap;
  if (t == 0) *p.ds_flag = fits ? 0 : 1;
  if (!fits) return;
  int32_t tot32 = 0;
  block_suffix_excl(p.ds_base, p.ds_base, p.B, &tot32);   // in place: later sequences' blocks
  sched_step_barrier();
  for (int b = t; b < p.B; b += 1024) {
    const int64_t nrb = (p.offs[b + 1] - p.offs[b] + 127) / 128;
    const int32_t cnt = (int32_t)((int64_t)p.H * nrb * (nrb + 1) / 2);
    p.ds_base[b] = (int32_t)total - p.ds_base[b] - cnt;
  }
}

// One launch for a call's plan: workgroups [0, npre) run the time pre-pass
// (and clear the backward's rab-gradient sums on the way), the next njobs
// build the work lists.
__global__ __launch_bounds__(1024) void k_plan(PlanArgs p) {
  extern __shared__ int32_t plan_lds[];
  const int wg = blockIdx.x;
  if (wg < p.npre) {
    for (int64_t i = (int64_t)wg * 1024 + threadIdx.x; i < p.nz; i += (int64_t)p.npre * 1024) {
      p.z0[i] = 0.0f;
      p.z1[i] = 0.0f;
    }
    if (p.mode == 0) prepass_seq(wg, p);
    else prepass_user(wg, p);
    return;
  }
  const int job = wg - p.npre;
  if (job == p.njobs) {
    ds_offsets(p);
    return;
  }
  build_schedule(p.B, p.sched_offs, p.job[job], p.lds_sched ? plan_lds : nullptr);
}

SchedJob sched_job(const Sched& s, int reverse) {
  SchedJob j;
  j.items = s.items;
  j.counters = s.counters;
  j.hist = s.hist;
  j.cnt = s.cnt;
  j.levelstart = s.levelstart;
  j.tie = s.tie;
  j.cap = (int)s.cap;
  j.bm = s.block_rows;
  j.reverse = reverse;
  return j;
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

// schedule arrays up to this many entries each live in LDS (4 x 12 KiB)
constexpr int SCHED_LDS_ENTRIES = 3072;

hipError_t launch_plan(PlanArgs p, hipStream_t st) {
  int max_e = 0;
  for (int k = 0; k < p.njobs; ++k) max_e = max(max_e, p.job[k].cap + 2);
  p.lds_sched = (p.njobs > 0 && max_e <= SCHED_LDS_ENTRIES) ? 1 : 0;
  if (p.npre == 0 && p.nz > 0) {
    hipError_t e = launch_zero_f32(p.z0, p.nz, st);
    if (e == hipSuccess) e = launch_zero_f32(p.z1, p.nz, st);
    if (e != hipSuccess) return e;
    p.nz = 0;
  }
  const int grid = p.npre + p.njobs + (p.ds_base ? 1 : 0);
  if (grid <= 0) return hipSuccess;
  const size_t lds = p.lds_sched ? (size_t)4 * max_e * sizeof(int32_t) : 0;
  k_plan<<<grid, 1024, lds, st>>>(p);
  return hipGetLastError();
}

PlanArgs plan_prepass(const TimeMeta& tm, int B, const int32_t* offs, const int64_t* ts,
                      float* z0, float* z1, int64_t nz) {
  PlanArgs p;
  p.npre = B > 0 ? B : 0;
  p.mode = 0;
  p.offs = offs;
  p.ts = ts;
  p.rel_t = tm.rel_t;
  p.flags = tm.seq_flags;
  p.z0 = z0;
  p.z1 = z1;
  p.nz = (z0 && z1) ? nz : 0;
  p.B = B;
  return p;
}

void plan_add_job(PlanArgs& p, const Sched& s, int reverse, const int32_t* sched_offs) {
  p.sched_offs = sched_offs;
  p.job[p.njobs++] = sched_job(s, reverse);
}

hipError_t launch_time_prepass(const TimeMeta& tm, int B, const int32_t* offs,
                               const int64_t* ts, hipStream_t st, float* z0, float* z1,
                               int64_t nz) {
  return launch_plan(plan_prepass(tm, B, offs, ts, z0, z1, nz), st);
}

hipError_t launch_sched(const Sched& s, int B, const int32_t* offs, int reverse, hipStream_t st) {
  PlanArgs p;
  p.B = B;
  plan_add_job(p, s, reverse, offs);
  return launch_plan(p, st);
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
