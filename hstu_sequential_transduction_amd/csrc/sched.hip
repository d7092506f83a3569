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
__global__ __launch_bounds__(1024) void k_time_prepass(const int32_t* __restrict__ offs,
                                                       const int64_t* __restrict__ ts,
                                                       int32_t* __restrict__ rel_t,
                                                       int32_t* __restrict__ flags,
                                                       float* __restrict__ z0,
                                                       float* __restrict__ z1, int64_t nz) {
  __shared__ int64_t smin[16], smax[16];
  __shared__ int sunsorted[16];
  const int b = blockIdx.x;
  // the backward's rab-gradient accumulators, cleared by the grid on the way
  for (int64_t i = (int64_t)b * 1024 + threadIdx.x; i < nz; i += (int64_t)gridDim.x * 1024) {
    z0[i] = 0.0f;
    z1[i] = 0.0f;
  }
  const int64_t o0 = offs[b], o1 = offs[b + 1];
  int64_t mn = INT64_MAX, mx = INT64_MIN;
  int unsorted = 0;
  // 1024 threads, four strided loads in flight per thread: a few memory round
  // trips per sequence rather than one per 256 tokens
#pragma unroll 4
  for (int64_t r = o0 + threadIdx.x; r < o1; r += 1024) {
    const int64_t t = ts[r];
    mn = t < mn ? t : mn;
    mx = t > mx ? t : mx;
    if (r > o0 && t < ts[r - 1]) unsorted = 1;
  }
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
  const bool wide = (o1 > o0) && (mx - mn > HSTU_NARROW_SPAN_MAX);
#pragma unroll 4
  for (int64_t r = o0 + threadIdx.x; r < o1; r += 1024)
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
                               const int64_t* ts, hipStream_t st, float* z0, float* z1,
                               int64_t nz) {
  if (B <= 0) {
    if (nz > 0) {
      hipError_t e = launch_zero_f32(z0, nz, st);
      if (e == hipSuccess) e = launch_zero_f32(z1, nz, st);
      return e;
    }
    return hipSuccess;
  }
  k_time_prepass<<<B, 1024, 0, st>>>(offs, ts, tm.rel_t, tm.seq_flags, z0, z1, nz);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Work list.
// ---------------------------------------------------------------------------
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

// One workgroup builds one schedule (the launch carries one or two): clear,
// count sequences per block count, the two suffix sums, then the items.  The
// steps communicate through global memory inside the workgroup, so each is
// separated by a barrier and an agent-scope acquire (the vector L1 holds no
// stale line of what other threads wrote or atomically updated).
struct SchedJob {
  int32_t* items;
  int32_t* counters;
  int32_t* hist;
  int32_t* cnt;
  int32_t* levelstart;
  int32_t* tie;
  int cap, bm, reverse;
};

__device__ void sched_step_barrier() {
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

__global__ __launch_bounds__(1024) void k_sched(int B, const int32_t* __restrict__ offs,
                                                SchedJob j0, SchedJob j1) {
  const SchedJob j = blockIdx.x == 0 ? j0 : j1;
  const int t = threadIdx.x;
  for (int i = t; i < j.cap + 2; i += 1024) {
    j.hist[i] = 0;
    j.tie[i] = 0;
  }
  if (t < 4) j.counters[t] = 0;
  sched_step_barrier();
  for (int b = t; b < B; b += 1024) {
    const int n = offs[b + 1] - offs[b];
    const int nb = (n + j.bm - 1) / j.bm;
    atomicAdd(&j.hist[nb], 1);
    atomicMax(&j.counters[1], nb);
  }
  sched_step_barrier();
  const int maxblk = j.counters[1];
  // cnt[m] = #sequences with more than m blocks, m in [0, maxblk]
  block_suffix_excl(j.hist, j.cnt, maxblk + 1, nullptr);
  sched_step_barrier();
  // levelstart[L] = sum of cnt[L'] for L' in (L, maxblk); n_items = sum over [0, maxblk)
  block_suffix_excl(j.cnt, j.levelstart, maxblk, &j.counters[0]);
  if (t == 0 && maxblk == 0) j.counters[0] = 0;
  sched_step_barrier();
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

static SchedJob sched_job(const Sched& s, int reverse) {
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

hipError_t launch_sched(const Sched& s, int B, const int32_t* offs, int reverse, hipStream_t st) {
  const SchedJob j = sched_job(s, reverse);
  k_sched<<<1, 1024, 0, st>>>(B, offs, j, j);
  return hipGetLastError();
}
hipError_t launch_sched2(const Sched& s0, int reverse0, const Sched& s1, int reverse1, int B,
                         const int32_t* offs, hipStream_t st) {
  k_sched<<<2, 1024, 0, st>>>(B, offs, sched_job(s0, reverse0), sched_job(s1, reverse1));
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
