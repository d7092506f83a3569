// Attention truncation ("Bending the Scaling Law Curve in Large-Scale
// Recommendation Systems", Attention Truncation: after the layers over whole
// sequences, further layers see only a segment of each history made of its
// most recent events).  The segment of sequence b is the contiguous tail of
// min(n_b - c_b, keep) history rows followed by its c_b candidate rows, so
// segment row r of sequence b comes from full row
//     src(r) = seq_offsets[b+1] - seg_offsets[b+1] + r.
// Three kernels: the segment offsets (one workgroup scan), the row gather
// into the truncated batch (activations and timestamps) and its backward,
// the row scatter of the gradient (zero outside the segments).  The copies
// are HBM-bound: 16-byte vectors, four in flight per lane, a wave per four
// rows so that each wave's row-to-sequence search runs once.
#include "common.h"
#include "internal.h"

namespace hstu {
namespace {

HSTU_DEV int seg_len(const int32_t* offs, const int32_t* nc, int keep, int b) {
  const int n = offs[b + 1] - offs[b];
  const int c = nc ? min(max(nc[b], 0), n) : 0;
  return min(n - c, keep) + c;
}

// seg_offsets[0] = 0, seg_offsets[b+1] = seg_offsets[b] + seg_len(b): each
// thread sums a contiguous run of sequences, the runs are scanned in LDS.
constexpr int SCAN_T = 1024;
__global__ __launch_bounds__(SCAN_T) void k_trunc_offsets(int B, const int32_t* offs,
                                                          const int32_t* nc, int keep,
                                                          int32_t* seg) {
  __shared__ int32_t part[SCAN_T];
  const int t = threadIdx.x;
  const int per = (B + SCAN_T - 1) / SCAN_T;
  const int b0 = min(t * per, B), b1 = min(b0 + per, B);
  int s = 0;
  for (int b = b0; b < b1; ++b) s += seg_len(offs, nc, keep, b);
  part[t] = s;
  __syncthreads();
  for (int o = 1; o < SCAN_T; o <<= 1) {  // inclusive Hillis-Steele scan
    const int v = t >= o ? part[t - o] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int run = t ? part[t - 1] : 0;
  if (t == 0) seg[0] = 0;
  for (int b = b0; b < b1; ++b) {
    run += seg_len(offs, nc, keep, b);
    seg[b + 1] = run;
  }
}

// Largest b in [0, B) with bounds[b] <= r (the non-empty sequence holding
// row r when r < bounds[B]).
HSTU_DEV int seq_of(const int32_t* bounds, int B, int r) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (bounds[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr int ROWS_PER_WAVE = 4;
constexpr int COPY_THREADS = 256;
constexpr int UNROLL = 4;

// Destination rows [0, rows), a row = cpr 16-byte chunks.  For destination
// row r of sequence b, map(r, b) returns the source row or -1 (write zeros);
// `bounds` are the destination's sequence offsets.  Rows at or past
// bounds[B] belong to no sequence and get map(r, B - 1), which the maps
// reject; every source row a map returns is range-checked by the map.
template <typename Map>
HSTU_DEV void copy_rows(int B, int64_t rows, int cpr, const int32_t* bounds, const u32x4* src,
                        u32x4* dst, Map map) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t(blockIdx.x) * COPY_THREADS + threadIdx.x) >> 6;
  const int64_t r0 = wave * ROWS_PER_WAVE;
  if (r0 >= rows) return;
  const int nr = int(min<int64_t>(ROWS_PER_WAVE, rows - r0));
  const int b0 = seq_of(bounds, B, int(r0));
  const int n = nr * cpr;
  for (int k0 = lane; k0 < n; k0 += 64 * UNROLL) {
    u32x4 v[UNROLL];
    int64_t at[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int k = k0 + 64 * u;
      at[u] = -1;
      if (k < n) {
        const int q = k / cpr, c = k - q * cpr;
        const int r = int(r0) + q;
        int b = b0;
        while (b < B - 1 && bounds[b + 1] <= r) ++b;
        const int64_t s = map(r, b);
        at[u] = int64_t(r) * cpr + c;
        v[u] = s >= 0 ? src[s * cpr + c] : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
      if (at[u] >= 0) dst[at[u]] = v[u];
  }
}

__global__ __launch_bounds__(COPY_THREADS) void k_trunc_gather(int B, int64_t T, int64_t Tseg,
                                                                int cpr, const int32_t* offs,
                                                                const int32_t* seg,
                                                                const u32x4* x, u32x4* xs,
                                                                const int64_t* ts, int64_t* tss) {
  // segment row r of sequence b (seg[b] <= r < seg[b+1]) comes from full row
  // offs[b+1] - seg[b+1] + r
  auto src_row = [&](int r, int b) -> int64_t {
    if (r >= seg[b + 1]) return -1;
    const int64_t i = int64_t(offs[b + 1]) - seg[b + 1] + r;
    return (i >= 0 && i < T) ? i : -1;
  };
  copy_rows(B, Tseg, cpr, seg, x, xs, src_row);
  if (tss) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (((int64_t(blockIdx.x) * COPY_THREADS + threadIdx.x) >> 6) *
                       ROWS_PER_WAVE) + lane;
    if (lane < ROWS_PER_WAVE && r < Tseg) {
      const int64_t i = src_row(int(r), seq_of(seg, B, int(r)));
      tss[r] = i >= 0 ? ts[i] : int64_t(0);
    }
  }
}

__global__ __launch_bounds__(COPY_THREADS) void k_trunc_scatter(int B, int64_t T, int64_t Tseg,
                                                                 int cpr, const int32_t* offs,
                                                                 const int32_t* seg,
                                                                 const u32x4* dxs, u32x4* dx) {
  // full row i of sequence b lies in its segment iff i >= offs[b+1] - len_b
  auto seg_row = [&](int i, int b) -> int64_t {
    if (i >= offs[b + 1]) return -1;
    const int64_t r = int64_t(seg[b + 1]) - offs[b + 1] + i;
    return (r >= seg[b] && r >= 0 && r < Tseg) ? r : -1;
  };
  copy_rows(B, T, cpr, offs, dxs, dx, seg_row);
}

int copy_grid(int64_t rows) {
  const int64_t waves = (rows + ROWS_PER_WAVE - 1) / ROWS_PER_WAVE;
  return int((waves * 64 + COPY_THREADS - 1) / COPY_THREADS);
}

}  // namespace

hipError_t launch_trunc_offsets(int B, const int32_t* offs, const int32_t* nc, int keep,
                                int32_t* seg, hipStream_t st) {
  k_trunc_offsets<<<1, SCAN_T, 0, st>>>(B, offs, nc, keep, seg);
  return hipGetLastError();
}

hipError_t launch_trunc_gather(int B, int64_t T, int64_t Tseg, int64_t row_bytes,
                               const int32_t* offs, const int32_t* seg, const void* x, void* xs,
                               const int64_t* ts, int64_t* tss, hipStream_t st) {
  if (Tseg <= 0 || B <= 0) return hipSuccess;
  k_trunc_gather<<<copy_grid(Tseg), COPY_THREADS, 0, st>>>(
      B, T, Tseg, int(row_bytes / 16), offs, seg, static_cast<const u32x4*>(x),
      static_cast<u32x4*>(xs), ts, tss);
  return hipGetLastError();
}

hipError_t launch_trunc_scatter(int B, int64_t T, int64_t Tseg, int64_t row_bytes,
                                const int32_t* offs, const int32_t* seg, const void* dxs,
                                void* dx, hipStream_t st) {
  if (T <= 0 || B <= 0) return hipSuccess;
  k_trunc_scatter<<<copy_grid(T), COPY_THREADS, 0, st>>>(
      B, T, Tseg, int(row_bytes / 16), offs, seg, static_cast<const u32x4*>(dxs),
      static_cast<u32x4*>(dx));
  return hipGetLastError();
}

}  // namespace hstu
