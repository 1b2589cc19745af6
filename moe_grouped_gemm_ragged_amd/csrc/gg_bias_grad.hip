// gg_bias_grad.hip -- the backward of the grouped bias with a per-token
// factor, y[i, :] += s[i] * bias[g, :] over the rows i of expert g:
//
//   dbias[g, n] = sum_{i in g} s[i] dY[i, n]        (s = 1 when absent)
//   ds[i]       = sum_n bias[g, n] dY[i, n]          (rows an expert owns)
//
// Both are reductions over bf16 dY in fp32, HBM-bound, in a fixed order per
// element (deterministic; no atomics).  Groups as everywhere: clamped end
// offsets (ragged) or masked_m (masked, rows e * max_m + r, r < masked_m[e]).
// An expert's row range and the per-row expert lookup come from cooperative
// maxima and scans over the offsets, never a serial walk.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gg_internal.h"

namespace gg {
namespace {

typedef uint32_t u32x4b __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// dbias: a workgroup owns COLS (64 or 128) columns of one expert -- COLS / 8
// column groups of 8 (16 bytes per lane) by the remaining row lanes, each
// thread with 8 rows in flight.
constexpr int kDbUnroll = 8;
// Average rows per expert from which a workgroup takes 128 columns: large
// experts stream better with 256 bytes of a row per workgroup, many small
// (and typically skewed) experts balance better over twice the workgroups.
constexpr int64_t kDbWideRows = 2048;

__device__ __forceinline__ void unpack8(const u32x4b q, float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __builtin_bit_cast(float, q[e] << 16);
    v[2 * e + 1] = __builtin_bit_cast(float, q[e] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ int imax(int a, int b) { return a > b ? a : b; }

// Rows [start, end) of expert g in the flat row index space, computed by
// the whole workgroup.  Ragged: end(g) = min(max(0, offs[0..g]), m) and
// start = end(g - 1) (0 for g = 0) -- two maxima over the offsets, strided
// over the threads, then reduced across lanes and waves.  red: kWaves * 2
// ints of LDS.
template <bool MASKED>
__device__ __forceinline__ void group_rows(const int32_t* groups, int g, int64_t m, int tid, int32_t* red,
                                           int64_t& start, int64_t& end) {
  if constexpr (MASKED) {
    int64_t a = groups[g];
    a = a < 0 ? 0 : (a > m ? m : a);
    start = (int64_t)g * m;
    end = start + a;
  } else {
    int upto = 0, before = 0;          // max over offs[0..g] and offs[0..g-1], floored at 0
    for (int h = tid; h <= g; h += kThreads) {
      const int o = groups[h];
      upto = imax(upto, o);
      if (h < g) before = imax(before, o);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      upto = imax(upto, __shfl_xor(upto, off, 64));
      before = imax(before, __shfl_xor(before, off, 64));
    }
    if ((tid & 63) == 0) {
      red[2 * (tid >> 6)] = upto;
      red[2 * (tid >> 6) + 1] = before;
    }
    __syncthreads();
    upto = 0;
    before = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      upto = imax(upto, red[2 * w]);
      before = imax(before, red[2 * w + 1]);
    }
    end = upto < m ? upto : m;
    start = before < m ? before : m;
  }
}

// One workgroup per (expert, COLS-column block).  Thread (c, l) = (tid mod
// G, tid / G), G = COLS / 8, sums columns 8 c .. 8 c + 7 over its rows
// start + l, start + l + L, ... (L = 256 / G row lanes) in increasing order,
// loading 8 of them at a time; the L row lanes of a column are then added in
// LDS in order l = 0..L-1: a fixed order per element.
template <bool MASKED, int COLS>
__global__ __launch_bounds__(kThreads) void dbias_kernel(const uint16_t* dy, const int32_t* groups,
                                                         const float* scale, int64_t m, int64_t n,
                                                         int32_t E, float* dbias) {
  constexpr int kDbCols = COLS;
  constexpr int kDbGroups = COLS / 8;
  constexpr int kDbLanes = kThreads / kDbGroups;
  __shared__ float part[kDbLanes][kDbCols];
  __shared__ int32_t red[2 * kWaves];
  const int col_blocks = (int)((n + kDbCols - 1) / kDbCols);
  const int g = blockIdx.x / col_blocks;
  const int cb = blockIdx.x - g * col_blocks;
  const int tid = threadIdx.x;
  const int c = tid % kDbGroups;
  const int l = tid / kDbGroups;
  const int64_t col = (int64_t)cb * kDbCols + 8 * c;
  int64_t start, end;
  group_rows<MASKED>(groups, g, m, tid, red, start, end);
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  if (col < n) {
    int64_t i = start + l;
    for (; i + (kDbUnroll - 1) * kDbLanes < end; i += kDbUnroll * kDbLanes) {
      u32x4b q[kDbUnroll];
      float s[kDbUnroll];
#pragma unroll
      for (int u = 0; u < kDbUnroll; ++u) {
        const int64_t r = i + u * kDbLanes;
        q[u] = *reinterpret_cast<const u32x4b*>(dy + r * n + col);
        s[u] = scale ? scale[r] : 1.0f;
      }
#pragma unroll
      for (int u = 0; u < kDbUnroll; ++u) {
        float v[8];
        unpack8(q[u], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += s[u] * v[e];
      }
    }
    for (; i < end; i += kDbLanes) {
      const float s = scale ? scale[i] : 1.0f;
      float v[8];
      unpack8(*reinterpret_cast<const u32x4b*>(dy + i * n + col), v);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += s * v[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[l][8 * c + e] = acc[e];
  __syncthreads();
  for (int j = tid; j < kDbCols; j += kThreads) {
    const int64_t cc = (int64_t)cb * kDbCols + j;
    if (cc < n) {
      float t = part[0][j];
#pragma unroll
      for (int q = 1; q < kDbLanes; ++q) t += part[q][j];
      dbias[(int64_t)g * n + cc] = t;
    }
  }
}

// One wave per row: ds[i] = sum_n bias[g, n] dY[i, n] for rows an expert
// owns (8 columns per lane, then a fixed-order reduction across the wave).
template <bool MASKED>
__global__ __launch_bounds__(kThreads) void dscale_kernel(const uint16_t* dy, const int32_t* groups,
                                                          const uint16_t* bias, int64_t m, int64_t n,
                                                          int32_t E, int64_t rows, float* ds) {
  __shared__ int32_t s_end[GG_MAX_GROUPS_DEV];
  __shared__ int32_t wave_max[kWaves];
  const int tid = threadIdx.x;
  // expert ends end(h) = min(max(0, offs[0..h]), m), so each row finds its
  // expert by binary search: thread t takes a run of consecutive experts,
  // writes its local prefix maxima, and raises them by the maximum of the
  // runs before its own (a shuffle scan within the wave, then the totals of
  // the earlier waves).
  if constexpr (!MASKED) {
    const int per = (E + kThreads - 1) / kThreads;
    const int h0 = tid * per;
    const int h1 = h0 + per < E ? h0 + per : E;
    int run = 0;
    for (int h = h0; h < h1; ++h) {
      run = imax(run, groups[h]);
      s_end[h] = run;
    }
    const int lane = tid & 63, w = tid >> 6;
    int incl = run;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, (unsigned)d, 64);
      if (lane >= d) incl = imax(incl, o);
    }
    int before = __shfl_up(incl, 1u, 64);
    if (lane == 0) before = 0;
    if (lane == 63) wave_max[w] = incl;
    __syncthreads();
    for (int q = 0; q < w; ++q) before = imax(before, wave_max[q]);
    const int mcap = m < 2147483647 ? (int)m : 2147483647;
    for (int h = h0; h < h1; ++h) {
      const int e = imax(s_end[h], before);
      s_end[h] = e < mcap ? e : mcap;
    }
    __syncthreads();
  }
  const int lane = tid & 63;
  const int64_t waves = (int64_t)gridDim.x * (kThreads / 64);
  for (int64_t i = (int64_t)blockIdx.x * (kThreads / 64) + (tid >> 6); i < rows; i += waves) {
    int g;
    bool owned;
    if constexpr (MASKED) {
      g = (int)(i / m);
      int64_t a = groups[g];
      a = a < 0 ? 0 : (a > m ? m : a);
      owned = (i - (int64_t)g * m) < a;
    } else {
      int lo = 0, hi = E;                       // first g with end(g) > i
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_end[mid] > i) hi = mid; else lo = mid + 1;
      }
      g = lo;
      owned = lo < E;
    }
    if (!owned) continue;                        // ds of rows no expert owns is untouched
    float acc = 0.f;
    for (int64_t col = 8 * lane; col < n; col += 8 * 64) {
      float v[8], b[8];
      unpack8(*reinterpret_cast<const u32x4b*>(dy + i * n + col), v);
      unpack8(*reinterpret_cast<const u32x4b*>(bias + (int64_t)g * n + col), b);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += b[e] * v[e];
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) ds[i] = acc;
  }
}

}  // namespace

hipError_t launch_dbias(bool masked, const void* dy, const int32_t* groups, const float* scale, int64_t m,
                        int64_t n, int32_t E, float* dbias, hipStream_t stream) {
  // rows per expert: max_m (masked), or the average m / E (ragged)
  const bool wide = (masked ? m : m / E) >= kDbWideRows;
  const int cols = wide ? 128 : 64;
  const dim3 grid((unsigned)(E * ((n + cols - 1) / cols)));
  const uint16_t* d = static_cast<const uint16_t*>(dy);
  if (masked && wide)
    return launch_kernel(dbias_kernel<true, 128>, grid, dim3(kThreads), stream, d, groups, scale, m, n, E, dbias);
  if (masked)
    return launch_kernel(dbias_kernel<true, 64>, grid, dim3(kThreads), stream, d, groups, scale, m, n, E, dbias);
  if (wide)
    return launch_kernel(dbias_kernel<false, 128>, grid, dim3(kThreads), stream, d, groups, scale, m, n, E, dbias);
  return launch_kernel(dbias_kernel<false, 64>, grid, dim3(kThreads), stream, d, groups, scale, m, n, E, dbias);
}

hipError_t launch_dscale(bool masked, const void* dy, const int32_t* groups, const void* bias, int64_t m,
                         int64_t n, int32_t E, float* ds, int num_cus, hipStream_t stream) {
  const int64_t rows = masked ? (int64_t)E * m : m;
  const int64_t want = (rows + 3) / 4;
  const int64_t cap = 8 * (int64_t)num_cus;
  const int grid = (int)(want < 1 ? 1 : (want < cap ? want : cap));
  if (masked)
    return launch_kernel(dscale_kernel<true>, dim3(grid), dim3(kThreads), stream,
                         static_cast<const uint16_t*>(dy), groups, static_cast<const uint16_t*>(bias), m, n, E,
                         rows, ds);
  return launch_kernel(dscale_kernel<false>, dim3(grid), dim3(kThreads), stream,
                       static_cast<const uint16_t*>(dy), groups, static_cast<const uint16_t*>(bias), m, n, E,
                       rows, ds);
}

}  // namespace gg
