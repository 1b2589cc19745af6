// gg_bias_grad.hip -- the backward of the grouped bias with a per-token
// factor, y[i, :] += s[i] * bias[g, :] over the rows i of expert g:
//
//   dbias[g, n] = sum_{i in g} s[i] dY[i, n]        (s = 1 when absent)
//   ds[i]       = sum_n bias[g, n] dY[i, n]          (rows an expert owns)
//
// Both are reductions over bf16 dY in fp32, HBM-bound, in a fixed order per
// element (deterministic; no atomics).  Groups as everywhere: clamped end
// offsets (ragged) or masked_m (masked, rows e * max_m + r, r < masked_m[e]).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gg_internal.h"

namespace gg {
namespace {

typedef uint32_t u32x4b __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRowLanes = 4;                       // threads along the rows of one column group
constexpr int kColsPerBlock = 8 * (kThreads / kRowLanes);   // 512 columns per workgroup

__device__ __forceinline__ void unpack8(const u32x4b q, float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __builtin_bit_cast(float, q[e] << 16);
    v[2 * e + 1] = __builtin_bit_cast(float, q[e] & 0xFFFF0000u);
  }
}

// Rows [start, end) of expert g in the flat row index space.
template <bool MASKED>
__device__ __forceinline__ void group_rows(const int32_t* groups, int g, int64_t m, int64_t& start,
                                           int64_t& end) {
  if constexpr (MASKED) {
    int64_t a = groups[g];
    a = a < 0 ? 0 : (a > m ? m : a);
    start = (int64_t)g * m;
    end = start + a;
  } else {
    // end(g) = min(max(offs[0..g]), m); start = end(g - 1)
    int64_t run = 0, prev = 0;
    for (int h = 0; h <= g; ++h) {
      prev = run;
      const int64_t o = groups[h];
      run = o > run ? o : run;
      run = run < m ? run : m;
    }
    start = prev;
    end = run;
  }
}

// One workgroup per (expert, 512-column block): thread (c, l) sums columns
// 8 c .. 8 c + 7 over rows start + l, start + l + 4, ...; the 4 partial sums
// of a column are added in LDS in order l = 0..3.
template <bool MASKED>
__global__ __launch_bounds__(kThreads) void dbias_kernel(const uint16_t* dy, const int32_t* groups,
                                                         const float* scale, int64_t m, int64_t n,
                                                         int32_t E, float* dbias) {
  __shared__ float part[kRowLanes][kColsPerBlock];
  const int col_blocks = (int)((n + kColsPerBlock - 1) / kColsPerBlock);
  const int g = blockIdx.x / col_blocks;
  const int cb = blockIdx.x - g * col_blocks;
  const int tid = threadIdx.x;
  const int l = tid % kRowLanes;
  const int c = tid / kRowLanes;
  const int64_t col = (int64_t)cb * kColsPerBlock + 8 * c;
  int64_t start, end;
  group_rows<MASKED>(groups, g, m, start, end);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (col < n) {
    for (int64_t i = start + l; i < end; i += kRowLanes) {
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
  for (int j = tid; j < kColsPerBlock; j += kThreads) {
    const int64_t cc = (int64_t)cb * kColsPerBlock + j;
    if (cc < n) {
      float t = part[0][j];
#pragma unroll
      for (int q = 1; q < kRowLanes; ++q) t += part[q][j];
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
  const int tid = threadIdx.x;
  // expert ends, so each row finds its expert by binary search
  if constexpr (!MASKED) {
    if (tid == 0) {
      int64_t run = 0;
      for (int h = 0; h < E; ++h) {
        const int64_t o = groups[h];
        run = o > run ? o : run;
        run = run < m ? run : m;
        s_end[h] = (int32_t)run;
      }
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
  const int col_blocks = (int)((n + kColsPerBlock - 1) / kColsPerBlock);
  const dim3 grid((unsigned)(E * col_blocks));
  if (masked)
    hipLaunchKernelGGL(dbias_kernel<true>, grid, dim3(kThreads), 0, stream, static_cast<const uint16_t*>(dy),
                       groups, scale, m, n, E, dbias);
  else
    hipLaunchKernelGGL(dbias_kernel<false>, grid, dim3(kThreads), 0, stream, static_cast<const uint16_t*>(dy),
                       groups, scale, m, n, E, dbias);
  return hipGetLastError();
}

hipError_t launch_dscale(bool masked, const void* dy, const int32_t* groups, const void* bias, int64_t m,
                         int64_t n, int32_t E, float* ds, int num_cus, hipStream_t stream) {
  const int64_t rows = masked ? (int64_t)E * m : m;
  const int64_t want = (rows + 3) / 4;
  const int64_t cap = 8 * (int64_t)num_cus;
  const int grid = (int)(want < 1 ? 1 : (want < cap ? want : cap));
  if (masked)
    hipLaunchKernelGGL(dscale_kernel<true>, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(dy), groups, static_cast<const uint16_t*>(bias), m, n, E,
                       rows, ds);
  else
    hipLaunchKernelGGL(dscale_kernel<false>, dim3(grid), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(dy), groups, static_cast<const uint16_t*>(bias), m, n, E,
                       rows, ds);
  return hipGetLastError();
}

}  // namespace gg
