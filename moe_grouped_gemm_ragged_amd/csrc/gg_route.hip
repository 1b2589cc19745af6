// gg_route.hip -- producing the grouped layout the GEMMs consume.
//
// PyTorch issue #152668 ("Describe the bug") builds the grouped GEMM's end
// offsets with a permute-indices kernel that rounds every expert's token
// count up to min_alignment_m (8 or 16 on that page) and, as its fix, pads
// empty experts too; TransformerEngine PR #3224 hands the grouped GEMM
// per-expert row counts (m_splits) on the device.  This file holds those
// steps, all on the device with no host sync:
//
//   offsets_from_splits  offs[g] = sum_{g' <= g} pad(m_splits[g'])
//   route                token-slot -> expert ids -> padded end offsets, the
//                        slot each grouped row holds (-1 for a padding row)
//                        and the row each slot went to; within an expert the
//                        slots keep their order (a stable counting sort)
//   gather_rows          the grouped activations: row r = X[slot(r) / topk],
//                        zero for a padding row
//   combine_rows         back to tokens: out[t] = sum_k w[t, k] Y[row(t, k)]
//
// pad(c) = c rounded up to a multiple of align, and at least align when
// pad_empty is set (an empty expert then gets align padding rows).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gg_internal.h"

namespace gg {
namespace {

typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

constexpr int kRouteThreads = 512;
constexpr int kChunk = 1024;          // slots per block in the route passes
constexpr int kPerThread = kChunk / kRouteThreads;

// End offsets saturate here: the grouped GEMMs take at most this many rows
// (2^31 - 2^16), and clamp every end offset to their row count, so a
// saturated sum stays monotone and reads as "up to the last row" instead of
// wrapping negative in int32.
constexpr int64_t kOffsetCap = (int64_t(1) << 31) - (int64_t(1) << 16);

__device__ __forceinline__ int32_t cap_offset(int64_t v) { return (int32_t)(v < kOffsetCap ? v : kOffsetCap); }

__device__ __forceinline__ int64_t pad_count(int64_t c, int align, bool pad_empty) {
  c = c < 0 ? 0 : c;
  c = c < kOffsetCap ? c : kOffsetCap;      // a sum of such counts stays far inside int64
  int64_t p = (c + align - 1) / align * align;
  if (pad_empty && p < align) p = align;
  return p;
}

// Block-wide exclusive scan of one int64 per thread; returns the total.
__device__ int64_t block_exclusive_scan(int64_t& v, int64_t* s, int tid, int nt) {
  s[tid] = v;
  __syncthreads();
  for (int d = 1; d < nt; d <<= 1) {
    const int64_t o = tid >= d ? s[tid - d] : 0;
    __syncthreads();
    s[tid] += o;
    __syncthreads();
  }
  const int64_t incl = s[tid];
  const int64_t total = s[nt - 1];
  __syncthreads();
  v = incl - v;
  return total;
}

// One workgroup: offs from per-expert counts (int64 m_splits).
__global__ __launch_bounds__(1024) void offsets_from_splits_kernel(const int64_t* splits, int32_t E,
                                                                   int32_t align, int pad_empty,
                                                                   int32_t* offs) {
  __shared__ int64_t s[1024];
  const int tid = threadIdx.x;
  const int per = (E + 1023) / 1024;
  const int g0 = tid * per;
  const int g1 = g0 + per < E ? g0 + per : E;
  int64_t local = 0;
  for (int g = g0; g < g1; ++g) local += pad_count(splits[g], align, pad_empty != 0);
  block_exclusive_scan(local, s, tid, 1024);
  for (int g = g0; g < g1; ++g) {
    local += pad_count(splits[g], align, pad_empty != 0);
    offs[g] = cap_offset(local);
  }
}

// Pass 1: per-block expert histograms, hist[e * nblocks + b].  Slots with an
// expert outside [0, E) are dropped.
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(const int32_t* expert, int64_t slots,
                                                                    int32_t E, int32_t* hist) {
  __shared__ int32_t h[GG_MAX_GROUPS_DEV];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kRouteThreads) h[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  for (int j = 0; j < kPerThread; ++j) {
    const int64_t s = base + j * kRouteThreads + tid;
    if (s < slots) {
      const int e = expert[s];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) hist[(int64_t)e * gridDim.x + blockIdx.x] = h[e];
}

// Pass 2 (one workgroup): per expert, the count, its padded size and end
// offset; hist becomes each block's first row for that expert; padding rows
// get -1 in row_slot.
__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* hist, int32_t nblocks, int32_t E,
                                                          int32_t align, int pad_empty, int32_t* offs,
                                                          int32_t* row_slot) {
  __shared__ int64_t s[1024];
  const int tid = threadIdx.x;
  const int per = (E + 1023) / 1024;
  const int g0 = tid * per;
  const int g1 = g0 + per < E ? g0 + per : E;
  int64_t local = 0;
  for (int g = g0; g < g1; ++g) {
    int64_t c = 0;
    const int32_t* hg = hist + (int64_t)g * nblocks;
#pragma unroll 8
    for (int b = 0; b < nblocks; ++b) c += hg[b];
    local += pad_count(c, align, pad_empty != 0);
  }
  block_exclusive_scan(local, s, tid, 1024);
  int64_t start = local;
  for (int g = g0; g < g1; ++g) {
    int64_t run = start;
    int32_t* hg = hist + (int64_t)g * nblocks;
#pragma unroll 8
    for (int b = 0; b < nblocks; ++b) {
      const int32_t c = hg[b];
      hg[b] = (int32_t)run;
      run += c;
    }
    const int64_t end = start + pad_count(run - start, align, pad_empty != 0);
    for (int64_t r = run; r < end; ++r) row_slot[r] = -1;
    offs[g] = cap_offset(end);   // below the cap: the host bounds the rows
    start = end;
  }
}

// Pass 3: each block sorts its slots by (expert, slot) in LDS (bitonic), so
// a slot's rank among the block's slots of its expert is its sorted position
// minus the position of that expert's first slot; row = the block's first
// row for the expert + rank.
__global__ __launch_bounds__(kRouteThreads) void route_place_kernel(const int32_t* expert, int64_t slots,
                                                                    int32_t E, const int32_t* hist,
                                                                    int32_t* row_slot, int32_t* slot_row) {
  __shared__ uint32_t key[kChunk];
  __shared__ int32_t first[GG_MAX_GROUPS_DEV];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kChunk;
  // key = expert (E for dropped or past the end) << 11 | local slot index
  static_assert(kChunk <= 2048, "the slot index takes 11 bits of the key");
  for (int j = 0; j < kPerThread; ++j) {
    const int i = j * kRouteThreads + tid;
    const int64_t s = base + i;
    int e = E;
    if (s < slots) {
      const int v = expert[s];
      e = (v >= 0 && v < E) ? v : E;
    }
    key[i] = ((uint32_t)e << 11) | (uint32_t)i;
  }
  __syncthreads();
  for (int size = 2; size <= kChunk; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int j = 0; j < kChunk / 2 / kRouteThreads; ++j) {
        const int t = j * kRouteThreads + tid;           // pair index
        const int lo = 2 * t - (t & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint32_t a = key[lo], b = key[hi];
        if ((a > b) == up) {
          key[lo] = b;
          key[hi] = a;
        }
      }
      __syncthreads();
    }
  }
  for (int j = 0; j < kPerThread; ++j) {
    const int p = j * kRouteThreads + tid;
    const int e = (int)(key[p] >> 11);
    if (e < E && (p == 0 || (int)(key[p - 1] >> 11) != e)) first[e] = p;
  }
  __syncthreads();
  for (int j = 0; j < kPerThread; ++j) {
    const int p = j * kRouteThreads + tid;
    const int e = (int)(key[p] >> 11);
    const int i = (int)(key[p] & 2047u);
    const int64_t s = base + i;
    if (s >= slots) continue;
    if (e >= E) {
      slot_row[s] = -1;
      continue;
    }
    const int32_t row = hist[(int64_t)e * gridDim.x + blockIdx.x] + (p - first[e]);
    row_slot[row] = (int32_t)s;
    slot_row[s] = row;
  }
}

// Grouped rows from token rows: dst[r] = src[row_slot[r] / topk] for r below
// the last end offset, zeros for a padding row (row_slot -1).  16 bytes per
// lane; row_bytes is a multiple of 16.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* src, int64_t row_bytes,
                                                          const int32_t* row_slot, int32_t topk,
                                                          const int32_t* offs, int32_t E, int64_t rows_cap,
                                                          int64_t tokens, uint8_t* dst) {
  // the last end offset, clamped as the GEMMs clamp it
  __shared__ int64_t s_rows;
  if (threadIdx.x == 0) {
    int64_t run = 0;
    for (int g = 0; g < E; ++g) run = offs[g] > run ? offs[g] : run;
    s_rows = run < rows_cap ? run : rows_cap;
  }
  __syncthreads();
  const int64_t rows = s_rows;
  const int64_t vec_per_row = row_bytes / 16;
  const int64_t total = rows * vec_per_row;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = v / vec_per_row;
    const int64_t c = v - r * vec_per_row;
    const int32_t s = row_slot[r];
    u32x4v out = {0u, 0u, 0u, 0u};
    if (s >= 0 && s / topk < tokens)
      out = *reinterpret_cast<const u32x4v*>(src + (int64_t)(s / topk) * row_bytes + 16 * c);
    *reinterpret_cast<u32x4v*>(dst + r * row_bytes + 16 * c) = out;
  }
}

// Back to tokens: out[t, :] = sum_k w[t, k] y[slot_row[t topk + k], :] in
// fp32 (w = 1 when null; dropped slots, row -1, add nothing), rounded once
// to bf16 (or stored as fp32).  8 columns per lane.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void combine_rows_kernel(const uint16_t* y, int64_t n, const int32_t* slot_row,
                                                           const float* w, int32_t topk, int64_t tokens,
                                                           int64_t rows_cap, void* out) {
  const int64_t groups = n / 8;
  const int64_t total = tokens * groups;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = v / groups;
    const int64_t c = (v - t * groups) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < topk; ++k) {
      const int32_t r = slot_row[t * topk + k];
      if (r < 0 || r >= rows_cap) continue;
      const float wk = w ? w[t * topk + k] : 1.0f;
      const u32x4v q = *reinterpret_cast<const u32x4v*>(y + r * n + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += wk * __builtin_bit_cast(float, q[e] << 16);
        acc[2 * e + 1] += wk * __builtin_bit_cast(float, q[e] & 0xFFFF0000u);
      }
    }
    if constexpr (OUT_F32) {
      float* o = static_cast<float*>(out) + t * n + c;
      *reinterpret_cast<f32x4v*>(o) = f32x4v{acc[0], acc[1], acc[2], acc[3]};
      *reinterpret_cast<f32x4v*>(o + 4) = f32x4v{acc[4], acc[5], acc[6], acc[7]};
    } else {
      u32x4v q;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f32x2v f = {acc[2 * e], acc[2 * e + 1]};
        q[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
      }
      *reinterpret_cast<u32x4v*>(static_cast<uint16_t*>(out) + t * n + c) = q;
    }
  }
}

int grid_for(int64_t work, int num_cus) {
  const int64_t want = (work + 255) / 256;
  const int64_t cap = 8 * (int64_t)num_cus;
  return (int)(want < 1 ? 1 : (want < cap ? want : cap));
}

}  // namespace

int64_t route_blocks(int64_t slots) { return (slots + kChunk - 1) / kChunk; }

hipError_t launch_offsets_from_splits(const int64_t* splits, int32_t E, int32_t align, bool pad_empty,
                                      int32_t* offs, hipStream_t stream) {
  return launch_kernel(offsets_from_splits_kernel, dim3(1), dim3(1024), stream, splits, E, align,
                       pad_empty ? 1 : 0, offs);
}

hipError_t launch_route(const int32_t* expert, int64_t slots, int32_t E, int32_t align, bool pad_empty,
                        int32_t* offs, int32_t* row_slot, int32_t* slot_row, int32_t* hist,
                        hipStream_t stream) {
  const int nb = (int)route_blocks(slots);
  if (nb > 0) {
    const hipError_t e = launch_kernel(route_count_kernel, dim3(nb), dim3(kRouteThreads), stream, expert, slots,
                                       E, hist);
    if (e != hipSuccess) return e;
  }
  const hipError_t e = launch_kernel(route_scan_kernel, dim3(1), dim3(1024), stream, hist, nb, E, align,
                                     pad_empty ? 1 : 0, offs, row_slot);
  if (e != hipSuccess || nb == 0) return e;
  return launch_kernel(route_place_kernel, dim3(nb), dim3(kRouteThreads), stream, expert, slots, E, hist,
                       row_slot, slot_row);
}

hipError_t launch_gather_rows(const void* src, int64_t row_bytes, const int32_t* row_slot, int32_t topk,
                              const int32_t* offs, int32_t E, int64_t rows_cap, int64_t tokens, void* dst,
                              int num_cus, hipStream_t stream) {
  return launch_kernel(gather_rows_kernel, dim3(grid_for(rows_cap * (row_bytes / 16), num_cus)), dim3(256),
                       stream, static_cast<const uint8_t*>(src), row_bytes, row_slot, topk, offs, E, rows_cap,
                       tokens, static_cast<uint8_t*>(dst));
}

hipError_t launch_combine_rows(const void* y, int64_t n, const int32_t* slot_row, const float* w, int32_t topk,
                               int64_t tokens, int64_t rows_cap, void* out, bool out_f32, int num_cus,
                               hipStream_t stream) {
  const int grid = grid_for(tokens * (n / 8), num_cus);
  if (out_f32)
    return launch_kernel(combine_rows_kernel<true>, dim3(grid), dim3(256), stream,
                         static_cast<const uint16_t*>(y), n, slot_row, w, topk, tokens, rows_cap, out);
  return launch_kernel(combine_rows_kernel<false>, dim3(grid), dim3(256), stream,
                       static_cast<const uint16_t*>(y), n, slot_row, w, topk, tokens, rows_cap, out);
}

}  // namespace gg
