// gg_fp8_scales.hip -- the scale-layout step of the fp8 block-scaled forward.
//
// The fp8 kernels read their power-of-two scales as E8M0 bytes (2^(e - 127))
// in a packed, tile-major layout (stated with the fp8 main loop in
// gg_kernels.hip): for every 256-row tile of an operand and every k-block of
// 128 reduction values, 256 bytes, tile row r at 128 (r / 128) + 4 (r mod 32)
// + (r / 32) mod 4.  This kernel writes that layout from the scales as a
// quantizer emits them -- fp32 values [rows, k-blocks] (sglang PR #32385,
// "Cause": the fp32 fallback branch) or one E8M0 byte each (the packed int32
// branch of the same table is four such bytes per word) -- and counts the
// scales that are not UE8M0.
//
// Only active rows are read or validated: rows past an expert's end offset,
// or at or past masked_m in the masked layout, are written as zero bytes and
// never looked at, whatever the caller left there (the page's "Cause" and
// "Rejected alternatives": validating the padding is what failed).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gg_internal.h"

namespace gg {
namespace {

constexpr int kRows = 256;     // rows per packed tile
constexpr int kThreads = 256;
constexpr int kChunk = 32;     // k-blocks of a tile staged in LDS at a time
constexpr int kPitch = kRows + 4;   // LDS bytes per staged k-block (padded: the 32 k-blocks of one row fall in 32 banks)

// Block-wide scan of one non-negative int per thread (sum, or max): a
// shuffle scan within each wave, then the totals of the earlier waves.
// Returns the inclusive value; *excl gets the exclusive one (0 for thread 0).
template <bool MAX>
__device__ __forceinline__ int block_scan(int v, int* wave_tot, int tid, int* excl) {
  const int lane = tid & 63, w = tid >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(v, (unsigned)d, 64);
    if (lane >= d) v = MAX ? (v > o ? v : o) : v + o;
  }
  int prev = __shfl_up(v, 1u, 64);
  if (lane == 0) prev = 0;
  if (lane == 63) wave_tot[w] = v;
  __syncthreads();
  int before = 0;
  for (int q = 0; q < w; ++q) {
    const int t = wave_tot[q];
    before = MAX ? (before > t ? before : t) : before + t;
  }
  __syncthreads();
  *excl = MAX ? (prev > before ? prev : before) : prev + before;
  return MAX ? (v > before ? v : before) : v + before;
}

// E8M0 byte of one scale, and whether the scale is UE8M0: an fp32 with
// sign and mantissa bits clear (+0.0 or a positive power of two; +0.0 maps
// to the smallest E8M0 value, 2^-127), or any byte but 0xFF (E8M0's NaN).
template <bool SRC_F32>
__device__ __forceinline__ uint32_t e8m0(const void* src, int64_t idx, int& bad) {
  if constexpr (SRC_F32) {
    const uint32_t bits = reinterpret_cast<const uint32_t*>(src)[idx];
    bad += (bits & 0x807FFFFFu) != 0u;
    return (bits >> 23) & 0xFFu;
  } else {
    const uint32_t b = reinterpret_cast<const uint8_t*>(src)[idx];
    bad += b == 0xFFu;
    return b;
  }
}

// LAYOUT 0: ragged activations (groups = end offsets, rows = M);
// 1: masked activations (groups = masked_m, rows = max_m per expert);
// 2: weights (rows = N per expert, groups unused).  VEC: fp32 scales read
// four k-blocks per 16-byte load (the row pitch and the k-block count are
// multiples of 4 and the source is 16-byte aligned).
typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
template <int LAYOUT, bool SRC_F32, bool VEC>
__global__ __launch_bounds__(kThreads) void pack_scales_kernel(const void* src, int64_t ld_src,
                                                               const int32_t* groups, int64_t rows,
                                                               int32_t kblocks, int32_t num_groups,
                                                               int64_t tiles, uint8_t* dst,
                                                               int32_t* bad_count) {
  __shared__ int32_t s_end[GG_MAX_GROUPS_DEV];
  __shared__ int32_t s_pref[GG_MAX_GROUPS_DEV + 1];
  __shared__ int32_t s_wave[kThreads / 64];
  __shared__ uint8_t s_bytes[kChunk * kPitch];
  __shared__ int32_t s_bad;
  const int tid = threadIdx.x;
  const int E = num_groups;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  int64_t total = tiles;
  if constexpr (LAYOUT == 0) {
    // clamped monotone ends (prefix max of the offsets, capped at rows) and
    // the prefix of per-expert 256-row tile counts, as the GEMM decodes them
    const int per = (E + kThreads - 1) / kThreads;
    const int g0 = tid * per;
    const int g1 = g0 + per < E ? g0 + per : E;
    int run = 0;
    for (int g = g0; g < g1; ++g) {
      const int o = groups[g];
      run = o > run ? o : run;
      s_end[g] = run;
    }
    int before;
    block_scan<true>(run, s_wave, tid, &before);
    int local = 0;
    for (int g = g0; g < g1; ++g) {
      int e = s_end[g] > before ? s_end[g] : before;
      e = e < rows ? e : (int)rows;
      s_end[g] = e;
    }
    __syncthreads();
    for (int g = g0; g < g1; ++g) {
      const int start = g == 0 ? 0 : s_end[g - 1];
      local += (s_end[g] - start + kRows - 1) / kRows;
    }
    int acc;
    const int incl = block_scan<false>(local, s_wave, tid, &acc);
    for (int g = g0; g < g1; ++g) {
      s_pref[g] = acc;
      const int start = g == 0 ? 0 : s_end[g - 1];
      acc += (s_end[g] - start + kRows - 1) / kRows;
    }
    if (tid == kThreads - 1) s_pref[E] = incl;
    __syncthreads();
    total = s_pref[E];
  }
  const int64_t tpe = (rows + kRows - 1) / kRows;   // layouts 1, 2: tiles per expert
  int bad = 0;
  // Thread t writes dword d = t mod 64 of k-blocks t / 64, t / 64 + 4, ...:
  // the bytes of tile rows 128 (d / 32) + d mod 32 + 32 b, b = 0..3.  VEC:
  // per tile and chunk of up to 32 k-blocks, thread (tid mod 8, tid / 8)
  // first reads k-blocks 4 (tid mod 8) .. + 3 of tile rows tid / 8, + 32,
  // ... with one 16-byte load each (a row's scales are consecutive, so the
  // loads of a wave cover 8 rows' chunks contiguously) and stores the E8M0
  // bytes transposed in LDS ([k-block][row]), from where the dwords are
  // assembled.  Otherwise each thread reads its dwords' four scales itself.
  const int d = tid & 63;
  const int kb0 = tid >> 6;
  for (int64_t T = blockIdx.x; T < total; T += gridDim.x) {
    int64_t first;     // source row of tile row 0
    int64_t valid;     // rows of the tile that are active
    if constexpr (LAYOUT == 0) {
      int lo = 0, hi = E;                 // largest g with s_pref[g] <= T
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= T) lo = mid; else hi = mid;
      }
      const int start = lo == 0 ? 0 : s_end[lo - 1];
      first = start + (T - s_pref[lo]) * kRows;
      valid = s_end[lo] - first;
    } else {
      const int64_t e = T / tpe;
      const int64_t r0 = (T - e * tpe) * kRows;
      first = e * rows + r0;
      int64_t active = rows;
      if constexpr (LAYOUT == 1) {
        int64_t a = groups[e];
        a = a < 0 ? 0 : a;
        active = a < rows ? a : rows;
      }
      valid = active - r0;
    }
    if constexpr (VEC) {
      const int nvalid = valid < 0 ? 0 : (valid > kRows ? kRows : (int)valid);
      const int q4 = 4 * (tid & 7);
      const float* srcf = reinterpret_cast<const float*>(src);
      for (int kc = 0; kc < kblocks; kc += kChunk) {
        const int nk = kblocks - kc < kChunk ? kblocks - kc : kChunk;
#pragma unroll 8
        for (int r = tid >> 3; r < kRows; r += kThreads / 8) {
          u32x4s v = {0u, 0u, 0u, 0u};
          const bool live = q4 < nk && r < nvalid;
          if (live) v = *reinterpret_cast<const u32x4s*>(srcf + (first + r) * ld_src + kc + q4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (live) bad += (v[i] & 0x807FFFFFu) != 0u;
            if (q4 < nk) s_bytes[(q4 + i) * kPitch + r] = (uint8_t)((v[i] >> 23) & 0xFFu);
          }
        }
        __syncthreads();
        for (int kb = kb0; kb < nk; kb += 4) {
          uint32_t word = 0;
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const int r = 128 * (d >> 5) + (d & 31) + 32 * b;
            word |= (uint32_t)s_bytes[kb * kPitch + r] << (8 * b);
          }
          reinterpret_cast<uint32_t*>(dst + (T * kblocks + kc + kb) * kRows)[d] = word;
        }
        __syncthreads();
      }
    } else {
      for (int kb = kb0; kb < kblocks; kb += 4) {
        uint32_t word = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int r = 128 * (d >> 5) + (d & 31) + 32 * b;
          if (r < valid) word |= e8m0<SRC_F32>(src, (first + r) * ld_src + kb, bad) << (8 * b);
        }
        reinterpret_cast<uint32_t*>(dst + (T * kblocks + kb) * kRows)[d] = word;
      }
    }
  }
  if (bad_count) {
    if (bad) atomicAdd(&s_bad, bad);
    __syncthreads();
    if (tid == 0 && s_bad) atomicAdd(bad_count, s_bad);
  }
}

template <int LAYOUT>
hipError_t launch_layout(bool src_f32, const void* src, int64_t ld_src, const int32_t* groups,
                         int64_t rows, int32_t kblocks, int32_t E, int64_t tiles, uint8_t* dst,
                         int32_t* bad, int num_cus, hipStream_t stream) {
  const int64_t want = tiles < 4 * (int64_t)num_cus ? tiles : 4 * (int64_t)num_cus;
  const int grid = (int)(want > 0 ? want : 1);
  const bool vec = src_f32 && ld_src % 4 == 0 && kblocks % 4 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0;
  if (vec)
    return launch_kernel(pack_scales_kernel<LAYOUT, true, true>, dim3(grid), dim3(kThreads), stream, src,
                         ld_src, groups, rows, kblocks, E, tiles, dst, bad);
  if (src_f32)
    return launch_kernel(pack_scales_kernel<LAYOUT, true, false>, dim3(grid), dim3(kThreads), stream, src,
                         ld_src, groups, rows, kblocks, E, tiles, dst, bad);
  return launch_kernel(pack_scales_kernel<LAYOUT, false, false>, dim3(grid), dim3(kThreads), stream, src,
                       ld_src, groups, rows, kblocks, E, tiles, dst, bad);
}

}  // namespace

int64_t fp8_scale_tiles(int layout, int64_t rows, int32_t num_groups) {
  const int64_t t = (rows + kRows - 1) / kRows;
  return layout == 0 ? t + num_groups : t * num_groups;
}

hipError_t launch_pack_scales(int layout, bool src_f32, const void* src, int64_t ld_src,
                              const int32_t* groups, int64_t rows, int32_t kblocks, int32_t num_groups,
                              uint8_t* dst, int32_t* bad, int num_cus, hipStream_t stream) {
  const int64_t tiles = fp8_scale_tiles(layout, rows, num_groups);
  switch (layout) {
    case 0: return launch_layout<0>(src_f32, src, ld_src, groups, rows, kblocks, num_groups, tiles, dst,
                                    bad, num_cus, stream);
    case 1: return launch_layout<1>(src_f32, src, ld_src, groups, rows, kblocks, num_groups, tiles, dst,
                                    bad, num_cus, stream);
    default: return launch_layout<2>(src_f32, src, ld_src, groups, rows, kblocks, num_groups, tiles, dst,
                                     bad, num_cus, stream);
  }
}

}  // namespace gg
