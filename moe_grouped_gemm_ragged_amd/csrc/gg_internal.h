// gg_internal.h -- declarations shared by the host API and the kernel file.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

// Experts per call the device-side decode holds in LDS.  Must equal
// GG_MAX_GROUPS in include/gg.h.
#define GG_MAX_GROUPS_DEV 2048

namespace gg {
// Launches `kernel` and returns the status of this launch itself, not the
// thread's last error: an error that earlier, unrelated HIP work left behind
// is not reported as this call's failure.  Arguments are converted to the
// kernel's parameter types and passed by address, as hipLaunchKernel takes
// them.
template <typename... KArgs, typename... Args, size_t... I>
inline hipError_t launch_kernel_impl(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                                     std::index_sequence<I...>, Args&&... args) {
  std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
  void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1] = {static_cast<void*>(&std::get<I>(vals))...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream);
}

template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                                Args&&... args) {
  static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count differs from the kernel's");
  return launch_kernel_impl(kernel, grid, block, stream, std::index_sequence_for<KArgs...>{},
                            std::forward<Args>(args)...);
}

// mode: 0 forward, 1 dgrad, 2 wgrad, 3 masked forward, 4 masked dgrad,
// 5 masked wgrad, 6 forward with the SiLU-mul activation, 7 masked forward
// with the SiLU-mul activation.  Arguments were
// validated by the caller.  Writes alpha * product + beta * (prior output)
// (the prior output is not read when beta == 0), plus bias_scale[row] *
// bias[expert, col] when bias is non-null (modes 0 and 3 only; bias is
// bf16 [E, output cols], bias_scale fp32 indexed by the output row, null for
// 1).  Launches one persistent grid of at most num_cus workgroups on `stream`.
hipError_t launch(int mode, const void* a, const void* b, const int32_t* groups, void* c,
                  bool out_f32, int64_t m, int64_t k, int64_t n, int32_t num_groups,
                  float alpha, float beta, const void* bias, const float* bias_scale, int num_cus,
                  hipStream_t stream);

// The fp8 (e4m3) block-scaled forward, ragged (groups = end offsets) or
// masked (groups = masked_m, m = max_m): x [rows, k] and w [E, n, k] e4m3,
// sx / sw their scales in the packed layout of gg_fp8_pack_scales, k a
// multiple of 128.  Arguments were validated by the caller.
hipError_t launch_fp8(bool masked, const void* x, const void* sx, const void* w, const void* sw,
                      const int32_t* groups, void* c, bool out_f32, int64_t m, int64_t k, int64_t n,
                      int32_t num_groups, int num_cus, hipStream_t stream);

// Packed fp8 scale tiles for `rows` rows of an operand: layout 0 ragged
// activations (an upper bound: ceil(rows / 256) + num_groups), 1 masked
// activations and 2 weights (num_groups * ceil(rows / 256)).  Each tile
// takes kblocks * 256 bytes.
int64_t fp8_scale_tiles(int layout, int64_t rows, int32_t num_groups);

// Writes the packed scales of one operand (gg_fp8_scales.hip).  src holds
// one scale per (row, k-block) at row * ld_src + kb, fp32 or E8M0 bytes;
// bad (nullable) is incremented by the number of active scales that are
// not UE8M0.
hipError_t launch_pack_scales(int layout, bool src_f32, const void* src, int64_t ld_src,
                              const int32_t* groups, int64_t rows, int32_t kblocks, int32_t num_groups,
                              uint8_t* dst, int32_t* bad, int num_cus, hipStream_t stream);

// Routing and layout steps (gg_route.hip).
int64_t route_blocks(int64_t slots);   // blocks of the route passes; hist holds E * this many ints
hipError_t launch_offsets_from_splits(const int64_t* splits, int32_t E, int32_t align, bool pad_empty,
                                      int32_t* offs, hipStream_t stream);
hipError_t launch_route(const int32_t* expert, int64_t slots, int32_t E, int32_t align, bool pad_empty,
                        int32_t* offs, int32_t* row_slot, int32_t* slot_row, int32_t* hist,
                        hipStream_t stream);
hipError_t launch_gather_rows(const void* src, int64_t row_bytes, const int32_t* row_slot, int32_t topk,
                              const int32_t* offs, int32_t E, int64_t rows_cap, int64_t tokens, void* dst,
                              int num_cus, hipStream_t stream);
hipError_t launch_combine_rows(const void* y, int64_t n, const int32_t* slot_row, const float* w, int32_t topk,
                               int64_t tokens, int64_t rows_cap, void* out, bool out_f32, int num_cus,
                               hipStream_t stream);

// Backward of the grouped bias (gg_bias_grad.hip): dbias fp32 [E, n] and
// the per-row factor's gradient ds fp32 [rows], both from bf16 dY.
hipError_t launch_dbias(bool masked, const void* dy, const int32_t* groups, const float* scale, int64_t m,
                        int64_t n, int32_t E, float* dbias, hipStream_t stream);
hipError_t launch_dscale(bool masked, const void* dy, const int32_t* groups, const void* bias, int64_t m,
                         int64_t n, int32_t E, float* ds, int num_cus, hipStream_t stream);
}  // namespace gg
