// gg_internal.h -- declarations shared by the host API and the kernel file.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Experts per call the device-side decode holds in LDS.  Must equal
// GG_MAX_GROUPS in include/gg.h.
#define GG_MAX_GROUPS_DEV 2048

namespace gg {
// mode: 0 forward, 1 dgrad, 2 wgrad, 3 masked forward, 4 masked dgrad,
// 5 masked wgrad, 6 forward with the SiLU-mul activation, 7 masked forward
// with the SiLU-mul activation.  Arguments were
// validated by the caller.  Writes alpha * product + beta * (prior output)
// (the prior output is not read when beta == 0).  Launches one persistent
// grid of at most num_cus workgroups on `stream`.
hipError_t launch(int mode, const void* a, const void* b, const int32_t* groups, void* c,
                  bool out_f32, int64_t m, int64_t k, int64_t n, int32_t num_groups,
                  float alpha, float beta, int num_cus, hipStream_t stream);
}  // namespace gg
