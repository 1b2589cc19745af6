// gg_api.hip -- the C ABI of include/gg.h: argument checks on the host, then
// one kernel launch on the caller's stream.  Nothing here allocates device
// memory, copies device -> host or synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstdio>
#include <mutex>
#include <string>

#include "gg.h"
#include "gg_internal.h"

static_assert(GG_MAX_GROUPS == GG_MAX_GROUPS_DEV, "group limit mismatch");

namespace {

thread_local std::string g_last_error;

gg_status fail(gg_status s, const char* what) {
  g_last_error = what;
  return s;
}

// Compute-unit count per device, read once (a device attribute query; no
// allocation, no synchronisation).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

gg_status device_cus(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_error = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return GG_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(GG_ERR_HIP, "device ordinal out of range");
  int cus = g_cus[dev].load(std::memory_order_relaxed);
  if (cus <= 0) {
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess || cus <= 0) {
      g_last_error = std::string("hipDeviceGetAttribute: ") + hipGetErrorString(e);
      return GG_ERR_HIP;
    }
    g_cus[dev].store(cus, std::memory_order_relaxed);
  }
  *out = cus;
  return GG_OK;
}

constexpr int64_t kRowLimit = (int64_t(1) << 31) - (int64_t(1) << 16);

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared checks.  rows = m (ragged) or max_m (masked).
gg_status check(const void* p0, const void* p1, const void* groups, const void* out, gg_dtype dt,
                int64_t rows, int64_t k, int64_t n, int32_t E) {
  if (!p0 || !p1 || !groups || !out) return fail(GG_ERR_NULL_PTR, "a required pointer is NULL");
  if (dt != GG_BF16 && dt != GG_F32) return fail(GG_ERR_BAD_DTYPE, "output dtype must be GG_BF16 or GG_F32");
  if (E < 1 || E > GG_MAX_GROUPS) return fail(GG_ERR_LIMIT, "num_groups must be in [1, GG_MAX_GROUPS]");
  if (rows < 0 || k < 8 || n < 8) return fail(GG_ERR_BAD_DIM, "need m >= 0, k >= 8, n >= 8");
  if (k % 8 != 0 || n % 8 != 0) return fail(GG_ERR_BAD_DIM, "k and n must be multiples of 8");
  // Row indices and reduction lengths are int32 on the device; element
  // offsets are int64.  Keep every count comfortably inside both.
  // (2^16 below 2^31, so that a row count plus a tile or a few stages of
  // reduction rows still fits an int32 on the device)
  if (rows >= kRowLimit) return fail(GG_ERR_BAD_DIM, "row count must be below 2^31 - 2^16");
  // Per-tile byte offsets are 32-bit: 256 rows of k or n fp32 values must
  // stay below 2^31 bytes.
  if (k > GG_MAX_KN || n > GG_MAX_KN) return fail(GG_ERR_BAD_DIM, "k and n must not exceed GG_MAX_KN");
  // A weight operand is read down its rows through one 32-bit buffer range
  // per stage that runs to its last row: one expert's k x n bf16 matrix
  // must stay below 2^32 bytes.
  if (k * n >= (int64_t(1) << 31))
    return fail(GG_ERR_BAD_DIM, "k * n must be below 2^31 (each expert's weights under 4 GiB)");
  if ((double)(rows + E) * (double)(k > n ? k : n) * 4.0 > 4.0e18)
    return fail(GG_ERR_BAD_DIM, "problem too large");
  if (!aligned16(p0) || !aligned16(p1) || !aligned16(out) || !aligned16(groups))
    return fail(GG_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
  return GG_OK;
}

gg_status run(int mode, const void* a, const void* b, const int32_t* groups, void* c, gg_dtype dt,
              int64_t m, int64_t k, int64_t n, int32_t E, float alpha, float beta, void* stream,
              const void* bias = nullptr, const float* bias_scale = nullptr) {
  int cus = 0;
  gg_status s = device_cus(&cus);
  if (s != GG_OK) return s;
  hipError_t e = gg::launch(mode, a, b, groups, c, dt == GG_F32, m, k, n, E, alpha, beta, bias, bias_scale, cus,
                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = std::string("kernel launch: ") + hipGetErrorString(e);
    return GG_ERR_HIP;
  }
  g_last_error.clear();
  return GG_OK;
}

gg_status masked_rows(int64_t max_m, int32_t E) {
  if ((double)E * (double)max_m >= (double)kRowLimit)
    return fail(GG_ERR_BAD_DIM, "num_groups * max_m must be below 2^31 - 2^16");
  return GG_OK;
}

}  // namespace

extern "C" {

gg_status gg_forward_ex(const void* x, const void* w, const int32_t* offs, void* y, gg_dtype y_dtype,
                        int64_t m, int64_t k, int64_t n, int32_t num_groups, float alpha,
                        float beta, void* stream) {
  gg_status s = check(x, w, offs, y, y_dtype, m, k, n, num_groups);
  if (s != GG_OK) return s;
  return run(0, x, w, offs, y, y_dtype, m, k, n, num_groups, alpha, beta, stream);
}

gg_status gg_dgrad_ex(const void* dy, const void* w, const int32_t* offs, void* dx, gg_dtype dx_dtype,
                      int64_t m, int64_t k, int64_t n, int32_t num_groups, float alpha, float beta,
                      void* stream) {
  gg_status s = check(dy, w, offs, dx, dx_dtype, m, k, n, num_groups);
  if (s != GG_OK) return s;
  return run(1, dy, w, offs, dx, dx_dtype, m, k, n, num_groups, alpha, beta, stream);
}

gg_status gg_wgrad_ex(const void* x, const void* dy, const int32_t* offs, void* dw, gg_dtype dw_dtype,
                      int64_t m, int64_t k, int64_t n, int32_t num_groups, float alpha, float beta,
                      void* stream) {
  gg_status s = check(x, dy, offs, dw, dw_dtype, m, k, n, num_groups);
  if (s != GG_OK) return s;
  return run(2, x, dy, offs, dw, dw_dtype, m, k, n, num_groups, alpha, beta, stream);
}

gg_status gg_masked_forward_ex(const void* x, const void* w, const int32_t* masked_m, void* y,
                               gg_dtype y_dtype, int64_t max_m, int64_t k, int64_t n,
                               int32_t num_groups, float alpha, float beta, void* stream) {
  gg_status s = check(x, w, masked_m, y, y_dtype, max_m, k, n, num_groups);
  if (s != GG_OK) return s;
  s = masked_rows(max_m, num_groups);
  if (s != GG_OK) return s;
  return run(3, x, w, masked_m, y, y_dtype, max_m, k, n, num_groups, alpha, beta, stream);
}

gg_status gg_masked_dgrad_ex(const void* dy, const void* w, const int32_t* masked_m, void* dx,
                             gg_dtype dx_dtype, int64_t max_m, int64_t k, int64_t n,
                             int32_t num_groups, float alpha, float beta, void* stream) {
  gg_status s = check(dy, w, masked_m, dx, dx_dtype, max_m, k, n, num_groups);
  if (s != GG_OK) return s;
  s = masked_rows(max_m, num_groups);
  if (s != GG_OK) return s;
  return run(4, dy, w, masked_m, dx, dx_dtype, max_m, k, n, num_groups, alpha, beta, stream);
}

gg_status gg_masked_wgrad_ex(const void* x, const void* dy, const int32_t* masked_m, void* dw,
                             gg_dtype dw_dtype, int64_t max_m, int64_t k, int64_t n,
                             int32_t num_groups, float alpha, float beta, void* stream) {
  gg_status s = check(x, dy, masked_m, dw, dw_dtype, max_m, k, n, num_groups);
  if (s != GG_OK) return s;
  s = masked_rows(max_m, num_groups);
  if (s != GG_OK) return s;
  return run(5, x, dy, masked_m, dw, dw_dtype, max_m, k, n, num_groups, alpha, beta, stream);
}

gg_status gg_masked_dgrad(const void* dy, const void* w, const int32_t* masked_m, void* dx,
                          gg_dtype dx_dtype, int64_t max_m, int64_t k, int64_t n,
                          int32_t num_groups, void* stream) {
  return gg_masked_dgrad_ex(dy, w, masked_m, dx, dx_dtype, max_m, k, n, num_groups, 1.0f, 0.0f,
                            stream);
}

gg_status gg_masked_wgrad(const void* x, const void* dy, const int32_t* masked_m, void* dw,
                          gg_dtype dw_dtype, int64_t max_m, int64_t k, int64_t n,
                          int32_t num_groups, void* stream) {
  return gg_masked_wgrad_ex(x, dy, masked_m, dw, dw_dtype, max_m, k, n, num_groups, 1.0f, 0.0f,
                            stream);
}

gg_status gg_forward_silu_mul(const void* x, const void* w13, const int32_t* offs, void* out,
                              gg_dtype out_dtype, int64_t m, int64_t k, int64_t n,
                              int32_t num_groups, void* stream) {
  gg_status s = check(x, w13, offs, out, out_dtype, m, k, n, num_groups);
  if (s != GG_OK) return s;
  if (n % 16 != 0) return fail(GG_ERR_BAD_DIM, "n (= 2 I) must be a multiple of 16");
  return run(6, x, w13, offs, out, out_dtype, m, k, n, num_groups, 1.0f, 0.0f, stream);
}

gg_status gg_masked_forward_silu_mul(const void* x, const void* w13, const int32_t* masked_m,
                                     void* out, gg_dtype out_dtype, int64_t max_m, int64_t k,
                                     int64_t n, int32_t num_groups, void* stream) {
  gg_status s = check(x, w13, masked_m, out, out_dtype, max_m, k, n, num_groups);
  if (s != GG_OK) return s;
  if (n % 16 != 0) return fail(GG_ERR_BAD_DIM, "n (= 2 I) must be a multiple of 16");
  s = masked_rows(max_m, num_groups);
  if (s != GG_OK) return s;
  return run(7, x, w13, masked_m, out, out_dtype, max_m, k, n, num_groups, 1.0f, 0.0f, stream);
}

gg_status gg_forward(const void* x, const void* w, const int32_t* offs, void* y, gg_dtype y_dtype,
                     int64_t m, int64_t k, int64_t n, int32_t num_groups, void* stream) {
  return gg_forward_ex(x, w, offs, y, y_dtype, m, k, n, num_groups, 1.0f, 0.0f, stream);
}

gg_status gg_dgrad(const void* dy, const void* w, const int32_t* offs, void* dx, gg_dtype dx_dtype,
                   int64_t m, int64_t k, int64_t n, int32_t num_groups, void* stream) {
  return gg_dgrad_ex(dy, w, offs, dx, dx_dtype, m, k, n, num_groups, 1.0f, 0.0f, stream);
}

gg_status gg_wgrad(const void* x, const void* dy, const int32_t* offs, void* dw, gg_dtype dw_dtype,
                   int64_t m, int64_t k, int64_t n, int32_t num_groups, void* stream) {
  return gg_wgrad_ex(x, dy, offs, dw, dw_dtype, m, k, n, num_groups, 1.0f, 0.0f, stream);
}

gg_status gg_masked_forward(const void* x, const void* w, const int32_t* masked_m, void* y,
                            gg_dtype y_dtype, int64_t max_m, int64_t k, int64_t n,
                            int32_t num_groups, void* stream) {
  return gg_masked_forward_ex(x, w, masked_m, y, y_dtype, max_m, k, n, num_groups, 1.0f, 0.0f,
                              stream);
}

// The [E, N, K] weight layout runs the [E, K, N] kernels with the roles of
// the dimensions exchanged: y = x W[g]^T is the dgrad form (x as its "dy",
// k as its n), dx = dy W[g] with W[g] [n, k] the forward form, dW[g]^T =
// dy^T x the wgrad form with its operands swapped, and the masked forward
// the masked dgrad form.
gg_status gg_forward_nk_ex(const void* x, const void* w, const int32_t* offs, void* y, gg_dtype y_dtype,
                           int64_t m, int64_t k, int64_t n, int32_t num_groups, float alpha, float beta,
                           void* stream) {
  gg_status s = check(x, w, offs, y, y_dtype, m, k, n, num_groups);
  if (s != GG_OK) return s;
  return run(1, x, w, offs, y, y_dtype, m, n, k, num_groups, alpha, beta, stream);
}

gg_status gg_dgrad_nk_ex(const void* dy, const void* w, const int32_t* offs, void* dx, gg_dtype dx_dtype,
                         int64_t m, int64_t k, int64_t n, int32_t num_groups, float alpha, float beta,
                         void* stream) {
  gg_status s = check(dy, w, offs, dx, dx_dtype, m, k, n, num_groups);
  if (s != GG_OK) return s;
  return run(0, dy, w, offs, dx, dx_dtype, m, n, k, num_groups, alpha, beta, stream);
}

gg_status gg_wgrad_nk_ex(const void* x, const void* dy, const int32_t* offs, void* dw, gg_dtype dw_dtype,
                         int64_t m, int64_t k, int64_t n, int32_t num_groups, float alpha, float beta,
                         void* stream) {
  gg_status s = check(x, dy, offs, dw, dw_dtype, m, k, n, num_groups);
  if (s != GG_OK) return s;
  return run(2, dy, x, offs, dw, dw_dtype, m, n, k, num_groups, alpha, beta, stream);
}

gg_status gg_masked_forward_nk_ex(const void* x, const void* w, const int32_t* masked_m, void* y,
                                  gg_dtype y_dtype, int64_t max_m, int64_t k, int64_t n,
                                  int32_t num_groups, float alpha, float beta, void* stream) {
  gg_status s = check(x, w, masked_m, y, y_dtype, max_m, k, n, num_groups);
  if (s != GG_OK) return s;
  s = masked_rows(max_m, num_groups);
  if (s != GG_OK) return s;
  return run(4, x, w, masked_m, y, y_dtype, max_m, n, k, num_groups, alpha, beta, stream);
}

gg_status gg_forward_nk(const void* x, const void* w, const int32_t* offs, void* y, gg_dtype y_dtype,
                        int64_t m, int64_t k, int64_t n, int32_t num_groups, void* stream) {
  return gg_forward_nk_ex(x, w, offs, y, y_dtype, m, k, n, num_groups, 1.0f, 0.0f, stream);
}

gg_status gg_dgrad_nk(const void* dy, const void* w, const int32_t* offs, void* dx, gg_dtype dx_dtype,
                      int64_t m, int64_t k, int64_t n, int32_t num_groups, void* stream) {
  return gg_dgrad_nk_ex(dy, w, offs, dx, dx_dtype, m, k, n, num_groups, 1.0f, 0.0f, stream);
}

gg_status gg_wgrad_nk(const void* x, const void* dy, const int32_t* offs, void* dw, gg_dtype dw_dtype,
                      int64_t m, int64_t k, int64_t n, int32_t num_groups, void* stream) {
  return gg_wgrad_nk_ex(x, dy, offs, dw, dw_dtype, m, k, n, num_groups, 1.0f, 0.0f, stream);
}

gg_status gg_masked_forward_nk(const void* x, const void* w, const int32_t* masked_m, void* y,
                               gg_dtype y_dtype, int64_t max_m, int64_t k, int64_t n, int32_t num_groups,
                               void* stream) {
  return gg_masked_forward_nk_ex(x, w, masked_m, y, y_dtype, max_m, k, n, num_groups, 1.0f, 0.0f, stream);
}

static gg_status bias_args(const void* bias, const float* bias_scale) {
  if (!bias) return fail(GG_ERR_NULL_PTR, "bias is NULL");
  if (!aligned16(bias) || (reinterpret_cast<uintptr_t>(bias_scale) & 3u))
    return fail(GG_ERR_ALIGNMENT, "bias must be 16-byte aligned and bias_scale 4-byte aligned");
  return GG_OK;
}

gg_status gg_forward_bias(const void* x, const void* w, const int32_t* offs, const void* bias,
                          const float* bias_scale, void* y, gg_dtype y_dtype, int64_t m, int64_t k, int64_t n,
                          int32_t num_groups, float alpha, float beta, void* stream) {
  gg_status s = check(x, w, offs, y, y_dtype, m, k, n, num_groups);
  if (s != GG_OK) return s;
  s = bias_args(bias, bias_scale);
  if (s != GG_OK) return s;
  return run(0, x, w, offs, y, y_dtype, m, k, n, num_groups, alpha, beta, stream, bias, bias_scale);
}

gg_status gg_masked_forward_bias(const void* x, const void* w, const int32_t* masked_m, const void* bias,
                                 const float* bias_scale, void* y, gg_dtype y_dtype, int64_t max_m, int64_t k,
                                 int64_t n, int32_t num_groups, float alpha, float beta, void* stream) {
  gg_status s = check(x, w, masked_m, y, y_dtype, max_m, k, n, num_groups);
  if (s != GG_OK) return s;
  s = masked_rows(max_m, num_groups);
  if (s != GG_OK) return s;
  s = bias_args(bias, bias_scale);
  if (s != GG_OK) return s;
  return run(3, x, w, masked_m, y, y_dtype, max_m, k, n, num_groups, alpha, beta, stream, bias, bias_scale);
}

static gg_status hip_result(hipError_t e) {
  if (e != hipSuccess) {
    g_last_error = std::string("kernel launch: ") + hipGetErrorString(e);
    return GG_ERR_HIP;
  }
  g_last_error.clear();
  return GG_OK;
}

static bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

constexpr int32_t kMaxAlignment = 4096;

gg_status gg_offsets_from_splits(const int64_t* m_splits, int32_t num_groups, int32_t min_alignment,
                                 int pad_empty, int32_t* offs, void* stream) {
  if (!m_splits || !offs) return fail(GG_ERR_NULL_PTR, "a required pointer is NULL");
  if (num_groups < 1 || num_groups > GG_MAX_GROUPS) return fail(GG_ERR_LIMIT, "num_groups must be in [1, GG_MAX_GROUPS]");
  if (min_alignment < 1 || min_alignment > kMaxAlignment)
    return fail(GG_ERR_BAD_DIM, "min_alignment must be in [1, 4096]");
  if ((reinterpret_cast<uintptr_t>(m_splits) & 7u) || !aligned4(offs))
    return fail(GG_ERR_ALIGNMENT, "m_splits must be 8-byte and offs 4-byte aligned");
  return hip_result(gg::launch_offsets_from_splits(m_splits, num_groups, min_alignment, pad_empty != 0, offs,
                                                   static_cast<hipStream_t>(stream)));
}

int64_t gg_route_rows_bound(int64_t slots, int32_t num_groups, int32_t min_alignment) {
  if (slots < 0 || num_groups < 1 || num_groups > GG_MAX_GROUPS || min_alignment < 1 ||
      min_alignment > kMaxAlignment)
    return -1;
  return slots + (int64_t)num_groups * min_alignment;
}

int64_t gg_route_workspace_bytes(int64_t slots, int32_t num_groups) {
  if (slots < 0 || num_groups < 1 || num_groups > GG_MAX_GROUPS) return -1;
  const int64_t b = gg::route_blocks(slots);
  return (b > 0 ? b : 1) * (int64_t)num_groups * 4;
}

gg_status gg_route(const int32_t* expert_of_slot, int64_t slots, int32_t num_groups, int32_t min_alignment,
                   int pad_empty, int32_t* offs, int32_t* row_slot, int64_t rows_cap, int32_t* slot_row,
                   void* workspace, void* stream) {
  if (!offs || !row_slot || !workspace || (slots > 0 && (!expert_of_slot || !slot_row)))
    return fail(GG_ERR_NULL_PTR, "a required pointer is NULL");
  if (num_groups < 1 || num_groups > GG_MAX_GROUPS) return fail(GG_ERR_LIMIT, "num_groups must be in [1, GG_MAX_GROUPS]");
  if (min_alignment < 1 || min_alignment > kMaxAlignment)
    return fail(GG_ERR_BAD_DIM, "min_alignment must be in [1, 4096]");
  if (slots < 0) return fail(GG_ERR_BAD_DIM, "slots must be >= 0");
  const int64_t bound = gg_route_rows_bound(slots, num_groups, min_alignment);
  // the rows it produces must be acceptable to the GEMMs (and fit int32)
  if (bound >= kRowLimit)
    return fail(GG_ERR_BAD_DIM, "slots + num_groups * min_alignment must be below 2^31 - 2^16");
  if (rows_cap < bound) return fail(GG_ERR_BAD_DIM, "rows_cap is below gg_route_rows_bound");
  if (!aligned4(expert_of_slot) || !aligned4(offs) || !aligned4(row_slot) || !aligned4(slot_row) ||
      !aligned16(workspace))
    return fail(GG_ERR_ALIGNMENT, "int32 arrays must be 4-byte aligned, workspace 16-byte aligned");
  return hip_result(gg::launch_route(expert_of_slot, slots, num_groups, min_alignment, pad_empty != 0, offs,
                                     row_slot, slot_row, static_cast<int32_t*>(workspace),
                                     static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---- routing without a workspace argument (gg_route_noalloc) -----------------------
//
// The route histograms live in this array instead of a caller's workspace:
// one copy per GPU, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not the device memory: the device address is
// taken once per device with hipGetSymbolAddress (that device current) and
// only that address is ever passed to a kernel.
static __device__ __align__(256) int32_t scratch[GG_ROUTE_NOALLOC_SCRATCH_BYTES / 4];

namespace {

constexpr int64_t kNoAllocScratchBytes = GG_ROUTE_NOALLOC_SCRATCH_BYTES;

std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices];   // per device, set once under g_scratch_mu

gg_status scratch_for_current_device(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_error = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return GG_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(GG_ERR_HIP, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_error = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return GG_ERR_HIP;
    }
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return GG_OK;
}

}  // namespace

extern "C" {

gg_status gg_route_noalloc(const int32_t* expert_of_slot, int64_t slots, int32_t num_groups,
                           int32_t min_alignment, int pad_empty, int32_t* offs, int32_t* row_slot,
                           int64_t rows_cap, int32_t* slot_row, void* stream) {
  if (!offs || !row_slot || (slots > 0 && (!expert_of_slot || !slot_row)))
    return fail(GG_ERR_NULL_PTR, "a required pointer is NULL");
  if (num_groups < 1 || num_groups > GG_MAX_GROUPS) return fail(GG_ERR_LIMIT, "num_groups must be in [1, GG_MAX_GROUPS]");
  if (min_alignment < 1 || min_alignment > kMaxAlignment)
    return fail(GG_ERR_BAD_DIM, "min_alignment must be in [1, 4096]");
  if (slots < 0) return fail(GG_ERR_BAD_DIM, "slots must be >= 0");
  const int64_t bound = gg_route_rows_bound(slots, num_groups, min_alignment);
  if (bound >= kRowLimit)
    return fail(GG_ERR_BAD_DIM, "slots + num_groups * min_alignment must be below 2^31 - 2^16");
  if (rows_cap < bound) return fail(GG_ERR_BAD_DIM, "rows_cap is below gg_route_rows_bound");
  if (gg_route_workspace_bytes(slots, num_groups) > kNoAllocScratchBytes)
    return fail(GG_ERR_LIMIT, "the route histograms exceed GG_ROUTE_NOALLOC_SCRATCH_BYTES; use gg_route");
  if (!aligned4(expert_of_slot) || !aligned4(offs) || !aligned4(row_slot) || !aligned4(slot_row))
    return fail(GG_ERR_ALIGNMENT, "int32 arrays must be 4-byte aligned");
  int32_t* hist = nullptr;
  const gg_status s = scratch_for_current_device(&hist);
  if (s != GG_OK) return s;
  return hip_result(gg::launch_route(expert_of_slot, slots, num_groups, min_alignment, pad_empty != 0, offs,
                                     row_slot, slot_row, hist, static_cast<hipStream_t>(stream)));
}

gg_status gg_gather_rows(const void* src, int64_t tokens, int64_t row_bytes, const int32_t* row_slot,
                         int32_t topk, const int32_t* offs, int32_t num_groups, int64_t rows_cap, void* dst,
                         void* stream) {
  if (!src || !row_slot || !offs || !dst) return fail(GG_ERR_NULL_PTR, "a required pointer is NULL");
  if (num_groups < 1 || num_groups > GG_MAX_GROUPS) return fail(GG_ERR_LIMIT, "num_groups must be in [1, GG_MAX_GROUPS]");
  if (tokens < 0 || rows_cap < 0 || topk < 1 || row_bytes < 16 || row_bytes % 16 != 0)
    return fail(GG_ERR_BAD_DIM, "need tokens, rows_cap >= 0, topk >= 1, row_bytes a positive multiple of 16");
  if (rows_cap >= kRowLimit || tokens * (int64_t)topk >= kRowLimit)
    return fail(GG_ERR_BAD_DIM, "row and slot counts must be below 2^31 - 2^16");
  if (!aligned16(src) || !aligned16(dst) || !aligned4(row_slot) || !aligned4(offs))
    return fail(GG_ERR_ALIGNMENT, "src and dst must be 16-byte aligned");
  int cus = 0;
  gg_status s = device_cus(&cus);
  if (s != GG_OK) return s;
  return hip_result(gg::launch_gather_rows(src, row_bytes, row_slot, topk, offs, num_groups, rows_cap, tokens,
                                           dst, cus, static_cast<hipStream_t>(stream)));
}

gg_status gg_combine_rows(const void* y, int64_t n, const int32_t* slot_row, const float* weights, int32_t topk,
                          int64_t tokens, int64_t rows_cap, void* out, gg_dtype out_dtype, void* stream) {
  if (!y || !slot_row || !out) return fail(GG_ERR_NULL_PTR, "a required pointer is NULL");
  if (out_dtype != GG_BF16 && out_dtype != GG_F32) return fail(GG_ERR_BAD_DTYPE, "output dtype must be GG_BF16 or GG_F32");
  if (n < 8 || n % 8 != 0 || tokens < 0 || topk < 1 || rows_cap < 0)
    return fail(GG_ERR_BAD_DIM, "need n a positive multiple of 8, tokens, rows_cap >= 0, topk >= 1");
  if (rows_cap >= kRowLimit || tokens * (int64_t)topk >= kRowLimit)
    return fail(GG_ERR_BAD_DIM, "row and slot counts must be below 2^31 - 2^16");
  if (!aligned16(y) || !aligned16(out) || !aligned4(slot_row) || !aligned4(weights))
    return fail(GG_ERR_ALIGNMENT, "y and out must be 16-byte aligned");
  int cus = 0;
  gg_status s = device_cus(&cus);
  if (s != GG_OK) return s;
  return hip_result(gg::launch_combine_rows(y, n, slot_row, weights, topk, tokens, rows_cap, out,
                                            out_dtype == GG_F32, cus, static_cast<hipStream_t>(stream)));
}

static gg_status bias_grad_check(const void* dy, const int32_t* groups, const void* out, int64_t rows, int64_t n,
                                 int32_t E, bool masked) {
  if (!dy || !groups || !out) return fail(GG_ERR_NULL_PTR, "a required pointer is NULL");
  if (E < 1 || E > GG_MAX_GROUPS) return fail(GG_ERR_LIMIT, "num_groups must be in [1, GG_MAX_GROUPS]");
  if (rows < 0 || n < 8 || n % 8 != 0 || n > GG_MAX_KN)
    return fail(GG_ERR_BAD_DIM, "need rows >= 0 and n a positive multiple of 8 up to GG_MAX_KN");
  const double total = masked ? (double)rows * E : (double)rows;
  if (total >= (double)kRowLimit) return fail(GG_ERR_BAD_DIM, "row count must be below 2^31 - 2^16");
  if (!aligned16(dy) || !aligned4(groups) || !aligned4(out))
    return fail(GG_ERR_ALIGNMENT, "dy must be 16-byte aligned");
  return GG_OK;
}

gg_status gg_bias_grad(const void* dy, const int32_t* offs, const float* bias_scale, float* dbias, int64_t m,
                       int64_t n, int32_t num_groups, void* stream) {
  gg_status s = bias_grad_check(dy, offs, dbias, m, n, num_groups, false);
  if (s != GG_OK) return s;
  if (!aligned4(bias_scale)) return fail(GG_ERR_ALIGNMENT, "bias_scale must be 4-byte aligned");
  return hip_result(gg::launch_dbias(false, dy, offs, bias_scale, m, n, num_groups, dbias,
                                     static_cast<hipStream_t>(stream)));
}

gg_status gg_masked_bias_grad(const void* dy, const int32_t* masked_m, const float* bias_scale, float* dbias,
                              int64_t max_m, int64_t n, int32_t num_groups, void* stream) {
  gg_status s = bias_grad_check(dy, masked_m, dbias, max_m, n, num_groups, true);
  if (s != GG_OK) return s;
  if (!aligned4(bias_scale)) return fail(GG_ERR_ALIGNMENT, "bias_scale must be 4-byte aligned");
  return hip_result(gg::launch_dbias(true, dy, masked_m, bias_scale, max_m, n, num_groups, dbias,
                                     static_cast<hipStream_t>(stream)));
}

static gg_status dscale_run(bool masked, const void* dy, const int32_t* groups, const void* bias, float* ds,
                            int64_t rows, int64_t n, int32_t E, void* stream) {
  gg_status s = bias_grad_check(dy, groups, ds, rows, n, E, masked);
  if (s != GG_OK) return s;
  if (!bias) return fail(GG_ERR_NULL_PTR, "bias is NULL");
  if (!aligned16(bias)) return fail(GG_ERR_ALIGNMENT, "bias must be 16-byte aligned");
  int cus = 0;
  s = device_cus(&cus);
  if (s != GG_OK) return s;
  return hip_result(gg::launch_dscale(masked, dy, groups, bias, rows, n, E, ds, cus,
                                      static_cast<hipStream_t>(stream)));
}

gg_status gg_bias_scale_grad(const void* dy, const int32_t* offs, const void* bias, float* ds, int64_t m,
                             int64_t n, int32_t num_groups, void* stream) {
  return dscale_run(false, dy, offs, bias, ds, m, n, num_groups, stream);
}

gg_status gg_masked_bias_scale_grad(const void* dy, const int32_t* masked_m, const void* bias, float* ds,
                                    int64_t max_m, int64_t n, int32_t num_groups, void* stream) {
  return dscale_run(true, dy, masked_m, bias, ds, max_m, n, num_groups, stream);
}

int64_t gg_fp8_scale_bytes(gg_fp8_scale_layout layout, int64_t rows, int64_t k, int32_t num_groups) {
  if (layout < GG_FP8_ACT_RAGGED || layout > GG_FP8_WEIGHT) return -1;
  if (rows < 0 || k < 128 || k % 128 != 0 || k > GG_MAX_KN) return -1;
  if (num_groups < 1 || num_groups > GG_MAX_GROUPS) return -1;
  if (rows >= kRowLimit) return -1;
  return gg::fp8_scale_tiles((int)layout, rows, num_groups) * (k / 128) * 256;
}

gg_status gg_fp8_pack_scales(gg_fp8_scale_layout layout, const void* src, int src_is_f32, int64_t ld_src,
                             const int32_t* groups, int64_t rows, int64_t k, int32_t num_groups,
                             void* dst, int32_t* bad_count, void* stream) {
  if (layout < GG_FP8_ACT_RAGGED || layout > GG_FP8_WEIGHT) return fail(GG_ERR_BAD_DIM, "unknown scale layout");
  if (!src || !dst || (layout != GG_FP8_WEIGHT && !groups))
    return fail(GG_ERR_NULL_PTR, "a required pointer is NULL");
  if (num_groups < 1 || num_groups > GG_MAX_GROUPS) return fail(GG_ERR_LIMIT, "num_groups must be in [1, GG_MAX_GROUPS]");
  if (rows < 0 || k < 128 || k % 128 != 0 || k > GG_MAX_KN)
    return fail(GG_ERR_BAD_DIM, "need rows >= 0 and k a positive multiple of 128 up to GG_MAX_KN");
  const int64_t kb = k / 128;
  if (ld_src < kb) return fail(GG_ERR_BAD_DIM, "ld_src must be at least k / 128");
  const double src_rows = layout == GG_FP8_ACT_RAGGED ? (double)rows : (double)rows * num_groups;
  if (src_rows >= (double)kRowLimit) return fail(GG_ERR_BAD_DIM, "row count must be below 2^31 - 2^16");
  if (src_rows * (double)ld_src * 4.0 > 4.0e18) return fail(GG_ERR_BAD_DIM, "problem too large");
  if (!aligned16(dst) || (groups && !aligned16(groups)) || (src_is_f32 && (reinterpret_cast<uintptr_t>(src) & 3u)))
    return fail(GG_ERR_ALIGNMENT, "dst and groups must be 16-byte aligned, fp32 src 4-byte aligned");
  int cus = 0;
  gg_status s = device_cus(&cus);
  if (s != GG_OK) return s;
  hipError_t e = gg::launch_pack_scales((int)layout, src_is_f32 != 0, src, ld_src, groups, rows, (int32_t)kb,
                                        num_groups, static_cast<uint8_t*>(dst), bad_count, cus,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = std::string("kernel launch: ") + hipGetErrorString(e);
    return GG_ERR_HIP;
  }
  g_last_error.clear();
  return GG_OK;
}

static gg_status fp8_run(bool masked, const void* x, const void* xs, const void* w, const void* ws,
                         const int32_t* groups, void* y, gg_dtype y_dtype, int64_t rows, int64_t k,
                         int64_t n, int32_t num_groups, void* stream) {
  gg_status s = check(x, w, groups, y, y_dtype, rows, k, n, num_groups);
  if (s != GG_OK) return s;
  if (!xs || !ws) return fail(GG_ERR_NULL_PTR, "a required pointer is NULL");
  if (k % 128 != 0) return fail(GG_ERR_BAD_DIM, "k must be a multiple of 128 (one scale per 128 values)");
  if (!aligned16(xs) || !aligned16(ws)) return fail(GG_ERR_ALIGNMENT, "pointers must be 16-byte aligned");
  if (masked) {
    s = masked_rows(rows, num_groups);
    if (s != GG_OK) return s;
  }
  int cus = 0;
  s = device_cus(&cus);
  if (s != GG_OK) return s;
  hipError_t e = gg::launch_fp8(masked, x, xs, w, ws, groups, y, y_dtype == GG_F32, rows, k, n, num_groups,
                                cus, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    g_last_error = std::string("kernel launch: ") + hipGetErrorString(e);
    return GG_ERR_HIP;
  }
  g_last_error.clear();
  return GG_OK;
}

gg_status gg_fp8_forward(const void* x, const void* x_scales, const void* w, const void* w_scales,
                         const int32_t* offs, void* y, gg_dtype y_dtype, int64_t m, int64_t k, int64_t n,
                         int32_t num_groups, void* stream) {
  return fp8_run(false, x, x_scales, w, w_scales, offs, y, y_dtype, m, k, n, num_groups, stream);
}

gg_status gg_fp8_masked_forward(const void* x, const void* x_scales, const void* w, const void* w_scales,
                                const int32_t* masked_m, void* y, gg_dtype y_dtype, int64_t max_m, int64_t k,
                                int64_t n, int32_t num_groups, void* stream) {
  return fp8_run(true, x, x_scales, w, w_scales, masked_m, y, y_dtype, max_m, k, n, num_groups, stream);
}

const char* gg_status_str(gg_status s) {
  switch (s) {
    case GG_OK: return "GG_OK";
    case GG_ERR_NULL_PTR: return "GG_ERR_NULL_PTR: a required pointer is NULL";
    case GG_ERR_BAD_DIM: return "GG_ERR_BAD_DIM: invalid dimension";
    case GG_ERR_ALIGNMENT: return "GG_ERR_ALIGNMENT: pointer not 16-byte aligned";
    case GG_ERR_BAD_DTYPE: return "GG_ERR_BAD_DTYPE: unknown output dtype";
    case GG_ERR_LIMIT: return "GG_ERR_LIMIT: num_groups out of range";
    case GG_ERR_HIP: return "GG_ERR_HIP: HIP runtime error";
  }
  return "unknown gg_status";
}

const char* gg_last_error(void) { return g_last_error.c_str(); }

const char* gg_version(void) { return "gg 0.1.0 (gfx950)"; }

}  // extern "C"
