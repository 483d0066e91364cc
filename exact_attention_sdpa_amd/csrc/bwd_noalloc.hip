// Allocation-free variant of sdpa_bwd: the row dots D_i = <dO_i, O_i> that
// sdpa_bwd keeps in the caller's workspace live in a file-scope device
// array instead, so the call needs neither a workspace argument nor any
// allocation.  Each device the library runs on holds its own copy of the
// array (SDPA_BWD_NOALLOC_MAX_ROWS floats) until the process ends.
#include <atomic>
#include <mutex>

#include "sdpa_internal.h"

namespace {

static __device__ __align__(256) float scratch[SDPA_BWD_NOALLOC_MAX_ROWS];

constexpr int kMaxDevices = 64;
// per device: the array's device address, found once with the device current
std::atomic<float*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, or null.  In host code
// `scratch` names a host-side stand-in, never the device memory, so only
// this address may be passed to kernels.
float* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  float* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (p == nullptr) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr)
      return nullptr;
    p = static_cast<float*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

sdpa_status sdpa_bwd_noalloc(const void* q, const void* k, const void* v, const void* out,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                             float scale, int is_causal, sdpa_dtype dtype, sdpa_dtype out_dtype,
                             sdpa_dtype grad_dtype, void* stream) {
  if (B < 1 || H < 1 || Nq < 1) return SDPA_ERR_INVALID;
  const int64_t bytes = sdpa_bwd_workspace_bytes(B, H, Nq);
  if (bytes < 0) return SDPA_ERR_INVALID;
  if (bytes > (int64_t)sizeof(float) * SDPA_BWD_NOALLOC_MAX_ROWS) return SDPA_ERR_UNSUPPORTED;
  if (!sdpa::current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  float* work = scratch_on_current_device();
  if (work == nullptr) return SDPA_ERR_DEVICE;
  sdpa::BwdArgs a;
  const sdpa_status st =
      sdpa::validate_bwd(q, k, v, out, dout, lse, dq, dk, dv, work, B, H, Nq, Nk, d, scale,
                         is_causal, dtype, out_dtype, grad_dtype, stream, &a);
  if (st != SDPA_OK) return st;
  // the dQ kernel writes every D_i before the dK/dV kernel, launched after
  // it, reads it, so nothing needs clearing
  const hipError_t e =
      dtype == SDPA_BF16 ? sdpa::launch_bwd_mfma_bf16(a) : sdpa::launch_bwd_mfma_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

}  // extern "C"
