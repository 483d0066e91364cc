// C-ABI entry points: validation, device check, kernel selection, launch.
#include <atomic>
#include <cstring>

#include "sdpa_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// per device: 0 = not yet checked, 1 = gfx950, 2 = anything else
std::atomic<int> g_arch[kMaxDevices];

}  // namespace

namespace sdpa {

bool current_device_is_gfx950() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  int st = g_arch[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1;
}

}  // namespace sdpa

using sdpa::current_device_is_gfx950;

extern "C" {

sdpa_status sdpa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                     int is_causal, const int32_t* cu_seqlens, sdpa_dtype dtype,
                     sdpa_dtype out_dtype, void* stream) {
  sdpa::FwdArgs a;
  const sdpa_status st = sdpa::validate(q, k, v, out, lse, B, H, Nq, Nk, d, scale, is_causal,
                                        cu_seqlens, dtype, out_dtype, stream, &a);
  if (st != SDPA_OK) return st;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  hipError_t e;
  switch (dtype) {
    case SDPA_F16: e = sdpa::launch_fwd_mfma_f16(a); break;
    case SDPA_BF16: e = sdpa::launch_fwd_mfma_bf16(a); break;
    default: e = sdpa::launch_fwd_f32(a); break;
  }
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

sdpa_status sdpa_fwd_strided(const void* q, const void* k, const void* v, void* out, float* lse,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                             const int64_t* q_strides, const int64_t* kv_strides,
                             const int64_t* out_strides, float scale, int is_causal,
                             sdpa_dtype dtype, sdpa_dtype out_dtype, void* stream) {
  sdpa::FwdArgs a;
  const sdpa_status st = sdpa::validate(q, k, v, out, lse, B, H, Nq, Nk, d, scale, is_causal,
                                        nullptr, dtype, out_dtype, stream, &a, false);
  if (st != SDPA_OK) return st;
  const sdpa_status ss = sdpa::validate_strides(q_strides, kv_strides, out_strides, &a);
  if (ss != SDPA_OK) return ss;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  const hipError_t e =
      dtype == SDPA_BF16 ? sdpa::launch_fwd_mfma_bf16(a) : sdpa::launch_fwd_mfma_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

sdpa_status sdpa_fwd_masked(const void* q, const void* k, const void* v, void* out, float* lse,
                            int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                            const int64_t* q_strides, const int64_t* kv_strides,
                            const int64_t* out_strides, float scale, int is_causal,
                            const void* mask, sdpa_mask_kind mask_kind,
                            const int64_t* mask_strides, sdpa_dtype dtype, sdpa_dtype out_dtype,
                            void* stream) {
  const bool strided = q_strides != nullptr || kv_strides != nullptr || out_strides != nullptr;
  sdpa::FwdArgs a;
  const sdpa_status st = sdpa::validate(q, k, v, out, lse, B, H, Nq, Nk, d, scale, is_causal,
                                        nullptr, dtype, out_dtype, stream, &a, !strided);
  if (st != SDPA_OK) return st;
  if (strided) {
    const sdpa_status ss = sdpa::validate_strides(q_strides, kv_strides, out_strides, &a);
    if (ss != SDPA_OK) return ss;
  }
  const sdpa_status sm = sdpa::validate_attn_mask(mask, mask_kind, mask_strides, &a);
  if (sm != SDPA_OK) return sm;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  const hipError_t e = dtype == SDPA_BF16 ? sdpa::launch_fwd_mfma_masked_bf16(a)
                                          : sdpa::launch_fwd_mfma_masked_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

sdpa_status sdpa_fwd_masked_dropout(const void* q, const void* k, const void* v, void* out,
                                    float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                    int64_t d, const int64_t* q_strides,
                                    const int64_t* kv_strides, const int64_t* out_strides,
                                    float scale, int is_causal, const void* mask,
                                    sdpa_mask_kind mask_kind, const int64_t* mask_strides,
                                    float dropout_p, uint64_t seed, uint32_t offset,
                                    sdpa_dtype dtype, sdpa_dtype out_dtype, void* stream) {
  const bool strided = q_strides != nullptr || kv_strides != nullptr || out_strides != nullptr;
  sdpa::FwdArgs a;
  const sdpa_status st = sdpa::validate(q, k, v, out, lse, B, H, Nq, Nk, d, scale, is_causal,
                                        nullptr, dtype, out_dtype, stream, &a, !strided);
  if (st != SDPA_OK) return st;
  if (strided) {
    const sdpa_status ss = sdpa::validate_strides(q_strides, kv_strides, out_strides, &a);
    if (ss != SDPA_OK) return ss;
  }
  const sdpa_status sm = sdpa::validate_attn_mask(mask, mask_kind, mask_strides, &a);
  if (sm != SDPA_OK) return sm;
  const sdpa_status sd = sdpa::validate_dropout(dropout_p, seed, offset, &a);
  if (sd != SDPA_OK) return sd;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  const hipError_t e = dtype == SDPA_BF16 ? sdpa::launch_fwd_mfma_masked_bf16(a)
                                          : sdpa::launch_fwd_mfma_masked_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

sdpa_status sdpa_fwd_block_sparse(const void* q, const void* k, const void* v, void* out,
                                  float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                  int64_t d, float scale, int is_causal,
                                  const uint8_t* block_mask, int64_t mask_heads, sdpa_dtype dtype,
                                  sdpa_dtype out_dtype, void* stream) {
  sdpa::FwdArgs a;
  const sdpa_status st = sdpa::validate(q, k, v, out, lse, B, H, Nq, Nk, d, scale, is_causal,
                                        nullptr, dtype, out_dtype, stream, &a);
  if (st != SDPA_OK) return st;
  const sdpa_status sm = sdpa::validate_block_mask(block_mask, mask_heads, &a);
  if (sm != SDPA_OK) return sm;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  const hipError_t e =
      dtype == SDPA_BF16 ? sdpa::launch_fwd_mfma_bf16(a) : sdpa::launch_fwd_mfma_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

sdpa_status sdpa_fwd_dropout(const void* q, const void* k, const void* v, void* out, float* lse,
                             int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                             int is_causal, const int32_t* cu_seqlens, float dropout_p,
                             uint64_t seed, uint32_t offset, sdpa_dtype dtype,
                             sdpa_dtype out_dtype, void* stream) {
  sdpa::FwdArgs a;
  const sdpa_status st = sdpa::validate(q, k, v, out, lse, B, H, Nq, Nk, d, scale, is_causal,
                                        cu_seqlens, dtype, out_dtype, stream, &a);
  if (st != SDPA_OK) return st;
  const sdpa_status sd = sdpa::validate_dropout(dropout_p, seed, offset, &a);
  if (sd != SDPA_OK) return sd;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  const hipError_t e =
      dtype == SDPA_BF16 ? sdpa::launch_fwd_mfma_bf16(a) : sdpa::launch_fwd_mfma_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

sdpa_status sdpa_bwd(const void* q, const void* k, const void* v, const void* out,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     float* workspace, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                     float scale, int is_causal, sdpa_dtype dtype, sdpa_dtype out_dtype,
                     sdpa_dtype grad_dtype, void* stream) {
  sdpa::BwdArgs a;
  const sdpa_status st =
      sdpa::validate_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale,
                         is_causal, dtype, out_dtype, grad_dtype, stream, &a);
  if (st != SDPA_OK) return st;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  const hipError_t e =
      dtype == SDPA_BF16 ? sdpa::launch_bwd_mfma_bf16(a) : sdpa::launch_bwd_mfma_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

sdpa_status sdpa_bwd_dropout(const void* q, const void* k, const void* v, const void* out,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             float* workspace, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                             int64_t d, float scale, int is_causal, float dropout_p,
                             uint64_t seed, uint32_t offset, sdpa_dtype dtype,
                             sdpa_dtype out_dtype, sdpa_dtype grad_dtype, void* stream) {
  sdpa::BwdArgs a;
  const sdpa_status st =
      sdpa::validate_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale,
                         is_causal, dtype, out_dtype, grad_dtype, stream, &a);
  if (st != SDPA_OK) return st;
  const sdpa_status sd = sdpa::validate_bwd_dropout(dropout_p, seed, offset, &a);
  if (sd != SDPA_OK) return sd;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  const hipError_t e =
      dtype == SDPA_BF16 ? sdpa::launch_bwd_mfma_bf16(a) : sdpa::launch_bwd_mfma_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

sdpa_status sdpa_bwd_masked(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            float* workspace, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                            int64_t d, float scale, int is_causal, const void* mask,
                            sdpa_mask_kind mask_kind, const int64_t* mask_strides,
                            sdpa_dtype dtype, sdpa_dtype out_dtype, sdpa_dtype grad_dtype,
                            void* stream) {
  sdpa::BwdArgs a;
  const sdpa_status st =
      sdpa::validate_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale,
                         is_causal, dtype, out_dtype, grad_dtype, stream, &a);
  if (st != SDPA_OK) return st;
  const sdpa_status sm = sdpa::validate_bwd_attn_mask(mask, mask_kind, mask_strides, &a);
  if (sm != SDPA_OK) return sm;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  const hipError_t e = dtype == SDPA_BF16 ? sdpa::launch_bwd_mfma_masked_bf16(a)
                                          : sdpa::launch_bwd_mfma_masked_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

sdpa_status sdpa_bwd_masked_dropout(const void* q, const void* k, const void* v, const void* out,
                                    const void* dout, const float* lse, void* dq, void* dk,
                                    void* dv, float* workspace, int64_t B, int64_t H, int64_t Nq,
                                    int64_t Nk, int64_t d, float scale, int is_causal,
                                    const void* mask, sdpa_mask_kind mask_kind,
                                    const int64_t* mask_strides, float dropout_p, uint64_t seed,
                                    uint32_t offset, sdpa_dtype dtype, sdpa_dtype out_dtype,
                                    sdpa_dtype grad_dtype, void* stream) {
  sdpa::BwdArgs a;
  const sdpa_status st =
      sdpa::validate_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale,
                         is_causal, dtype, out_dtype, grad_dtype, stream, &a);
  if (st != SDPA_OK) return st;
  const sdpa_status sm = sdpa::validate_bwd_attn_mask(mask, mask_kind, mask_strides, &a);
  if (sm != SDPA_OK) return sm;
  const sdpa_status sd = sdpa::validate_bwd_dropout(dropout_p, seed, offset, &a);
  if (sd != SDPA_OK) return sd;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  const hipError_t e = dtype == SDPA_BF16 ? sdpa::launch_bwd_mfma_masked_bf16(a)
                                          : sdpa::launch_bwd_mfma_masked_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

sdpa_status sdpa_bwd_block_sparse(const void* q, const void* k, const void* v, const void* out,
                                  const void* dout, const float* lse, void* dq, void* dk,
                                  void* dv, float* workspace, int64_t B, int64_t H, int64_t Nq,
                                  int64_t Nk, int64_t d, float scale, int is_causal,
                                  const uint8_t* block_mask, int64_t mask_heads, sdpa_dtype dtype,
                                  sdpa_dtype out_dtype, sdpa_dtype grad_dtype, void* stream) {
  sdpa::BwdArgs a;
  const sdpa_status st =
      sdpa::validate_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale,
                         is_causal, dtype, out_dtype, grad_dtype, stream, &a);
  if (st != SDPA_OK) return st;
  const sdpa_status sm = sdpa::validate_bwd_block_mask(block_mask, mask_heads, &a);
  if (sm != SDPA_OK) return sm;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  const hipError_t e = dtype == SDPA_BF16 ? sdpa::launch_bwd_mfma_masked_bf16(a)
                                          : sdpa::launch_bwd_mfma_masked_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

sdpa_status sdpa_bwd_packed(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            float* workspace, int64_t B, int64_t H, int64_t T,
                            int64_t max_seqlen, int64_t d, float scale, int is_causal,
                            const int32_t* cu_seqlens, float dropout_p, uint64_t seed,
                            uint32_t offset, sdpa_dtype dtype, sdpa_dtype out_dtype,
                            sdpa_dtype grad_dtype, void* stream) {
  sdpa::BwdArgs a;
  const sdpa_status st = sdpa::validate_bwd_packed(
      q, k, v, out, dout, lse, dq, dk, dv, workspace, B, H, T, max_seqlen, d, scale, is_causal,
      cu_seqlens, dtype, out_dtype, grad_dtype, stream, &a);
  if (st != SDPA_OK) return st;
  const sdpa_status sd = sdpa::validate_bwd_dropout(dropout_p, seed, offset, &a);
  if (sd != SDPA_OK) return sd;
  if (!current_device_is_gfx950()) return SDPA_ERR_DEVICE;
  const hipError_t e =
      dtype == SDPA_BF16 ? sdpa::launch_bwd_mfma_bf16(a) : sdpa::launch_bwd_mfma_f16(a);
  return e == hipSuccess ? SDPA_OK : SDPA_ERR_LAUNCH;
}

int64_t sdpa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq) {
  if (B < 0 || H < 0 || Nq < 0) return -1;
  if (B != 0 && H > INT64_MAX / B) return -1;
  const int64_t bh = B * H;
  if (bh != 0 && Nq > INT64_MAX / 4 / bh) return -1;
  return bh * Nq * 4;
}

int sdpa_supports(sdpa_dtype dtype, int64_t d, int is_causal, int varlen) {
  // every supported (dtype, d) serves causal masking and packed batches
  if ((is_causal != 0 && is_causal != 1) || (varlen != 0 && varlen != 1)) return -1;
  return sdpa::path_for(dtype, d);
}

const char* sdpa_status_str(sdpa_status s) {
  switch (s) {
    case SDPA_OK: return "ok";
    case SDPA_ERR_INVALID: return "invalid argument";
    case SDPA_ERR_UNSUPPORTED: return "not supported";
    case SDPA_ERR_LAUNCH: return "kernel launch failed";
    case SDPA_ERR_DEVICE: return "current device is not gfx950";
  }
  return "unknown status";
}

int sdpa_abi_version(void) { return SDPA_ABI_VERSION; }

}  // extern "C"
