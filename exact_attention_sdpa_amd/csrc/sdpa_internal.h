// Internal interface between the C-ABI entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sdpa.h"

namespace sdpa {

// Validated arguments of one forward call.  Sizes are already checked to be
// positive and small enough for the kernels' int32 tile arithmetic.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;               // may be null
  const int32_t* cu;        // null for dense
  int64_t B, H, Nq, Nk, d;  // packed: Nq == Nk == max sequence length
  // dense layouts: (batch, head, row) strides in elements of q, of k and v
  // (shared), of out; contiguous [B,H,N,d] unless set by the strided entry
  int64_t q_str[3], kv_str[3], o_str[3];
  float scale;
  bool causal;
  bool out_f32;             // out element type is f32 (else the input type)
  sdpa_dtype dtype;         // SDPA_F16, SDPA_BF16 or SDPA_F32
  hipStream_t stream;       // null = the null stream
  const uint8_t* bmask;     // block-sparse mask, or null
  int64_t mask_heads;       // 1 (shared) or H
  bool dropout;             // dropout on the attention weights
  uint64_t drop_seed;       // Philox key
  uint32_t drop_offset;     // last Philox counter word
  uint32_t drop_t;          // keep iff the 16-bit number < drop_t
  float drop_scale;         // 65536 / drop_t, the inverse keep probability
  const void* amask;        // elementwise mask, or null
  int amask_kind;           // sdpa_mask_kind
  int64_t am_str[3];        // mask (batch, head, row) strides, elements
};

// Validated arguments of one backward call (dense layouts only).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;          // forward output O
  const void* dout;         // upstream gradient dO (input dtype)
  const float* lse;         // forward logsumexp, natural log
  void* dq;
  void* dk;
  void* dv;
  float* work;              // B*H*Nq floats (packed: T*H)
  const int32_t* cu;        // packed batches: B+1 sequence offsets, else null
  int64_t T;                // packed batches: total rows
  int64_t B, H, Nq, Nk, d;  // packed: Nq == Nk == the longest sequence
  float scale;
  bool causal;
  bool out_f32;             // O is f32 (else the input type)
  bool grad_f32;            // dq/dk/dv are f32 (else the input type)
  sdpa_dtype dtype;         // SDPA_F16 or SDPA_BF16
  hipStream_t stream;
  bool dropout;             // the forward ran with dropout (same contract)
  uint64_t drop_seed;
  uint32_t drop_offset;
  uint32_t drop_t;
  float drop_scale;
  const void* amask;        // elementwise mask, or null
  int amask_kind;           // sdpa_mask_kind
  int64_t am_str[3];        // mask (batch, head, row) strides, elements
  const uint8_t* bmask;     // block-sparse mask, or null
  int64_t mask_heads;       // 1 (shared) or H
};

// Host-only argument checks (no HIP calls).  Fills `a` on success.
sdpa_status validate(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                     int is_causal, const int32_t* cu_seqlens, sdpa_dtype dtype,
                     sdpa_dtype out_dtype, void* stream, FwdArgs* a,
                     bool check_overlap = true);

// Host-only checks of a backward call.  Fills `a` on success.
// Replaces the contiguous strides of validated dense forward arguments with
// caller strides (batch, head, row; elements): non-negative multiples of 8
// (inputs) or 4 (out), rows of one head within 32-bit buffer offsets, out
// non-overlapping in itself and clear of q, k, v and lse.
sdpa_status validate_strides(const int64_t* q_strides, const int64_t* kv_strides,
                             const int64_t* out_strides, FwdArgs* a);

// Adds a block-sparse mask to validated forward arguments: mask non-null,
// mask_heads 1 or H, f16/bf16 inputs, dense layout, and the mask
// [mask_heads][ceil(Nq/128)][ceil(Nk/128)] bytes clear of out and lse.
sdpa_status validate_block_mask(const uint8_t* mask, int64_t mask_heads, FwdArgs* a);

// Adds an elementwise mask to validated dense forward arguments: kind
// known, f16/bf16 inputs, strides non-negative multiples of 4, base aligned
// to 4 elements, a workgroup's rows within 32-bit offsets, and the mask
// clear of out and lse.
sdpa_status validate_attn_mask(const void* mask, sdpa_mask_kind kind,
                               const int64_t* mask_strides, FwdArgs* a);

// Adds an elementwise mask to validated dense backward arguments: as
// validate_attn_mask, with each (batch, head) unit's mask rows within
// 32-bit offsets, and the mask clear of dq, dk, dv and the workspace.
sdpa_status validate_bwd_attn_mask(const void* mask, sdpa_mask_kind kind,
                                   const int64_t* mask_strides, BwdArgs* a);

// Adds a block-sparse mask to validated dense backward arguments: as
// validate_block_mask, and the mask clear of dq, dk, dv and the workspace.
sdpa_status validate_bwd_block_mask(const uint8_t* mask, int64_t mask_heads, BwdArgs* a);

// Adds dropout to validated backward arguments (same rules as the forward).
sdpa_status validate_bwd_dropout(float p, uint64_t seed, uint32_t offset, BwdArgs* a);

// Adds dropout to validated forward arguments: 0 <= p < 1 (p = 0 leaves the
// plain kernel), f16/bf16 inputs; the keep threshold T = floor((1-p) 65536 +
// 1/2) and the scale 65536 / T are computed here, in double (T = 0 is
// refused as unsupported).
sdpa_status validate_dropout(float p, uint64_t seed, uint32_t offset, FwdArgs* a);

// Host-only checks of a packed-batch backward call (q, k, v, out, dout,
// dq, dk, dv [T,H,d]; lse and workspace [T,H]).  Fills `a` on success.
sdpa_status validate_bwd_packed(const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                float* workspace, int64_t B, int64_t H, int64_t T,
                                int64_t max_seqlen, int64_t d, float scale, int is_causal,
                                const int32_t* cu_seqlens, sdpa_dtype dtype,
                                sdpa_dtype out_dtype, sdpa_dtype grad_dtype, void* stream,
                                BwdArgs* a);

sdpa_status validate_bwd(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* workspace, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                         int64_t d, float scale, int is_causal, sdpa_dtype dtype,
                         sdpa_dtype out_dtype, sdpa_dtype grad_dtype, void* stream,
                         BwdArgs* a);

// 1 = matrix-core path, 0 = plain f32 path, -1 = unsupported.
int path_for(sdpa_dtype dtype, int64_t d);

// True if the calling thread's current HIP device is a gfx950 (cached per
// device after the first query).
bool current_device_is_gfx950();

// Kernel launchers: queue the kernel on a.stream and return the launch status.
hipError_t launch_fwd_mfma_f16(const FwdArgs& a);
hipError_t launch_fwd_mfma_bf16(const FwdArgs& a);
hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_fwd_mfma_masked_f16(const FwdArgs& a);
hipError_t launch_fwd_mfma_masked_bf16(const FwdArgs& a);
hipError_t launch_bwd_mfma_f16(const BwdArgs& a);
hipError_t launch_bwd_mfma_bf16(const BwdArgs& a);
hipError_t launch_bwd_mfma_masked_f16(const BwdArgs& a);
hipError_t launch_bwd_mfma_masked_bf16(const BwdArgs& a);

}  // namespace sdpa
