/*
 * sdpa.h -- C ABI of the fused, exact scaled dot-product attention forward
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every (batch, head) -- or (sequence, head) of a
 * packed variable-length batch -- and every query row i:
 *
 *     s_ij  = scale * <q_i, k_j>                  for j in A_i
 *     out_i = sum_j softmax_j(s_i.) * v_j
 *     lse_i = ln sum_{j in A_i} exp(s_ij)
 *
 * with A_i = every key, or the keys j <= i when is_causal is set (a
 * lower-triangular mask aligned at the top-left corner).  This is the
 * scaled dot-product attention of the PyTorch SDPA tutorial ("Overview";
 * the example calls in "Fused implementations" and the CausalSelfAttention
 * block under "Causal self-attention"), computed the FlashAttention way:
 * tile by tile with a running softmax, so that the N x N score matrix is
 * never written to device memory (FlashAttention article, method
 * paragraph and its tiling figure).  The result is exact attention up to
 * floating-point rounding; there is no approximation.
 *
 * Ownership and side effects.  The caller owns every buffer.  The library
 * never allocates, frees or synchronises, keeps no state between calls and
 * may be called concurrently from several host threads.  Work is queued on
 * `stream`; faults during kernel execution surface at the caller's next
 * synchronisation.  No C++ exception crosses this interface.
 */
#ifndef SDPA_MI355X_H
#define SDPA_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SDPA_ABI_VERSION 12

#if defined(__GNUC__)
#define SDPA_API __attribute__((visibility("default")))
#else
#define SDPA_API
#endif

/* Element types.  SDPA_SAME is only valid as an output type and means
 * "the input type".  Every enum of this interface spans the whole int32
 * range (the *_RANGE_* enumerators), so that any 32-bit value a caller
 * passes is a value of the type, which the library then checks and
 * refuses if unknown. */
typedef enum {
  SDPA_DTYPE_RANGE_MIN = -2147483647 - 1,
  SDPA_F16 = 0,
  SDPA_BF16 = 1,
  SDPA_F32 = 2,
  SDPA_SAME = 255,
  SDPA_DTYPE_RANGE_MAX = 2147483647
} sdpa_dtype;

/* Status codes.  Mirrors the tutorial's convention that an unsupported
 * input raises an error instead of computing ("Explicit dispatcher
 * control": a backend that cannot serve the input reports "not
 * supported"). */
typedef enum {
  SDPA_STATUS_RANGE_MIN = -2147483647 - 1,
  SDPA_OK = 0,
  SDPA_ERR_INVALID = 1,     /* malformed arguments (see sdpa_fwd)          */
  SDPA_ERR_UNSUPPORTED = 2, /* well-formed but outside what is implemented */
  SDPA_ERR_LAUNCH = 3,      /* the HIP runtime refused the launch          */
  SDPA_ERR_DEVICE = 4,      /* no usable gfx950 device is current          */
  SDPA_STATUS_RANGE_MAX = 2147483647
} sdpa_status;

/*
 * sdpa_fwd -- one attention forward, queued on `stream`.
 *
 * q, k, v   device pointers, element type `dtype`.
 *           Dense (cu_seqlens == NULL): q is [B, H, Nq, d], k and v are
 *           [B, H, Nk, d], all contiguous row-major.
 *           Packed (cu_seqlens != NULL): q, k, v are [T, H, d] contiguous,
 *           where sequence s owns rows cu_seqlens[s] .. cu_seqlens[s+1]-1
 *           and attends only to itself (the tutorial's NestedTensor batches,
 *           "NestedTensor and dense tensor support"); T = cu_seqlens[B].
 * out       device pointer, element type out_dtype (SDPA_SAME -> dtype),
 *           same shape as q.  Must not overlap q, k, v or lse.
 * lse       device pointer to float, or NULL to skip.  Natural-log
 *           logsumexp of the scaled, masked scores of each query row:
 *           [B, H, Nq] dense, [T, H] packed (the output's shape without d).
 * B, H      batch (number of sequences when packed) and heads, >= 1.
 * Nq, Nk    query and key rows per (batch, head), >= 1.  Packed: both must
 *           equal max_s(len_s); used only to size the launch grid.
 * d         head dimension, >= 1.
 * scale     multiplier of <q_i, k_j>; finite and >= 0 (1/sqrt(d) is the
 *           usual choice), with scale * log2(e) finite in fp32; every
 *           scale * <q_i, k_j> must be finite in fp32.
 * is_causal 0 or 1.
 * cu_seqlens device pointer to B+1 int32 offsets, or NULL for dense.  The
 *           caller guarantees cu_seqlens[0] = 0, non-decreasing entries and
 *           every length <= Nq; the library cannot check device memory.
 *           Zero-length sequences are allowed and write nothing.
 * dtype     SDPA_F16, SDPA_BF16 or SDPA_F32.
 * out_dtype SDPA_SAME or SDPA_F32.
 * stream    hipStream_t, or NULL for the null stream.
 *
 * Supported: f16 and bf16 with d in {32, 64, 128}; f32 with 1 <= d <= 128.
 * For bf16 inputs the P.V product runs on the f16 matrix cores with V
 * converted to f16, which requires |v| <= 65504 (larger values overflow).
 *
 * Alignment: q, k, v and out must be 16-byte aligned (f16/bf16 paths).
 *
 * Returns SDPA_OK, or
 *   SDPA_ERR_INVALID     null q/k/v/out, B/H/Nq/Nk/d < 1, non-finite scale,
 *                        is_causal not 0/1, unknown dtype, SDPA_SAME as
 *                        dtype, packed with Nq != Nk, misaligned pointers,
 *                        or element counts overflowing int64;
 *   SDPA_ERR_UNSUPPORTED d or dtype outside the supported set, negative
 *                        scale or scale * log2(e) above the fp32 range,
 *                        out_dtype other than SDPA_SAME/SDPA_F32;
 *   SDPA_ERR_DEVICE      the current device is not gfx950;
 *   SDPA_ERR_LAUNCH      the kernel launch failed.
 * Nothing is launched unless SDPA_OK is returned.
 */
SDPA_API sdpa_status sdpa_fwd(const void* q, const void* k, const void* v, void* out, float* lse,
                              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                              float scale, int is_causal, const int32_t* cu_seqlens,
                              sdpa_dtype dtype, sdpa_dtype out_dtype, void* stream);

/* Forward on strided dense layouts, e.g. the q, k, v views that a packed
 * QKV projection yields (SDPA tutorial, "Causal self-attention": c_attn(x)
 * [B, N, 3E] chunked into three and viewed as [B, H, N, d]) with the output
 * written straight into a [B, N, H*d] buffer.  Element (b, h, n, c) of a
 * tensor with strides s lives at base + b*s[0] + h*s[1] + n*s[2] + c
 * (elements; the stride along d is 1).
 *
 * q_strides, kv_strides, out_strides  host arrays of 3 int64 (batch, head,
 *             row); k and v share kv_strides.  Input strides: non-negative
 *             multiples of 8, bases 16-byte aligned; out strides: multiples
 *             of 4, and no two output elements may share an address.
 * lse         [B, H, Nq] contiguous (or null).
 * Other arguments as sdpa_fwd (no packed batches); f16/bf16 only.
 * SDPA_ERR_INVALID for bad strides or an output that overlaps itself or an
 * input; SDPA_ERR_UNSUPPORTED if a head's rows exceed 32-bit offsets.
 */
SDPA_API sdpa_status sdpa_fwd_strided(const void* q, const void* k, const void* v, void* out,
                                      float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                      int64_t d, const int64_t* q_strides,
                                      const int64_t* kv_strides, const int64_t* out_strides,
                                      float scale, int is_causal, sdpa_dtype dtype,
                                      sdpa_dtype out_dtype, void* stream);

/* Element types of an elementwise attention mask (sdpa_fwd_masked). */
typedef enum {
  SDPA_MASK_KIND_RANGE_MIN = -2147483647 - 1,
  SDPA_MASK_BOOL = 0,    /* one byte per pair (torch.bool storage): nonzero = attend */
  SDPA_MASK_ADD = 1,     /* additive, in the input element type (f16 or bf16)    */
  SDPA_MASK_ADD_F32 = 2, /* additive, f32                                          */
  SDPA_MASK_KIND_RANGE_MAX = 2147483647
} sdpa_mask_kind;

/* Forward with an elementwise attention mask.  The SDPA tutorial's
 * functional call takes an `attn_mask` argument (its CausalSelfAttention
 * passes None; "Fused implementations" and "Causal self-attention") but the
 * pages do not define it; the reading taken is the functional API's
 * convention.  A boolean mask says which (query, key) pairs take part; an
 * additive mask a is added to the scaled scores before the softmax:
 *     s_ij = scale * <q_i, k_j> + a_ij    (a_ij = 0 or -inf for a boolean mask)
 * then out and lse as sdpa_fwd, over the keys the causal rule leaves when
 * is_causal is set (both restrictions apply).  A row whose every score is
 * -inf gets out = 0 and lse = -inf.
 *
 * mask       device pointer; element (b, h, i, j) lives at
 *            mask + b*ms[0] + h*ms[1] + i*ms[2] + j (elements).  Base aligned
 *            to 4 elements.  Rows are read in blocks of 16 elements: elements
 *            j in [Nk, roundup(Nk, 16)) of every row must be readable (their
 *            values are ignored).  Additive values must be finite or -inf.
 * mask_kind  SDPA_MASK_BOOL, SDPA_MASK_ADD (the input type) or
 *            SDPA_MASK_ADD_F32.
 * mask_strides  host array of 3 int64 (ms[0..2]: batch, head, row), each a
 *            non-negative multiple of 4; 0 broadcasts that dimension (e.g.
 *            a key-padding mask [B, 1, 1, Nk] has ms[1] = ms[2] = 0).
 * q_strides, kv_strides, out_strides  all NULL (contiguous layouts, as
 *            sdpa_fwd) or all given (as sdpa_fwd_strided).
 * Other arguments as sdpa_fwd; dense layouts only, dtype SDPA_F16 or
 * SDPA_BF16.  The mask must not overlap out or lse.
 *
 * Returns SDPA_ERR_INVALID for a null mask or strides, an unknown kind,
 * misaligned mask or strides, or overlap; SDPA_ERR_UNSUPPORTED for f32
 * inputs or rows too far apart for 32-bit offsets (256 * ms[2] elements
 * beyond 2^31 bytes); otherwise as sdpa_fwd / sdpa_fwd_strided.
 */
SDPA_API sdpa_status sdpa_fwd_masked(const void* q, const void* k, const void* v, void* out,
                                     float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                     int64_t d, const int64_t* q_strides,
                                     const int64_t* kv_strides, const int64_t* out_strides,
                                     float scale, int is_causal, const void* mask,
                                     sdpa_mask_kind mask_kind, const int64_t* mask_strides,
                                     sdpa_dtype dtype, sdpa_dtype out_dtype, void* stream);

/* Block size of block-sparse masks: 128 query rows x 128 keys. */
#define SDPA_BLOCK_SPARSE_BLOCK 128

/* Block-sparse forward.  The FlashAttention article (results paragraph)
 * benchmarks a block-sparse FlashAttention but gives no mask format; here
 * query i may attend key j only if block_mask[h][i / 128][j / 128] is
 * nonzero (and j <= i when is_causal).  Within the visible set the result is
 * exact attention as in sdpa_fwd.  A row that sees no key gets O = 0 and
 * lse = -inf.  Blocks no row of a tile needs are neither computed nor read.
 *
 * block_mask  device pointer, uint8 [mask_heads][ceil(Nq/128)][ceil(Nk/128)],
 *             row-major; 0 = masked block.
 * mask_heads  1 (one mask for every head) or H.
 * Other arguments as sdpa_fwd, dense layouts only (no cu_seqlens), dtype
 * SDPA_F16 or SDPA_BF16.  Returns SDPA_ERR_INVALID for a null mask or
 * mask_heads not in {1, H}, SDPA_ERR_UNSUPPORTED for f32 inputs, otherwise
 * as sdpa_fwd.
 */
SDPA_API sdpa_status sdpa_fwd_block_sparse(const void* q, const void* k, const void* v, void* out,
                                           float* lse, int64_t B, int64_t H, int64_t Nq,
                                           int64_t Nk, int64_t d, float scale, int is_causal,
                                           const uint8_t* block_mask, int64_t mask_heads,
                                           sdpa_dtype dtype, sdpa_dtype out_dtype, void* stream);

/* Forward with dropout on the attention weights (the SDPA tutorial's
 * CausalSelfAttention passes its dropout rate to the functional call in
 * training).  Each softmax weight P_ij is kept with probability 1 - p and
 * kept weights are divided by the keep probability kappa:
 *     O_i = sum_j P_ij z_ij / kappa v_j;   lse as sdpa_fwd (undropped).
 * z comes from Philox4x32-10 (Salmon et al., SC 2011), key = (seed low 32
 * bits, seed high 32 bits), counter = (n(j), i, u, offset) with
 * u = b*H + h (packed: sequence*H + h, i counted from the sequence start),
 * n(j) = 2*(j >> 4) + ((j >> 2) & 1); the 16-bit half e(j) =
 * 4*((j >> 3) & 1) + (j & 3) of the output (word e >> 1, bits 16*(e & 1)..)
 * is compared with T = floor((1 - p) * 65536 + 1/2): kept iff below, so
 * kappa = T / 65536 (1 - p to within 2^-17), and the expected output is the
 * undropped one.  The same (seed, offset) gives the same mask on every
 * call.
 *
 * dropout_p  0 <= p < 1 (else SDPA_ERR_INVALID); p = 0 is exactly sdpa_fwd;
 *           a p that rounds T to 0 (1 - p below 2^-17) keeps nothing and
 *           returns SDPA_ERR_UNSUPPORTED.
 * seed, offset  as above.
 * Other arguments as sdpa_fwd; dtype SDPA_F16 or SDPA_BF16 (SDPA_F32:
 * SDPA_ERR_UNSUPPORTED).
 */
SDPA_API sdpa_status sdpa_fwd_dropout(const void* q, const void* k, const void* v, void* out,
                                      float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                      int64_t d, float scale, int is_causal,
                                      const int32_t* cu_seqlens, float dropout_p, uint64_t seed,
                                      uint32_t offset, sdpa_dtype dtype, sdpa_dtype out_dtype,
                                      void* stream);

/* Forward with an elementwise attention mask and dropout together: the
 * tutorial's module in training on padded batches passes both.  The mask
 * decides which pairs enter the softmax, exactly as in sdpa_fwd_masked;
 * dropout then acts on the resulting weights with the draws and scaling of
 * sdpa_fwd_dropout (the draws depend only on the pair's position, so a
 * mask changes none of them):
 *     P = softmax(scale q k^T + a),  O_i = sum_j P_ij z_ij / kappa v_j,
 *     lse = that of the masked scores (undropped).
 * A row whose every score is -inf gets out = 0 and lse = -inf.
 *
 * mask, mask_kind, mask_strides  as sdpa_fwd_masked.
 * dropout_p, seed, offset  as sdpa_fwd_dropout (unit u = b*H + h).
 * q_strides, kv_strides, out_strides  all NULL or all given, as
 *           sdpa_fwd_masked.  Other arguments as sdpa_fwd; dense layouts,
 *           dtype SDPA_F16 or SDPA_BF16.
 * Returns the errors of sdpa_fwd_masked and sdpa_fwd_dropout; p = 0 is
 * exactly sdpa_fwd_masked.
 */
SDPA_API sdpa_status sdpa_fwd_masked_dropout(
    const void* q, const void* k, const void* v, void* out, float* lse, int64_t B, int64_t H,
    int64_t Nq, int64_t Nk, int64_t d, const int64_t* q_strides, const int64_t* kv_strides,
    const int64_t* out_strides, float scale, int is_causal, const void* mask,
    sdpa_mask_kind mask_kind, const int64_t* mask_strides, float dropout_p, uint64_t seed,
    uint32_t offset, sdpa_dtype dtype, sdpa_dtype out_dtype, void* stream);

/* Backward pass of sdpa_fwd: the gradients dq, dk, dv of sum(dout * out)
 * with respect to q, k and v.  The FlashAttention article (method
 * paragraph) names recomputation in the backward pass as its second
 * technique: the attention probabilities are rebuilt tile by tile from q, k
 * and the forward's lse instead of being stored.  What is computed is the
 * chain rule of the forward definition above:
 *     P = exp(s - lse),   dV = P^T dO,   dP = dO V^T,
 *     dS = P * (dP - rowsum(dO * O)),   dQ = scale dS K,   dK = scale dS^T Q
 * (masked pairs have P = 0).
 *
 * q, k, v   the forward's inputs, dense [B,H,Nq,d] / [B,H,Nk,d], dtype.
 * out       the forward's output O [B,H,Nq,d] in out_dtype.
 * dout      upstream gradient dO [B,H,Nq,d] in dtype.
 * lse       the forward's logsumexp [B,H,Nq] (fp32, natural log).
 * dq, dk, dv  outputs [B,H,Nq,d] / [B,H,Nk,d] in grad_dtype; every element
 *           is written (keys no query attends get zero gradients).
 * workspace B*H*Nq floats owned by the caller (sdpa_bwd_workspace_bytes);
 *           overwritten.
 * B, H, Nq, Nk, d, scale, is_causal  as in sdpa_fwd (dense layouts only).
 * dtype     SDPA_F16 or SDPA_BF16; d in {32, 64, 128}.
 * out_dtype / grad_dtype  SDPA_SAME or SDPA_F32.
 * stream    hipStream_t, or NULL.  All pointers are device pointers, 16-byte
 *           aligned (lse and workspace: 4-byte); outputs must not overlap
 *           any input or each other.
 *
 * Precision: every product accumulates in fp32; q, k, v and dout enter the
 * matrix cores exactly.  P and dS are rounded to the input type before the
 * dV, dK and dQ products (f16: relative 2^-11, with f16's subnormal range
 * below 2^-14; bf16: relative 2^-8 over bf16's whole exponent range, so
 * upstream gradients as small as bf16 itself holds are not flushed).
 *
 * Returns SDPA_OK, or SDPA_ERR_INVALID / SDPA_ERR_UNSUPPORTED /
 * SDPA_ERR_DEVICE / SDPA_ERR_LAUNCH with the meanings of sdpa_fwd (f32
 * inputs and packed batches are unsupported).  Queues two kernels on
 * `stream` (dQ, which also writes the row dots into `workspace`, then dK
 * and dV); allocates nothing.  Nothing is launched unless SDPA_OK is
 * returned.
 */
SDPA_API sdpa_status sdpa_bwd(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv,
                              float* workspace, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                              int64_t d, float scale, int is_causal, sdpa_dtype dtype,
                              sdpa_dtype out_dtype, sdpa_dtype grad_dtype, void* stream);

/* Backward pass of sdpa_fwd_dropout: the gradients of sum(dO * O) where
 * O = sum_j P_ij z_ij / kappa v_j and the mask z is the one the forward
 * drew (it is regenerated from the same dropout_p, seed and offset, never
 * stored).  With W = P z / kappa: dV = W^T dO, dP = (dO V^T) z / kappa,
 * dS = P (dP - <dO, O>), dQ = scale dS K, dK = scale dS^T Q.  `out` and
 * `lse` are the dropout forward's.  Arguments otherwise as sdpa_bwd;
 * 0 <= dropout_p < 1 (else SDPA_ERR_INVALID), p = 0 is exactly sdpa_bwd.
 */
SDPA_API sdpa_status sdpa_bwd_dropout(const void* q, const void* k, const void* v,
                                      const void* out, const void* dout, const float* lse,
                                      void* dq, void* dk, void* dv, float* workspace, int64_t B,
                                      int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                      int is_causal, float dropout_p, uint64_t seed,
                                      uint32_t offset, sdpa_dtype dtype, sdpa_dtype out_dtype,
                                      sdpa_dtype grad_dtype, void* stream);

/* Backward pass of sdpa_fwd_masked: the gradients of sum(dout * out) for
 * attention with an elementwise mask, the chain rule of sdpa_bwd with the
 * mask's bias a constant (not differentiated):
 *     P = softmax(scale q k^T + a),  dV = P^T dO,  dP = dO V^T,
 *     dS = P (dP - rowsum(dO * O)),  dQ = scale dS K,  dK = scale dS^T Q.
 * Rows the forward found empty (lse = -inf) contribute nothing.
 *
 * mask, mask_kind, mask_strides  as sdpa_fwd_masked (the same mask the
 *           forward used); in addition one (batch, head) unit's mask,
 *           (Nq + 256) * mask_strides[2] elements plus a row, must fit
 *           32-bit byte offsets (else SDPA_ERR_UNSUPPORTED).
 * Other arguments as sdpa_bwd: dense contiguous layouts, f16/bf16.  The
 * mask must not overlap dq, dk, dv or the workspace.
 */
SDPA_API sdpa_status sdpa_bwd_masked(const void* q, const void* k, const void* v,
                                     const void* out, const void* dout, const float* lse,
                                     void* dq, void* dk, void* dv, float* workspace, int64_t B,
                                     int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                     int is_causal, const void* mask, sdpa_mask_kind mask_kind,
                                     const int64_t* mask_strides, sdpa_dtype dtype,
                                     sdpa_dtype out_dtype, sdpa_dtype grad_dtype, void* stream);

/* Backward pass of sdpa_fwd_masked_dropout: the gradients of
 * sum(dout * out) with the mask's bias and the dropout mask z constants:
 *     P = softmax(scale q k^T + a),  W = P z / kappa,  dV = W^T dO,
 *     dP = (dO V^T) z / kappa,  dS = P (dP - rowsum(dO * O)),
 *     dQ = scale dS K,  dK = scale dS^T Q.
 * `out` and `lse` are the forward's; z is regenerated from the same
 * dropout_p, seed and offset.  mask arguments as sdpa_bwd_masked, dropout
 * arguments as sdpa_bwd_dropout, the rest as sdpa_bwd.  p = 0 is exactly
 * sdpa_bwd_masked.
 */
SDPA_API sdpa_status sdpa_bwd_masked_dropout(
    const void* q, const void* k, const void* v, const void* out, const void* dout,
    const float* lse, void* dq, void* dk, void* dv, float* workspace, int64_t B, int64_t H,
    int64_t Nq, int64_t Nk, int64_t d, float scale, int is_causal, const void* mask,
    sdpa_mask_kind mask_kind, const int64_t* mask_strides, float dropout_p, uint64_t seed,
    uint32_t offset, sdpa_dtype dtype, sdpa_dtype out_dtype, sdpa_dtype grad_dtype,
    void* stream);

/* Backward pass of sdpa_fwd_block_sparse: the gradients of sum(dout * out)
 * for exact attention restricted to the pairs the block mask keeps (the
 * chain rule of sdpa_bwd over the visible pairs).  Only the tiles whose
 * 128x128 mask block is kept are read or computed; rows that see no key
 * (lse = -inf) contribute nothing, and keys no row sees get zero
 * gradients.
 *
 * block_mask, mask_heads  as sdpa_fwd_block_sparse (the forward's mask).
 * Other arguments as sdpa_bwd: dense contiguous layouts, f16/bf16, no
 * dropout.  The mask must not overlap dq, dk, dv or the workspace.
 * Returns SDPA_ERR_INVALID for a null mask or mask_heads not in {1, H},
 * otherwise as sdpa_bwd.
 */
SDPA_API sdpa_status sdpa_bwd_block_sparse(const void* q, const void* k, const void* v,
                                           const void* out, const void* dout, const float* lse,
                                           void* dq, void* dk, void* dv, float* workspace,
                                           int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                           int64_t d, float scale, int is_causal,
                                           const uint8_t* block_mask, int64_t mask_heads,
                                           sdpa_dtype dtype, sdpa_dtype out_dtype,
                                           sdpa_dtype grad_dtype, void* stream);

/* Backward pass of a packed variable-length batch: the gradients of
 * sdpa_fwd (or sdpa_fwd_dropout) with cu_seqlens, the chain rule of
 * sdpa_bwd applied to each (sequence, head) unit.  The tutorial's
 * NestedTensor batches ("NestedTensor and dense tensor support") run its
 * module in training as well as in inference.
 *
 * q, k, v, out, dout  [T, H, d] as in the packed forward (out in
 *           out_dtype, dout in dtype); sequence s owns rows
 *           cu_seqlens[s] .. cu_seqlens[s+1]-1.
 * lse       the packed forward's [T, H] logsumexp.
 * dq, dk, dv  outputs [T, H, d] in grad_dtype; every row of a sequence is
 *           written (rows outside every sequence are not touched).
 * workspace T*H floats owned by the caller (sdpa_bwd_workspace_bytes(1, H,
 *           T)); overwritten.
 * B         number of sequences; cu_seqlens holds B+1 int32 offsets (device
 *           memory, as in sdpa_fwd: cu_seqlens[0] = 0, non-decreasing,
 *           cu_seqlens[B] = T, every length <= max_seqlen).
 * T         total rows (the tensors' first dimension).
 * max_seqlen  the longest sequence; sizes the grid.
 * dropout_p, seed, offset  the packed forward's dropout contract (p = 0:
 *           none); unit u = s*H + h, rows counted from the sequence start.
 * Other arguments as sdpa_bwd.  Returns SDPA_ERR_INVALID for a null or
 * misaligned cu_seqlens, B, T or max_seqlen < 1, a bad dropout_p, or the
 * conditions of sdpa_bwd on [T, H, d] tensors; SDPA_ERR_UNSUPPORTED when a
 * sequence's rows exceed 32-bit offsets ((max_seqlen + 256) * H * d * 2
 * bytes beyond 2^31) or as sdpa_bwd.
 */
SDPA_API sdpa_status sdpa_bwd_packed(const void* q, const void* k, const void* v,
                                     const void* out, const void* dout, const float* lse,
                                     void* dq, void* dk, void* dv, float* workspace, int64_t B,
                                     int64_t H, int64_t T, int64_t max_seqlen, int64_t d,
                                     float scale, int is_causal, const int32_t* cu_seqlens,
                                     float dropout_p, uint64_t seed, uint32_t offset,
                                     sdpa_dtype dtype, sdpa_dtype out_dtype,
                                     sdpa_dtype grad_dtype, void* stream);

/* Largest B*H*Nq that sdpa_bwd_noalloc serves (16 MiB of floats). */
#define SDPA_BWD_NOALLOC_MAX_ROWS (4 * 1024 * 1024)

/* sdpa_bwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight training loops, harnesses that forbid hipMalloc.
 * The same gradients, bit for bit, as sdpa_bwd; the B*H*Nq row dots that
 * sdpa_bwd keeps in the caller's workspace live in a fixed device array
 * that the library holds, one copy per device, until the process ends.
 *
 * Arguments as sdpa_bwd without `workspace`.  The call allocates and frees
 * nothing and calls no allocating library routine.  Every call on one
 * device shares that device's array, so calls that overlap in time on one
 * device (e.g. on two streams) race and give undefined results; calls on
 * one stream, or on different devices, do not.
 *
 * Returns as sdpa_bwd, and SDPA_ERR_UNSUPPORTED when B*H*Nq exceeds
 * SDPA_BWD_NOALLOC_MAX_ROWS (checked before any device work); the size
 * limits are checked first, so an oversized call is refused even without a
 * device. */
SDPA_API sdpa_status sdpa_bwd_noalloc(const void* q, const void* k, const void* v,
                                      const void* out, const void* dout, const float* lse,
                                      void* dq, void* dk, void* dv, int64_t B, int64_t H,
                                      int64_t Nq, int64_t Nk, int64_t d, float scale,
                                      int is_causal, sdpa_dtype dtype, sdpa_dtype out_dtype,
                                      sdpa_dtype grad_dtype, void* stream);

/* Bytes of the workspace sdpa_bwd needs (B*H*Nq floats), or -1 if the sizes
 * overflow.  Pure host function. */
SDPA_API int64_t sdpa_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Nq);

/* Which path would serve a call, asked before making it: the SDPA
 * tutorial's dispatcher ("Explicit dispatcher control") tries backends in
 * turn and a backend that cannot serve an input reports "not supported";
 * here there is one backend per input type, and this query says in
 * advance whether sdpa_fwd would refuse.  Returns 1 if (dtype, d,
 * is_causal, varlen) is served by the matrix-core path (f16 / bf16, d in
 * {32, 64, 128}), 0 if by the plain f32 path (1 <= d <= 128), -1 if
 * unsupported or if is_causal or varlen is not 0 or 1.  Causal masking and
 * packed batches are served by every supported (dtype, d).  Pure host
 * function; touches no device. */
SDPA_API int sdpa_supports(sdpa_dtype dtype, int64_t d, int is_causal, int varlen);

/* Static string naming a status code, never NULL: "ok", "invalid
 * argument", "not supported" (the tutorial's wording for an input a backend
 * cannot serve, "Explicit dispatcher control"), "kernel launch failed",
 * "current device is not gfx950", or "unknown status". */
SDPA_API const char* sdpa_status_str(sdpa_status s);

/* SDPA_ABI_VERSION of the built library, so that a caller built against
 * this header can refuse a library whose entry points differ.  Bookkeeping
 * of this interface; the pages define no versioning. */
SDPA_API int sdpa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_H */
