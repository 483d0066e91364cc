// Host-side argument checks of sdpa_fwd and sdpa_bwd.  Makes no HIP calls, so every
// error path can be exercised without a GPU.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "sdpa_internal.h"

namespace sdpa {

namespace {

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

int elem_bytes(sdpa_dtype t) { return t == SDPA_F32 ? 4 : 2; }

// bytes from the base of a strided [B,H,N,d] tensor to one past its last
// element (strides in elements, all non-negative); -1 if that overflows
int64_t span_bytes(int64_t B, int64_t H, int64_t N, int64_t d, const int64_t* s, int64_t eb) {
  const __int128 e = ((__int128)(B - 1) * s[0] + (__int128)(H - 1) * s[1] +
                      (__int128)(N - 1) * s[2] + d) * eb;
  return e > (__int128)(INT64_MAX / 2) ? -1 : (int64_t)e;
}

// no two (b, h, n, c) of a strided [B,H,N,d] tensor share an element:
// along ascending strides, each stride clears the extent of the dims below
bool no_self_overlap(int64_t B, int64_t H, int64_t N, int64_t d, const int64_t* s) {
  int64_t st[3] = {s[0], s[1], s[2]}, sz[3] = {B, H, N};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (st[j] < st[i] || (st[j] == st[i] && sz[j] < sz[i])) {
        std::swap(st[i], st[j]);
        std::swap(sz[i], sz[j]);
      }
  int64_t extent = d;   // elements covered by the dims below, plus one
  for (int i = 0; i < 3; ++i) {
    if (sz[i] == 1) continue;
    if (st[i] < extent) return false;
    extent = (sz[i] - 1) * st[i] + extent;
  }
  return true;
}

}  // namespace

int path_for(sdpa_dtype dtype, int64_t d) {
  if (dtype == SDPA_F16 || dtype == SDPA_BF16) return (d == 32 || d == 64 || d == 128) ? 1 : -1;
  if (dtype == SDPA_F32) return (d >= 1 && d <= 128) ? 0 : -1;
  return -1;
}

sdpa_status validate(const void* q, const void* k, const void* v, void* out, float* lse,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                     int is_causal, const int32_t* cu_seqlens, sdpa_dtype dtype,
                     sdpa_dtype out_dtype, void* stream, FwdArgs* a, bool check_overlap) {
  if (!q || !k || !v || !out) return SDPA_ERR_INVALID;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return SDPA_ERR_INVALID;
  if (is_causal != 0 && is_causal != 1) return SDPA_ERR_INVALID;
  if (dtype != SDPA_F16 && dtype != SDPA_BF16 && dtype != SDPA_F32) return SDPA_ERR_INVALID;
  if (!std::isfinite(scale)) return SDPA_ERR_INVALID;
  const bool varlen = cu_seqlens != nullptr;
  if (varlen && Nq != Nk) return SDPA_ERR_INVALID;

  // sizes must fit the kernels' int32 row and tile arithmetic
  const int64_t lim = (int64_t)1 << 30;
  if (H > lim || Nq > lim || Nk > lim || B > lim) return SDPA_ERR_INVALID;
  int64_t rows_q, rows_k, eq, ek, tmp;
  if (!mul_ok(B, H, &tmp) || !mul_ok(tmp, Nq, &rows_q) || !mul_ok(tmp, Nk, &rows_k) ||
      !mul_ok(rows_q, d, &eq) || !mul_ok(rows_k, d, &ek) || eq > INT64_MAX / 4 ||
      ek > INT64_MAX / 4)
    return SDPA_ERR_INVALID;
  // one workgroup per (batch, head, 32-row block) at most
  if (tmp * ((Nq + 31) / 32) > INT32_MAX) return SDPA_ERR_INVALID;

  bool out_f32;
  if (out_dtype == SDPA_SAME || out_dtype == dtype)
    out_f32 = dtype == SDPA_F32;
  else if (out_dtype == SDPA_F32)
    out_f32 = true;
  else if (out_dtype == SDPA_F16 || out_dtype == SDPA_BF16)
    return SDPA_ERR_UNSUPPORTED;
  else
    return SDPA_ERR_INVALID;

  const int path = path_for(dtype, d);
  if (path < 0) return SDPA_ERR_UNSUPPORTED;
  if (scale < 0.f) return SDPA_ERR_UNSUPPORTED;
  // the kernels work in base 2 with scale * log2(e), which must be finite
  if (!std::isfinite(scale * 1.4426950408889634f)) return SDPA_ERR_UNSUPPORTED;

  // matrix-core path: one head's rows (plus a query tile of slack) must fit
  // the 32-bit byte offsets of its buffer loads
  if (path == 1) {
    const int64_t row_bytes = (varlen ? H * d : d) * 2;
    if ((std::max(Nq, Nk) + 256) * row_bytes > (int64_t)INT32_MAX) return SDPA_ERR_UNSUPPORTED;
  }

  const uintptr_t al = path == 1 ? 16 : 4;
  if (!aligned(q, al) || !aligned(k, al) || !aligned(v, al) || !aligned(out, al))
    return SDPA_ERR_INVALID;
  if (lse && !aligned(lse, 4)) return SDPA_ERR_INVALID;
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return SDPA_ERR_INVALID;

  if (!varlen && check_overlap) {
    const int64_t ib = elem_bytes(dtype), ob = out_f32 ? 4 : elem_bytes(dtype);
    const int64_t obytes = eq * ob;
    if (overlap(out, obytes, q, eq * ib) || overlap(out, obytes, k, ek * ib) ||
        overlap(out, obytes, v, ek * ib))
      return SDPA_ERR_INVALID;
    if (lse && overlap(out, obytes, lse, rows_q * 4)) return SDPA_ERR_INVALID;
  }

  a->q = q;
  a->k = k;
  a->v = v;
  a->out = out;
  a->lse = lse;
  a->cu = cu_seqlens;
  a->B = B;
  a->H = H;
  a->Nq = Nq;
  a->Nk = Nk;
  a->d = d;
  a->scale = scale;
  a->causal = is_causal != 0;
  a->out_f32 = out_f32;
  a->dtype = dtype;
  a->stream = static_cast<hipStream_t>(stream);
  a->q_str[0] = H * Nq * d;
  a->q_str[1] = Nq * d;
  a->q_str[2] = d;
  a->kv_str[0] = H * Nk * d;
  a->kv_str[1] = Nk * d;
  a->kv_str[2] = d;
  a->o_str[0] = H * Nq * d;
  a->o_str[1] = Nq * d;
  a->o_str[2] = d;
  a->bmask = nullptr;
  a->mask_heads = 0;
  a->dropout = false;
  a->drop_seed = 0;
  a->drop_offset = 0;
  a->drop_t = 65536;
  a->drop_scale = 1.f;
  a->amask = nullptr;
  a->amask_kind = SDPA_MASK_BOOL;
  a->am_str[0] = a->am_str[1] = a->am_str[2] = 0;
  return SDPA_OK;
}

sdpa_status validate_strides(const int64_t* q_strides, const int64_t* kv_strides,
                             const int64_t* out_strides, FwdArgs* a) {
  if (!q_strides || !kv_strides || !out_strides) return SDPA_ERR_INVALID;
  if (a->cu != nullptr) return SDPA_ERR_INVALID;
  if (a->dtype == SDPA_F32) return SDPA_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 40;
  for (int i = 0; i < 3; ++i) {
    // 16-byte input loads; output stores of 4 elements
    if (q_strides[i] < 0 || kv_strides[i] < 0 || out_strides[i] < 0) return SDPA_ERR_INVALID;
    if (q_strides[i] > lim || kv_strides[i] > lim || out_strides[i] > lim) return SDPA_ERR_INVALID;
    if (q_strides[i] % 8 || kv_strides[i] % 8 || out_strides[i] % 4) return SDPA_ERR_INVALID;
  }
  // one head's rows (plus a tile of slack) within 32-bit buffer offsets
  if ((a->Nq + 256) * q_strides[2] * 2 > (int64_t)INT32_MAX ||
      (a->Nk + 256) * kv_strides[2] * 2 > (int64_t)INT32_MAX)
    return SDPA_ERR_UNSUPPORTED;
  if (!no_self_overlap(a->B, a->H, a->Nq, a->d, out_strides)) return SDPA_ERR_INVALID;
  const int64_t ib = elem_bytes(a->dtype), ob = a->out_f32 ? 4 : ib;
  const int64_t os = span_bytes(a->B, a->H, a->Nq, a->d, out_strides, ob);
  const int64_t qs = span_bytes(a->B, a->H, a->Nq, a->d, q_strides, ib);
  const int64_t ks = span_bytes(a->B, a->H, a->Nk, a->d, kv_strides, ib);
  if (os < 0 || qs < 0 || ks < 0) return SDPA_ERR_INVALID;
  if (overlap(a->out, os, a->q, qs) || overlap(a->out, os, a->k, ks) ||
      overlap(a->out, os, a->v, ks))
    return SDPA_ERR_INVALID;
  if (a->lse && overlap(a->out, os, a->lse, a->B * a->H * a->Nq * 4)) return SDPA_ERR_INVALID;
  for (int i = 0; i < 3; ++i) {
    a->q_str[i] = q_strides[i];
    a->kv_str[i] = kv_strides[i];
    a->o_str[i] = out_strides[i];
  }
  return SDPA_OK;
}

sdpa_status validate_block_mask(const uint8_t* mask, int64_t mask_heads, FwdArgs* a) {
  if (mask == nullptr || (mask_heads != 1 && mask_heads != a->H)) return SDPA_ERR_INVALID;
  if (a->cu != nullptr) return SDPA_ERR_INVALID;
  if (a->dtype == SDPA_F32) return SDPA_ERR_UNSUPPORTED;
  constexpr int64_t blk = SDPA_BLOCK_SPARSE_BLOCK;
  const int64_t nqb = (a->Nq + blk - 1) / blk, nkb = (a->Nk + blk - 1) / blk;
  int64_t mb = 0, ob = 0;
  if (!mul_ok(mask_heads * nqb, nkb, &mb) || mb > INT32_MAX) return SDPA_ERR_INVALID;
  if (!mul_ok(a->B * a->H * a->Nq, a->d * (a->out_f32 ? 4 : elem_bytes(a->dtype)), &ob))
    return SDPA_ERR_INVALID;
  if (overlap(mask, mb, a->out, ob)) return SDPA_ERR_INVALID;
  if (a->lse && overlap(mask, mb, a->lse, a->B * a->H * a->Nq * 4)) return SDPA_ERR_INVALID;
  a->bmask = mask;
  a->mask_heads = mask_heads;
  return SDPA_OK;
}

sdpa_status validate_attn_mask(const void* mask, sdpa_mask_kind kind,
                               const int64_t* mask_strides, FwdArgs* a) {
  if (mask == nullptr || mask_strides == nullptr) return SDPA_ERR_INVALID;
  if (kind != SDPA_MASK_BOOL && kind != SDPA_MASK_ADD && kind != SDPA_MASK_ADD_F32)
    return SDPA_ERR_INVALID;
  if (a->cu != nullptr) return SDPA_ERR_INVALID;
  if (a->dtype == SDPA_F32) return SDPA_ERR_UNSUPPORTED;
  const int64_t eb = kind == SDPA_MASK_BOOL ? 1 : kind == SDPA_MASK_ADD ? 2 : 4;
  const int64_t lim = (int64_t)1 << 40;
  for (int i = 0; i < 3; ++i)
    if (mask_strides[i] < 0 || mask_strides[i] > lim || mask_strides[i] % 4 != 0)
      return SDPA_ERR_INVALID;
  if (!aligned(mask, (uintptr_t)(4 * eb))) return SDPA_ERR_INVALID;
  // rows are read in blocks of 16 elements
  const int64_t nk16 = (a->Nk + 15) / 16 * 16;
  // a workgroup reads its rows through 32-bit byte offsets
  if ((256 * mask_strides[2] + nk16) * eb > (int64_t)INT32_MAX) return SDPA_ERR_UNSUPPORTED;
  const __int128 span = ((__int128)(a->B - 1) * mask_strides[0] +
                         (__int128)(a->H - 1) * mask_strides[1] +
                         (__int128)(a->Nq - 1) * mask_strides[2] + nk16) * eb;
  if (span > (__int128)(INT64_MAX / 2)) return SDPA_ERR_INVALID;
  const int64_t ob = a->out_f32 ? 4 : elem_bytes(a->dtype);
  const int64_t os = span_bytes(a->B, a->H, a->Nq, a->d, a->o_str, ob);
  if (os < 0 || overlap(mask, (int64_t)span, a->out, os)) return SDPA_ERR_INVALID;
  if (a->lse && overlap(mask, (int64_t)span, a->lse, a->B * a->H * a->Nq * 4))
    return SDPA_ERR_INVALID;
  a->amask = mask;
  a->amask_kind = kind;
  for (int i = 0; i < 3; ++i) a->am_str[i] = mask_strides[i];
  return SDPA_OK;
}

sdpa_status validate_bwd_attn_mask(const void* mask, sdpa_mask_kind kind,
                                   const int64_t* mask_strides, BwdArgs* a) {
  if (mask == nullptr || mask_strides == nullptr) return SDPA_ERR_INVALID;
  if (kind != SDPA_MASK_BOOL && kind != SDPA_MASK_ADD && kind != SDPA_MASK_ADD_F32)
    return SDPA_ERR_INVALID;
  if (a->cu != nullptr) return SDPA_ERR_INVALID;
  const int64_t eb = kind == SDPA_MASK_BOOL ? 1 : kind == SDPA_MASK_ADD ? 2 : 4;
  const int64_t lim = (int64_t)1 << 40;
  for (int i = 0; i < 3; ++i)
    if (mask_strides[i] < 0 || mask_strides[i] > lim || mask_strides[i] % 4 != 0)
      return SDPA_ERR_INVALID;
  if (!aligned(mask, (uintptr_t)(4 * eb))) return SDPA_ERR_INVALID;
  const int64_t nk16 = (a->Nk + 15) / 16 * 16;
  // a unit's whole mask (plus a tile of slack) is read through 32-bit byte
  // offsets
  if ((a->Nq + 256) * mask_strides[2] * eb + (nk16 + 256) * eb > (int64_t)INT32_MAX)
    return SDPA_ERR_UNSUPPORTED;
  const __int128 span = ((__int128)(a->B - 1) * mask_strides[0] +
                         (__int128)(a->H - 1) * mask_strides[1] +
                         (__int128)(a->Nq - 1) * mask_strides[2] + nk16) * eb;
  if (span > (__int128)(INT64_MAX / 2)) return SDPA_ERR_INVALID;
  const int64_t gb = a->grad_f32 ? 4 : 2;
  const int64_t eq = a->B * a->H * a->Nq * a->d, ek = a->B * a->H * a->Nk * a->d;
  if (overlap(mask, (int64_t)span, a->dq, eq * gb) || overlap(mask, (int64_t)span, a->dk, ek * gb) ||
      overlap(mask, (int64_t)span, a->dv, ek * gb) ||
      overlap(mask, (int64_t)span, a->work, a->B * a->H * a->Nq * 4))
    return SDPA_ERR_INVALID;
  a->amask = mask;
  a->amask_kind = kind;
  for (int i = 0; i < 3; ++i) a->am_str[i] = mask_strides[i];
  return SDPA_OK;
}

sdpa_status validate_bwd_block_mask(const uint8_t* mask, int64_t mask_heads, BwdArgs* a) {
  if (mask == nullptr || (mask_heads != 1 && mask_heads != a->H)) return SDPA_ERR_INVALID;
  if (a->cu != nullptr) return SDPA_ERR_INVALID;
  constexpr int64_t blk = SDPA_BLOCK_SPARSE_BLOCK;
  const int64_t nqb = (a->Nq + blk - 1) / blk, nkb = (a->Nk + blk - 1) / blk;
  int64_t mb = 0;
  if (!mul_ok(mask_heads * nqb, nkb, &mb) || mb > INT32_MAX) return SDPA_ERR_INVALID;
  const int64_t gb = a->grad_f32 ? 4 : 2;
  const int64_t eq = a->B * a->H * a->Nq * a->d, ek = a->B * a->H * a->Nk * a->d;
  if (overlap(mask, mb, a->dq, eq * gb) || overlap(mask, mb, a->dk, ek * gb) ||
      overlap(mask, mb, a->dv, ek * gb) || overlap(mask, mb, a->work, a->B * a->H * a->Nq * 4))
    return SDPA_ERR_INVALID;
  a->bmask = mask;
  a->mask_heads = mask_heads;
  return SDPA_OK;
}

sdpa_status validate_dropout(float p, uint64_t seed, uint32_t offset, FwdArgs* a) {
  if (!(p >= 0.f && p < 1.f)) return SDPA_ERR_INVALID;   // NaN fails too
  if (a->dtype == SDPA_F32) return SDPA_ERR_UNSUPPORTED;
  if (p == 0.f) return SDPA_OK;   // no dropout: the plain kernel
  // keep iff a 16-bit number is below T: the keep probability is T / 65536
  // (1 - p rounded to 16 bits), and kept weights are divided by exactly
  // that, so the expected output is the undropped one.  p so close to 1
  // that T rounds to 0 would drop everything: refused.
  const double t = std::floor((1.0 - (double)p) * 65536.0 + 0.5);
  if (t < 1.0) return SDPA_ERR_UNSUPPORTED;
  a->dropout = true;
  a->drop_seed = seed;
  a->drop_offset = offset;
  a->drop_t = (uint32_t)t;
  a->drop_scale = (float)(65536.0 / t);
  return SDPA_OK;
}

sdpa_status validate_bwd_dropout(float p, uint64_t seed, uint32_t offset, BwdArgs* a) {
  if (!(p >= 0.f && p < 1.f)) return SDPA_ERR_INVALID;
  if (p == 0.f) return SDPA_OK;
  // keep iff a 16-bit number is below T: the keep probability is T / 65536
  // (1 - p rounded to 16 bits), and kept weights are divided by exactly
  // that, so the expected output is the undropped one.  p so close to 1
  // that T rounds to 0 would drop everything: refused.
  const double t = std::floor((1.0 - (double)p) * 65536.0 + 0.5);
  if (t < 1.0) return SDPA_ERR_UNSUPPORTED;
  a->dropout = true;
  a->drop_seed = seed;
  a->drop_offset = offset;
  a->drop_t = (uint32_t)t;
  a->drop_scale = (float)(65536.0 / t);
  return SDPA_OK;
}

sdpa_status validate_bwd(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* workspace, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                         int64_t d, float scale, int is_causal, sdpa_dtype dtype,
                         sdpa_dtype out_dtype, sdpa_dtype grad_dtype, void* stream,
                         BwdArgs* a) {
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv || !workspace)
    return SDPA_ERR_INVALID;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return SDPA_ERR_INVALID;
  if (is_causal != 0 && is_causal != 1) return SDPA_ERR_INVALID;
  if (dtype != SDPA_F16 && dtype != SDPA_BF16 && dtype != SDPA_F32) return SDPA_ERR_INVALID;
  if (!std::isfinite(scale)) return SDPA_ERR_INVALID;
  const int64_t lim = (int64_t)1 << 30;
  if (H > lim || Nq > lim || Nk > lim || B > lim) return SDPA_ERR_INVALID;
  int64_t rows_q, rows_k, eq, ek, tmp;
  if (!mul_ok(B, H, &tmp) || !mul_ok(tmp, Nq, &rows_q) || !mul_ok(tmp, Nk, &rows_k) ||
      !mul_ok(rows_q, d, &eq) || !mul_ok(rows_k, d, &ek) || eq > INT64_MAX / 4 ||
      ek > INT64_MAX / 4)
    return SDPA_ERR_INVALID;
  if (tmp * ((std::max(Nq, Nk) + 31) / 32) > INT32_MAX) return SDPA_ERR_INVALID;
  auto kind = [&](sdpa_dtype t, bool* f32) -> sdpa_status {
    if (t == SDPA_SAME || t == dtype) {
      *f32 = dtype == SDPA_F32;
      return SDPA_OK;
    }
    if (t == SDPA_F32) {
      *f32 = true;
      return SDPA_OK;
    }
    return (t == SDPA_F16 || t == SDPA_BF16) ? SDPA_ERR_UNSUPPORTED : SDPA_ERR_INVALID;
  };
  bool out_f32, grad_f32;
  sdpa_status st = kind(out_dtype, &out_f32);
  if (st != SDPA_OK) return st;
  st = kind(grad_dtype, &grad_f32);
  if (st != SDPA_OK) return st;
  // the backward runs on the matrix cores only
  if (dtype == SDPA_F32 || path_for(dtype, d) != 1) return SDPA_ERR_UNSUPPORTED;
  if (scale < 0.f || !std::isfinite(scale * 1.4426950408889634f)) return SDPA_ERR_UNSUPPORTED;
  if ((std::max(Nq, Nk) + 256) * d * 2 > (int64_t)INT32_MAX) return SDPA_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 4))
    return SDPA_ERR_INVALID;
  // outputs must not overlap the inputs or each other
  const int64_t ib = 2, gb = grad_f32 ? 4 : 2, obb = out_f32 ? 4 : 2;
  const void* ins[] = {q, k, v, out, dout, lse, workspace};
  const int64_t inb[] = {eq * ib, ek * ib, ek * ib, eq * obb, eq * ib, rows_q * 4, rows_q * 4};
  const void* outs[] = {dq, dk, dv};
  const int64_t outb[] = {eq * gb, ek * gb, ek * gb};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 7; ++i)
      if (overlap(outs[o], outb[o], ins[i], inb[i])) return SDPA_ERR_INVALID;
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlap(outs[o], outb[o], outs[o2], outb[o2])) return SDPA_ERR_INVALID;
  }
  for (int i = 0; i < 6; ++i)
    if (overlap(workspace, rows_q * 4, ins[i], inb[i])) return SDPA_ERR_INVALID;

  a->q = q;
  a->k = k;
  a->v = v;
  a->out = out;
  a->dout = dout;
  a->lse = lse;
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  a->work = workspace;
  a->cu = nullptr;
  a->T = 0;
  a->amask = nullptr;
  a->amask_kind = SDPA_MASK_BOOL;
  a->am_str[0] = a->am_str[1] = a->am_str[2] = 0;
  a->bmask = nullptr;
  a->mask_heads = 0;
  a->B = B;
  a->H = H;
  a->Nq = Nq;
  a->Nk = Nk;
  a->d = d;
  a->scale = scale;
  a->causal = is_causal != 0;
  a->out_f32 = out_f32;
  a->grad_f32 = grad_f32;
  a->dtype = dtype;
  a->stream = static_cast<hipStream_t>(stream);
  a->dropout = false;
  a->drop_seed = 0;
  a->drop_offset = 0;
  a->drop_t = 65536;
  a->drop_scale = 1.f;
  return SDPA_OK;
}

sdpa_status validate_bwd_packed(const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                float* workspace, int64_t B, int64_t H, int64_t T,
                                int64_t max_seqlen, int64_t d, float scale, int is_causal,
                                const int32_t* cu_seqlens, sdpa_dtype dtype,
                                sdpa_dtype out_dtype, sdpa_dtype grad_dtype, void* stream,
                                BwdArgs* a) {
  if (cu_seqlens == nullptr || !aligned(cu_seqlens, 4)) return SDPA_ERR_INVALID;
  if (B < 1 || max_seqlen < 1 || T < 1) return SDPA_ERR_INVALID;
  const int64_t lim = (int64_t)1 << 30;
  if (B > lim || max_seqlen > lim || T > lim) return SDPA_ERR_INVALID;
  // the [T,H,d] tensors as one unit of T rows: null pointers, types,
  // alignment, sizes and every overlap between outputs and inputs
  const sdpa_status st =
      validate_bwd(q, k, v, out, dout, lse, dq, dk, dv, workspace, 1, H, T, T, d, scale,
                   is_causal, dtype, out_dtype, grad_dtype, stream, a);
  if (st != SDPA_OK) return st;
  int64_t units;
  if (!mul_ok(B, H, &units) || units * ((max_seqlen + 31) / 32) > INT32_MAX)
    return SDPA_ERR_INVALID;
  // one sequence's rows (row stride H*d) within 32-bit buffer offsets
  if ((max_seqlen + 256) * H * d * 2 > (int64_t)INT32_MAX) return SDPA_ERR_UNSUPPORTED;
  a->cu = cu_seqlens;
  a->T = T;
  a->B = B;
  a->Nq = a->Nk = max_seqlen;
  return SDPA_OK;
}

}  // namespace sdpa
