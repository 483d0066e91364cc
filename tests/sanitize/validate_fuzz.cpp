// Host fuzz driver for the C ABI's argument checks (sdpa_validate.cpp),
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_validate_sanitized.py.  The checks make no HIP calls and never
// dereference the device pointers they are given, so fake addresses serve.
//
// Every call runs on seeded random arguments mixing ordinary sizes with
// edge values (0, 1, negative, powers of two around the int32 and int64
// limits) and fake pointers (null, misaligned, overlapping).  The driver
// checks the few outcomes that are fixed regardless of the other
// arguments and otherwise relies on the sanitizers: any signed overflow,
// shift out of range, or out-of-bounds access aborts the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "sdpa_internal.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;

uint64_t next() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int64_t edge_int() {
  static const int64_t edges[] = {0,
                                  1,
                                  2,
                                  3,
                                  7,
                                  31,
                                  32,
                                  33,
                                  64,
                                  128,
                                  129,
                                  1000,
                                  65536,
                                  (int64_t)1 << 30,
                                  ((int64_t)1 << 30) + 1,
                                  (int64_t)1 << 31,
                                  INT32_MAX,
                                  (int64_t)INT32_MAX + 1,
                                  (int64_t)1 << 40,
                                  (int64_t)1 << 62,
                                  INT64_MAX,
                                  -1,
                                  -8,
                                  INT64_MIN};
  const uint64_t r = next();
  if (r % 3 == 0) return (int64_t)(next() % 4096);
  return edges[r % (sizeof(edges) / sizeof(edges[0]))];
}

float edge_float() {
  static const float edges[] = {0.f,  0.125f, 1.f, -1.f, 1e-30f, 1e30f, 3.4e38f,
                                -0.f, 0.5f,   0.99999f, 1.0f - 1e-7f,
                                std::numeric_limits<float>::infinity(),
                                std::numeric_limits<float>::quiet_NaN()};
  return edges[next() % (sizeof(edges) / sizeof(edges[0]))];
}

// fake device addresses: far apart and 256-byte aligned, or null, or
// misaligned, or equal to another one (overlap)
const void* fake_ptr(int slot) {
  const uint64_t r = next() % 16;
  if (r == 0) return nullptr;
  uintptr_t base = (uintptr_t)(slot + 1) << 40;
  if (r == 1) base += 2;          // misaligned
  if (r == 2) base = (uintptr_t)1 << 40;  // collides with slot 0
  return reinterpret_cast<const void*>(base);
}

sdpa_dtype any_dtype() {
  static const int v[] = {SDPA_F16, SDPA_BF16, SDPA_F32, SDPA_SAME, 7, -1, INT32_MIN, INT32_MAX};
  return (sdpa_dtype)v[next() % 8];
}

int failures = 0;
long accepted_fwd = 0, accepted_bwd = 0;
void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "unexpected outcome: %s\n", what);
    ++failures;
  }
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 200000;
  for (long it = 0; it < iters; ++it) {
    // half the draws take plausible sizes, so that the deeper checks (strides,
    // masks, dropout) see accepted arguments often
    const bool sane = (next() & 1) != 0;
    static const int64_t dims[] = {8, 24, 32, 64, 128};
    const int64_t B = sane ? 1 + (int64_t)(next() % 4) : edge_int();
    const int64_t H = sane ? 1 + (int64_t)(next() % 8) : edge_int();
    const int64_t Nq = sane ? 1 + (int64_t)(next() % 2048) : edge_int();
    const int64_t Nk = sane ? (next() & 1 ? Nq : 1 + (int64_t)(next() % 2048)) : edge_int();
    const int64_t d = sane ? dims[next() % 5] : edge_int();
    const float scale = sane ? 0.125f : edge_float();
    const int causal = (int)(next() % (sane ? 2 : 3));
    const sdpa_dtype dt = sane ? (sdpa_dtype)(next() % 3) : any_dtype();
    const sdpa_dtype odt = sane ? (next() & 1 ? SDPA_SAME : SDPA_F32) : any_dtype();
    const int32_t* cu = (next() & 1) ? reinterpret_cast<const int32_t*>(fake_ptr(6)) : nullptr;

    sdpa::FwdArgs a;
    const sdpa_status st =
        sdpa::validate(fake_ptr(0), fake_ptr(1), fake_ptr(2), const_cast<void*>(fake_ptr(3)),
                       reinterpret_cast<float*>(const_cast<void*>(fake_ptr(4))), B, H, Nq, Nk, d,
                       scale, causal, cu, dt, odt, nullptr, &a, (next() & 1) != 0);
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) expect(st == SDPA_ERR_INVALID, "bad sizes");
    if (!std::isfinite(scale)) expect(st == SDPA_ERR_INVALID, "non-finite scale");
    if (causal > 1) expect(st == SDPA_ERR_INVALID, "is_causal not 0/1");
    if (st == SDPA_OK) {
      ++accepted_fwd;
      // strides, masks and dropout on accepted forward arguments
      int64_t qs[3], ks[3], os[3];
      for (int i = 0; i < 3; ++i) {
        qs[i] = edge_int();
        ks[i] = edge_int();
        os[i] = edge_int();
      }
      sdpa::FwdArgs b = a;
      (void)sdpa::validate_strides(qs, ks, os, &b);
      b = a;
      (void)sdpa::validate_block_mask(reinterpret_cast<const uint8_t*>(fake_ptr(7)), edge_int(),
                                      &b);
      b = a;
      int64_t ms[3] = {edge_int(), edge_int(), edge_int()};
      (void)sdpa::validate_attn_mask(fake_ptr(8), (sdpa_mask_kind)(int32_t)next(), ms, &b);
      b = a;
      const float p = edge_float();
      const sdpa_status sd = sdpa::validate_dropout(p, next(), (uint32_t)next(), &b);
      if (!(p >= 0.f && p < 1.f)) expect(sd == SDPA_ERR_INVALID, "dropout p outside [0, 1)");
      if (sd == SDPA_OK && b.dropout)
        expect(b.drop_t >= 1 && b.drop_t <= 65536 && std::isfinite(b.drop_scale),
               "dropout threshold and scale");
    }

    sdpa::BwdArgs g;
    const sdpa_status sb = sdpa::validate_bwd(
        fake_ptr(0), fake_ptr(1), fake_ptr(2), fake_ptr(3), fake_ptr(9),
        reinterpret_cast<const float*>(fake_ptr(4)), const_cast<void*>(fake_ptr(10)),
        const_cast<void*>(fake_ptr(11)), const_cast<void*>(fake_ptr(12)),
        reinterpret_cast<float*>(const_cast<void*>(fake_ptr(13))), B, H, Nq, Nk, d, scale, causal,
        dt, odt, any_dtype(), nullptr, &g);
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) expect(sb == SDPA_ERR_INVALID, "bwd sizes");
    if (sb == SDPA_OK) {
      ++accepted_bwd;
      sdpa::BwdArgs c = g;
      (void)sdpa::validate_bwd_dropout(edge_float(), next(), (uint32_t)next(), &c);
      c = g;
      int64_t ms[3] = {edge_int(), edge_int(), edge_int()};
      (void)sdpa::validate_bwd_attn_mask(fake_ptr(8), (sdpa_mask_kind)(int32_t)next(), ms, &c);
      c = g;
      (void)sdpa::validate_bwd_block_mask(reinterpret_cast<const uint8_t*>(fake_ptr(7)),
                                          edge_int(), &c);
    }

    sdpa::BwdArgs pk;
    (void)sdpa::validate_bwd_packed(
        fake_ptr(0), fake_ptr(1), fake_ptr(2), fake_ptr(3), fake_ptr(9),
        reinterpret_cast<const float*>(fake_ptr(4)), const_cast<void*>(fake_ptr(10)),
        const_cast<void*>(fake_ptr(11)), const_cast<void*>(fake_ptr(12)),
        reinterpret_cast<float*>(const_cast<void*>(fake_ptr(13))), B, H, edge_int(), Nq, d, scale,
        causal, reinterpret_cast<const int32_t*>(fake_ptr(6)), dt, odt, any_dtype(), nullptr, &pk);
    (void)sdpa::path_for(dt, d);
  }
  std::printf("validate fuzz: %ld iterations, accepted %ld forward and %ld backward calls, "
              "%d unexpected outcomes\n", iters, accepted_fwd, accepted_bwd, failures);
  return failures == 0 ? 0 : 1;
}
