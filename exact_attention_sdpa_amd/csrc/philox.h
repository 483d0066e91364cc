// Philox4x32-10 counter-based generator on the GPU.
//
// From its published definition: J. K. Salmon, M. A. Moraes, R. O. Dror and
// D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011.  One
// round maps the counter (c0, c1, c2, c3) under the key (k0, k1) to
//   (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1, lo(M0*c0))
// with 32x32 -> 64-bit products; the key advances by the Weyl constants (the
// 32-bit fractions of the golden ratio and of sqrt(3)) between rounds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

// a ^ b ^ k in one instruction (gfx950's three-input bitwise op; table 0x96
// is the odd-parity function), with k wave-uniform.
__device__ __forceinline__ uint32_t xor3_uniform(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1, uint32_t (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = xor3_uniform((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3_uniform((uint32_t)(p0 >> 32), c3, k1);
    c0 = n0;
    c1 = (uint32_t)p1;
    c2 = n2;
    c3 = (uint32_t)p0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

}  // namespace sdpa
