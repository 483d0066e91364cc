// Grid set-up and instantiation of the matrix-core backward for one head dim.
#pragma once

#include "bwd_mfma.h"
#include "sdpa_internal.h"

namespace sdpa {

// Tile shapes: dq -- NW waves of 32 query rows, BN keys per step;
// dkdv -- NW waves of 32 key rows, BQ query rows per step.
constexpr int kBwdDqWaves = 4, kBwdDqKeys = 32;
constexpr int kBwdKvWaves = 4, kBwdKvRows = 32;

template <bool BF16, int D, bool CAUSAL, bool GF32, bool DROP, bool VARLEN>
hipError_t launch_bwd_tiles(const BwdArgs& a, BwdParams p) {
  using Q = BwdDq<BF16, D, kBwdDqWaves, kBwdDqKeys, CAUSAL, GF32, DROP, VARLEN>;
  using KV = BwdDkdv<BF16, D, kBwdKvWaves, kBwdKvRows, CAUSAL, GF32, DROP, VARLEN>;
  p.n_tiles = (int)((a.Nq + Q::BM - 1) / Q::BM);
  p.total = (int)(a.B * a.H * p.n_tiles);
  hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, kBwdDqWaves, kBwdDqKeys, CAUSAL, GF32, DROP, VARLEN>),
                     dim3(p.total), dim3(kBwdDqWaves * 64), 0, a.stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  p.n_tiles = (int)((a.Nk + KV::BK - 1) / KV::BK);
  p.total = (int)(a.B * a.H * p.n_tiles);
  hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D, kBwdKvWaves, kBwdKvRows, CAUSAL, GF32, DROP, VARLEN>),
                     dim3(p.total), dim3(kBwdKvWaves * 64), 0, a.stream, p);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_bwd_d(const BwdArgs& a) {
  BwdParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.out = a.out;
  p.dout = static_cast<const uint16_t*>(a.dout);
  p.lse = a.lse;
  p.dsum = a.work;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.H = (int)a.H;
  p.Nq = (int)a.Nq;
  p.Nk = (int)a.Nk;
  p.cu = a.cu;
  // scale 0 is carried as a tiny positive multiplier, as in the forward
  p.c = fmaxf(a.scale * 1.4426950408889634f, 1e-30f);
  p.scale = a.scale;
  p.seed_lo = (uint32_t)(a.drop_seed & 0xffffffffu);
  p.seed_hi = (uint32_t)(a.drop_seed >> 32);
  p.drop_offset = a.drop_offset;
  p.drop_t = a.drop_t;
  p.drop_scale = a.drop_scale;
  // D_i = <dO_i, O_i> (with dropout O is the dropped output, and D is still
  // sum_j P_ij dP_ij with dP the gradient of the undropped weights)
  // rows of O / dO: [B,H,Nq] dense, [T,H] packed (both flat, row stride d)
  const int64_t rows = a.cu != nullptr ? a.T * a.H : a.B * a.H * a.Nq;
  const dim3 grid((unsigned)((rows + 255) / 256));
  if (a.out_f32)
    hipLaunchKernelGGL((bwd_rowdot_kernel<BF16, D, true>), grid, dim3(256), 0, a.stream, p, rows);
  else
    hipLaunchKernelGGL((bwd_rowdot_kernel<BF16, D, false>), grid, dim3(256), 0, a.stream, p, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool varlen = a.cu != nullptr;
#define SDPA_BCASE(C, G, X, V)                                                \
  if (a.causal == C && a.grad_f32 == G && a.dropout == X && varlen == V)      \
    return launch_bwd_tiles<BF16, D, C, G, X, V>(a, p);
#define SDPA_BCASES(V)        \
  SDPA_BCASE(false, false, false, V) \
  SDPA_BCASE(false, true, false, V)  \
  SDPA_BCASE(true, false, false, V)  \
  SDPA_BCASE(true, true, false, V)   \
  SDPA_BCASE(false, false, true, V)  \
  SDPA_BCASE(false, true, true, V)   \
  SDPA_BCASE(true, false, true, V)   \
  SDPA_BCASE(true, true, true, V)
  SDPA_BCASES(false)
  SDPA_BCASES(true)
#undef SDPA_BCASES
#undef SDPA_BCASE
  return hipErrorInvalidValue;
}

}  // namespace sdpa
