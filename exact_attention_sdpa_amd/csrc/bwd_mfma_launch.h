// Grid set-up and instantiation of the matrix-core backward for one head dim.
#pragma once

#include "bwd_mfma.h"
#include "sdpa_internal.h"

namespace sdpa {

// Tile shapes: dq -- NW waves of 32 query rows, BN keys per step;
// dkdv -- NW waves of 32 key rows, BQ query rows per step.
constexpr int kBwdDqWaves = 4, kBwdDqKeys = 32;
constexpr int kBwdKvWaves = 4, kBwdKvRows = 32;

template <bool BF16, int D, bool CAUSAL, bool GF32>
hipError_t launch_bwd_tiles(const BwdArgs& a, BwdParams p) {
  using Q = BwdDq<BF16, D, kBwdDqWaves, kBwdDqKeys, CAUSAL, GF32>;
  using KV = BwdDkdv<BF16, D, kBwdKvWaves, kBwdKvRows, CAUSAL, GF32>;
  p.n_tiles = (int)((a.Nq + Q::BM - 1) / Q::BM);
  p.total = (int)(a.B * a.H * p.n_tiles);
  hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, kBwdDqWaves, kBwdDqKeys, CAUSAL, GF32>),
                     dim3(p.total), dim3(kBwdDqWaves * 64), 0, a.stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  p.n_tiles = (int)((a.Nk + KV::BK - 1) / KV::BK);
  p.total = (int)(a.B * a.H * p.n_tiles);
  hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D, kBwdKvWaves, kBwdKvRows, CAUSAL, GF32>),
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
  // scale 0 is carried as a tiny positive multiplier, as in the forward
  p.c = fmaxf(a.scale * 1.4426950408889634f, 1e-30f);
  p.scale = a.scale;
  // D_i = <dO_i, O_i>
  const int64_t rows = a.B * a.H * a.Nq;
  const dim3 grid((unsigned)((rows + 255) / 256));
  if (a.out_f32)
    hipLaunchKernelGGL((bwd_rowdot_kernel<BF16, D, true>), grid, dim3(256), 0, a.stream, p, rows);
  else
    hipLaunchKernelGGL((bwd_rowdot_kernel<BF16, D, false>), grid, dim3(256), 0, a.stream, p, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.causal)
    return a.grad_f32 ? launch_bwd_tiles<BF16, D, true, true>(a, p)
                      : launch_bwd_tiles<BF16, D, true, false>(a, p);
  return a.grad_f32 ? launch_bwd_tiles<BF16, D, false, true>(a, p)
                    : launch_bwd_tiles<BF16, D, false, false>(a, p);
}

}  // namespace sdpa
