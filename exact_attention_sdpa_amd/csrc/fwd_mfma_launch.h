// Grid set-up and instantiation of the matrix-core forward for one head dim.
#pragma once

#include "fwd_mfma.h"
#include "sdpa_internal.h"

namespace sdpa {

// Tile shape per head dimension: NB blocks of 32 query rows per wave, NW waves.
template <int D> struct MfmaShape { static constexpr int NB = 1, NW = 4; };

template <bool BF16, int D, bool CAUSAL, bool VARLEN, bool OUTF32>
hipError_t launch_mfma_inst(const FwdArgs& a) {
  constexpr int NB = MfmaShape<D>::NB, NW = MfmaShape<D>::NW;
  using K = MfmaFwd<BF16, D, NB, NW, CAUSAL, VARLEN, OUTF32>;
  MfmaParams p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.k = static_cast<const uint16_t*>(a.k);
  p.v = static_cast<const uint16_t*>(a.v);
  p.out = a.out;
  p.lse = a.lse;
  p.cu = a.cu;
  p.H = (int)a.H;
  p.Nq = (int)a.Nq;
  p.Nk = (int)a.Nk;
  p.n_qtiles = (int)((a.Nq + K::BM - 1) / K::BM);
  p.total = (int)(a.B * a.H * p.n_qtiles);
  p.c = a.scale * 1.4426950408889634f;
  hipLaunchKernelGGL((fwd_mfma_kernel<BF16, D, NB, NW, CAUSAL, VARLEN, OUTF32>), dim3(p.total),
                     dim3(NW * 64), 0, a.stream, p);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_mfma_d(const FwdArgs& a) {
  const bool varlen = a.cu != nullptr;
#define SDPA_CASE(C, V, O)                                                   \
  if (a.causal == C && varlen == V && a.out_f32 == O)                        \
    return launch_mfma_inst<BF16, D, C, V, O>(a);
  SDPA_CASE(false, false, false)
  SDPA_CASE(false, false, true)
  SDPA_CASE(false, true, false)
  SDPA_CASE(false, true, true)
  SDPA_CASE(true, false, false)
  SDPA_CASE(true, false, true)
  SDPA_CASE(true, true, false)
  SDPA_CASE(true, true, true)
#undef SDPA_CASE
  return hipErrorInvalidValue;
}

}  // namespace sdpa
