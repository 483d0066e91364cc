// Grid set-up and instantiation of the matrix-core backward for one head dim.
#pragma once

#include "bwd_mfma.h"
#include "sdpa_internal.h"

namespace sdpa {

// Tile shapes: dq -- NW waves of 32 query rows, BN keys per step;
// dkdv -- NW waves of 32 key rows, BQ query rows per step.
#ifndef SDPA_BWD_DQ_KEYS_D32
#define SDPA_BWD_DQ_KEYS_D32 64
#endif
#ifndef SDPA_BWD_DQ_KEYS_D64
#define SDPA_BWD_DQ_KEYS_D64 32
#endif
#ifndef SDPA_BWD_KV_ROWS_D32
#define SDPA_BWD_KV_ROWS_D32 64
#endif
#ifndef SDPA_BWD_KV_ROWS_D64
#define SDPA_BWD_KV_ROWS_D64 32
#endif
// Waves per workgroup (32 rows or keys each).  8 for the unmasked d = 32
// kernels without dropout: a step's staged tile is shared by twice the
// waves at the same occupancy, +5% on B32 H32 N1024.  Block-sparse kernels
// need exactly one 128-row mask block per workgroup; masked ones stage a
// mask tile that grows with the workgroup's keys; the dropout dK/dV kernel
// runs at 3 waves per SIMD, where an 8-wave workgroup leaves room for only
// one per CU (-12% measured).
#ifndef SDPA_BWD_WAVES_D32
#define SDPA_BWD_WAVES_D32 8
#endif
template <int D, int MK, bool DROP>
constexpr int kBwdWaves = MK == kPlain && !DROP && D == 32 ? SDPA_BWD_WAVES_D32 : 4;
// Keys (dQ) and query rows (dK/dV) per step.  64 at d = 32 for the unmasked
// kernels: half the steps and barriers, +5.5% on B32 H32 N1024; the masked
// ones stage a mask tile per step in LDS, which at 64 rows would halve
// their resident workgroups, and at d = 64 the doubled K/V and Q/dO tiles
// cost occupancy the same way (-35...-45% measured).
template <int D, int MK>
constexpr int kBwdDqKeys =
    MK != kPlain ? 32 : D == 32 ? SDPA_BWD_DQ_KEYS_D32 : D == 64 ? SDPA_BWD_DQ_KEYS_D64 : 32;
template <int D, int MK>
constexpr int kBwdKvRows =
    MK != kPlain ? 32 : D == 32 ? SDPA_BWD_KV_ROWS_D32 : D == 64 ? SDPA_BWD_KV_ROWS_D64 : 32;

// dQ and dK/dV with two groups of waves on grids of few tiles: 8 waves
// over 128 query rows (dQ) or keys (dK/dV), in two groups of 4 that take
// alternate key (query) tiles and add their sums at the end, so that small
// grids hold twice the waves.  The
// thresholds count tiles of 256 rows over the keys, as the forward's do
// over the queries.  Plain and dropout kernels (unmasked) at d = 32 and 64,
// and dQ at d = 128 (there an 8-wave dK/dV workgroup spills 15-42 VGPRs
// even at 2 waves per SIMD).  Measured on the whole backward (f16, one MI355X, A/B):
// B1 H16 N2048 d = 64 +26/30% plain and +21/25% with dropout
// (non-causal/causal), d = 32 with dropout +22/29%; causal grids of 256
// tiles +17...32%.  Non-causal grids of 256 tiles lost 8-10% at d = 32
// with dropout (dK/dV split alone), hence 128 there.
#ifndef SDPA_BWD_SPLIT_TILES_D32
#define SDPA_BWD_SPLIT_TILES_D32 128
#endif
#ifndef SDPA_BWD_SPLIT_TILES_D64
#define SDPA_BWD_SPLIT_TILES_D64 128
#endif
#ifndef SDPA_BWD_SPLIT_TILES_D128
#define SDPA_BWD_SPLIT_TILES_D128 128
#endif
#ifndef SDPA_BWD_SPLIT_TILES_CAUSAL
#define SDPA_BWD_SPLIT_TILES_CAUSAL 256
#endif
template <int D>
constexpr int64_t kBwdSplitTiles(bool causal) {
  return causal ? SDPA_BWD_SPLIT_TILES_CAUSAL
                : D == 32 ? SDPA_BWD_SPLIT_TILES_D32
                          : (D == 64 ? SDPA_BWD_SPLIT_TILES_D64 : SDPA_BWD_SPLIT_TILES_D128);
}

template <bool BF16, int D, bool CAUSAL, bool GF32, bool DROP, bool VARLEN, int MK = kPlain>
hipError_t launch_bwd_tiles(const BwdArgs& a, BwdParams p) {
  using Q = BwdDq<BF16, D, kBwdWaves<D, MK, DROP>, kBwdDqKeys<D, MK>, CAUSAL, GF32, DROP, VARLEN, MK>;
  using KV = BwdDkdv<BF16, D, kBwdWaves<D, MK, DROP>, kBwdKvRows<D, MK>, CAUSAL, GF32, DROP, VARLEN, MK>;
  constexpr int NWK = kBwdWaves<D, MK, DROP>;
  // the split kernels: 8 waves in two groups of 4 (128 rows or keys per
  // workgroup; the 8-wave d = 32 kernels cover 256, so their split grid has
  // twice the workgroups).  d = 128: the dQ kernel's two groups fit 2
  // waves per SIMD, the dK/dV kernel's do not.
  constexpr bool kCanSplitDq = MK != kBlockSparse;
  constexpr bool kCanSplit = kCanSplitDq && D != 128;
  bool dq_done = false;
  if constexpr (kCanSplitDq) {
    // dQ with two key groups over the same 128 query rows
    if (a.B * a.H * ((a.Nq + 255) / 256) <= kBwdSplitTiles<D>(CAUSAL)) {
      using Q2 = BwdDq<BF16, D, 8, kBwdDqKeys<D, MK>, CAUSAL, GF32, DROP, VARLEN, MK, 2>;
      p.n_tiles = (int)((a.Nq + Q2::BM - 1) / Q2::BM);
      p.total = (int)(a.B * a.H * p.n_tiles);
      hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, 8, kBwdDqKeys<D, MK>, CAUSAL, GF32, DROP, VARLEN, MK, 2>),
                         dim3(p.total), dim3(8 * 64), 0, a.stream, p);
      dq_done = true;
    }
  }
  if (!dq_done) {
    p.n_tiles = (int)((a.Nq + Q::BM - 1) / Q::BM);
    p.total = (int)(a.B * a.H * p.n_tiles);
    hipLaunchKernelGGL((bwd_dq_kernel<BF16, D, NWK, kBwdDqKeys<D, MK>, CAUSAL, GF32, DROP, VARLEN, MK>),
                       dim3(p.total), dim3(NWK * 64), 0, a.stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (kCanSplit) {
    if (a.B * a.H * ((a.Nk + 255) / 256) <= kBwdSplitTiles<D>(CAUSAL)) {
      using KV2 = BwdDkdv<BF16, D, 8, kBwdKvRows<D, MK>, CAUSAL, GF32, DROP, VARLEN, MK, 2>;
      p.n_tiles = (int)((a.Nk + KV2::BK - 1) / KV2::BK);
      p.total = (int)(a.B * a.H * p.n_tiles);
      hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D, 8, kBwdKvRows<D, MK>, CAUSAL, GF32, DROP, VARLEN, MK, 2>),
                         dim3(p.total), dim3(8 * 64), 0, a.stream, p);
      return hipGetLastError();
    }
  }
  p.n_tiles = (int)((a.Nk + KV::BK - 1) / KV::BK);
  p.total = (int)(a.B * a.H * p.n_tiles);
  hipLaunchKernelGGL((bwd_dkdv_kernel<BF16, D, NWK, kBwdKvRows<D, MK>, CAUSAL, GF32, DROP, VARLEN, MK>),
                     dim3(p.total), dim3(NWK * 64), 0, a.stream, p);
  return hipGetLastError();
}

// Elementwise-mask backward (dense layouts, no dropout): one instantiation
// per mask kind, causal flag and gradient type.  Defined in
// bwd_mfma_mask_*.hip.
template <bool BF16, int D>
hipError_t launch_bwd_masked_tiles(const BwdArgs& a, const BwdParams& p);
template <> hipError_t launch_bwd_masked_tiles<false, 32>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_masked_tiles<false, 64>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_masked_tiles<false, 128>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_masked_tiles<true, 32>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_masked_tiles<true, 64>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_masked_tiles<true, 128>(const BwdArgs&, const BwdParams&);

// Elementwise mask together with dropout.  Defined in bwd_mfma_maskdrop_*.hip.
template <bool BF16, int D>
hipError_t launch_bwd_masked_drop_tiles(const BwdArgs& a, const BwdParams& p);
template <> hipError_t launch_bwd_masked_drop_tiles<false, 32>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_masked_drop_tiles<false, 64>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_masked_drop_tiles<false, 128>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_masked_drop_tiles<true, 32>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_masked_drop_tiles<true, 64>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_masked_drop_tiles<true, 128>(const BwdArgs&, const BwdParams&);

// Block-sparse backward (dense layouts, no dropout).  Defined in
// bwd_mfma_mask_*.hip.
template <bool BF16, int D>
hipError_t launch_bwd_bsp_tiles(const BwdArgs& a, const BwdParams& p);
template <> hipError_t launch_bwd_bsp_tiles<false, 32>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_bsp_tiles<false, 64>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_bsp_tiles<false, 128>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_bsp_tiles<true, 32>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_bsp_tiles<true, 64>(const BwdArgs&, const BwdParams&);
template <> hipError_t launch_bwd_bsp_tiles<true, 128>(const BwdArgs&, const BwdParams&);

template <bool BF16, int D>
hipError_t launch_bwd_bsp_tiles_impl(const BwdArgs& a, const BwdParams& p) {
  if (a.causal)
    return a.grad_f32 ? launch_bwd_tiles<BF16, D, true, true, false, false, kBlockSparse>(a, p)
                      : launch_bwd_tiles<BF16, D, true, false, false, false, kBlockSparse>(a, p);
  return a.grad_f32 ? launch_bwd_tiles<BF16, D, false, true, false, false, kBlockSparse>(a, p)
                    : launch_bwd_tiles<BF16, D, false, false, false, false, kBlockSparse>(a, p);
}

// DROP: the mask together with dropout (compiled in translation units of
// their own).
template <bool BF16, int D, bool DROP = false>
hipError_t launch_bwd_masked_tiles_impl(const BwdArgs& a, const BwdParams& p) {
#define SDPA_MBCASE(KIND, MK)                                                            \
  if (a.amask_kind == KIND) {                                                           \
    if (a.causal)                                                                       \
      return a.grad_f32 ? launch_bwd_tiles<BF16, D, true, true, DROP, false, MK>(a, p)   \
                        : launch_bwd_tiles<BF16, D, true, false, DROP, false, MK>(a, p); \
    return a.grad_f32 ? launch_bwd_tiles<BF16, D, false, true, DROP, false, MK>(a, p)    \
                      : launch_bwd_tiles<BF16, D, false, false, DROP, false, MK>(a, p);  \
  }
  SDPA_MBCASE(SDPA_MASK_BOOL, kMaskBool)
  SDPA_MBCASE(SDPA_MASK_ADD, kMaskAdd)
  SDPA_MBCASE(SDPA_MASK_ADD_F32, kMaskAddF32)
#undef SDPA_MBCASE
  return hipErrorInvalidValue;
}

template <bool BF16, int D>
hipError_t launch_bwd_d(const BwdArgs& a, bool with_mask = false) {
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
  p.rc = 1.f / p.c;
  p.scale = a.scale;
  p.seed_lo = (uint32_t)(a.drop_seed & 0xffffffffu);
  p.seed_hi = (uint32_t)(a.drop_seed >> 32);
  p.drop_offset = a.drop_offset;
  p.drop_t = a.drop_t;
  p.drop_scale = a.drop_scale;
  p.bmask = a.bmask;
  p.bm_nqb = (int)((a.Nq + kSparseBlock - 1) / kSparseBlock);
  p.bm_nkb = (int)((a.Nk + kSparseBlock - 1) / kSparseBlock);
  p.bm_hstride = a.mask_heads > 1 ? p.bm_nqb * p.bm_nkb : 0;
  p.amask = a.amask;
  p.am_bs = a.am_str[0];
  p.am_hs = a.am_str[1];
  p.am_rs = (int)a.am_str[2];
  // D_i = <dO_i, O_i> (with dropout O is the dropped output, and D is still
  // sum_j P_ij dP_ij with dP the gradient of the undropped weights)
  // rows of O / dO: [B,H,Nq] dense, [T,H] packed (both flat, row stride d)
  // (computed by the dQ kernel, which runs first, unless built without)
  p.out_f32 = a.out_f32 ? 1 : 0;
  if constexpr (!SDPA_BWD_FUSED_ROWDOT) {
    const int64_t rows = a.cu != nullptr ? a.T * a.H : a.B * a.H * a.Nq;
    const dim3 grid((unsigned)((rows + 255) / 256));
    if (a.out_f32)
      hipLaunchKernelGGL((bwd_rowdot_kernel<BF16, D, true>), grid, dim3(256), 0, a.stream, p, rows);
    else
      hipLaunchKernelGGL((bwd_rowdot_kernel<BF16, D, false>), grid, dim3(256), 0, a.stream, p, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (with_mask)
    return a.bmask != nullptr ? launch_bwd_bsp_tiles<BF16, D>(a, p)
           : a.dropout        ? launch_bwd_masked_drop_tiles<BF16, D>(a, p)
                              : launch_bwd_masked_tiles<BF16, D>(a, p);
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
