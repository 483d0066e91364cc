// Grid set-up and instantiation of the matrix-core forward for one head dim.
#pragma once

#include <type_traits>

#include "fwd_mfma.h"
#include "sdpa_internal.h"

static_assert(sdpa::kSparseBlock == SDPA_BLOCK_SPARSE_BLOCK, "mask block size");

namespace sdpa {

// Tile shape per head dimension: NB blocks of 32 query rows per wave, NW
// waves, BN keys per step (overridable at build time for tuning sweeps).
#ifndef SDPA_SHAPE_D32
#define SDPA_SHAPE_D32 1, 8, 64
#endif
#ifndef SDPA_SHAPE_D64
#define SDPA_SHAPE_D64 1, 8, 64
#endif
#ifndef SDPA_SHAPE_D128
#define SDPA_SHAPE_D128 1, 8, 32
#endif
template <int NB_, int NW_, int BN_> struct ShapeOf {
  static constexpr int NB = NB_, NW = NW_, BN = BN_;
};
template <int D> struct MfmaShape;
template <> struct MfmaShape<32> : ShapeOf<SDPA_SHAPE_D32> {};
template <> struct MfmaShape<64> : ShapeOf<SDPA_SHAPE_D64> {};
template <> struct MfmaShape<128> : ShapeOf<SDPA_SHAPE_D128> {};

// The wide d = 32 shape for large dense grids: two blocks of 32 query rows
// per wave and 4 waves (256 rows per workgroup), three workgroups per CU.
// A wave's K and V fragment reads and the workgroup's staging then serve
// twice the rows, which measured +1...6% on d = 32 grids of at least 2048
// query tiles of 256 rows (B32 H32 N1024, B16 H16 N4096, B128 H16 N512,
// ...) and +5% with dropout (B32 H32 N1024, against its 128-row shape), but
// 12 resident waves per CU instead of 16 lose 3-15% on smaller grids
// (B2 H16 N4096, B1 H16 N16384), which keep the other shapes.
#ifndef SDPA_WIDE_SHAPE_D32
#define SDPA_WIDE_SHAPE_D32 2, 4, 64
#endif
#ifndef SDPA_WIDE_MIN_TILES
#define SDPA_WIDE_MIN_TILES 2048
#endif
template <int D> struct WideShape : MfmaShape<D> {};
template <> struct WideShape<32> : ShapeOf<SDPA_WIDE_SHAPE_D32> {};

// Packed (variable-length) batches.
#ifndef SDPA_VARLEN_SHAPE_D32
#define SDPA_VARLEN_SHAPE_D32 SDPA_SHAPE_D32
#endif
#ifndef SDPA_VARLEN_SHAPE_D64
#define SDPA_VARLEN_SHAPE_D64 SDPA_SHAPE_D64
#endif
#ifndef SDPA_VARLEN_SHAPE_D128
#define SDPA_VARLEN_SHAPE_D128 SDPA_SHAPE_D128
#endif
template <int D> struct VarlenShape;
template <> struct VarlenShape<32> : ShapeOf<SDPA_VARLEN_SHAPE_D32> {};
template <> struct VarlenShape<64> : ShapeOf<SDPA_VARLEN_SHAPE_D64> {};
template <> struct VarlenShape<128> : ShapeOf<SDPA_VARLEN_SHAPE_D128> {};

// Key groups for grids of few query tiles: 8 waves over 128 query rows, in
// two groups of 4 that take alternate key tiles and merge their states at
// the end.  Against the 256-row shape a workgroup's chain of key steps is
// half as long and the grid has twice the waves, which pays where that grid
// would leave most CUs with one workgroup or none (f16, one MI355X: B1 H16
// N2048 +66/69% at d = 32, +15/21% at d = 64, +33/36% at d = 128,
// non-causal/causal; 256 tiles of 256 rows: d = 32 +16%, causal d = 64 and
// 128 +13...19%, but non-causal d = 64 and 128 -9...25%, as do larger
// grids).  With dropout (same kernels, keep decisions by position) B1 H16
// N2048 gains +26/30%, +54/59% and +46/48%.  Thresholds in query tiles of
// 256 rows (plain and dropout launches, dense or packed):
#ifndef SDPA_SPLIT_TILES_D32
#define SDPA_SPLIT_TILES_D32 256
#endif
#ifndef SDPA_SPLIT_TILES_D64
#define SDPA_SPLIT_TILES_D64 128
#endif
#ifndef SDPA_SPLIT_TILES_D128
#define SDPA_SPLIT_TILES_D128 128
#endif
#ifndef SDPA_SPLIT_TILES_CAUSAL
#define SDPA_SPLIT_TILES_CAUSAL 256
#endif
template <int D> struct SplitShape : ShapeOf<1, 8, MfmaShape<D>::BN> {};
template <int D>
constexpr int64_t kSplitTiles(bool causal) {
  return D == 32 ? SDPA_SPLIT_TILES_D32
                 : causal ? SDPA_SPLIT_TILES_CAUSAL
                          : (D == 64 ? SDPA_SPLIT_TILES_D64 : SDPA_SPLIT_TILES_D128);
}

// Block-sparse shapes: 128 query rows per workgroup, one mask row, so every
// wave of a workgroup needs the same key tiles.
#ifndef SDPA_BSP_SHAPE_D32
#define SDPA_BSP_SHAPE_D32 1, 4, 64
#endif
#ifndef SDPA_BSP_SHAPE_D64
#define SDPA_BSP_SHAPE_D64 1, 4, 32
#endif
#ifndef SDPA_BSP_SHAPE_D128
#define SDPA_BSP_SHAPE_D128 1, 4, 64
#endif
template <int D> struct BspShape;
template <> struct BspShape<32> : ShapeOf<SDPA_BSP_SHAPE_D32> {};
template <> struct BspShape<64> : ShapeOf<SDPA_BSP_SHAPE_D64> {};
template <> struct BspShape<128> : ShapeOf<SDPA_BSP_SHAPE_D128> {};

// Dropout shapes.
#ifndef SDPA_DROP_SHAPE_D32
#define SDPA_DROP_SHAPE_D32 1, 4, 64
#endif
#ifndef SDPA_DROP_SHAPE_D64
#define SDPA_DROP_SHAPE_D64 SDPA_SHAPE_D64
#endif
#ifndef SDPA_DROP_SHAPE_D128
#define SDPA_DROP_SHAPE_D128 SDPA_SHAPE_D128
#endif
template <int D> struct DropShape;
template <> struct DropShape<32> : ShapeOf<SDPA_DROP_SHAPE_D32> {};
template <> struct DropShape<64> : ShapeOf<SDPA_DROP_SHAPE_D64> {};
template <> struct DropShape<128> : ShapeOf<SDPA_DROP_SHAPE_D128> {};

// Elementwise-mask shapes.
#ifndef SDPA_MASK_SHAPE_D32
#define SDPA_MASK_SHAPE_D32 1, 4, 64
#endif
#ifndef SDPA_MASK_SHAPE_D64
#define SDPA_MASK_SHAPE_D64 SDPA_SHAPE_D64
#endif
#ifndef SDPA_MASK_SHAPE_D128
#define SDPA_MASK_SHAPE_D128 SDPA_SHAPE_D128
#endif
template <int D> struct MaskShape;
template <> struct MaskShape<32> : ShapeOf<SDPA_MASK_SHAPE_D32> {};
template <> struct MaskShape<64> : ShapeOf<SDPA_MASK_SHAPE_D64> {};
template <> struct MaskShape<128> : ShapeOf<SDPA_MASK_SHAPE_D128> {};

template <bool BF16, int D, bool CAUSAL, bool VARLEN, bool OUTF32, int VAR = kPlain,
          bool WIDE = false, int KS = 1>
hipError_t launch_mfma_inst(const FwdArgs& a) {
  using S = std::conditional_t<
      VAR == kBlockSparse, BspShape<D>,
      std::conditional_t<
          (KS > 1), SplitShape<D>,
      std::conditional_t<
          WIDE, WideShape<D>,
          std::conditional_t<VAR == kDropout, DropShape<D>,
                             std::conditional_t<(VAR >= kMaskBool), MaskShape<D>,
                                                std::conditional_t<VARLEN, VarlenShape<D>,
                                                                   MfmaShape<D>>>>>>>;
  constexpr int NB = S::NB, NW = S::NW, BN = S::BN;
  using K = MfmaFwd<BF16, D, NB, NW, BN, CAUSAL, VARLEN, OUTF32, VAR, KS>;
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
  p.q_bs = a.q_str[0];
  p.q_hs = a.q_str[1];
  p.q_rs = (int)a.q_str[2];
  p.kv_bs = a.kv_str[0];
  p.kv_hs = a.kv_str[1];
  p.kv_rs = (int)a.kv_str[2];
  p.o_bs = a.o_str[0];
  p.o_hs = a.o_str[1];
  p.o_rs = (int)a.o_str[2];
  p.n_qtiles = (int)((a.Nq + K::BM - 1) / K::BM);
  p.total = (int)(a.B * a.H * p.n_qtiles);
  // scale 0 is carried as a tiny positive multiplier: every visible score
  // becomes 0 to within 1e-30 relative, masked scores stay -inf
  p.c = fmaxf(a.scale * 1.4426950408889634f, 1e-30f);
  p.bmask = a.bmask;
  p.bm_nqb = (int)((a.Nq + kSparseBlock - 1) / kSparseBlock);
  p.bm_nkb = (int)((a.Nk + kSparseBlock - 1) / kSparseBlock);
  p.bm_hstride = a.mask_heads > 1 ? p.bm_nqb * p.bm_nkb : 0;
  p.seed_lo = (uint32_t)(a.drop_seed & 0xffffffffu);
  p.seed_hi = (uint32_t)(a.drop_seed >> 32);
  p.drop_offset = a.drop_offset;
  p.drop_t = a.drop_t;
  p.drop_scale = a.drop_scale;
  p.amask = a.amask;
  p.am_bs = a.am_str[0];
  p.am_hs = a.am_str[1];
  p.am_rs = (int)a.am_str[2];
  hipLaunchKernelGGL((fwd_mfma_kernel<BF16, D, NB, NW, BN, CAUSAL, VARLEN, OUTF32, VAR, KS>), dim3(p.total),
                     dim3(NW * 64), 0, a.stream, p);
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_mfma_d(const FwdArgs& a) {
  const bool varlen = a.cu != nullptr;
  if (a.bmask != nullptr) {   // block-sparse: dense layouts only
    if (varlen) return hipErrorInvalidValue;
    if (a.causal)
      return a.out_f32 ? launch_mfma_inst<BF16, D, true, false, true, kBlockSparse>(a)
                       : launch_mfma_inst<BF16, D, true, false, false, kBlockSparse>(a);
    return a.out_f32 ? launch_mfma_inst<BF16, D, false, false, true, kBlockSparse>(a)
                     : launch_mfma_inst<BF16, D, false, false, false, kBlockSparse>(a);
  }
  // the wide d = 32 shape for large dense grids (plain and dropout)
  if constexpr (D == 32) {
    static_assert(WideShape<32>::NW * WideShape<32>::NB * 32 == 256, "wide tile rows");
    const int64_t tiles = a.B * a.H * ((a.Nq + 255) / 256);
    if (!varlen && tiles >= SDPA_WIDE_MIN_TILES) {
#define SDPA_WCASE(VAR)                                                                     \
      if (a.causal)                                                                         \
        return a.out_f32 ? launch_mfma_inst<BF16, D, true, false, true, VAR, true>(a)       \
                         : launch_mfma_inst<BF16, D, true, false, false, VAR, true>(a);     \
      return a.out_f32 ? launch_mfma_inst<BF16, D, false, false, true, VAR, true>(a)        \
                       : launch_mfma_inst<BF16, D, false, false, false, VAR, true>(a);
      if (a.dropout) {
        SDPA_WCASE(kDropout)
      }
      SDPA_WCASE(kPlain)
#undef SDPA_WCASE
    }
  }
  // key groups for grids of few query tiles (B counts sequences and Nq is
  // the longest one for packed batches)
  const bool split = a.B * a.H * ((a.Nq + 255) / 256) <= kSplitTiles<D>(a.causal);
  if (a.dropout) {
    if (split) {
#define SDPA_SDCASE(C, V, O)                                                 \
      if (a.causal == C && varlen == V && a.out_f32 == O)                    \
        return launch_mfma_inst<BF16, D, C, V, O, kDropout, false, 2>(a);
      SDPA_SDCASE(false, false, false)
      SDPA_SDCASE(false, false, true)
      SDPA_SDCASE(false, true, false)
      SDPA_SDCASE(false, true, true)
      SDPA_SDCASE(true, false, false)
      SDPA_SDCASE(true, false, true)
      SDPA_SDCASE(true, true, false)
      SDPA_SDCASE(true, true, true)
#undef SDPA_SDCASE
    }
#define SDPA_DCASE(C, V, O)                                                  \
    if (a.causal == C && varlen == V && a.out_f32 == O)                      \
      return launch_mfma_inst<BF16, D, C, V, O, kDropout>(a);
    SDPA_DCASE(false, false, false)
    SDPA_DCASE(false, false, true)
    SDPA_DCASE(false, true, false)
    SDPA_DCASE(false, true, true)
    SDPA_DCASE(true, false, false)
    SDPA_DCASE(true, false, true)
    SDPA_DCASE(true, true, false)
    SDPA_DCASE(true, true, true)
#undef SDPA_DCASE
  }
  if (split) {
#define SDPA_SCASE(C, V, O)                                                  \
    if (a.causal == C && varlen == V && a.out_f32 == O)                      \
      return launch_mfma_inst<BF16, D, C, V, O, kPlain, false, 2>(a);
    SDPA_SCASE(false, false, false)
    SDPA_SCASE(false, false, true)
    SDPA_SCASE(false, true, false)
    SDPA_SCASE(false, true, true)
    SDPA_SCASE(true, false, false)
    SDPA_SCASE(true, false, true)
    SDPA_SCASE(true, true, false)
    SDPA_SCASE(true, true, true)
#undef SDPA_SCASE
  }
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

// Elementwise-mask launches (dense layouts, any strides): the dense tile
// shapes, one instantiation per mask kind, causal flag and output type.
template <bool BF16, int D>
hipError_t launch_mfma_masked_d(const FwdArgs& a) {
  if (a.cu != nullptr || a.amask == nullptr) return hipErrorInvalidValue;
  // key groups for grids of few query tiles, as for the plain launches
  if (a.B * a.H * ((a.Nq + 255) / 256) <= kSplitTiles<D>(a.causal)) {
#define SDPA_MSCASE(KIND, VAR)                                                                 \
    if (a.amask_kind == KIND) {                                                               \
      if (a.causal)                                                                           \
        return a.out_f32 ? launch_mfma_inst<BF16, D, true, false, true, VAR, false, 2>(a)     \
                         : launch_mfma_inst<BF16, D, true, false, false, VAR, false, 2>(a);   \
      return a.out_f32 ? launch_mfma_inst<BF16, D, false, false, true, VAR, false, 2>(a)      \
                       : launch_mfma_inst<BF16, D, false, false, false, VAR, false, 2>(a);    \
    }
    SDPA_MSCASE(SDPA_MASK_BOOL, kMaskBool)
    SDPA_MSCASE(SDPA_MASK_ADD, kMaskAdd)
    SDPA_MSCASE(SDPA_MASK_ADD_F32, kMaskAddF32)
#undef SDPA_MSCASE
    return hipErrorInvalidValue;
  }
#define SDPA_MCASE(KIND, VAR)                                                          \
  if (a.amask_kind == KIND) {                                                         \
    if (a.causal)                                                                     \
      return a.out_f32 ? launch_mfma_inst<BF16, D, true, false, true, VAR>(a)         \
                       : launch_mfma_inst<BF16, D, true, false, false, VAR>(a);       \
    return a.out_f32 ? launch_mfma_inst<BF16, D, false, false, true, VAR>(a)          \
                     : launch_mfma_inst<BF16, D, false, false, false, VAR>(a);        \
  }
  SDPA_MCASE(SDPA_MASK_BOOL, kMaskBool)
  SDPA_MCASE(SDPA_MASK_ADD, kMaskAdd)
  SDPA_MCASE(SDPA_MASK_ADD_F32, kMaskAddF32)
  return hipErrorInvalidValue;
}

// An elementwise mask together with dropout (dense layouts, any strides):
// the mask shapes, one instantiation per mask kind, causal flag and output
// type (compiled in translation units of their own).
template <bool BF16, int D>
hipError_t launch_mfma_masked_drop_d(const FwdArgs& a) {
  if (a.cu != nullptr || a.amask == nullptr || !a.dropout) return hipErrorInvalidValue;
  // key groups for grids of few query tiles, as for the plain launches
  if (a.B * a.H * ((a.Nq + 255) / 256) <= kSplitTiles<D>(a.causal)) {
#define SDPA_MSCASE(KIND, VAR)                                                                 \
    if (a.amask_kind == KIND) {                                                               \
      if (a.causal)                                                                           \
        return a.out_f32 ? launch_mfma_inst<BF16, D, true, false, true, VAR, false, 2>(a)     \
                         : launch_mfma_inst<BF16, D, true, false, false, VAR, false, 2>(a);   \
      return a.out_f32 ? launch_mfma_inst<BF16, D, false, false, true, VAR, false, 2>(a)      \
                       : launch_mfma_inst<BF16, D, false, false, false, VAR, false, 2>(a);    \
    }
    SDPA_MSCASE(SDPA_MASK_BOOL, kMaskBoolDrop)
    SDPA_MSCASE(SDPA_MASK_ADD, kMaskAddDrop)
    SDPA_MSCASE(SDPA_MASK_ADD_F32, kMaskAddF32Drop)
#undef SDPA_MSCASE
    return hipErrorInvalidValue;
  }
  SDPA_MCASE(SDPA_MASK_BOOL, kMaskBoolDrop)
  SDPA_MCASE(SDPA_MASK_ADD, kMaskAddDrop)
  SDPA_MCASE(SDPA_MASK_ADD_F32, kMaskAddF32Drop)
#undef SDPA_MCASE
  return hipErrorInvalidValue;
}

}  // namespace sdpa
