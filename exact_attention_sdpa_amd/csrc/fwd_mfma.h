// Fused attention forward on gfx950 matrix cores (f16 / bf16 inputs).
//
// Method: the FlashAttention tiling (FlashAttention article, method
// paragraph and tiling figure): key/value blocks are staged in on-chip
// memory and the softmax is accumulated block by block, so the N x N score
// matrix never reaches device memory.  The loop order differs from the
// article's figure, which walks key/value blocks in the outer loop and
// writes partial outputs back per block: here one workgroup owns a block
// of query rows for its whole life, streams every key/value block past it
// and writes the output and the row logsumexp exactly once.
//
// Work decomposition
//   grid     one workgroup per (batch or sequence, head, query tile of BM
//            rows); the block index is remapped so that each of the eight
//            XCDs (dispatched round-robin) owns a contiguous range of tiles,
//            and the tiles of one head run back to back on one XCD, sharing
//            K/V in that XCD's L2.  Causal dense grids of up to 16 query
//            tiles per head instead run every head's heaviest query tile
//            first, then the next heaviest, and so on (longest-processing-
//            time order), each XCD keeping its own heads.
//   waves    NW waves; wave w owns NB blocks of 32 query rows.
//   tile     BN keys per step, read with buffer loads whose range check
//            returns zeros past the last key, staged through double-buffered
//            LDS: K row-major [BN][D+8]; V transposed to [D][BN+8] f16 with
//            keys permuted inside each group of 16, so that a lane's V
//            fragment is one 16-byte read.  The row padding and the lane to
//            key-pair assignment of the transposing writes were chosen by
//            measuring LDS bank conflicts on gfx950: both the fragment reads
//            and the writes are conflict-free.
//
// Register dataflow per 32x32 block (v_mfma_f32_32x32x16, wave64):
//   S^T = K . Q^T      A = K rows from LDS, B = Q rows held in VGPRs.
//                      Lane l owns query l%32 and keys 8(r/4)+4(l/32)+r%4,
//                      r = 0..15, so a row max is 15 in-lane ops plus one
//                      v_permlane32_swap exchange with lane l^32.
//   softmax (exp2)     t = s*c - m with c = scale*log2(e) and m a per-row
//                      reference (one fma per score); P = exp2(t).  The
//                      first 32 keys set m to their row maximum.  After that
//                      no maximum is computed at all: every lane's fp32 sum
//                      of its P values bounds each of them, and only if a sum
//                      exceeds 2^15 (an f16 P could overflow) is the block
//                      redone with m raised to the block maximum.  Row sums
//                      accumulate the fp32 P, so the logsumexp is exact to
//                      fp32 rounding.
//   P                  converted to f16 straight from the accumulator
//                      registers (no LDS round trip).
//   O^T += V^T . P^T   A = V^T read from LDS in the key order of P's
//                      registers.  bf16 inputs: V is converted to f16 when
//                      staged (exact for |v| <= 65504).
//   epilogue           O = acc / l, lse = ln2 * (m + log2 l), one store.
//
// Step j: S(j) = K(j) Q^T, the softmax of tile j, P(j) V(j) (the P.V products
// of the first 32 keys are issued under the exponentials of the next 32).
// LDS holds two K and two V buffers, filled from registers loaded one step
// earlier, with one barrier per step.
//
// Block-sparse instantiation (BSP; the FlashAttention article's results
// section benchmarks a block-sparse variant without fixing a mask format):
// a uint8 mask over 128x128 blocks says which key blocks each block of 128
// query rows attends.  A workgroup is then exactly one mask row (128 rows),
// steps only through the key tiles its row keeps (found from a 64-column
// bit set built by one ballot), and never loads the others.  A row's
// reference m is set by the first block in which it sees a key; a row that
// sees none writes O = 0 and lse = -inf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "philox.h"

namespace sdpa {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct MfmaParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* out;
  float* lse;
  const int32_t* cu;   // packed batches: B+1 offsets
  int H;
  int Nq, Nk;          // dense sizes; packed: max sequence length
  // dense layouts: (batch, head, row) strides in elements; k and v share
  // theirs (the element stride along d is 1)
  int64_t q_bs, q_hs, kv_bs, kv_hs, o_bs, o_hs;
  int q_rs, kv_rs, o_rs;
  int n_qtiles;        // query tiles per (batch, head)
  int total;           // grid size
  float c;             // scale * log2(e), at least 1e-30
  // block-sparse launches: mask [Hm][ceil(Nq/128)][ceil(Nk/128)], nonzero =
  // the 128x128 block of (query, key) pairs is visible
  const uint8_t* bmask;
  int bm_hstride;      // bytes between the heads' masks (0: one mask for all)
  int bm_nqb, bm_nkb;  // mask rows and columns
  // dropout launches: keep (query i, key j) of unit u iff a 16-bit number
  // of Philox4x32-10(key = seed, counter = (n(j), i, u, offset)) is below
  // drop_t; kept weights are scaled by drop_scale = 65536 / drop_t
  uint32_t seed_lo, seed_hi, drop_offset, drop_t;
  float drop_scale;
  // elementwise-mask launches: mask element (b, h, i, j) at
  // amask + (b*am_bs + h*am_hs + i*am_rs + j) elements (strides may be 0)
  const void* amask;
  int64_t am_bs, am_hs;
  int am_rs;
};

// Block size of block-sparse masks (query rows x keys).
constexpr int kSparseBlock = 128;

// Kernel variants: plain, block-sparse, dropout on the attention weights,
// and an elementwise attention mask: boolean (one byte per pair, nonzero =
// attend), or additive in the input type or in f32.
enum FwdVariant : int {
  kPlain = 0,
  kBlockSparse = 1,
  kDropout = 2,
  kMaskBool = 3,
  kMaskAdd = 4,
  kMaskAddF32 = 5,
  // an elementwise mask together with dropout (kind + 3)
  kMaskBoolDrop = 6,
  kMaskAddDrop = 7,
  kMaskAddF32Drop = 8
};
// the mask kind of a variant (kMaskBool / kMaskAdd / kMaskAddF32), else VAR
constexpr int mask_kind_of(int var) { return var >= kMaskBoolDrop ? var - 3 : var; }

// Build option: raise the wave priority while it issues matrix-core work
// (measured a few percent faster on MI355X).
#ifndef SDPA_SETPRIO
#define SDPA_SETPRIO 1
#endif
// Build option: waves skip tiles their boolean mask drops entirely.
#ifndef SDPA_MASK_SKIP
#define SDPA_MASK_SKIP 1
#endif
// Debug build option: fill LDS with NaN before it is written (the whole of
// it when a tile starts, and each thread's staging slots after the barrier
// that ends their reads), so that a read of LDS before its data has been
// written -- a missing or misplaced barrier -- turns the output into NaN.
// Built into libsdpa_debug.so only.
#ifndef SDPA_LDS_POISON
#define SDPA_LDS_POISON 0
#endif
// Build option: 16-bit outputs leave through LDS as whole-row segments.
#ifndef SDPA_EPI_LDS
#define SDPA_EPI_LDS 1
#endif
// Build option: causal dense grids in longest-processing-time order.
#ifndef SDPA_CAUSAL_LPT
#define SDPA_CAUSAL_LPT 1
#endif

// A lane whose tile sum of P exceeds this redoes the tile with a raised
// reference, so no f16 P ever exceeds 2^15 (f16 max 65504).
constexpr float kLaneSumLimit = 32768.0f;
// Buffer descriptor word 3 for raw (untyped) 32-bit accesses on gfx9.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ f32x16 mfma_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// max / sum of x over the lane pair (l, l^32).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  f16x2 h = {(_Float16)a, (_Float16)b};  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 h = {(__bf16)a, (__bf16)b};     // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}


// Position of key k (0..BN-1) inside its LDS V^T row: within each group of
// 16 keys, lane half 0 reads keys {0-3, 8-11} and half 1 keys {4-7, 12-15},
// each as 8 contiguous elements.
__host__ __device__ constexpr int vt_key_pos(int k) {
  return (k & ~15) | (k & 3) | ((k & 4) << 1) | ((k & 8) >> 1);
}

template <bool BF16, int D, int NB, int NW, int BN, bool CAUSAL, bool VARLEN, bool OUTF32,
          int VAR = kPlain, int KS = 1>
struct MfmaFwd {
  static constexpr bool BSP = VAR == kBlockSparse;
  static constexpr int MK = mask_kind_of(VAR);
  static constexpr bool DROP = VAR == kDropout || VAR >= kMaskBoolDrop;
  static constexpr bool MASK = VAR >= kMaskBool;
  // mask element bytes = 32-bit words a lane loads per group of 4 keys
  static constexpr int MW = MK == kMaskBool ? 1 : MK == kMaskAdd ? 2 : 4;
  // KS key groups: the workgroup's waves form KS groups of NWG waves over
  // the same query rows; group g takes key tiles g, g + KS, ... and the
  // groups' partial states are merged at the end
  static constexpr int NWG = NW / KS;
  static constexpr int BM = NWG * NB * 32;  // query rows per workgroup
  // epilogue: a wave's 16-bit output rows staged in LDS, rows padded by 16
  // bytes (the LDS area is sized for every wave's rows)
  static constexpr int OROW = D + 8;
  static constexpr int KB = BN / 32;       // 32-key blocks per step
  static constexpr int DS = D / 16;        // k-steps of S = Q K^T
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
  static constexpr int NT = NW * 64;
  static constexpr int NTG = NWG * 64;     // threads of a key group (staging)
  static constexpr int NC = D / 8;         // 16-byte chunks per row
  static constexpr int KROW = D + 8;       // LDS K row, elements
  static constexpr int VRW = BN / 2 + 4;   // LDS V^T row, 32-bit words
  static constexpr int KCHUNKS = BN * NC;        // 16-byte K chunks per tile
  static constexpr int VPAIRS = (BN / 2) * NC;   // (2 rows x 16 bytes) V chunks
  static constexpr int KPT = (KCHUNKS + NTG - 1) / NTG;
  static constexpr int VPT = (VPAIRS + NTG - 1) / NTG;
  static_assert(KS == 1 || (KS == 2 && NW % 2 == 0 && !BSP), "key groups");
  static_assert(D % 32 == 0 && D <= 128, "head dim");
  static_assert(BN % 32 == 0 && BN <= 128, "key block");
  // block-sparse: a workgroup's rows are exactly one mask row, and a key
  // tile never straddles two mask columns
  static_assert(!BSP || (NW * NB * 32 == kSparseBlock && kSparseBlock % BN == 0 && !VARLEN),
                "block-sparse tile shape");
  static_assert(!MASK || !VARLEN, "elementwise masks take dense layouts");

  static constexpr bool EPI_LDS = SDPA_EPI_LDS && !OUTF32;
  static constexpr int KV_BYTES = 2 * KS * (BN * KROW * 2 + D * VRW * 4);
  // key groups: the other group's state (per lane: O, m, l) for the merge,
  // after the epilogue's rows
  static constexpr int MITEMS = 16 * DB + 2;
  static constexpr int MERGE_OFF = EPI_LDS ? NWG * NB * 32 * OROW * 2 : 0;
  static constexpr int EPI_BYTES = MERGE_OFF + (KS > 1 ? NWG * NB * MITEMS * 64 * 4 : 0);
  struct __attribute__((aligned(16))) Smem {
    uint16_t k[2 * KS][BN * KROW];
    uint32_t vt[2 * KS][D * VRW];
    // room for the epilogue's rows where the K/V buffers are smaller
    uint8_t pad[EPI_BYTES > KV_BYTES ? EPI_BYTES - KV_BYTES : 16];
  };
  static_assert(!EPI_LDS || EPI_BYTES <= (int)sizeof(Smem), "epilogue rows fit in LDS");

  struct KRegs { u32x4 k[KPT]; };
  struct VRegs { u32x4 v0[VPT], v1[VPT]; };
  // a lane's mask elements of one tile: per 32-key block, per query block,
  // the 4 groups of 4 keys it owns (keys 8g + 4hl + 0..3)
  struct MaskRegs { uint32_t w[KB][NB][4][MW]; };

  // per-thread constant addressing of the staging copies
  struct Staging {
    int kg[KPT];   // K chunk: byte offset within the tile
    int kl[KPT];   // K chunk: element offset in an LDS K buffer
    int vg[VPT];   // V pair: byte offset of the even row within the tile
    int vl[VPT];   // V pair: word offset in an LDS V^T buffer (d offset 0)
  };

  // per-lane LDS read bases
  struct Lanes {
    int kl;      // K fragment, elements
    int vl[2];   // V^T fragment for hs = 0, 1, words
  };

  // per-head view used by the staging copies
  struct Head {
    const char* k;
    const char* v;
    int kv_bytes;   // byte length of the valid key rows
    int rs_bytes;   // row stride in bytes
  };

  static __device__ __forceinline__ void setup_staging(Staging& st, int64_t rs, int tid) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int c = tid + i * NTG;
      const int row = c / NC, col = (c % NC) * 8;
      st.kg[i] = (int)(((int64_t)row * rs + col) * 2);
      st.kl[i] = row * KROW + col;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int c = tid + i * NTG;
      // consecutive lanes take consecutive key pairs of one column chunk
      const int pr = c % (BN / 2);
      const int col = (c / (BN / 2)) * 8;
      st.vg[i] = (int)(((int64_t)(2 * pr) * rs + col) * 2);
      st.vl[i] = col * VRW + vt_key_pos(2 * pr) / 2;
    }
  }

  static __device__ __forceinline__ Lanes setup_lanes(int l32, int hl) {
    Lanes ln;
    ln.kl = l32 * KROW + hl * 8;
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) ln.vl[hs] = l32 * VRW + hl * 4 + 8 * hs;
    return ln;
  }

  // Buffer view of tile `t` of a head: it starts at the tile and ends at the
  // last valid key row, so rows past it read as zeros (the range check never
  // relies on the hardware applying an offset register).
  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int t,
                                                                     const Head& hd) {
    const int toff = t * BN * hd.rs_bytes;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + toff), (short)0,
                                             max(hd.kv_bytes - toff, 0), kBufferWord3);
  }

  static __device__ __forceinline__ void load_k(KRegs& r, const Staging& st, const Head& hd, int t,
                                                int tid) {
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(hd.k, t, hd);
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (KCHUNKS % NTG == 0 || tid + i * NTG < KCHUNKS)
        r.k[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(kr, st.kg[i], 0, 0));
  }

  static __device__ __forceinline__ void load_v(VRegs& r, const Staging& st, const Head& hd, int t,
                                                int tid) {
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(hd.v, t, hd);
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      if (VPAIRS % NTG == 0 || tid + i * NTG < VPAIRS) {
        r.v0[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, st.vg[i], 0, 0));
        r.v1[i] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(vr, st.vg[i] + hd.rs_bytes, 0, 0));
      }
  }

  static __device__ __forceinline__ void store_k(Smem& sm, int buf, const KRegs& r,
                                                 const Staging& st, int tid) {
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (KCHUNKS % NTG == 0 || tid + i * NTG < KCHUNKS)
        *reinterpret_cast<u32x4*>(&sm.k[buf][st.kl[i]]) = r.k[i];
  }

  // V transposed to [d][key] (f16), keys in vt_key_pos order
  static __device__ __forceinline__ void store_v(Smem& sm, int buf, const VRegs& r,
                                                 const Staging& st, int tid) {
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      if (VPAIRS % NTG == 0 || tid + i * NTG < VPAIRS) {
        uint32_t* dst = &sm.vt[buf][st.vl[i]];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a = r.v0[i][w], b = r.v1[i][w];  // (d 2w, d 2w+1) of keys 2pr, 2pr+1
          if (BF16) {
            // a bf16 value is the upper half of its f32, so one byte
            // permute both widens it and picks it out of the pair (the
            // transpose), and a packing conversion makes the f16 pair
            const auto f = [&](uint32_t sel) { return __uint_as_float(__builtin_amdgcn_perm(b, a, sel)); };
            dst[(2 * w) * VRW] = pack_f16(f(0x01000c0cu), f(0x05040c0cu));
            dst[(2 * w + 1) * VRW] = pack_f16(f(0x03020c0cu), f(0x07060c0cu));
          } else {
            dst[(2 * w) * VRW] = __builtin_amdgcn_perm(b, a, 0x05040100u);
            dst[(2 * w + 1) * VRW] = __builtin_amdgcn_perm(b, a, 0x07060302u);
          }
        }
      }
  }

  // Debug (LDS poisoning): NaN (f16 0x7e00, bf16 0x7fc0) written into every
  // LDS slot this thread stores tiles into, after the barrier that ends the
  // reads of buffer `buf` and before the step that stores the buffer's next
  // tile, so that a wave reading a buffer before its tile has been written
  // -- a missing or misplaced barrier -- computes NaN instead of stale
  // values.  Single 32-bit writes of one constant keep it light on registers.
  static __device__ __forceinline__ void poison_slots(Smem& sm, int buf, const Staging& st,
                                                      int tid) {
    const uint32_t kn = BF16 ? 0x7fc07fc0u : 0x7e007e00u;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      if (KCHUNKS % NTG == 0 || tid + i * NTG < KCHUNKS) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(&sm.k[buf][st.kl[i]]);
#pragma unroll
        for (int w = 0; w < 4; ++w) dst[w] = kn;
      }
#pragma unroll
    for (int i = 0; i < VPT; ++i)
      if (VPAIRS % NTG == 0 || tid + i * NTG < VPAIRS) {
        uint32_t* dst = &sm.vt[buf][st.vl[i]];
#pragma unroll
        for (int w = 0; w < 8; ++w) dst[w * VRW] = 0x7e007e00u;
      }
  }
  // ... and the whole of both buffers, padding included, at the start
  static __device__ __forceinline__ void poison_all(Smem& sm, int tid) {
    uint32_t* w = reinterpret_cast<uint32_t*>(&sm);
    constexpr int NWORDS = (int)(sizeof(Smem) / 4);
    for (int i = tid; i < NWORDS; i += NT) w[i] = 0x7e007e00u;
  }

  // Raw scores S^T = K Q^T for key block kk (32 keys) of the tile in LDS K
  // buffer `buf`.
  static __device__ __forceinline__ void scores(f32x16 (&s)[NB], const Smem& sm, int buf, int kk,
                                                const Lanes& ln, const u32x4 (&qf)[NB][DS]) {
    u32x4 kf[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      kf[ds] = *reinterpret_cast<const u32x4*>(&sm.k[buf][ln.kl + kk * 32 * KROW + ds * 16]);
    if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      f32x16 acc = {};
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        acc = BF16 ? mfma_bf16(kf[ds], qf[qb][ds], acc) : mfma_f16(kf[ds], qf[qb][ds], acc);
      s[qb] = acc;
    }
    if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(0);
  }

  struct State {
    f32x16 o[NB][DB];
    float m[NB];   // row reference, log2 units: t = s*c - m
    float l[NB];
  };

  struct Ctx {
    Staging st;
    Lanes ln;
    Head hd;
    int ntiles, nk, wq0, l32, hl, tid;
    int gtid, bb;   // thread index within its key group; the group's first LDS buffer
    bool wave_live;
    float c;
    const uint8_t* mrow;       // block-sparse: the workgroup's mask row
    int nkb;                   // block-sparse: mask columns
    int mchunk;                // block-sparse: which 64 columns mbits holds
    uint64_t mbits;            // block-sparse: those columns, bit set = kept
    uint32_t unit;             // dropout: b*H + h (packed: sequence*H + h)
    uint32_t seed_lo, seed_hi, doff, dt;   // dropout: key, offset, threshold
    const char* mbase;         // mask: row wq0 of the unit's mask
    int mbytes;                // mask: readable bytes from mbase
    int moff[NB];              // mask: byte offset of the lane's row and first key
  };

  static __device__ __forceinline__ bool skip_tile(const Ctx& x, int t) {
    return !x.wave_live || (KS > 1 && t >= x.ntiles) || (CAUSAL && t * BN > x.wq0 + NB * 32 - 1);
  }

  // Elementwise mask: the lane's elements of tile t, by 32-key block.  The
  // view ends at the wave's last row (keys rounded up to 16), so loads past
  // it read zeros; elements past the last key are never used.
  //   bool, 16-bit: the lane pair (l, l^32) reads the row's block as two
  //   contiguous halves (keys 16hl..16hl+15: one 16-byte load for bytes, two
  //   for 16-bit values), then v_permlane32_swap trades the 4-key groups each
  //   lane does not own for those it does, so that a load instruction
  //   touches each row's cache line once per half block rather than once
  //   per group.
  //   f32: one 16-byte load per 4-key group (a group is 16 bytes already).
  static __device__ __forceinline__ void load_mask(MaskRegs& r, const Ctx& x, int t) {
    const __amdgpu_buffer_rsrc_t mr =
        __builtin_amdgcn_make_buffer_rsrc((void*)x.mbase, (short)0, x.mbytes, kBufferWord3);
#pragma unroll
    for (int kk = 0; kk < KB; ++kk)
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) {
        const int off = x.moff[qb] + (t * BN + kk * 32) * MW;
        uint32_t(&w)[4][MW] = r.w[kk][qb];
        if constexpr (MW == 1) {
          // d[i] = keys 16hl + 4i..4i+3; after the swaps lane hl holds
          // groups g = 0, 2 in d0, d1 and g = 1, 3 in d2, d3
          const u32x4 d = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(mr, off, 0, 0));
          const auto s01 = __builtin_amdgcn_permlane32_swap(d[0], d[1], false, false);
          const auto s23 = __builtin_amdgcn_permlane32_swap(d[2], d[3], false, false);
          w[0][0] = s01[0];
          w[2][0] = s01[1];
          w[1][0] = s23[0];
          w[3][0] = s23[1];
        } else if constexpr (MW == 2) {
          // a = keys 16hl + 0..7, b = keys 16hl + 8..15 (2 per word); after
          // the swaps words 0-1 of a and b hold groups 0 and 1, words 2-3
          // groups 2 and 3
          const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(mr, off, 0, 0));
          const u32x4 b =
              __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(mr, off + 16, 0, 0));
          const auto a0 = __builtin_amdgcn_permlane32_swap(a[0], a[2], false, false);
          const auto a1 = __builtin_amdgcn_permlane32_swap(a[1], a[3], false, false);
          const auto b0 = __builtin_amdgcn_permlane32_swap(b[0], b[2], false, false);
          const auto b1 = __builtin_amdgcn_permlane32_swap(b[1], b[3], false, false);
          w[0][0] = a0[0];
          w[0][1] = a1[0];
          w[2][0] = a0[1];
          w[2][1] = a1[1];
          w[1][0] = b0[0];
          w[1][1] = b1[0];
          w[3][0] = b0[1];
          w[3][1] = b1[1];
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const u32x4 v = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(mr, off + 32 * g, 0, 0));
#pragma unroll
            for (int i = 0; i < MW; ++i) w[g][i] = v[i];
          }
        }
      }
  }

  // Score r of the lane (key 8(r/4) + 4hl + r%4 of its block) in log2
  // units relative to the reference: s c + a log2(e) - mref for an additive
  // mask a, s c - mref or -inf for a boolean one.
  static __device__ __forceinline__ float mask_score(float s, float c, float mref,
                                                     const uint32_t (&w)[4][MW], int r) {
    const int g = r / 4, e = r % 4;
    if (MK == kMaskBool) {
      const uint32_t byte = (w[g][0] >> (8 * e)) & 0xffu;
      return byte != 0u ? __builtin_fmaf(s, c, -mref) : -INFINITY;
    }
    float a;
    if (MK == kMaskAdd) {
      const uint32_t h = (w[g][e / 2] >> (16 * (e & 1))) & 0xffffu;
      a = BF16 ? __uint_as_float(h << 16)
               : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
    } else {
      a = __uint_as_float(w[g][e]);
    }
    return __builtin_fmaf(s, c, __builtin_fmaf(a, 1.4426950408889634f, -mref));
  }

  // Block-sparse: the first tile >= t whose key block the mask row keeps
  // (>= ntiles if none).  The row is read 64 columns at a time, one byte
  // per lane, into a wave-uniform bit set, so the scan waits on memory once
  // per 64 columns rather than once per tile.
  static __device__ __forceinline__ int next_tile(Ctx& x, int t) {
    if (!BSP) return t;
    constexpr int TPB = kSparseBlock / BN;   // key tiles per mask column
    while (t < x.ntiles) {
      const int kc = t / TPB;
      const int chunk = kc >> 6;
      if (chunk != x.mchunk) {
        const int c = chunk * 64 + (int)(x.tid & 63);
        x.mbits = __builtin_amdgcn_ballot_w64(c < x.nkb && x.mrow[c] != 0);
        x.mchunk = chunk;
      }
      const uint64_t rest = x.mbits >> (kc & 63);
      if (rest != 0) return max(t, (kc + (int)__builtin_ctzll(rest)) * TPB);
      t = (chunk + 1) * 64 * TPB;
    }
    return t;
  }

  // ---- softmax update of one tile, one block of 32 keys at a time

  // Causal / key-tail mask on the raw scores of the block at key kb0.
  static __device__ __forceinline__ void mask_block(f32x16 (&s)[NB], int kb0, int nk, int wq0,
                                                    int l32, int hl) {
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      const int qi = wq0 + qb * 32 + l32;
      // register r holds key base + 8(r/4) + r%4; it is visible iff that
      // offset is at most lim (below nk and, when causal, at most qi), so
      // each score costs one compare with a constant and one select
      const int base = kb0 + 4 * hl;
      const int lim = CAUSAL ? min(nk - 1, qi) - base : nk - 1 - base;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r / 4) + (r % 4) > lim) s[qb][r] = -INFINITY;
    }
  }

  // Row maximum over the block (4 chains, then the lane pair l, l^32).
  static __device__ __forceinline__ float row_max(const f32x16& t) {
    float x[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int r = 0; r < 16; ++r) x[r & 3] = fmaxf(x[r & 3], t[r]);
    return pair_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  }

  // P = exp2(t) of a block: the lane's fp32 sums (two partial sums per row)
  // and the f16 B operands of P V.
  static __device__ __forceinline__ void exp_block(const f32x16 (&t)[NB], float (&bs)[NB][2],
                                                   u32x4 (&pf)[NB][2]) {
#pragma unroll
    for (int qb = 0; qb < NB; ++qb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e0 = __builtin_amdgcn_exp2f(t[qb][8 * hs + 2 * i]);
          const float e1 = __builtin_amdgcn_exp2f(t[qb][8 * hs + 2 * i + 1]);
          if (hs == 0 && i == 0) {
            bs[qb][0] = e0;
            bs[qb][1] = e1;
          } else {
            bs[qb][0] += e0;
            bs[qb][1] += e1;
          }
          w[i] = pack_f16(e0, e1);
        }
        pf[qb][hs] = u32x4{w[0], w[1], w[2], w[3]};
      }
  }

  // Dropout on the block of 32 keys at kb0: zero the f16 P of the dropped
  // (query, key) pairs.  Lane (row i, half hl) holds, in pf[qb][hs] word w,
  // keys kb0 + 16 hs + 4 hl + {0, 1, 2, 3} + 8 (w >> 1) as pairs (2(w&1),
  // 2(w&1)+1): exactly the 8 keys of Philox call n = kb0/8 + 2 hs + hl of
  // row i, whose output word w carries their two 16-bit numbers (low half
  // = first key of the pair).  The row sums keep the undropped P; the
  // 65536/T scale (the inverse keep probability) is applied to O at the end.
  static __device__ __forceinline__ void drop_block(u32x4 (&pf)[NB][2], int kb0, const Ctx& x) {
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      const uint32_t row = (uint32_t)(x.wq0 + qb * 32 + x.l32);
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        uint32_t r[4];
        philox4x32_10((uint32_t)(kb0 >> 3) + 2 * hs + x.hl, row, x.unit, x.doff, x.seed_lo,
                      x.seed_hi, r);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          // r16 - T has its upper 16 bits all set iff r16 < T (T <= 65536);
          // one byte permute gathers both halves' upper bytes into the
          // pair's mask
          const uint32_t dlo = (r[w] & 0xffffu) - x.dt;
          const uint32_t dhi = (r[w] >> 16) - x.dt;
          pf[qb][hs][w] &= __builtin_amdgcn_perm(dhi, dlo, 0x07060302u);
        }
      }
    }
  }

  // One tile, one block of 32 keys at a time: S of block kk, its softmax,
  // P V of block kk, then S of block kk+1 (issuing S(kk+1) ahead of the
  // softmax of block kk took 16 more VGPRs and measured 1.5% slower on long
  // sequences: the other waves of the SIMD already overlap the two).
  //   t = s*c - m (one fma per score), P = exp2(t).
  // The first block of the first tile sets m to its row maximum (finite:
  // key 0 is visible to every row).  After that no row maximum is taken:
  // each P is at most its lane's block sum, so one compare per block proves
  // that no f16 P can overflow.  A lane over the limit (rare) raises its
  // row to the block maximum, O and l are rescaled in place, and the
  // block's exponentials are redone.
  static __device__ __forceinline__ void tile(const Smem& sm, int buf, int kb, bool first,
                                              bool masked, const Ctx& x, const u32x4 (&qf)[NB][DS],
                                              State& S, const MaskRegs& mr) {
    f32x16 sc[NB];
    scores(sc, sm, buf, 0, x.ln, qf);
#pragma unroll
    for (int kk = 0; kk < KB; ++kk) {
      if (masked && !MASK) mask_block(sc, kb + kk * 32, x.nk, x.wq0, x.l32, x.hl);
      if (MASK) {
        // the mask's bias is folded into the scaled scores first; pairs the
        // causal rule or the key tail excludes are then set to -inf whatever
        // the mask holds there.  A row's reference is set by the first block
        // in which it has a finite score.
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
          const float mref = S.m[qb] == -INFINITY ? 0.f : S.m[qb];
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sc[qb][r] = mask_score(sc[qb][r], x.c, mref, mr.w[kk][qb], r);
        }
        if (masked) mask_block(sc, kb + kk * 32, x.nk, x.wq0, x.l32, x.hl);
        bool unset = false;
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) unset = unset || S.m[qb] == -INFINITY;
        if (__builtin_amdgcn_ballot_w64(unset) != 0) {
#pragma unroll
          for (int qb = 0; qb < NB; ++qb) {
            const float mm = row_max(sc[qb]);
            const bool set_now = S.m[qb] == -INFINITY && mm > -INFINITY;
            const float sub = set_now ? mm : 0.f;
            if (set_now) S.m[qb] = mm;
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[qb][r] -= sub;
          }
        }
      } else if (BSP) {
        // block-sparse: a row's reference is set by the first block in
        // which it sees a key (its first visible block can be anywhere)
        bool unset = false;
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) unset = unset || S.m[qb] == -INFINITY;
        if (__builtin_amdgcn_ballot_w64(unset) != 0) {
#pragma unroll
          for (int qb = 0; qb < NB; ++qb) {
            const float mm = row_max(sc[qb]) * x.c;
            if (S.m[qb] == -INFINITY) S.m[qb] = mm;
          }
        }
      } else if (kk == 0 && first) {
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) S.m[qb] = row_max(sc[qb]) * x.c;
      }
      if (!MASK) {
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
          // rows that have not seen a key yet have only -inf scores here
          const float mref = (BSP && S.m[qb] == -INFINITY) ? 0.f : S.m[qb];
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[qb][r] = __builtin_fmaf(sc[qb][r], x.c, -mref);
        }
      }
      float bs[NB][2];
      u32x4 pf[NB][2];
      exp_block(sc, bs, pf);
      bool over = false;
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) over = over || !(bs[qb][0] + bs[qb][1] <= kLaneSumLimit);
      if (__builtin_amdgcn_ballot_w64(over) != 0) {
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
          // rows with nothing to raise take y = 0 (a no-op), so no per-lane
          // branch splits the accumulators' live ranges
          const float y = fmaxf(row_max(sc[qb]), 0.f);
          const float alpha = __builtin_amdgcn_exp2f(-y);
          S.m[qb] += y;
          S.l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) S.o[qb][db][r] *= alpha;
#pragma unroll
          for (int r = 0; r < 16; ++r) sc[qb][r] -= y;
        }
        exp_block(sc, bs, pf);
      }
      if (DROP) drop_block(pf, kb + kk * 32, x);
      if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x4 vf = *reinterpret_cast<const u32x4*>(
              &sm.vt[buf][x.ln.vl[hs] + db * 32 * VRW + 16 * kk]);
#pragma unroll
          for (int qb = 0; qb < NB; ++qb) S.o[qb][db] = mfma_f16(vf, pf[qb][hs], S.o[qb][db]);
        }
      if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) S.l[qb] += bs[qb][0] + bs[qb][1];
      if (kk + 1 < KB) scores(sc, sm, buf, kk + 1, x.ln, qf);
    }
  }

  // Step j (K and V of tile j in buffers B): loads tile jn (the next tile
  // to process, j+1 unless block-sparse) into registers; S(j), softmax and
  // P.V of tile j; stores tile jn into buffers B^1; barrier.
  template <int B>
  static __device__ __forceinline__ void step(Smem& sm, const Ctx& x, State& S,
                                              const u32x4 (&qf)[NB][DS], int j, int jn) {
    KRegs kr;
    VRegs vr;
    MaskRegs mr;
    const bool nxt = jn < x.ntiles;
    const bool live = !skip_tile(x, j);
    // the mask of tile j is requested before the next tile's K and V, so
    // its wait does not include theirs (requesting it a step ahead, into a
    // second register set, measured slower)
    if (MASK && live) load_mask(mr, x, j);
    if (nxt) {
      load_k(kr, x.st, x.hd, jn, x.gtid);
      load_v(vr, x.st, x.hd, jn, x.gtid);
    }
    // boolean masks: a tile whose mask drops every pair of the wave's rows
    // adds nothing (its P would be exactly 0), so the wave skips it, e.g.
    // the keys past a sequence's end under a key-padding mask
    bool run_tile = live;
    if (MK == kMaskBool && SDPA_MASK_SKIP && live) {
      uint32_t any = 0;
#pragma unroll
      for (int kk = 0; kk < KB; ++kk)
#pragma unroll
        for (int qb = 0; qb < NB; ++qb)
#pragma unroll
          for (int g = 0; g < 4; ++g) any |= mr.w[kk][qb][g][0];
      run_tile = __builtin_amdgcn_ballot_w64(any != 0u) != 0;
    }
    if (run_tile) {
      const int kb = j * BN;
      const bool masked = (kb + BN > x.nk) || (CAUSAL && kb + BN - 1 > x.wq0);
      tile(sm, x.bb + B, kb, !BSP && (KS == 1 ? j == 0 : j < KS), masked, x, qf, S, mr);
    }
    if (nxt) {
      store_k(sm, x.bb + (B ^ 1), kr, x.st, x.gtid);
      store_v(sm, x.bb + (B ^ 1), vr, x.st, x.gtid);
    }
    __syncthreads();
    // every read of buffer B ended at this barrier; the step after next
    // stores its next tile there
    if (SDPA_LDS_POISON) poison_slots(sm, x.bb + B, x.st, x.gtid);
  }

  static __device__ void run(const MfmaParams& p, Smem& sm) {
    Ctx x;
    x.tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(x.tid / 64);   // wave-uniform
    const int grp = KS > 1 ? wave / NWG : 0;   // key group
    x.gtid = KS > 1 ? x.tid % NTG : x.tid;
    x.bb = KS > 1 ? 2 * grp : 0;
    x.hl = (x.tid >> 5) & 1;
    x.l32 = x.tid & 31;
    x.c = p.c;

    // ---- which tile: XCD-contiguous ranges; causal: heaviest tiles first
    int qt, bh;
    if (CAUSAL && !VARLEN && SDPA_CAUSAL_LPT && p.n_qtiles * BM <= 16 * 256) {
      // causal, short sequences (at most 4096 rows): every head's heaviest
      // query tiles first,
      // then the next heaviest of every head, ... (longest-processing-time
      // order, which shortens the tail when many heads have few tiles);
      // each XCD keeps its own eighth of the heads when the head count
      // allows.  Long sequences keep a head's tiles back to back: their
      // order is already near the ideal, and interleaving heads doubles the
      // K/V re-reads that reach past L2.
      const int nbh = p.total / p.n_qtiles;
      int rank;
      if ((nbh & 7) == 0) {
        const int hp = nbh >> 3, j = blockIdx.x >> 3;
        bh = (blockIdx.x & 7) * hp + j % hp;
        rank = j / hp;
      } else {
        bh = blockIdx.x % nbh;
        rank = blockIdx.x / nbh;
      }
      qt = p.n_qtiles - 1 - rank;
    } else {
      int tile = blockIdx.x;
      if ((p.total & 7) == 0) {
        const int per = p.total >> 3;
        tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
      }
      qt = tile % p.n_qtiles;
      bh = tile / p.n_qtiles;
      if (CAUSAL) qt = p.n_qtiles - 1 - qt;
    }
    const int b = bh / p.H, h = bh % p.H;

    int nq, nk;
    int64_t qoff, kvoff, ooff, rs, qrs, ors;
    if (VARLEN) {
      const int s0 = p.cu[b], s1 = p.cu[b + 1];
      nq = nk = s1 - s0;
      rs = qrs = ors = (int64_t)p.H * D;
      qoff = kvoff = ooff = (int64_t)s0 * rs + (int64_t)h * D;
    } else {
      nq = p.Nq;
      nk = p.Nk;
      rs = p.kv_rs;
      qrs = p.q_rs;
      ors = p.o_rs;
      qoff = (int64_t)b * p.q_bs + (int64_t)h * p.q_hs;
      kvoff = (int64_t)b * p.kv_bs + (int64_t)h * p.kv_hs;
      ooff = (int64_t)b * p.o_bs + (int64_t)h * p.o_hs;
    }
    const int q0 = qt * BM;
    if (q0 >= nq) return;  // whole workgroup: tile past the sequence end
    x.nk = nk;

    x.hd.rs_bytes = (int)(rs * 2);
    x.hd.kv_bytes = (int)(((int64_t)(nk - 1) * rs + D) * 2);
    x.hd.k = reinterpret_cast<const char*>(p.k + kvoff);
    x.hd.v = reinterpret_cast<const char*>(p.v + kvoff);
    const int q_bytes = (int)(((int64_t)(nq - 1) * qrs + D) * 2);
    const int q_rs_bytes = (int)(qrs * 2);
    const __amdgpu_buffer_rsrc_t qr =
        __builtin_amdgcn_make_buffer_rsrc((void*)(p.q + qoff), (short)0, q_bytes, kBufferWord3);

    const int kend = CAUSAL ? min(nk, q0 + BM) : nk;
    x.ntiles = (kend + BN - 1) / BN;
    x.wq0 = q0 + (KS > 1 ? wave % NWG : wave) * NB * 32;   // first query row of this wave
    x.wave_live = x.wq0 < nq;
    if (DROP) {
      x.unit = (uint32_t)bh;
      x.seed_lo = p.seed_lo;
      x.seed_hi = p.seed_hi;
      x.doff = p.drop_offset;
      x.dt = p.drop_t;
    }
    if (MASK && x.wave_live) {
      const int rows = min(NB * 32, nq - x.wq0);
      x.mbase = reinterpret_cast<const char*>(p.amask) +
                ((int64_t)b * p.am_bs + (int64_t)h * p.am_hs + (int64_t)x.wq0 * p.am_rs) * MW;
      x.mbytes = (int)(((int64_t)(rows - 1) * p.am_rs + ((nk + 15) & ~15)) * MW);
      // bool / 16-bit: the lane's half block starts at key 16hl; f32: its
      // first group at key 4hl
      const int k0 = MW == 4 ? 4 * x.hl : 16 * x.hl;
#pragma unroll
      for (int qb = 0; qb < NB; ++qb) x.moff[qb] = ((qb * 32 + x.l32) * p.am_rs + k0) * MW;
    }
    if (BSP) {
      x.mrow = p.bmask + (int64_t)(bh % p.H) * p.bm_hstride + (int64_t)qt * p.bm_nkb;
      x.nkb = p.bm_nkb;
      x.mchunk = -1;
      x.mbits = 0;
    }

    // ---- Q rows as the B operand of S^T = K Q^T
    u32x4 qf[NB][DS];
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      const int qi = x.wq0 + qb * 32 + x.l32;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        qf[qb][ds] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, qi * q_rs_bytes + (ds * 16 + x.hl * 8) * 2, 0, 0));
    }

    State S;
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      S.m[qb] = (BSP || MASK) ? -INFINITY : 0.f;
      S.l[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) S.o[qb][db][r] = 0.f;
    }

    setup_staging(x.st, rs, x.gtid);
    x.ln = setup_lanes(x.l32, x.hl);

    if (SDPA_LDS_POISON) {
      poison_all(sm, x.tid);
      __syncthreads();
    }

    // ---- prologue: the first tile staged
    int j = KS > 1 ? grp : next_tile(x, 0);
    if (j < x.ntiles) {
      KRegs k0;
      VRegs v0;
      load_k(k0, x.st, x.hd, j, x.gtid);
      load_v(v0, x.st, x.hd, j, x.gtid);
      store_k(sm, x.bb, k0, x.st, x.gtid);
      store_v(sm, x.bb, v0, x.st, x.gtid);
    }
    __syncthreads();

    if (!BSP && KS == 1) {
      for (; j < x.ntiles; j += 2) {
        step<0>(sm, x, S, qf, j, j + 1);
        if (j + 1 < x.ntiles) step<1>(sm, x, S, qf, j + 1, j + 2);
      }
    } else if (!BSP) {
      // every group makes the same number of steps (one barrier each); a
      // group past its last tile only waits at them
      const int nsteps = (x.ntiles + KS - 1) / KS;
      for (int s = 0; s < nsteps; s += 2, j += 2 * KS) {
        step<0>(sm, x, S, qf, j, j + KS);
        if (s + 1 < nsteps) step<1>(sm, x, S, qf, j + KS, j + 2 * KS);
      }
    } else {
      while (j < x.ntiles) {
        int jn = next_tile(x, j + 1);
        step<0>(sm, x, S, qf, j, jn);
        if (jn >= x.ntiles) break;
        j = jn;
        jn = next_tile(x, j + 1);
        step<1>(sm, x, S, qf, j, jn);
        j = jn;
      }
    }

    // ---- epilogue: normalise, store O and lse once
    // (debug poisoning: the last step's poison writes end before any wave
    // stages its output rows in LDS)
    if (SDPA_LDS_POISON && EPI_LDS) __syncthreads();
    if constexpr (KS > 1) {
      // key groups: group 1 hands its state to group 0 through LDS (every
      // read of the K/V buffers ended at the last step's barrier); group 0
      // brings both states to the larger reference m and adds them
      float* mg = reinterpret_cast<float*>(reinterpret_cast<char*>(&sm) + MERGE_OFF) +
                  (wave % NWG) * NB * MITEMS * 64 + x.tid % 64;
      if (grp == 1 && x.wave_live) {
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
          float* e = mg + qb * MITEMS * 64;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) e[(db * 16 + r) * 64] = S.o[qb][db][r];
          e[(16 * DB) * 64] = S.m[qb];
          e[(16 * DB + 1) * 64] = S.l[qb];
        }
      }
      __syncthreads();
      if (grp != 0) return;
      // group 1 starts at tile 1; a wave that skips it skips every tile of
      // that group (causal: its rows end before key BN)
      if (!skip_tile(x, 1)) {
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
          const float* e = mg + qb * MITEMS * 64;
          const float m1 = e[(16 * DB) * 64], l1 = e[(16 * DB + 1) * 64];
          const float m = fmaxf(S.m[qb], m1);
          // masks: a group in which the row saw no key has m = -inf and
          // nothing to add (both: the row stays empty, m = -inf)
          const float a0 = (MASK && S.m[qb] == -INFINITY) ? 0.f
                                                          : __builtin_amdgcn_exp2f(S.m[qb] - m);
          const float a1 = (MASK && m1 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
          S.m[qb] = m;
          S.l[qb] = S.l[qb] * a0 + l1 * a1;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              S.o[qb][db][r] = S.o[qb][db][r] * a0 + e[(db * 16 + r) * 64] * a1;
        }
      }
    }
    if (!x.wave_live) return;
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      const int qi = x.wq0 + qb * 32 + x.l32;
      const float lt = pair_sum(S.l[qb]);
      // block-sparse or masked rows that saw no key: O = 0, lse = -inf
      const float inv = ((BSP || MASK) && !(lt > 0.f)) ? 0.f : (DROP ? p.drop_scale : 1.f) / lt;
      if (EPI_LDS) {
        // 16-bit output: the block's 32 rows go through this wave's own LDS
        // area (every read of the K/V buffers ended at the last step's
        // barrier) and leave as whole-row segments, 16 bytes per lane, so
        // that one store covers 1 KB of rows instead of 16 bytes of each of
        // 32 rows
        uint16_t* ow = reinterpret_cast<uint16_t*>(&sm) + ((x.tid / 64) * NB + qb) * 32 * OROW;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dcol = db * 32 + 8 * g + 4 * x.hl;
            const float x0 = S.o[qb][db][4 * g + 0] * inv, x1 = S.o[qb][db][4 * g + 1] * inv;
            const float x2 = S.o[qb][db][4 * g + 2] * inv, x3 = S.o[qb][db][4 * g + 3] * inv;
            *reinterpret_cast<u32x2*>(&ow[x.l32 * OROW + dcol]) =
                BF16 ? u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)}
                     : u32x2{pack_f16(x0, x1), pack_f16(x2, x3)};
          }
        const int lane = x.tid % 64;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) {
          const int c = i * 64 + lane;              // 16-byte chunk of the block
          const int row = c / (D / 8), col = (c % (D / 8)) * 8;
          const int qr = x.wq0 + qb * 32 + row;
          const u32x4 v = *reinterpret_cast<const u32x4*>(&ow[row * OROW + col]);
          if (qr < nq)
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + ooff +
                                      (int64_t)qr * ors + col) = v;
        }
      }
      if (qi < nq) {
#pragma unroll
        for (int db = 0; db < (EPI_LDS ? 0 : DB); ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dcol = db * 32 + 8 * g + 4 * x.hl;
            const float x0 = S.o[qb][db][4 * g + 0] * inv, x1 = S.o[qb][db][4 * g + 1] * inv;
            const float x2 = S.o[qb][db][4 * g + 2] * inv, x3 = S.o[qb][db][4 * g + 3] * inv;
            const int64_t off = ooff + (int64_t)qi * ors + dcol;
            if (OUTF32) {
              *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + off) =
                  f32x4{x0, x1, x2, x3};
            } else {
              const u32x2 w = BF16 ? u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)}
                                   : u32x2{pack_f16(x0, x1), pack_f16(x2, x3)};
              *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + off) = w;
            }
          }
        if (p.lse != nullptr && x.hl == 0) {
          const float lse = (S.m[qb] + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f;
          if (VARLEN)
            p.lse[(int64_t)(p.cu[b] + qi) * p.H + h] = lse;
          else
            p.lse[(int64_t)bh * p.Nq + qi] = lse;
        }
      }
    }
  }
};

// Waves per SIMD the register allocation is fitted to, per head dimension.
// An 8-wave workgroup takes 2 waves of every SIMD, so only 4 (two
// workgroups per CU) or 2 (one) are worth fitting to: d = 128 holds 168-170
// VGPRs at 2 without spilling, where a bound of 3 spilled 8-12 and ran 24-29%
// slower.
#ifndef SDPA_WAVES_D32
#define SDPA_WAVES_D32 4
#endif
#ifndef SDPA_WAVES_D64
#define SDPA_WAVES_D64 4
#endif
#ifndef SDPA_WAVES_D128
#define SDPA_WAVES_D128 2
#endif
template <int D>
constexpr int kWavesPerSimd = D == 32 ? SDPA_WAVES_D32 : D == 64 ? SDPA_WAVES_D64 : SDPA_WAVES_D128;
// the block-sparse kernels (4 waves of 128 rows: twice the staging
// registers per lane of the 8-wave dense shapes)
#ifndef SDPA_BSP_WAVES_D32
#define SDPA_BSP_WAVES_D32 4
#endif
#ifndef SDPA_BSP_WAVES_D64
#define SDPA_BSP_WAVES_D64 4
#endif
#ifndef SDPA_BSP_WAVES_D128
#define SDPA_BSP_WAVES_D128 2
#endif
template <int D>
constexpr int kBspWavesPerSimd =
    D == 32 ? SDPA_BSP_WAVES_D32 : D == 64 ? SDPA_BSP_WAVES_D64 : SDPA_BSP_WAVES_D128;
// the dropout kernels (the Philox rounds need about ten more live
// registers).  At d = 64 the bound of 4 waves keeps them within 128 VGPRs,
// so two 8-wave workgroups share a CU: a kernel of 129 registers runs one
// workgroup per CU and measured 20% slower on the causal workload.
#ifndef SDPA_DROP_WAVES_D32
#define SDPA_DROP_WAVES_D32 4
#endif
#ifndef SDPA_DROP_WAVES_D64
#define SDPA_DROP_WAVES_D64 4
#endif
#ifndef SDPA_DROP_WAVES_D128
#define SDPA_DROP_WAVES_D128 2
#endif
template <int D>
constexpr int kDropWavesPerSimd =
    D == 32 ? SDPA_DROP_WAVES_D32 : D == 64 ? SDPA_DROP_WAVES_D64 : SDPA_DROP_WAVES_D128;
// the elementwise-mask kernels (a tile's mask elements are held in
// registers while it is processed).  Two 8-wave workgroups share a CU only
// at 4 waves per SIMD (at most 128 VGPRs): boolean and 16-bit additive
// masks fit at d = 64 without spilling; f32 masks (32 more registers of
// mask per tile) would spill 28 VGPRs and keep 3.
#ifndef SDPA_MASK_WAVES_D32
#define SDPA_MASK_WAVES_D32 4
#endif
#ifndef SDPA_MASK_WAVES_D64
#define SDPA_MASK_WAVES_D64 4
#endif
#ifndef SDPA_MASK_WAVES_D128
#define SDPA_MASK_WAVES_D128 2
#endif
#ifndef SDPA_MASKF_WAVES_D32
#define SDPA_MASKF_WAVES_D32 4
#endif
#ifndef SDPA_MASKF_WAVES_D64
#define SDPA_MASKF_WAVES_D64 3
#endif
#ifndef SDPA_MASKF_WAVES_D128
#define SDPA_MASKF_WAVES_D128 2
#endif
#ifndef SDPA_MASKB_WAVES_D32
#define SDPA_MASKB_WAVES_D32 4
#endif
#ifndef SDPA_MASKB_WAVES_D64
#define SDPA_MASKB_WAVES_D64 4
#endif
#ifndef SDPA_MASKB_WAVES_D128
#define SDPA_MASKB_WAVES_D128 2
#endif
template <int D, int VAR>
constexpr int kMaskWavesPerSimd =
    mask_kind_of(VAR) == kMaskBool
        ? (D == 32 ? SDPA_MASKB_WAVES_D32 : D == 64 ? SDPA_MASKB_WAVES_D64 : SDPA_MASKB_WAVES_D128)
    : mask_kind_of(VAR) == kMaskAddF32
        ? (D == 32 ? SDPA_MASKF_WAVES_D32 : D == 64 ? SDPA_MASKF_WAVES_D64 : SDPA_MASKF_WAVES_D128)
        : (D == 32 ? SDPA_MASK_WAVES_D32 : D == 64 ? SDPA_MASK_WAVES_D64 : SDPA_MASK_WAVES_D128);
// a 16-bit additive mask with dropout holds both register sets: it takes
// the f32 masks' bound (4 waves per SIMD at d = 64 would spill)
template <int D, int VAR>
constexpr int kVariantWavesPerSimd = VAR == kBlockSparse  ? kBspWavesPerSimd<D>
                                     : VAR == kDropout    ? kDropWavesPerSimd<D>
                                     : VAR == kMaskAddDrop ? kMaskWavesPerSimd<D, kMaskAddF32>
                                     : VAR >= kMaskBool   ? kMaskWavesPerSimd<D, VAR>
                                                          : kWavesPerSimd<D>;

// two query blocks per wave (the wide d = 32 shape: 4-wave workgroups, three
// per CU): 149 VGPRs at 3 waves per SIMD, 24-33 spilled at 4
#ifndef SDPA_WIDE_WAVES
#define SDPA_WIDE_WAVES 3
#endif
template <int NB, int D, int VAR>
constexpr int kKernelWavesPerSimd = NB > 1 ? SDPA_WIDE_WAVES : kVariantWavesPerSimd<D, VAR>;

template <bool BF16, int D, int NB, int NW, int BN, bool CAUSAL, bool VARLEN, bool OUTF32,
          int VAR = kPlain, int KS = 1>
__global__ __launch_bounds__(NW * 64, (kKernelWavesPerSimd<NB, D, VAR>)) void
fwd_mfma_kernel(MfmaParams p) {
  using K = MfmaFwd<BF16, D, NB, NW, BN, CAUSAL, VARLEN, OUTF32, VAR, KS>;
  __shared__ typename K::Smem sm;
  K::run(p, sm);
}

}  // namespace sdpa
