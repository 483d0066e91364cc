// Attention backward on gfx950 matrix cores (f16 / bf16 inputs).
//
// Method: the FlashAttention article (method paragraph) names recomputation
// in the backward pass as its second technique: the N x N probabilities are
// not kept from the forward pass but rebuilt tile by tile from Q, K and the
// stored logsumexp.  The gradients are the chain rule of the exact forward
// definition:
//   P = exp(scale*Q K^T - lse)          (rows already normalised)
//   dV = P^T dO,   dP = dO V^T,   D_i = <dO_i, O_i> = sum_j P_ij dP_ij
//   dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q
//
// Two kernels, no atomics (deterministic):
//   dq       one wave per 32 query rows (lanes own queries, as in the
//            forward): D_i = <dO_i, O_i> in fp32 from the wave's dO operand
//            registers and its rows of O (written out for dkdv); S^T = K Q^T
//            and dP^T = V dO^T on the matrix cores, P and dS in registers,
//            dQ^T += K^T dS^T with K^T staged in LDS in the key order of
//            dS's registers.
//   dkdv     one wave per 32 key rows (lanes own keys): S = Q K^T and
//            dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS, with Q^T
//            and dO^T staged in LDS in the query order of P's registers;
//            launched after dq, whose D it reads.
// (Built with SDPA_BWD_FUSED_ROWDOT=0, a third kernel, rowdot, computes D
// first, one thread per row.)
// Matrix-core layout of v_mfma_f32_32x32x16 (measured, see the forward):
// A lane l holds row l%32, k-slots 8(l/32)..+7; B lane l holds column l%32,
// the same k-slots; C lane l, register r holds row 8(r/4)+4(l/32)+r%4,
// column l%32.  Products whose k index comes from an accumulator use the
// accumulator's register order as the k order, and the other operand is
// staged permuted to match (vt_key_pos).
// Operand types of the products dV = P^T dO, dK = Q^T dS and dQ = dS K:
// the input type.  bf16 inputs keep the transposed copies of Q, dO and K in
// bf16 and round P and dS to bf16, so these products run on the bf16
// matrix cores with dO, Q and K exact and the whole bf16 exponent range
// (upstream gradients of 1e-8 and below stay exact operands; f16 copies
// would flush them); P and dS carry bf16's relative rounding, 2^-8.
// f16 inputs round P and dS to f16 (2^-11).
#pragma once

#include <type_traits>

#include "fwd_mfma.h"

namespace sdpa {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const void* out;        // forward output O (input dtype or f32)
  const uint16_t* dout;   // upstream gradient dO (input dtype)
  const float* lse;       // [B,H,Nq] dense, [T,H] packed; natural log
  float* dsum;            // workspace of the same layout: <dO_i, O_i>
  const int32_t* cu;      // packed batches: B+1 sequence offsets
  void* dq;
  void* dk;
  void* dv;
  int H, Nq, Nk;          // packed: Nq = Nk = the longest sequence
  int n_tiles;            // tiles per head of the launched kernel
  int total;              // grid size
  float c;                // scale * log2(e)
  float rc;               // 1 / c
  float scale;
  // dropout (the forward's Philox contract): key, last counter word, keep
  // threshold on the 16-bit numbers, 65536 / T (the inverse keep probability)
  uint32_t seed_lo, seed_hi, drop_offset, drop_t;
  float drop_scale;
  // elementwise mask (dense layouts): element (b, h, i, j) at
  // amask + (b*am_bs + h*am_hs + i*am_rs + j) elements; bool bytes, or an
  // additive bias in the input type or f32
  const void* amask;
  int64_t am_bs, am_hs;
  int am_rs;
  // block-sparse mask (dense layouts): uint8 [Hm][nqb][nkb] over 128x128
  // blocks, nonzero = the block's pairs are visible
  const uint8_t* bmask;
  int bm_hstride, bm_nqb, bm_nkb;
  int out_f32;            // O is f32 (else the input type)
};

// Build option: the dQ kernel computes D_i = <dO_i, O_i> for its own rows
// (it holds dO already) and writes it for the dK/dV kernel, which runs
// after it, instead of a separate pass over dO and O.
#ifndef SDPA_BWD_FUSED_ROWDOT
#define SDPA_BWD_FUSED_ROWDOT 1
#endif

// Block-sparse scan: the first tile index >= t whose 128x128 mask block is
// kept, tiles of 128/tpb rows or keys, mask entries base[b * stride] for
// blocks b < n.  A wave reads 64 entries per ballot into a wave-uniform bit
// set, so a scan waits on memory once per 64 blocks.  Every wave of a
// workgroup computes the same sequence.
struct BlockScan {
  const uint8_t* base;
  int stride, n, chunk;
  uint64_t bits;
};

__device__ __forceinline__ int block_scan_next(BlockScan& sc, int t, int tpb, int ntiles,
                                               int lane) {
  while (t < ntiles) {
    const int blk = t / tpb;
    const int chunk = blk >> 6;
    if (chunk != sc.chunk) {
      const int c = chunk * 64 + lane;
      sc.bits = __builtin_amdgcn_ballot_w64(c < sc.n && sc.base[(int64_t)c * sc.stride] != 0);
      sc.chunk = chunk;
    }
    const uint64_t rest = sc.bits >> (blk & 63);
    if (rest != 0) return max(t, (blk + (int)__builtin_ctzll(rest)) * tpb);
    t = (chunk + 1) * 64 * tpb;
  }
  return t;
}

// Buffer view of one unit's mask (rows 0..nq-1, keys rounded up to 16), and
// the bias in log2 units of element `e` (0..3) of the 4-element group held
// in w: bool -> 0 or -inf, additive -> a*log2(e).
template <int MK>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mask_unit_rsrc(const BwdParams& p, int b, int h,
                                                                 int nq, int nk) {
  constexpr int EB = MK == kMaskBool ? 1 : MK == kMaskAdd ? 2 : 4;
  const char* base = reinterpret_cast<const char*>(p.amask) +
                     ((int64_t)b * p.am_bs + (int64_t)h * p.am_hs) * EB;
  const int bytes = (int)(((int64_t)(nq - 1) * p.am_rs + ((nk + 15) & ~15)) * EB);
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, bytes, kBufferWord3);
}

// The 4-key groups g (keys 8g + 4hl .. +3 of a 32-key block) of one mask
// row, as the forward reads them: bool and 16-bit masks as two contiguous
// half blocks per lane pair (keys 16hl .. 16hl+15 at byte offset `off`),
// exchanged through v_permlane32_swap; f32 masks one 16-byte load per group
// (`off` at key 4hl).  w[g] holds group g's elements (1, 2 or 4 words).
template <int MK>
__device__ __forceinline__ void load_mask_groups(__amdgpu_buffer_rsrc_t r, int off,
                                                 uint32_t (&w)[4][MK == kMaskBool ? 1 : MK == kMaskAdd ? 2 : 4]) {
  if constexpr (MK == kMaskBool) {
    const u32x4 d = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    const auto s01 = __builtin_amdgcn_permlane32_swap(d[0], d[1], false, false);
    const auto s23 = __builtin_amdgcn_permlane32_swap(d[2], d[3], false, false);
    w[0][0] = s01[0];
    w[2][0] = s01[1];
    w[1][0] = s23[0];
    w[3][0] = s23[1];
  } else if constexpr (MK == kMaskAdd) {
    const u32x4 a = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    const u32x4 b = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
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
      const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 32 * g, 0, 0));
#pragma unroll
      for (int e = 0; e < 4; ++e) w[g][e] = v[e];
    }
  }
}

template <int MK, bool BF16>
__device__ __forceinline__ float mask_bias2(uint32_t word, int half) {
  if (MK == kMaskBool) return ((word >> (8 * half)) & 0xffu) != 0u ? 0.f : -INFINITY;
  if (MK == kMaskAdd) {
    const uint32_t hb = (word >> (16 * half)) & 0xffffu;
    const float a = BF16 ? __uint_as_float(hb << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)hb);
    return a * 1.4426950408889634f;
  }
  return __uint_as_float(word) * 1.4426950408889634f;
}

// 65536/T (the inverse keep probability) if the 16-bit number u is below
// the keep threshold T, else 0: the sign of u - T (T <= 65536) selects the
// bits of the scale.
__device__ __forceinline__ float keep_scale(uint32_t u, uint32_t t, float rp) {
  const uint32_t m = (uint32_t)((int32_t)(u - t) >> 31);
  return __uint_as_float(__float_as_uint(rp) & m);
}

// unpack 8 16-bit values (f16 or bf16) to fp32
template <bool BF16>
__device__ __forceinline__ void unpack8(u32x4 w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (BF16) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    } else {
      const uint32_t e = w[i];
      x[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(e & 0xffffu));
      x[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(e >> 16));
    }
  }
}

// ---- D_i = <dO_i, O_i>, one thread per row (builds without the fused row
// dot of the dQ kernel)
template <bool BF16, int D, bool OF32>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(BwdParams p, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D; c += 8) {
    float g[8], o[8];
    unpack8<BF16>(*reinterpret_cast<const u32x4*>(p.dout + r * D + c), g);
    if (OF32) {
      const float* op = reinterpret_cast<const float*>(p.out) + r * D + c;
      const f32x4 a = *reinterpret_cast<const f32x4*>(op);
      const f32x4 b = *reinterpret_cast<const f32x4*>(op + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[i] = a[i];
        o[4 + i] = b[i];
      }
    } else {
      unpack8<BF16>(*reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.out) + r * D + c), o);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(g[i], o[i], acc);
  }
  p.dsum[r] = acc;
}

// ---- shared pieces of the two tile kernels

// XCD-contiguous tile order (blocks are dispatched round-robin over the 8
// XCDs): each XCD gets a contiguous range, so a head's tiles share an L2.
__device__ __forceinline__ int bwd_tile_of_block(int total) {
  int t = blockIdx.x;
  if ((total & 7) == 0) t = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  return t;
}

// Build option: causal grids in longest-processing-time order.
#ifndef SDPA_BWD_CAUSAL_LPT
#define SDPA_BWD_CAUSAL_LPT 1
#endif

// The rows of one (batch, head) unit -- or (sequence, head) of a packed
// batch, whose rows are cu[s]..cu[s+1]-1 of [T, H, d] tensors (row stride
// H*d): row counts, row stride in elements, element offsets of the first
// q and k/v rows, and the index of the first row in the lse / workspace
// layout ([B,H,N] dense, [T,H] packed) with its stride per row.
struct BwdUnit {
  int nq, nk, rs, ls;
  int64_t qoff, kvoff, l0;
};

template <bool VARLEN>
__device__ __forceinline__ BwdUnit bwd_unit(const BwdParams& p, int bh, int D) {
  BwdUnit u;
  if (VARLEN) {
    const int s = bh / p.H, h = bh % p.H;
    const int s0 = p.cu[s];
    u.nq = u.nk = p.cu[s + 1] - s0;
    u.rs = p.H * D;
    u.l0 = (int64_t)s0 * p.H + h;
    u.qoff = u.kvoff = u.l0 * D;
    u.ls = p.H;
  } else {
    u.nq = p.Nq;
    u.nk = p.Nk;
    u.rs = D;
    u.qoff = (int64_t)bh * p.Nq * D;
    u.kvoff = (int64_t)bh * p.Nk * D;
    u.l0 = (int64_t)bh * p.Nq;
    u.ls = 1;
  }
  return u;
}

// Causal grids: rank r of head bh, where rank 0 is every head's heaviest
// tile, rank 1 the next heaviest, ... (longest-processing-time order, which
// shortens the grid's tail); each XCD keeps its own eighth of the heads
// when the head count allows.
__device__ __forceinline__ void bwd_causal_rank_of_block(int total, int n_tiles, int& bh,
                                                         int& rank) {
  const int nbh = total / n_tiles;
  if ((nbh & 7) == 0) {
    const int hp = nbh >> 3, j = blockIdx.x >> 3;
    bh = (blockIdx.x & 7) * hp + j % hp;
    rank = j / hp;
  } else {
    bh = blockIdx.x % nbh;
    rank = blockIdx.x / nbh;
  }
}

// Buffer view of `rows` rows of a head starting at row r0; rows past `nrows`
// read as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* head, int r0, int nrows,
                                                            int rs_bytes, int D) {
  const int off = r0 * rs_bytes;
  const int valid = max(((nrows - 1) * rs_bytes + D * 2) - off, 0);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(reinterpret_cast<const char*>(head) + off),
                                           (short)0, valid, kBufferWord3);
}

// 16-byte chunk of row `row` (relative to the view), columns c..c+7
__device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, int row, int col, int rs_bytes) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, row * rs_bytes + col * 2, 0, 0));
}

// Two rows (2pr, 2pr+1) x 8 columns -> 8 words of the transposed copy: word
// e holds (row 2pr, row 2pr+1) of column e, in the input type.
__device__ __forceinline__ void store_pair_t(uint32_t* dst, int tw, u32x4 a, u32x4 b) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t x = a[w], y = b[w];
    dst[(2 * w) * tw] = __builtin_amdgcn_perm(y, x, 0x05040100u);
    dst[(2 * w + 1) * tw] = __builtin_amdgcn_perm(y, x, 0x07060302u);
  }
}

// Debug (LDS poisoning, SDPA_LDS_POISON): all-ones words are NaN in f16,
// bf16 and f32.  The whole LDS is filled when a kernel starts, and after
// the barrier that ends the reads of a staging buffer each thread refills
// the slots it stores that buffer's next tile into (same thread, so the
// refill and the later store are ordered), so that a read of a buffer
// before its tile has been written turns the gradients into NaN.
template <class Smem>
__device__ __forceinline__ void poison_whole_lds(Smem& sm, int tid, int nt) {
  uint32_t* w = reinterpret_cast<uint32_t*>(&sm);
  for (int i = tid; i < (int)(sizeof(Smem) / 4); i += nt) w[i] = 0xffffffffu;
}
template <class Regs>
__device__ __forceinline__ Regs poison_regs() {
  Regs r;
  __builtin_memset(&r, 0xff, sizeof(r));
  return r;
}

// Two fp32 values packed as operands of the dV / dK / dQ products (the
// input type, round to nearest even), and those products.
template <bool BF16>
__device__ __forceinline__ uint32_t pack_grad_operand(float a, float b) {
  return BF16 ? pack_bf16(a, b) : pack_f16(a, b);
}
template <bool BF16>
__device__ __forceinline__ f32x16 mfma_in(u32x4 a, u32x4 b, f32x16 c) {
  return BF16 ? mfma_bf16(a, b, c) : mfma_f16(a, b, c);
}

// Store a d-major accumulator (lane = row of the output, registers = d) of
// one 32-row block: rows row0 + l%32 < nrows, scaled by `mul`.
template <bool BF16, bool GF32, int DB>
__device__ __forceinline__ void store_rows(void* base, int64_t off0, int64_t rs, int row, int nrows,
                                           int hl, const f32x16 (&acc)[DB], float mul) {
  if (row >= nrows) return;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dcol = db * 32 + 8 * g + 4 * hl;
      const float x0 = acc[db][4 * g] * mul, x1 = acc[db][4 * g + 1] * mul;
      const float x2 = acc[db][4 * g + 2] * mul, x3 = acc[db][4 * g + 3] * mul;
      const int64_t off = off0 + (int64_t)row * rs + dcol;
      if (GF32) {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(base) + off) = f32x4{x0, x1, x2, x3};
      } else {
        const u32x2 w = BF16 ? u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)}
                             : u32x2{pack_f16(x0, x1), pack_f16(x2, x3)};
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + off) = w;
      }
    }
}

// The same rows in 16-bit types, through the wave's own LDS area `ow`
// (32 rows of D + 8 elements; free once the kernel's last barrier has
// passed): each lane stages its row's values, then stores 16-byte segments
// along the rows, so that one store covers 1 KB of rows instead of 16 bytes
// of each of 32 rows.  row0 is the wave's first row.
template <bool BF16, int D>
__device__ __forceinline__ void store_rows_lds(void* base, int64_t off0, int64_t rs, int row0,
                                               int nrows, int l32, int hl,
                                               const f32x16 (&acc)[D / 32], float mul,
                                               uint16_t* ow) {
  constexpr int OROW = D + 8;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dcol = db * 32 + 8 * g + 4 * hl;
      const float x0 = acc[db][4 * g] * mul, x1 = acc[db][4 * g + 1] * mul;
      const float x2 = acc[db][4 * g + 2] * mul, x3 = acc[db][4 * g + 3] * mul;
      *reinterpret_cast<u32x2*>(&ow[l32 * OROW + dcol]) =
          BF16 ? u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)} : u32x2{pack_f16(x0, x1), pack_f16(x2, x3)};
    }
  const int lane = hl * 32 + l32;
#pragma unroll
  for (int i = 0; i < D / 16; ++i) {
    const int c = i * 64 + lane;   // 16-byte chunk of the wave's 32 rows
    const int row = c / (D / 8), col = (c % (D / 8)) * 8;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&ow[row * OROW + col]);
    if (row0 + row < nrows)
      *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(base) + off0 +
                                (int64_t)(row0 + row) * rs + col) = v;
  }
}

// ---- dQ: one wave per 32 query rows, key tiles of BN rows streamed
template <bool BF16, int D, int NW, int BN, bool CAUSAL, bool GF32, bool DROP = false,
          bool VARLEN = false, int MK = kPlain, int KS = 1>
struct BwdDq {
  // KS key groups: the workgroup's waves form KS groups of NWG waves over
  // the same query rows; group g takes key tiles g, g + KS, ... and the
  // groups' dQ partial sums are added at the end
  static constexpr int NWG = NW / KS;
  static constexpr int BM = NWG * 32;
  static constexpr int KB = BN / 32;
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int NT = NW * 64;
  static constexpr int NTG = NWG * 64;          // threads of a key group (staging)
  static constexpr int NC = D / 8;
  static constexpr int KROW = D + 8;            // row-major LDS row, elements
  static constexpr int TW = BN / 2 + 4;         // transposed LDS row, words
  static constexpr int PAIRS = (BN / 2) * NC;   // K: (2 rows x 16 bytes) tasks
  static constexpr int VCH = BN * NC;           // V: 16-byte tasks
  static constexpr int PPT = (PAIRS + NTG - 1) / NTG;
  static constexpr int VPT = (VCH + NTG - 1) / NTG;
  static_assert(BN % 32 == 0 && D % 32 == 0, "shape");
  static_assert(KS == 1 || (KS == 2 && NW % 2 == 0 && MK != kBlockSparse), "key groups");

  struct __attribute__((aligned(16))) Buf {
    uint16_t k[BN * KROW];
    uint16_t v[BN * KROW];
    uint32_t kt[D * TW];   // K^T (input type), keys in vt_key_pos order
  };
  struct __attribute__((aligned(16))) Smem {
    Buf b[2 * KS];
  };
  // key groups: group 1's dQ sums (per lane) for the merge
  static constexpr int MERGE_BYTES = KS > 1 ? NWG * DB * 16 * 64 * 4 : 0;
  static_assert(MERGE_BYTES <= (int)sizeof(Smem), "merged sums fit in LDS");
  struct Regs {
    u32x4 k0[PPT], k1[PPT], v[VPT];
  };
  struct Stage {
    int kg[PPT], kl[PPT], kt[PPT], vg[VPT], vl[VPT];
  };

  static __device__ void run(const BwdParams& p, Smem& sm) {
    const int tid = threadIdx.x, wave = tid / 64, lane = tid & 63;
    const int l32 = tid & 31, hl = (tid >> 5) & 1;
    const int grp = KS > 1 ? wave / NWG : 0;      // key group
    const int gtid = KS > 1 ? tid % NTG : tid;    // thread index within the group
    const int bb = KS > 1 ? 2 * grp : 0;          // the group's first LDS buffer
    int qt, bh;
    if (CAUSAL && SDPA_BWD_CAUSAL_LPT) {   // the last query tiles see the most keys
      int rank;
      bwd_causal_rank_of_block(p.total, p.n_tiles, bh, rank);
      qt = p.n_tiles - 1 - rank;
    } else {
      const int tile = bwd_tile_of_block(p.total);
      qt = tile % p.n_tiles;
      bh = tile / p.n_tiles;
    }
    const BwdUnit un = bwd_unit<VARLEN>(p, bh, D);
    const int nq = un.nq, nk = un.nk;
    const int rs_bytes = un.rs * 2;
    const int64_t qoff = un.qoff, kvoff = un.kvoff;
    const int q0 = qt * BM, q0w = q0 + (KS > 1 ? wave % NWG : wave) * 32;
    if (VARLEN && q0 >= nq) return;   // whole workgroup: past the sequence end
    const int kend = CAUSAL ? min(nk, q0 + BM) : nk;
    const int ntiles = (kend + BN - 1) / BN;

    // this wave's Q and dO rows as B operands; lse and D of its row
    const __amdgpu_buffer_rsrc_t qr = rows_rsrc(p.q + qoff, 0, nq, rs_bytes, D);
    const __amdgpu_buffer_rsrc_t gr = rows_rsrc(p.dout + qoff, 0, nq, rs_bytes, D);
    u32x4 qf[DS], gf[DS];
    const int qi = q0w + l32;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      qf[ds] = ld16(qr, qi, ds * 16 + hl * 8, rs_bytes);
      gf[ds] = ld16(gr, qi, ds * 16 + hl * 8, rs_bytes);
    }
    const bool qok = qi < nq;
    const int64_t li = un.l0 + (int64_t)qi * un.ls;
    float lse2 = qok ? p.lse[li] * 1.4426950408889634f : 0.f;
    // masks, block-sparse: a row that saw no key (lse = -inf) has P = 0
    if (MK != kPlain && lse2 == -INFINITY) lse2 = INFINITY;
    float dd;
    if (SDPA_BWD_FUSED_ROWDOT) {
      // D of the lane's row: the lane holds 8 columns of dO per k-step (the
      // other half of the row is in lane l^32); rows past the end read as
      // zeros, so their D is 0
      float part = 0.f;
      if (p.out_f32) {
        const int rs4 = rs_bytes * 2;
        const __amdgpu_buffer_rsrc_t orr = rows_rsrc(
            reinterpret_cast<const uint16_t*>(reinterpret_cast<const float*>(p.out) + qoff), 0,
            nq, rs4, 2 * D);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          float g[8];
          unpack8<BF16>(gf[ds], g);
          const int c = 2 * (ds * 16 + hl * 8);   // 16-bit units
          const u32x4 oa = ld16(orr, qi, c, rs4), ob = ld16(orr, qi, c + 8, rs4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            part = __builtin_fmaf(g[i], __uint_as_float(oa[i]), part);
            part = __builtin_fmaf(g[4 + i], __uint_as_float(ob[i]), part);
          }
        }
      } else {
        const __amdgpu_buffer_rsrc_t orr =
            rows_rsrc(reinterpret_cast<const uint16_t*>(p.out) + qoff, 0, nq, rs_bytes, D);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          float g[8], o[8];
          unpack8<BF16>(gf[ds], g);
          unpack8<BF16>(ld16(orr, qi, ds * 16 + hl * 8, rs_bytes), o);
#pragma unroll
          for (int i = 0; i < 8; ++i) part = __builtin_fmaf(g[i], o[i], part);
        }
      }
      dd = pair_sum(part);
      // (key groups: both groups hold D of the same rows; group 0 writes it)
      if (hl == 0 && qok && grp == 0) p.dsum[li] = dd;
    } else {
      dd = qok ? p.dsum[li] : 0.f;
    }
    // masks: the lane's row of the unit's mask, read per 32-key block as
    // the forward reads it (load_mask_groups)
    constexpr int MW = MK == kMaskBool ? 1 : MK == kMaskAdd ? 2 : 4;
    __amdgpu_buffer_rsrc_t mrs;
    int moff = 0;
    if (MK >= kMaskBool) {
      mrs = mask_unit_rsrc<MK>(p, bh / p.H, bh % p.H, nq, nk);
      moff = (qi * p.am_rs + (MW == 4 ? 4 : 16) * hl) * MW;
    }

    Stage st;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int t = gtid + i * NTG;
      const int pr = t % (BN / 2), c = t / (BN / 2);
      st.kg[i] = 2 * pr;
      st.kl[i] = 2 * pr * KROW + c * 8;
      st.kt[i] = c * 8 * TW + vt_key_pos(2 * pr) / 2;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int t = gtid + i * NTG;
      st.vg[i] = t / NC;
      st.vl[i] = (t / NC) * KROW + (t % NC) * 8;
    }
    auto col_of_pair = [&](int i) { return ((gtid + i * NTG) / (BN / 2)) * 8; };
    auto col_of_v = [&](int i) { return ((gtid + i * NTG) % NC) * 8; };

    auto load = [&](Regs& r, int j) {
      const __amdgpu_buffer_rsrc_t kr = rows_rsrc(p.k + kvoff, j * BN, nk, rs_bytes, D);
      const __amdgpu_buffer_rsrc_t vr = rows_rsrc(p.v + kvoff, j * BN, nk, rs_bytes, D);
#pragma unroll
      for (int i = 0; i < PPT; ++i)
        if (PAIRS % NTG == 0 || gtid + i * NTG < PAIRS) {
          r.k0[i] = ld16(kr, st.kg[i], col_of_pair(i), rs_bytes);
          r.k1[i] = ld16(kr, st.kg[i] + 1, col_of_pair(i), rs_bytes);
        }
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        if (VCH % NTG == 0 || gtid + i * NTG < VCH) r.v[i] = ld16(vr, st.vg[i], col_of_v(i), rs_bytes);
    };
    auto store = [&](int buf, const Regs& r) {
      Buf& b = sm.b[bb + buf];
#pragma unroll
      for (int i = 0; i < PPT; ++i)
        if (PAIRS % NTG == 0 || gtid + i * NTG < PAIRS) {
          *reinterpret_cast<u32x4*>(&b.k[st.kl[i]]) = r.k0[i];
          *reinterpret_cast<u32x4*>(&b.k[st.kl[i] + KROW]) = r.k1[i];
          store_pair_t(&b.kt[st.kt[i]], TW, r.k0[i], r.k1[i]);
        }
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        if (VCH % NTG == 0 || gtid + i * NTG < VCH) *reinterpret_cast<u32x4*>(&b.v[st.vl[i]]) = r.v[i];
    };

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

    // block-sparse: only the key tiles the workgroup's mask row keeps (the
    // workgroup's BM = 128 rows are one mask row)
    constexpr bool BSP = MK == kBlockSparse;
    static_assert(!BSP || (BM == kSparseBlock && kSparseBlock % BN == 0 && !VARLEN && !DROP),
                  "block-sparse dQ shape");
    BlockScan bsc;
    if (BSP) {
      bsc.base = p.bmask + (int64_t)(bh % p.H) * p.bm_hstride + (int64_t)qt * p.bm_nkb;
      bsc.stride = 1;
      bsc.n = p.bm_nkb;
      bsc.chunk = -1;
      bsc.bits = 0;
    }
    auto next_tile = [&](int t) {
      return BSP ? block_scan_next(bsc, t, kSparseBlock / BN, ntiles, lane) : t;
    };
    if (SDPA_LDS_POISON) {
      poison_whole_lds(sm, tid, NT);
      __syncthreads();
    }
    int j = KS > 1 ? grp : next_tile(0);
    if (j < ntiles) {
      Regs r0;
      load(r0, j);
      store(0, r0);
    }
    __syncthreads();

    const int kl = l32 * KROW + hl * 8;
    // key groups: every group makes the same number of steps (one barrier
    // each); a group past its last tile only waits at them
    const int nsteps = KS > 1 ? (ntiles + KS - 1) / KS : 0;
    for (int step = 0; KS > 1 ? step < nsteps : j < ntiles; ++step) {
      const int buf = step & 1;
      Regs rn;
      const int jn = KS > 1 ? j + KS : next_tile(j + 1);
      const bool nxt = jn < ntiles;
      if (nxt) load(rn, jn);
      const int kb = j * BN;
      const bool live = (KS == 1 || j < ntiles) && !(CAUSAL && kb > q0w + 31);
      if (live) {
        const Buf& b = sm.b[bb + buf];
        const bool masked = (kb + BN > nk) || (CAUSAL && kb + BN - 1 > q0w);
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
          f32x16 s = {}, dp = {};
          if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int ds = 0; ds < DS; ++ds) {
            const u32x4 ka = *reinterpret_cast<const u32x4*>(&b.k[kl + kk * 32 * KROW + ds * 16]);
            const u32x4 va = *reinterpret_cast<const u32x4*>(&b.v[kl + kk * 32 * KROW + ds * 16]);
            s = BF16 ? mfma_bf16(ka, qf[ds], s) : mfma_f16(ka, qf[ds], s);
            dp = BF16 ? mfma_bf16(va, gf[ds], dp) : mfma_f16(va, gf[ds], dp);
          }
          if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(0);
          // masks: s becomes log2 units relative to the row's lse, in place,
          // plus the mask's bias (the plain kernel forms that in the exp)
          if (MK >= kMaskBool) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = __builtin_fmaf(s[r], p.c, -lse2);
            uint32_t gw[4][MW];
            load_mask_groups<MK>(mrs, moff + (kb + kk * 32) * MW, gw);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const uint32_t* mw = gw[g];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const uint32_t word = MW == 1 ? mw[0] : MW == 2 ? mw[e / 2] : mw[e];
                const int half = MW == 1 ? e : MW == 2 ? (e & 1) : 0;
                s[4 * g + e] += mask_bias2<MK, BF16>(word, half);
              }
            }
          }
          if (masked) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kb + kk * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
              if (key >= nk || (CAUSAL && key > qi)) s[r] = -INFINITY;
            }
          }
          u32x4 dsf[2];
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            // dropout: the forward's keep decisions of these 8 keys of row
            // qi (same lane layout as the forward), dP scaled by z/kappa (kappa = T/65536, the keep probability)
            uint32_t rr[4];
            if (DROP)
              philox4x32_10((uint32_t)((kb + kk * 32) >> 3) + 2 * hs + hl, (uint32_t)qi,
                            (uint32_t)bh, p.drop_offset, p.seed_lo, p.seed_hi, rr);
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 8 * hs + 2 * i;
              const float p0 = __builtin_amdgcn_exp2f(
                  MK >= kMaskBool ? s[r] : __builtin_fmaf(s[r], p.c, -lse2));
              const float p1 = __builtin_amdgcn_exp2f(
                  MK >= kMaskBool ? s[r + 1] : __builtin_fmaf(s[r + 1], p.c, -lse2));
              float d0 = dp[r] - dd, d1 = dp[r + 1] - dd;
              if (DROP) {
                d0 = __builtin_fmaf(keep_scale(rr[i] & 0xffffu, p.drop_t, p.drop_scale), dp[r], -dd);
                d1 = __builtin_fmaf(keep_scale(rr[i] >> 16, p.drop_t, p.drop_scale), dp[r + 1], -dd);
              }
              w[i] = pack_grad_operand<BF16>(p0 * d0, p1 * d1);
            }
            dsf[hs] = u32x4{w[0], w[1], w[2], w[3]};
          }
          if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int hs = 0; hs < 2; ++hs)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const u32x4 kta = *reinterpret_cast<const u32x4*>(
                  &b.kt[l32 * TW + hl * 4 + 8 * hs + db * 32 * TW + 16 * kk]);
              acc[db] = mfma_in<BF16>(kta, dsf[hs], acc[db]);
            }
          if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(0);
        }
      }
      if (nxt) store(buf ^ 1, rn);
      __syncthreads();
      // every read of buffer buf ended at this barrier; the next step
      // stores the tile after next there
      if (SDPA_LDS_POISON) store(buf, poison_regs<Regs>());
      j = jn;
    }
    // (debug poisoning: the last refills end before any wave stages its
    // gradient rows in LDS)
    if (SDPA_LDS_POISON) __syncthreads();
    if constexpr (KS > 1) {
      // key groups: group 1 hands its dQ sums to group 0 through LDS (every
      // read of the K/V buffers ended at the last step's barrier); the
      // second barrier ends the reads before group 0 stages its rows there
      float* mg = reinterpret_cast<float*>(&sm) + (wave % NWG) * DB * 16 * 64 + lane;
      if (grp == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) mg[(db * 16 + r) * 64] = acc[db][r];
      }
      __syncthreads();
      if (grp == 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] += mg[(db * 16 + r) * 64];
      }
      __syncthreads();
      if (grp != 0) return;
    }
    static_assert(NWG * 32 * (D + 8) * 2 <= (int)sizeof(Smem), "dQ rows fit in LDS");
    // (the masked kernels keep direct stores: through LDS they measured
    // 5% slower on a key-padding mask)
    if (GF32 || MK != kPlain)
      store_rows<BF16, GF32, DB>(p.dq, qoff, un.rs, qi, nq, hl, acc, p.scale);
    else
      store_rows_lds<BF16, D>(p.dq, qoff, un.rs, q0w, nq, l32, hl, acc, p.scale,
                              reinterpret_cast<uint16_t*>(&sm) + wave * 32 * (D + 8));
  }
};

// ---- dK, dV: one wave per 32 key rows, query tiles of BQ rows streamed
// Dropout keep bits in the transposed layout of the dK/dV kernel.  Lane
// (l32, hl) owns key key0 + l32 and needs the decisions of the 32 queries
// q0 .. q0+31 of a block.  Each lane first draws, as the forward does, the
// two Philox calls of query q0 + l32 for keys key0 .. key0+31; then each of
// the 16 (call, word, half) positions is turned into a 64-lane ballot whose
// bit L is the decision of query q0 + L%32 for one key (lanes L < 32) or
// for the key 4 above it (L >= 32).  The 32 ballot halves are spread over
// lanes 0..31 and every lane fetches the one of its key.  Returns bit q =
// keep (query q0 + q, key key0 + l32).
// v with lane `lane` replaced by the wave-uniform value s.  s is typically
// a ballot just written by a vector compare, and a vector instruction that
// reads an SGPR written by a vector instruction needs two wait states on
// gfx950; the compiler cannot see inside the asm, so the nop is written here.
template <int lane>
__device__ __forceinline__ uint32_t write_lane(uint32_t v, uint32_t s) {
  asm("s_nop 1\n\tv_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(s), "i"(lane));
  return v;
}

__device__ __forceinline__ uint32_t keep_bits_of_key(int q0, int key0, int l32, int hl,
                                                     uint32_t unit, const BwdParams& p) {
  uint32_t r[2][4];
#pragma unroll
  for (int hs = 0; hs < 2; ++hs)
    philox4x32_10((uint32_t)(key0 >> 3) + 2 * hs + hl, (uint32_t)(q0 + l32), unit, p.drop_offset,
                  p.seed_lo, p.seed_hi, r[hs]);
  uint32_t v = 0;
  auto put = [&](auto idx_c, uint32_t u) {
    constexpr int idx = decltype(idx_c)::value;
    const uint64_t bal = __builtin_amdgcn_ballot_w64(u < p.drop_t);
    v = write_lane<2 * idx>(v, (uint32_t)bal);
    v = write_lane<2 * idx + 1>(v, (uint32_t)(bal >> 32));
  };
  // ballot index hs * 8 + w * 2 + b for half b of word w of call hs
#define SDPA_PUT(HS, W)                                                         \
  put(std::integral_constant<int, HS * 8 + W * 2>{}, r[HS][W] & 0xffffu);       \
  put(std::integral_constant<int, HS * 8 + W * 2 + 1>{}, r[HS][W] >> 16);
  SDPA_PUT(0, 0) SDPA_PUT(0, 1) SDPA_PUT(0, 2) SDPA_PUT(0, 3)
  SDPA_PUT(1, 0) SDPA_PUT(1, 1) SDPA_PUT(1, 2) SDPA_PUT(1, 3)
#undef SDPA_PUT
  // key offset l32 = 16 hs + 8 (w >> 1) + 4 h + 2 (w & 1) + b
  const int w = 2 * ((l32 >> 3) & 1) + ((l32 >> 1) & 1);
  const int idx = ((l32 >> 4) & 1) * 8 + w * 2 + (l32 & 1);
  const int src = 2 * idx + ((l32 >> 2) & 1);
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src * 4, (int)v);
}

template <bool BF16, int D, int NW, int BQ, bool CAUSAL, bool GF32, bool DROP = false,
          bool VARLEN = false, int MK = kPlain, int KS = 1>
struct BwdDkdv {
  // KS query groups: the workgroup's waves form KS groups of NWG waves over
  // the same keys; group g takes query tiles i0 + g, i0 + g + KS, ... and
  // the groups' dK and dV partial sums are added at the end
  static constexpr int NWG = NW / KS;
  static constexpr int BK = NWG * 32;
  static constexpr int KB = BQ / 32;
  static constexpr int DS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int NT = NW * 64;
  static constexpr int NTG = NWG * 64;   // threads of a query group (staging)
  static constexpr int NC = D / 8;
  static constexpr int KROW = D + 8;
  static constexpr int TW = BQ / 2 + 4;
  static constexpr int PAIRS = (BQ / 2) * NC;   // Q and dO: (2 rows x 16 bytes) tasks
  static constexpr int PPT = (PAIRS + NTG - 1) / NTG;
  static_assert(BQ % 32 == 0 && D % 32 == 0 && BQ <= NTG, "shape");
  static_assert(KS == 1 || (KS == 2 && NW % 2 == 0 && MK != kBlockSparse), "query groups");
  // masks: the step's [BQ queries x BK keys] mask tile is staged through LDS
  // with the Q and dO rows (16-byte chunks, rows padded by 16 bytes)
  static constexpr bool HASM = MK >= kMaskBool;
  static constexpr int MEB = MK == kMaskBool ? 1 : MK == kMaskAdd ? 2 : 4;
  static constexpr int MROWB = BK * MEB + 16;            // LDS row, bytes
  static constexpr int MCPR = BK * MEB / 16;             // 16-byte chunks per row
  static constexpr int MPT = HASM ? (BQ * MCPR + NTG - 1) / NTG : 1;

  struct __attribute__((aligned(16))) Buf {
    uint16_t q[BQ * KROW];
    uint16_t g[BQ * KROW];     // dO rows
    uint32_t qt[D * TW];       // Q^T (input type), queries in vt_key_pos order
    uint32_t gt[D * TW];       // dO^T, likewise
    float nl[BQ];              // -lse * log2(e) / c; -inf past the last row
    float nd[BQ];              // -<dO_i, O_i>; 0 past the last row
    uint32_t mk[HASM ? BQ * MROWB / 4 : 4];   // mask tile (masked kernels)
  };
  struct __attribute__((aligned(16))) Smem {
    Buf b[2 * KS];
  };
  // query groups: group 1's dK and dV (per lane) for the merge
  static constexpr int MERGE_BYTES = KS > 1 ? NWG * 2 * DB * 16 * 64 * 4 : 0;
  static_assert(MERGE_BYTES <= (int)sizeof(Smem), "merged sums fit in LDS");
  struct Regs {
    u32x4 q0[PPT], q1[PPT], g0[PPT], g1[PPT];
    u32x4 m[MPT];
    float l2, dd;
  };

  static __device__ void run(const BwdParams& p, Smem& sm) {
    const int tid = threadIdx.x, wave = tid / 64, lane = tid & 63;
    const int l32 = tid & 31, hl = (tid >> 5) & 1;
    const int grp = KS > 1 ? wave / NWG : 0;      // query group
    const int gtid = KS > 1 ? tid % NTG : tid;    // thread index within the group
    const int bb = KS > 1 ? 2 * grp : 0;          // the group's first LDS buffer
    int kt, bh;
    if (CAUSAL && SDPA_BWD_CAUSAL_LPT) {   // the first key tiles are seen by the most queries
      bwd_causal_rank_of_block(p.total, p.n_tiles, bh, kt);
    } else {
      const int tile = bwd_tile_of_block(p.total);
      kt = tile % p.n_tiles;
      bh = tile / p.n_tiles;
    }
    const BwdUnit un = bwd_unit<VARLEN>(p, bh, D);
    const int nq = un.nq, nk = un.nk;
    const int rs_bytes = un.rs * 2;
    const int64_t qoff = un.qoff, kvoff = un.kvoff;
    const int k0 = kt * BK, k0w = k0 + (KS > 1 ? wave % NWG : wave) * 32;
    if (VARLEN && k0 >= nk) return;   // whole workgroup: past the sequence end
    const int ki = k0w + l32;
    const int nqt = (nq + BQ - 1) / BQ;
    // causal: query tiles before the one holding query k0 see none of the
    // workgroup's keys
    const int i0 = CAUSAL ? min(k0 / BQ, nqt) : 0;

    // masks: the unit's mask, read a [BQ x BK] tile per step
    __amdgpu_buffer_rsrc_t mrs;
    if (MK >= kMaskBool) mrs = mask_unit_rsrc<MK>(p, bh / p.H, bh % p.H, nq, nk);

    // this wave's K and V rows as B operands
    const __amdgpu_buffer_rsrc_t kr = rows_rsrc(p.k + kvoff, 0, nk, rs_bytes, D);
    const __amdgpu_buffer_rsrc_t vr = rows_rsrc(p.v + kvoff, 0, nk, rs_bytes, D);
    u32x4 kf[DS], vf[DS];
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      kf[ds] = ld16(kr, ki, ds * 16 + hl * 8, rs_bytes);
      vf[ds] = ld16(vr, ki, ds * 16 + hl * 8, rs_bytes);
    }

    int pg[PPT], pl[PPT], ptl[PPT], pc[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int t = gtid + i * NTG;
      const int pr = t % (BQ / 2), c = t / (BQ / 2);
      pg[i] = 2 * pr;
      pc[i] = c * 8;
      pl[i] = 2 * pr * KROW + c * 8;
      ptl[i] = c * 8 * TW + vt_key_pos(2 * pr) / 2;
    }

    auto load = [&](Regs& r, int i) {
      const int r0 = i * BQ;
      const __amdgpu_buffer_rsrc_t qv = rows_rsrc(p.q + qoff, r0, nq, rs_bytes, D);
      const __amdgpu_buffer_rsrc_t gv = rows_rsrc(p.dout + qoff, r0, nq, rs_bytes, D);
#pragma unroll
      for (int t = 0; t < PPT; ++t)
        if (PAIRS % NTG == 0 || gtid + t * NTG < PAIRS) {
          r.q0[t] = ld16(qv, pg[t], pc[t], rs_bytes);
          r.q1[t] = ld16(qv, pg[t] + 1, pc[t], rs_bytes);
          r.g0[t] = ld16(gv, pg[t], pc[t], rs_bytes);
          r.g1[t] = ld16(gv, pg[t] + 1, pc[t], rs_bytes);
        }
      if (HASM) {
#pragma unroll
        for (int t = 0; t < MPT; ++t) {
          const int c = gtid + t * NTG;
          if ((BQ * MCPR) % NTG == 0 || c < BQ * MCPR) {
            const int row = c / MCPR, cc = c % MCPR;
            const int off = (r0 + row) * p.am_rs * MEB + k0 * MEB + cc * 16;
            r.m[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(mrs, off, 0, 0));
          }
        }
      }
      if (gtid < BQ) {
        const int row = r0 + gtid;
        const bool ok = row < nq;
        const int64_t li = un.l0 + (int64_t)row * un.ls;
        // masks: a row that saw no key (lse = -inf) has P = 0 everywhere
        r.l2 = (ok && (MK == kPlain || p.lse[li] > -INFINITY))
                   ? -p.lse[li] * 1.4426950408889634f / p.c
                   : -INFINITY;
        r.dd = ok ? -p.dsum[li] : 0.f;
      }
    };
    auto store = [&](int buf, const Regs& r) {
      Buf& b = sm.b[bb + buf];
#pragma unroll
      for (int t = 0; t < PPT; ++t)
        if (PAIRS % NTG == 0 || gtid + t * NTG < PAIRS) {
          *reinterpret_cast<u32x4*>(&b.q[pl[t]]) = r.q0[t];
          *reinterpret_cast<u32x4*>(&b.q[pl[t] + KROW]) = r.q1[t];
          *reinterpret_cast<u32x4*>(&b.g[pl[t]]) = r.g0[t];
          *reinterpret_cast<u32x4*>(&b.g[pl[t] + KROW]) = r.g1[t];
          store_pair_t(&b.qt[ptl[t]], TW, r.q0[t], r.q1[t]);
          store_pair_t(&b.gt[ptl[t]], TW, r.g0[t], r.g1[t]);
        }
      if (gtid < BQ) {
        b.nl[gtid] = r.l2;
        b.nd[gtid] = r.dd;
      }
      if (HASM) {
#pragma unroll
        for (int t = 0; t < MPT; ++t) {
          const int c = gtid + t * NTG;
          if ((BQ * MCPR) % NTG == 0 || c < BQ * MCPR) {
            const int row = c / MCPR, cc = c % MCPR;
            *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(b.mk) + row * MROWB + cc * 16) = r.m[t];
          }
        }
      }
    };

    f32x16 dk[DB], dv[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dk[db][r] = dv[db][r] = 0.f;

    // block-sparse: only the query tiles whose mask block keeps the
    // workgroup's keys (its BK = 128 keys are one mask column)
    constexpr bool BSP = MK == kBlockSparse;
    static_assert(!BSP || (BK == kSparseBlock && kSparseBlock % BQ == 0 && !VARLEN && !DROP),
                  "block-sparse dK/dV shape");
    BlockScan bsc;
    if (BSP) {
      bsc.base = p.bmask + (int64_t)(bh % p.H) * p.bm_hstride + kt;
      bsc.stride = p.bm_nkb;
      bsc.n = p.bm_nqb;
      bsc.chunk = -1;
      bsc.bits = 0;
    }
    auto next_tile = [&](int t) {
      return BSP ? block_scan_next(bsc, t, kSparseBlock / BQ, nqt, lane) : t;
    };
    if (SDPA_LDS_POISON) {
      poison_whole_lds(sm, tid, NT);
      __syncthreads();
    }
    int i = KS > 1 ? i0 + grp : next_tile(i0);
    if (i < nqt) {
      Regs r0;
      load(r0, i);
      store(0, r0);
    }
    __syncthreads();

    const int ql = l32 * KROW + hl * 8;
    // query groups: every group makes the same number of steps (one
    // barrier each); a group past its last tile only waits at them
    const int nsteps = KS > 1 ? (nqt - i0 + KS - 1) / KS : 0;
    for (int step = 0; KS > 1 ? step < nsteps : i < nqt; ++step) {
      const int buf = step & 1;
      Regs rn;
      const int in_ = KS > 1 ? i + KS : next_tile(i + 1);
      const bool nxt = in_ < nqt;
      if (nxt) load(rn, in_);
      const int qb = i * BQ;
      const bool live = (KS == 1 || i < nqt) && !(CAUSAL && qb + BQ - 1 < k0w);
      if (live) {
        const Buf& b = sm.b[bb + buf];
        const bool masked = CAUSAL && qb < k0w + 31;
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
          // The accumulators start at -lse*log2(e)/c and -D of the lane's 16
          // query rows (register r holds query 8(r/4) + 4*hl + r%4 of the
          // block), so the matrix cores return S - lse/scale and dP - D.
          // With dropout dP starts at 0 and -D stays in registers, since
          // dS = P (z dP / kappa - D) needs D on its own (kappa = T/65536).
          f32x16 s, dp;
          f32x4 ndv[4];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int idx = kk * 32 + 8 * g + 4 * hl;
            const f32x4 a = *reinterpret_cast<const f32x4*>(&b.nl[idx]);
            const f32x4 c = *reinterpret_cast<const f32x4*>(&b.nd[idx]);
            if (DROP) ndv[g] = c;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              s[4 * g + e] = a[e];
              dp[4 * g + e] = DROP ? 0.f : c[e];
            }
          }
          if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int ds = 0; ds < DS; ++ds) {
            const u32x4 qa = *reinterpret_cast<const u32x4*>(&b.q[ql + kk * 32 * KROW + ds * 16]);
            const u32x4 ga = *reinterpret_cast<const u32x4*>(&b.g[ql + kk * 32 * KROW + ds * 16]);
            s = BF16 ? mfma_bf16(qa, kf[ds], s) : mfma_f16(qa, kf[ds], s);
            dp = BF16 ? mfma_bf16(ga, vf[ds], dp) : mfma_f16(ga, vf[ds], dp);
          }
          if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(0);
          // masks: add the bias in the units of s (the exponent is c s)
          if (MK >= kMaskBool) {
            // the lane's key column of the staged mask tile, its 16 rows
            const char* mcol = reinterpret_cast<const char*>(b.mk) + (k0w - k0 + l32) * MEB;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int row = kk * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
              const char* e = mcol + row * MROWB;
              const uint32_t word = MEB == 1   ? (uint32_t)*reinterpret_cast<const uint8_t*>(e)
                                    : MEB == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(e)
                                               : *reinterpret_cast<const uint32_t*>(e);
              s[r] += mask_bias2<MK, BF16>(word, 0) * p.rc;
            }
          }
          if (masked) {
            // register r holds query qb + 32 kk + 4 hl + 8(r/4) + r%4, which
            // sees key ki iff that offset is at least ki - base
            const int lo = ki - (qb + kk * 32 + 4 * hl);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (8 * (r / 4) + (r % 4) < lo) s[r] = -INFINITY;
          }
          uint32_t zb = 0;
          if (DROP) zb = keep_bits_of_key(qb + kk * 32, k0w, l32, hl, (uint32_t)bh, p) >> (4 * hl);
          u32x4 pf[2], dsf[2];
#pragma unroll
          for (int hs = 0; hs < 2; ++hs) {
            uint32_t wp[4], wd[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 8 * hs + 2 * e;
              const float p0 = __builtin_amdgcn_exp2f(s[r] * p.c);
              const float p1 = __builtin_amdgcn_exp2f(s[r + 1] * p.c);
              if (DROP) {
                // register r holds query 8 (r >> 2) + 4 hl + (r & 3) of the block
                const float z0 = (zb >> (8 * (r >> 2) + (r & 3))) & 1u ? p.drop_scale : 0.f;
                const float z1 = (zb >> (8 * (r >> 2) + (r & 3) + 1)) & 1u ? p.drop_scale : 0.f;
                wp[e] = pack_grad_operand<BF16>(p0 * z0, p1 * z1);
                wd[e] = pack_grad_operand<BF16>(
                    p0 * __builtin_fmaf(z0, dp[r], ndv[r >> 2][r & 3]),
                    p1 * __builtin_fmaf(z1, dp[r + 1], ndv[(r + 1) >> 2][(r + 1) & 3]));
              } else {
                wp[e] = pack_grad_operand<BF16>(p0, p1);
                wd[e] = pack_grad_operand<BF16>(p0 * dp[r], p1 * dp[r + 1]);
              }
            }
            pf[hs] = u32x4{wp[0], wp[1], wp[2], wp[3]};
            dsf[hs] = u32x4{wd[0], wd[1], wd[2], wd[3]};
          }
          if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
          for (int hs = 0; hs < 2; ++hs)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const int wofs = l32 * TW + hl * 4 + 8 * hs + db * 32 * TW + 16 * kk;
              const u32x4 ga = *reinterpret_cast<const u32x4*>(&b.gt[wofs]);
              const u32x4 qa = *reinterpret_cast<const u32x4*>(&b.qt[wofs]);
              dv[db] = mfma_in<BF16>(ga, pf[hs], dv[db]);
              dk[db] = mfma_in<BF16>(qa, dsf[hs], dk[db]);
            }
          if (SDPA_SETPRIO) __builtin_amdgcn_s_setprio(0);
        }
      }
      if (nxt) store(buf ^ 1, rn);
      __syncthreads();
      // every read of buffer buf ended at this barrier
      if (SDPA_LDS_POISON) store(buf, poison_regs<Regs>());
      i = in_;
    }
    if (SDPA_LDS_POISON) __syncthreads();
    if constexpr (KS > 1) {
      // query groups: group 1 hands its dK and dV sums to group 0 through
      // LDS (every read of the Q/dO buffers ended at the last step's
      // barrier); the second barrier ends the reads before group 0 stages
      // its output rows over the same LDS
      float* mg = reinterpret_cast<float*>(&sm) + (wave % NWG) * 2 * DB * 16 * 64 + lane;
      if (grp == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            mg[(db * 16 + r) * 64] = dk[db][r];
            mg[((DB + db) * 16 + r) * 64] = dv[db][r];
          }
      }
      __syncthreads();
      if (grp == 0) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            dk[db][r] += mg[(db * 16 + r) * 64];
            dv[db][r] += mg[((DB + db) * 16 + r) * 64];
          }
      }
      __syncthreads();
      if (grp != 0) return;
    }
    static_assert(NWG * 32 * (D + 8) * 2 <= (int)sizeof(Smem), "dK, dV rows fit in LDS");
    if (GF32 || MK != kPlain) {
      store_rows<BF16, GF32, DB>(p.dk, kvoff, un.rs, ki, nk, hl, dk, p.scale);
      store_rows<BF16, GF32, DB>(p.dv, kvoff, un.rs, ki, nk, hl, dv, 1.f);
    } else {
      uint16_t* ow = reinterpret_cast<uint16_t*>(&sm) + wave * 32 * (D + 8);
      store_rows_lds<BF16, D>(p.dk, kvoff, un.rs, k0w, nk, l32, hl, dk, p.scale, ow);
      store_rows_lds<BF16, D>(p.dv, kvoff, un.rs, k0w, nk, l32, hl, dv, 1.f, ow);
    }
  }
};

// waves per SIMD the dQ kernel's registers are fitted to.  At d = 64 the
// kernels with 16-bit gradients (staged through LDS for their stores)
// spilled 3-4 VGPRs at 4, and the masked and block-sparse ones 4-21; at 3
// none spills (134-160 VGPRs) and the plain ones measured 2-4% faster.  The
// plain kernels with f32 gradients fit 4 without spilling, and 3 measured
// 6% slower for them.
#ifndef SDPA_BWD_DQ_WAVES_D64
#define SDPA_BWD_DQ_WAVES_D64 3
#endif
#ifndef SDPA_BWD_DQ_WAVES_D64_GF32
#define SDPA_BWD_DQ_WAVES_D64_GF32 4
#endif
template <int D, bool GF32, int MK>
constexpr int kBwdDqWavesPerSimd =
    D == 32   ? 4
    : D == 64 ? (GF32 && MK == kPlain ? SDPA_BWD_DQ_WAVES_D64_GF32 : SDPA_BWD_DQ_WAVES_D64)
              : 2;
// with dropout the Philox state needs more registers
template <int D>
constexpr int kBwdDqDropWavesPerSimd = D == 32 ? 4 : D == 64 ? 3 : 2;

// key groups (8 waves): one workgroup per CU, 256 VGPRs
template <bool BF16, int D, int NW, int BN, bool CAUSAL, bool GF32, bool DROP, bool VARLEN,
          int MK, int KS = 1>
__global__ __launch_bounds__(NW * 64, (KS > 1 ? 2 : DROP ? kBwdDqDropWavesPerSimd<D> : kBwdDqWavesPerSimd<D, GF32, MK>))
void bwd_dq_kernel(BwdParams p) {
  using K = BwdDq<BF16, D, NW, BN, CAUSAL, GF32, DROP, VARLEN, MK, KS>;
  __shared__ typename K::Smem sm;
  K::run(p, sm);
}

// waves per SIMD the dK/dV kernel's registers are fitted to (d = 128: one
// wave per SIMD would hold it without spilling, but halves the resident
// workgroups and measured 20% slower than two with a few spilled VGPRs)
#ifndef SDPA_BWD_KV_WAVES_D128
#define SDPA_BWD_KV_WAVES_D128 2
#endif
template <int D>
constexpr int kBwdKvWavesPerSimd = D == 32 ? 4 : D == 64 ? 3 : SDPA_BWD_KV_WAVES_D128;
// with dropout: -D of 16 queries and the Philox state stay live
template <int D>
constexpr int kBwdKvDropWavesPerSimd = D == 32 ? 3 : D == 64 ? 2 : 1;

// with an elementwise mask (its elements of a step are held in registers):
// bounds that do not spill, except for boolean masks at d = 32 (2-4 VGPRs
// spilled at 4 waves measured 3-4% faster than 3 waves without).  Against
// the dense bounds, measured on B32 H8 N1024 d = 64 and B32 H32 N1024
// d = 32 (f16): d = 64 +4-8% for boolean and additive masks, +17% on the
// key-padding workload (B32 H8 N512); additive masks at d = 32 +7-13%.
#ifndef SDPA_BWD_KVM_WAVES_D32
#define SDPA_BWD_KVM_WAVES_D32 3
#endif
#ifndef SDPA_BWD_KVMB_WAVES_D32
#define SDPA_BWD_KVMB_WAVES_D32 4
#endif
#ifndef SDPA_BWD_KVM_WAVES_D64
#define SDPA_BWD_KVM_WAVES_D64 2
#endif
template <int D, int MK>
constexpr int kBwdKvMaskWavesPerSimd =
    MK < kMaskBool ? kBwdKvWavesPerSimd<D>
    : D == 32      ? (MK == kMaskBool ? SDPA_BWD_KVMB_WAVES_D32 : SDPA_BWD_KVM_WAVES_D32)
    : D == 64      ? SDPA_BWD_KVM_WAVES_D64
                   : kBwdKvWavesPerSimd<D>;

// query groups (8 waves): one workgroup per CU, 256 VGPRs
template <bool BF16, int D, int NW, int BQ, bool CAUSAL, bool GF32, bool DROP, bool VARLEN,
          int MK, int KS = 1>
__global__ __launch_bounds__(NW * 64, (KS > 1 ? 2 : DROP ? kBwdKvDropWavesPerSimd<D> : kBwdKvMaskWavesPerSimd<D, MK>))
void bwd_dkdv_kernel(BwdParams p) {
  using K = BwdDkdv<BF16, D, NW, BQ, CAUSAL, GF32, DROP, VARLEN, MK, KS>;
  __shared__ typename K::Smem sm;
  K::run(p, sm);
}

}  // namespace sdpa
