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
//            K/V in that XCD's L2.  Causal tiles of a head run heaviest
//            first.
//   waves    NW waves; wave w owns NB blocks of 32 query rows.
//   tile     BN keys per step, staged through double-buffered LDS:
//            K row-major [BN][D+8], V transposed [D][BN+4] (f16 always).
//
// Register dataflow per 32x32 block (v_mfma_f32_32x32x16, wave64):
//   S^T = K . Q^T      A = K rows from LDS, B = Q rows held in VGPRs.
//                      Lane l owns query l%32 and keys 8(r/4)+4(l/32)+r%4,
//                      r = 0..15, so a row max/sum is 15 in-lane ops plus
//                      one v_permlane32_swap exchange with lane l^32.
//   P = exp2(S*c - m)  c = scale*log2(e); running max m and per-lane
//                      partial row sums l in fp32 registers.
//   O^T += V^T . P^T   B = P converted to f16 straight from the S^T
//                      accumulator registers (no LDS round trip); A = V^T
//                      read from the transposed LDS tile with the matching
//                      key order.  bf16 inputs: V is converted to f16 when
//                      it is staged (exact for |v| <= 65504), P is f16.
//   epilogue           O = acc / l, lse = ln2 * (m + log2 l), one store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
  int n_qtiles;        // query tiles per (batch, head)
  int total;           // grid size
  float c;             // scale * log2(e)
};

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

// bf16 bit pattern -> f16 bit pattern (exact for normal f16 magnitudes).
__device__ __forceinline__ uint32_t bf16_to_f16_bits(uint32_t b) {
  _Float16 h = (_Float16)__uint_as_float(b << 16);
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

template <bool BF16, int D, int NB, int NW, bool CAUSAL, bool VARLEN, bool OUTF32>
struct MfmaFwd {
  static constexpr int BM = NW * NB * 32;  // query rows per workgroup
  static constexpr int BN = (D >= 128) ? 32 : 64;  // keys per step
  static constexpr int KB = BN / 32;       // 32-key blocks per step
  static constexpr int DS = D / 16;        // k-steps of S = Q K^T
  static constexpr int DB = D / 32;        // 32-row blocks of O^T
  static constexpr int NT = NW * 64;
  static constexpr int KROW = D + 8;       // LDS K row, elements
  static constexpr int VROW = BN + 4;      // LDS V^T row, elements
  static constexpr int KCHUNKS = BN * D / 8;         // 16-byte K chunks per tile
  static constexpr int VPAIRS = (BN / 2) * (D / 8);  // (2 rows x 16 bytes) V chunks
  static constexpr int KPT = (KCHUNKS + NT - 1) / NT;
  static constexpr int VPT = (VPAIRS + NT - 1) / NT;
  static_assert(D % 32 == 0 && D <= 128, "head dim");

  struct __attribute__((aligned(16))) Smem {
    uint16_t k[2][BN * KROW];
    uint16_t vt[2][D * VROW];
  };

  struct Prefetch {
    u32x4 k[KPT];
    u32x4 v0[VPT], v1[VPT];
  };

  // Global -> registers for key tile starting at key kb (rows >= nk read as 0).
  static __device__ __forceinline__ void load_tile(Prefetch& pf, const uint16_t* kbase,
                                                   const uint16_t* vbase, int64_t rs, int kb,
                                                   int nk, int tid) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      int c = tid + i * NT;
      pf.k[i] = u32x4{0, 0, 0, 0};
      if (KCHUNKS % NT == 0 || c < KCHUNKS) {
        int row = c / (D / 8), col = (c % (D / 8)) * 8;
        if (kb + row < nk)
          pf.k[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)(kb + row) * rs + col);
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int c = tid + i * NT;
      pf.v0[i] = u32x4{0, 0, 0, 0};
      pf.v1[i] = u32x4{0, 0, 0, 0};
      if (VPAIRS % NT == 0 || c < VPAIRS) {
        int pr = c / (D / 8), col = (c % (D / 8)) * 8;
        int r0 = kb + 2 * pr;
        if (r0 < nk)
          pf.v0[i] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)r0 * rs + col);
        if (r0 + 1 < nk)
          pf.v1[i] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)(r0 + 1) * rs + col);
      }
    }
  }

  // Registers -> LDS buffer `buf` (K as is, V transposed to [d][key], f16).
  static __device__ __forceinline__ void store_tile(Smem& sm, int buf, const Prefetch& pf,
                                                    int tid) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      int c = tid + i * NT;
      if (KCHUNKS % NT == 0 || c < KCHUNKS) {
        int row = c / (D / 8), col = (c % (D / 8)) * 8;
        *reinterpret_cast<u32x4*>(&sm.k[buf][row * KROW + col]) = pf.k[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      int c = tid + i * NT;
      if (VPAIRS % NT == 0 || c < VPAIRS) {
        int pr = c / (D / 8), col = (c % (D / 8)) * 8;
        uint32_t* dst = reinterpret_cast<uint32_t*>(&sm.vt[buf][col * VROW + 2 * pr]);
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          uint32_t a = (pf.v0[i][t / 2] >> (16 * (t & 1))) & 0xffffu;
          uint32_t b = (pf.v1[i][t / 2] >> (16 * (t & 1))) & 0xffffu;
          if (BF16) {
            a = bf16_to_f16_bits(a);
            b = bf16_to_f16_bits(b);
          }
          dst[t * (VROW / 2)] = a | (b << 16);
        }
      }
    }
  }

  static __device__ void run(const MfmaParams& p, Smem& sm) {
    const int tid = threadIdx.x;
    const int wave = tid / 64;
    const int lane = tid % 64;
    const int hl = lane / 32;
    const int l32 = lane % 32;

    // ---- which tile: XCD-contiguous ranges, heads' tiles back to back
    int tile = blockIdx.x;
    if ((p.total & 7) == 0) {
      const int per = p.total >> 3;
      tile = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    }
    int qt = tile % p.n_qtiles;
    const int bh = tile / p.n_qtiles;
    if (CAUSAL) qt = p.n_qtiles - 1 - qt;
    const int b = bh / p.H, h = bh % p.H;

    int nq, nk;
    int64_t qoff, kvoff, rs;
    if (VARLEN) {
      const int s0 = p.cu[b], s1 = p.cu[b + 1];
      nq = nk = s1 - s0;
      rs = (int64_t)p.H * D;
      qoff = kvoff = (int64_t)s0 * rs + (int64_t)h * D;
    } else {
      nq = p.Nq;
      nk = p.Nk;
      rs = D;
      qoff = (int64_t)bh * p.Nq * D;
      kvoff = (int64_t)bh * p.Nk * D;
    }
    const int q0 = qt * BM;
    if (q0 >= nq) return;  // whole workgroup: tile past the sequence end

    const uint16_t* qbase = p.q + qoff;
    const uint16_t* kbase = p.k + kvoff;
    const uint16_t* vbase = p.v + kvoff;
    const int kend = CAUSAL ? min(nk, q0 + BM) : nk;
    const int ntiles = (kend + BN - 1) / BN;

    const int wq0 = q0 + wave * NB * 32;   // first query row of this wave
    const bool wave_live = wq0 < nq;

    // ---- Q rows as the B operand of S^T = K Q^T
    u32x4 qf[NB][DS];
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      const int qi = wq0 + qb * 32 + l32;
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        qf[qb][ds] = u32x4{0, 0, 0, 0};
        if (qi < nq)
          qf[qb][ds] = *reinterpret_cast<const u32x4*>(qbase + (int64_t)qi * rs + ds * 16 + hl * 8);
      }
    }

    f32x16 o[NB][DB];
    float m[NB], l[NB];
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      m[qb] = -INFINITY;
      l[qb] = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[qb][db][r] = 0.f;
    }

    Prefetch pf;
    load_tile(pf, kbase, vbase, rs, 0, nk, tid);
    store_tile(sm, 0, pf, tid);
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
      const int buf = j & 1;
      const int kb = j * BN;
      const bool has_next = j + 1 < ntiles;
      if (has_next) load_tile(pf, kbase, vbase, rs, kb + BN, nk, tid);

      const bool skip = !wave_live || (CAUSAL && kb > wq0 + NB * 32 - 1);
      if (!skip) {
        const bool need_mask = (kb + BN > nk) || (CAUSAL && kb + BN - 1 > wq0);
        // ---- S^T = K Q^T
        f32x16 s[NB][KB];
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
          u32x4 kf[DS];
#pragma unroll
          for (int ds = 0; ds < DS; ++ds)
            kf[ds] = *reinterpret_cast<const u32x4*>(
                &sm.k[buf][(kk * 32 + l32) * KROW + ds * 16 + hl * 8]);
#pragma unroll
          for (int qb = 0; qb < NB; ++qb) {
            f32x16 acc;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
            for (int ds = 0; ds < DS; ++ds)
              acc = BF16 ? mfma_bf16(kf[ds], qf[qb][ds], acc) : mfma_f16(kf[ds], qf[qb][ds], acc);
            s[qb][kk] = acc;
          }
        }

        // ---- online softmax (exp2 domain)
        u32x4 pf16[NB][KB][2];
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
          const int qi = wq0 + qb * 32 + l32;
          if (need_mask) {
#pragma unroll
            for (int kk = 0; kk < KB; ++kk)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int key = kb + kk * 32 + 8 * (r / 4) + 4 * hl + (r % 4);
                const bool ok = key < nk && (!CAUSAL || key <= qi);
                if (!ok) s[qb][kk][r] = -INFINITY;
              }
          }
          float mt = -INFINITY;
#pragma unroll
          for (int kk = 0; kk < KB; ++kk)
#pragma unroll
            for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[qb][kk][r]);
          mt = pair_max(mt);
          // scaled tile max; a row with every key masked here keeps its max
          const float ms = (mt == -INFINITY) ? -INFINITY : mt * p.c;
          const float mnew = fmaxf(m[qb], ms);
          const float mref = (mnew == -INFINITY) ? 0.f : mnew;
          const float alpha = __builtin_amdgcn_exp2f(m[qb] - mref);
          m[qb] = mnew;
          const float nm = -mref;
          float rsum = 0.f;
#pragma unroll
          for (int kk = 0; kk < KB; ++kk) {
            float pv[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][kk][r], p.c, nm));
              if (need_mask && s[qb][kk][r] == -INFINITY) e = 0.f;
              pv[r] = e;
              rsum += e;
            }
#pragma unroll
            for (int hs = 0; hs < 2; ++hs)
              pf16[qb][kk][hs] = u32x4{pack_f16(pv[8 * hs + 0], pv[8 * hs + 1]),
                                       pack_f16(pv[8 * hs + 2], pv[8 * hs + 3]),
                                       pack_f16(pv[8 * hs + 4], pv[8 * hs + 5]),
                                       pack_f16(pv[8 * hs + 6], pv[8 * hs + 7])};
          }
          l[qb] = l[qb] * alpha + rsum;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[qb][db][r] *= alpha;
        }

        // ---- O^T += V^T P^T
#pragma unroll
        for (int kk = 0; kk < KB; ++kk)
#pragma unroll
          for (int hs = 0; hs < 2; ++hs)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const uint16_t* vrow = &sm.vt[buf][(db * 32 + l32) * VROW + kk * 32 + 16 * hs + 4 * hl];
              const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
              const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 8);
              const u32x4 vf = u32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
              for (int qb = 0; qb < NB; ++qb) o[qb][db] = mfma_f16(vf, pf16[qb][kk][hs], o[qb][db]);
            }
      }

      if (has_next) store_tile(sm, buf ^ 1, pf, tid);
      __syncthreads();
    }

    // ---- epilogue: normalise, store O and lse once
    if (!wave_live) return;
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      const int qi = wq0 + qb * 32 + l32;
      const float lt = pair_sum(l[qb]);
      const float inv = 1.f / lt;
      if (qi < nq) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dcol = db * 32 + 8 * g + 4 * hl;
            const float x0 = o[qb][db][4 * g + 0] * inv, x1 = o[qb][db][4 * g + 1] * inv;
            const float x2 = o[qb][db][4 * g + 2] * inv, x3 = o[qb][db][4 * g + 3] * inv;
            const int64_t off = qoff + (int64_t)qi * rs + dcol;
            if (OUTF32) {
              *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + off) =
                  f32x4{x0, x1, x2, x3};
            } else {
              const u32x2 w = BF16 ? u32x2{pack_bf16(x0, x1), pack_bf16(x2, x3)}
                                   : u32x2{pack_f16(x0, x1), pack_f16(x2, x3)};
              *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.out) + off) = w;
            }
          }
        if (p.lse != nullptr && hl == 0) {
          const float lse = (m[qb] + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f;
          if (VARLEN)
            p.lse[(int64_t)(p.cu[b] + qi) * p.H + h] = lse;
          else
            p.lse[(int64_t)bh * p.Nq + qi] = lse;
        }
      }
    }
  }
};

template <bool BF16, int D, int NB, int NW, bool CAUSAL, bool VARLEN, bool OUTF32>
__global__ __launch_bounds__(NW * 64, 2) void fwd_mfma_kernel(MfmaParams p) {
  using K = MfmaFwd<BF16, D, NB, NW, CAUSAL, VARLEN, OUTF32>;
  __shared__ typename K::Smem sm;
  K::run(p, sm);
}

}  // namespace sdpa
