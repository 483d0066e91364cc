// Attention forward for f32 inputs on the vector ALUs.
//
// f32 has no dense-contraction fast path worth the complexity here (its
// use is small problems such as the tutorial's 2x3x8 example), so this is
// a direct fp32 kernel: one lane per query row, key/value blocks of 32 rows
// staged in LDS and broadcast to the wave, the same running-max / running-
// sum recurrence as the matrix-core kernel, output and logsumexp written
// once.
#include "sdpa_internal.h"

namespace sdpa {

namespace {

constexpr int F32_ROWS = 64;  // query rows per workgroup (one wave)
constexpr int F32_KEYS = 32;  // keys per LDS block

struct F32Params {
  const float* q;
  const float* k;
  const float* v;
  float* out;
  float* lse;
  const int32_t* cu;
  int H, Nq, Nk, d;
  int n_qtiles;
  float c;  // scale * log2(e)
  int causal;
};

template <int DMAX, bool VARLEN>
__global__ __launch_bounds__(F32_ROWS) void fwd_f32_kernel(F32Params p) {
  __shared__ __attribute__((aligned(16))) float ks[F32_KEYS][DMAX];
  __shared__ float vs[F32_KEYS][DMAX];
  const int tid = threadIdx.x;
  const int qt = blockIdx.x % p.n_qtiles;
  const int bh = blockIdx.x / p.n_qtiles;
  const int b = bh / p.H, h = bh % p.H;
  const int d = p.d;

  int nq, nk;
  int64_t qoff, kvoff, rs;
  if (VARLEN) {
    const int s0 = p.cu[b], s1 = p.cu[b + 1];
    nq = nk = s1 - s0;
    rs = (int64_t)p.H * d;
    qoff = kvoff = (int64_t)s0 * rs + (int64_t)h * d;
  } else {
    nq = p.Nq;
    nk = p.Nk;
    rs = d;
    qoff = (int64_t)bh * p.Nq * d;
    kvoff = (int64_t)bh * p.Nk * d;
  }
  const int q0 = qt * F32_ROWS;
  if (q0 >= nq) return;
  const int qi = q0 + tid;
  const bool live = qi < nq;

  float q[DMAX], acc[DMAX];
#pragma unroll
  for (int c = 0; c < DMAX; ++c) {
    q[c] = (live && c < d) ? p.q[qoff + (int64_t)qi * rs + c] : 0.f;
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kend = p.causal ? min(nk, q0 + F32_ROWS) : nk;

  for (int kb = 0; kb < kend; kb += F32_KEYS) {
    __syncthreads();
    for (int e = tid; e < F32_KEYS * DMAX; e += F32_ROWS) {
      const int r = e / DMAX, c = e % DMAX;
      const bool in = (kb + r < nk) && c < d;
      ks[r][c] = in ? p.k[kvoff + (int64_t)(kb + r) * rs + c] : 0.f;
      vs[r][c] = in ? p.v[kvoff + (int64_t)(kb + r) * rs + c] : 0.f;
    }
    __syncthreads();

    float s[F32_KEYS];
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < F32_KEYS; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < DMAX; ++c) dot = __builtin_fmaf(q[c], ks[j][c], dot);
      const int key = kb + j;
      const bool ok = key < nk && (!p.causal || key <= qi);
      s[j] = ok ? dot : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float ms = (mt == -INFINITY) ? -INFINITY : mt * p.c;
    const float mnew = fmaxf(m, ms);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = __builtin_amdgcn_exp2f(m - mref);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < DMAX; ++c) acc[c] *= alpha;
#pragma unroll
    for (int j = 0; j < F32_KEYS; ++j) {
      const float e = (s[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], p.c, -mref));
      l += e;
#pragma unroll
      for (int c = 0; c < DMAX; ++c) acc[c] = __builtin_fmaf(e, vs[j][c], acc[c]);
    }
  }

  if (!live) return;
  const float inv = 1.f / l;
  for (int c = 0; c < d; ++c) p.out[qoff + (int64_t)qi * rs + c] = acc[c] * inv;
  if (p.lse != nullptr) {
    const float lse = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
    if (VARLEN)
      p.lse[(int64_t)(p.cu[b] + qi) * p.H + h] = lse;
    else
      p.lse[(int64_t)bh * p.Nq + qi] = lse;
  }
}

template <int DMAX>
hipError_t launch_dmax(const FwdArgs& a, const F32Params& p, int grid) {
  if (a.cu != nullptr)
    hipLaunchKernelGGL((fwd_f32_kernel<DMAX, true>), dim3(grid), dim3(F32_ROWS), 0, a.stream, p);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<DMAX, false>), dim3(grid), dim3(F32_ROWS), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a) {
  F32Params p;
  p.q = static_cast<const float*>(a.q);
  p.k = static_cast<const float*>(a.k);
  p.v = static_cast<const float*>(a.v);
  p.out = static_cast<float*>(a.out);
  p.lse = a.lse;
  p.cu = a.cu;
  p.H = (int)a.H;
  p.Nq = (int)a.Nq;
  p.Nk = (int)a.Nk;
  p.d = (int)a.d;
  p.n_qtiles = (int)((a.Nq + F32_ROWS - 1) / F32_ROWS);
  p.c = a.scale * 1.4426950408889634f;
  p.causal = a.causal ? 1 : 0;
  const int grid = (int)(a.B * a.H * p.n_qtiles);
  if (a.d <= 8) return launch_dmax<8>(a, p, grid);
  if (a.d <= 16) return launch_dmax<16>(a, p, grid);
  if (a.d <= 32) return launch_dmax<32>(a, p, grid);
  if (a.d <= 64) return launch_dmax<64>(a, p, grid);
  return launch_dmax<128>(a, p, grid);
}

}  // namespace sdpa
