// Per-token comparison of the two streams.
//   dist(t)    = ||o_full(t) - o_sparse(t)||_2 over the head dim (paper sec. 5, pp. 6-7:
//                the counterpart outputs are compared at every layer);
//   dropped(t) = clamp(-expm1(lse_sparse(t) - lse_full(t)), 0, 1): the full-attention mass
//                on tokens the sparse stream leaves out (App. B p. 19, sec. 4.2 p. 6),
//                since exp(lse_s - lse_f) is the full-attention mass the sparse set keeps.
//   retained_hist (optional): per (b, h), the number of rows whose retained mass
//                1 - dropped(t) falls in [m/16, (m+1)/16) (m = 15 also holding 1), the
//                distribution of the sparse stream's kept attention mass the pages
//                report (App. H, Table A9: attention sparsity as the mass kept).
// HBM-bound streaming reduction: a row of D elements is D/E lanes wide (E elements per
// 16-byte load); each wave handles 64/(D/E) tokens per step and loops over 4 steps.  A
// step's tokens lie in one (b, h) (64 divides L); the wave counts its rows per bin with
// ballots and adds each non-zero count to the histogram with one float atomic (whole
// numbers, so the sums do not depend on the order).
#include "launch.hpp"

namespace ssa {

constexpr int kRetainedBins = 16;

__global__ __launch_bounds__(256) void align_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void align_kernel(const T* __restrict__ of, const T* __restrict__ os,
                                                    const float* __restrict__ lf, const float* __restrict__ ls,
                                                    float* __restrict__ dist, float* __restrict__ drop,
                                                    float* __restrict__ rhist, int64_t ntok, int L) {
  constexpr int E = Elem<T>::kPer16B;
  constexpr int LPR = D / E;
  constexpr int TPW = kWave / LPR;  // tokens per wave step
  constexpr int STEPS = 4;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t first = ((int64_t)blockIdx.x * 4 + wave) * (TPW * STEPS);
  const int c = lane % LPR;
#pragma unroll
  for (int u = 0; u < STEPS; ++u) {
    const int64_t tok = first + u * TPW + lane / LPR;
    const bool ok = tok < ntok;
    if (dist) {
      float acc = 0.f;
      if (ok) {
        float a[E], b[E];
        Elem<T>::unpack(load16(of + tok * D + c * E), a);
        Elem<T>::unpack(load16(os + tok * D + c * E), b);
#pragma unroll
        for (int e = 0; e < E; ++e) { const float df = a[e] - b[e]; acc = fmaf(df, df, acc); }
      }
#pragma unroll
      for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o);
      if (ok && c == 0) dist[tok] = sqrtf(acc);
    }
    if ((drop || rhist) && ok && c == 0) {
      const float x = ls[tok] - lf[tok];
      const float dm = fminf(fmaxf(-expm1f(x), 0.f), 1.f);
      if (drop) drop[tok] = dm;
    }
    if (rhist) {
      int bin = -1;
      if (ok && c == 0) {
        const float dm = fminf(fmaxf(-expm1f(ls[tok] - lf[tok]), 0.f), 1.f);
        bin = min((int)((1.f - dm) * kRetainedBins), kRetainedBins - 1);
      }
      const int64_t t0 = first + u * TPW;  // the step's first token: its (b, h) holds them all
      if (t0 < ntok) {
        float* hb = rhist + (t0 / L) * kRetainedBins;
#pragma unroll
        for (int b = 0; b < kRetainedBins; ++b) {
          const uint64_t mk = __builtin_amdgcn_ballot_w64(bin == b);
          if (mk && lane == 0) atomicAdd(hb + b, (float)__builtin_popcountll(mk));
        }
      }
    }
  }
}

template <typename T, int D>
static hipError_t run_align(const Dims& d, const void* of, const void* os, const float* lf, const float* ls,
                            float* dist, float* drop, float* rhist, hipStream_t st) {
  constexpr int LPR = D / Elem<T>::kPer16B;
  const int64_t per_block = 4 * (kWave / LPR) * 4;
  const int64_t ntok = d.tokens();
  const int64_t grid = (ntok + per_block - 1) / per_block;
  if (rhist) {  // the counts start at zero (a kernel, not a memset: callers may capture this in a graph)
    const int64_t nb = d.bh() * kRetainedBins;
    hipLaunchKernelGGL(align_zero_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st, rhist, nb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((align_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, st, static_cast<const T*>(of),
                     static_cast<const T*>(os), lf, ls, dist, drop, rhist, ntok, d.L);
  return hipGetLastError();
}

LaunchResult launch_align(const Dims& d, const void* of, const void* os, const float* lf, const float* ls,
                          float* dist, float* drop, hipStream_t st, float* rhist) {
  LaunchResult r;
  if (d.dtype == 1)
    r.err = d.D == 128 ? run_align<uint16_t, 128>(d, of, os, lf, ls, dist, drop, rhist, st)
                       : run_align<uint16_t, 64>(d, of, os, lf, ls, dist, drop, rhist, st);
  else
    r.err = d.D == 128 ? run_align<float, 128>(d, of, os, lf, ls, dist, drop, rhist, st)
                       : run_align<float, 64>(d, of, os, lf, ls, dist, drop, rhist, st);
  return r;
}

}  // namespace ssa
