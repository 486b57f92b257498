// Exact online-softmax attention for a single query row, one wave per row: each lane
// scores one key of a 64-key chunk (float32 dot product with q held in LDS), the wave
// keeps the running max / sum, and each lane accumulates D/64 output columns.
#pragma once
#include "common.hpp"

namespace ssa {

// Process keys [c*64, c*64+64) for one query row; `limit` = last key index allowed.
template <typename T, int D>
__device__ __forceinline__ void attend_chunk(const T* __restrict__ kh, const T* __restrict__ vh,
                                             const float* qs, int c, int limit, float scale, float& m,
                                             float& l, float* o) {
  constexpr int E = Elem<T>::kPer16B;
  const int lane = threadIdx.x & 63;
  const int key = c * 64 + lane;
  const bool valid = key <= limit;
  float s = -__builtin_huge_valf();
  if (valid) {
    const T* kr = kh + (int64_t)key * D;
    float acc = 0.f;
#pragma unroll 4
    for (int d = 0; d < D; d += E) {
      float x[E];
      Elem<T>::unpack(load16(kr + d), x);
#pragma unroll
      for (int e = 0; e < E; ++e) acc = fmaf(qs[d + e], x[e], acc);
    }
    s = acc * scale;
  }
  const float mc = wave_max(s);
  const float m_new = fmaxf(m, mc);
  const float alpha = expf(m - m_new);
  const float p = valid ? expf(s - m_new) : 0.f;
  l = l * alpha + wave_sum(p);
#pragma unroll
  for (int e = 0; e < D / 64; ++e) o[e] *= alpha;
  const int nkeys = min(64, limit - c * 64 + 1);
  for (int kk = 0; kk < nkeys; ++kk) {
    const float pk = __shfl(p, kk);
    const T* vr = vh + (int64_t)(c * 64 + kk) * D;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) o[e] = fmaf(pk, Elem<T>::load1(vr + lane + 64 * e), o[e]);
  }
  m = m_new;
}

// The sparse stream for one query row t: the chunk holding t first (causal), then the
// rest of the own block, then every listed block below the own block (entries outside
// [0, b_t) or not above the previous used entry are skipped).
template <typename T, int D>
__device__ __forceinline__ void attend_sparse_row(const T* __restrict__ kh, const T* __restrict__ vh,
                                                  const float* qs, const int32_t* __restrict__ ir, int topk,
                                                  int t, int S, float scale, float& m, float& l, float* acc) {
  const int ct = t / 64;
  attend_chunk<T, D>(kh, vh, qs, ct, t, scale, m, l, acc);
  const int bt = t / S, cpb = S / 64;
  for (int c = bt * cpb; c < ct; ++c) attend_chunk<T, D>(kh, vh, qs, c, t, scale, m, l, acc);
  int prev = -1;
  for (int e = 0; e < topk; ++e) {
    const int j = ir[e];
    if (j > prev && j < bt) {
      prev = j;
      for (int ch = 0; ch < cpb; ++ch) attend_chunk<T, D>(kh, vh, qs, j * cpb + ch, t, scale, m, l, acc);
    }
  }
}

}  // namespace ssa
