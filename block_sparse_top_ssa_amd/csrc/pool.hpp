// Sum of the first `rows` keys of one block, shared by the block pooling kernel and the
// cache append (paper sec. 3, p. 4: one mean-pooled key per block of s tokens).
//
// One wave per block: lanes read 16-byte pieces of consecutive rows (a row of D elements
// is D/E lanes wide, E = elements per 16 bytes), so one wave-wide load covers 64/(D/E)
// whole rows.  Rows at or after `rows` add +0; row `sub` (if >= 0) is read from `subp`
// instead of the block.  Partial sums are float32 per lane, folded across the row groups
// with xor-shuffles, so every lane ends with the sums of its E columns (lane % (D/E)).
// The order of the additions depends only on (s, rows), so a full block summed here
// gives the same bits whichever kernel asks.
#pragma once
#include "common.hpp"

namespace ssa {

template <typename T, int D>
__device__ __forceinline__ void block_key_sum(const T* __restrict__ base, int s, int rows, int sub,
                                              const T* __restrict__ subp, float (&acc)[Elem<T>::kPer16B]) {
  constexpr int E = Elem<T>::kPer16B;
  constexpr int LPR = D / E;       // lanes per row
  constexpr int RPI = kWave / LPR; // rows per wave-wide load
  const int lane = threadIdx.x & 63;
  const int r0 = lane / LPR, c = lane % LPR;
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int r = r0; r < s; r += RPI * 4) {
    u32x4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int rr = r + u * RPI;
      const T* src = rr == sub ? subp + c * E : base + (int64_t)rr * D + c * E;
      w[u] = rr < rows ? load16(src) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float x[E];
      Elem<T>::unpack(w[u], x);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] += x[e];
    }
  }
#pragma unroll
  for (int o = LPR; o < kWave; o <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += __shfl_xor(acc[e], o);
}

}  // namespace ssa
