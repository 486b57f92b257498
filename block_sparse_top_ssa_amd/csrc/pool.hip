// Block mean-pooling of keys: kbar[b,h,j,:] = (1/s) sum_{i=js}^{js+s-1} k[b,h,i,:].
// Paper sec. 3 (p. 4): contiguous blocks of s tokens, one mean-pooled key per block.
//
// HBM-bound: each wave owns one block and sums it with block_key_sum (16-byte loads of
// whole rows, float32 partial sums per lane, xor-shuffle fold).
#include "launch.hpp"
#include "pool.hpp"

namespace ssa {

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_kernel(const T* __restrict__ k, float* __restrict__ km,
                                                   int64_t nblocks, int s, float inv_s) {
  constexpr int E = Elem<T>::kPer16B;
  constexpr int LPR = D / E;  // lanes per row
  const int lane = threadIdx.x & 63;
  const int64_t blk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= nblocks) return;
  // Blocks are contiguous in [B,H,L,D] because L = n*s: block blk starts at row blk*s.
  float acc[E];
  block_key_sum<T, D>(k + blk * (int64_t)s * D, s, s, -1, k, acc);
  if (lane < LPR) {
    float* dst = km + blk * D + lane * E;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      u32x4 w;
      w[0] = __float_as_uint(acc[e] * inv_s);
      w[1] = __float_as_uint(acc[e + 1] * inv_s);
      w[2] = __float_as_uint(acc[e + 2] * inv_s);
      w[3] = __float_as_uint(acc[e + 3] * inv_s);
      store16(dst + e, w);
    }
  }
}

template <typename T, int D>
static hipError_t run_pool(const Dims& d, const void* k, float* km, hipStream_t st) {
  const int64_t nblocks = d.bh() * d.n();
  const int64_t grid = (nblocks + 3) / 4;
  hipLaunchKernelGGL((pool_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, st,
                     static_cast<const T*>(k), km, nblocks, d.S, 1.0f / (float)d.S);
  return hipGetLastError();
}

LaunchResult launch_pool(const Dims& d, const void* k, float* km, hipStream_t st) {
  LaunchResult r;
  if (d.dtype == 1) r.err = d.D == 128 ? run_pool<uint16_t, 128>(d, k, km, st) : run_pool<uint16_t, 64>(d, k, km, st);
  else r.err = d.D == 128 ? run_pool<float, 128>(d, k, km, st) : run_pool<float, 64>(d, k, km, st);
  return r;
}

}  // namespace ssa
