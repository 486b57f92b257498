// V (and, for the sparse stream, K) rewritten once into the MFMA fragment order the
// attention kernels read as A operands -- of O^T = V^T P^T and S^T = K Q^T (paper sec. 3,
// pp. 3-4: both streams score the keys against the query and weight V) -- and the
// stream-ordered workspace that holds them.
#include <mutex>

#include "launch.hpp"
#include "mfma.hpp"

namespace ssa {

// ---------------------------------------------------------------- one chunk through LDS
// The 64 rows of a 64-key chunk (contiguous in a [B,H,L,D] tensor) read with 16-byte
// loads of consecutive words, so each wave instruction moves 1 KB of whole cache lines,
// into LDS rows of D/8 + 1 words (the extra word staggers neighbouring rows over the
// banks; rows 16 apart still meet, a 2-way conflict on the fragment reads that costs
// nothing next to the HBM traffic).  Both copies below then take each lane's 16 bytes,
// one word of one row, from LDS.
template <int D>
struct ChunkTile {
  static constexpr int RW = D / 8, RS = RW + 1;  // 16-byte words per row; LDS row stride
  u32x4 w[64 * RS];
};
template <int D>
__device__ __forceinline__ void stage_chunk(ChunkTile<D>& t, const uint16_t* __restrict__ x, int64_t bh, int L,
                                            int c) {
  constexpr int RW = ChunkTile<D>::RW, RS = ChunkTile<D>::RS;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + (bh * (int64_t)L + 64 * c) * D);
#pragma unroll
  for (int i = threadIdx.x; i < 64 * RW; i += 256) t.w[(i / RW) * RS + i % RW] = src[i];
  __syncthreads();
}

// ---------------------------------------------------------------- V in fragment order
// Fragment (chunk c, d tile dt, key half kc) of a head: 64 lanes x 16 bytes; lane
// l = 16 g + i holds V[64 c + kappa(kc, g, 0..7)][16 dt + i], the A operand of
// O^T = V^T P^T.  One workgroup per 64-key chunk: lane 16 g + 8 h + p takes row
// kappa(kc, g, p), columns 16 dt + 8 h .. +7, and an 8x8 transpose inside each group of
// 8 lanes turns rows into columns.
template <int D>
__global__ __launch_bounds__(256) void vfrag_kernel(const uint16_t* __restrict__ v, u32x4* __restrict__ vt, int L) {
  constexpr int F = 2 * (D / 16), RS = ChunkTile<D>::RS;  // fragments per chunk
  __shared__ ChunkTile<D> tile;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, h = (lane >> 3) & 1, p = lane & 7;
  const int64_t chunk = blockIdx.x;  // over B*H*(L/64), head-major
  const int nck = L / 64;
  stage_chunk<D>(tile, v, chunk / nck, L, (int)(chunk % nck));
  for (int f = w; f < F; f += 4) {
    const int dt = f >> 1, kc = f & 1;
    vt[(chunk * F + f) * 64 + lane] = transpose8x8_b16_dpp(tile.w[kappa(kc, g, p) * RS + 2 * dt + h]);
  }
}

// ---------------------------------------------------------------- K in fragment order
// Fragment (chunk c, key tile kt, contraction chunk cc) of a head: 64 lanes x 16 bytes;
// lane l = 16 g + i holds K[64 c + 16 kt + i][32 cc + 8 g .. + 7], the A operand of
// S^T = K Q^T.  Read from here a fragment is one contiguous 1 KB load (8 full cache
// lines) instead of 16 half lines of K's rows.  One workgroup per 64-key chunk.
template <int D>
__global__ __launch_bounds__(256) void kfrag_kernel(const uint16_t* __restrict__ k, u32x4* __restrict__ kt, int L) {
  constexpr int NC = D / 32, F = 4 * NC, RS = ChunkTile<D>::RS;  // fragments per chunk
  __shared__ ChunkTile<D> tile;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t chunk = blockIdx.x;  // over B*H*(L/64), head-major
  const int nck = L / 64;
  stage_chunk<D>(tile, k, chunk / nck, L, (int)(chunk % nck));
  for (int f = w; f < F; f += 4)
    kt[(chunk * F + f) * 64 + lane] = tile.w[(16 * (f / NC) + (lane & 15)) * RS + 4 * (f % NC) + (lane >> 4)];
}

// ---------------------------------------------------------------- workspace
// The V^T copy lives in stream-ordered memory from a pool the library keeps per
// device: freed blocks stay in the pool, so after the first call of a size the
// allocation is a pool hit that neither blocks the host nor synchronises the device.
static hipError_t workspace_pool(hipMemPool_t* out) {
  static std::mutex mu;
  static hipMemPool_t pools[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!pools[dev]) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t p = nullptr;
    e = hipMemPoolCreate(&p, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = ~0ull;
    e = hipMemPoolSetAttribute(p, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) return e;
    pools[dev] = p;
  }
  *out = pools[dev];
  return hipSuccess;
}

template <int D>
static hipError_t run_vfrag(const Dims& d, const void* v, u32x4* vt, hipStream_t st) {
  const int64_t grid = d.bh() * (d.L / 64);
  hipLaunchKernelGGL((vfrag_kernel<D>), dim3((unsigned)grid), dim3(256), 0, st, static_cast<const uint16_t*>(v), vt,
                     d.L);
  return hipGetLastError();
}

hipError_t vfrag_acquire(const Dims& d, const void* v, void** ws, hipStream_t st) {
  *ws = nullptr;
  hipMemPool_t pool = nullptr;
  hipError_t e = workspace_pool(&pool);
  if (e != hipSuccess) return e;
  e = hipMallocFromPoolAsync(ws, (size_t)d.tokens() * d.D * 2, pool, st);
  if (e != hipSuccess) return e;
  e = d.D == 128 ? run_vfrag<128>(d, v, static_cast<u32x4*>(*ws), st)
                 : run_vfrag<64>(d, v, static_cast<u32x4*>(*ws), st);
  if (e != hipSuccess) {
    (void)hipFreeAsync(*ws, st);
    *ws = nullptr;
  }
  return e;
}

hipError_t vfrag_release(void* ws, hipStream_t st) { return ws ? hipFreeAsync(ws, st) : hipSuccess; }

template <int D>
static hipError_t run_kfrag(const Dims& d, const void* k, u32x4* kt, hipStream_t st) {
  const int64_t grid = d.bh() * (d.L / 64);
  hipLaunchKernelGGL((kfrag_kernel<D>), dim3((unsigned)grid), dim3(256), 0, st, static_cast<const uint16_t*>(k), kt,
                     d.L);
  return hipGetLastError();
}

hipError_t kfrag_acquire(const Dims& d, const void* k, void** ws, hipStream_t st) {
  *ws = nullptr;
  hipMemPool_t pool = nullptr;
  hipError_t e = workspace_pool(&pool);
  if (e != hipSuccess) return e;
  e = hipMallocFromPoolAsync(ws, (size_t)d.tokens() * d.D * 2, pool, st);
  if (e != hipSuccess) return e;
  e = d.D == 128 ? run_kfrag<128>(d, k, static_cast<u32x4*>(*ws), st)
                 : run_kfrag<64>(d, k, static_cast<u32x4*>(*ws), st);
  if (e != hipSuccess) {
    (void)hipFreeAsync(*ws, st);
    *ws = nullptr;
  }
  return e;
}

hipError_t kv_frag_into(const Dims& d, const void* k, const void* v, void* kf, void* vf, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (kf)
    e = d.D == 128 ? run_kfrag<128>(d, k, static_cast<u32x4*>(kf), st) : run_kfrag<64>(d, k, static_cast<u32x4*>(kf), st);
  if (e == hipSuccess && vf)
    e = d.D == 128 ? run_vfrag<128>(d, v, static_cast<u32x4*>(vf), st) : run_vfrag<64>(d, v, static_cast<u32x4*>(vf), st);
  return e;
}

hipError_t frag_order_into(const Dims& d, const void* x, void* out, hipStream_t st) {
  return d.D == 128 ? run_vfrag<128>(d, x, static_cast<u32x4*>(out), st)
                    : run_vfrag<64>(d, x, static_cast<u32x4*>(out), st);
}

hipError_t workspace_alloc(size_t bytes, void** ws, hipStream_t st) {
  *ws = nullptr;
  hipMemPool_t pool = nullptr;
  hipError_t e = workspace_pool(&pool);
  if (e != hipSuccess) return e;
  return hipMallocFromPoolAsync(ws, bytes, pool, st);
}

hipError_t workspace_free(void* ws, hipStream_t st) { return ws ? hipFreeAsync(ws, st) : hipSuccess; }

}  // namespace ssa
