// V rewritten once into the MFMA fragment order the attention kernels read as the A
// operand of O^T = V^T P^T (paper sec. 3, p. 3-4: both streams multiply the attention
// weights with V), and the stream-ordered workspace that holds it.
#include <mutex>

#include "launch.hpp"
#include "mfma.hpp"

namespace ssa {

// ---------------------------------------------------------------- V in fragment order
// Fragment (chunk c, d tile dt, key half kc) of a head: 64 lanes x 16 bytes; lane
// l = 16 g + i holds V[64 c + kappa(kc, g, 0..7)][16 dt + i], the A operand of
// O^T = V^T P^T.  One workgroup per 64-key chunk.
template <int D>
__global__ __launch_bounds__(256) void vfrag_kernel(const uint16_t* __restrict__ v, u32x4* __restrict__ vt, int L) {
  constexpr int F = 2 * (D / 16);  // fragments per chunk
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t chunk = blockIdx.x;  // over B*H*(L/64), head-major
  const int nck = L / 64;
  const int64_t bh = chunk / nck;
  const int c = (int)(chunk % nck);
  const uint16_t* vh = v + bh * (int64_t)L * D;
  for (int f = w; f < F; f += 4)
    vt[(chunk * F + f) * 64 + lane] = transpose8x8_b16_dpp(load_v_raw<D>(vh, c * 64, f >> 1, f & 1));
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
