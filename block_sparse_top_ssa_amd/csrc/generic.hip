// Portable vector-ALU kernels for every op of the attention forward.  They serve the
// float32 element type, shapes the MFMA kernels do not take, and the tests that check
// each code path against the CPU oracle.  Plain float32 arithmetic throughout.
//
//  topk_generic   one workgroup per query row: scores sigma_j = q . kbar_j of every block
//                 before the query's own (paper sec. 3, p. 4), a bitonic sort of 64-bit
//                 (score, index) keys in LDS, ascending listing of the kept blocks.
//  attn_generic   one wave per query row: online softmax over 64-key chunks; each lane
//                 scores one key, and each lane accumulates D/64 output columns.  Full
//                 stream: every chunk up to the query (sec. 3, p. 3).  Sparse stream: the
//                 own block causally plus the listed blocks (sec. 3, p. 4).
#include "launch.hpp"
#include "rowattn.hpp"

namespace ssa {

constexpr int kTopkGenericMaxN = 4096;  // LDS holds 12 bytes per candidate

template <typename T, int D>
__global__ __launch_bounds__(256) void topk_generic_kernel(const T* __restrict__ q, const float* __restrict__ km,
                                                           int32_t* __restrict__ idx, float* __restrict__ sel,
                                                           int L, int S, int topk, int P, int G) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* qs = reinterpret_cast<float*>(smem);                   // [D]
  uint64_t* keys = reinterpret_cast<uint64_t*>(qs + D);         // [P]
  float* sc = reinterpret_cast<float*>(keys + P);               // [P]
  const int64_t row = blockIdx.x;                              // (b*H + h)*L + t
  const int64_t bh = row / L;
  const int t = (int)(row % L);
  const int bt = t / S;
  const int m = min(topk - 1, bt);
  const int n = L / S;
  const int tid = threadIdx.x;
  for (int d = tid; d < D; d += 256) qs[d] = Elem<T>::load1(q + row * D + d);
  __syncthreads();
  const float* kmh = km + (bh / G) * (int64_t)n * D;  // pooled keys of this head's K/V head
  for (int j = tid; j < P; j += 256) {
    if (j < bt) {
      float acc = 0.f;
      const float* kr = kmh + (int64_t)j * D;
      for (int d = 0; d < D; ++d) acc = fmaf(qs[d], kr[d], acc);
      sc[j] = acc;
      keys[j] = make_key(acc, j);
    } else {
      keys[j] = 0;
    }
  }
  __syncthreads();
  if (m < bt) {
    // bitonic sort, descending, over P (power of two) keys
    for (int k2 = 2; k2 <= P; k2 <<= 1) {
      for (int j2 = k2 >> 1; j2 > 0; j2 >>= 1) {
        for (int i = tid; i < P; i += 256) {
          const int p = i ^ j2;
          if (p > i) {
            const uint64_t a = keys[i], b = keys[p];
            const bool desc = (i & k2) == 0;
            if (desc ? (a < b) : (a > b)) { keys[i] = b; keys[p] = a; }
          }
        }
        __syncthreads();
      }
    }
  }
  // mark the kept candidates, then list them in ascending order
  unsigned char* kept = reinterpret_cast<unsigned char*>(sc + P);  // [P]
  for (int j = tid; j < P; j += 256) kept[j] = 0;
  __syncthreads();
  if (m < bt) {
    for (int r = tid; r < m; r += 256) kept[key_index(keys[r])] = 1;
  } else {
    for (int j = tid; j < bt; j += 256) kept[j] = 1;
  }
  __syncthreads();
  if (tid == 0) {
    int32_t* out = idx + row * topk;
    float* so = sel ? sel + row * topk : nullptr;
    int c = 0;
    for (int j = 0; j < bt; ++j)
      if (kept[j]) {
        out[c] = j;
        if (so) so[c] = sc[j];
        ++c;
      }
    out[c] = bt;
    if (so) so[c] = __builtin_huge_valf();
    for (int r = c + 1; r < topk; ++r) {
      out[r] = -1;
      if (so) so[r] = -__builtin_huge_valf();
    }
  }
}

template <typename T, int D, bool SPARSE>
__global__ __launch_bounds__(256) void attn_generic_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, const int32_t* __restrict__ idx,
                                                           int topk, int L, int S, float scale, int64_t nrows,
                                                           T* __restrict__ o, float* __restrict__ lse, int G) {
  __shared__ float qsh[4][D];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row >= nrows) return;
  const int64_t bh = row / L;
  const int t = (int)(row % L);
  float* qs = qsh[wave];
  for (int d = lane; d < D; d += 64) qs[d] = Elem<T>::load1(q + row * D + d);
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  const T* kh = k + (bh / G) * (int64_t)L * D;  // K/V head of this query head
  const T* vh = v + (bh / G) * (int64_t)L * D;
  float m = -__builtin_huge_valf(), l = 0.f, acc[D / 64];
#pragma unroll
  for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
  if (!SPARSE) {
    // the chunk holding the query itself first, so the running max is finite from the start
    const int ct = t / 64;
    attend_chunk<T, D>(kh, vh, qs, ct, t, scale, m, l, acc);
    for (int c = 0; c < ct; ++c) attend_chunk<T, D>(kh, vh, qs, c, t, scale, m, l, acc);
  } else {
    attend_sparse_row<T, D>(kh, vh, qs, idx + row * topk, topk, t, S, scale, m, l, acc);
  }
  if (o) {
    const float inv = 1.f / l;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) Elem<T>::store1(o + row * D + lane + 64 * e, acc[e] * inv);
  }
  if (lse && lane == 0) lse[row] = m + logf(l);
}

static int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

template <typename T, int D>
static hipError_t run_topk_generic(const Dims& d, const void* q, const float* km, int topk, int32_t* idx,
                                   float* sel, hipStream_t st) {
  const int P = next_pow2(max(1, d.n()));
  const size_t shm = D * sizeof(float) + (size_t)P * (8 + 4 + 1);
  hipLaunchKernelGGL((topk_generic_kernel<T, D>), dim3((unsigned)d.tokens()), dim3(256), shm, st,
                     static_cast<const T*>(q), km, idx, sel, d.L, d.S, topk, P, d.G());
  return hipGetLastError();
}

LaunchResult launch_topk_generic(const Dims& d, const void* q, const float* km, int topk, int32_t* idx,
                                 float* sel, hipStream_t st) {
  LaunchResult r;
  if (d.n() > kTopkGenericMaxN) {
    r.unsupported = "portable top-k kernel holds at most 4096 blocks per sequence";
    return r;
  }
  if (d.dtype == 1)
    r.err = d.D == 128 ? run_topk_generic<uint16_t, 128>(d, q, km, topk, idx, sel, st)
                       : run_topk_generic<uint16_t, 64>(d, q, km, topk, idx, sel, st);
  else
    r.err = d.D == 128 ? run_topk_generic<float, 128>(d, q, km, topk, idx, sel, st)
                       : run_topk_generic<float, 64>(d, q, km, topk, idx, sel, st);
  return r;
}

template <typename T, int D, bool SPARSE>
static hipError_t run_attn_generic(const Dims& d, const void* q, const void* k, const void* v, const int32_t* idx,
                                   int topk, float scale, void* o, float* lse, hipStream_t st) {
  const int64_t nrows = d.tokens();
  hipLaunchKernelGGL((attn_generic_kernel<T, D, SPARSE>), dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v), idx, topk, d.L,
                     d.S, scale, nrows, static_cast<T*>(o), lse, d.G());
  return hipGetLastError();
}

template <bool SPARSE>
static hipError_t dispatch_attn_generic(const Dims& d, const void* q, const void* k, const void* v,
                                        const int32_t* idx, int topk, float scale, void* o, float* lse,
                                        hipStream_t st) {
  if (d.dtype == 1)
    return d.D == 128 ? run_attn_generic<uint16_t, 128, SPARSE>(d, q, k, v, idx, topk, scale, o, lse, st)
                      : run_attn_generic<uint16_t, 64, SPARSE>(d, q, k, v, idx, topk, scale, o, lse, st);
  return d.D == 128 ? run_attn_generic<float, 128, SPARSE>(d, q, k, v, idx, topk, scale, o, lse, st)
                    : run_attn_generic<float, 64, SPARSE>(d, q, k, v, idx, topk, scale, o, lse, st);
}

LaunchResult launch_sparse_generic(const Dims& d, const void* q, const void* k, const void* v, const int32_t* idx,
                                   int topk, float scale, void* o, float* lse, hipStream_t st) {
  LaunchResult r;
  r.err = dispatch_attn_generic<true>(d, q, k, v, idx, topk, scale, o, lse, st);
  return r;
}

LaunchResult launch_full_generic(const Dims& d, const void* q, const void* k, const void* v, float scale, void* o,
                                 float* lse, hipStream_t st) {
  LaunchResult r;
  r.err = dispatch_attn_generic<false>(d, q, k, v, nullptr, 1, scale, o, lse, st);
  return r;
}

}  // namespace ssa
