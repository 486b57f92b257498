// Training both streams: the backward of the attention forward and the bidirectional
// alignment loss.
//
// SSA trains the full and the sparse stream of every layer (paper sec. 5, pp. 6-7; App. C,
// p. 20): the sampled main stream receives the language-model gradient, both receive the
// gradient of the alignment loss, so both attention forwards need their backward.  For
// o = softmax(scale q k^T) v over a key set A(t) (all i <= t for the full stream, the kept
// blocks' tokens for the sparse one, the selection held fixed) the chain rule gives, per
// row t and key i, with p the attention weights and delta_t = sum_d do_t,d o_t,d:
//     dv_i += p_ti do_t,   ds_ti = p_ti (do_t . v_i - delta_t),
//     dq_t += scale sum_i ds_ti k_i,   dk_i += scale ds_ti q_t.
// p is recomputed from the forward's log-sum-exp: p_ti = exp(scale q_t . k_i - lse_t).
//
// The dense stream in bf16 runs on the matrix cores (bwd_mfma.hip); the kernels here
// (vector ALU, float32 arithmetic; every key or query row is read with 16-byte coalesced
// loads, a row of D elements being D/E lanes wide) serve the sparse stream, fp32, and
// shapes the matrix-core kernels do not take:
//   delta:  delta_t from the forward output o and do;
//   dq:     one wave per query row walks the row's 64-key chunks (as the forward does)
//           and accumulates scale sum_i ds_ti k_i;
//   dk/dv:  one workgroup per 64-key chunk of a key/value head, a wave per 16 keys held
//           in registers, walks every query row that attends the chunk (all query heads
//           of the group): for the full stream the rows t >= the chunk's first key, for
//           the sparse stream the rows of the key's own block plus the rows that kept it,
//           taken from an inverted index (block -> rows) built by three small kernels.
//   align:  SmoothL1 terms and their gradients, a two-stage deterministic sum.
#include <cmath>

#include "launch.hpp"

namespace ssa {

namespace {

constexpr int kKeysPerWave = 16;

// Walk the valid entries of one idx row: blocks below b_t, each greater than the one
// used before it (the forward's rule for malformed rows).
template <typename F>
__device__ __forceinline__ void for_kept(const int32_t* __restrict__ ir, int topk, int bt, F&& fn) {
  int prev = -1;
  for (int e = 0; e < topk; ++e) {
    const int j = ir[e];
    if (j > prev && j < bt) {
      prev = j;
      fn(j);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------- delta
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                                        float* __restrict__ delta, int64_t ntok) {
  constexpr int E = Elem<T>::kPer16B, LPR = D / E, RPW = kWave / LPR;
  const int lane = threadIdx.x & 63;
  const int64_t tok = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / LPR;
  const int c = lane % LPR;
  float acc = 0.f;
  if (tok < ntok) {
    float a[E], b[E];
    Elem<T>::unpack(load16(o + tok * D + c * E), a);
    Elem<T>::unpack(load16(dout + tok * D + c * E), b);
#pragma unroll
    for (int e = 0; e < E; ++e) acc = fmaf(a[e], b[e], acc);
  }
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off);
  if (tok < ntok && c == 0) delta[tok] = acc;
}

// ---------------------------------------------------------------- dq
// One wave per query row.  Chunks of the row: sparse -- the valid kept blocks (listed
// first into LDS), then the own block's chunks up to t; full -- chunks 0 .. t/64.
template <typename T, int D, bool SPARSE>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                     const T* __restrict__ v, const T* __restrict__ dout,
                                                     const float* __restrict__ lse, const float* __restrict__ delta,
                                                     const int32_t* __restrict__ idx, int topk, float* __restrict__ dq,
                                                     int L, int G, int s, float scale, float sl2) {
  constexpr int E = Elem<T>::kPer16B, LPR = D / E, RPW = kWave / LPR, NI = 64 / RPW;
  extern __shared__ int kept_lds[];  // [4][topk]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;  // flat (b, h, t)
  const int64_t bh = row / L;
  const int t = (int)(row - bh * L);
  const int64_t kvbh = bh / G;
  const T* kh = k + kvbh * (int64_t)L * D;
  const T* vh = v + kvbh * (int64_t)L * D;
  const int col = (lane % LPR) * E, krow = lane / LPR;
  const int bt = t / s, cpb = s / 64;
  int* kept = kept_lds + wv * topk;
  int m = 0;
  if (SPARSE) {
    if (lane == 0) for_kept(idx + row * topk, topk, bt, [&](int j) { kept[m++] = j; });
    m = __shfl(m, 0);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
  const int own = (t - bt * s) / 64 + 1;
  const int nch = SPARSE ? m * cpb + own : t / 64 + 1;
  float qv[E], dov[E], acc[E];
  Elem<T>::unpack(load16(q + row * D + col), qv);
  Elem<T>::unpack(load16(dout + row * D + col), dov);
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  const float lse2 = lse[row] * kLog2e, dl = delta[row];
  for (int ch = 0; ch < nch; ++ch) {
    int key0;
    if (SPARSE) {
      const int slot = ch / cpb, sub = ch - slot * cpb;
      key0 = (slot < m ? kept[slot] : bt) * s + sub * 64;
    } else {
      key0 = ch * 64;
    }
    u32x4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = load16(kh + (int64_t)(key0 + i * RPW + krow) * D + col);
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = load16(vh + (int64_t)(key0 + i * RPW + krow) * D + col);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kx[E], vx[E];
      Elem<T>::unpack(kr[i], kx);
      Elem<T>::unpack(vr[i], vx);
      float sdot = 0.f, pdot = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        sdot = fmaf(qv[e], kx[e], sdot);
        pdot = fmaf(dov[e], vx[e], pdot);
      }
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) {
        sdot += __shfl_xor(sdot, off);
        pdot += __shfl_xor(pdot, off);
      }
      const bool live = key0 + i * RPW + krow <= t;
      const float p = live ? fast_exp2(fmaf(sdot, sl2, -lse2)) : 0.f;
      const float ds = p * (pdot - dl);
#pragma unroll
      for (int e = 0; e < E; ++e) acc[e] = fmaf(ds, kx[e], acc[e]);
    }
  }
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += __shfl_xor(acc[e], off);
  if (lane < LPR) {
    float* dst = dq + row * D + col;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] += scale * acc[e];
  }
}

// ---------------------------------------------------------------- sparse inverted index
// For each (b, query head) and block j, the rows t that kept j (valid entries only).
// The counters are cleared by a kernel (not a memset), so the sequence can be captured
// into a graph.
__global__ __launch_bounds__(256) void bwd_zero_kernel(int* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void bwd_index_count_kernel(const int32_t* __restrict__ idx, int topk,
                                                              int* __restrict__ cnt, int64_t rows, int L, int s,
                                                              int n) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int64_t bh = row / L;
  const int t = (int)(row - bh * L);
  int* c = cnt + bh * n;
  for_kept(idx + row * topk, topk, t / s, [&](int j) { atomicAdd(&c[j], 1); });
}

// The same count and fill with the counting done in LDS first: a workgroup takes 1024
// rows of one (b, h), counts its entries per block in LDS and adds each nonzero count to
// the global counter once (fill: reserves its range with one global atomic per block,
// then places its rows with LDS cursors).  For n <= kIndexLdsBlocks.
constexpr int kIndexLdsBlocks = 4096;
constexpr int kIndexRows = 1024;

__global__ __launch_bounds__(256) void bwd_index_count_lds_kernel(const int32_t* __restrict__ idx, int topk,
                                                                  int* __restrict__ cnt, int L, int s, int n) {
  __shared__ int lc[kIndexLdsBlocks];
  const int tiles = (L + kIndexRows - 1) / kIndexRows;
  const int64_t bh = blockIdx.x / tiles;
  const int t0 = (int)(blockIdx.x - bh * tiles) * kIndexRows;
  for (int j = threadIdx.x; j < n; j += 256) lc[j] = 0;
  __syncthreads();
  for (int t = t0 + threadIdx.x; t < min(L, t0 + kIndexRows); t += 256)
    for_kept(idx + (bh * L + t) * topk, topk, t / s, [&](int j) { atomicAdd(&lc[j], 1); });
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += 256)
    if (lc[j]) atomicAdd(&cnt[bh * n + j], lc[j]);
}

__global__ __launch_bounds__(256) void bwd_index_fill_lds_kernel(const int32_t* __restrict__ idx, int topk,
                                                                 int* __restrict__ cur, int* __restrict__ list, int L,
                                                                 int s, int n) {
  __shared__ int lc[kIndexLdsBlocks];
  const int tiles = (L + kIndexRows - 1) / kIndexRows;
  const int64_t bh = blockIdx.x / tiles;
  const int t0 = (int)(blockIdx.x - bh * tiles) * kIndexRows;
  const int t1 = min(L, t0 + kIndexRows);
  int* li = list + bh * (int64_t)L * topk;
  for (int j = threadIdx.x; j < n; j += 256) lc[j] = 0;
  __syncthreads();
  for (int t = t0 + threadIdx.x; t < t1; t += 256)
    for_kept(idx + (bh * L + t) * topk, topk, t / s, [&](int j) { atomicAdd(&lc[j], 1); });
  __syncthreads();
  for (int j = threadIdx.x; j < n; j += 256)
    if (lc[j]) lc[j] = atomicAdd(&cur[bh * n + j], lc[j]);  // this workgroup's first slot of block j
  __syncthreads();
  for (int t = t0 + threadIdx.x; t < t1; t += 256)
    for_kept(idx + (bh * L + t) * topk, topk, t / s, [&](int j) { li[atomicAdd(&lc[j], 1)] = t; });
}

// Exclusive prefix sum of cnt over the n blocks of one (b, h); cnt becomes the fill
// cursor.  One workgroup per (b, h).
__global__ __launch_bounds__(256) void bwd_index_scan_kernel(int* __restrict__ cnt, int* __restrict__ off, int n) {
  __shared__ int wsum[4];
  const int64_t bh = blockIdx.x;
  int* c = cnt + bh * n;
  int* o = off + bh * (int64_t)(n + 1);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int seg = (n + 255) / 256;
  const int j0 = min(n, tid * seg), j1 = min(n, j0 + seg);
  int local = 0;
  for (int j = j0; j < j1; ++j) local += c[j];
  int incl = local;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  if (lane == kWave - 1) wsum[wv] = incl;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < wv; ++i) base += wsum[i];
  int run = base + incl - local;
  for (int j = j0; j < j1; ++j) {
    const int x = c[j];
    o[j] = run;
    c[j] = run;
    run += x;
  }
  if (tid == 255) o[n] = base + incl;
}

__global__ __launch_bounds__(256) void bwd_index_fill_kernel(const int32_t* __restrict__ idx, int topk,
                                                             int* __restrict__ cur, int* __restrict__ list,
                                                             int64_t rows, int L, int s, int n) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= rows) return;
  const int64_t bh = row / L;
  const int t = (int)(row - bh * L);
  int* c = cur + bh * n;
  int* li = list + bh * (int64_t)L * topk;  // per (b, h) region, offsets from the scan
  for_kept(idx + row * topk, topk, t / s, [&](int j) { li[atomicAdd(&c[j], 1)] = t; });
}

// ---------------------------------------------------------------- dk, dv
// One workgroup per 64-key chunk of a key/value head; wave w holds keys 16w .. 16w+15 of
// the chunk (K and V rows in registers: key row i*RPW + lane/LPR, columns of lane % LPR)
// and their dk, dv accumulators.  Every query row that attends the chunk is processed by
// all four waves: its q, do, lse and delta are broadcast loads.
template <typename T, int D, bool SPARSE>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                       const T* __restrict__ v, const T* __restrict__ dout,
                                                       const float* __restrict__ lse, const float* __restrict__ delta,
                                                       const int* __restrict__ off, const int* __restrict__ list,
                                                       int topk, float* __restrict__ dk, float* __restrict__ dv,
                                                       int L, int G, int s, float scale, float sl2) {
  constexpr int E = Elem<T>::kPer16B, LPR = D / E, RPW = kWave / LPR, NK = kKeysPerWave / RPW;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nck = L / 64;
  const int64_t kvbh = blockIdx.x / nck;
  const int c = (int)(blockIdx.x - kvbh * nck);
  const int col = (lane % LPR) * E, krow = lane / LPR;
  const int key_base = c * 64 + kKeysPerWave * wv + krow;  // key of load i: key_base + i*RPW
  const T* kh = k + kvbh * (int64_t)L * D;
  const T* vh = v + kvbh * (int64_t)L * D;
  float kx[NK][E], vx[NK][E], dka[NK][E], dva[NK][E];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    Elem<T>::unpack(load16(kh + (int64_t)(key_base + i * RPW) * D + col), kx[i]);
    Elem<T>::unpack(load16(vh + (int64_t)(key_base + i * RPW) * D + col), vx[i]);
#pragma unroll
    for (int e = 0; e < E; ++e) dka[i][e] = dva[i][e] = 0.f;
  }
  auto one_row = [&](int64_t qrow, int t) {
    float qv[E], dov[E];
    Elem<T>::unpack(load16(q + qrow * D + col), qv);
    Elem<T>::unpack(load16(dout + qrow * D + col), dov);
    const float lse2 = lse[qrow] * kLog2e, dl = delta[qrow];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
      float sdot = 0.f, pdot = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        sdot = fmaf(qv[e], kx[i][e], sdot);
        pdot = fmaf(dov[e], vx[i][e], pdot);
      }
#pragma unroll
      for (int o2 = 1; o2 < LPR; o2 <<= 1) {
        sdot += __shfl_xor(sdot, o2);
        pdot += __shfl_xor(pdot, o2);
      }
      const float p = key_base + i * RPW <= t ? fast_exp2(fmaf(sdot, sl2, -lse2)) : 0.f;
      const float ds = p * (pdot - dl);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        dva[i][e] = fmaf(p, dov[e], dva[i][e]);
        dka[i][e] = fmaf(ds, qv[e], dka[i][e]);
      }
    }
  };
  const int c0 = c * 64;
  for (int gq = 0; gq < G; ++gq) {
    const int64_t bh = kvbh * G + gq;  // query heads of this key/value head
    if (SPARSE) {
      // rows of the keys' own block (causal), then the rows that kept the block
      const int j = c0 / s;
      const int r1 = min(L, j * s + s);
      for (int t = c0; t < r1; ++t) one_row(bh * L + t, t);
      const int* o = off + bh * (int64_t)(L / s + 1);
      const int* li = list + bh * (int64_t)L * topk;
      for (int e = o[j]; e < o[j + 1]; ++e) {
        const int t = li[e];
        one_row(bh * L + t, t);
      }
    } else {
      for (int t = c0; t < L; ++t) one_row(bh * L + t, t);
    }
  }
  float* dkh = dk + kvbh * (int64_t)L * D;
  float* dvh = dv + kvbh * (int64_t)L * D;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    float* pk = dkh + (int64_t)(key_base + i * RPW) * D + col;
    float* pv = dvh + (int64_t)(key_base + i * RPW) * D + col;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      pk[e] += scale * dka[i][e];
      pv[e] += dva[i][e];
    }
  }
}

// ---------------------------------------------------------------- alignment loss
// SmoothL1(x) = 0.5 x^2 / beta for |x| < beta, |x| - beta / 2 otherwise; its derivative
// is x / beta clipped to [-1, 1].  Stage 1: per-workgroup partial sums of SmoothL1 and the
// gradients; stage 2: one workgroup sums the partials in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void align_loss_kernel(const T* __restrict__ of, const T* __restrict__ os,
                                                         float* __restrict__ gf, float* __restrict__ gs,
                                                         float* __restrict__ partial, int64_t nvec, float beta,
                                                         float gscale) {
  constexpr int E = Elem<T>::kPer16B;
  __shared__ float red[256];
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  float sum = 0.f;
  if (i < nvec) {
    float a[E], b[E], g[E];
    Elem<T>::unpack(load16(of + i * E), a);
    Elem<T>::unpack(load16(os + i * E), b);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float x = a[e] - b[e], ax = fabsf(x);
      sum += ax < beta ? 0.5f * x * x / beta : ax - 0.5f * beta;
      g[e] = fminf(fmaxf(x / beta, -1.f), 1.f) * gscale;
    }
    if (gf)
#pragma unroll
      for (int e = 0; e < E; ++e) gf[i * E + e] = g[e];
    if (gs)
#pragma unroll
      for (int e = 0; e < E; ++e) gs[i * E + e] = -g[e];
  }
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void align_loss_sum_kernel(const float* __restrict__ partial, int64_t np,
                                                             float* __restrict__ loss, float lscale) {
  __shared__ double red[256];
  double sum = 0.0;
  for (int64_t i = threadIdx.x; i < np; i += 256) sum += partial[i];
  red[threadIdx.x] = sum;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = (float)(red[0] * lscale);
}

// ---------------------------------------------------------------- launchers
namespace {

template <typename F>
hipError_t dispatch_td(const Dims& d, F&& f) {
  if (d.dtype == 1) return d.D == 128 ? f(uint16_t{}, std::integral_constant<int, 128>{})
                                      : f(uint16_t{}, std::integral_constant<int, 64>{});
  return d.D == 128 ? f(float{}, std::integral_constant<int, 128>{}) : f(float{}, std::integral_constant<int, 64>{});
}

template <typename T, int D>
hipError_t run_delta(const Dims& d, const void* o, const void* dout, float* delta, hipStream_t st) {
  constexpr int RPW = kWave / (D / Elem<T>::kPer16B);
  const int64_t ntok = d.tokens();
  const int64_t grid = (ntok + 4 * RPW - 1) / (4 * RPW);
  hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, st, static_cast<const T*>(o),
                     static_cast<const T*>(dout), delta, ntok);
  return hipGetLastError();
}

template <typename T, int D, bool SPARSE>
hipError_t run_attn_bwd(const Dims& d, const void* q, const void* k, const void* v, const void* dout, const float* lse,
                        const float* delta, const int32_t* idx, int topk, const int* off, const int* list, float scale,
                        float* dq, float* dk, float* dv, hipStream_t st) {
  const float sl2 = scale * kLog2e;
  const int64_t rows = d.tokens();
  const size_t lds = SPARSE ? 4 * (size_t)topk * sizeof(int) : 0;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, SPARSE>), dim3((unsigned)(rows / 4)), dim3(256), lds, st,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<const T*>(dout), lse, delta, idx, topk, dq, d.L, d.G(), d.S, scale, sl2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t chunks = (int64_t)d.B * d.Hkv * (d.L / 64);
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, SPARSE>), dim3((unsigned)chunks), dim3(256), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<const T*>(dout), lse, delta, off, list, topk, dk, dv, d.L, d.G(), d.S, scale, sl2);
  return hipGetLastError();
}

}  // namespace

LaunchResult launch_attn_bwd(const Dims& d, bool sparse, bool mfma, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* dout, const int32_t* idx, int topk,
                             float scale, float* dq, float* dk, float* dv, hipStream_t st) {
  LaunchResult r;
  const int64_t rows = d.tokens();
  const int n = d.n();
  // workspace: delta [B*H*L]; sparse adds the inverted index: counts/cursors [B*H*n],
  // offsets [B*H*(n+1)] and row lists [B*H*L*topk]
  size_t bytes = (size_t)rows * sizeof(float);
  size_t o_cnt = 0, o_off = 0, o_list = 0;
  if (sparse) {
    o_cnt = bytes;
    bytes += (size_t)d.bh() * n * sizeof(int);
    o_off = bytes;
    bytes += (size_t)d.bh() * (n + 1) * sizeof(int);
    o_list = bytes;
    bytes += (size_t)rows * topk * sizeof(int);
  }
  void* ws = nullptr;
  r.err = workspace_alloc(bytes, &ws, st);
  if (r.err != hipSuccess) return r;
  char* base = static_cast<char*>(ws);
  float* delta = reinterpret_cast<float*>(base);
  int* cnt = reinterpret_cast<int*>(base + o_cnt);
  int* off = reinterpret_cast<int*>(base + o_off);
  int* list = reinterpret_cast<int*>(base + o_list);
  r.err = dispatch_td(d, [&](auto t, auto dd) {
    using T = decltype(t);
    constexpr int D = decltype(dd)::value;
    hipError_t e = run_delta<T, D>(d, o, dout, delta, st);
    if (e != hipSuccess || !sparse) {
      if (e != hipSuccess) return e;
      if (mfma && full_bwd_mfma_supported(d))
        return launch_full_bwd_mfma(d, nullptr, 0, nullptr, nullptr, q, k, v, dout, lse, delta, scale, dq, dk, dv,
                                    st);
      return run_attn_bwd<T, D, false>(d, q, k, v, dout, lse, delta, nullptr, 1, nullptr, nullptr, scale, dq, dk, dv,
                                       st);
    }
    const int64_t ncnt = d.bh() * n;
    hipLaunchKernelGGL(bwd_zero_kernel, dim3((unsigned)((ncnt + 255) / 256)), dim3(256), 0, st, cnt, ncnt);
    const unsigned g = (unsigned)((rows + 255) / 256);
    const unsigned gl = (unsigned)(d.bh() * ((d.L + kIndexRows - 1) / kIndexRows));
    if (n <= kIndexLdsBlocks)
      hipLaunchKernelGGL(bwd_index_count_lds_kernel, dim3(gl), dim3(256), 0, st, idx, topk, cnt, d.L, d.S, n);
    else
      hipLaunchKernelGGL(bwd_index_count_kernel, dim3(g), dim3(256), 0, st, idx, topk, cnt, rows, d.L, d.S, n);
    hipLaunchKernelGGL(bwd_index_scan_kernel, dim3((unsigned)d.bh()), dim3(256), 0, st, cnt, off, n);
    if (n <= kIndexLdsBlocks)
      hipLaunchKernelGGL(bwd_index_fill_lds_kernel, dim3(gl), dim3(256), 0, st, idx, topk, cnt, list, d.L, d.S, n);
    else
      hipLaunchKernelGGL(bwd_index_fill_kernel, dim3(g), dim3(256), 0, st, idx, topk, cnt, list, rows, d.L, d.S, n);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (mfma && sparse_bwd_mfma_supported(d, topk))
      return launch_full_bwd_mfma(d, idx, topk, off, list, q, k, v, dout, lse, delta, scale, dq, dk, dv, st);
    return run_attn_bwd<T, D, true>(d, q, k, v, dout, lse, delta, idx, topk, off, list, scale, dq, dk, dv, st);
  });
  const hipError_t fe = workspace_free(ws, st);
  if (r.err == hipSuccess) r.err = fe;
  return r;
}

LaunchResult launch_align_loss(const Dims& d, const void* of, const void* os, float alpha, float beta, float* loss,
                               float* gf, float* gs, hipStream_t st) {
  LaunchResult r;
  const int64_t nel = d.tokens() * d.D;
  const int E = d.dtype == 1 ? 8 : 4;
  const int64_t nvec = nel / E;
  const int64_t np = (nvec + 255) / 256;
  void* ws = nullptr;
  r.err = workspace_alloc((size_t)np * sizeof(float), &ws, st);
  if (r.err != hipSuccess) return r;
  float* partial = static_cast<float*>(ws);
  const float gscale = alpha / (float)nel;
  if (d.dtype == 1)
    hipLaunchKernelGGL(align_loss_kernel<uint16_t>, dim3((unsigned)np), dim3(256), 0, st,
                       static_cast<const uint16_t*>(of), static_cast<const uint16_t*>(os), gf, gs, partial, nvec,
                       beta, gscale);
  else
    hipLaunchKernelGGL(align_loss_kernel<float>, dim3((unsigned)np), dim3(256), 0, st, static_cast<const float*>(of),
                       static_cast<const float*>(os), gf, gs, partial, nvec, beta, gscale);
  r.err = hipGetLastError();
  if (r.err == hipSuccess) {
    hipLaunchKernelGGL(align_loss_sum_kernel, dim3(1), dim3(256), 0, st, partial, np, loss,
                       2.0f * alpha / (float)nel);
    r.err = hipGetLastError();
  }
  const hipError_t fe = workspace_free(ws, st);
  if (r.err == hipSuccess) r.err = fe;
  return r;
}

}  // namespace ssa
