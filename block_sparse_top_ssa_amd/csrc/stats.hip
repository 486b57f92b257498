// Attention-pattern measurements of either stream: the entropy of each row's attention
// weights and, per (b, h), the attention mass by block distance.  The pages report
// attention sparsity and entropy (App. H, Table A9) and distance histograms (App. K.2,
// p. 31, Fig. A4) to compare how the methods spread attention.
//
// With the stream's log-sum-exp known, the weights are exact in one pass:
//   p_ti = exp(scale q_t . k_i - lse_t),  entropy_t = lse_t - sum_i p_ti scale q_t . k_i,
//   hist[m] += p_ti for m = bucket(b_t - b_i), bucket(0) = 0, bucket(d) = 1 + floor(log2 d)
// (the last of the 16 buckets collects the rest).  Only the scores are needed, so the
// matrix-core kernel (bf16) of the full stream is the query-stationary backward kernel's
// first product alone (the sparse stream visits only its kept blocks: stats_gather.hip;
// the masked form below remains for tiles whose index does not fit in LDS):
// four waves x 32 rows, 64-key chunks of K streamed through two LDS stages.  Every row of a
// wave lies in one block, so a chunk's distance bucket is the same for the whole wave.
// Histogram partials go to one slot per (b, h, row group) and are summed in a fixed order.
#include <cmath>

#include "launch.hpp"
#include "mfma.hpp"

namespace ssa {

namespace {

constexpr int kBuckets = kDistBuckets;

// hist[m] += x for a wave-uniform bucket m (registers cannot be indexed at run time)
__device__ __forceinline__ void add_bucket(float (&h)[kBuckets], int m, float x) {
#pragma unroll
  for (int i = 0; i < kBuckets; ++i)
    if (i == m) h[i] += x;
}

template <typename F>
__device__ __forceinline__ void for_kept_blocks(const int32_t* __restrict__ ir, int topk, int bt, F&& fn) {
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

// ---------------------------------------------------------------- matrix cores (bf16)
template <int D, bool SPARSE>
__global__ __launch_bounds__(256) void attn_stats_mfma_kernel(const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              const float* __restrict__ lse,
                                                              const uint32_t* __restrict__ mask, int W,
                                                              float* __restrict__ entropy, float* __restrict__ part,
                                                              int L, int G, int BH, int s, float scale, float sl2) {
  constexpr int NC = D / 32, NF = 4 * NC;  // K fragments per 64-key chunk
  constexpr int PT = NF * 64 / 256;
  __shared__ u32x4 st[2][NF][64];
  __shared__ float hs[4][kBuckets];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int nqb = L / 128;
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);
  const int64_t bh = blockIdx.x % BH;
  const int64_t kvbh = bh / G;
  const int rw0 = qb * 128 + 32 * w;
  const int bt = rw0 / s;  // every row of this wave lies in block bt
  const uint16_t* qh = q + bh * (int64_t)L * D;
  const uint16_t* kh = k + kvbh * (int64_t)L * D;
  u32x4 qf[2][NC];
  float l2[2], ent[2] = {0.f, 0.f};
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t row = rw0 + 16 * nt + n;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) qf[nt][cc] = load_q_frag<D>(qh + row * D, cc);
    l2[nt] = lse[bh * L + row] * kLog2e;
  }
  float hacc[kBuckets];
#pragma unroll
  for (int m = 0; m < kBuckets; ++m) hacc[m] = 0.f;
  auto keeps = [&](int nt, int c) -> bool {
    if (!SPARSE) return true;
    const int j = c * 64 / s;
    return (mask[(bh * L + rw0 + 16 * nt + n) * (int64_t)W + j / 32] >> (j % 32)) & 1u;
  };
  const int items = (qb * 128 + 127) / 64 + 1;
  u32x4 pr[PT];
  auto load_item = [&](int c) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int p = tid + 256 * i, f = p >> 6, ll = p & 63, kt = f / NC, cc = f % NC;
      pr[i] = load16(kh + (int64_t)(c * 64 + 16 * kt + (ll & 15)) * D + 32 * cc + 8 * (ll >> 4));
    }
  };
  auto store_item = [&](int b) {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int p = tid + 256 * i;
      st[b][p >> 6][p & 63] = pr[i];
    }
  };
  load_item(0);
  store_item(0);
  __syncthreads();
  for (int c = 0; c < items; ++c) {
    const int b = c & 1;
    load_item(min(c + 1, items - 1));
    const int k0 = c * 64;
    if (k0 <= rw0 + 31) {
      float mass = 0.f;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const bool kept = keeps(nt, c);
        f32x4 sa[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) sa[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) sa[kt] = mfma_bf16(st[b][kt * NC + cc][lane], qf[nt][cc], sa[kt]);
        const int row = rw0 + 16 * nt + n;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool live = kept && k0 + 16 * kt + 4 * g + i <= row;
            const float p = live ? fast_exp2(fmaf(sa[kt][i], sl2, -l2[nt])) : 0.f;
            ent[nt] = fmaf(p, sa[kt][i] * scale, ent[nt]);
            mass += p;
          }
      }
      add_bucket(hacc, dist_bucket(bt - k0 / s), mass);
    }
    store_item(b ^ 1);
    __syncthreads();
  }
  if (entropy) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      float e = ent[nt];
      e += __shfl_xor(e, 16);
      e += __shfl_xor(e, 32);
      if (g == 0) {
        const int64_t row = bh * L + rw0 + 16 * nt + n;
        entropy[row] = lse[row] - e;
      }
    }
  }
  if (part) {
#pragma unroll
    for (int m = 0; m < kBuckets; ++m) {
      float x = hacc[m];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
      if (lane == 0) hs[w][m] = x;
    }
    __syncthreads();
    if (tid < kBuckets)
      part[(bh * nqb + qb) * kBuckets + tid] = hs[0][tid] + hs[1][tid] + hs[2][tid] + hs[3][tid];
  }
}

// ---------------------------------------------------------------- vector ALU (any dtype)
// One wave per row, the row's chunks as in the forward (sparse: the valid kept blocks,
// then the own block's chunks up to t); histogram partials per workgroup (4 rows).
template <typename T, int D, bool SPARSE>
__global__ __launch_bounds__(256) void attn_stats_generic_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                 const float* __restrict__ lse,
                                                                 const int32_t* __restrict__ idx, int topk,
                                                                 float* __restrict__ entropy,
                                                                 float* __restrict__ part, int L, int G, int s,
                                                                 float scale, float sl2) {
  constexpr int E = Elem<T>::kPer16B, LPR = D / E, RPW = kWave / LPR, NI = 64 / RPW;
  extern __shared__ int kept_stats[];  // [4][topk]
  __shared__ float hs[4][kBuckets];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  const int64_t bh = row / L;
  const int t = (int)(row - bh * L);
  const T* kh = k + (bh / G) * (int64_t)L * D;
  const int col = (lane % LPR) * E, krow = lane / LPR;
  const int bt = t / s, cpb = s / 64;
  int* kept = kept_stats + wv * topk;
  int m = 0;
  if (SPARSE) {
    if (lane == 0) for_kept_blocks(idx + row * topk, topk, bt, [&](int j) { kept[m++] = j; });
    m = __shfl(m, 0);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
  const int nch = SPARSE ? m * cpb + (t - bt * s) / 64 + 1 : t / 64 + 1;
  float qv[E];
  Elem<T>::unpack(load16(q + row * D + col), qv);
  const float lse2 = lse[row] * kLog2e;
  float ent = 0.f, hacc[kBuckets];
#pragma unroll
  for (int i = 0; i < kBuckets; ++i) hacc[i] = 0.f;
  for (int ch = 0; ch < nch; ++ch) {
    int key0;
    if (SPARSE) {
      const int slot = ch / cpb, sub = ch - slot * cpb;
      key0 = (slot < m ? kept[slot] : bt) * s + sub * 64;
    } else {
      key0 = ch * 64;
    }
    float mass = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kx[E];
      Elem<T>::unpack(load16(kh + (int64_t)(key0 + i * RPW + krow) * D + col), kx);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) d = fmaf(qv[e], kx[e], d);
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) d += __shfl_xor(d, off);
      const float p = key0 + i * RPW + krow <= t ? fast_exp2(fmaf(d, sl2, -lse2)) : 0.f;
      ent = fmaf(p, d * scale, ent);
      mass += p;
    }
    add_bucket(hacc, dist_bucket(bt - key0 / s), mass);
  }
  // each row group's lanes hold the same values: sum over the row groups only
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
    ent += __shfl_xor(ent, off);
#pragma unroll
    for (int i = 0; i < kBuckets; ++i) hacc[i] += __shfl_xor(hacc[i], off);
  }
  if (entropy && lane == 0) entropy[row] = lse[row] - ent;
  if (part) {
    if (lane < kBuckets) {
      float x = 0.f;
#pragma unroll
      for (int i = 0; i < kBuckets; ++i)
        if (i == lane) x = hacc[i];
      hs[wv][lane] = x;
    }
    __syncthreads();
    if (threadIdx.x < kBuckets)
      part[(int64_t)blockIdx.x * kBuckets + threadIdx.x] =
          hs[0][threadIdx.x] + hs[1][threadIdx.x] + hs[2][threadIdx.x] + hs[3][threadIdx.x];
  }
}

// hist[bh][m] = sum over the P partials of (b, h), in order.
__global__ __launch_bounds__(64) void attn_stats_sum_kernel(const float* __restrict__ part, float* __restrict__ hist,
                                                            int P) {
  const int64_t bh = blockIdx.x;
  const int m = threadIdx.x;
  if (m >= kBuckets) return;
  double x = 0.0;
  for (int p = 0; p < P; ++p) x += part[(bh * P + p) * kBuckets + m];
  hist[bh * kBuckets + m] = (float)x;
}

hipError_t launch_hist_sum(const float* part, float* hist, int64_t bh, int P, hipStream_t st) {
  hipLaunchKernelGGL(attn_stats_sum_kernel, dim3((unsigned)bh), dim3(64), 0, st, part, hist, P);
  return hipGetLastError();
}

// The full forward then the measurement pass, for the shapes and dtypes the fused
// matrix-core sweep does not take (a transient lse when the caller wants none).
LaunchResult launch_full_stats_unfused(const Dims& d, const void* q, const void* k, const void* v, float scale,
                                       void* o, float* lse, float* entropy, float* hist, hipStream_t st) {
  LaunchResult r;
  void* ws = nullptr;
  float* l = lse;
  if (!l) {
    r.err = workspace_alloc((size_t)d.tokens() * sizeof(float), &ws, st);
    if (r.err != hipSuccess) return r;
    l = static_cast<float*>(ws);
  }
  r = launch_full_generic(d, q, k, v, scale, o, l, st);
  if (r.err == hipSuccess && !r.unsupported)
    r = launch_attn_stats(d, false, q, k, l, nullptr, 1, scale, entropy, hist, st);
  if (ws) {
    const hipError_t ef = vfrag_release(ws, st);
    if (r.err == hipSuccess) r.err = ef;
  }
  return r;
}

// The sparse forward then the measurement pass over its lse, for the dtypes and shapes
// the fused matrix-core kernel does not take (a transient lse when the caller wants none).
LaunchResult launch_sparse_stats_unfused(const Dims& d, bool mfma, const void* q, const void* k, const void* v,
                                         const int32_t* idx, int topk, float scale, void* o, float* lse,
                                         float* entropy, float* hist, hipStream_t st) {
  LaunchResult r;
  void* ws = nullptr;
  float* l = lse;
  if (!l) {
    r.err = workspace_alloc((size_t)d.tokens() * sizeof(float), &ws, st);
    if (r.err != hipSuccess) return r;
    l = static_cast<float*>(ws);
  }
  r = mfma && sparse_mfma_supported(d, topk) ? launch_sparse_mfma(d, q, k, v, idx, topk, scale, o, l, st)
                                             : launch_sparse_generic(d, q, k, v, idx, topk, scale, o, l, st);
  if (r.err == hipSuccess && !r.unsupported) r = launch_attn_stats(d, mfma, q, k, l, idx, topk, scale, entropy, hist, st);
  if (ws) {
    const hipError_t ef = vfrag_release(ws, st);
    if (r.err == hipSuccess) r.err = ef;
  }
  return r;
}

// ---------------------------------------------------------------- launcher
LaunchResult launch_attn_stats(const Dims& d, bool mfma, const void* q, const void* k, const float* lse,
                               const int32_t* idx, int topk, float scale, float* entropy, float* hist,
                               hipStream_t st) {
  LaunchResult r;
  // the sparse stream over gathered rows (stats_gather.hip) where its tile index fits in LDS
  const int gT = mfma && idx ? stats_gather_tile(d, topk) : 0;
  const bool use_mfma = gT == 0 && mfma && d.dtype == 1 && d.L % 128 == 0 && (!idx || d.n() <= 4096);
  const int P = gT ? (d.L + gT - 1) / gT : use_mfma ? d.L / 128 : d.L / 4;  // histogram partials per (b, h)
  const int W = (d.n() + 31) / 32;
  const size_t pbytes = hist ? (size_t)d.bh() * P * kBuckets * sizeof(float) : 0;
  const size_t mbytes = use_mfma && idx ? (size_t)d.tokens() * W * sizeof(uint32_t) : 0;
  void* ws = nullptr;
  if (pbytes + mbytes) {
    r.err = workspace_alloc(pbytes + mbytes, &ws, st);
    if (r.err != hipSuccess) return r;
  }
  float* part = hist ? static_cast<float*>(ws) : nullptr;
  uint32_t* mask = mbytes ? reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + pbytes) : nullptr;
  const float sl2 = scale * kLog2e;
  auto go = [&]() -> hipError_t {
    if (gT) return launch_stats_gather(d, q, k, lse, idx, topk, scale, entropy, part, st);
    if (use_mfma) {
      if (idx) {
        hipError_t e = build_block_mask(d, idx, topk, mask, st);
        if (e != hipSuccess) return e;
      }
      const unsigned grid = (unsigned)(d.bh() * (d.L / 128));
      const uint16_t* qq = static_cast<const uint16_t*>(q);
      const uint16_t* kk = static_cast<const uint16_t*>(k);
      if (d.D == 128) {
        if (idx)
          hipLaunchKernelGGL((attn_stats_mfma_kernel<128, true>), dim3(grid), dim3(256), 0, st, qq, kk, lse, mask, W,
                             entropy, part, d.L, d.G(), (int)d.bh(), d.S, scale, sl2);
        else
          hipLaunchKernelGGL((attn_stats_mfma_kernel<128, false>), dim3(grid), dim3(256), 0, st, qq, kk, lse, mask, W,
                             entropy, part, d.L, d.G(), (int)d.bh(), d.S, scale, sl2);
      } else {
        if (idx)
          hipLaunchKernelGGL((attn_stats_mfma_kernel<64, true>), dim3(grid), dim3(256), 0, st, qq, kk, lse, mask, W,
                             entropy, part, d.L, d.G(), (int)d.bh(), d.S, scale, sl2);
        else
          hipLaunchKernelGGL((attn_stats_mfma_kernel<64, false>), dim3(grid), dim3(256), 0, st, qq, kk, lse, mask, W,
                             entropy, part, d.L, d.G(), (int)d.bh(), d.S, scale, sl2);
      }
      return hipGetLastError();
    }
    const unsigned grid = (unsigned)(d.tokens() / 4);
    const size_t lds = idx ? 4 * (size_t)topk * sizeof(int) : 0;
    auto launch = [&](auto t, auto dd, auto sp) {
      using T = decltype(t);
      constexpr int D = decltype(dd)::value;
      constexpr bool SP = decltype(sp)::value;
      hipLaunchKernelGGL((attn_stats_generic_kernel<T, D, SP>), dim3(grid), dim3(256), lds, st,
                         static_cast<const T*>(q), static_cast<const T*>(k), lse, idx, topk, entropy, part, d.L,
                         d.G(), d.S, scale, sl2);
    };
    using BT = std::integral_constant<bool, true>;
    using BF = std::integral_constant<bool, false>;
    using D128 = std::integral_constant<int, 128>;
    using D64 = std::integral_constant<int, 64>;
    if (d.dtype == 1) {
      if (d.D == 128) idx ? launch(uint16_t{}, D128{}, BT{}) : launch(uint16_t{}, D128{}, BF{});
      else idx ? launch(uint16_t{}, D64{}, BT{}) : launch(uint16_t{}, D64{}, BF{});
    } else {
      if (d.D == 128) idx ? launch(float{}, D128{}, BT{}) : launch(float{}, D128{}, BF{});
      else idx ? launch(float{}, D64{}, BT{}) : launch(float{}, D64{}, BF{});
    }
    return hipGetLastError();
  };
  r.err = go();
  if (r.err == hipSuccess && hist) {
    hipLaunchKernelGGL(attn_stats_sum_kernel, dim3((unsigned)d.bh()), dim3(64), 0, st, part, hist, P);
    r.err = hipGetLastError();
  }
  if (ws) {
    const hipError_t fe = workspace_free(ws, st);
    if (r.err == hipSuccess) r.err = fe;
  }
  return r;
}

}  // namespace ssa
