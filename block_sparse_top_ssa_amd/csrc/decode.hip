// Decoding with a key/value cache: one new query per sequence per step.
//
// The paper's sparse kernel has no key/value cache, which makes its decoding slow (App. E,
// p. 22).  These kernels are the cached form of the per-layer forward of sec. 3 (pp. 3-4)
// for the query at position t = pos[b]: the same block selection over the complete
// blocks before t's own, the same sparse attention over the kept blocks, and dense
// attention over 0..t, reading a cache of capacity L instead of the whole sequence.
//
// Everything here is bound by memory traffic and latency, not arithmetic: one query row
// per (b, h) makes every product a matrix-vector product, so the kernels use 16-byte
// coalesced loads of whole key/value rows, float32 vector arithmetic and short
// xor-shuffle reductions, and spread a row's keys over many workgroups (split keys,
// combined afterwards through per-split log-sum-exps) so that a small batch still
// fills the chip.
#include <cmath>

#include <mutex>

#include "launch.hpp"
#include "mfma.hpp"
#include "pool.hpp"

namespace ssa {

namespace {

constexpr int kDecodeMaxBlocks = 8192;  // candidates held in LDS by the selection kernel
constexpr int kChunk = 64;              // keys per wave step of the attention kernel
constexpr int kTopkThreads = 1024;      // selection workgroup: 16 waves share the scoring loads

// Position of the new token of sequence b, or -1 when it lies outside the cache.
__device__ __forceinline__ int cache_pos(const int32_t* pos, int b, int L) {
  const int p = pos[b];
  return (p >= 0 && p < L) ? p : -1;
}

// Number of 64-key chunks a row attends and the chunks per split, identical in the
// attention and combine kernels.  Sparse: the m = min(topk-1, b_t) kept blocks, then the
// chunks of the own block up to t.  Full: chunks 0 .. t/64.
template <bool SPARSE>
__device__ __forceinline__ int row_chunks(int p, int s, int topk) {
  if (SPARSE) {
    const int bt = p / s;
    const int m = min(topk - 1, bt);
    return m * (s / kChunk) + (p - bt * s) / kChunk + 1;
  }
  return p / kChunk + 1;
}

}  // namespace

// ---------------------------------------------------------------- append
// One wave per (b, key/value head): writes the new key and value at p = pos[b] and
// rewrites the pooled key of block p / s as the mean of the c = p % s + 1 tokens it holds
// (the new key read from k_new, the others from the cache), summed exactly as the block
// pooling kernel sums a block, so a block completed by appends holds the same bits as one
// pooled from the whole sequence.  A sequence whose pos is outside [0, L) is skipped.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_append_kernel(const int32_t* __restrict__ pos,
                                                            const T* __restrict__ k_new,
                                                            const T* __restrict__ v_new, T* __restrict__ kc,
                                                            T* __restrict__ vc, float* __restrict__ km, int B,
                                                            int Hkv, int L, int s, float inv_s) {
  constexpr int E = Elem<T>::kPer16B;
  constexpr int LPR = D / E;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // flat (b, kv head)
  if (w >= (int64_t)B * Hkv) return;
  const int p = cache_pos(pos, (int)(w / Hkv), L);
  if (p < 0) return;
  const T* kn = k_new + w * D;
  const T* vn = v_new + w * D;
  T* kh = kc + w * (int64_t)L * D;
  T* vh = vc + w * (int64_t)L * D;
  if (lane < LPR) {
    store16(kh + (int64_t)p * D + lane * E, load16(kn + lane * E));
    store16(vh + (int64_t)p * D + lane * E, load16(vn + lane * E));
  }
  const int bt = p / s, c = p - bt * s + 1;
  float acc[E];
  block_key_sum<T, D>(kh + (int64_t)bt * s * D, s, c, c - 1, kn, acc);
  if (lane < LPR) {
    float* dst = km + (w * (L / s) + bt) * D + lane * E;
    const float cf = (float)c;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(c == s ? acc[e + i] * inv_s : acc[e + i] / cf);
      store16(dst + e, o);
    }
  }
}

// ---------------------------------------------------------------- selection
// One workgroup of 16 waves per (b, query head).  Scores sigma_j = q . kbar_j of the
// complete blocks j < b_t in float32 (a kbar row is D/4 lanes wide, several rows per
// wave-wide load, eight loads in flight per lane, xor-shuffle sums), held in LDS as
// order-preserving 32-bit keys.  The m = min(topk-1,
// b_t) best by (score descending, j ascending) are found by a radix select, 8 bits per
// pass from the top: a 256-bin histogram of the keys that match the digits chosen so far,
// then the digit where the running count from the top reaches the wanted rank.  After
// four passes the m-th key T is known with r = the number of keys equal to T to keep;
// those are the r lowest indices among the keys equal to T.  A block-wide scan in index
// order then writes the kept blocks in ascending order, b_t after them, -1 after that.
template <typename T, int D>
__global__ __launch_bounds__(kTopkThreads) void decode_topk_kernel(const int32_t* __restrict__ pos, const T* __restrict__ q,
                                                          const float* __restrict__ km, int32_t* __restrict__ idx,
                                                          int H, int G, int L, int s, int topk) {
  __shared__ uint32_t keys[kDecodeMaxBlocks];
  __shared__ uint32_t hist[256];
  constexpr int NT = kTopkThreads, NW = NT / kWave;
  __shared__ uint32_t wsum[NW];
  __shared__ int sel[2];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t bh = blockIdx.x;
  const int p = cache_pos(pos, (int)(bh / H), L);
  int32_t* out = idx + bh * topk;
  if (p < 0) {
    for (int i = tid; i < topk; i += NT) out[i] = -1;
    return;
  }
  const int bt = p / s;
  const int m = min(topk - 1, bt);
  if (m == bt || m == 0) {  // every candidate is kept, or none (topk = 1)
    for (int i = tid; i < topk; i += NT) out[i] = i < m ? i : (i == m ? bt : -1);
    return;
  }
  // ---- scores (bt >= 1 here)
  constexpr int LK = D / 4, RK = kWave / LK;  // lanes per kbar row, rows per load
  const float* kmh = km + (bh / G) * (int64_t)(L / s) * D;
  float qv[4];
  {
    const T* qp = q + bh * D + (lane % LK) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[e] = Elem<T>::load1(qp + e);
  }
  const int nc = bt;
  constexpr int U = 8;  // loads in flight per lane
  for (int j0 = wv * RK * U; j0 < nc; j0 += NW * RK * U) {
    f32x4 x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * RK + lane / LK;
      x[u] = j < nc ? *reinterpret_cast<const f32x4*>(kmh + (int64_t)j * D + (lane % LK) * 4) : f32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d = qv[0] * x[u][0];
      d = fmaf(qv[1], x[u][1], d);
      d = fmaf(qv[2], x[u][2], d);
      d = fmaf(qv[3], x[u][3], d);
#pragma unroll
      for (int o = 1; o < LK; o <<= 1) d += __shfl_xor(d, o);
      const int j = j0 + u * RK + lane / LK;
      if (lane % LK == 0 && j < nc) keys[j] = orderable_f32(d);
    }
  }
  __syncthreads();
  // ---- radix select of the m-th largest key
  uint32_t prefix = 0;
  int rank = m;  // 1-based rank wanted among the keys that match `prefix`
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int j = tid; j < nc; j += NT) {
      const uint32_t u = keys[j];
      if (pass == 0 || (u >> (shift + 8)) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wv == 0) {
      // lane l holds digits 255-4l .. 252-4l, so lanes run from the top digit down
      uint32_t c4[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c4[i] = hist[255 - 4 * lane - i];
        tot += c4[i];
      }
      uint32_t incl = tot;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
      }
      const uint64_t hit = __ballot(incl >= (uint32_t)rank);
      if (lane == __ffsll((unsigned long long)hit) - 1) {
        uint32_t before = incl - tot;
        int digit = 255 - 4 * lane - 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (before + c4[i] >= (uint32_t)rank) {
            digit = 255 - 4 * lane - i;
            break;
          }
          before += c4[i];
        }
        sel[0] = digit;
        sel[1] = rank - (int)before;
      }
    }
    __syncthreads();
    prefix = (prefix << 8) | (uint32_t)sel[0];
    rank = sel[1];
  }
  const uint32_t kth = prefix;
  const int take_eq = rank;  // keys equal to kth that are kept (lowest indices first)
  // ---- write the kept blocks in index order: each thread owns a contiguous range
  const int C = (nc + NT - 1) / NT;
  const int jlo = min(tid * C, nc), jhi = min(jlo + C, nc);
  uint32_t gt = 0, eq = 0;
  for (int j = jlo; j < jhi; ++j) {
    const uint32_t u = keys[j];
    gt += u > kth;
    eq += u == kth;
  }
  // exclusive scan of (gt, eq) packed in 16-bit halves (each total <= 8192)
  const uint32_t mine = (gt << 16) | eq;
  uint32_t incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) wsum[wv] = incl;
  __syncthreads();
  uint32_t excl = incl - mine;
  for (int i = 0; i < wv; ++i) excl += wsum[i];
  const int gt_before = (int)(excl >> 16), eq_before = (int)(excl & 0xFFFFu);
  int o = gt_before + min(eq_before, take_eq);
  int e = eq_before;
  for (int j = jlo; j < jhi; ++j) {
    const uint32_t u = keys[j];
    if (u > kth) {
      out[o++] = j;
    } else if (u == kth) {
      if (e < take_eq) out[o++] = j;
      ++e;
    }
  }
  for (int i = m + tid; i < topk; i += NT) out[i] = i == m ? bt : -1;
}

// ---------------------------------------------------------------- attention (split keys)
// Grid (splits, B*H), four waves per workgroup.  Split x of a row takes its chunks
// [x*cps, (x+1)*cps); a wave takes every fourth of them.  Per 64-key chunk a wave loads
// all keys (and values) at once: a row of D elements is D/E lanes wide, so load i covers
// keys i*RPW .. i*RPW+RPW-1 of the chunk, 1 KB contiguous.  Each lane forms its part of
// q . k_i, an xor-shuffle over the row's lanes completes the dot product, and an online
// softmax in base 2 (running maximum, rescaled sum and o) folds the chunk in.  The four
// waves' (max, sum, o) are merged through LDS into the split's partial result
// part[(bh, x)] = {max, sum, o[0..D)} (o not normalised), combined later.
template <typename T, int D, bool SPARSE, bool WANT_O>
__global__ __launch_bounds__(256) void decode_attn_kernel(const int32_t* __restrict__ pos, const T* __restrict__ q,
                                                          const T* __restrict__ kc, const T* __restrict__ vc,
                                                          const int32_t* __restrict__ idx, float* __restrict__ part,
                                                          int H, int G, int L, int s, int topk, int cps, float sl2) {
  constexpr int E = Elem<T>::kPer16B;
  constexpr int LPR = D / E;        // lanes per key row
  constexpr int RPW = kWave / LPR;  // key rows per wave-wide load
  constexpr int NI = kChunk / RPW;  // loads per chunk
  __shared__ float red[4][D + 2];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int split = blockIdx.x, nsplit = gridDim.x;
  const int64_t bh = blockIdx.y;
  const int p = cache_pos(pos, (int)(bh / H), L);
  if (p < 0) return;
  const int nch = row_chunks<SPARSE>(p, s, topk);
  const int c0 = split * cps, c1 = min(nch, c0 + cps);
  if (c0 >= nch) return;
  const int bt = p / s, cpb = s / kChunk;
  const int m_sel = min(topk - 1, bt);
  const int32_t* ir = idx + bh * topk;
  const int64_t kvbh = bh / G;
  const T* kh = kc + kvbh * (int64_t)L * D;
  const T* vh = WANT_O ? vc + kvbh * (int64_t)L * D : nullptr;  // v is not read for lse only
  const int col = (lane % LPR) * E, krow = lane / LPR;
  float qv[E];
  Elem<T>::unpack(load16(q + bh * D + col), qv);
  float mrun = -INFINITY, lrun = 0.f, o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int ch = c0 + wv; ch < c1; ch += 4) {
    int key0;
    if (SPARSE) {
      const int slot = ch / cpb, sub = ch - slot * cpb;
      key0 = (slot < m_sel ? ir[slot] : bt) * s + sub * kChunk;
    } else {
      key0 = ch * kChunk;
    }
    const T* kp = kh + (int64_t)(key0 + krow) * D + col;
    const T* vp = WANT_O ? vh + (int64_t)(key0 + krow) * D + col : nullptr;
    u32x4 kr[NI], vr[WANT_O ? NI : 1];
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = load16(kp + (int64_t)i * RPW * D);
    if (WANT_O) {
#pragma unroll
      for (int i = 0; i < NI; ++i) vr[i] = load16(vp + (int64_t)i * RPW * D);
    }
    float sc[NI];
    float cmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float x[E];
      Elem<T>::unpack(kr[i], x);
      float d = qv[0] * x[0];
#pragma unroll
      for (int e = 1; e < E; ++e) d = fmaf(qv[e], x[e], d);
#pragma unroll
      for (int off = 1; off < LPR; off <<= 1) d += __shfl_xor(d, off);
      sc[i] = (key0 + i * RPW + krow <= p) ? d * sl2 : -INFINITY;
      cmax = fmaxf(cmax, sc[i]);
    }
#pragma unroll
    for (int off = LPR; off < kWave; off <<= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off));
    // cmax is finite: the chunk's first key is at or before p
    const float mnew = fmaxf(mrun, cmax);
    const float alpha = mrun == -INFINITY ? 0.f : fast_exp2(mrun - mnew);
    lrun *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= alpha;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const float pr = fast_exp2(sc[i] - mnew);
      lrun += pr;
      if (WANT_O) {
        float y[E];
        Elem<T>::unpack(vr[WANT_O ? i : 0], y);
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] = fmaf(pr, y[e], o[e]);
      }
    }
    mrun = mnew;
  }
  // sum over the key rows of the wave (each row group holds one share)
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
    lrun += __shfl_xor(lrun, off);
    if (WANT_O) {
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] += __shfl_xor(o[e], off);
    }
  }
  if (lane == 0) {
    red[wv][0] = mrun;
    red[wv][1] = lrun;
  }
  if (WANT_O && lane < LPR) {
#pragma unroll
    for (int e = 0; e < E; ++e) red[wv][2 + col + e] = o[e];
  }
  __syncthreads();
  float* pp = part + (bh * nsplit + split) * (int64_t)(D + 2);
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) M = fmaxf(M, red[w][0]);  // finite: wave 0 has a chunk
  float wt[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) wt[w] = red[w][0] == -INFINITY ? 0.f : fast_exp2(red[w][0] - M);
  const int t = threadIdx.x;
  if (t == 0) {
    pp[0] = M;
    pp[1] = wt[0] * red[0][1] + wt[1] * red[1][1] + wt[2] * red[2][1] + wt[3] * red[3][1];
  }
  if (WANT_O && t < D)
    pp[2 + t] = wt[0] * red[0][2 + t] + wt[1] * red[1][2 + t] + wt[2] * red[2][2 + t] + wt[3] * red[3][2 + t];
}


// ---------------------------------------------------------------- dense stream, grouped heads
// With G query heads per key/value head, the dense stream's G rows of one sequence read the
// same keys and values, so they are one small matrix product on the matrix cores: the
// group's heads are the N (column) dimension, S^T (64 keys x 16 heads) = K Q^T, an online
// softmax per column, O^T (D x 16 heads) += V^T P^T with V^T fragments formed from the
// cache rows on the fly (8x8 transposes of 16-bit values across 8 lanes, the kappa key
// order in which the S^T layout is the B operand).  Each key/value row is read once per
// group instead of once per query head.  Up to 16 heads per pass; columns past G hold no
// query.  Split partials as in decode_attn_kernel (same layout, merged by the same
// combine kernel).
template <int D, bool WANT_O>
__global__ __launch_bounds__(256) void decode_full_group_kernel(const int32_t* __restrict__ pos,
                                                                const uint16_t* __restrict__ q,
                                                                const uint16_t* __restrict__ kc,
                                                                const uint16_t* __restrict__ vc,
                                                                float* __restrict__ part, int H, int G, int L,
                                                                int cps, float sl2) {
  constexpr int NC = D / 32, NDT = D / 16;
  __shared__ float red[4][16][D + 2];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x, nsplit = gridDim.x;
  const int nhg = (G + 15) / 16;
  const int64_t kvbh = blockIdx.y / nhg;
  const int hg = (int)(blockIdx.y - kvbh * nhg);
  const int Hkv = H / G;
  const int b = (int)(kvbh / Hkv), kvh = (int)(kvbh - (int64_t)b * Hkv);
  const int p = cache_pos(pos, b, L);
  if (p < 0) return;
  const int nch = p / kChunk + 1;
  const int c0 = split * cps, c1 = min(nch, c0 + cps);
  if (c0 >= nch) return;
  const int hl = 16 * hg + n;  // this lane's head within the group (column n)
  const bool hv = hl < G;
  const int64_t bhq = (int64_t)b * H + kvh * G + (hv ? hl : 0);
  const uint16_t* kh = kc + kvbh * (int64_t)L * D;
  const uint16_t* vh = vc + kvbh * (int64_t)L * D;
  u32x4 qf[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) qf[cc] = hv ? load_q_frag<D>(q + bhq * D, cc) : u32x4{0, 0, 0, 0};
  float mrun = -INFINITY, lrun = 0.f;
  f32x4 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x4{0, 0, 0, 0};
  for (int ch = c0 + wv; ch < c1; ch += 4) {
    const int key0 = ch * kChunk;
    u32x4 kf[4][NC], vt[WANT_O ? NDT : 1][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) kf[kt][cc] = load_k_frag<D>(kh, key0 + 16 * kt, cc);
    if (WANT_O) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) vt[WANT_O ? dt : 0][c2] = load_v_raw<D>(vh, key0, dt, c2);
    }
    f32x4 sa[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sa[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) sa[kt] = mfma_bf16(kf[kt][cc], qf[cc], sa[kt]);
    }
    // element i of sa[kt]: key key0 + 16 kt + 4 g + i, head column n
    float sc[4][4], cmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[kt][i] = key0 + 16 * kt + 4 * g + i <= p ? sa[kt][i] * sl2 : -INFINITY;
        cmax = fmaxf(cmax, sc[kt][i]);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float mnew = fmaxf(mrun, cmax);  // finite: the chunk's first key is at or before p
    const float alpha = mrun == -INFINITY ? 0.f : fast_exp2(mrun - mnew);
    float pr[4][4], ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[kt][i] = fast_exp2(sc[kt][i] - mnew);
        ps += pr[kt][i];
      }
    lrun = lrun * alpha + ps;
    if (WANT_O) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) oacc[dt] = oacc[dt] * alpha;
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const u32x4 pb = pack_p(pr[2 * c2], pr[2 * c2 + 1]);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          oacc[dt] = mfma_bf16(transpose8x8_b16_dpp(vt[WANT_O ? dt : 0][c2]), pb, oacc[dt]);
      }
    }
    mrun = mnew;
  }
  lrun += __shfl_xor(lrun, 16);
  lrun += __shfl_xor(lrun, 32);
  if (g == 0) {
    red[wv][n][0] = mrun;
    red[wv][n][1] = lrun;
  }
  if (WANT_O) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wv][n][2 + 16 * dt + 4 * g + i] = oacc[dt][i];
  }
  __syncthreads();
  // merge the four waves per head; part[(query head, split)] = {max, sum, o}
  for (int e = threadIdx.x; e < 16 * (D + 2); e += 256) {
    const int hn = e / (D + 2), c = e - hn * (D + 2);
    if (16 * hg + hn >= G || (!WANT_O && c >= 2)) continue;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red[w][hn][0]);
    float x = 0.f;
    if (c == 0) {
      x = M;
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = red[w][hn][0];
        if (mw != -INFINITY) x += fast_exp2(mw - M) * red[w][hn][c];
      }
    }
    const int64_t bq = (int64_t)b * H + kvh * G + 16 * hg + hn;
    part[(bq * nsplit + split) * (int64_t)(D + 2) + c] = x;
  }
}

// ---------------------------------------------------------------- combine
// One workgroup per (b, h): merges the row's split partials, o = sum_x 2^(m_x - M) o_x /
// sum_x 2^(m_x - M) l_x, lse = ln 2 * (M + log2 l), with M the largest split maximum (the
// logits are in base 2).  A sequence whose pos is outside [0, L) gets NaN outputs.
template <typename T, int D, bool SPARSE, bool WANT_O>
__global__ __launch_bounds__(256) void decode_combine_kernel(const int32_t* __restrict__ pos,
                                                             const float* __restrict__ part, T* __restrict__ o,
                                                             float* __restrict__ lse, int H, int L, int s, int topk,
                                                             int cps, int nsplit) {
  __shared__ float red[256];
  __shared__ float acc[256 / D][D];
  const int t = threadIdx.x;
  const int64_t bh = blockIdx.x;
  const int p = cache_pos(pos, (int)(bh / H), L);
  if (p < 0) {
    if (WANT_O && t < D) Elem<T>::store1(o + bh * D + t, NAN);
    if (t == 0 && lse) lse[bh] = NAN;
    return;
  }
  const int ns = (row_chunks<SPARSE>(p, s, topk) + cps - 1) / cps;  // splits that wrote
  const float* pr = part + bh * nsplit * (int64_t)(D + 2);
  float mx = -INFINITY;
  for (int x = t; x < ns; x += 256) mx = fmaxf(mx, pr[(int64_t)x * (D + 2)]);
  red[t] = mx;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (t < h) red[t] = fmaxf(red[t], red[t + h]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();
  float l = 0.f;
  for (int x = t; x < ns; x += 256) {
    const float* px = pr + (int64_t)x * (D + 2);
    l += fast_exp2(px[0] - M) * px[1];
  }
  red[t] = l;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (t < h) red[t] += red[t + h];
    __syncthreads();
  }
  const float lsum = red[0];
  if (WANT_O) {
    constexpr int NG = 256 / D;  // split groups
    const int c = t % D, g = t / D;
    float a = 0.f;
    for (int x = g; x < ns; x += NG) {
      const float* px = pr + (int64_t)x * (D + 2);
      a = fmaf(fast_exp2(px[0] - M), px[2 + c], a);
    }
    acc[g][c] = a;
    __syncthreads();
    if (t < D) {
      float v = 0.f;
#pragma unroll
      for (int i = 0; i < NG; ++i) v += acc[i][t];
      Elem<T>::store1(o + bh * D + t, v / lsum);
    }
  }
  if (t == 0 && lse) lse[bh] = (M + log2f(lsum)) * kLn2;
}

// ---------------------------------------------------------------- launchers
namespace {

template <typename T, int D>
hipError_t run_append(const Dims& d, const int32_t* pos, const void* kn, const void* vn, void* kc, void* vc,
                      float* km, hipStream_t st) {
  const int64_t waves = (int64_t)d.B * d.Hkv;
  hipLaunchKernelGGL((decode_append_kernel<T, D>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, pos,
                     static_cast<const T*>(kn), static_cast<const T*>(vn), static_cast<T*>(kc), static_cast<T*>(vc),
                     km, d.B, d.Hkv, d.L, d.S, 1.0f / (float)d.S);
  return hipGetLastError();
}

// Splits of a row: sparse rows have at most topk * s / 64 chunks, full rows L / 64.
constexpr int kSparseCps = 4;  // one chunk per wave
constexpr int kFullCps = 16;   // four chunks per wave (fewer split results to merge)
constexpr int kGroupCps = 16;  // grouped heads (4 measured slower: more partials to merge)
int max_chunks(const Dims& d, bool sparse, int topk) { return sparse ? topk * (d.S / kChunk) : d.L / kChunk; }
int splits(const Dims& d, bool sparse, int topk) {
  const int cps = sparse ? kSparseCps : kFullCps;
  return (max_chunks(d, sparse, topk) + cps - 1) / cps;
}

template <typename T, int D, bool SPARSE, bool WANT_O>
hipError_t run_attn(const Dims& d, const int32_t* pos, const void* q, const void* kc, const void* vc,
                    const int32_t* idx, int topk, float scale, void* o, float* lse, float* part, hipStream_t st) {
  const int cps = SPARSE ? kSparseCps : kFullCps;
  const int ns = splits(d, SPARSE, topk);
  hipLaunchKernelGGL((decode_attn_kernel<T, D, SPARSE, WANT_O>), dim3((unsigned)ns, (unsigned)d.bh()), dim3(256), 0,
                     st, pos, static_cast<const T*>(q), static_cast<const T*>(kc), static_cast<const T*>(vc), idx,
                     part, d.H, d.G(), d.L, d.S, topk, cps, scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<T, D, SPARSE, WANT_O>), dim3((unsigned)d.bh()), dim3(256), 0, st, pos,
                     part, static_cast<T*>(o), lse, d.H, d.L, d.S, topk, cps, ns);
  return hipGetLastError();
}

template <int D, bool WANT_O>
hipError_t run_group(const Dims& d, const int32_t* pos, const void* q, const void* kc, const void* vc, float scale,
                     void* o, float* lse, float* part, hipStream_t st) {
  const int ns = (max_chunks(d, false, 1) + kGroupCps - 1) / kGroupCps;
  const int nhg = (d.G() + 15) / 16;
  hipLaunchKernelGGL((decode_full_group_kernel<D, WANT_O>), dim3((unsigned)ns, (unsigned)(d.kv().bh() * nhg)),
                     dim3(256), 0, st, pos, static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(kc),
                     static_cast<const uint16_t*>(vc), part, d.H, d.G(), d.L, kGroupCps, scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<uint16_t, D, false, WANT_O>), dim3((unsigned)d.bh()), dim3(256), 0, st,
                     pos, part, static_cast<uint16_t*>(o), lse, d.H, d.L, d.S, 1, kGroupCps, ns);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_topk(const Dims& d, const int32_t* pos, const void* q, const float* km, int topk, int32_t* idx,
                    hipStream_t st) {
  hipLaunchKernelGGL((decode_topk_kernel<T, D>), dim3((unsigned)d.bh()), dim3(kTopkThreads), 0, st, pos,
                     static_cast<const T*>(q), km, idx, d.H, d.G(), d.L, d.S, topk);
  return hipGetLastError();
}

template <typename F>
hipError_t dispatch(const Dims& d, F&& f) {
  if (d.dtype == 1) return d.D == 128 ? f(uint16_t{}, std::integral_constant<int, 128>{})
                                      : f(uint16_t{}, std::integral_constant<int, 64>{});
  return d.D == 128 ? f(float{}, std::integral_constant<int, 128>{}) : f(float{}, std::integral_constant<int, 64>{});
}

}  // namespace

bool decode_sparse_supported(const Dims& d) { return d.n() <= kDecodeMaxBlocks; }

LaunchResult launch_decode_append(const Dims& d, const int32_t* pos, const void* k_new, const void* v_new,
                                  void* k_cache, void* v_cache, float* k_mean, hipStream_t st) {
  LaunchResult r;
  r.err = dispatch(d, [&](auto t, auto dd) {
    return run_append<decltype(t), decltype(dd)::value>(d, pos, k_new, v_new, k_cache, v_cache, k_mean, st);
  });
  return r;
}

size_t decode_sparse_scratch_bytes(const Dims& d, int topk, bool own_idx) {
  const int ns = splits(d, true, topk);
  const size_t part_bytes = (size_t)d.bh() * ns * (d.D + 2) * sizeof(float);
  return part_bytes + (own_idx ? 0 : (size_t)d.bh() * topk * sizeof(int32_t));
}

// Selection, split attention and combine; `ws` holds the split results and, when the
// caller passes no idx, the kept blocks.  The combine reads only the splits the same
// call wrote, so ws needs no clearing.
static hipError_t decode_sparse_into(const Dims& d, const int32_t* pos, const void* q, const void* k_cache,
                                     const void* v_cache, const float* k_mean, int topk, float scale, void* o,
                                     float* lse, int32_t* idx, void* ws, hipStream_t st) {
  const size_t part_bytes = decode_sparse_scratch_bytes(d, topk, true);
  float* part = static_cast<float*>(ws);
  int32_t* sel = idx ? idx : reinterpret_cast<int32_t*>(static_cast<char*>(ws) + part_bytes);
  return dispatch(d, [&](auto t, auto dd) {
    using T = decltype(t);
    constexpr int D = decltype(dd)::value;
    hipError_t e = run_topk<T, D>(d, pos, q, k_mean, topk, sel, st);
    if (e != hipSuccess) return e;
    return run_attn<T, D, true, true>(d, pos, q, k_cache, v_cache, sel, topk, scale, o, lse, part, st);
  });
}

LaunchResult launch_decode_sparse(const Dims& d, const int32_t* pos, const void* q, const void* k_cache,
                                  const void* v_cache, const float* k_mean, int topk, float scale, void* o, float* lse,
                                  int32_t* idx, hipStream_t st) {
  LaunchResult r;
  if (!decode_sparse_supported(d)) {
    r.unsupported = "decoding selects over at most 8192 blocks (L / block)";
    return r;
  }
  void* ws = nullptr;
  r.err = workspace_alloc(decode_sparse_scratch_bytes(d, topk, idx != nullptr), &ws, st);
  if (r.err != hipSuccess) return r;
  r.err = decode_sparse_into(d, pos, q, k_cache, v_cache, k_mean, topk, scale, o, lse, idx, ws, st);
  const hipError_t fe = workspace_free(ws, st);
  if (r.err == hipSuccess) r.err = fe;
  return r;
}

// ---------------------------------------------------------------- allocation-free variant
// The same work with its scratch in a fixed device array instead of the pool, for
// callers that cannot allocate (graph capture, serving loops).  Each device holds its
// own copy of the array, at an address found once per device with that device current;
// host code uses that address, never the array's name (a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[kDecodeScratchMax];

static hipError_t scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

LaunchResult launch_decode_sparse_noalloc(const Dims& d, const int32_t* pos, const void* q, const void* k_cache,
                                          const void* v_cache, const float* k_mean, int topk, float scale, void* o,
                                          float* lse, int32_t* idx, hipStream_t st) {
  LaunchResult r;
  if (!decode_sparse_supported(d)) {
    r.unsupported = "decoding selects over at most 8192 blocks (L / block)";
    return r;
  }
  if (decode_sparse_scratch_bytes(d, topk, idx != nullptr) > kDecodeScratchMax) {
    r.unsupported = "needs more than the 16 MiB of fixed scratch (B*H*ceil(topk*block/256)*(D+2)*4 bytes, plus "
                    "B*H*topk*4 when idx is NULL)";
    return r;
  }
  void* ws = nullptr;
  r.err = scratch_address(&ws);
  if (r.err != hipSuccess) return r;
  r.err = decode_sparse_into(d, pos, q, k_cache, v_cache, k_mean, topk, scale, o, lse, idx, ws, st);
  return r;
}

LaunchResult launch_decode_full(const Dims& d, const int32_t* pos, const void* q, const void* k_cache,
                                const void* v_cache, float scale, void* o, float* lse, hipStream_t st) {
  LaunchResult r;
  const bool group = d.dtype == 1 && d.G() > 1;
  const int ns = group ? (max_chunks(d, false, 1) + kGroupCps - 1) / kGroupCps : splits(d, false, 1);
  void* ws = nullptr;
  r.err = workspace_alloc((size_t)d.bh() * ns * (d.D + 2) * sizeof(float), &ws, st);
  if (r.err != hipSuccess) return r;
  float* part = static_cast<float*>(ws);
  if (group) {  // grouped heads: one pass over K/V per group on the matrix cores
    r.err = d.D == 128 ? (o ? run_group<128, true>(d, pos, q, k_cache, v_cache, scale, o, lse, part, st)
                            : run_group<128, false>(d, pos, q, k_cache, v_cache, scale, o, lse, part, st))
                       : (o ? run_group<64, true>(d, pos, q, k_cache, v_cache, scale, o, lse, part, st)
                            : run_group<64, false>(d, pos, q, k_cache, v_cache, scale, o, lse, part, st));
  } else {
    r.err = dispatch(d, [&](auto t, auto dd) {
      using T = decltype(t);
      constexpr int D = decltype(dd)::value;
      return o ? run_attn<T, D, false, true>(d, pos, q, k_cache, v_cache, nullptr, 1, scale, o, lse, part, st)
               : run_attn<T, D, false, false>(d, pos, q, k_cache, v_cache, nullptr, 1, scale, o, lse, part, st);
    });
  }
  const hipError_t fe = workspace_free(ws, st);
  if (r.err == hipSuccess) r.err = fe;
  return r;
}

}  // namespace ssa
