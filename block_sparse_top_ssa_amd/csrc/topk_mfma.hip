// Per-query causal top-k block selection (paper sec. 3, p. 4: each query scores the
// blocks before its own with their mean-pooled keys and keeps the best k, its own
// block always included; App. D, p. 21: the block-scoring stage).
//
// All rows of one query block share the same candidates (the blocks before it), so a
// workgroup owns one query block of one (b, h) and streams the candidates in chunks
// of 64.  Scores are on MFMA: sigma = q . kbar with kbar (float32) split exactly into
// three bf16 terms hi + mid + lo (each the bf16 rounding of what is left), so three
// bf16 products per element give the float32 dot product (bf16 x bf16 products are
// exact in the float32 accumulator).  Each wave scores 16 candidates against 64 rows
// of the block and leaves the scores in LDS.  Candidates are ordered by 64-bit keys
// (score, then lower block index first), so all keys of a row are distinct.
//
// Selection of the m = topk - 1 best keys per row:
//  * m <= 40 (two passes over the scores, computed twice; kbar is split once, ahead,
//    into MFMA fragments).  A row's 64 candidates of a chunk go to the four lanes of a
//    quad, 16 consecutive ones each:
//    1. every lane keeps the largest score of each of its 16 candidate classes (block
//       index mod 64); the m-th largest t of the row's 64 class maxima gives a lower
//       bound (t, any block) on the row's m-th largest key, because m of its keys have
//       scores >= t;
//    2. the keys at or above that bound are collected in index order (about 31-45 for
//       m = 31 on unstructured scores); their m-th largest is exactly the row's m-th
//       largest key, and the keys at or above it are emitted in index order.  If more
//       than 64 keys reach the bound, the m-th largest of the first 64 collected is a
//       strictly higher bound and pass 2 runs again (only for such rows).
//    Both m-th largest values come from a 32-bit sort of the score bits (a quad's 64
//    values sorted in registers); equal scores at the cut are then settled by index
//    with a ballot, which is exact because the collected keys sit in index order;
//  * m > 40: each chunk's 64 keys are sorted across the wave with a bitonic network and
//    merged into the row's running list of the best 64*E keys in LDS; the result is
//    re-sorted by block index.  (For m close to 64 the first pass's bound is weak: rows
//    would collect far more than 64 keys and refine many times.)
// Output per row: the selected blocks in ascending order, then b_t, then -1.
#include <type_traits>

#include "launch.hpp"
#include "mfma.hpp"

namespace ssa {

// The value held by lane l ^ J, moved with DPP inside 16-lane rows (J <= 8), a
// swizzle inside 32-lane halves (J = 16) or a permute (J = 32).
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const int x = (int)v;
  if constexpr (J == 1) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  if constexpr (J == 2) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  if constexpr (J == 4) {
    const int t = __builtin_amdgcn_update_dpp(x, x, 0x104, 0xF, 0x5, false);  // row_shl:4 into lanes 0-3, 8-11
    return (uint32_t)__builtin_amdgcn_update_dpp(t, x, 0x114, 0xF, 0xA, false);  // row_shr:4 into 4-7, 12-15
  }
  if constexpr (J == 8) return (uint32_t)__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false);  // row_ror:8
  if constexpr (J == 16) return (uint32_t)__builtin_amdgcn_ds_swizzle(x, 0x401F);  // and 31, xor 16
  return (uint32_t)__shfl_xor(x, 32);
}

// Bitonic compare-exchange with lane l ^ J: the lane keeps the larger key of the pair
// if keep_max, else the smaller.
template <int J>
__device__ __forceinline__ uint64_t cx_lanes(uint64_t x, bool keep_max) {
  const uint64_t y = ((uint64_t)xor_lane<J>((uint32_t)(x >> 32)) << 32) | xor_lane<J>((uint32_t)x);
  return (x > y) == keep_max ? x : y;
}
template <int J>
__device__ __forceinline__ uint64_t cx_lanes_dir(uint64_t x, bool desc) {
  const int lane = threadIdx.x & 63;
  return cx_lanes<J>(x, ((lane & J) == 0) == desc);
}

// one bitonic stage (block size K2, distance J) of a full sort in direction `asc`
template <int K2, int J>
__device__ __forceinline__ uint64_t sort_stage(uint64_t x, bool asc) {
  const int lane = threadIdx.x & 63;
  const bool blk_asc = ((lane & K2) == 0) == asc;
  return cx_lanes_dir<J>(x, !blk_asc);
}
template <int K2, int J>
struct SortStages {
  __device__ static __forceinline__ uint64_t run(uint64_t x, bool asc) {
    x = sort_stage<K2, J>(x, asc);
    if constexpr (J > 1) return SortStages<K2, J / 2>::run(x, asc);
    else if constexpr (K2 < 64) return SortStages<K2 * 2, K2>::run(x, asc);
    else return x;
  }
};

// full bitonic sort of 64 lane values; ascending if `asc`
__device__ __forceinline__ uint64_t sort64(uint64_t x, bool asc) { return SortStages<2, 1>::run(x, asc); }

// ---------------------------------------------------------------- m-th largest of 64 values per quad
// With a row's 64 values spread over the four lanes of a quad, 16 each, one sorting
// network in registers orders all 16 rows a wave holds at once: each lane sorts its 16
// values, and two bitonic merges with the partner lane's values in reverse order join
// them into the row's 64 values in descending order.
__device__ __forceinline__ void minmax_u32(uint32_t& hi, uint32_t& lo) {
  const uint32_t a = hi, b = lo;
  hi = a > b ? a : b;
  lo = a > b ? b : a;
}
__device__ __forceinline__ void sort16_desc(uint32_t (&x)[16]) {
#pragma unroll
  for (int k2 = 2; k2 <= 16; k2 <<= 1)
#pragma unroll
    for (int j = k2 >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int l = i ^ j;
        if (l > i) {
          if ((i & k2) == 0) minmax_u32(x[i], x[l]);  // descending block
          else minmax_u32(x[l], x[i]);
        }
      }
}
// half-cleaners 8, 4, 2, 1: a bitonic sequence of 16 into descending order
__device__ __forceinline__ void clean16_desc(uint32_t (&x)[16]) {
#pragma unroll
  for (int j = 8; j > 0; j >>= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & j) == 0) minmax_u32(x[i], x[i ^ j]);
}
// v_max_f32 / v_med3_u32 as single instructions (the library max of floats adds a
// quieting step per operand; the scores are never NaN)
__device__ __forceinline__ float max_f32(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float med3_f32(float a, float b, float c) {
  float r;
  asm("v_med3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
template <int PERM>
__device__ __forceinline__ uint32_t quad_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, PERM, 0xF, 0xF, false);
}
// Sorts the 64 values a quad holds (16 per lane) into descending order, element
// 16 p + i in register i of lane p: each lane sorts its 16 by an in-register network,
// then bitonic merges with the partner lanes (p^1, then p^3 and p^1) join them.  About
// 30 instructions per quad, against about 125 for a 64-lane network.
__device__ __forceinline__ void sort64_quad_desc(uint32_t (&x)[16]) {
  const int p = threadIdx.x & 3;
  sort16_desc(x);
  {  // lanes p, p^1: two descending 16-lists into one descending 32-list over the pair
    uint32_t y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = quad_lane<0xB1>(x[15 - i]);  // quad_perm 1,0,3,2
    const uint32_t keep = (p & 1) == 0 ? 0xFFFFFFFFu : 0u;  // med3 with it: max, else min
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = med3_u32(x[i], y[i], keep);
    clean16_desc(x);
  }
  {  // lanes 0,1 and 2,3: two descending 32-lists into the quad's descending 64
    uint32_t y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = quad_lane<0x1B>(x[15 - i]);  // quad_perm 3,2,1,0
    const uint32_t top = p < 2 ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = med3_u32(x[i], y[i], top);
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = quad_lane<0xB1>(x[i]);
    const uint32_t keep = (p & 1) == 0 ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = med3_u32(x[i], y[i], keep);
    clean16_desc(x);
  }
}
// Element e (0 <= e < 64) of a quad's sorted 64, in every lane of the quad.
__device__ __forceinline__ uint32_t quad_element(const uint32_t (&x)[16], int e) {
  const int lane = threadIdx.x & 63, ii = e & 15;
  uint32_t sel = x[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) sel = i == ii ? x[i] : sel;
  return (uint32_t)__shfl((int)sel, (lane & ~3) | (e >> 4));
}
// The m-th largest (1 <= m <= 64) of the 64 values a quad holds, in every lane of it.
__device__ __forceinline__ uint32_t mth_largest_quad(uint32_t (&x)[16], int m) {
  sort64_quad_desc(x);
  return quad_element(x, m - 1);
}
// The m-th largest (1 <= m <= 64) of the 128 values a quad holds (a and b, 16 + 16
// per lane): both sorted, the top 64 of the two lists is max(a[e], b[63 - e]) (a
// bitonic sequence), put in order by half-cleaners 32 (lanes p^2), 16 (lanes p^1)
// and 8 .. 1 (registers).
__device__ __forceinline__ uint32_t mth_largest_quad128(uint32_t (&a)[16], uint32_t (&b)[16], int m) {
  const int p = threadIdx.x & 3;
  sort64_quad_desc(a);
  sort64_quad_desc(b);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t y = quad_lane<0x1B>(b[15 - i]);  // element 63 - e: lane 3 - p, register 15 - i
    a[i] = a[i] > y ? a[i] : y;
  }
  {
    uint32_t y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = quad_lane<0x4E>(a[i]);  // quad_perm 2,3,0,1
    const uint32_t top = p < 2 ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = med3_u32(a[i], y[i], top);
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = quad_lane<0xB1>(a[i]);
    const uint32_t keep = (p & 1) == 0 ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = med3_u32(a[i], y[i], keep);
    clean16_desc(a);
  }
  return quad_element(a, m - 1);
}

// Exclusive prefix sum of x over the lanes of a quad (in lane order), and the quad's
// total in *total.
__device__ __forceinline__ int quad_excl_sum(int x, int* total) {
  const int p = threadIdx.x & 3;
  int s = x;
  int y = (int)quad_lane<0x90>((uint32_t)s);  // quad_perm 0,0,1,2: lane p - 1
  s += p >= 1 ? y : 0;
  y = (int)quad_lane<0x40>((uint32_t)s);  // quad_perm 0,0,0,1: lane p - 2
  s += p >= 2 ? y : 0;
  *total = (int)quad_lane<0xFF>((uint32_t)s);  // quad_perm 3,3,3,3
  return s - x;
}

// bitonic merge (half-cleaners) of KP = 64*E values laid out as p = e*64 + lane,
// into descending order
template <int E>
__device__ __forceinline__ void merge_desc(uint64_t (&x)[E]) {
#pragma unroll
  for (int je = E / 2; je > 0; je >>= 1)
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((e & je) == 0) {
        const uint64_t a = x[e], b = x[e + je];
        x[e] = a > b ? a : b;
        x[e + je] = a > b ? b : a;
      }
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = cx_lanes_dir<32>(x[e], true);
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = cx_lanes_dir<16>(x[e], true);
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = cx_lanes_dir<8>(x[e], true);
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = cx_lanes_dir<4>(x[e], true);
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = cx_lanes_dir<2>(x[e], true);
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = cx_lanes_dir<1>(x[e], true);
}

// full bitonic sort ascending of KP = 64*E values (p = e*64 + lane)
template <int E>
__device__ __forceinline__ void sort_asc(uint64_t (&x)[E]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k2 = 2; k2 <= 64 * E; k2 <<= 1)
#pragma unroll
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      if (j >= 64) {
        const int je = j / 64;
#pragma unroll
        for (int e = 0; e < E; ++e)
          if ((e & je) == 0) {
            const int p = e * 64 + lane;
            const bool asc = (p & k2) == 0;
            const uint64_t a = x[e], b = x[e + je];
            const bool sw = asc ? (a > b) : (a < b);
            x[e] = sw ? b : a;
            x[e + je] = sw ? a : b;
          }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int p = e * 64 + lane;
          const bool desc = (p & k2) != 0;
          switch (j) {
            case 32: x[e] = cx_lanes_dir<32>(x[e], desc); break;
            case 16: x[e] = cx_lanes_dir<16>(x[e], desc); break;
            case 8: x[e] = cx_lanes_dir<8>(x[e], desc); break;
            case 4: x[e] = cx_lanes_dir<4>(x[e], desc); break;
            case 2: x[e] = cx_lanes_dir<2>(x[e], desc); break;
            default: x[e] = cx_lanes_dir<1>(x[e], desc); break;
          }
        }
      }
    }
}

__device__ __forceinline__ void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f32_to_bf16_bits(x);
  const float r1 = x - bf16_bits_to_f32(hi);
  mid = f32_to_bf16_bits(r1);
  const float r2 = r1 - bf16_bits_to_f32(mid);
  lo = f32_to_bf16_bits(r2);
}
// The same split for two values at once, packed as a bf16 pair per term (x0 in the low
// half): one paired conversion per term, the same nearest-even rounding as split3.
__device__ __forceinline__ void split3x2(float x0, float x1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = pack_bf16x2(x0, x1);
  const float r0 = x0 - lo_bf16(hi), r1 = x1 - hi_bf16(hi);
  mid = pack_bf16x2(r0, r1);
  const float s0 = r0 - lo_bf16(mid), s1 = r1 - hi_bf16(mid);
  lo = pack_bf16x2(s0, s1);
}

template <int D, int S, int E>
__global__ __launch_bounds__(256) void topk_merge_kernel(const uint16_t* __restrict__ q, const float* __restrict__ km,
                                                        int32_t* __restrict__ idx, float* __restrict__ sel, int L,
                                                        int n, int BH, int topk, int G) {
  constexpr int NC = D / 32, NT = S / 16, KP = 64 * E, SCS = 65;
  __shared__ float sc[S][SCS];
  __shared__ uint64_t lists[S][KP];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
  const int nn = lane & 15, g = lane >> 4;
  const int64_t wg = xcd_logical(blockIdx.x, (int64_t)gridDim.x);  // one head per XCD at a time
  const int64_t bh = wg / n;
  const int qb = n - 1 - (int)(wg % n);
  const int m = min(topk - 1, qb);
  const uint16_t* qh = q + (bh * L + (int64_t)qb * S) * D;
  const float* kmh = km + (bh / G) * (int64_t)n * D;  // pooled keys of this head's K/V head
  int32_t* ih = idx + (bh * L + (int64_t)qb * S) * topk;
  float* sh = sel ? sel + (bh * L + (int64_t)qb * S) * topk : nullptr;
  const float inf = __builtin_huge_valf();

  if (m == qb || m == 0) {
    // every candidate kept (or none to keep): no selection needed
    for (int it = tid; it < S * topk; it += 256) {
      const int r = it / topk, p = it % topk;
      ih[it] = p < qb && m == qb ? p : (p == m ? qb : -1);
      if (sh) {
        float v = p == m ? inf : -inf;
        if (p < m) {
          float acc = 0.f;
          const uint16_t* qr = qh + (int64_t)r * D;
          const float* kr = kmh + (int64_t)p * D;
          for (int d = 0; d < D; ++d) acc = fmaf(bf16_bits_to_f32(qr[d]), kr[d], acc);
          v = acc;
        }
        sh[it] = v;
      }
    }
    return;
  }

  for (int it = tid; it < S * KP; it += 256) (&lists[0][0])[it] = 0;
  u32x4 qf[NT][NC];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) qf[nt][cc] = load_q_frag<D>(qh + (int64_t)(16 * nt + nn) * D, cc);

  const int nchunks = (qb + 63) / 64;
  for (int chunk = 0; chunk < nchunks; ++chunk) {
    const int cb = chunk * 64;
    // ---- scores: wave w takes candidates cb + 16w .. +15 against every row
    {
      const int j = cb + 16 * w + nn;
      const bool valid = j < qb;
      u32x4 ah[NC], am[NC], al[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        float x[8];
        if (valid) {
          const float* src = kmh + (int64_t)j * D + 32 * cc + 8 * g;
          const u32x4 w0 = load16(src), w1 = load16(src + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = __uint_as_float(w0[e]);
            x[4 + e] = __uint_as_float(w1[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.f;
        }
        uint32_t h[8], md[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) split3(x[e], h[e], md[e], lo[e]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ah[cc][e] = h[2 * e] | (h[2 * e + 1] << 16);
          am[cc][e] = md[2 * e] | (md[2 * e + 1] << 16);
          al[cc][e] = lo[2 * e] | (lo[2 * e + 1] << 16);
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        f32x4 acc = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          acc = mfma_bf16(al[cc], qf[nt][cc], acc);
          acc = mfma_bf16(am[cc], qf[nt][cc], acc);
          acc = mfma_bf16(ah[cc], qf[nt][cc], acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[16 * nt + nn][16 * w + 4 * g + i] = acc[i];
      }
    }
    __syncthreads();
    // ---- selection: wave w merges the chunk into rows w, w+4, ...
    for (int r = w; r < S; r += 4) {
      const int j = cb + lane;
      uint64_t key = j < qb ? make_key(sc[r][lane], j) : 0ull;
      key = sort64(key, true);
      uint64_t x[E];
#pragma unroll
      for (int e = 0; e < E; ++e) x[e] = lists[r][e * 64 + lane];
      x[E - 1] = x[E - 1] > key ? x[E - 1] : key;
      merge_desc<E>(x);
#pragma unroll
      for (int e = 0; e < E; ++e) lists[r][e * 64 + lane] = x[e];
    }
    __syncthreads();
  }

  // ---- output: the best m blocks in ascending block order, then qb, then -1
  for (int r = w; r < S; r += 4) {
    uint64_t x[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int p = e * 64 + lane;
      const uint64_t kk = lists[r][p];
      x[e] = p < m ? (((uint64_t)key_index(kk) << 32) | (kk >> 32)) : ~0ull;
    }
    sort_asc<E>(x);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int p = e * 64 + lane;
      if (p < topk) {
        ih[(int64_t)r * topk + p] = p < m ? (int)(x[e] >> 32) : (p == m ? qb : -1);
        if (sh) sh[(int64_t)r * topk + p] = p < m ? unorderable_f32((uint32_t)x[e]) : (p == m ? inf : -inf);
      }
    }
  }
}


// kbar split into its three bf16 terms once per launch and stored as the MFMA A
// fragments the selection kernel reads: fragment (chunk, w, cc, term) of a K/V head
// gives lane (nn, g) that term's 8 values of candidate 64 chunk + 16 w + nn, columns
// 32 cc + 8 g .. +7 (term 0 = hi, 1 = mid, 2 = lo; rows past the pooled keys are zero).
// Each fragment is one contiguous 1 KB load, and the selection kernel, which scores
// every chunk at least twice, does no splitting.  kn2[chunk] gets the largest squared
// norm of the chunk's pooled keys (rounded up), for the first pass's error margin.
template <int D>
__global__ __launch_bounds__(256) void ksplit_kernel(const float* __restrict__ km, u32x4* __restrict__ ks,
                                                     float* __restrict__ kn2, int n, int nck) {
  constexpr int NC = D / 32;
  __shared__ float wmax[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nn = lane & 15, g = lane >> 4;
  const int64_t ch = blockIdx.x;  // (K/V head, chunk)
  const int64_t kvh = ch / nck;
  const int j = (int)(ch % nck) * 64 + 16 * w + nn;
  const float* src = km + (kvh * n + j) * (int64_t)D + 8 * g;
  u32x4* out = ks + (ch * 4 + w) * (3 * NC * 64) + lane;
  float ss = 0.f;
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    u32x4 w0 = {0, 0, 0, 0}, w1 = {0, 0, 0, 0};
    if (j < n) {
      w0 = load16(src + 32 * cc);
      w1 = load16(src + 32 * cc + 4);
    }
    u32x4 h, md, lo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t a = e < 2 ? w0[2 * e] : w1[2 * e - 4], b = e < 2 ? w0[2 * e + 1] : w1[2 * e - 3];
      uint32_t th, tm, tl;
      split3x2(__uint_as_float(a), __uint_as_float(b), th, tm, tl);
      h[e] = th;
      md[e] = tm;
      lo[e] = tl;
      ss = fmaf(__uint_as_float(a), __uint_as_float(a), ss);
      ss = fmaf(__uint_as_float(b), __uint_as_float(b), ss);
    }
    out[(3 * cc + 0) * 64] = h;
    out[(3 * cc + 1) * 64] = md;
    out[(3 * cc + 2) * 64] = lo;
  }
  ss += __shfl_xor(ss, 16);  // the four lanes of candidate nn
  ss += __shfl_xor(ss, 32);
  ss = wave_max(ss);
  if (lane == 0) wmax[w] = ss;
  __syncthreads();
  if (threadIdx.x == 0)  // rounded up past the float sums' error
    kn2[ch] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])) * (1.f + 0x1p-16f);
}

// Two-pass selection, exact for m = topk - 1 <= 64 (see the top of the file).
// S / 16 waves: for scoring, wave w takes candidates 16 (w & 3) .. +15 of each chunk
// against rows 64 (w >> 2) .. +63; for selection, lane (r, p) = (lane >> 2, lane & 3)
// of wave w takes row 16 w + r and, of each chunk, the 16 candidates 16 p .. +15, so a
// row's 64 candidates sit in one quad and every selection step is per-lane arithmetic
// or a move inside the quad.
//   T: approximate scores kept per candidate class in the first pass (1: the largest,
// for m <= 40; 2: the two largest, so that the bound stays tight up to m = 64).
//   CAP: entries collected per row (64 or 128); NB: score buffers (2: one barrier per
// chunk; 1: two, for the larger workgroups).
template <int D, int S, int T, int CAP, int NB>
__global__ __launch_bounds__(S * 4, 2) void topk_select_kernel(const uint16_t* __restrict__ q,
                                                            const u32x4* __restrict__ ks,
                                                            const float* __restrict__ kn2,
                                                            const float* __restrict__ km, int32_t* __restrict__ idx,
                                                            float* __restrict__ sel, int L, int n, int nck, int topk,
                                                            int G) {
  constexpr int NC = D / 32, NF = 3 * NC, NT = 4, NTH = S * 4, SCS = 68, NH = CAP / 64;
  // Scores of a chunk; rows 68 words apart: 16-byte aligned, and the quads' 16-byte
  // reads fall in distinct banks.
  __shared__ __align__(16) float scb[NB][S][SCS];
  // Collected entries, in index order: raw score and block index (rows start in
  // different banks).
  __shared__ float esc[S][CAP + 1];
  __shared__ uint16_t eix[S][CAP + 2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
  const int nn = lane & 15, g = lane >> 4;
  const int cw = w & 3, rh = w >> 2;
  const int rq = lane >> 2, p = lane & 3, row = 16 * w + rq;
  const int64_t wg = xcd_logical(blockIdx.x, (int64_t)gridDim.x);  // one head per XCD at a time
  const int64_t bh = wg / n;
  const int qb = n - 1 - (int)(wg % n);
  const int m = min(topk - 1, qb);
  const uint16_t* qh = q + (bh * L + (int64_t)qb * S) * D;
  const int64_t kvh = bh / G;  // this head's K/V head
  int32_t* ih = idx + (bh * L + (int64_t)qb * S) * topk;
  float* sh = sel ? sel + (bh * L + (int64_t)qb * S) * topk : nullptr;
  const float inf = __builtin_huge_valf();

  if (m == qb || m == 0) {
    // every candidate kept (or none to keep): no selection needed
    const float* kmh = km + kvh * (int64_t)n * D;
    for (int it = tid; it < S * topk; it += NTH) {
      const int r = it / topk, pp = it % topk;
      ih[it] = pp < qb && m == qb ? pp : (pp == m ? qb : -1);
      if (sh) {
        float v = pp == m ? inf : -inf;
        if (pp < m) {
          float acc = 0.f;
          const uint16_t* qr = qh + (int64_t)r * D;
          const float* kr = kmh + (int64_t)pp * D;
          for (int d = 0; d < D; ++d) acc = fmaf(bf16_bits_to_f32(qr[d]), kr[d], acc);
          v = acc;
        }
        sh[it] = v;
      }
    }
    return;
  }

  u32x4 qf[NT][NC];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) qf[nt][cc] = load_q_frag<D>(qh + (int64_t)(64 * rh + 16 * nt + nn) * D, cc);
  const u32x4* kst = ks + ((kvh * nck) * 4 + cw) * (NF * 64) + lane;
  const int nchunks = (qb + 63) / 64;
  // kbar fragments of the next chunk to score, loaded one chunk ahead
  u32x4 kf[NF];
  auto load_frags = [&](int c) {
#pragma unroll
    for (int f = 0; f < NF; ++f) kf[f] = kst[((int64_t)c * 4 * NF + f) * 64];
  };
  // Scores of one chunk against this wave's 64 rows: four independent accumulation
  // chains (one per 16 rows), each in the order lo, mid, hi per 32 columns.  The MFMAs
  // of the next chunk are issued before the current chunk is selected, so they run
  // under the selection's vector work.
  f32x4 acc[NT];
  auto mfma_chunk = [&]() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int t = 2; t >= 0; --t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_bf16(kf[3 * cc + t], qf[nt][cc], acc[nt]);
  };
  // the scores into sc; candidates past the block's own score -inf, below every score
  auto store_scores = [&](int cb, float (*sc)[SCS]) {
    const bool tail = cb + 64 > qb;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 a4 = acc[nt];
      if (tail) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a4[i] = cb + 16 * cw + 4 * g + i < qb ? a4[i] : -inf;
      }
      *reinterpret_cast<f32x4*>(&sc[64 * rh + 16 * nt + nn][16 * cw + 4 * g]) = a4;
    }
  };
  auto buffer = [&](int chunk) { return scb[NB == 2 ? (chunk & 1) : 0]; };
  // One pass over the chunks: select(cb, sc) sees each chunk's scores in turn.  On
  // entry kf holds chunk 0, and on return again (the last prefetch wraps to chunk 0).
  auto pass = [&](auto&& select) {
    mfma_chunk();
    load_frags(nchunks > 1 ? 1 : 0);
    for (int chunk = 0; chunk < nchunks; ++chunk) {
      float (*sc)[SCS] = buffer(chunk);
      if (NB == 1 && chunk > 0) __syncthreads();  // the previous chunk's scores are read
      store_scores(chunk * 64, sc);
      if (chunk + 1 < nchunks) {
        mfma_chunk();
        load_frags(chunk + 2 < nchunks ? chunk + 2 : 0);
      }
      __syncthreads();
      select(chunk * 64, sc);
    }
  };
  auto read_scores = [&](const float (*sc)[SCS], float (&v)[16]) {
    const f32x4* src = reinterpret_cast<const f32x4*>(&sc[row][16 * p]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 v4 = src[k];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * k + e] = v4[e];
    }
  };

  // ---- pass 1: approximate scores from the hi term alone (a third of the loads and
  // MFMAs).  The T largest of each of the row's 64 candidate classes (block index mod
  // 64, 16 per lane) and the m-th largest t of those mean that m distinct keys have
  // approximate scores >= t.  An approximate score is within eps of the float32 score
  // used for the keys, so (t - eps, any block) is at most the row's m-th key.
  //   The hi term differs from kbar by at most 2^-8 |kbar| per element (nearest-even
  // rounding to 8 significant bits); the float32 accumulations add at most D 2^-24
  // (approximate score) and 3 D 2^-24 (score) of sum_d |q_d kbar_d|, below
  // 2^-8 (2^-9 + 2^-7.4) of it for D <= 128; so with Cauchy-Schwarz
  // |approx - score| <= 1.008 2^-8 |q| |kbar|, and eps = 1.02 2^-8 |q| max|kbar|
  // (the norms' own float32 rounding is far inside the difference).
  // two register sets of hi-term fragments, so the loads run two chunks ahead (the
  // pass-2 fragment registers are free during this pass)
  u32x4 khA[NC], khB[NC];
  auto load_hi = [&](u32x4 (&kh)[NC], int c) {
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) kh[cc] = kst[((int64_t)c * 4 * NF + 3 * cc) * 64];
  };
  auto mfma_hi = [&](const u32x4 (&kh)[NC]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_bf16(kh[cc], qf[nt][cc], acc[nt]);
  };
  // The class maxima are kept where the products leave them: lane (nn, g) of wave w
  // holds, for row 64 rh + 16 nt + nn, the candidates 16 cw + 4 g + i of every chunk,
  // i.e. the classes 16 cw + 4 g + i.  So this pass needs no LDS and no barrier per
  // chunk (the other wave on the SIMD covers the products' latency).  At the end the
  // maxima go through LDS once to the selection layout.
  float m1[NT][4], m2[NT][4];  // the largest (and for T = 2 the second largest) per class
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) m1[nt][i] = m2[nt][i] = -inf;
  auto take_maxima = [&](int cb) {
    const bool tail = cb + 64 > qb;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = !tail || cb + 16 * cw + 4 * g + i < qb ? acc[nt][i] : -inf;
        if constexpr (T == 2) m2[nt][i] = med3_f32(m1[nt][i], m2[nt][i], v);
        m1[nt][i] = max_f32(m1[nt][i], v);
      }
  };
  load_hi(khA, 0);
  if (nchunks > 1) load_hi(khB, 1);
  for (int chunk = 0; chunk < nchunks; chunk += 2) {
    mfma_hi(khA);
    if (chunk + 2 < nchunks) load_hi(khA, chunk + 2);
    take_maxima(chunk * 64);
    if (chunk + 1 < nchunks) {
      mfma_hi(khB);
      if (chunk + 3 < nchunks) load_hi(khB, chunk + 3);
      take_maxima((chunk + 1) * 64);
    }
  }
  load_frags(0);  // pass 2 starts with chunk 0
  // to the selection layout: row r's classes 16 p .. +15 in lane (r, p)
  float c1[16], c2[16];
  auto to_rows = [&](const float (&mx)[NT][4], float (&out)[16]) {
    float (*sc)[SCS] = scb[0];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      *reinterpret_cast<f32x4*>(&sc[64 * rh + 16 * nt + nn][16 * cw + 4 * g]) =
          f32x4{mx[nt][0], mx[nt][1], mx[nt][2], mx[nt][3]};
    __syncthreads();
    read_scores(sc, out);
    __syncthreads();
  };
  to_rows(m1, c1);
  if constexpr (T == 2) to_rows(m2, c2);
  // The bound as a float tf and a block limit jmax: key (x, j) is at or above it iff
  // x > tf, or x == tf and j <= jmax (float comparison folds -0 onto +0 as the keys do).
  float tf;
  int jmax = 0x7FFFFFFF;
  {
    // |q| of the lane's row (its quad sums the squares of D / 4 elements each)
    float qq = 0.f;
    const uint16_t* qr = qh + (int64_t)row * D + (D / 4) * p;
#pragma unroll
    for (int k = 0; k < D / 32; ++k) {
      const u32x4 w4 = load16(qr + 8 * k);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = lo_bf16(w4[e]), b = hi_bf16(w4[e]);
        qq = fmaf(a, a, fmaf(b, b, qq));
      }
    }
    qq += __shfl_xor(qq, 1);
    qq += __shfl_xor(qq, 2);
    float kk = 0.f;  // largest squared norm of the block's pooled keys
    const float* kn2h = kn2 + kvh * nck;
    for (int c = 0; c < nchunks; ++c) kk = fmaxf(kk, kn2h[c]);
    const float eps = 1.02f * 0x1p-8f * __builtin_sqrtf(qq * kk);
    uint32_t u1[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) u1[s] = orderable_f32(c1[s]);
    uint32_t t;
    if constexpr (T == 2) {
      uint32_t u2[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) u2[s] = orderable_f32(c2[s]);
      t = mth_largest_quad128(u1, u2, m);
    } else {
      t = mth_largest_quad(u1, m);
    }
    tf = unorderable_f32(t) - eps;
  }
  bool act = true;  // rows done keep tf = +inf, so that nothing reaches their bound

  // ---- pass 2: collect the keys at or above the bound, in index order
  int cnt = 0;
  float* erow = &esc[row][0];
  uint16_t* irow = &eix[row][0];
  auto collect = [&](auto first_c) {
    constexpr bool kFirst = decltype(first_c)::value;  // every block index at tf qualifies
    pass([&](int cb, const float (*sc)[SCS]) {
      float v[16];
      read_scores(sc, v);
      const int j0 = cb + 16 * p;
      // f[s]: candidate j0 + s is at or above the bound (lane masks, no branches)
      bool f[16];
      if constexpr (kFirst) {
#pragma unroll
        for (int s = 0; s < 16; ++s) f[s] = v[s] >= tf;
      } else {
        const int lim = jmax - j0;
#pragma unroll
        for (int s = 0; s < 16; ++s) f[s] = (v[s] > tf) | ((v[s] == tf) & (s <= lim));
      }
      int c = 0;
#pragma unroll
      for (int s = 0; s < 16; ++s) c += f[s];
      int tot;
      int pos = cnt + quad_excl_sum(c, &tot);
      if (__builtin_amdgcn_ballot_w64(cnt + tot > CAP) == 0) {
#pragma unroll
        for (int s = 0; s < 16; ++s)
          if (f[s]) {
            erow[pos] = v[s];
            irow[pos] = (uint16_t)(j0 + s);
            ++pos;
          }
      } else {  // some row of the wave overflows: keep its first CAP entries
#pragma unroll
        for (int s = 0; s < 16; ++s)
          if (f[s]) {
            if (pos < CAP) {
              erow[pos] = v[s];
              irow[pos] = (uint16_t)(j0 + s);
            }
            ++pos;
          }
      }
      cnt += tot;
    });
  };
  // The cut of the lane's row among its first min(count, CAP) entries (in index order;
  // lane (r, p) holds entries 64 h + 16 p + k in hv[h][k], as order-preserving score
  // bits, absent ones 0): t = the m-th largest score bits; the entries above t, and
  // the first `need` at t, are the row's m best.  Returns the row's m-th key (in every
  // lane of the quad); with kOut the m best are written to the outputs in index order.
  // Output staging: the block's rows of idx (and of sel) in the score buffer when they fit.
  constexpr int kScbBytes = NB * S * SCS * 4;
  const bool stage_i = S * topk * 4 <= kScbBytes;          // uniform
  const bool stage_f = sh && S * topk * 8 <= kScbBytes;
  int32_t* const ob_i = reinterpret_cast<int32_t*>(&scb[0][0][0]);
  float* const ob_f = reinterpret_cast<float*>(ob_i + S * topk);
  auto put = [&](int pos, int32_t bi, float sv) {
    if (stage_i) ob_i[row * topk + pos] = bi;
    else ih[(int64_t)row * topk + pos] = bi;
    if (sh) {
      if (stage_f) ob_f[row * topk + pos] = sv;
      else sh[(int64_t)row * topk + pos] = sv;
    }
  };
  auto cut = [&](auto out_c) -> uint64_t {
    constexpr bool kOut = decltype(out_c)::value;
    const int cl = min(cnt, CAP);
    uint32_t hv[NH][16];
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int e = 64 * h + 16 * p + k;
        hv[h][k] = e < cl ? orderable_f32(erow[e]) : 0u;
      }
    uint32_t t;
    {
      uint32_t ha[16], hb[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        ha[k] = hv[0][k];
        hb[k] = hv[NH - 1][k];
      }
      if constexpr (NH == 2) t = mth_largest_quad128(ha, hb, m);
      else t = mth_largest_quad(ha, m);
    }
    int gt = 0, eqn[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      eqn[h] = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        gt += hv[h][k] > t;
        eqn[h] += hv[h][k] == t;
      }
    }
    int tot;
    quad_excl_sum(gt, &tot);
    const int need = m - tot;  // >= 1
    int rank_base = 0, pos_base = 0, kj = -1;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      int eq_tot;
      const int rank0 = rank_base + quad_excl_sum(eqn[h], &eq_tot);
      int rank = rank0, tk = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const bool at = hv[h][k] == t;
        tk += hv[h][k] > t || (at && rank < need);
        if (at && rank == need - 1) kj = 64 * h + 16 * p + k;
        rank += at;
      }
      if constexpr (kOut) {
        int tk_tot;
        int pos = pos_base + quad_excl_sum(tk, &tk_tot);
        rank = rank0;
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const bool at = hv[h][k] == t;
          if (hv[h][k] > t || (at && rank < need)) {
            const int e = 64 * h + 16 * p + k;
            put(pos, (int32_t)irow[e], erow[e]);
            ++pos;
          }
          rank += at;
        }
        pos_base += tk_tot;
      }
      rank_base += eq_tot;
    }
    // the m-th key's entry: held by one lane of the quad
    kj = max(kj, (int)quad_lane<0xB1>((uint32_t)kj));
    kj = max(kj, (int)quad_lane<0x4E>((uint32_t)kj));
    return ((uint64_t)t << 32) | (0xFFFFFFFFu - (uint32_t)irow[max(kj, 0)]);
  };
  collect(std::true_type{});
  for (;;) {
    __syncthreads();  // the entries are complete; a repeated pass scores chunk 0 again
    // rows that collected more than CAP keys: raise the bound to the m-th largest of
    // the first CAP collected (a strictly higher bound) and collect again
    if (!__syncthreads_or(act && cnt > CAP)) break;
    const uint64_t kth = cut(std::false_type{});
    if (act && cnt > CAP) {
      tf = key_score(kth);
      jmax = key_index(kth);
    } else {
      act = false;
      tf = inf;
    }
    __syncthreads();  // every row's entries are read before they are collected again
    if (act) cnt = 0;
    collect(std::false_type{});
  }

  // ---- output: the m keys at or above the row's exact m-th key, in index order, then
  // the own block, then -1.  The S rows are assembled in the score buffer (free now)
  // and stored with 16-byte writes of the block's contiguous rows; written one entry
  // per lane instead, each store would touch 16 rows' lines.
  (void)cut(std::true_type{});
  for (int pp = m + p; pp < topk; pp += 4) put(pp, pp == m ? qb : -1, pp == m ? inf : -inf);
  if (stage_i) {
    __syncthreads();  // uniform: the block's rows are assembled
    const int total = S * topk;
    const bool vec = (total % 4 == 0) & ((reinterpret_cast<uintptr_t>(ih) & 15) == 0) &
                     (!stage_f || (reinterpret_cast<uintptr_t>(sh) & 15) == 0);
    if (vec) {
      for (int i = 4 * tid; i < total; i += 4 * NTH) {
        *reinterpret_cast<int4*>(ih + i) = *reinterpret_cast<const int4*>(ob_i + i);
        if (stage_f) *reinterpret_cast<f32x4*>(sh + i) = *reinterpret_cast<const f32x4*>(ob_f + i);
      }
    } else {
      for (int i = tid; i < total; i += NTH) {
        ih[i] = ob_i[i];
        if (stage_f) sh[i] = ob_f[i];
      }
    }
  }
}

// Largest m = topk - 1 given to the two-pass selection with one approximate score per
// candidate class, and with two (above that the class maxima alone bound the m-th key
// loosely: rows would collect several times m keys).
constexpr int kSelectMaxM1 = 40, kSelectMaxM2 = 64;

static int e_for(int topk) {
  const int need = topk - 1;
  int e = 1;
  while (64 * e < need) e <<= 1;
  return e;
}

bool topk_mfma_supported(const Dims& d, int topk) {
  if (d.dtype != 1 || (d.D != 64 && d.D != 128)) return false;
  if (d.n() > 65536) return false;  // block indices are collected as 16 bits
  if (topk - 1 <= kSelectMaxM2) return true;
  return d.S * 64 * e_for(topk) <= 8192;  // running lists: S rows x KP keys x 8 bytes <= 64 KB
}

template <int D, int S, int T, int CAP, int NB>
static hipError_t run_select(const Dims& d, const void* q, const float* km, int topk, int32_t* idx, float* sel,
                             hipStream_t st) {
  const int n = d.n(), nck = (n + 63) / 64;
  const int64_t kvheads = (int64_t)d.B * d.Hkv;
  void* ws = nullptr;
  const size_t frag_bytes = (size_t)kvheads * nck * 4 * 3 * (D / 32) * 64 * sizeof(u32x4);
  hipError_t e = workspace_alloc(frag_bytes + (size_t)kvheads * nck * sizeof(float), &ws, st);
  if (e != hipSuccess) return e;
  u32x4* ks = static_cast<u32x4*>(ws);
  float* kn2 = reinterpret_cast<float*>(static_cast<char*>(ws) + frag_bytes);
  hipLaunchKernelGGL((ksplit_kernel<D>), dim3((unsigned)(kvheads * nck)), dim3(256), 0, st, km, ks, kn2, n, nck);
  e = hipGetLastError();
  if (e == hipSuccess) {
    const int64_t grid = (int64_t)n * d.bh();
    hipLaunchKernelGGL((topk_select_kernel<D, S, T, CAP, NB>), dim3((unsigned)grid), dim3(S * 4), 0, st,
                       static_cast<const uint16_t*>(q), ks, kn2, km, idx, sel, d.L, n, nck, topk, d.G());
    e = hipGetLastError();
  }
  const hipError_t ef = vfrag_release(ws, st);
  return e != hipSuccess ? e : ef;
}

template <int D, int S, int E>
static hipError_t run_topk(const Dims& d, const void* q, const float* km, int topk, int32_t* idx, float* sel,
                           hipStream_t st) {
  const int64_t grid = (int64_t)d.n() * d.bh();
  hipLaunchKernelGGL((topk_merge_kernel<D, S, E>), dim3((unsigned)grid), dim3(256), 0, st,
                     static_cast<const uint16_t*>(q), km, idx, sel, d.L, d.n(), (int)d.bh(), topk, d.G());
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_topk(const Dims& d, const void* q, const float* km, int topk, int32_t* idx, float* sel,
                                hipStream_t st) {
  if (topk - 1 <= kSelectMaxM1)
    return d.S == 64 ? run_select<D, 64, 1, 64, 2>(d, q, km, topk, idx, sel, st)
                     : run_select<D, 128, 1, 64, 2>(d, q, km, topk, idx, sel, st);
  if (topk - 1 <= kSelectMaxM2)
    return d.S == 64 ? run_select<D, 64, 2, 128, 1>(d, q, km, topk, idx, sel, st)
                     : run_select<D, 128, 2, 128, 1>(d, q, km, topk, idx, sel, st);
  return run_topk<D, 64, 2>(d, q, km, topk, idx, sel, st);  // m > 64: S = 64 only (see supported)
}

LaunchResult launch_topk_mfma(const Dims& d, const void* q, const float* km, int topk, int32_t* idx, float* sel,
                              hipStream_t st) {
  LaunchResult r;
  r.err = d.D == 128 ? dispatch_topk<128>(d, q, km, topk, idx, sel, st)
                     : dispatch_topk<64>(d, q, km, topk, idx, sel, st);
  return r;
}

}  // namespace ssa
