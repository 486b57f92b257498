// Per-query causal top-k block selection (paper sec. 3, p. 4: each query scores the
// blocks before its own with their mean-pooled keys and keeps the best k, its own
// block always included; App. D, p. 21: the block-scoring stage).
//
// All rows of one query block share the same candidates (the blocks before it), so a
// workgroup owns one query block of one (b, h) and streams the candidates in chunks
// of 64.  Scores are on MFMA: sigma = q . kbar with kbar (float32) split exactly into
// three bf16 terms hi + mid + lo (each the bf16 rounding of what is left), so three
// bf16 products per element give the float32 dot product (bf16 x bf16 products are
// exact in the float32 accumulator).  Each wave scores 16 candidates against all rows
// of the block and leaves the scores in LDS.  Candidates are ordered by 64-bit keys
// (score, then lower block index first), so all keys of a row are distinct.
//
// Selection of the m = topk - 1 best keys per row (one wave per row at a time):
//  * m <= 40 (two passes over the scores, computed twice):
//    1. every lane keeps the largest score (as order-preserving bits) among the
//       candidates it sees (j = lane mod 64); the m-th largest t of these 64 lane
//       maxima gives a lower bound (t, 0) on the row's m-th largest key, because m of
//       its keys have score bits >= t;
//    2. the keys at or above that bound are collected in index order (about 31-45 for
//       m = 31 on unstructured scores); their m-th largest is exactly the row's m-th
//       largest key, and the keys at or above it are emitted in index order.  If more
//       than 64 keys reach the bound, the m-th largest of the first 64 collected is a
//       strictly higher bound and pass 2 runs again (only for such rows).
//    Both m-th largest values come from a 32-bit sort of the score bits across the
//    wave; equal scores at the cut are then settled by index with a ballot, which is
//    exact because the collected keys sit in index order;
//  * m > 40: each chunk's 64 keys are sorted across the wave with a bitonic network and
//    merged into the row's running list of the best 64*E keys in LDS; the result is
//    re-sorted by block index.  (For m close to 64 the first pass's bound is weak: rows
//    would collect far more than 64 keys and refine many times.)
// Output per row: the selected blocks in ascending order, then b_t, then -1.
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

// The same network on 32-bit values (one lane move and a min/max per stage).
template <int K2, int J>
struct SortStages32 {
  __device__ static __forceinline__ uint32_t run(uint32_t x, bool asc) {
    const int lane = threadIdx.x & 63;
    const bool blk_asc = ((lane & K2) == 0) == asc;
    const bool keep_max = ((lane & J) == 0) == !blk_asc;
    uint32_t a, y;
    if constexpr (J >= 16) {
      // the row swaps leave the lane's value and its partner's in the two results
      const auto pr = J == 16 ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                              : __builtin_amdgcn_permlane32_swap(x, x, false, false);
      a = pr[0];
      y = pr[1];
    } else {
      a = x;
      y = xor_lane<J>(x);
    }
    x = keep_max ? (a > y ? a : y) : (a < y ? a : y);
    if constexpr (J > 1) return SortStages32<K2, J / 2>::run(x, asc);
    else if constexpr (K2 < 64) return SortStages32<K2 * 2, K2>::run(x, asc);
    else return x;
  }
};
__device__ __forceinline__ uint32_t sort64_u32(uint32_t x, bool asc) { return SortStages32<2, 1>::run(x, asc); }

// The m-th largest (1 <= m <= 64) of the 64-bit keys held by the lanes, where absent
// lanes hold 0, at least m keys are present, and the present keys with equal score
// bits sit in ascending block order along the lanes (true of keys collected in index
// order).  Only the 32 score bits are sorted: with t the m-th largest of them, the
// m-th key is the (m - #{score > t})-th key with score t in lane order.  Returns the
// key; *t_out and *need_out describe the cut for the caller.
__device__ __forceinline__ uint64_t kth_key_index_ordered(uint64_t y, int m, uint32_t* t_out, int* need_out,
                                                          uint64_t* eq_out) {
  const uint32_t hi = (uint32_t)(y >> 32);
  const uint32_t t = (uint32_t)__shfl((int)sort64_u32(hi, false), m - 1);  // descending
  const int n_gt = __builtin_popcountll(__builtin_amdgcn_ballot_w64(hi > t));
  const int need = m - n_gt;  // >= 1
  const uint64_t eq = __builtin_amdgcn_ballot_w64(hi == t);
  const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0));
  const uint64_t pick = __builtin_amdgcn_ballot_w64(hi == t && rank == need - 1);
  const int src = (int)__builtin_ctzll(pick);
  *t_out = t;
  *need_out = need;
  *eq_out = eq;
  return shfl_u64(y, src);
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


// The float32 kbar values a lane needs for one 64-candidate chunk (wave w takes the
// candidates cb + 16 w .. +15; lane (nn, g) the columns 32 cc + 8 g .. +7).  The row
// index is clamped into the pooled keys, so rows past the candidates load valid memory;
// their scores are never used.
template <int D>
__device__ __forceinline__ void load_kchunk(const float* __restrict__ kmh, int cb, int n, float (&xk)[D / 32][8]) {
  constexpr int NC = D / 32;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nn = lane & 15, g = lane >> 4;
  const int j = min(cb + 16 * w + nn, n - 1);
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    const float* src = kmh + (int64_t)j * D + 32 * cc + 8 * g;
    const u32x4 w0 = load16(src), w1 = load16(src + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xk[cc][e] = __uint_as_float(w0[e]);
      xk[cc][4 + e] = __uint_as_float(w1[e]);
    }
  }
}

// Scores of one 64-candidate chunk (its kbar values in xk) against all S rows of the
// block into sc.
template <int D, int S>
__device__ __forceinline__ void score_chunk(const u32x4 (&qf)[S / 16][D / 32], const float (&xk)[D / 32][8],
                                            float (*sc)[65]) {
  constexpr int NC = D / 32, NT = S / 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nn = lane & 15, g = lane >> 4;
  u32x4 ah[NC], am[NC], al[NC];
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t h, md, lo;
      split3x2(xk[cc][2 * e], xk[cc][2 * e + 1], h, md, lo);
      ah[cc][e] = h;
      am[cc][e] = md;
      al[cc][e] = lo;
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

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// Two-pass selection, exact for m = topk - 1 <= 64; dispatched for m <= kSelectMaxM
// (see the top of the file).
template <int D, int S>
__global__ __launch_bounds__(256) void topk_select_kernel(const uint16_t* __restrict__ q, const float* __restrict__ km,
                                                          int32_t* __restrict__ idx, float* __restrict__ sel, int L,
                                                          int n, int BH, int topk, int G) {
  constexpr int NC = D / 32, NT = S / 16, RPW = S / 4;  // rows per wave
  // Scores of a chunk go to one of two buffers (chunk parity), so scoring the next chunk
  // never overwrites scores other waves may still read: one barrier per chunk.
  __shared__ float scb[2][S][65];
  __shared__ uint64_t buf[S][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
  const int nn = lane & 15;
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

  u32x4 qf[NT][NC];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) qf[nt][cc] = load_q_frag<D>(qh + (int64_t)(16 * nt + nn) * D, cc);
  const int nchunks = (qb + 63) / 64;
  // kbar of the next chunk to score, loaded one chunk ahead (after the last chunk of a
  // pass, chunk 0 again for the next pass)
  float xk[NC][8];
  load_kchunk<D>(kmh, 0, n, xk);

  // ---- pass 1: lane maxima of the score bits, and from them a lower bound on each
  // row's m-th key (the m lanes whose maximum reaches the m-th largest lane maximum t
  // hold m distinct keys with score bits >= t, so (t, 0) is at most the m-th key)
  uint32_t lmax[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) lmax[i] = 0;
  for (int chunk = 0; chunk < nchunks; ++chunk) {
    const int cb = chunk * 64;
    float (*sc)[65] = scb[chunk & 1];
    score_chunk<D, S>(qf, xk, sc);
    load_kchunk<D>(kmh, chunk + 1 < nchunks ? cb + 64 : 0, n, xk);
    __syncthreads();
    const int j = cb + lane;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = w + 4 * i;
      const uint32_t h = j < qb ? orderable_f32(sc[r][lane]) : 0u;
      lmax[i] = lmax[i] > h ? lmax[i] : h;
    }
  }
  __syncthreads();  // pass 2 scores chunk 0 into buffer 0 again
  uint64_t thr[RPW];
  bool act[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    thr[i] = (uint64_t)(uint32_t)__shfl((int)sort64_u32(lmax[i], false), m - 1) << 32;  // descending: lane m-1
    act[i] = true;
  }

  // ---- pass 2: collect the keys at or above the bound, in index order
  int cnt[RPW];
  for (;;) {
#pragma unroll
    for (int i = 0; i < RPW; ++i)
      if (act[i]) cnt[i] = 0;
    for (int chunk = 0; chunk < nchunks; ++chunk) {
      const int cb = chunk * 64;
      float (*sc)[65] = scb[chunk & 1];
      score_chunk<D, S>(qf, xk, sc);
      load_kchunk<D>(kmh, chunk + 1 < nchunks ? cb + 64 : 0, n, xk);
      __syncthreads();
      const int j = cb + lane;
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        if (!act[i]) continue;
        const int r = w + 4 * i;
        const uint64_t key = j < qb ? make_key(sc[r][lane], j) : 0ull;
        const bool pass = key >= thr[i];
        const uint64_t mask = __builtin_amdgcn_ballot_w64(pass);
        const int pos = cnt[i] + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
        if (pass && pos < 64) buf[r][pos] = key;
        cnt[i] += __builtin_popcountll(mask);
      }
    }
    __syncthreads();  // buf complete; a repeated pass scores chunk 0 into buffer 0 again
    // rows that collected more than 64 keys: raise the bound to the m-th largest of
    // the first 64 collected (a strictly higher bound) and collect again
    bool again = false;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      if (!act[i]) continue;
      if (cnt[i] > 64) {
        const int r = w + 4 * i;
        uint32_t t;
        int need;
        uint64_t eq;
        thr[i] = kth_key_index_ordered(buf[r][lane], m, &t, &need, &eq);  // the first 64, index order
        again = true;
      } else {
        act[i] = false;
      }
    }
    if (!__syncthreads_or(again)) break;
  }

  // ---- output: the m keys at or above the row's exact m-th key, in index order
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int r = w + 4 * i;
    const int c = cnt[i];
    const uint64_t y = lane < c ? buf[r][lane] : 0ull;
    uint32_t t;
    int need;
    uint64_t eq;
    (void)kth_key_index_ordered(y, m, &t, &need, &eq);
    // all keys with score bits above t, and the first `need` (lowest blocks) at t
    const uint32_t hi = (uint32_t)(y >> 32);
    const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0));
    const bool take = lane < c && (hi > t || (hi == t && rank < need));
    const uint64_t mask = __builtin_amdgcn_ballot_w64(take);
    const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
    int32_t* orow = ih + (int64_t)r * topk;
    float* srow = sh ? sh + (int64_t)r * topk : nullptr;
    if (take) {
      orow[pos] = key_index(y);
      if (srow) srow[pos] = key_score(y);
    }
    for (int p = m + lane; p < topk; p += 64) {
      orow[p] = p == m ? qb : -1;
      if (srow) srow[p] = p == m ? inf : -inf;
    }
  }
}

constexpr int kSelectMaxM = 40;  // largest m = topk - 1 given to the two-pass selection

static int e_for(int topk) {
  const int need = topk - 1;
  int e = 1;
  while (64 * e < need) e <<= 1;
  return e;
}

bool topk_mfma_supported(const Dims& d, int topk) {
  if (d.dtype != 1 || (d.D != 64 && d.D != 128)) return false;
  const int e = e_for(topk);
  return d.S * 64 * e <= 8192;  // running lists: S rows x KP keys x 8 bytes <= 64 KB
}

template <int D, int S>
static hipError_t run_select(const Dims& d, const void* q, const float* km, int topk, int32_t* idx, float* sel,
                             hipStream_t st) {
  const int64_t grid = (int64_t)d.n() * d.bh();
  hipLaunchKernelGGL((topk_select_kernel<D, S>), dim3((unsigned)grid), dim3(256), 0, st,
                     static_cast<const uint16_t*>(q), km, idx, sel, d.L, d.n(), (int)d.bh(), topk, d.G());
  return hipGetLastError();
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
  // Two-pass selection while its first bound is tight (m well below 64); above that the
  // bound from 64 lane maxima is weak, rows collect far more than 64 keys and refine
  // many times, so the sort-and-merge kernel is faster (measured: m = 39 select 1.68 ms
  // vs merge 1.93 ms; m = 47 select 2.25 ms vs merge 1.91 ms at L = 32768, 32 heads).
  if (topk - 1 <= kSelectMaxM) return d.S == 64 ? run_select<D, 64>(d, q, km, topk, idx, sel, st)
                                                 : run_select<D, 128>(d, q, km, topk, idx, sel, st);
  const int e = e_for(topk);
  if (e == 1) return d.S == 64 ? run_topk<D, 64, 1>(d, q, km, topk, idx, sel, st)
                                : run_topk<D, 128, 1>(d, q, km, topk, idx, sel, st);
  return run_topk<D, 64, 2>(d, q, km, topk, idx, sel, st);  // S = 128 with E = 2 is not supported
}

LaunchResult launch_topk_mfma(const Dims& d, const void* q, const float* km, int topk, int32_t* idx, float* sel,
                              hipStream_t st) {
  LaunchResult r;
  r.err = d.D == 128 ? dispatch_topk<128>(d, q, km, topk, idx, sel, st)
                     : dispatch_topk<64>(d, q, km, topk, idx, sel, st);
  return r;
}

}  // namespace ssa
