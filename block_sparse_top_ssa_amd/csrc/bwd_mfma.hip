// Backward of the dense causal stream on MFMA (bf16 in, float32 accumulate); the chain
// rule is the one stated in bwd.hip (training both streams, paper sec. 5, pp. 6-7).
//
// Two kernels, each keeping one side resident and streaming the other through LDS:
//
//  dk, dv (key-stationary): a workgroup of four waves owns 128 keys of a key/value
//  head, wave w keys 32w .. 32w+31 (two 16-key column tiles).  For every query head of
//  the group and every 64-row query chunk at or after the keys, per 32-row pair of row
//  tiles:
//      S  = Q K^T,  dP = dO V^T            (A = Q / dO rows from LDS, B = K / V rows held
//                                            in registers; lane = key column)
//      P  = exp2(S sl2 - lse2_row), dS = P (dP - delta_row)     (vector ALU)
//      dV^T += dO^T P,  dK^T += Q^T dS     (A = dO, Q in fragment order, B = P, dS packed
//                                            to bf16 straight from the S layout)
//  The fragment order (rows kappa-permuted, as in the forward's V^T) makes the S layout
//  of two row tiles exactly the B operand of the second pair of products, so P and dS
//  need no lane movement.
//
//  dq (query-stationary): a workgroup of eight waves (two per SIMD; four where L is not a
//  multiple of 256) owns 256 (128) query rows, wave w rows 32w .. 32w+31 (two 16-row
//  column tiles), and walks the 64-key chunks 0 .. its last row's chunk; each K / V
//  fragment read from LDS serves both row tiles, and the next chunk is staged in two
//  halves around the two groups of products:
//      S^T = K Q^T, dP^T = V dO^T          (A = K / V rows from LDS, B = Q / dO rows held)
//      P^T, dS^T as above
//      dQ^T += K^T dS^T                    (A = K in fragment order from LDS)
//
//  Operands of the next chunk are loaded into registers while the current one is
//  multiplied, then written to the other LDS stage (last read before the previous
//  barrier): one barrier per chunk.
//
//  The sparse stream: dk, dv visit only the rows that attend each block -- a workgroup
//  per (key/value head, block) walks the block's own rows (causally) and the rows that
//  kept it (an inverted index block -> rows), gathered 64 at a time; dq visits, for a
//  tile of rows, each attended block once with the rows that attend it (bwd_dq_gather.hip).
#include "launch.hpp"
#include "mfma.hpp"

namespace ssa {

namespace {

constexpr int kRows = 64;  // query rows per chunk (kernel dk/dv) and keys per chunk (kernel dq)

// A fragment of a row-major [.., D] bf16 matrix for lane l (any lane may load it):
// row key0 + l%16, columns 32 cc + 8 (l/16) .. +7.
template <int D>
__device__ __forceinline__ u32x4 load_k_frag_lane(const uint16_t* __restrict__ base, int key0, int cc, int l) {
  return load16(base + (int64_t)(key0 + (l & 15)) * D + 32 * cc + 8 * (l >> 4));
}

}  // namespace

// ---------------------------------------------------------------- dk, dv
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_kv_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const u32x4* __restrict__ qt, const u32x4* __restrict__ dot,
    const float* __restrict__ lse, const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv,
    int L, int G, int BHkv, float sl2, float scale) {
  constexpr int NC = D / 32, NDT = D / 16;
  constexpr int FQ = 4 * NC;          // A fragments of Q (and of dO) per 64-row chunk: 4 row tiles x NC
  constexpr int FT = 2 * NDT;         // fragment-order fragments per chunk: NDT x 2 row halves
  constexpr int NF = 2 * FQ + 2 * FT;  // per stage
  constexpr int PT = NF * 64 / 256;    // 16-byte pieces per thread per stage
  extern __shared__ __align__(16) unsigned char smem_kv[];
  u32x4* st = reinterpret_cast<u32x4*>(smem_kv);                     // [2][NF][64]
  float* sv = reinterpret_cast<float*>(smem_kv + 2 * NF * 64 * 16);  // [2][2][64]: lse2, delta

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int nkb = L / 128, nqc = L / kRows;
  const int kb = (int)(blockIdx.x / BHkv);  // key blocks with the most query rows first
  const int64_t kvbh = blockIdx.x - (int64_t)kb * BHkv;
  const int kw0 = kb * 128 + 32 * w;        // this wave's first key
  const uint16_t* kh = k + kvbh * (int64_t)L * D;
  const uint16_t* vh = v + kvbh * (int64_t)L * D;

  u32x4 kf[2][NC], vf[2][NC];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      kf[kt][cc] = load_k_frag<D>(kh, kw0 + 16 * kt, cc);
      vf[kt][cc] = load_k_frag<D>(vh, kw0 + 16 * kt, cc);
    }
  f32x4 dva[2][NDT], dka[2][NDT];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dva[kt][dt] = dka[kt][dt] = f32x4{0, 0, 0, 0};

  const int qc0 = kb * 2;                 // first query chunk that sees these keys
  const int per_head = nqc - qc0;
  const int items = G * per_head;
  (void)nkb;
  // staging registers of the next item, filled and stored in two halves (one per pair of
  // row tiles) to keep register pressure down
  constexpr int PH = PT / 2;
  u32x4 pr[PH];
  float ps = 0.f;
  auto load_half = [&](int it, int half) {
    const int gq = it / per_head, qc = qc0 + (it - gq * per_head);
    const int64_t bh = kvbh * G + gq;
    const int r0 = qc * kRows;
    const uint16_t* qh = q + bh * (int64_t)L * D;
    const uint16_t* dh = dout + bh * (int64_t)L * D;
    const int64_t fbase = (bh * nqc + qc) * (int64_t)FT;  // fragment-order index of (head, chunk)
#pragma unroll
    for (int i = 0; i < PH; ++i) {
      const int p = tid + 256 * (half * PH + i), f = p >> 6, ll = p & 63;
      if (f < 2 * FQ) {
        const int ff = f < FQ ? f : f - FQ, rt = ff / NC, cc = ff % NC;
        const uint16_t* src = (f < FQ ? qh : dh) + (int64_t)(r0 + 16 * rt + (ll & 15)) * D + 32 * cc + 8 * (ll >> 4);
        pr[i] = load16(src);
      } else {
        const int ff = f - 2 * FQ;
        pr[i] = ff < FT ? qt[(fbase + ff) * 64 + ll] : dot[(fbase + ff - FT) * 64 + ll];
      }
    }
    if (half == 0 && tid < 2 * kRows) {
      const int64_t row = bh * L + r0 + (tid & (kRows - 1));
      ps = tid < kRows ? lse[row] * kLog2e : delta[row];
    }
  };
  auto store_half = [&](int b, int half) {
#pragma unroll
    for (int i = 0; i < PH; ++i) st[(b * NF) * 64 + tid + 256 * (half * PH + i)] = pr[i];
    if (half == 0 && tid < 2 * kRows) sv[b * 2 * kRows + tid] = ps;
  };
  // rows 32 rc .. 32 rc + 31 of the chunk in stage b against this wave's keys
  auto compute_rc = [&](int b, int r0, int rc) {
    const u32x4* sb = st + b * NF * 64;
    const float* lse2 = sv + b * 2 * kRows;
    const float* dl = lse2 + kRows;
    f32x4 s[2][2], dp[2][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s[h][kt] = dp[h][kt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rt = 2 * rc + h;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const u32x4 aq = sb[(rt * NC + cc) * 64 + lane];
        const u32x4 ad = sb[(FQ + rt * NC + cc) * 64 + lane];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          s[h][kt] = mfma_bf16(aq, kf[kt][cc], s[h][kt]);
          dp[h][kt] = mfma_bf16(ad, vf[kt][cc], dp[h][kt]);
        }
      }
    }
    // element i of s[h][kt]: row r0 + 32 rc + 16 h + 4 g + i, key kw0 + 16 kt + n
    float pv[2][2][4], dsv[2][2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 32 * rc + 16 * h + 4 * g + i;
        const float l2 = lse2[rl], de = dl[rl];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const bool live = r0 + rl >= kw0 + 16 * kt + n;
          const float p = live ? fast_exp2(fmaf(s[h][kt][i], sl2, -l2)) : 0.f;
          pv[h][kt][i] = p;
          dsv[h][kt][i] = p * (dp[h][kt][i] - de);
        }
      }
    u32x4 pb[2], sbf[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      pb[kt] = pack_p(pv[0][kt], pv[1][kt]);
      sbf[kt] = pack_p(dsv[0][kt], dsv[1][kt]);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const u32x4 aqt = sb[(2 * FQ + dt * 2 + rc) * 64 + lane];
      const u32x4 adt = sb[(2 * FQ + FT + dt * 2 + rc) * 64 + lane];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        dva[kt][dt] = mfma_bf16(adt, pb[kt], dva[kt][dt]);
        dka[kt][dt] = mfma_bf16(aqt, sbf[kt], dka[kt][dt]);
      }
    }
  };

  load_half(0, 0);
  store_half(0, 0);
  load_half(0, 1);
  store_half(0, 1);
  __syncthreads();
  for (int it = 0; it < items; ++it) {
    const int b = it & 1;
    const int nxt = min(it + 1, items - 1);  // unconditional loads (a repeat on the last item)
    const int gq = it / per_head, qc = qc0 + (it - gq * per_head);
    const int r0 = qc * kRows;
    const bool live = r0 + kRows - 1 >= kw0;  // some row of the chunk sees some key of this wave
    // stage b ^ 1 was last read in the previous iteration, before its barrier
#pragma unroll
    for (int rc = 0; rc < 2; ++rc) {
      load_half(nxt, rc);
      if (live) compute_rc(b, r0, rc);
      store_half(b ^ 1, rc);
    }
    __syncthreads();
  }
  // dva[kt][dt] element i: d = 16 dt + 4 g + i, key kw0 + 16 kt + n
  float* dkh = dk + kvbh * (int64_t)L * D;
  float* dvh = dv + kvbh * (int64_t)L * D;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int64_t key = kw0 + 16 * kt + n;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f32x4* pk = reinterpret_cast<f32x4*>(dkh + key * D + 16 * dt + 4 * g);
      f32x4* pv = reinterpret_cast<f32x4*>(dvh + key * D + 16 * dt + 4 * g);
      *pk = *pk + dka[kt][dt] * scale;
      *pv = *pv + dva[kt][dt];
    }
  }
}

// ---------------------------------------------------------------- dq
// NW waves of 32 rows each (NW / 4 waves per SIMD)
template <int D, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void bwd_q_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const u32x4* __restrict__ kt_frag, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dq, int L, int G, int BH, float sl2, float scale) {
  constexpr int NC = D / 32, NDT = D / 16;
  constexpr int FK = 4 * NC;          // A fragments of K (and of V) per 64-key chunk
  constexpr int FT = 2 * NDT;         // fragment-order K^T fragments per chunk
  constexpr int NF = 2 * FK + FT;
  constexpr int NTH = 64 * NW, RB = 32 * NW;  // threads, rows per workgroup
  constexpr int PT = NF * 64 / NTH;  // staging pieces per thread: PH0 in the first half, the rest in the second
  constexpr int PH0 = (PT + 1) / 2;
  static_assert(NF * 64 % NTH == 0, "staging pieces per thread");
  extern __shared__ __align__(16) unsigned char smem_q[];
  u32x4* st = reinterpret_cast<u32x4*>(smem_q);  // [2][NF][64]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int nqb = L / RB, nck = L / 64;
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);  // row blocks with the most keys first
  const int64_t bh = blockIdx.x % BH;
  const int64_t kvbh = bh / G;
  const int rw0 = qb * RB + 32 * w;  // this wave's first row
  const uint16_t* qh = q + bh * (int64_t)L * D;
  const uint16_t* dh = dout + bh * (int64_t)L * D;
  const uint16_t* kh = k + kvbh * (int64_t)L * D;
  const uint16_t* vh = v + kvbh * (int64_t)L * D;

  u32x4 qf[2][NC], df[2][NC];
  float l2[2], de[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t row = rw0 + 16 * nt + n;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      qf[nt][cc] = load_q_frag<D>(qh + row * D, cc);
      df[nt][cc] = load_q_frag<D>(dh + row * D, cc);
    }
    l2[nt] = lse[bh * L + row] * kLog2e;
    de[nt] = delta[bh * L + row];
  }
  f32x4 dqa[2][NDT];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dqa[nt][dt] = f32x4{0, 0, 0, 0};

  const int items = (qb * RB + RB - 1) / 64 + 1;  // key chunks 0 .. the block's last row's chunk
  // The next chunk is staged in two halves, each loaded before and stored after one group
  // of products, so only half of the staging registers are live at a time.
  u32x4 pr[PH0];
  auto load_half = [&](int c, int half) {
#pragma unroll
    for (int i = 0; i < (half ? PT - PH0 : PH0); ++i) {
      const int p = tid + NTH * (half * PH0 + i), f = p >> 6, ll = p & 63;
      if (f < 2 * FK) {
        const int ff = f < FK ? f : f - FK, kt = ff / NC, cc = ff % NC;
        pr[i] = load_k_frag_lane<D>(f < FK ? kh : vh, c * 64 + 16 * kt, cc, ll);
      } else {
        pr[i] = kt_frag[((kvbh * nck + c) * (int64_t)FT + (f - 2 * FK)) * 64 + ll];
      }
    }
  };
  auto store_half = [&](int b, int half) {
#pragma unroll
    for (int i = 0; i < (half ? PT - PH0 : PH0); ++i) st[(b * NF) * 64 + tid + NTH * (half * PH0 + i)] = pr[i];
  };
  load_half(0, 0);
  store_half(0, 0);
  load_half(0, 1);
  store_half(0, 1);
  __syncthreads();
  for (int c = 0; c < items; ++c) {
    const int b = c & 1;
    const int cn = min(c + 1, items - 1);  // unconditional loads (a repeat at the end)
    const u32x4* sb = st + b * NF * 64;
    const int k0 = c * 64;
    const bool act = k0 <= rw0 + 31;  // some key of the chunk is at or before some row of this wave
    // S^T and dP^T: each fragment read from LDS feeds the products of both row tiles
    load_half(cn, 0);
    f32x4 sa[2][4], dp[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) sa[nt][kt] = dp[nt][kt] = f32x4{0, 0, 0, 0};
    if (act) {
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const u32x4 ak = sb[(kt * NC + cc) * 64 + lane];
          const u32x4 av = sb[(FK + kt * NC + cc) * 64 + lane];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            sa[nt][kt] = mfma_bf16(ak, qf[nt][cc], sa[nt][kt]);
            dp[nt][kt] = mfma_bf16(av, df[nt][cc], dp[nt][kt]);
          }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    store_half(b ^ 1, 0);
    // dS^T (element i of sa[nt][kt]: key k0 + 16 kt + 4 g + i, row rw0 + 16 nt + n), then
    // dQ^T += K^T dS^T
    load_half(cn, 1);
    if (act) {
      u32x4 bs[2][2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int row = rw0 + 16 * nt + n;
        float dsv[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool live = k0 + 16 * kt + 4 * g + i <= row;
            const float p = live ? fast_exp2(fmaf(sa[nt][kt][i], sl2, -l2[nt])) : 0.f;
            dsv[kt][i] = p * (dp[nt][kt][i] - de[nt]);
          }
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) bs[nt][kc] = pack_p(dsv[2 * kc], dsv[2 * kc + 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const u32x4 at = sb[(2 * FK + dt * 2 + kc) * 64 + lane];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) dqa[nt][dt] = mfma_bf16(at, bs[nt][kc], dqa[nt][dt]);
        }
    }
    store_half(b ^ 1, 1);
    __syncthreads();
  }
  // dqa[nt][dt] element i: d = 16 dt + 4 g + i, row rw0 + 16 nt + n
  float* dqh = dq + bh * (int64_t)L * D;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int64_t row = rw0 + 16 * nt + n;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f32x4* pq = reinterpret_cast<f32x4*>(dqh + row * D + 16 * dt + 4 * g);
      *pq = *pq + dqa[nt][dt] * scale;
    }
  }
}


// ---------------------------------------------------------------- sparse dk, dv (gathered rows)
// One workgroup per (key/value head, block j): wave w owns keys j*S + (S/4) w .. +S/4-1
// (S/64 column tiles).  The rows that attend block j are the rows of the block itself
// (causally) and the rows that kept it (from the inverted index); they are processed 64 at
// a time for every query head of the group.  The staging builds, for each gathered 64-row
// item, the A fragments of Q and dO (row-major rows) and of Q^T and dO^T in the kappa row
// order (16-byte loads of the gathered rows, then an 8x8 transpose of 16-bit values across
// 8 lanes), so the products are those of the dense kernel with gathered rows.
template <int D, int S>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_kv_sparse_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const int* __restrict__ off, const int* __restrict__ list, int topk, float* __restrict__ dk,
    float* __restrict__ dv, int L, int G, int BHkv, float sl2, float scale) {
  constexpr int NC = D / 32, NDT = D / 16, NKT = S / 64;
  constexpr int FQ = 4 * NC, FT = 2 * NDT, NF = 2 * FQ + 2 * FT, PT = NF * 64 / 256, PH = PT / 2;
  extern __shared__ __align__(16) unsigned char smem_ks[];
  u32x4* st = reinterpret_cast<u32x4*>(smem_ks);                     // [2][NF][64]
  float* sv = reinterpret_cast<float*>(smem_ks + 2 * NF * 64 * 16);  // [2][2][64]: lse2, delta
  int* srow = reinterpret_cast<int*>(sv + 2 * 2 * 64);               // [3][64]: row ids of items it % 3

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int nb = L / S;
  const int j = (int)(blockIdx.x / BHkv);
  const int64_t kvbh = blockIdx.x - (int64_t)j * BHkv;
  const int kw0 = j * S + (S / 4) * w;
  const uint16_t* kh = k + kvbh * (int64_t)L * D;
  const uint16_t* vh = v + kvbh * (int64_t)L * D;
  u32x4 kf[NKT][NC], vf[NKT][NC];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      kf[kt][cc] = load_k_frag<D>(kh, kw0 + 16 * kt, cc);
      vf[kt][cc] = load_k_frag<D>(vh, kw0 + 16 * kt, cc);
    }
  f32x4 dva[NKT][NDT], dka[NKT][NDT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) dva[kt][dt] = dka[kt][dt] = f32x4{0, 0, 0, 0};

  // items of query head gq: S/64 items of the block's own rows, then the kept-by list
  constexpr int OWN = S / 64;
  auto list_count = [&](int gq) {
    const int* o = off + (kvbh * G + gq) * (int64_t)(nb + 1);
    return o[j + 1] - o[j];
  };
  int items = 0;
  for (int gq = 0; gq < G; ++gq) items += OWN + (list_count(gq) + 63) / 64;
  struct Item {
    int64_t bh;
    int ii, first, cnt;  // item index within the head, first list entry, list length
  };
  auto item_of = [&](int it) {
    Item x;
    int gq = 0;
    for (;; ++gq) {
      const int c = list_count(gq), ni = OWN + (c + 63) / 64;
      if (it < ni || gq == G - 1) {
        x.bh = kvbh * G + gq;
        x.ii = it;
        x.cnt = c;
        x.first = off[(kvbh * G + gq) * (int64_t)(nb + 1) + j];
        return x;
      }
      it -= ni;
    }
  };
  // row of position r (0..63) of an item; -1 past the end of the list.  The row ids of
  // item it + 2 are fetched during item it and kept in LDS (srow[(it + 2) % 3]), so the
  // operand loads of item it + 1 read their rows from LDS, not behind a list lookup.
  auto row_of = [&](const Item& x, int r) -> int {
    if (x.ii < OWN) return j * S + 64 * x.ii + r;
    const int e = (x.ii - OWN) * 64 + r;
    return e < x.cnt ? list[x.bh * (int64_t)L * topk + x.first + e] : -1;
  };

  u32x4 pr[PH];  // staging registers for one half of the next item
  float ps = 0.f;
  auto load_half = [&](const Item& x, const int* rows, int half) {
    const uint16_t* qh = q + x.bh * (int64_t)L * D;
    const uint16_t* dh = dout + x.bh * (int64_t)L * D;
#pragma unroll
    for (int i = 0; i < PH; ++i) {
      const int f = (tid >> 6) + 4 * (half * PH + i);  // uniform per wave; lane = tid & 63
      if (f < 2 * FQ) {
        const int ff = f < FQ ? f : f - FQ, rt = ff / NC, cc = ff % NC;
        const int row = max(rows[16 * rt + n], 0);
        pr[i] = load16((f < FQ ? qh : dh) + (int64_t)row * D + 32 * cc + 8 * g);
      } else {
        const int ff = (f - 2 * FQ) % FT, dt = ff >> 1, rc = ff & 1;
        const int h8 = (lane >> 3) & 1, p8 = lane & 7;
        const int row = max(rows[kappa(rc, g, p8)], 0);
        pr[i] = transpose8x8_b16_dpp(
            load16((f < 2 * FQ + FT ? qh : dh) + (int64_t)row * D + 16 * dt + 8 * h8));
      }
    }
    if (half == 0 && tid < 128) {
      const int row = rows[tid & 63];
      const int64_t gr = x.bh * L + max(row, 0);
      if (tid < 64) ps = row < 0 ? __builtin_huge_valf() : lse[gr] * kLog2e;
      else ps = row < 0 ? 0.f : delta[gr];
    }
  };
  auto store_half = [&](int b, int half) {
#pragma unroll
    for (int i = 0; i < PH; ++i) st[(b * NF + (tid >> 6) + 4 * (half * PH + i)) * 64 + lane] = pr[i];
    if (half == 0 && tid < 128) sv[b * 128 + tid] = ps;
  };
  auto compute_rc = [&](int b, const int* rows, int rc, bool causal) {
    const u32x4* sb = st + b * NF * 64;
    const float* lse2 = sv + b * 128;
    const float* dl = lse2 + 64;
    f32x4 sa[2][NKT], dp[2][NKT];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) sa[h][kt] = dp[h][kt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rt = 2 * rc + h;
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        const u32x4 aq = sb[(rt * NC + cc) * 64 + lane];
        const u32x4 ad = sb[(FQ + rt * NC + cc) * 64 + lane];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          sa[h][kt] = mfma_bf16(aq, kf[kt][cc], sa[h][kt]);
          dp[h][kt] = mfma_bf16(ad, vf[kt][cc], dp[h][kt]);
        }
      }
    }
    float pv[2][NKT][4], dsv[2][NKT][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rl = 32 * rc + 16 * h + 4 * g + i;
        const int row = rows[rl];
        const float l2 = lse2[rl], de = dl[rl];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const bool live = row >= 0 && (!causal || row >= kw0 + 16 * kt + n);
          const float p = live ? fast_exp2(fmaf(sa[h][kt][i], sl2, -l2)) : 0.f;
          pv[h][kt][i] = p;
          dsv[h][kt][i] = p * (dp[h][kt][i] - de);
        }
      }
    u32x4 pb[NKT], sbf[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      pb[kt] = pack_p(pv[0][kt], pv[1][kt]);
      sbf[kt] = pack_p(dsv[0][kt], dsv[1][kt]);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const u32x4 aqt = sb[(2 * FQ + dt * 2 + rc) * 64 + lane];
      const u32x4 adt = sb[(2 * FQ + FT + dt * 2 + rc) * 64 + lane];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        dva[kt][dt] = mfma_bf16(adt, pb[kt], dva[kt][dt]);
        dka[kt][dt] = mfma_bf16(aqt, sbf[kt], dka[kt][dt]);
      }
    }
  };

  {
    const Item x0 = item_of(0), x1 = item_of(min(1, items - 1));
    if (tid < 64) srow[tid] = row_of(x0, tid);
    else if (tid < 128) srow[64 + tid - 64] = row_of(x1, tid - 64);
    __syncthreads();
    load_half(x0, srow, 0);
    store_half(0, 0);
    load_half(x0, srow, 1);
    store_half(0, 1);
  }
  __syncthreads();
  for (int it = 0; it < items; ++it) {
    const int b = it & 1;
    const Item cur = item_of(it);
    const Item nxt = item_of(min(it + 1, items - 1));  // unconditional (a repeat at the end)
    int nid = -1;
    if (tid >= 192) nid = row_of(item_of(min(it + 2, items - 1)), tid - 192);
    const int* rows_cur = srow + (it % 3) * 64;
    const int* rows_nxt = srow + ((it + 1) % 3) * 64;
#pragma unroll
    for (int rc = 0; rc < 2; ++rc) {
      load_half(nxt, rows_nxt, rc);
      compute_rc(b, rows_cur, rc, cur.ii < OWN);
      store_half(b ^ 1, rc);
    }
    // srow[(it + 2) % 3] held item it - 1's rows, last read before the previous barrier
    if (tid >= 192) srow[((it + 2) % 3) * 64 + tid - 192] = nid;
    __syncthreads();
  }
  float* dkh = dk + kvbh * (int64_t)L * D;
  float* dvh = dv + kvbh * (int64_t)L * D;
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const int64_t key = kw0 + 16 * kt + n;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      f32x4* pk = reinterpret_cast<f32x4*>(dkh + key * D + 16 * dt + 4 * g);
      f32x4* pv = reinterpret_cast<f32x4*>(dvh + key * D + 16 * dt + 4 * g);
      *pk = *pk + dka[kt][dt] * scale;
      *pv = *pv + dva[kt][dt];
    }
  }
}

// ---------------------------------------------------------------- launcher
bool full_bwd_mfma_supported(const Dims& d) {
  return d.dtype == 1 && (d.D == 64 || d.D == 128) && d.L % 128 == 0;
}

bool sparse_bwd_mfma_supported(const Dims& d, int topk) {
  return full_bwd_mfma_supported(d) && dq_gather_supported(d, topk);
}

// Bit j of word j / 32 of row t's mask: the sparse stream attends block j (a valid kept
// entry of idx, or the own block).  One thread per (row, word).
__global__ __launch_bounds__(256) void bwd_mask_kernel(const int32_t* __restrict__ idx, int topk,
                                                       uint32_t* __restrict__ mask, int64_t rows, int W, int L,
                                                       int s) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * W) return;
  const int64_t row = i / W;
  const int wd = (int)(i - row * W);
  const int t = (int)(row % L), bt = t / s;
  uint32_t m = 0;
  auto set = [&](int j) {
    if (j / 32 == wd) m |= 1u << (j % 32);
  };
  set(bt);
  const int32_t* ir = idx + row * topk;
  int prev = -1;
  for (int e = 0; e < topk; ++e) {
    const int j = ir[e];
    if (j > prev && j < bt) {
      prev = j;
      set(j);
    }
  }
  mask[i] = m;
}

hipError_t build_block_mask(const Dims& d, const int32_t* idx, int topk, uint32_t* mask, hipStream_t st) {
  const int W = (d.n() + 31) / 32;
  const int64_t n = d.tokens() * W;
  hipLaunchKernelGGL(bwd_mask_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, idx, topk, mask, d.tokens(),
                     W, d.L, d.S);
  return hipGetLastError();
}

template <int D, bool SPARSE>
static hipError_t run_full_bwd_mfma(const Dims& d, const void* q, const void* k, const void* v, const void* dout,
                                    const float* lse, const float* delta, const int32_t* idx, const int* off,
                                    const int* list, int topk, float scale, float* dq, float* dk, float* dv,
                                    u32x4* qt, u32x4* dot, u32x4* ktf, hipStream_t st) {
  constexpr int NC = D / 32, NDT = D / 16;
  const Dims kv = d.kv();
  hipError_t e = hipSuccess;
  if (!SPARSE) {
    e = frag_order_into(d, q, qt, st);
    if (e == hipSuccess) e = frag_order_into(d, dout, dot, st);
  }
  if (e == hipSuccess) e = frag_order_into(kv, k, ktf, st);
  if (e != hipSuccess) return e;
  const float sl2 = scale * kLog2e;
  if constexpr (SPARSE) {  // dk, dv over the gathered rows of each block
    constexpr int NF = 2 * (4 * NC) + 2 * (2 * NDT);
    const int lds = 2 * NF * 64 * 16 + 2 * 2 * 64 * 4 + 3 * 64 * 4;
    auto kern = d.S == 64 ? bwd_kv_sparse_mfma_kernel<D, 64> : bwd_kv_sparse_mfma_kernel<D, 128>;
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    const int64_t grid = (int64_t)kv.bh() * d.n();
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                       static_cast<const uint16_t*>(dout), lse, delta, off, list, topk, dk, dv, d.L, d.G(),
                       (int)kv.bh(), sl2, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    constexpr int NF = 2 * (4 * NC) + 2 * (2 * NDT);
    const int lds = 2 * NF * 64 * 16 + 2 * 2 * 64 * 4;
    auto kern = bwd_kv_mfma_kernel<D>;
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    const int64_t grid = (int64_t)kv.bh() * (d.L / 128);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                       static_cast<const uint16_t*>(dout), qt, dot, lse, delta, dk, dv, d.L, d.G(), (int)kv.bh(),
                       sl2, scale);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (SPARSE) {
    e = launch_dq_gather(d, q, k, v, dout, ktf, lse, delta, idx, topk, scale, dq, st);
  } else {
    constexpr int NF = 2 * (4 * NC) + 2 * NDT;
    const int lds = 2 * NF * 64 * 16;
    // 256 rows (two waves per SIMD) where L allows, else 128
    const bool wide = d.L % 256 == 0;
    auto kern = wide ? bwd_q_mfma_kernel<D, 8> : bwd_q_mfma_kernel<D, 4>;
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    const int64_t grid = d.bh() * (d.L / (wide ? 256 : 128));
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(wide ? 512 : 256), lds, st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                       static_cast<const uint16_t*>(dout), ktf, lse, delta, dq, d.L, d.G(), (int)d.bh(), sl2, scale);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_full_bwd_mfma(const Dims& d, const int32_t* idx, int topk, const int* off, const int* list,
                                const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                const float* delta, float scale, float* dq, float* dk, float* dv, hipStream_t st) {
  // fragment-order copies of K (key/value heads) and, for the dense stream, of Q and dO
  const size_t qbytes = idx ? 0 : (size_t)d.tokens() * d.D * 2, kbytes = (size_t)d.kv().tokens() * d.D * 2;
  void* ws = nullptr;
  hipError_t e = workspace_alloc(2 * qbytes + kbytes, &ws, st);
  if (e != hipSuccess) return e;
  char* base = static_cast<char*>(ws);
  u32x4* qt = reinterpret_cast<u32x4*>(base);
  u32x4* dot = reinterpret_cast<u32x4*>(base + qbytes);
  u32x4* ktf = reinterpret_cast<u32x4*>(base + 2 * qbytes);
  if (idx)
    e = d.D == 128 ? run_full_bwd_mfma<128, true>(d, q, k, v, dout, lse, delta, idx, off, list, topk, scale, dq, dk,
                                                  dv, qt, dot, ktf, st)
                   : run_full_bwd_mfma<64, true>(d, q, k, v, dout, lse, delta, idx, off, list, topk, scale, dq, dk,
                                                 dv, qt, dot, ktf, st);
  else
    e = d.D == 128 ? run_full_bwd_mfma<128, false>(d, q, k, v, dout, lse, delta, nullptr, nullptr, nullptr, 1, scale,
                                                   dq, dk, dv, qt, dot, ktf, st)
                   : run_full_bwd_mfma<64, false>(d, q, k, v, dout, lse, delta, nullptr, nullptr, nullptr, 1, scale,
                                                  dq, dk, dv, qt, dot, ktf, st);
  const hipError_t fe = workspace_free(ws, st);
  return e != hipSuccess ? e : fe;
}

}  // namespace ssa
