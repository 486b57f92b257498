// dq of the sparse stream on MFMA bf16, over gathered rows (training both streams, paper
// sec. 5, pp. 6-7; the chain rule as stated in bwd.hip): dq_t = scale sum_{i in A(t)} ds_ti k_i
// with A(t) the tokens of row t's kept blocks and, causally, of its own block.
//
// Neighbouring rows attend largely different blocks, so a query-stationary sweep over
// every earlier chunk would do the dense amount of work under a mask.  This kernel is
// organised like the sparse forward (sparse_mfma.hip): a workgroup owns T consecutive
// query rows of one (b, h), keeps their dQ state (float32) in LDS, and visits every key
// block that some of its rows attend exactly once, multiplying only those rows (gathered
// into 16-row MFMA column tiles).  Two things are simpler than in the forward: p comes
// from the forward's log-sum-exp (no exponent reference, no recompute), and a row's own
// block is one more entry of the block -> rows index, masked per element (key <= row).
//
//  1. inverted index: per block the rows of the tile that attend it (LDS, a byte per
//     entry);
//  2. lockstep rounds of two roles per SIMD (one barrier per round, slots double-buffered):
//     * four score waves take the blocks j = s (mod 4) in ascending order and, per round,
//       one 16-row tile of the rows attending the current 64-key chunk:
//           S^T = K Q^T,  dP^T = V dO^T,  P^T = exp2(S^T sl2 - lse2_row),
//           dS^T = P^T (dP^T - delta_row)  rounded to bf16 -> the wave's slot;
//     * four value waves each own 32 columns of dQ for every row; per round they read the
//       four slots of the previous round and add dQ^T += K^T dS^T for their columns (K^T
//       from a copy of K in fragment order) with plain 16-byte read-add-write, slot after
//       slot (a row can sit in several slots of a round);
//  3. dq[t] += scale dQ[t].
#include "launch.hpp"
#include "mfma.hpp"

namespace ssa {

namespace {

constexpr int kDqSlotBytes = 2128;  // dS^T fragments (2 KB), 16 row ids, chunk ids

struct DqSlot {
  u32x4 p[2][64];
  int rows[16];
  int chunk, next_chunk, pad0, pad1;
};
static_assert(sizeof(DqSlot) == kDqSlotBytes, "slot layout");

struct DqLds {
  int dqs, l2, de, off, misc, slots, list, total;  // byte offsets inside the dynamic LDS block
};

// nb: blocks a row of the tile may attend (those up to the last row's own block)
template <int D>
__host__ __device__ inline DqLds dq_lds_layout(int T, int nb, int topk) {
  DqLds s;
  int o = 0;
  s.dqs = o;  o += T * D * 4;  // dQ state, rows of D floats, 16-byte granules XOR-swizzled by row
  s.l2 = o;   o += T * 4;      // lse of the row in log2 units
  s.de = o;   o += T * 4;      // delta of the row
  s.off = o;  o += (nb + 1) * 4;
  s.misc = o; o += 32;
  o = (o + 15) & ~15;
  s.slots = o;  // 2 sets x 4 slots; the per-block counters of the index build live here first
  o += 8 * kDqSlotBytes > nb * 4 ? 8 * kDqSlotBytes : nb * 4;
  s.list = o;  o += T * (topk + 1);  // up to topk kept blocks and the own block per row
  s.total = (o + 15) & ~15;
  return s;
}

template <int D>
__device__ __forceinline__ int dq_granule(int r, int d) {
  return r * D + ((((d >> 2) ^ (r & 15))) << 2);
}

constexpr int kMaxLds = 160 * 1024 - 256;  // room for the static LDS of the scan

}  // namespace

template <int D, int S, int T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_gather_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const u32x4* __restrict__ ktf, const float* __restrict__ lse,
    const float* __restrict__ delta, const int32_t* __restrict__ idx, int topk, float* __restrict__ dq, int L,
    int ntile, float sl2, float scale, int G) {
  constexpr int NW = 8, NTH = 512;
  constexpr int NC = D / 32, NDT = D / 16, CPB = S / 64;
  constexpr int DTW = NDT / 4;  // d tiles per value wave
  extern __shared__ __align__(16) unsigned char smem_dq[];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  // head-major order, the tiles with the most blocks first (as in the forward)
  const int64_t wg = xcd_logical(blockIdx.x, (int64_t)gridDim.x);
  const int64_t bh = wg / ntile;
  const int tile = ntile - 1 - (int)(wg % ntile);
  const int t0 = tile * T;
  const int rows = min(T, L - t0);
  const int nb = (t0 + rows - 1) / S + 1;  // blocks 0 .. the last row's own block
  const DqLds lay = dq_lds_layout<D>(T, nb, topk);
  float* dqs = reinterpret_cast<float*>(smem_dq + lay.dqs);
  float* l2s = reinterpret_cast<float*>(smem_dq + lay.l2);
  float* des = reinterpret_cast<float*>(smem_dq + lay.de);
  int* cnt = reinterpret_cast<int*>(smem_dq + lay.slots);  // index build only
  int* off = reinterpret_cast<int*>(smem_dq + lay.off);
  int* misc = reinterpret_cast<int*>(smem_dq + lay.misc);
  DqSlot* slots = reinterpret_cast<DqSlot*>(smem_dq + lay.slots);  // [2][4]: set, score wave
  uint8_t* list = smem_dq + lay.list;

  const uint16_t* qh = q + bh * (int64_t)L * D;
  const uint16_t* dh = dout + bh * (int64_t)L * D;
  const int64_t kvh = bh / G;
  const uint16_t* kh = k + kvh * (int64_t)L * D;
  const uint16_t* vh = v + kvh * (int64_t)L * D;
  const u32x4* kth = ktf + kvh * (int64_t)(L / 64) * NDT * 2 * 64;
  const int32_t* ih = idx + bh * (int64_t)L * topk;
  auto kt_frag = [&](int c, int dt, int kc) -> u32x4 { return kth[((int64_t)(c * NDT + dt) * 2 + kc) * 64 + lane]; };

  // Blocks attended by row t = t0 + tid: the valid kept entries (distinct, below b_t,
  // each greater than the entry used before it: the forward's rule) and then b_t itself.
  // Rows of at most 32 entries are read once into registers (two entries per register as
  // 16-bit values; values outside [0, 2^15) are never valid here and become -1) and walked
  // from there by both passes of the index build; longer rows are re-read in batches.
  const bool idx_regs = topk <= 32 && L / S < 32768;
  const bool idx_vec = idx_regs && topk % 4 == 0 && ((reinterpret_cast<uintptr_t>(ih) & 15) == 0);
  auto pack16 = [](int32_t a, int32_t b) -> uint32_t {
    const uint32_t ua = (a >= 0 && a < 32768) ? (uint32_t)a : 0xFFFFu;
    const uint32_t ub = (b >= 0 && b < 32768) ? (uint32_t)b : 0xFFFFu;
    return ua | (ub << 16);
  };
  uint32_t ent[16];
  if (idx_regs && tid < rows) {
    const int32_t* ir = ih + (int64_t)(t0 + tid) * topk;
    if (idx_vec) {
#pragma unroll
      for (int u4 = 0; u4 < 8; ++u4) {
        u32x4 x = u32x4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
        if (4 * u4 < topk) x = *reinterpret_cast<const u32x4*>(ir + 4 * u4);
        ent[2 * u4] = pack16((int32_t)x[0], (int32_t)x[1]);
        ent[2 * u4 + 1] = pack16((int32_t)x[2], (int32_t)x[3]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < 16; ++u) ent[u] = pack16(2 * u < topk ? ir[2 * u] : -1, 2 * u + 1 < topk ? ir[2 * u + 1] : -1);
    }
  }
  auto for_each_block = [&](int t, auto&& fn) {
    const int bt = t / S;
    int prev = -1;
    if (idx_regs) {
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int j = (int)(int16_t)(ent[u >> 1] >> (16 * (u & 1)));
        if (j > prev && j < bt) {
          prev = j;
          fn(j);
        }
      }
    } else {
      const int32_t* ir = ih + (int64_t)t * topk;
      for (int e0 = 0; e0 < topk; e0 += 32) {
        int jj[32];
#pragma unroll
        for (int u = 0; u < 32; ++u) jj[u] = e0 + u < topk ? ir[e0 + u] : -1;
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          const int j = jj[u];
          if (j > prev && j < bt) {
            prev = j;
            fn(j);
          }
        }
      }
    }
    fn(bt);
  };

  // ---------------------------------------------------------------- 1. inverted index
  for (int j = tid; j < nb; j += NTH) cnt[j] = 0;
  for (int r = tid; r < rows; r += NTH) {
    l2s[r] = lse[bh * (int64_t)L + t0 + r] * kLog2e;
    des[r] = delta[bh * (int64_t)L + t0 + r];
  }
  for (int i = tid; i < T * D / 4; i += NTH) reinterpret_cast<f32x4*>(dqs)[i] = f32x4{0, 0, 0, 0};
  __syncthreads();
  if (tid < rows) for_each_block(t0 + tid, [&](int j) { atomicAdd(&cnt[j], 1); });
  __syncthreads();
  {  // exclusive prefix sum of cnt[0..nb) into off[0..nb]; thread-contiguous segments
    const int seg = (nb + NTH - 1) / NTH;
    const int b0 = min(nb, tid * seg), b1 = min(nb, b0 + seg);
    int local = 0;
    for (int j = b0; j < b1; ++j) local += cnt[j];
    int incl = local;
#pragma unroll
    for (int o2 = 1; o2 < 64; o2 <<= 1) {
      const int y = __shfl_up(incl, o2);
      if (lane >= o2) incl += y;
    }
    __shared__ int wsum[NW];
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < w; ++i) base += wsum[i];
    int run = base + incl - local;
    for (int j = b0; j < b1; ++j) {
      off[j] = run;
      run += cnt[j];
    }
    if (tid == NTH - 1) off[nb] = base + incl;
  }
  __syncthreads();
  for (int j = tid; j < nb; j += NTH) cnt[j] = off[j];  // cnt becomes the fill cursor
  __syncthreads();
  if (tid < rows) for_each_block(t0 + tid, [&](int j) { list[atomicAdd(&cnt[j], 1)] = (uint8_t)tid; });
  __syncthreads();  // (the order of a block's rows only sets the order of float additions)
  // ---------------------------------------------------------------- 2. lockstep rounds
  auto next_block = [&](int from) -> int {  // next non-empty block >= from, same residue
    int j = from;
    while (j < nb && off[j + 1] == off[j]) j += 4;
    return j < nb ? j : nb;
  };
  if (w < 4) {  // items of score wave w: tiles of the blocks j = w (mod 4), all lanes counting
    int items = 0;
    for (int j = w + 4 * lane; j < nb; j += 256) items += CPB * ((off[j + 1] - off[j] + 15) / 16);
#pragma unroll
    for (int o2 = 32; o2 > 0; o2 >>= 1) items += __shfl_xor(items, o2);
    if (lane == 0) misc[w] = items;
  }
  __syncthreads();
  const int my_items = w < 4 ? misc[w] : 0;
  const int rounds = max(max(misc[0], misc[1]), max(misc[2], misc[3]));

  int j = w < 4 ? next_block(w) : nb, ch = 0, it = 0, r_cur = -1;
  // ra: a score wave's K fragments of its current chunk, a value wave's K^T fragments;
  // rb: a score wave's V fragments
  constexpr int RA = 4 * NC > 8 * DTW ? 4 * NC : 8 * DTW;
  u32x4 ra[RA], rb[4 * NC], qf[NC], df[NC];
  u32x4 pub0 = u32x4{0, 0, 0, 0}, pub1 = u32x4{0, 0, 0, 0};
  int pub_r = -1, pub_c = -1, pub_nc = -1;
  int scored = 0;
  auto load_item = [&](bool new_chunk) {
    const int beg = off[j], count = off[j + 1] - beg;
    const int e = it * 16 + n;
    r_cur = e < count ? (int)list[beg + e] : -1;
    if (new_chunk) {
      const int c = j * CPB + ch;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
          ra[kt * NC + cc] = load_k_frag<D>(kh, c * 64 + 16 * kt, cc);
          rb[kt * NC + cc] = load_k_frag<D>(vh, c * 64 + 16 * kt, cc);
        }
    }
    const int64_t row = t0 + (r_cur < 0 ? 0 : r_cur);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      qf[cc] = load_q_frag<D>(qh + row * D, cc);
      df[cc] = load_q_frag<D>(dh + row * D, cc);
    }
  };
  auto score_item = [&]() {
    const int r = r_cur;
    const int c = j * CPB + ch;
    f32x4 sacc[4], dacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = dacc[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) {
        sacc[kt] = mfma_bf16(ra[kt * NC + cc], qf[cc], sacc[kt]);
        dacc[kt] = mfma_bf16(rb[kt * NC + cc], df[cc], dacc[kt]);
      }
    }
    // element i of sacc[kt]: key 64 c + 16 kt + 4 g + i, row r (column n)
    const float l2 = r >= 0 ? l2s[r] : __builtin_huge_valf();  // no row: every p is 0
    const float de = r >= 0 ? des[r] : 0.f;
    const int tq = t0 + r;
    float ds[16];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool live = 64 * c + 16 * kt + 4 * g + i <= tq;
        const float p = live ? fast_exp2(fmaf(sacc[kt][i], sl2, -l2)) : 0.f;
        ds[kt * 4 + i] = p * (dacc[kt][i] - de);
      }
    pub0 = pack_p(&ds[0], &ds[4]);
    pub1 = pack_p(&ds[8], &ds[12]);
    pub_r = r;
    pub_c = c;
    // advance to the next tile and issue its loads (scored next round)
    const int ntl = (off[j + 1] - off[j] + 15) / 16;
    bool new_chunk = false;
    if (++it == ntl) {
      it = 0;
      new_chunk = true;
      if (++ch == CPB) {
        ch = 0;
        j = next_block(j + 4);
      }
    }
    ++scored;
    const bool more = scored < my_items;
    pub_nc = more ? j * CPB + ch : -1;
    if (more) load_item(new_chunk);
  };
  if (w < 4 && my_items > 0) {
    load_item(true);
    score_item();
  }
  const int pw = w - 4;
  int vchunk[4] = {-1, -1, -1, -1};
  auto load_kt = [&](int s, int c) {
#pragma unroll
    for (int dl = 0; dl < DTW; ++dl)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) ra[(s * DTW + dl) * 2 + kc] = kt_frag(c, pw * DTW + dl, kc);
  };
  auto publish = [&](int set, bool have) {
    DqSlot& sl = slots[set * 4 + w];
    if (have) {
      sl.p[0][lane] = pub0;
      sl.p[1][lane] = pub1;
      if (g == 0) sl.rows[n] = pub_r;
    }
    if (lane == 0) {
      sl.chunk = have ? pub_c : -1;
      sl.next_chunk = have ? pub_nc : -1;
    }
  };
  if (w < 4) publish(0, my_items > 0);
  __syncthreads();
  // Round rd: the value waves fold slot set rd % 2 while the score waves fill the other.
  if (w < 4) {
    for (int rd = 0; rd < rounds; ++rd) {
      const bool more = rd + 1 < my_items;
      if (more) score_item();
      publish((rd + 1) & 1, more);
      __syncthreads();
    }
  } else {
    for (int rd = 0; rd < rounds; ++rd) {
      const DqSlot* const cs = slots + (rd & 1) * 4;
      int sc[4], sn[4], sr[4];
      u32x4 sp[4][2];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sc[s] = __builtin_amdgcn_readfirstlane(cs[s].chunk);
        sn[s] = __builtin_amdgcn_readfirstlane(cs[s].next_chunk);
        sr[s] = cs[s].rows[n];
        sp[s][0] = cs[s].p[0][lane];
        sp[s][1] = cs[s].p[1][lane];
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (sc[s] >= 0 && sc[s] != vchunk[s]) {  // first tile of a stream: not prefetched
          load_kt(s, sc[s]);
          vchunk[s] = sc[s];
        }
      }
      f32x4 acc[4][DTW];
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int dl = 0; dl < DTW; ++dl) {
          acc[s][dl] = mfma_bf16(ra[(s * DTW + dl) * 2], sp[s][0], f32x4{0, 0, 0, 0});
          acc[s][dl] = mfma_bf16(ra[(s * DTW + dl) * 2 + 1], sp[s][1], acc[s][dl]);
        }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (sc[s] >= 0 && sn[s] >= 0 && sn[s] != sc[s]) {
          load_kt(s, sn[s]);  // used next round
          vchunk[s] = sn[s];
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = sr[s];
        if (sc[s] >= 0 && r >= 0) {
          f32x4 cv[DTW];
          f32x4* gp[DTW];
#pragma unroll
          for (int dl = 0; dl < DTW; ++dl) {
            gp[dl] = reinterpret_cast<f32x4*>(dqs + dq_granule<D>(r, 16 * (pw * DTW + dl) + 4 * g));
            cv[dl] = *gp[dl];
          }
#pragma unroll
          for (int dl = 0; dl < DTW; ++dl) *gp[dl] = cv[dl] + acc[s][dl];
        }
      }
      __syncthreads();
    }
  }

  // ---------------------------------------------------------------- 3. dq += scale dQ
  float* dqh = dq + (bh * (int64_t)L + t0) * D;
  for (int i = tid; i < rows * (D / 4); i += NTH) {
    const int r = i / (D / 4), c4 = i % (D / 4);
    const f32x4 a = *reinterpret_cast<const f32x4*>(dqs + dq_granule<D>(r, 4 * c4));
    f32x4* p = reinterpret_cast<f32x4*>(dqh + (int64_t)r * D + 4 * c4);
    *p = *p + a * scale;
  }
}

namespace {

template <int D>
int dq_pick_tile(const Dims& d, int topk) {
  for (int T : {256, 128})
    if (dq_lds_layout<D>(T, d.n(), topk).total <= kMaxLds) return T;
  return 0;
}

template <int D, int S, int T>
hipError_t run_dq_gather(const Dims& d, const void* q, const void* k, const void* v, const void* dout,
                         const u32x4* ktf, const float* lse, const float* delta, const int32_t* idx, int topk,
                         float scale, float* dq, hipStream_t st) {
  const int ntile = (d.L + T - 1) / T;
  const int64_t grid = (int64_t)ntile * d.bh();
  const int lds = dq_lds_layout<D>(T, d.n(), topk).total;
  auto kern = bwd_dq_gather_kernel<D, S, T>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, st, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(dout), ktf, lse, delta, idx, topk, dq, d.L, ntile, scale * kLog2e,
                     scale, d.G());
  return hipGetLastError();
}

template <int D, int S>
hipError_t dq_dispatch_t(const Dims& d, const void* q, const void* k, const void* v, const void* dout,
                         const u32x4* ktf, const float* lse, const float* delta, const int32_t* idx, int topk,
                         float scale, float* dq, hipStream_t st) {
  if (dq_pick_tile<D>(d, topk) == 256)
    return run_dq_gather<D, S, 256>(d, q, k, v, dout, ktf, lse, delta, idx, topk, scale, dq, st);
  return run_dq_gather<D, S, 128>(d, q, k, v, dout, ktf, lse, delta, idx, topk, scale, dq, st);
}

}  // namespace

bool dq_gather_supported(const Dims& d, int topk) {
  if (d.dtype != 1 || (d.D != 64 && d.D != 128) || d.L % 64 || (d.S != 64 && d.S != 128)) return false;
  return (d.D == 128 ? dq_pick_tile<128>(d, topk) : dq_pick_tile<64>(d, topk)) > 0;
}

hipError_t launch_dq_gather(const Dims& d, const void* q, const void* k, const void* v, const void* dout,
                            const u32x4* ktf, const float* lse, const float* delta, const int32_t* idx, int topk,
                            float scale, float* dq, hipStream_t st) {
  if (d.D == 128)
    return d.S == 64 ? dq_dispatch_t<128, 64>(d, q, k, v, dout, ktf, lse, delta, idx, topk, scale, dq, st)
                     : dq_dispatch_t<128, 128>(d, q, k, v, dout, ktf, lse, delta, idx, topk, scale, dq, st);
  return d.S == 64 ? dq_dispatch_t<64, 64>(d, q, k, v, dout, ktf, lse, delta, idx, topk, scale, dq, st)
                   : dq_dispatch_t<64, 128>(d, q, k, v, dout, ktf, lse, delta, idx, topk, scale, dq, st);
}

}  // namespace ssa
