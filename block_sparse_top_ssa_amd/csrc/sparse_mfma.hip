// Sparse-stream attention forward on MFMA bf16 (paper sec. 3, p. 4: each query attends
// the tokens of its kept blocks -- the "reduced K and V" -- causally inside its own
// block; App. D, p. 21: the attend-over-selected-tokens stage).
//
// Neighbouring queries keep largely different blocks, so a dense tile over the union
// of their blocks would waste most of its products.  Instead a workgroup owns T
// consecutive query rows of one (b, h), keeps their output state in LDS, and visits
// each key block that any of its rows kept exactly once, multiplying only the rows
// that kept it (gathered into 16-row MFMA column tiles):
//
//  0. (separate passes) V and K are rewritten once into MFMA fragment order, so the PV
//     operand V^T is loaded with one coalesced 16-byte load per lane and no lane
//     transposes, and every K fragment is one contiguous 1 KB load (8 full cache lines
//     instead of 16 half lines: the CU's address unit, the busiest resource here, pays
//     per line);
//  1. inverted index: from idx, count per block the rows that kept it, prefix-sum,
//     and list the row ids per block (LDS, one byte per entry).  The tile is as tall as
//     the O state allows (256 rows at D = 128); when its lists exceed the LDS left
//     over (long idx rows, e.g. 64 blocks per row), they are built and consumed in
//     batches of consecutive blocks, phase 3 running once per batch;
//  2. own-block phase: each 64-row query chunk against its own 64-key chunk (causal)
//     on MFMA; the row max of these logits becomes the row's fixed reference m_ref,
//     and O, l start from this chunk;
//  3. kept-block phase, in lockstep rounds of two roles per SIMD:
//     * four score waves each take the blocks j = s (mod 4) in ascending order and,
//       per round, one 16-row tile of the rows that kept the current 64-key chunk:
//       S^T = K Q^T, p = exp2(s - m_ref) rounded to bf16, row sums of the rounded p;
//       P^T, the row ids and the sums go to the wave's slot in a double-buffered set;
//     * four value waves each own a 32-column slice of the O state of every row; per
//       round they read the four slots of the previous round, load the V^T fragments
//       of their slice (prefetched one round ahead), form O^T = V^T P^T for their
//       columns and add it into the O state with plain 16-byte read-add-write.
//     Each O element has a single writer, so no atomics are needed (LDS float atomics
//     run at a fraction of a lane per clock on this chip).  While the value waves fold
//     one slot set, the score waves fill the other: one barrier per round.
//     Because every row uses the fixed reference m_ref, partial sums from different
//     blocks simply add, in any order, with no rescaling.
//  4. finalize: o = O / l (bf16), lse = m_ref + log l.
// A 64-row query chunk whose rows all keep every block below their own (the leading
// rows t < topk * s, every row when topk covers all blocks; a row can only do so if
// b_t <= topk) is plain causal attention; this kernel skips it and the dense kernel,
// launched next on the same stream over the rows t < (topk + 1) * s, writes it (it
// keeps each row's O in registers, which gathered rows cannot).
//
// A second instance (STATS) also measures the sparse stream (App. H, Table A9: entropy;
// App. K.2, p. 31: attention mass by distance) from the same probabilities: beside l each
// row keeps sum p x (x = log2 p against m_ref; entropy = ln l - ln 2 sum p x / l) and its
// mass in each block-distance bucket, and each tile sums its rows' bucket masses over l
// into one partial.  That state takes 16 floats per row, so this instance runs on 192-row
// tiles.
//
// m_ref is an attained logit of the row, so l >= 1 and nothing underflows.  If any
// kept logit exceeds m_ref by more than kGuard (log2 units, i.e. exp would pass
// 2^kGuard), the row is flagged and recomputed exactly by one wave with a running-max
// softmax at the end; with unit-scale inputs this does not happen.
#include <algorithm>
#include <type_traits>

#include "launch.hpp"
#include "mfma.hpp"
#include "rowattn.hpp"

namespace ssa {

constexpr float kGuard = 90.f;  // log2 units
constexpr int kSlotBytes = 2256;  // P^T fragments (2 KB), 16 row ids, 2 x 16 row sums, chunk ids

struct SparseLds {
  // byte offsets inside the dynamic LDS block
  int ost, lst, lse2, mref, lent, hbk, off, misc, slots, flag, list, total;
};

// STATS: the layout also holds each row's sum of p x (x = log2 p against m_ref, for the
// entropy) and its mass in each block-distance bucket, and the slots carry four row sums.
constexpr int kSlotBytesStats = 2384;  // P^T fragments (2 KB), 16 row ids, 4 x 16 row sums, chunk ids
template <int D, bool STATS = false>
__host__ __device__ inline SparseLds sparse_lds_layout(int T, int nb, int list_cap) {
  SparseLds s;
  int o = 0;
  s.ost = o;   o += T * D * 4;   // O state, rows of D floats, 16-byte granules XOR-swizzled by row
  s.lst = o;   o += T * 4;   // row sums of the bf16-rounded p (normalise o)
  s.lse2 = o;  o += T * 4;   // row sums of the float32 p (log-sum-exp)
  s.mref = o;  o += T * 4;
  s.lent = o;  o += STATS ? T * 4 : 0;
  s.hbk = o;   o += STATS ? T * kDistBuckets * 4 : 0;
  s.off = o;   o += (nb + 1) * 4;
  s.misc = o;  o += 48;  // 4 item counts, 4 chunk flags
  o = (o + 15) & ~15;
  s.slots = o;  // 2 sets x 4 slots; the per-block counters of the index build live here first
  const int slot_bytes = STATS ? kSlotBytesStats : kSlotBytes;
  o += 8 * slot_bytes > nb * 4 ? 8 * slot_bytes : nb * 4;
  s.flag = o;  o += T;
  s.list = o;  o += list_cap;  // row lists of one batch of blocks (at least T entries)
  s.total = (o + 15) & ~15;
  return s;
}

// float offset of the 16-byte granule holding O[r][d .. d+3] (d % 4 == 0)
template <int D>
__device__ __forceinline__ int ost_granule(int r, int d) {
  return r * D + ((((d >> 2) ^ (r & 15))) << 2);
}

struct Slot {
  u32x4 p[2][64];
  int rows[16];
  float ps_round[16], ps_exact[16];  // row sums of the bf16-rounded and of the float32 p
  int chunk, next_chunk, pad0, pad1;
};
static_assert(sizeof(Slot) == kSlotBytes, "slot layout");
// The slot of the measuring instance: the rounded and exact p sums, the p x sums and the
// exact sums again, so value wave i adds sums[i] (its own row array) with no selection.
struct SlotStats {
  u32x4 p[2][64];
  int rows[16];
  float sums[4][16];
  int chunk, next_chunk, pad0, pad1;
};
static_assert(sizeof(SlotStats) == kSlotBytesStats, "slot layout");

// sum of the 8 bf16 values packed in a P^T fragment
__device__ __forceinline__ float sum_bf16x8(const u32x4& w) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += lo_bf16(w[i]) + hi_bf16(w[i]);
  return s;
}

// The sparse stream's measurements of one query row t from its exact log-sum-exp (nats),
// one wave: returns the entropy -sum p ln p over A(t) and adds the mass of each
// block-distance bucket to hb (lane 0), walking the keys as attend_sparse_row does (the
// row's own block causally, then each valid listed block below it).  qs holds q in float.
template <int D>
__device__ float sparse_row_stats(const uint16_t* __restrict__ kh, const float* qs, const int32_t* __restrict__ ir,
                                  int topk, int t, int S, float scale, float lse, float* hb) {
  const int lane = threadIdx.x & 63;
  const int bt = t / S, cpb = S / 64;
  float ent = 0.f;
  auto chunk = [&](int c, int bucket) {
    const int key = c * 64 + lane;
    float p = 0.f, pl = 0.f;
    if (key <= t) {
      const uint16_t* kr = kh + (int64_t)key * D;
      float acc = 0.f;
      for (int d = 0; d < D; d += 8) {
        float x[8];
        Elem<uint16_t>::unpack(load16(kr + d), x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(qs[d + e], x[e], acc);
      }
      const float lg = acc * scale - lse;  // ln p
      p = expf(lg);
      pl = p * lg;
    }
    const float mass = wave_sum(p);
    ent -= wave_sum(pl);
    if (lane == 0) hb[bucket] += mass;
  };
  for (int c = bt * cpb; c <= t / 64; ++c) chunk(c, 0);
  int prev = -1;
  for (int e = 0; e < topk; ++e) {
    const int j = ir[e];
    if (j > prev && j < bt) {
      prev = j;
      for (int ch = 0; ch < cpb; ++ch) chunk(j * cpb + ch, dist_bucket(bt - j));
    }
  }
  return ent;
}

template <int D, int S, int T, bool BATCHED, bool STATS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void sparse_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const u32x4* __restrict__ vt, const u32x4* __restrict__ ktf, const int32_t* __restrict__ idx, int topk,
    uint16_t* __restrict__ o,
    float* __restrict__ lse, int L, int BH, int ntile, float sl2, float scale, int G, int list_cap,
    float* __restrict__ ent_out, float* __restrict__ hpart) {
  constexpr int NW = 8, NTH = 512;
  constexpr int NC = D / 32, NDT = D / 16, CPB = S / 64;
  constexpr int DTW = NDT / 4;  // d tiles per value wave
  extern __shared__ __align__(16) unsigned char smem[];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  // head-major order: the resident workgroups cover few heads, so their K/V stay in
  // the L2 / last-level cache; within a head the tiles with the most work go first
  const int64_t wg = xcd_logical(blockIdx.x, (int64_t)gridDim.x);  // one head per XCD at a time
  const int64_t bh = wg / ntile;
  const int tile = ntile - 1 - (int)(wg % ntile);
  const int t0 = tile * T;
  const int rows = min(T, L - t0);
  const int nb = (t0 + rows - 1) / S;  // candidate blocks: those below the last row's block
  const SparseLds lay = sparse_lds_layout<D, STATS>(T, nb, list_cap);
  float* ost = reinterpret_cast<float*>(smem + lay.ost);
  float* lst = reinterpret_cast<float*>(smem + lay.lst);
  float* lsx = reinterpret_cast<float*>(smem + lay.lse2);
  float* mrf = reinterpret_cast<float*>(smem + lay.mref);
  int* cnt = reinterpret_cast<int*>(smem + lay.slots);  // index build only
  int* off = reinterpret_cast<int*>(smem + lay.off);
  int* misc = reinterpret_cast<int*>(smem + lay.misc);
  int* chunk_full = misc + 4;  // per 64-row query chunk: its rows all keep every earlier block
  using SlotT = std::conditional_t<STATS, SlotStats, Slot>;
  SlotT* slots = reinterpret_cast<SlotT*>(smem + lay.slots);  // [2][4]: set, score wave
  uint8_t* flag = smem + lay.flag;
  uint8_t* list = smem + lay.list;
  float* lent = reinterpret_cast<float*>(smem + lay.lent);  // STATS: per row sum of p x
  float* hbk = reinterpret_cast<float*>(smem + lay.hbk);    // STATS: [row][bucket] mass

  const uint16_t* qh = q + bh * (int64_t)L * D;
  const int64_t kvh = bh / G;  // K/V head of this query head
  const uint16_t* kh = k + kvh * (int64_t)L * D;
  const uint16_t* vh = v + kvh * (int64_t)L * D;
  const u32x4* vth = vt + kvh * (int64_t)(L / 64) * NDT * 2 * 64;
  const int32_t* ih = idx + bh * (int64_t)L * topk;
  auto vt_frag = [&](int c, int dt, int kc) -> u32x4 { return vth[((int64_t)(c * NDT + dt) * 2 + kc) * 64 + lane]; };
  const u32x4* kth = ktf + kvh * (int64_t)(L / 64) * 4 * NC * 64;
  // K fragment (key tile kt4, contraction chunk cc) of chunk c: one contiguous 1 KB load
  auto k_frag = [&](int c, int kt4, int cc) -> u32x4 { return kth[((int64_t)(c * 4 + kt4) * NC + cc) * 64 + lane]; };

  // Walk the valid entries of one row's idx list: distinct blocks below b_t, each
  // greater than the entry used before it.  Entries are loaded 32 at a time.
  // Rows of at most 32 entries (the usual case) are read once into registers, two
  // entries per register as 16-bit values (block indices stay below 2^15 then; other
  // values, which are never valid here, become -1), and walked from there by both
  // passes of the index build; 16-byte loads when the rows are 16-byte aligned.
  // Longer rows are re-read in batches of 32.
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
  auto for_each_entry = [&](int t, auto&& fn) {
    const int bt = t / S;
    if (idx_regs) {  // this thread's row (t = t0 + tid), from registers
      int prev = -1;
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        const int j = (int)(int16_t)(ent[u >> 1] >> (16 * (u & 1)));
        if (j > prev && j < bt) {
          prev = j;
          fn(j);
        }
      }
      return;
    }
    const int32_t* ir = ih + (int64_t)t * topk;
    int prev = -1;
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
  };

  // Operands of this wave's first own-block unit (phase 2), loaded before the index
  // build so their latency passes while the index is built: K and V^T of the unit's
  // diagonal chunk and Q of its 32 rows.
  constexpr int NQ = 2 * NC;
  u32x4 okf[4][NC], ovf[NDT][2], oqf[NQ];
  auto own_load = [&](int u) __attribute__((always_inline)) {
    const int r0 = 32 * u, qc = r0 / 64;
    const int c_diag = (t0 + 64 * qc) / 64;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) okf[kt][cc] = k_frag(c_diag, kt, cc);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) ovf[dt][kc] = vt_frag(c_diag, dt, kc);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc)
        oqf[nt * NC + cc] = load_q_frag<D>(qh + (int64_t)(t0 + r0 + 16 * nt + n) * D, cc);
  };
  if (32 * w < rows && w < T / 32) own_load(w);

  // ---------------------------------------------------------------- 1. inverted index
  // A row whose kept blocks are all the blocks below its own block is plain causal
  // attention.  A 64-row query chunk made only of such rows is left to the dense kernel
  // (launched after this one, it applies the same test) and takes no part here.
  for (int j = tid; j < nb; j += NTH) cnt[j] = 0;
  for (int r = tid; r < T; r += NTH) flag[r] = 0;
  if constexpr (STATS)
    for (int i = tid; i < T * kDistBuckets; i += NTH) hbk[i] = 0.f;
  if (tid < 4) chunk_full[tid] = 1;
  __syncthreads();
  if (tid < rows) {
    int kept = 0;
    for_each_entry(t0 + tid, [&](int) { ++kept; });
    if (kept != (t0 + tid) / S) chunk_full[tid / 64] = 0;
  }
  __syncthreads();
  bool tile_full = true;
  for (int c = 0; c < rows / 64; ++c) tile_full = tile_full && chunk_full[c];
  if (tile_full) {  // uniform: the dense kernel writes (and measures) every row of this tile
    if constexpr (STATS)
      if (hpart && tid < kDistBuckets) hpart[((int64_t)bh * ntile + tile) * kDistBuckets + tid] = 0.f;
    return;
  }
  auto row_here = [&](int r) { return !chunk_full[r / 64]; };
  if (tid < rows && row_here(tid)) for_each_entry(t0 + tid, [&](int j) { atomicAdd(&cnt[j], 1); });
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
  // off[] now holds every block's offset in one virtual row list.  When the whole list
  // fits the list area it is built here, where its LDS atomics overlap the own-block
  // phase; otherwise phase 3 builds it batch by batch, as many blocks as fit at a time.
  __syncthreads();
  const bool one_batch = !BATCHED || off[nb] <= list_cap;  // uniform
  if (one_batch) {
    for (int j = tid; j < nb; j += NTH) cnt[j] = off[j];  // cnt becomes the fill cursor
    __syncthreads();
    if (tid < rows && row_here(tid)) for_each_entry(t0 + tid, [&](int j) { list[atomicAdd(&cnt[j], 1)] = (uint8_t)tid; });
  }

  // ---------------------------------------------------------------- 2. own-block phase
  // Unit = 32 rows (two 16-row column tiles) of one 64-row query chunk against the
  // 64-key chunk holding them (causal).  These rows belong to this wave alone here.
  for (int u = w; u < T / 32; u += NW) {
    const int r0 = 32 * u;  // tile-relative first row of the unit
    if (r0 >= rows) break;
    if (!row_here(r0)) continue;
    const int qc = r0 / 64, rq = r0 % 64;  // query chunk and row offset inside it
    const int c_diag = (t0 + 64 * qc) / 64;
    if (u != w) own_load(u);  // the first unit's operands were loaded before phase 1
    auto& kf = okf;
    auto& vf = ovf;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int rl = rq + 16 * nt;  // row offset inside the 64-row chunk
      const int r = r0 + 16 * nt + n;
      u32x4 qf[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) qf[cc] = oqf[nt * NC + cc];
      f32x4 sacc[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        sacc[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) sacc[kt] = mfma_bf16(kf[kt][cc], qf[cc], sacc[kt]);
      }
      float p[16];
      float mx = -__builtin_huge_valf();
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = sacc[kt][i] * sl2;
          if (16 * kt + 4 * g + i > rl + n) x = -__builtin_huge_valf();
          p[kt * 4 + i] = x;
          mx = fmaxf(mx, x);
        }
      mx = max_over_rows(mx);
      float px = 0.f, pe = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = p[i] - mx;
        p[i] = fast_exp2(e);
        px += p[i];
        if constexpr (STATS) pe = fmaf(p[i], fmaxf(e, -0x1p100f), pe);  // masked keys: p = 0
      }
      const u32x4 pf0 = pack_p(&p[0], &p[4]), pf1 = pack_p(&p[8], &p[12]);
      const float ps = sum_over_rows(sum_bf16x8(pf0) + sum_bf16x8(pf1));  // sum of the rounded p the products use
      px = sum_over_rows(px);
      if constexpr (STATS) pe = sum_over_rows(pe);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        f32x4 acc = f32x4{0, 0, 0, 0};
        acc = mfma_bf16(vf[dt][0], pf0, acc);
        acc = mfma_bf16(vf[dt][1], pf1, acc);
        *reinterpret_cast<f32x4*>(ost + ost_granule<D>(r, 16 * dt + 4 * g)) = acc;
      }
      if (g == 0) {
        lst[r] = ps;
        lsx[r] = px;
        mrf[r] = mx;
        if constexpr (STATS) {
          lent[r] = pe;
          hbk[r * kDistBuckets] = px;  // distance bucket 0: the own block
        }
      }
    }
    if (CPB == 2 && (c_diag & 1)) {
      // a 128-token block: rows in its second half also see its first half, unmasked
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // m_ref written by other lanes
      const int c = c_diag - 1;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) kf[kt][cc] = k_frag(c, kt, cc);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) vf[dt][kc] = vt_frag(c, dt, kc);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const int r = r0 + 16 * nt + n;
        u32x4 qf[NC];
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) qf[cc] = load_q_frag<D>(qh + (int64_t)(t0 + r) * D, cc);
        f32x4 sacc[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          sacc[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) sacc[kt] = mfma_bf16(kf[kt][cc], qf[cc], sacc[kt]);
        }
        const float mr = mrf[r];
        float p[16], mx = -__builtin_huge_valf(), px = 0.f, pe = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = sacc[kt][i] * sl2 - mr;
            mx = fmaxf(mx, x);
            p[kt * 4 + i] = fast_exp2(x);
            px += p[kt * 4 + i];
            if constexpr (STATS) pe = fmaf(p[kt * 4 + i], x, pe);
          }
        if (mx > kGuard) flag[r] = 1;
        const u32x4 pf0 = pack_p(&p[0], &p[4]), pf1 = pack_p(&p[8], &p[12]);
        const float ps = sum_over_rows(sum_bf16x8(pf0) + sum_bf16x8(pf1));
        px = sum_over_rows(px);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          f32x4 acc = f32x4{0, 0, 0, 0};
          acc = mfma_bf16(vf[dt][0], pf0, acc);
          acc = mfma_bf16(vf[dt][1], pf1, acc);
          f32x4* gp = reinterpret_cast<f32x4*>(ost + ost_granule<D>(r, 16 * dt + 4 * g));
          *gp = *gp + acc;
        }
        if constexpr (STATS) pe = sum_over_rows(pe);
        if (g == 0) {
          lst[r] += ps;
          lsx[r] += px;
          if constexpr (STATS) {
            lent[r] += pe;
            hbk[r * kDistBuckets] += px;
          }
        }
      }
    }
  }

  // ---------------------------------------------------------------- 3. kept-block phase
  // score wave s (w < 4) owns blocks j = s (mod 4); its items are (block, chunk, tile)
  // The blocks are taken in batches [jb, je) whose row lists fit the list area (lbase:
  // the batch's first entry in the virtual list).
  int jb = 0, je = 0, lbase = 0, my_items = 0, rounds = 0;
  auto next_block = [&](int from) -> int {  // next non-empty block >= from in the batch, same residue
    int j = from;
    while (j < je && off[j + 1] == off[j]) j += 4;
    return j < je ? j : je;
  };

  // score-wave state (waves 0-3): the loaded operands of the next tile to score, and
  // the scored tile waiting to be published
  int j = je, ch = 0, it = 0, r_cur = -1;
  // Operand registers live across rounds: a score wave keeps the K fragments of its
  // current chunk in `ra`, a value wave its V^T fragments; one array serves both roles
  // so the two never hold registers at the same time.
  constexpr int RA = 4 * NC > 8 * DTW ? 4 * NC : 8 * DTW;
  u32x4 ra[RA], qf[NC];
  u32x4 pub0 = u32x4{0, 0, 0, 0}, pub1 = u32x4{0, 0, 0, 0};
  int pub_r = -1, pub_c = -1, pub_nc = -1;
  float pub_ps = 0.f, pub_px = 0.f, pub_pe = 0.f;
  int scored = 0;
  auto load_item = [&](bool new_chunk) {
    const int beg = off[j] - lbase, count = off[j + 1] - off[j];
    const int e = it * 16 + n;
    r_cur = e < count ? (int)list[beg + e] : -1;
    if (new_chunk) {
      const int c = j * CPB + ch;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) ra[kt * NC + cc] = k_frag(c, kt, cc);
    }
    const uint16_t* qrow = qh + (int64_t)(t0 + (r_cur < 0 ? 0 : r_cur)) * D;
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) qf[cc] = load_q_frag<D>(qrow, cc);
  };
  auto score_item = [&]() {
    const int r = r_cur;
    const float mr = r >= 0 ? mrf[r] : __builtin_huge_valf();  // no row: every p is 0
    f32x4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) sacc[kt] = mfma_bf16(ra[kt * NC + cc], qf[cc], sacc[kt]);
    }
    float p[16], mx = -__builtin_huge_valf(), px = 0.f, pe = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = fmaf(sacc[kt][i], sl2, -mr);
        mx = fmaxf(mx, x);
        p[kt * 4 + i] = fast_exp2(x);
        px += p[kt * 4 + i];
        if constexpr (STATS) pe = fmaf(p[kt * 4 + i], fmaxf(x, -0x1p100f), pe);  // r < 0: x = -inf, p = 0
      }
    if (mx > kGuard) flag[r] = 1;  // mx is -inf for r < 0
    pub0 = pack_p(&p[0], &p[4]);
    pub1 = pack_p(&p[8], &p[12]);
    pub_ps = sum_over_rows(sum_bf16x8(pub0) + sum_bf16x8(pub1));  // sum of the rounded p the products use
    pub_px = sum_over_rows(px);
    if constexpr (STATS) pub_pe = sum_over_rows(pe);
    pub_r = r;
    pub_c = j * CPB + ch;
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
  // value-wave state (waves 4-7): V^T fragments of its column slice, per score-wave stream
  const int pw = w - 4;
  // the same as a scalar (the compiler cannot see that w is uniform across the wave);
  // STATS: value wave i keeps the row sums sums[i] of the slots in lsum: the rounded and
  // the exact p sums, the p x sums, and per row and distance bucket the exact p sums
  const int pu = __builtin_amdgcn_readfirstlane(pw);
  float* const lsum = pu == 0 ? lst : pu == 1 ? lsx : pu == 2 ? lent : hbk;
  int vchunk[4] = {-1, -1, -1, -1};
  auto load_v = [&](int s, int c) {
#pragma unroll
    for (int dl = 0; dl < DTW; ++dl)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) ra[(s * DTW + dl) * 2 + kc] = vt_frag(c, pw * DTW + dl, kc);
  };

  // The tile scored last goes to the wave's slot in set `set` (chunk -1: nothing).
  auto publish = [&](int set, bool have) {
    SlotT& sl = slots[set * 4 + w];
    if (have) {
      sl.p[0][lane] = pub0;
      sl.p[1][lane] = pub1;
      if (g == 0) {
        sl.rows[n] = pub_r;
        if constexpr (STATS) {
          sl.sums[0][n] = pub_ps;
          sl.sums[1][n] = pub_px;
          sl.sums[2][n] = pub_pe;
          sl.sums[3][n] = pub_px;
        } else {
          sl.ps_round[n] = pub_ps;
          sl.ps_exact[n] = pub_px;
        }
      }
    }
    if (lane == 0) {
      sl.chunk = have ? pub_c : -1;
      sl.next_chunk = have ? pub_nc : -1;
    }
  };
  __syncthreads();  // off[] and the own-block state are complete
  do {
    // ------------------------------------------------------------ one batch of blocks
    lbase = off[jb];
    if (one_batch) {
      je = nb;
    } else {
      {  // the largest je with off[je] - off[jb] <= list_cap (one block lists at most T rows)
        int lo = jb + 1, hi = nb;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (off[mid] - lbase <= list_cap) lo = mid;
          else hi = mid - 1;
        }
        je = lo;
      }
      for (int jj = jb + tid; jj < je; jj += NTH) cnt[jj - jb] = off[jj] - lbase;  // fill cursors
      __syncthreads();
      if (tid < rows && row_here(tid))
        for_each_entry(t0 + tid, [&](int jj) {
          if (jj >= jb && jj < je) list[atomicAdd(&cnt[jj - jb], 1)] = (uint8_t)tid;
        });
    }
    if (w < 4) {  // items of score wave w: tiles of the batch's blocks j = w (mod 4), all lanes counting
      int items = 0;
      for (int jj = jb + ((w - jb) & 3) + 4 * lane; jj < je; jj += 256) items += CPB * ((off[jj + 1] - off[jj] + 15) / 16);
#pragma unroll
      for (int o2 = 32; o2 > 0; o2 >>= 1) items += __shfl_xor(items, o2);
      if (lane == 0) misc[w] = items;
    }
    __syncthreads();  // row lists, item counts
    my_items = w < 4 ? misc[w] : 0;
    rounds = max(max(misc[0], misc[1]), max(misc[2], misc[3]));
    j = w < 4 ? next_block(jb + ((w - jb) & 3)) : je;
    ch = 0;
    it = 0;
    scored = 0;
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) vchunk[s2] = -1;
    if (w < 4 && my_items > 0) {
      load_item(true);
      score_item();
    }
    if (w < 4) publish(0, my_items > 0);
    __syncthreads();
    // Round rd: the value waves fold slot set rd % 2 while the score waves score their
    // next tile and publish it in the other set; one barrier per round.  Each role runs
    // its own loop (same number of rounds, so the barriers pair up), which keeps the
    // compiler's load counting of one role free of the other's pending loads.
    if (w < 4) {
      for (int rd = 0; rd < rounds; ++rd) {
        // ------------------------------------------------------------ score wave: next tile
        const bool more = rd + 1 < my_items;
        if (more) score_item();
        publish((rd + 1) & 1, more);
        __syncthreads();
      }
    } else {
      for (int rd = 0; rd < rounds; ++rd) {
        // ------------------------------------------------------------ value wave
        const SlotT* const cs = slots + (rd & 1) * 4;
        // (1) slot headers and P^T; (2) V^T of a stream's first chunk (later chunks were
        // loaded a round ahead); (3) all products; (4) next round's V^T loads (registers
        // are free once the products are issued); (5) read-add-write into the owned
        // columns, slot by slot (slots may share rows).
        int sc[4], sn[4], sr[4];
        float sps[4];  // value wave 0: rounded-p row sums, wave 1: exact ones
        u32x4 sp[4][2];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          sc[s] = __builtin_amdgcn_readfirstlane(cs[s].chunk);  // uniform: scalar branches
          sn[s] = __builtin_amdgcn_readfirstlane(cs[s].next_chunk);
          sr[s] = cs[s].rows[n];
          if constexpr (STATS)
            sps[s] = cs[s].sums[pu][n];
          else
            sps[s] = pw == 0 ? cs[s].ps_round[n] : cs[s].ps_exact[n];
          sp[s][0] = cs[s].p[0][lane];
          sp[s][1] = cs[s].p[1][lane];
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (sc[s] >= 0 && sc[s] != vchunk[s]) {  // first tile of a stream: not prefetched
            load_v(s, sc[s]);
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
            load_v(s, sn[s]);  // used next round
            vchunk[s] = sn[s];
          }
        }
        // (5) read-add-write, slot by slot: a row can sit in several slots of a round (at
        // any lane), and the in-order LDS queue of the wave makes each slot's writes land
        // before the next slot's reads.  Value wave 0 also adds the rounded-p row sums,
        // wave 1 the exact ones: the sum is read with the O granules and written after
        // them, so the O writes wait for one LDS round trip only.
        float* const ls = pw == 0 ? lst : lsx;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int r = sr[s];
          if (sc[s] >= 0 && r >= 0) {
            f32x4 cv[DTW];
            f32x4* gp[DTW];
#pragma unroll
            for (int dl = 0; dl < DTW; ++dl) {
              gp[dl] = reinterpret_cast<f32x4*>(ost + ost_granule<D>(r, 16 * (pw * DTW + dl) + 4 * g));
              cv[dl] = *gp[dl];
            }
            if constexpr (STATS) {
              // value waves 2 and 3 also keep a row sum each: the p x sums (entropy) and
              // the mass in the distance bucket of this slot's block
              const int li = pu == 3 ? r * kDistBuckets + dist_bucket((t0 + r) / S - sc[s] / CPB) : r;
              const float lv = lsum[li];
#pragma unroll
              for (int dl = 0; dl < DTW; ++dl) *gp[dl] = cv[dl] + acc[s][dl];
              if (g == 0) lsum[li] = lv + sps[s];
            } else {
              const float lv = pw < 2 ? ls[r] : 0.f;
#pragma unroll
              for (int dl = 0; dl < DTW; ++dl) *gp[dl] = cv[dl] + acc[s][dl];
              if (pw < 2 && g == 0) ls[r] = lv + sps[s];
            }
          }
        }
        __syncthreads();
      }
    }
    jb = je;
  } while (BATCHED && jb < nb);  // batches

  // ---------------------------------------------------------------- 4. finalize
  for (int it = tid; it < rows * (D / 8); it += NTH) {
    const int r = it / (D / 8), c8 = it % (D / 8);
    if (flag[r] || !row_here(r)) continue;
    const float inv = 1.f / lst[r];
    const f32x4 a = *reinterpret_cast<const f32x4*>(ost + ost_granule<D>(r, 8 * c8));
    const f32x4 b = *reinterpret_cast<const f32x4*>(ost + ost_granule<D>(r, 8 * c8 + 4));
    float x[8] = {a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv, b[0] * inv, b[1] * inv, b[2] * inv, b[3] * inv};
    store16(o + (bh * (int64_t)L + t0 + r) * D + 8 * c8, Elem<uint16_t>::pack(x));
  }
  if (lse)
    for (int r = tid; r < rows; r += NTH)
      if (!flag[r] && row_here(r)) lse[bh * (int64_t)L + t0 + r] = (mrf[r] + log2f(lsx[r])) * kLn2;
  if constexpr (STATS)  // entropy = ln l - ln 2 sum(p x) / l, with p = 2^x against m_ref
    if (ent_out)
      for (int r = tid; r < rows; r += NTH)
        if (!flag[r] && row_here(r)) ent_out[bh * (int64_t)L + t0 + r] = logf(lsx[r]) - kLn2 * lent[r] / lsx[r];

  // ---------------------------------------------------------------- 5. exact recompute of flagged rows
  int any = 0;
  for (int r = tid; r < rows; r += NTH) any |= flag[r];
  const bool any_flag = __syncthreads_or(any);
  if constexpr (!STATS) {
    if (!any_flag) return;
  }
  if (any_flag) {
    float* qs = reinterpret_cast<float*>(smem + lay.ost) + w * D;  // O state no longer needed
    for (int r = w; r < rows; r += NW) {
      if (!flag[r]) continue;
      const int t = t0 + r;
      for (int d = lane; d < D; d += 64) qs[d] = bf16_bits_to_f32(qh[(int64_t)t * D + d]);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      float m = -__builtin_huge_valf(), l = 0.f, acc[D / 64];
#pragma unroll
      for (int e = 0; e < D / 64; ++e) acc[e] = 0.f;
      attend_sparse_row<uint16_t, D>(kh, vh, qs, ih + (int64_t)t * topk, topk, t, S, scale, m, l, acc);
      const float inv = 1.f / l;
#pragma unroll
      for (int e = 0; e < D / 64; ++e)
        o[(bh * (int64_t)L + t) * D + lane + 64 * e] = (uint16_t)f32_to_bf16_bits(acc[e] * inv);
      if (lse && lane == 0) lse[bh * (int64_t)L + t] = m + logf(l);
      if constexpr (STATS) {
        // the row's measurements from its exact log-sum-exp; its bucket masses are then
        // normalised already, so its divisor becomes 1
        float* hr = hbk + r * kDistBuckets;
        if (lane < kDistBuckets) hr[lane] = 0.f;
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        const float e = sparse_row_stats<D>(kh, qs, ih + (int64_t)t * topk, topk, t, S, scale, m + logf(l), hr);
        if (lane == 0) {
          if (ent_out) ent_out[bh * (int64_t)L + t] = e;
          lsx[r] = 1.f;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
  if constexpr (STATS) {
    // this tile's distance histogram: each row's bucket masses divided by its l, summed
    // over the rows in a fixed order (row groups, then the groups) into one partial
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem + lay.ost);  // [row group][bucket]; the O state is done
    constexpr int RG = NTH / kDistBuckets;
    {
      const int b = tid % kDistBuckets, rg = tid / kDistBuckets;
      float x = 0.f;
      for (int r = rg; r < rows; r += RG)
        if (row_here(r)) x += hbk[r * kDistBuckets + b] / lsx[r];
      red[rg * kDistBuckets + b] = x;
    }
    __syncthreads();
    if (hpart && tid < kDistBuckets) {
      float y = 0.f;
      for (int i = 0; i < RG; ++i) y += red[i * kDistBuckets + tid];
      hpart[((int64_t)bh * ntile + tile) * kDistBuckets + tid] = y;
    }
  }
}

static constexpr int kMaxLds = 160 * 1024 - 512;  // leave room for the static LDS (scan partials, 288 bytes)

struct SparseTile {
  int T, list_cap;
};
// Rows per tile: the most (so each visited block serves the most rows) whose LDS fits
// with a list area of at least T entries; the list area takes what is left, up to a
// tile's whole row lists (T * topk entries), so long idx rows only add batches.
template <int D, bool STATS = false>
static SparseTile pick_tile(const Dims& d, int topk) {
  for (int T : {256, 192, 128}) {
    const int fixed = sparse_lds_layout<D, STATS>(T, d.n(), 0).total;  // d.n(): bound on any tile's blocks
    const int room = (kMaxLds - fixed) & ~15;
    if (room >= T) return {T, min((T * topk + 15) & ~15, room)};
  }
  return {0, 0};
}

bool sparse_mfma_supported(const Dims& d, int topk) {
  if (d.dtype != 1 || (d.D != 64 && d.D != 128) || d.L % 64) return false;
  return (d.D == 128 ? pick_tile<128>(d, topk) : pick_tile<64>(d, topk)).T > 0;
}

bool sparse_mfma_stats_supported(const Dims& d, int topk) {
  if (!sparse_mfma_supported(d, topk)) return false;
  return (d.D == 128 ? pick_tile<128, true>(d, topk) : pick_tile<64, true>(d, topk)).T > 0;
}

template <int D, int S, int T, bool BATCHED, bool STATS>
static hipError_t run_sparse(const Dims& d, const void* q, const void* k, const void* v, const u32x4* vt,
                             const u32x4* kt, const int32_t* idx, int topk, int list_cap, float scale, void* o,
                             float* lse, float* ent, float* hpart, hipStream_t st) {
  const int ntile = (d.L + T - 1) / T;
  const int64_t grid = (int64_t)ntile * d.bh();
  const int lds = sparse_lds_layout<D, STATS>(T, d.n(), list_cap).total;
  auto kern = sparse_fwd_kernel<D, S, T, BATCHED, STATS>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), lds, st, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), vt, kt, idx, topk,
                     static_cast<uint16_t*>(o), lse, d.L, (int)d.bh(), ntile, scale * kLog2e, scale, d.G(), list_cap,
                     ent, hpart);
  return hipGetLastError();
}

template <int D, int S, bool STATS>
static hipError_t dispatch_t(const Dims& d, const void* q, const void* k, const void* v, const u32x4* vt,
                             const u32x4* kt, const int32_t* idx, int topk, float scale, void* o, float* lse,
                             float* ent, float* hpart, hipStream_t st) {
  const SparseTile t = pick_tile<D, STATS>(d, topk);
  // the batched kernel only where a tile's row lists (T * topk entries at most) may not fit
  if (t.list_cap >= t.T * topk) {
    if (t.T == 256)
      return run_sparse<D, S, 256, false, STATS>(d, q, k, v, vt, kt, idx, topk, t.list_cap, scale, o, lse, ent, hpart, st);
    if (t.T == 192)
      return run_sparse<D, S, 192, false, STATS>(d, q, k, v, vt, kt, idx, topk, t.list_cap, scale, o, lse, ent, hpart, st);
    return run_sparse<D, S, 128, false, STATS>(d, q, k, v, vt, kt, idx, topk, t.list_cap, scale, o, lse, ent, hpart, st);
  }
  if (t.T == 256)
    return run_sparse<D, S, 256, true, STATS>(d, q, k, v, vt, kt, idx, topk, t.list_cap, scale, o, lse, ent, hpart, st);
  if (t.T == 192)
    return run_sparse<D, S, 192, true, STATS>(d, q, k, v, vt, kt, idx, topk, t.list_cap, scale, o, lse, ent, hpart, st);
  return run_sparse<D, S, 128, true, STATS>(d, q, k, v, vt, kt, idx, topk, t.list_cap, scale, o, lse, ent, hpart, st);
}

template <bool STATS>
static hipError_t dispatch_sparse(const Dims& d, const void* q, const void* k, const void* v, const u32x4* vt,
                                  const u32x4* kt, const int32_t* idx, int topk, float scale, void* o, float* lse,
                                  float* ent, float* hpart, hipStream_t st) {
  if (d.D == 128)
    return d.S == 64 ? dispatch_t<128, 64, STATS>(d, q, k, v, vt, kt, idx, topk, scale, o, lse, ent, hpart, st)
                     : dispatch_t<128, 128, STATS>(d, q, k, v, vt, kt, idx, topk, scale, o, lse, ent, hpart, st);
  return d.S == 64 ? dispatch_t<64, 64, STATS>(d, q, k, v, vt, kt, idx, topk, scale, o, lse, ent, hpart, st)
                   : dispatch_t<64, 128, STATS>(d, q, k, v, vt, kt, idx, topk, scale, o, lse, ent, hpart, st);
}

LaunchResult launch_sparse_mfma_frag(const Dims& d, const void* q, const void* k, const void* v, const u32x4* kt,
                                     const u32x4* vt, const int32_t* idx, int topk, float scale, void* o, float* lse,
                                     hipStream_t st) {
  LaunchResult r;
  r.err = dispatch_sparse<false>(d, q, k, v, vt, kt, idx, topk, scale, o, lse, nullptr, nullptr, st);
  if (r.err == hipSuccess) r.err = launch_full_rows_of_sparse(d, q, k, vt, idx, topk, scale, o, lse, st);
  return r;
}

LaunchResult launch_sparse_mfma(const Dims& d, const void* q, const void* k, const void* v, const int32_t* idx,
                                int topk, float scale, void* o, float* lse, hipStream_t st) {
  LaunchResult r;
  void* ws = nullptr;
  r.err = vfrag_acquire(d.kv(), v, &ws, st);
  if (r.err != hipSuccess) return r;
  void* kws = nullptr;
  r.err = kfrag_acquire(d.kv(), k, &kws, st);
  if (r.err != hipSuccess) {
    (void)vfrag_release(ws, st);
    return r;
  }
  r = launch_sparse_mfma_frag(d, q, k, v, static_cast<const u32x4*>(kws), static_cast<const u32x4*>(ws), idx, topk,
                              scale, o, lse, st);
  const hipError_t ef = vfrag_release(ws, st);
  const hipError_t ek = vfrag_release(kws, st);
  if (r.err == hipSuccess) r.err = ef != hipSuccess ? ef : ek;
  return r;
}

// hist[bh][m] = the sum of the sparse kernel's Ps partials of (b, h), then of the dense
// kernel's Pd partials, in order.
__global__ __launch_bounds__(64) void sparse_hist_sum_kernel(const float* __restrict__ ps, int Ps,
                                                             const float* __restrict__ pd, int Pd,
                                                             float* __restrict__ hist) {
  const int64_t bh = blockIdx.x;
  const int m = threadIdx.x;
  if (m >= kDistBuckets) return;
  double x = 0.0;
  for (int p = 0; p < Ps; ++p) x += ps[(bh * Ps + p) * kDistBuckets + m];
  for (int p = 0; p < Pd; ++p) x += pd[(bh * Pd + p) * kDistBuckets + m];
  hist[bh * kDistBuckets + m] = (float)x;
}

LaunchResult launch_sparse_mfma_stats(const Dims& d, const void* q, const void* k, const void* v, const int32_t* idx,
                                      int topk, float scale, void* o, float* lse, float* ent, float* hist,
                                      hipStream_t st) {
  LaunchResult r;
  const int T = (d.D == 128 ? pick_tile<128, true>(d, topk) : pick_tile<64, true>(d, topk)).T;
  const int Ps = (d.L + T - 1) / T;                                                 // sparse kernel tiles
  const int Pd = (int)((std::min<int64_t>(d.L, ((int64_t)topk + 1) * d.S) + 255) / 256);  // dense-chunk tiles
  void* hws = nullptr;
  float *ps = nullptr, *pd = nullptr;
  if (hist) {
    r.err = workspace_alloc((size_t)d.bh() * (Ps + Pd) * kDistBuckets * sizeof(float), &hws, st);
    if (r.err != hipSuccess) return r;
    ps = static_cast<float*>(hws);
    pd = ps + (size_t)d.bh() * Ps * kDistBuckets;
  }
  void* ws = nullptr;
  void* kws = nullptr;
  r.err = vfrag_acquire(d.kv(), v, &ws, st);
  if (r.err == hipSuccess) r.err = kfrag_acquire(d.kv(), k, &kws, st);
  if (r.err == hipSuccess) {
    const u32x4* vt = static_cast<const u32x4*>(ws);
    r.err = dispatch_sparse<true>(d, q, k, v, vt, static_cast<const u32x4*>(kws), idx, topk, scale, o, lse, ent, ps,
                                  st);
    if (r.err == hipSuccess) r.err = launch_full_rows_of_sparse(d, q, k, vt, idx, topk, scale, o, lse, st, ent, pd);
    if (r.err == hipSuccess && hist) {
      hipLaunchKernelGGL(sparse_hist_sum_kernel, dim3((unsigned)d.bh()), dim3(64), 0, st, ps, Ps, pd, Pd, hist);
      r.err = hipGetLastError();
    }
  }
  for (void* p : {ws, kws, hws}) {
    const hipError_t e = vfrag_release(p, st);
    if (r.err == hipSuccess) r.err = e;
  }
  return r;
}

}  // namespace ssa
