// Attention-pattern measurements of the sparse stream on MFMA bf16 over gathered rows
// (the quantities of stats.hip: per-row entropy and, per (b, h), the attention mass by
// block distance; the pages report them in App. H, Table A9 and App. K.2, Fig. A4).
//
// A query-stationary sweep under per-row block masks scores every earlier chunk although
// each row attends only its kept blocks.  Here, as in the sparse forward, a workgroup owns
// T consecutive rows of one (b, h), builds the block -> rows index of its tile in LDS (the
// rows' kept blocks and own blocks) and visits each attended block once with the rows that
// attend it.  Only the scores are needed, so the eight waves work independently: wave w
// takes the blocks j = w (mod 8) and, per 16 gathered rows and 64-key chunk,
//     S^T = K Q^T (MFMA),  p = exp2(S^T sl2 - lse2_row), 0 for keys after the row,
//     row sums of p * scale q.k and of p;
// the first go to the row's entropy accumulator in LDS (one atomic add per row and item),
// the second to a per-lane 16-bucket histogram in registers, the bucket being that of the
// block distance b_t - j.  At the end entropy_t = lse_t - acc_t, and the workgroup's
// histogram (lanes, then waves, in a fixed order) is one partial of the head's histogram.
#include "launch.hpp"
#include "mfma.hpp"

namespace ssa {

namespace {

constexpr int kGBuckets = kDistBuckets;
constexpr int kGWaves = 8, kGThreads = 512;

struct GatherLds {
  int ent, off, cnt, hs, list, total;  // byte offsets inside the dynamic LDS block
};

// nb: blocks a row of the tile may attend (those up to the last row's own block)
__host__ __device__ inline GatherLds gather_lds_layout(int T, int nb, int topk) {
  GatherLds s;
  int o = 0;
  s.ent = o;  o += T * 4;                   // per-row sum of p * scale q.k
  s.off = o;  o += (nb + 1) * 4;            // index: first entry of each block
  s.cnt = o;  o += nb * 4;                  // index: counts, then fill cursors
  s.hs = o;   o += kGWaves * kGBuckets * 4;  // per-wave histograms
  o = (o + 15) & ~15;
  s.list = o; o += T * (topk + 1) * 2;      // row ids (16-bit), up to topk kept blocks and the own block per row
  s.total = (o + 15) & ~15;
  return s;
}

constexpr int kGatherMaxLds = 160 * 1024 - 256;  // room for the static LDS of the scan


}  // namespace

template <int D, int S, int T>
__global__ __launch_bounds__(kGThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_stats_gather_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ lse,
    const int32_t* __restrict__ idx, int topk, float* __restrict__ entropy, float* __restrict__ part, int L,
    int ntile, float scale, float sl2, int G) {
  constexpr int NC = D / 32, CPB = S / 64;
  constexpr int RPT = (T + kGThreads - 1) / kGThreads;  // rows per thread in the index build
  extern __shared__ __align__(16) unsigned char smem_sg[];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  const int64_t wg = xcd_logical(blockIdx.x, (int64_t)gridDim.x);  // head-major, most work first
  const int64_t bh = wg / ntile;
  const int tile = ntile - 1 - (int)(wg % ntile);
  const int t0 = tile * T;
  const int rows = min(T, L - t0);
  const int nb = (t0 + rows - 1) / S + 1;
  const GatherLds lay = gather_lds_layout(T, nb, topk);
  float* ent = reinterpret_cast<float*>(smem_sg + lay.ent);
  int* off = reinterpret_cast<int*>(smem_sg + lay.off);
  int* cnt = reinterpret_cast<int*>(smem_sg + lay.cnt);
  float* hs = reinterpret_cast<float*>(smem_sg + lay.hs);
  uint16_t* list = reinterpret_cast<uint16_t*>(smem_sg + lay.list);

  const uint16_t* qh = q + bh * (int64_t)L * D;
  const uint16_t* kh = k + (bh / G) * (int64_t)L * D;
  const int32_t* ih = idx + bh * (int64_t)L * topk;
  const float* lh = lse + bh * (int64_t)L;

  // Blocks attended by row t: the valid kept entries (distinct, below b_t, each greater
  // than the entry used before it: the forward's rule) and then b_t itself.
  auto for_each_block = [&](int t, auto&& fn) {
    const int bt = t / S;
    const int32_t* ir = ih + (int64_t)t * topk;
    int prev = -1;
    for (int e = 0; e < topk; ++e) {
      const int j = ir[e];
      if (j > prev && j < bt) {
        prev = j;
        fn(j);
      }
    }
    fn(bt);
  };

  // ---------------------------------------------------------------- index
  for (int j = tid; j < nb; j += kGThreads) cnt[j] = 0;
  for (int r = tid; r < T; r += kGThreads) ent[r] = 0.f;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int r = tid + kGThreads * u;
    if (r < rows) for_each_block(t0 + r, [&](int j) { atomicAdd(&cnt[j], 1); });
  }
  __syncthreads();
  {  // exclusive prefix sum of cnt[0..nb) into off[0..nb]; thread-contiguous segments
    const int seg = (nb + kGThreads - 1) / kGThreads;
    const int b0 = min(nb, tid * seg), b1 = min(nb, b0 + seg);
    int local = 0;
    for (int j = b0; j < b1; ++j) local += cnt[j];
    int incl = local;
#pragma unroll
    for (int o2 = 1; o2 < 64; o2 <<= 1) {
      const int y = __shfl_up(incl, o2);
      if (lane >= o2) incl += y;
    }
    __shared__ int wsum[kGWaves];
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    int base = 0;
    for (int i = 0; i < w; ++i) base += wsum[i];
    int run = base + incl - local;
    for (int j = b0; j < b1; ++j) {
      off[j] = run;
      run += cnt[j];
    }
    if (tid == kGThreads - 1) off[nb] = base + incl;
  }
  __syncthreads();
  for (int j = tid; j < nb; j += kGThreads) cnt[j] = off[j];  // fill cursors
  __syncthreads();
#pragma unroll
  for (int u = 0; u < RPT; ++u) {
    const int r = tid + kGThreads * u;
    if (r < rows) for_each_block(t0 + r, [&](int j) { list[atomicAdd(&cnt[j], 1)] = (uint16_t)r; });
  }
  __syncthreads();

  // ---------------------------------------------------------------- items of this wave
  // item = (block j = w mod 8, chunk ch of the block, 16-row tile it of its rows)
  auto next_block = [&](int from) -> int {
    int j = from;
    while (j < nb && off[j + 1] == off[j]) j += kGWaves;
    return j;
  };
  float hacc[kGBuckets];
#pragma unroll
  for (int i = 0; i < kGBuckets; ++i) hacc[i] = 0.f;
  u32x4 kf[4 * NC], qf[NC];
  int j = next_block(w), ch = 0, it = 0, r = -1;
  auto load = [&](bool new_chunk) {
    const int beg = off[j], count = off[j + 1] - beg;
    const int e = it * 16 + n;
    r = e < count ? (int)list[beg + e] : -1;
    if (new_chunk) {
      const int c = j * CPB + ch;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) kf[kt * NC + cc] = load_k_frag<D>(kh, c * 64 + 16 * kt, cc);
    }
    const int64_t row = t0 + (r < 0 ? 0 : r);
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) qf[cc] = load_q_frag<D>(qh + row * D, cc);
  };
  if (j < nb) load(true);
  while (j < nb) {
    f32x4 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      sacc[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) sacc[kt] = mfma_bf16(kf[kt * NC + cc], qf[cc], sacc[kt]);
    }
    // element i of sacc[kt]: key 64 c + 16 kt + 4 g + i, row r (column n)
    const int c = j * CPB + ch, rr = r, jj = j;
    const int tq = t0 + rr;
    const float lv = lh[t0 + (rr < 0 ? 0 : rr)];
    const float l2 = rr >= 0 ? lv * kLog2e : __builtin_huge_valf();  // no row: every p is 0
    float es = 0.f, ms = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool live = 64 * c + 16 * kt + 4 * g + i <= tq;
        const float p = live ? fast_exp2(fmaf(sacc[kt][i], sl2, -l2)) : 0.f;
        es = fmaf(p, sacc[kt][i] * scale, es);
        ms += p;
      }
    // advance to the next item and issue its loads before folding this one
    const int ntl = (off[j + 1] - off[j] + 15) / 16;
    bool new_chunk = false;
    if (++it == ntl) {
      it = 0;
      new_chunk = true;
      if (++ch == CPB) {
        ch = 0;
        j = next_block(j + kGWaves);
      }
    }
    if (j < nb) load(new_chunk);
    // the four lanes of a row (n, n + 16, n + 32, n + 48) hold its 64 keys between them
    es += __shfl_xor(es, 16);
    es += __shfl_xor(es, 32);
    ms += __shfl_xor(ms, 16);
    ms += __shfl_xor(ms, 32);
    if (rr >= 0) {
      if (g == 0) atomicAdd(&ent[rr], es);
      const int m = dist_bucket(tq / S - jj);
#pragma unroll
      for (int b2 = 0; b2 < kGBuckets; ++b2)
        if (b2 == m && g == 0) hacc[b2] += ms;
    }
  }

  // ---------------------------------------------------------------- outputs
  if (part) {  // lanes, then waves, in a fixed order
#pragma unroll
    for (int b2 = 0; b2 < kGBuckets; ++b2) {
      float x = hacc[b2];
#pragma unroll
      for (int o2 = 32; o2 > 0; o2 >>= 1) x += __shfl_xor(x, o2);
      if (lane == 0) hs[w * kGBuckets + b2] = x;
    }
  }
  __syncthreads();
  if (entropy)
    for (int rr = tid; rr < rows; rr += kGThreads) entropy[bh * (int64_t)L + t0 + rr] = lh[t0 + rr] - ent[rr];
  if (part && tid < kGBuckets) {
    float x = 0.f;
    for (int ww = 0; ww < kGWaves; ++ww) x += hs[ww * kGBuckets + tid];
    part[wg * kGBuckets + tid] = x;
  }
}

namespace {

template <int T>
bool gather_fits(const Dims& d, int topk) {
  return gather_lds_layout(T, d.n(), topk).total <= kGatherMaxLds;
}

}  // namespace

// Tile of 512 rows where the index fits in LDS, else 256; 0 when neither does.
int stats_gather_tile(const Dims& d, int topk) {
  if (d.dtype != 1 || (d.D != 64 && d.D != 128) || (d.S != 64 && d.S != 128)) return 0;
  if (gather_fits<512>(d, topk)) return 512;
  if (gather_fits<256>(d, topk)) return 256;
  return 0;
}

// part: [B*H][ceil(L / tile)][16] histogram partials (tiles of a head in order)
hipError_t launch_stats_gather(const Dims& d, const void* q, const void* k, const float* lse, const int32_t* idx,
                               int topk, float scale, float* entropy, float* part, hipStream_t st) {
  const int T = stats_gather_tile(d, topk);
  if (T == 0) return hipErrorInvalidValue;
  const int ntile = (d.L + T - 1) / T;
  const int64_t grid = (int64_t)ntile * d.bh();
  const int lds = gather_lds_layout(T, d.n(), topk).total;
  auto pick = [&](auto dd, auto ss, auto tt) {
    constexpr int D = decltype(dd)::value, S = decltype(ss)::value, TT = decltype(tt)::value;
    auto kern = attn_stats_gather_kernel<D, S, TT>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kGThreads), lds, st, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), lse, idx, topk, entropy, part, d.L, ntile, scale,
                       scale * kLog2e, d.G());
    return hipGetLastError();
  };
  using I64 = std::integral_constant<int, 64>;
  using I128 = std::integral_constant<int, 128>;
  using I256 = std::integral_constant<int, 256>;
  using I512 = std::integral_constant<int, 512>;
  if (d.D == 128) {
    if (d.S == 64) return T == 512 ? pick(I128{}, I64{}, I512{}) : pick(I128{}, I64{}, I256{});
    return T == 512 ? pick(I128{}, I128{}, I512{}) : pick(I128{}, I128{}, I256{});
  }
  if (d.S == 64) return T == 512 ? pick(I64{}, I64{}, I512{}) : pick(I64{}, I64{}, I256{});
  return T == 512 ? pick(I64{}, I128{}, I512{}) : pick(I64{}, I128{}, I256{});
}

}  // namespace ssa
