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
//  1. inverted index: from idx, count per block the rows that kept it, prefix-sum,
//     and list the row ids per block (LDS, one byte per entry);
//  2. own-block phase: each 64-row query chunk against its own 64-key chunk (causal)
//     on MFMA; the row max of these logits becomes the row's fixed reference m_ref,
//     and O, l start from this chunk;
//  3. kept-block phase: waves take blocks in ascending order; for each 64-key chunk
//     of the block they hold its K and V^T fragments in registers and sweep the rows
//     that kept it in 16-row tiles: S^T = K Q^T, p = exp2(s - m_ref), O^T = V^T P^T,
//     then add O and l into LDS with float atomics.  Because every row uses the fixed
//     reference m_ref, the partial sums from different waves and blocks simply add,
//     in any order, with no rescaling.  K of the next chunk is loaded while the
//     current one's V products run, and V of the next chunk while its K products run.
//  4. finalize: o = O / l (bf16), lse = m_ref + log l.
//
// m_ref is an attained logit of the row, so l >= 1 and nothing underflows.  If any
// kept logit exceeds m_ref by more than kGuard (log2 units, i.e. exp would pass
// 2^kGuard), the row is flagged and recomputed exactly by one wave with a running-max
// softmax at the end; with unit-scale inputs this does not happen.
#include "launch.hpp"
#include "mfma.hpp"
#include "rowattn.hpp"

namespace ssa {

constexpr float kGuard = 90.f;  // log2 units

struct SparseLds {
  // byte offsets inside the dynamic LDS block
  int ost, lst, mref, flag, cnt, off, list, next, total;
};

template <int D>
__host__ __device__ inline SparseLds sparse_lds_layout(int T, int nb, int topk) {
  SparseLds s;
  int o = 0;
  s.ost = o;  o += T * (D + 1) * 4;   // O state, row stride D+1 floats
  s.lst = o;  o += T * 4;
  s.mref = o; o += T * 4;
  s.flag = o; o += T * 4;
  s.cnt = o;  o += nb * 4;
  s.off = o;  o += (nb + 1) * 4;
  s.next = o; o += 16;
  s.list = o; o += T * topk;  // malformed rows may list up to topk blocks below b_t
  s.total = (o + 15) & ~15;
  return s;
}

template <int D, int S, int T, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4))) void sparse_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ idx, int topk, uint16_t* __restrict__ o, float* __restrict__ lse, int L, int BH,
    int ntile, float sl2, float scale) {
  constexpr int NC = D / 32, NDT = D / 16, CPB = S / 64, NTH = NW * 64;
  constexpr int RS = D + 1;  // O state row stride (floats)
  extern __shared__ __align__(16) unsigned char smem[];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, tid = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  const int tile = ntile - 1 - (int)(blockIdx.x / BH);
  const int64_t bh = blockIdx.x % BH;
  const int t0 = tile * T;
  const int rows = min(T, L - t0);
  const int nb = (t0 + rows - 1) / S;  // candidate blocks: those below the last row's block
  const SparseLds lay = sparse_lds_layout<D>(T, nb, topk);
  float* ost = reinterpret_cast<float*>(smem + lay.ost);
  float* lst = reinterpret_cast<float*>(smem + lay.lst);
  float* mrf = reinterpret_cast<float*>(smem + lay.mref);
  int* flag = reinterpret_cast<int*>(smem + lay.flag);
  int* cnt = reinterpret_cast<int*>(smem + lay.cnt);
  int* off = reinterpret_cast<int*>(smem + lay.off);
  int* nextp = reinterpret_cast<int*>(smem + lay.next);
  uint8_t* list = smem + lay.list;

  const uint16_t* qh = q + bh * (int64_t)L * D;
  const uint16_t* kh = k + bh * (int64_t)L * D;
  const uint16_t* vh = v + bh * (int64_t)L * D;
  const int32_t* ih = idx + bh * (int64_t)L * topk;

  // Walk the valid entries of one row's idx list: distinct blocks below b_t, each
  // greater than the entry used before it.  Entries are loaded 8 at a time.
  auto for_each_entry = [&](int t, auto&& fn) {
    const int bt = t / S;
    const int32_t* ir = ih + (int64_t)t * topk;
    int prev = -1;
    for (int e0 = 0; e0 < topk; e0 += 8) {
      int jj[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) jj[u] = e0 + u < topk ? ir[e0 + u] : -1;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = jj[u];
        if (j > prev && j < bt) {
          prev = j;
          fn(j);
        }
      }
    }
  };

  // ---------------------------------------------------------------- 1. inverted index
  for (int j = tid; j < nb; j += NTH) cnt[j] = 0;
  for (int r = tid; r < T; r += NTH) flag[r] = 0;
  if (tid == 0) *nextp = 0;
  __syncthreads();
  if (tid < rows) for_each_entry(t0 + tid, [&](int j) { atomicAdd(&cnt[j], 1); });
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
  if (tid < rows) for_each_entry(t0 + tid, [&](int j) { list[atomicAdd(&cnt[j], 1)] = (uint8_t)tid; });

  // ---------------------------------------------------------------- 2. own-block phase
  // Unit = 32 rows (two 16-row column tiles) of one 64-row query chunk against the
  // 64-key chunk holding them (causal).  These rows belong to this wave alone here.
  for (int u = w; u < T / 32; u += NW) {
    const int r0 = 32 * u;  // tile-relative first row of the unit
    if (r0 >= rows) break;
    const int qc = r0 / 64, rq = r0 % 64;  // query chunk and row offset inside it
    const int c_diag = (t0 + 64 * qc) / 64;
    u32x4 kf[4][NC], vf[NDT][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) kf[kt][cc] = load_k_frag<D>(kh, c_diag * 64 + 16 * kt, cc);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) vf[dt][kc] = load_v_raw<D>(vh, c_diag * 64, dt, kc);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      vf[dt][0] = transpose8x8_b16_dpp(vf[dt][0]);
      vf[dt][1] = transpose8x8_b16_dpp(vf[dt][1]);
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int rl = rq + 16 * nt;  // row offset inside the 64-row chunk (relative to key 0 of the chunk)
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
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        p[i] = fast_exp2(p[i] - mx);
        ps += p[i];
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      const u32x4 pf0 = pack_p(&p[0], &p[4]), pf1 = pack_p(&p[8], &p[12]);
      float* orow = ost + r * RS;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        f32x4 acc = f32x4{0, 0, 0, 0};
        acc = mfma_bf16(vf[dt][0], pf0, acc);
        acc = mfma_bf16(vf[dt][1], pf1, acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) orow[16 * dt + 4 * g + i] = acc[i];
      }
      if (g == 0) {
        lst[r] = ps;
        mrf[r] = mx;
      }
    }
    if (CPB == 2 && (c_diag & 1)) {
      // a 128-token block: rows in its second half also see its first half, unmasked
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");  // m_ref written by other lanes
      const int c = c_diag - 1;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) kf[kt][cc] = load_k_frag<D>(kh, c * 64 + 16 * kt, cc);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) vf[dt][kc] = transpose8x8_b16_dpp(load_v_raw<D>(vh, c * 64, dt, kc));
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
        float p[16], ps = 0.f, mx = -__builtin_huge_valf();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = sacc[kt][i] * sl2 - mr;
            mx = fmaxf(mx, x);
            p[kt * 4 + i] = fast_exp2(x);
            ps += p[kt * 4 + i];
          }
        if (mx > kGuard) flag[r] = 1;
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        const u32x4 pf0 = pack_p(&p[0], &p[4]), pf1 = pack_p(&p[8], &p[12]);
        float* orow = ost + r * RS;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          f32x4 acc = f32x4{0, 0, 0, 0};
          acc = mfma_bf16(vf[dt][0], pf0, acc);
          acc = mfma_bf16(vf[dt][1], pf1, acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) orow[16 * dt + 4 * g + i] += acc[i];
        }
        if (g == 0) lst[r] += ps;
      }
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- 3. kept-block phase
  // Each wave takes the next block with rows (ascending), holds one 64-key chunk's K
  // and V^T fragments in registers and sweeps its rows 16 at a time; the next tile's
  // query fragments are loaded while the current one is in flight.
  auto grab = [&]() -> int {
    int j = 0;
    if (lane == 0) {
      do {
        j = atomicAdd(nextp, 1);
      } while (j < nb && off[j + 1] == off[j]);
    }
    return __shfl(j, 0);
  };
  for (int j = grab(); j < nb; j = grab()) {
    const int beg = off[j], count = off[j + 1] - beg;
    const int ntiles = (count + 15) / 16;
    for (int ch = 0; ch < CPB; ++ch) {
      const int c = j * CPB + ch;
      // issue order matters for the in-order load counter: K, then the first tile's
      // rows and Q, then V (only needed after the first score tile)
      u32x4 kf[4][NC], vf[NDT][2];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) kf[kt][cc] = load_k_frag<D>(kh, c * 64 + 16 * kt, cc);
      int r = n < count ? list[beg + n] : -1;
      u32x4 qf[NC];
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) qf[cc] = load_q_frag<D>(qh + (int64_t)(t0 + (r < 0 ? 0 : r)) * D, cc);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) vf[dt][kc] = load_v_raw<D>(vh, c * 64, dt, kc);
      for (int it = 0; it < ntiles; ++it) {
        // prefetch the next tile's rows and Q
        const int e2 = (it + 1) * 16 + n;
        const int r2 = (it + 1 < ntiles && e2 < count) ? list[beg + e2] : -1;
        u32x4 qn[NC];
        if (it + 1 < ntiles) {
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) qn[cc] = load_q_frag<D>(qh + (int64_t)(t0 + (r2 < 0 ? 0 : r2)) * D, cc);
        }
        const float mr = mrf[r < 0 ? 0 : r];
        f32x4 sacc[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          sacc[kt] = f32x4{0, 0, 0, 0};
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) sacc[kt] = mfma_bf16(kf[kt][cc], qf[cc], sacc[kt]);
        }
        float p[16], ps = 0.f, mx = -__builtin_huge_valf();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = sacc[kt][i] * sl2 - mr;
            mx = fmaxf(mx, x);
            p[kt * 4 + i] = r >= 0 ? fast_exp2(x) : 0.f;
            ps += p[kt * 4 + i];
          }
        if (r >= 0 && mx > kGuard) flag[r] = 1;
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        if (r >= 0 && g == 0) atomicAdd(&lst[r], ps);
        const u32x4 pf0 = pack_p(&p[0], &p[4]), pf1 = pack_p(&p[8], &p[12]);
        if (it == 0) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            vf[dt][0] = transpose8x8_b16_dpp(vf[dt][0]);
            vf[dt][1] = transpose8x8_b16_dpp(vf[dt][1]);
          }
        }
        float* orow = ost + (r < 0 ? 0 : r) * RS;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          f32x4 acc = f32x4{0, 0, 0, 0};
          acc = mfma_bf16(vf[dt][0], pf0, acc);
          acc = mfma_bf16(vf[dt][1], pf1, acc);
          if (r >= 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              __hip_atomic_fetch_add(orow + 16 * dt + 4 * g + i, acc[i], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
        r = r2;
        if (it + 1 < ntiles) {
#pragma unroll
          for (int cc = 0; cc < NC; ++cc) qf[cc] = qn[cc];
        }
      }
    }
  }
  __syncthreads();

  // ---------------------------------------------------------------- 4. finalize
  for (int it = tid; it < rows * (D / 8); it += NTH) {
    const int r = it / (D / 8), c8 = it % (D / 8);
    if (flag[r]) continue;
    const float inv = 1.f / lst[r];
    const float* src = ost + r * RS + 8 * c8;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = src[e] * inv;
    store16(o + (bh * (int64_t)L + t0 + r) * D + 8 * c8, Elem<uint16_t>::pack(x));
  }
  if (lse)
    for (int r = tid; r < rows; r += NTH)
      if (!flag[r]) lse[bh * (int64_t)L + t0 + r] = (mrf[r] + log2f(lst[r])) * kLn2;

  // ---------------------------------------------------------------- 5. exact recompute of flagged rows
  int any = 0;
  for (int r = tid; r < rows; r += NTH) any |= flag[r];
  if (!__syncthreads_or(any)) return;
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
    __builtin_amdgcn_wave_barrier();
  }
}

static constexpr int kMaxLds = 160 * 1024;

template <int D>
static int pick_tile(const Dims& d, int topk) {
  for (int T : {256, 128}) {
    const int nb = d.n();  // upper bound on candidate blocks of any tile
    if (sparse_lds_layout<D>(T, nb, topk).total <= kMaxLds) return T;
  }
  return 0;
}

bool sparse_mfma_supported(const Dims& d, int topk) {
  if (d.dtype != 1 || (d.D != 64 && d.D != 128) || d.L % 64) return false;
  return (d.D == 128 ? pick_tile<128>(d, topk) : pick_tile<64>(d, topk)) > 0;
}

constexpr int kSparseWaves = 8;

template <int D, int S, int T>
static hipError_t run_sparse(const Dims& d, const void* q, const void* k, const void* v, const int32_t* idx,
                             int topk, float scale, void* o, float* lse, hipStream_t st) {
  const int ntile = (d.L + T - 1) / T;
  const int64_t grid = (int64_t)ntile * d.bh();
  const int lds = sparse_lds_layout<D>(T, d.n(), topk).total;
  auto kern = sparse_fwd_kernel<D, S, T, kSparseWaves>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kSparseWaves * 64), lds, st, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), idx, topk,
                     static_cast<uint16_t*>(o), lse, d.L, (int)d.bh(), ntile, scale * kLog2e, scale);
  return hipGetLastError();
}

template <int D, int S>
static hipError_t dispatch_t(const Dims& d, const void* q, const void* k, const void* v, const int32_t* idx,
                             int topk, float scale, void* o, float* lse, hipStream_t st) {
  const int T = pick_tile<D>(d, topk);
  if (T == 256) return run_sparse<D, S, 256>(d, q, k, v, idx, topk, scale, o, lse, st);
  return run_sparse<D, S, 128>(d, q, k, v, idx, topk, scale, o, lse, st);
}

LaunchResult launch_sparse_mfma(const Dims& d, const void* q, const void* k, const void* v, const int32_t* idx,
                                int topk, float scale, void* o, float* lse, hipStream_t st) {
  LaunchResult r;
  if (d.D == 128)
    r.err = d.S == 64 ? dispatch_t<128, 64>(d, q, k, v, idx, topk, scale, o, lse, st)
                      : dispatch_t<128, 128>(d, q, k, v, idx, topk, scale, o, lse, st);
  else
    r.err = d.S == 64 ? dispatch_t<64, 64>(d, q, k, v, idx, topk, scale, o, lse, st)
                      : dispatch_t<64, 128>(d, q, k, v, idx, topk, scale, o, lse, st);
  return r;
}

}  // namespace ssa
