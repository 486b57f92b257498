// Dense causal attention forward (the full stream; paper sec. 3, p. 3: each query
// attends to every preceding token), flash-style on MFMA bf16 with fp32 online softmax.
//
// Work split: a workgroup owns 256 consecutive query rows of one (b, h); each of its 8
// waves owns 32 rows (2 column tiles of 16; two waves per SIMD) and keeps their O^T
// accumulators, running max and partial sums in registers for the whole sweep.  The workgroup sweeps 64-key
// chunks from key 0 to its last row; chunk c+1 is loaded from HBM/L2 into registers
// while chunk c is being used, then written to the other half of a double-buffered
// LDS stage in MFMA-fragment order (K as is; V transposed in registers first), so
// every wave reads its fragments with conflict-free 16-byte LDS reads.  V comes from a
// copy already in fragment order (written by a short pass before this kernel), so
// staging V^T is a plain copy.  A wave stops at its own diagonal chunk, which is masked
// causally.
// Grid order: head-major, tiles with the most chunks first, remapped so that each XCD
// works through a contiguous range (one head at a time), keeping that head's K/V in its
// L2.  The softmax exponent reference is set by the first chunk and moves only when a
// chunk's probabilities would pass 2^64 (seen from their row sums, so no per-element row
// maximum is formed off the diagonal), so the O accumulators are rarely rescaled.
// With o == NULL only the running max and sums are kept (log-sum-exp only).
// Given a sparse stream's idx (full rows of the sparse stream), a workgroup writes only
// the 64-row query chunks whose rows all keep every earlier block -- those rows of the
// sparse stream are exactly causal attention -- and leaves the rest to the sparse kernel.
// With STATS the sweep also gives the attention-pattern measurements of the full stream
// (paper App. H, Table A9: entropy; App. K.2, p. 31: mass by distance) from its own
// probabilities: per row B = sum_i p_i e_i (e_i = log2 p_i against the reference, kept
// through reference moves like l), so entropy = ln l - ln 2 B / l; and per row the mass
// of each distance bucket -- a wave's rows share one block, so a chunk's bucket is the
// same for the whole wave and, chunks coming in order, changes at most 16 times: the
// running bucket mass is kept beside l and flushed to LDS when the bucket changes.  At
// the end each row's bucket masses are divided by its l and summed over the workgroup's
// rows into one partial per (b, h, tile), summed in a fixed order by a second kernel.
// With a sparse stream's idx as well, only the rows of the chunks the workgroup writes are
// measured (the sparse stream's measurements of those rows; a tile with none writes a zero
// partial).
#include <algorithm>

#include "launch.hpp"
#include "mfma.hpp"

namespace ssa {

constexpr float kLag = 8.f;  // max path: log2 units the row max may pass the reference before it moves

// Each wave owns NT = 2 column tiles of 16 rows; waves w and w + 4 share a SIMD and own
// the two 32-row halves of the same 64-row block.  Per 64-key chunk a wave does three
// steps: S (scores, MFMA), X (softmax, VALU) and A (accumulate P V, MFMA).  Between two
// barriers the first wave of a SIMD runs A(c-1), S(c), X(c) and the second runs
// X(c-1), A(c-1), S(c): one wave's matrix products run while its partner's softmax
// does, instead of both waves queueing on the same unit at the same time.  The stage
// of chunk c-1 (its V) is still read while chunk c+1 is written, hence three stages.
template <int D, bool WANT_O, bool STATS>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void full_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const u32x4* __restrict__ vt,
    uint16_t* __restrict__ o, float* __restrict__ lse, int L, int BH, int ntile, float sl2, int G,
    const int32_t* __restrict__ didx, int dtopk, int dS, float* __restrict__ ent, float* __restrict__ hpart) {
  constexpr int NT = 2;        // 16-row column tiles per wave
  constexpr int NW = 8;        // waves per workgroup (256 rows)
  constexpr int NC = D / 32;   // contraction chunks of d for S^T
  constexpr int NDT = D / 16;  // d tiles of O^T
  constexpr int KF = 4 * NC;   // K fragments per 64-key chunk
  constexpr int VF = 2 * NDT;  // V^T fragments per 64-key chunk
  constexpr int KF_W = KF / NW, VF_W = VF / NW;  // fragments each wave loads
  __shared__ u32x4 sk[3][KF][64];
  __shared__ u32x4 sv[WANT_O ? 3 : 1][WANT_O ? VF : 1][64];
  // STATS: per wave, per distance bucket, per row of the wave: flushed bucket masses
  __shared__ float hst[STATS ? NW : 1][STATS ? kDistBuckets : 1][STATS ? 32 : 1];
  __shared__ float hred[STATS ? NW : 1][STATS ? kDistBuckets : 1];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int n = lane & 15, g = lane >> 4;
  const bool late = w >= 4;  // second wave on its SIMD
  // head-major order: the resident workgroups cover few heads, so their K/V stay in
  // the L2 / last-level cache; within a head the tiles with the most work go first
  const int64_t wg = xcd_logical(blockIdx.x, (int64_t)gridDim.x);
  const int64_t bh = wg / ntile;
  const int tile = ntile - 1 - (int)(wg % ntile);
  const uint16_t* qh = q + bh * (int64_t)L * D;
  const int64_t kvh = bh / G;  // K/V head of this query head
  const uint16_t* kh = k + kvh * (int64_t)L * D;
  const u32x4* vth = vt + kvh * (int64_t)(L / 64) * VF * 64;  // per chunk: VF fragments of 64 lanes
  __shared__ int chunk_full[4];  // with didx: 64-row query chunks this workgroup writes
  if (didx) {
    if (threadIdx.x < 4) chunk_full[threadIdx.x] = 1;
    __syncthreads();
    const int t = tile * 256 + (int)threadIdx.x;
    if (threadIdx.x < 256 && t < L && !row_keeps_all(didx + (bh * (int64_t)L + t) * dtopk, dtopk, t / dS))
      chunk_full[threadIdx.x / 64] = 0;
    __syncthreads();
    if (!(chunk_full[0] | chunk_full[1] | chunk_full[2] | chunk_full[3])) {  // uniform
      if constexpr (STATS)
        if (hpart && threadIdx.x < kDistBuckets) hpart[((int64_t)bh * ntile + tile) * kDistBuckets + threadIdx.x] = 0.f;
      return;
    }
  }
  const int rq = late ? 32 : 0;              // row offset inside the diagonal chunk
  const int r0 = tile * 256 + 64 * (w & 3) + rq;  // first row of this wave
  const bool active = r0 < L;
  const int cw = r0 / 64;                    // this wave's diagonal chunk
  const int cmax = min(tile * 4 + 3, L / 64 - 1);

  u32x4 qf[NT][NC];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int cc = 0; cc < NC; ++cc)
      qf[nt][cc] = active ? load_q_frag<D>(qh + (int64_t)(r0 + 16 * nt + n) * D, cc) : u32x4{0, 0, 0, 0};

  f32x4 oacc[WANT_O ? NDT : 1][NT];
  float m[NT], lsum[NT];
  float eb[NT], hb[NT];  // STATS: sum p e and the running bucket's mass (lane partials)
  int cur_b = -1;        // STATS: the running bucket (wave-uniform)
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m[nt] = -__builtin_huge_valf();
    lsum[nt] = 0.f;
    eb[nt] = hb[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < (WANT_O ? NDT : 1); ++dt) oacc[dt][nt] = f32x4{0, 0, 0, 0};
  }
  if constexpr (STATS) {
#pragma unroll
    for (int i = 0; i < kDistBuckets * 32 / 64; ++i) (&hst[w][0][0])[i * 64 + lane] = 0.f;
  }
  const int bt = r0 / dS;  // the block of this wave's rows
  // STATS: the running bucket's mass of each row goes to LDS (summed over its 4 lanes)
  auto flush = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float x = hb[nt];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      if (g == 0) hst[w][b][16 * nt + n] += x;
      hb[nt] = 0.f;
    }
  };

  // Each wave copies its share of every chunk's K and V^T fragments from global memory
  // into the LDS stages, through one of two register sets: the loads for chunk c + 2
  // are issued during interval c, and the set loaded one interval earlier
  // (chunk c + 1) is written out at its end.  The loads are unconditional (the chunk
  // index is clamped) so the compiler can count them exactly and wait only for the
  // older set.
  u32x4 kA[KF_W], vA[VF_W], kB[KF_W], vB[VF_W];
  auto issue_loads = [&](u32x4* kr, u32x4* vr, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < KF_W; ++i) {
      const int f = w * KF_W + i;
      kr[i] = load_k_frag<D>(kh, c * 64 + 16 * (f / NC), f % NC);
    }
    if (WANT_O) {
#pragma unroll
      for (int i = 0; i < VF_W; ++i) vr[i] = vth[((int64_t)c * VF + w * VF_W + i) * 64 + lane];
    }
  };
  auto stage_store = [&](const u32x4* kr, const u32x4* vr, int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < KF_W; ++i) sk[st][w * KF_W + i][lane] = kr[i];
    if (WANT_O) {
#pragma unroll
      for (int i = 0; i < VF_W; ++i) sv[st][w * VF_W + i][lane] = vr[i];
    }
  };

  f32x4 sacc[4][NT];
  u32x4 pf[NT][2];
  // S: S^T tiles of the chunk in stage st.  The first half of the K fragments is read
  // before any product; the second half is read one fragment per pair of products of
  // the first half (scheduling-group barriers keep that order), so the LDS latency is
  // paid once per chunk and the reads run eight fragments ahead of their use.
  auto scores = [&](int st) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[kt][nt] = f32x4{0, 0, 0, 0};
    u32x4 kf[KF];
#pragma unroll
    for (int f = 0; f < KF / 2; ++f) kf[f] = sk[st][(f % 4) * NC + f / 4][lane];  // cc-major order
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < KF / 2; ++f) {  // first half's products, second half's reads between them
      const int cc = f / 4, kt = f % 4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[kt][nt] = mfma_bf16(kf[f], qf[nt][cc], sacc[kt][nt]);
      const int fg = KF / 2 + f;
      kf[fg] = sk[st][(fg % 4) * NC + fg / 4][lane];
      __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = KF / 2; f < KF; ++f) {
      const int cc = f / 4, kt = f % 4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[kt][nt] = mfma_bf16(kf[f], qf[nt][cc], sacc[kt][nt]);
    }
  };
  // X: online softmax of sacc into pf (bf16 P^T fragments), m, lsum and O rescaling.
  // Off the diagonal the exponents are taken against the current reference m straight
  // away, and the row sums of the result show whether that was safe: a first chunk
  // (m = -inf gives p = +inf) or a chunk whose p would pass 2^64 redoes the chunk on the
  // max path, as does the diagonal chunk (masked).  The max path moves m only when the
  // row maximum passes it by more than kLag (the row maximum across the four lanes of a
  // row is formed only when some lane's own maximum passes), rescaling O and l.  p up to
  // 2^64 keeps O and l far from the float32 range even over the longest rows.
  auto softmax = [&](bool diag, int c) __attribute__((always_inline)) {
    if constexpr (STATS) {
      const int bk = dist_bucket(bt - c * 64 / dS);
      if (bk != cur_b) {
        if (cur_b >= 0) flush(cur_b);
        cur_b = bk;
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float sr[16];
      float ps = 0.f, pe = 0.f;
      if (!diag) {
        const float mneg = -m[nt];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float e = fmaf(sacc[kt][nt][i], sl2, mneg);
            sr[kt * 4 + i] = fast_exp2(e);
            ps += sr[kt * 4 + i];
            if constexpr (STATS) pe = fmaf(sr[kt * 4 + i], e, pe);
          }
      }
      if (diag || __builtin_amdgcn_ballot_w64(!(ps <= 0x1p64f))) {
        float mx = -__builtin_huge_valf();
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = sacc[kt][nt][i];
            if (diag && (16 * kt + 4 * g + i > rq + 16 * nt + n)) x = -__builtin_huge_valf();
            sr[kt * 4 + i] = x;
            mx = fmaxf(mx, x);
          }
        if (__builtin_amdgcn_ballot_w64(mx * sl2 > m[nt] + kLag)) {
          const float mxs = max_over_rows(mx) * sl2;
          const bool need = mxs > m[nt] + kLag;
          const float mnew = need ? mxs : m[nt];
          const float alpha = fast_exp2(m[nt] - mnew);
          if constexpr (STATS) {  // e moves by m - mnew: B' = alpha (B + (m - mnew) l)
            eb[nt] = lsum[nt] > 0.f ? alpha * fmaf(m[nt] - mnew, lsum[nt], eb[nt]) : 0.f;  // first chunk: m = -inf
            hb[nt] *= alpha;
            if (g == 0)
#pragma unroll
              for (int b = 0; b < kDistBuckets; ++b) hst[w][b][16 * nt + n] *= alpha;
          }
          lsum[nt] *= alpha;
          if (WANT_O) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) oacc[dt][nt] *= alpha;
          }
          m[nt] = mnew;
        }
        const float mneg = -m[nt];
        ps = 0.f;
        pe = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float e = fmaf(sr[i], sl2, mneg);
          sr[i] = fast_exp2(e);
          ps += sr[i];
          if constexpr (STATS) pe = fmaf(sr[i], fmaxf(e, -0x1p100f), pe);  // masked keys: p = 0
        }
      }
      lsum[nt] += ps;
      if constexpr (STATS) {
        eb[nt] += pe;
        hb[nt] += ps;
      }
      if (WANT_O) {
        pf[nt][0] = pack_p(&sr[0], &sr[4]);
        pf[nt][1] = pack_p(&sr[8], &sr[12]);
      }
    }
  };
  // A: O^T += V^T P^T for the chunk in stage st (V^T fragments read as for S)
  auto accumulate = [&](int st) {
    u32x4 vf[VF];
#pragma unroll
    for (int f = 0; f < VF / 2; ++f) vf[f] = sv[st][f][lane];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < VF / 2; ++f) {  // fragment dt * 2 + kc
      const int dt = f / 2, kc = f % 2;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) oacc[dt][nt] = mfma_bf16(vf[f], pf[nt][kc], oacc[dt][nt]);
      vf[VF / 2 + f] = sv[st][VF / 2 + f][lane];
      __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = VF / 2; f < VF; ++f) {
      const int dt = f / 2, kc = f % 2;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) oacc[dt][nt] = mfma_bf16(vf[f], pf[nt][kc], oacc[dt][nt]);
    }
  };

  // A then S in one stream: the V^T fragments of stage sv_st and then the K fragments
  // of stage sk_st, every read eight fragments ahead of its products except the first
  // eight; mid() runs between the two halves of the value products.
  auto acc_scores = [&](int sv_st, int sk_st, auto&& mid) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[kt][nt] = f32x4{0, 0, 0, 0};
    u32x4 vf[VF], kf[KF];
#pragma unroll
    for (int f = 0; f < VF / 2; ++f) vf[f] = sv[sv_st][f][lane];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < VF / 2; ++f) {
      const int dt = f / 2, kc = f % 2;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) oacc[dt][nt] = mfma_bf16(vf[f], pf[nt][kc], oacc[dt][nt]);
      vf[VF / 2 + f] = sv[sv_st][VF / 2 + f][lane];
      __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    mid();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = VF / 2; f < VF; ++f) {
      const int dt = f / 2, kc = f % 2;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) oacc[dt][nt] = mfma_bf16(vf[f], pf[nt][kc], oacc[dt][nt]);
      const int fk = f - VF / 2;
      if (fk < KF / 2) {
        kf[fk] = sk[sk_st][(fk % 4) * NC + fk / 4][lane];
        __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < KF / 2; ++f) {
      const int cc = f / 4, kt = f % 4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[kt][nt] = mfma_bf16(kf[f], qf[nt][cc], sacc[kt][nt]);
      const int fg = KF / 2 + f;
      kf[fg] = sk[sk_st][(fg % 4) * NC + fg / 4][lane];
      __builtin_amdgcn_sched_group_barrier(0x008, NT, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = KF / 2; f < KF; ++f) {
      const int cc = f / 4, kt = f % 4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sacc[kt][nt] = mfma_bf16(kf[f], qf[nt][cc], sacc[kt][nt]);
    }
  };

  issue_loads(kA, vA, 0);
  issue_loads(kB, vB, min(1, cmax));
  stage_store(kA, vA, 0);
  __syncthreads();

  int s0 = 0;  // stage holding chunk c; chunk c - 1 is in sp, chunk c + 1 goes to s1
  // one interval: loads into set (kL, vL), chunk c + 1 written out from set (kS, vS)
  auto interval = [&](int c, u32x4* kL, u32x4* vL, const u32x4* kS, const u32x4* vS)
                      __attribute__((always_inline)) {
    const int s1 = s0 == 2 ? 0 : s0 + 1;
    const int sp = s0 == 0 ? 2 : s0 - 1;
    const bool prev = active && c >= 1 && c - 1 <= cw;  // chunk c - 1 still to finish
    const bool cur = active && c <= cw;                 // chunk c to start
    // (the causal mask is compiled only into the diagonal chunk's softmax)
    if (late && prev) {
      if (c - 1 == cw) softmax(true, c - 1);
      else softmax(false, c - 1);
    }
    // Steady state: the value products of chunk c - 1 and the score products of chunk c
    // as one pipelined stream (acc_scores); the loads for chunk c + 2 go out between
    // them rather than at the start: the compiler waits for the older set before
    // reusing the registers, and by then it has landed.
    if (WANT_O && prev && cur) {
      acc_scores(sp, s0, [&]() __attribute__((always_inline)) { issue_loads(kL, vL, min(c + 2, cmax)); });
    } else {
      if (WANT_O && prev) accumulate(sp);
      issue_loads(kL, vL, min(c + 2, cmax));
      if (cur) scores(s0);
    }
    if (!late && cur) {
      if (c == cw) softmax(true, c);
      else softmax(false, c);
    }
    // Unconditional, like the loads, so the compiler's load counting stays exact: past
    // the last chunk the stage written holds a chunk that no wave reads again.
    stage_store(kS, vS, s1);
    __syncthreads();
    s0 = s1;
  };
  for (int c = 0; c <= cmax + 1; c += 2) {
    interval(c, kA, vA, kB, vB);
    if (c + 1 <= cmax + 1) interval(c + 1, kB, vB, kA, vA);
  }

  if constexpr (STATS) {
    // entropy of each row; the workgroup's bucket masses, each row's divided by its l
    // (with didx only the rows of the chunks this workgroup writes)
    float hw[4] = {0.f, 0.f, 0.f, 0.f};  // buckets 4 g .. 4 g + 3, this lane's rows
    if (active && (!didx || chunk_full[w & 3])) {
      if (cur_b >= 0) flush(cur_b);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float l = lsum[nt], e = eb[nt];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        e += __shfl_xor(e, 16);
        e += __shfl_xor(e, 32);
        const float inv = 1.f / l;
        if (ent && g == 0) ent[bh * (int64_t)L + r0 + 16 * nt + n] = logf(l) - kLn2 * e * inv;
#pragma unroll
        for (int j = 0; j < 4; ++j) hw[j] = fmaf(hst[w][4 * g + j][16 * nt + n], inv, hw[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // sum over the wave's rows (lanes n)
      float x = hw[j];
      x += __shfl_xor(x, 1);
      x += __shfl_xor(x, 2);
      x += __shfl_xor(x, 4);
      x += __shfl_xor(x, 8);
      if (n == 0) hred[w][4 * g + j] = x;
    }
    __syncthreads();
    if (hpart && threadIdx.x < kDistBuckets) {
      float x = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) x += hred[ww][threadIdx.x];
      hpart[((int64_t)bh * ntile + tile) * kDistBuckets + threadIdx.x] = x;
    }
  }
  if (!active || (didx && !chunk_full[w & 3])) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = lsum[nt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int row = r0 + 16 * nt + n;
    if (WANT_O) {
      const float inv = 1.f / l;
      uint16_t* orow = o + (bh * (int64_t)L + row) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        u32x2 pk;
        pk[0] = pack_bf16x2(oacc[dt][nt][0] * inv, oacc[dt][nt][1] * inv);
        pk[1] = pack_bf16x2(oacc[dt][nt][2] * inv, oacc[dt][nt][3] * inv);
        *reinterpret_cast<u32x2*>(orow + 16 * dt + 4 * g) = pk;
      }
    }
    if (lse && g == 0) lse[bh * (int64_t)L + row] = (m[nt] + log2f(l)) * kLn2;
  }
}

bool full_mfma_supported(const Dims& d) { return d.dtype == 1 && (d.D == 64 || d.D == 128) && d.L % 64 == 0; }

template <int D, bool WANT_O, bool STATS = false>
static hipError_t run_full(const Dims& d, const void* q, const void* k, const u32x4* vt, float scale, void* o,
                           float* lse, hipStream_t st, const int32_t* didx = nullptr, int dtopk = 0,
                           float* ent = nullptr, float* hpart = nullptr) {
  // with didx only rows whose block b_t <= topk can keep every earlier block (b_t
  // distinct valid entries below b_t), i.e. t < (topk + 1) * s
  const int rows = didx ? (int)std::min<int64_t>(d.L, ((int64_t)dtopk + 1) * d.S) : d.L;
  const int ntile = (rows + 255) / 256;
  const int64_t grid = (int64_t)ntile * d.bh();
  hipLaunchKernelGGL((full_fwd_kernel<D, WANT_O, STATS>), dim3((unsigned)grid), dim3(512), 0, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     vt, static_cast<uint16_t*>(o), lse, d.L, (int)d.bh(), ntile,
                     scale * kLog2e, d.G(), didx, dtopk, d.S, ent, hpart);
  return hipGetLastError();
}

hipError_t launch_full_rows_of_sparse(const Dims& d, const void* q, const void* k, const u32x4* vt,
                                      const int32_t* idx, int topk, float scale, void* o, float* lse,
                                      hipStream_t st, float* ent, float* hpart) {
  if (ent || hpart)
    return d.D == 128 ? run_full<128, true, true>(d, q, k, vt, scale, o, lse, st, idx, topk, ent, hpart)
                      : run_full<64, true, true>(d, q, k, vt, scale, o, lse, st, idx, topk, ent, hpart);
  return d.D == 128 ? run_full<128, true>(d, q, k, vt, scale, o, lse, st, idx, topk)
                    : run_full<64, true>(d, q, k, vt, scale, o, lse, st, idx, topk);
}

LaunchResult launch_full_mfma_stats(const Dims& d, const void* q, const void* k, const void* v, float scale,
                                    void* o, float* lse, float* entropy, float* hist, hipStream_t st) {
  LaunchResult r;
  const int ntile = (d.L + 255) / 256;
  void* hws = nullptr;
  float* hpart = nullptr;
  if (hist) {
    r.err = workspace_alloc((size_t)d.bh() * ntile * kDistBuckets * sizeof(float), &hws, st);
    if (r.err != hipSuccess) return r;
    hpart = static_cast<float*>(hws);
  }
  if (o) {
    void* ws = nullptr;
    r.err = vfrag_acquire(d.kv(), v, &ws, st);
    if (r.err == hipSuccess) {
      const u32x4* vt = static_cast<const u32x4*>(ws);
      r.err = d.D == 128 ? run_full<128, true, true>(d, q, k, vt, scale, o, lse, st, nullptr, 0, entropy, hpart)
                         : run_full<64, true, true>(d, q, k, vt, scale, o, lse, st, nullptr, 0, entropy, hpart);
      const hipError_t ef = vfrag_release(ws, st);
      if (r.err == hipSuccess) r.err = ef;
    }
  } else {
    r.err = d.D == 128 ? run_full<128, false, true>(d, q, k, nullptr, scale, o, lse, st, nullptr, 0, entropy, hpart)
                       : run_full<64, false, true>(d, q, k, nullptr, scale, o, lse, st, nullptr, 0, entropy, hpart);
  }
  if (r.err == hipSuccess && hist) r.err = launch_hist_sum(hpart, hist, d.bh(), ntile, st);
  if (hws) {
    const hipError_t ef = vfrag_release(hws, st);
    if (r.err == hipSuccess) r.err = ef;
  }
  return r;
}

LaunchResult launch_full_mfma_frag(const Dims& d, const void* q, const void* k, const u32x4* vt, float scale,
                                   void* o, float* lse, hipStream_t st) {
  LaunchResult r;
  if (o)
    r.err = d.D == 128 ? run_full<128, true>(d, q, k, vt, scale, o, lse, st)
                       : run_full<64, true>(d, q, k, vt, scale, o, lse, st);
  else  // log-sum-exp only: V is not read
    r.err = d.D == 128 ? run_full<128, false>(d, q, k, nullptr, scale, o, lse, st)
                       : run_full<64, false>(d, q, k, nullptr, scale, o, lse, st);
  return r;
}

LaunchResult launch_full_mfma(const Dims& d, const void* q, const void* k, const void* v, float scale, void* o,
                              float* lse, hipStream_t st) {
  if (!o) return launch_full_mfma_frag(d, q, k, nullptr, scale, o, lse, st);
  LaunchResult r;
  void* ws = nullptr;
  r.err = vfrag_acquire(d.kv(), v, &ws, st);
  if (r.err != hipSuccess) return r;
  r = launch_full_mfma_frag(d, q, k, static_cast<const u32x4*>(ws), scale, o, lse, st);
  const hipError_t ef = vfrag_release(ws, st);
  if (r.err == hipSuccess) r.err = ef;
  return r;
}

}  // namespace ssa
