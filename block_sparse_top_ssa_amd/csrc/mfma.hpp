// MFMA tile helpers shared by the attention and top-k kernels (gfx950, bf16 in, fp32 acc).
//
// All products use v_mfma_f32_16x16x32_bf16, oriented so that query rows are the N
// (column) dimension:  S^T[key][row] = sum_d K[key][d] Q[row][d]  and
// O^T[d][row] = sum_key V^T[d][key] P^T[key][row].
// Fragment layout (lane l, g = l / 16): an A fragment holds row l%16 and 8 contraction
// elements, a B fragment holds column l%16 and 8 contraction elements, both in slot
// group g; the contraction index given to (g, j) is the same for A and B, so any
// assignment of contraction indices to slots is valid as long as both operands use it.
// The 16x16 fp32 result holds, in lane l, column l%16 and rows 4g .. 4g+3.
//
// Key order inside a 32-key contraction chunk kc: slot (g, j) carries key
//   kappa(kc, g, j) = 32 kc + 4 g + j          for j < 4
//                   = 32 kc + 16 + 4 g + j - 4 for j >= 4,
// which is exactly where the S^T result tiles 2kc and 2kc+1 leave the probabilities of
// row l%16 in lane l, so P^T needs no data movement between lanes.
#pragma once
#include "common.hpp"

namespace ssa {

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ int kappa(int kc, int g, int j) {
  return 32 * kc + (j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4));
}

// Transpose an 8x8 matrix of 16-bit values held by 8 consecutive lanes (lane p of the
// group holds row p as 4 dwords); afterwards lane p holds column p.
__device__ __forceinline__ u32x4 transpose8x8_b16(u32x4 x) {
  const int p = threadIdx.x & 7;
  {  // swap the off-diagonal 4x4 blocks between lanes p and p^4
    const bool top = (p & 4) == 0;
    const uint32_t s0 = top ? x[2] : x[0], s1 = top ? x[3] : x[1];
    const uint32_t r0 = __shfl_xor(s0, 4), r1 = __shfl_xor(s1, 4);
    if (top) { x[2] = r0; x[3] = r1; } else { x[0] = r0; x[1] = r1; }
  }
  {  // swap the off-diagonal 2x2 blocks inside each 4x4 between lanes p and p^2
    const bool up = (p & 2) == 0;
    const uint32_t s0 = up ? x[1] : x[0], s1 = up ? x[3] : x[2];
    const uint32_t r0 = __shfl_xor(s0, 2), r1 = __shfl_xor(s1, 2);
    if (up) { x[1] = r0; x[3] = r1; } else { x[0] = r0; x[2] = r1; }
  }
  {  // swap single elements inside each 2x2 between lanes p and p^1
    const bool up = (p & 1) == 0;
    const uint32_t h01 = (x[0] >> 16) | (x[1] & 0xFFFF0000u), h23 = (x[2] >> 16) | (x[3] & 0xFFFF0000u);
    const uint32_t l01 = (x[0] & 0xFFFFu) | (x[1] << 16), l23 = (x[2] & 0xFFFFu) | (x[3] << 16);
    const uint32_t r0 = __shfl_xor(up ? h01 : l01, 1), r1 = __shfl_xor(up ? h23 : l23, 1);
    if (up) {
      x[0] = (x[0] & 0xFFFFu) | (r0 << 16);
      x[1] = (x[1] & 0xFFFFu) | (r0 & 0xFFFF0000u);
      x[2] = (x[2] & 0xFFFFu) | (r1 << 16);
      x[3] = (x[3] & 0xFFFFu) | (r1 & 0xFFFF0000u);
    } else {
      x[0] = (r0 & 0xFFFFu) | (x[0] & 0xFFFF0000u);
      x[1] = (r0 >> 16) | (x[1] & 0xFFFF0000u);
      x[2] = (r1 & 0xFFFFu) | (x[2] & 0xFFFF0000u);
      x[3] = (r1 >> 16) | (x[3] & 0xFFFF0000u);
    }
  }
  return x;
}

// Same transpose with DPP lane moves only (no LDS crossbar traffic).
__device__ __forceinline__ u32x4 transpose8x8_b16_dpp(u32x4 x) {
  const int p = threadIdx.x & 7;
  {  // lanes p and p^4: rows shifted by 4 inside each 16-lane row; banks 0,2 hold p < 4
    const int x0 = (int)x[0], x1 = (int)x[1], x2 = (int)x[2], x3 = (int)x[3];
    x[2] = (uint32_t)__builtin_amdgcn_update_dpp(x2, x0, 0x104, 0xF, 0x5, false);  // row_shl:4
    x[3] = (uint32_t)__builtin_amdgcn_update_dpp(x3, x1, 0x104, 0xF, 0x5, false);
    x[0] = (uint32_t)__builtin_amdgcn_update_dpp(x0, x2, 0x114, 0xF, 0xA, false);  // row_shr:4
    x[1] = (uint32_t)__builtin_amdgcn_update_dpp(x1, x3, 0x114, 0xF, 0xA, false);
  }
  {  // lanes p and p^2: quad_perm [2,3,0,1]
    const bool up = (p & 2) == 0;
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(up ? x[1] : x[0]), 0x4E, 0xF, 0xF, false);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(up ? x[3] : x[2]), 0x4E, 0xF, 0xF, false);
    if (up) { x[1] = r0; x[3] = r1; } else { x[0] = r0; x[2] = r1; }
  }
  {  // lanes p and p^1: quad_perm [1,0,3,2], 16-bit halves
    const bool up = (p & 1) == 0;
    const uint32_t h01 = (x[0] >> 16) | (x[1] & 0xFFFF0000u), h23 = (x[2] >> 16) | (x[3] & 0xFFFF0000u);
    const uint32_t l01 = (x[0] & 0xFFFFu) | (x[1] << 16), l23 = (x[2] & 0xFFFFu) | (x[3] << 16);
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(up ? h01 : l01), 0xB1, 0xF, 0xF, false);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)(up ? h23 : l23), 0xB1, 0xF, 0xF, false);
    if (up) {
      x[0] = (x[0] & 0xFFFFu) | (r0 << 16);
      x[1] = (x[1] & 0xFFFFu) | (r0 & 0xFFFF0000u);
      x[2] = (x[2] & 0xFFFFu) | (r1 << 16);
      x[3] = (x[3] & 0xFFFFu) | (r1 & 0xFFFF0000u);
    } else {
      x[0] = (r0 & 0xFFFFu) | (x[0] & 0xFFFF0000u);
      x[1] = (r0 >> 16) | (x[1] & 0xFFFF0000u);
      x[2] = (r1 & 0xFFFFu) | (x[2] & 0xFFFF0000u);
      x[3] = (r1 >> 16) | (x[3] & 0xFFFF0000u);
    }
  }
  return x;
}

// A fragment of K for S^T: keys key0 + l%16, contraction chunk cc (32 values of d),
// slot group g = l/16 holds d = 32 cc + 8 g .. +7 (one 16-byte load).
template <int D>
__device__ __forceinline__ u32x4 load_k_frag(const uint16_t* __restrict__ kh, int key0, int cc) {
  const int l = threadIdx.x & 63;
  return load16(kh + (int64_t)(key0 + (l & 15)) * D + 32 * cc + 8 * (l >> 4));
}

// B fragment of Q^T for S^T: query row `row` (already l%16-specific), chunk cc.
template <int D>
__device__ __forceinline__ u32x4 load_q_frag(const uint16_t* __restrict__ qrow, int cc) {
  const int l = threadIdx.x & 63;
  return load16(qrow + 32 * cc + 8 * (l >> 4));
}

// Raw (untransposed) load for an A fragment of V^T: d-tile dt, key chunk kc.
// Lane l = 16 g + 8 h + p loads V[key0 + kappa(kc, g, p)][16 dt + 8 h .. +7]; after
// transpose8x8_b16 lane l holds V[key0 + kappa(kc, g, 0..7)][16 dt + l%16].
template <int D>
__device__ __forceinline__ u32x4 load_v_raw(const uint16_t* __restrict__ vh, int key0, int dt, int kc) {
  const int l = threadIdx.x & 63;
  const int g = l >> 4, h = (l >> 3) & 1, p = l & 7;
  return load16(vh + (int64_t)(key0 + kappa(kc, g, p)) * D + 16 * dt + 8 * h);
}

// Pack the probabilities of S^T tiles 2kc (p0) and 2kc+1 (p1) into the P^T B fragment.
__device__ __forceinline__ u32x4 pack_p(const float* p0, const float* p1) {
  u32x4 w;
  w[0] = pack_bf16x2(p0[0], p0[1]);
  w[1] = pack_bf16x2(p0[2], p0[3]);
  w[2] = pack_bf16x2(p1[0], p1[1]);
  w[3] = pack_bf16x2(p1[2], p1[3]);
  return w;
}

}  // namespace ssa
