// Internal launcher interface between the C ABI (api.hip) and the kernel files.
#pragma once
#include "common.hpp"

namespace ssa {

struct Dims {
  int B, H, L, D, S, dtype;  // S = block size; dtype 0 = f32, 1 = bf16
  int Hkv;                   // key/value heads (divides H); query head h reads K/V head h / G
  int n() const { return L / S; }
  int64_t bh() const { return (int64_t)B * H; }
  int64_t tokens() const { return (int64_t)B * H * L; }
  // query heads per K/V head; flat query head bh = b*H + h reads flat K/V head bh / G()
  int G() const { return H / Hkv; }
  // the same shape seen from the K/V heads (for k, v and the pooled keys)
  Dims kv() const {
    Dims k = *this;
    k.H = Hkv;
    return k;
  }
};

// Reports the reason a launcher refused a shape it cannot handle (no launch done).
struct LaunchResult {
  hipError_t err = hipSuccess;
  const char* unsupported = nullptr;
};

LaunchResult launch_pool(const Dims& d, const void* k, float* k_mean, hipStream_t st);
LaunchResult launch_align(const Dims& d, const void* o_full, const void* o_sparse, const float* lse_full,
                          const float* lse_sparse, float* dist, float* dropped, hipStream_t st,
                          float* retained_hist = nullptr);

// Portable vector-ALU kernels (any dtype, D in {64,128}).
LaunchResult launch_topk_generic(const Dims& d, const void* q, const float* k_mean, int topk, int32_t* idx,
                                 float* sel, hipStream_t st);
LaunchResult launch_sparse_generic(const Dims& d, const void* q, const void* k, const void* v,
                                   const int32_t* idx, int topk, float scale, void* o, float* lse,
                                   hipStream_t st);
LaunchResult launch_full_generic(const Dims& d, const void* q, const void* k, const void* v, float scale,
                                 void* o, float* lse, hipStream_t st);

// V of a bf16 [B,H,L,D] tensor rewritten into MFMA fragment order: per (b,h), 64-key
// chunk c, 16-column tile dt and key half kc, 64 lanes x 16 bytes, lane 16 g + i holding
// V[64 c + kappa(kc, g, 0..7)][16 dt + i].  d holds the key/value head count in H (callers
// pass Dims::kv()), so the buffer is B*Hkv*L*D*2 bytes; it comes from a stream-ordered
// pool kept per device; give it back with vfrag_release on the same stream.
hipError_t vfrag_acquire(const Dims& d, const void* v, void** ws, hipStream_t st);
hipError_t vfrag_release(void* ws, hipStream_t st);
// K of a bf16 [B,H,L,D] tensor in MFMA fragment order (the A operand of S^T = K Q^T):
// per (b,h), 64-key chunk c, key tile kt and contraction chunk cc, 64 lanes x 16 bytes,
// lane 16 g + i holding K[64 c + 16 kt + i][32 cc + 8 g .. +7]; B*H*L*D*2 bytes from the
// same pool (d holds the key/value head count in H), given back with vfrag_release.
hipError_t kfrag_acquire(const Dims& d, const void* k, void** ws, hipStream_t st);
// Both rewrites into caller-given buffers of B*H*L*D*2 bytes each (d holds the key/value
// head count in H): kf as kfrag_acquire's copy of k, vf as vfrag_acquire's copy of v;
// a null kf or vf skips that copy.
hipError_t kv_frag_into(const Dims& d, const void* k, const void* v, void* kf, void* vf, hipStream_t st);
// The same rewrite of any bf16 [B,H,L,D] tensor (d.H heads) into a caller-given buffer.
hipError_t frag_order_into(const Dims& d, const void* x, void* out, hipStream_t st);

// Transient device memory from the same per-device stream-ordered pool: valid for work
// enqueued on `st` after the call, given back with workspace_free on the same stream.
hipError_t workspace_alloc(size_t bytes, void** ws, hipStream_t st);
hipError_t workspace_free(void* ws, hipStream_t st);

// Decoding with a key/value cache (one query per sequence; d.L = cache capacity).
bool decode_sparse_supported(const Dims& d);
LaunchResult launch_decode_append(const Dims& d, const int32_t* pos, const void* k_new, const void* v_new,
                                  void* k_cache, void* v_cache, float* k_mean, hipStream_t st);
LaunchResult launch_decode_sparse(const Dims& d, const int32_t* pos, const void* q, const void* k_cache,
                                  const void* v_cache, const float* k_mean, int topk, float scale, void* o, float* lse,
                                  int32_t* idx, hipStream_t st);
// The same selection and sparse attention with its scratch in a fixed 16 MiB device array
// (no allocation); bytes it needs (decode_sparse_scratch_bytes) above that are refused.
constexpr size_t kDecodeScratchMax = size_t(16) << 20;
size_t decode_sparse_scratch_bytes(const Dims& d, int topk, bool own_idx);
LaunchResult launch_decode_sparse_noalloc(const Dims& d, const int32_t* pos, const void* q, const void* k_cache,
                                          const void* v_cache, const float* k_mean, int topk, float scale, void* o,
                                          float* lse, int32_t* idx, hipStream_t st);
LaunchResult launch_decode_full(const Dims& d, const int32_t* pos, const void* q, const void* k_cache,
                                const void* v_cache, float scale, void* o, float* lse, hipStream_t st);

// Training: backward of one stream's attention forward (gradients accumulated into the
// float32 dq [B,H,L,D], dk and dv [B,Hkv,L,D]) and the SmoothL1 alignment loss.
LaunchResult launch_attn_bwd(const Dims& d, bool sparse, bool mfma, const void* q, const void* k, const void* v,
                             const void* o, const float* lse, const void* dout, const int32_t* idx, int topk,
                             float scale, float* dq, float* dk, float* dv, hipStream_t st);
// MFMA backward (bf16): dq, dk, dv += ..., given delta [B*H*L]; with idx (the sparse
// stream) dk, dv use the inverted index off/list (block -> rows that kept it, as built in
// bwd.hip) and dq the gathered-row kernel, which builds its own per-tile index from idx.
bool full_bwd_mfma_supported(const Dims& d);
bool sparse_bwd_mfma_supported(const Dims& d, int topk);
hipError_t launch_full_bwd_mfma(const Dims& d, const int32_t* idx, int topk, const int* off, const int* list,
                                const void* q, const void* k, const void* v, const void* dout, const float* lse,
                                const float* delta, float scale, float* dq, float* dk, float* dv, hipStream_t st);
// Sparse-stream dq on MFMA over gathered rows: dq += scale sum ds k over each row's kept
// blocks and own block; ktf is K in fragment order (frag_order_into of the K/V heads).
bool dq_gather_supported(const Dims& d, int topk);
hipError_t launch_dq_gather(const Dims& d, const void* q, const void* k, const void* v, const void* dout,
                            const u32x4* ktf, const float* lse, const float* delta, const int32_t* idx, int topk,
                            float scale, float* dq, hipStream_t st);
// Per-row bit masks of the blocks the sparse stream attends (word j / 32, bit j % 32 of
// row t: a valid kept entry of idx, or the own block); [B*H*L][ceil(n/32)] words.
hipError_t build_block_mask(const Dims& d, const int32_t* idx, int topk, uint32_t* mask, hipStream_t st);

// Sparse-stream measurements over gathered rows: the tile (512 or 256 rows) whose index fits
// in LDS, 0 if none; part gets ceil(L / tile) histogram partials per (b, h), in order.
int stats_gather_tile(const Dims& d, int topk);
hipError_t launch_stats_gather(const Dims& d, const void* q, const void* k, const float* lse, const int32_t* idx,
                               int topk, float scale, float* entropy, float* part, hipStream_t st);
// Attention-pattern measurements: row entropy and attention mass by block distance.
LaunchResult launch_attn_stats(const Dims& d, bool mfma, const void* q, const void* k, const float* lse,
                               const int32_t* idx, int topk, float scale, float* entropy, float* hist,
                               hipStream_t st);
LaunchResult launch_align_loss(const Dims& d, const void* of, const void* os, float alpha, float beta, float* loss,
                               float* gf, float* gs, hipStream_t st);

// MFMA kernels (bf16 only).  *_supported() tells whether the shape fits.
bool topk_mfma_supported(const Dims& d, int topk);
LaunchResult launch_topk_mfma(const Dims& d, const void* q, const float* k_mean, int topk, int32_t* idx,
                              float* sel, hipStream_t st);
bool full_mfma_supported(const Dims& d);
LaunchResult launch_full_mfma(const Dims& d, const void* q, const void* k, const void* v, float scale,
                              void* o, float* lse, hipStream_t st);
// The same with v already in fragment order (vt as written by vfrag_acquire; unused, and
// may be null, when o is null): no workspace.
LaunchResult launch_full_mfma_frag(const Dims& d, const void* q, const void* k, const u32x4* vt, float scale,
                                   void* o, float* lse, hipStream_t st);
// The same with the full stream's measurements from the sweep's own probabilities:
// entropy [B,H,L] and the distance histogram [B,H,kDistBuckets] (either may be null).
LaunchResult launch_full_mfma_stats(const Dims& d, const void* q, const void* k, const void* v, float scale,
                                    void* o, float* lse, float* entropy, float* hist, hipStream_t st);
// The unfused sparse form: the sparse forward (matrix-core kernel if mfma and the shape
// fits, else the portable one), then the measurement pass over its lse.
LaunchResult launch_sparse_stats_unfused(const Dims& d, bool mfma, const void* q, const void* k, const void* v,
                                         const int32_t* idx, int topk, float scale, void* o, float* lse,
                                         float* entropy, float* hist, hipStream_t st);
// The unfused form: the full forward, then the measurement pass over its lse.
LaunchResult launch_full_stats_unfused(const Dims& d, const void* q, const void* k, const void* v, float scale,
                                       void* o, float* lse, float* entropy, float* hist, hipStream_t st);
// hist[bh][m] = sum over the P partials part[bh][p][m], in order (one kernel).
hipError_t launch_hist_sum(const float* part, float* hist, int64_t bh, int P, hipStream_t st);
// The dense kernel over the sparse stream's full rows: writes o and lse of the 64-row
// query chunks whose rows all keep every earlier block (row_keeps_all), nothing else.
// With ent or hpart it also writes those rows' entropy and one distance-histogram partial
// per (b, h, 256-row tile) of the rows t < (topk + 1) * block (0 where it writes no row).
hipError_t launch_full_rows_of_sparse(const Dims& d, const void* q, const void* k, const u32x4* vt,
                                      const int32_t* idx, int topk, float scale, void* o, float* lse,
                                      hipStream_t st, float* ent = nullptr, float* hpart = nullptr);
bool sparse_mfma_supported(const Dims& d, int topk);
// The sparse forward with the sparse stream's measurements from its own sweep (entropy
// [B,H,L], distance histogram [B,H,kDistBuckets]; either may be null): the tile that fits
// the measurement state in LDS, and the launcher (transient copies and partials from the pool).
bool sparse_mfma_stats_supported(const Dims& d, int topk);
LaunchResult launch_sparse_mfma_stats(const Dims& d, const void* q, const void* k, const void* v, const int32_t* idx,
                                      int topk, float scale, void* o, float* lse, float* ent, float* hist,
                                      hipStream_t st);
LaunchResult launch_sparse_mfma(const Dims& d, const void* q, const void* k, const void* v,
                                const int32_t* idx, int topk, float scale, void* o, float* lse,
                                hipStream_t st);
// The same with k and v already in fragment order (kt, vt as kfrag_acquire and
// vfrag_acquire write them): no workspace.
LaunchResult launch_sparse_mfma_frag(const Dims& d, const void* q, const void* k, const void* v, const u32x4* kt,
                                     const u32x4* vt, const int32_t* idx, int topk, float scale, void* o, float* lse,
                                     hipStream_t st);

}  // namespace ssa
