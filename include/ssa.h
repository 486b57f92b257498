/*
 * ssa.h -- C ABI of libssa: the per-layer causal attention forward of both streams of
 * SSA ("Sparse Sparse Attention", Shen et al., arXiv 2511.20102) on AMD Instinct
 * MI355X (gfx950), plus the per-token comparison of the two streams.
 *
 * Citations name the paper's sections as tagged on its v4 summary page.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Tensors      q and o are [B, H, L, D], k and v are [B, Hkv, L, D], row-major
 *               contiguous (D innermost), element type given by ssa_dims.dtype (SSA_BF16
 *               or SSA_F32).  Hkv = ssa_dims.Hkv key/value heads (0 means H) divide the
 *               H query heads into groups of G = H / Hkv consecutive heads that share
 *               one key/value head: query head h reads key/value head h / G (grouped-
 *               query attention, as in the paper's training setup with two key-value
 *               heads, App. C, p. 20).  Every query head selects its own blocks.
 *               Blocks: block size s = ssa_dims.block, n = L / s blocks per sequence; the
 *               query at position t lies in block b_t = t / s.
 *  Pointers     every data pointer is a DEVICE pointer (hipMalloc'd, or torch CUDA
 *               memory); q, k, v, o and k_mean 16-byte aligned, idx, lse, sel_score,
 *               l2_dist and dropped 4-byte aligned.  The caller owns every buffer it
 *               passes.  The library keeps no pointer to them after a call returns and
 *               writes nothing outside the outputs named by a call.  Two calls allocate:
 *               ssa_sparse_attn_fwd on bf16, and ssa_full_attn_fwd on bf16 with o given,
 *               take a transient workspace (see ssa_sparse_attn_fwd).
 *  Stream       `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *               Calls only enqueue work on that stream and return; there is no hidden
 *               synchronisation.  Outputs are valid once the stream reaches that point.
 *  Errors       arguments are checked before anything is enqueued, so a call that
 *               returns an error has done no work.  Checks: required pointers non-NULL
 *               and aligned as above; B, H, L >= 1; Hkv = 0 or Hkv >= 1 dividing H;
 *               D in {64, 128}; block in {64, 128};
 *               L % block == 0; 1 <= topk <= n; dtype known; scale finite and > 0;
 *               B*H*L <= 2^24; the current device is gfx950.  A failed launch returns
 *               SSA_ERR_LAUNCH.  ssa_last_error() gives a thread-local message for the
 *               last failing call.  The library never prints, aborts or throws.
 *  Threads      stateless apart from a per-device properties cache and a per-device
 *               workspace pool, each created once under a lock; calls from several
 *               threads are safe.
 *  Determinism  ssa_block_pool, ssa_block_topk, ssa_full_attn_fwd and ssa_align_stats
 *               are deterministic.  ssa_sparse_attn_fwd accumulates partial sums in an
 *               order that can differ between runs (last-bit fp32 differences, which
 *               can show as one-ulp differences of bf16 outputs).
 */
#ifndef SSA_H_
#define SSA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSA_ABI_VERSION 2 /* 2: ssa_dims.Hkv (grouped-query attention) */

typedef int32_t ssa_status;
enum {
  SSA_OK = 0,
  SSA_ERR_NULL = 1,        /* a required pointer is NULL (or an output pair incomplete) */
  SSA_ERR_SHAPE = 2,       /* bad B/H/L/D/block/topk, L % block != 0, sizes too large */
  SSA_ERR_DTYPE = 3,       /* unknown dtype */
  SSA_ERR_UNSUPPORTED = 4, /* valid but not supported (misaligned pointer, bad scale) */
  SSA_ERR_DEVICE = 5,      /* no device, or the current device is not gfx950 */
  SSA_ERR_LAUNCH = 6       /* the HIP runtime rejected a kernel launch */
};

enum { SSA_F32 = 0, SSA_BF16 = 1 };

typedef struct {
  int32_t B, H, L, D; /* batch, query heads, sequence length, head dim */
  int32_t block;      /* block size s (tokens per block) */
  int32_t dtype;      /* SSA_F32 or SSA_BF16: element type of q, k, v and o */
  int32_t Hkv;        /* key/value heads: 0 (= H) or a divisor of H */
} ssa_dims;

/*
 * ssa_block_pool -- mean-pooled block keys.
 *   Paper sec. 3 (p. 4): tokens are split into contiguous blocks of s, and each block
 *   is represented by the mean of its keys.
 *   k       [B,Hkv,L,D] (dtype)             in
 *   k_mean  [B,Hkv,n,D] float32             out: k_mean[b,h,j,:] = (1/s) sum_{i=js}^{js+s-1}
 *                                           k[b,h,i,:], summed in float32.
 */
ssa_status ssa_block_pool(const ssa_dims* dims, const void* k, float* k_mean, void* stream);

/*
 * ssa_block_topk -- per-query causal top-k block selection.
 *   Paper sec. 3 (p. 4) and App. D (p. 21, the block-scoring stage): each query scores
 *   the blocks before its own with their pooled keys and keeps the best k; its own
 *   block is always kept and counts toward k.
 *   q          [B,H,L,D] (dtype)            in
 *   k_mean     [B,Hkv,n,D] float32          in (as written by ssa_block_pool); query head h
 *                                           scores the pooled keys of key/value head h / G
 *   topk       1 <= topk <= n               blocks kept per query (k)
 *   idx        [B,H,L,topk] int32           out: for the query at t, the blocks j < b_t with
 *              the m = min(topk-1, b_t) largest scores sigma_tj = q_t . k_mean_j (raw dot
 *              product, float32; equal scores go to the lower j), plus b_t, listed in
 *              ascending order; slots m+1..topk-1 hold -1.
 *   sel_score  [B,H,L,topk] float32 or NULL out (optional): the score of each listed block;
 *              +inf for b_t, -inf for the -1 slots.
 */
ssa_status ssa_block_topk(const ssa_dims* dims, const void* q, const float* k_mean, int32_t topk,
                          int32_t* idx, float* sel_score, void* stream);

/*
 * ssa_sparse_attn_fwd -- softmax attention over the tokens of the kept blocks.
 *   Paper sec. 3 (p. 4): the kept blocks' tokens form reduced key and value matrices
 *   for the query; App. D (p. 21, the attend-over-selected-tokens stage).
 *   q        [B,H,L,D] (dtype)               in
 *   k, v     [B,Hkv,L,D] (dtype)             in (query head h attends key/value head h / G)
 *   idx      [B,H,L,topk] int32              in: rows as written by ssa_block_topk (distinct
 *            blocks in ascending order, -1 in unused slots).  The query's own block b_t
 *            is always attended, causally (keys i <= t), whether or not it is listed.
 *            Entries outside [0, b_t), and entries not greater than the entry used before
 *            them, are skipped, so malformed rows cannot make the kernel read outside k/v.
 *   scale    softmax scale (> 0, finite), normally 1/sqrt(D)
 *   o        [B,H,L,D] (dtype)               out: o(t) = sum_{i in A(t)} softmax_i(scale q_t.k_i) v_i,
 *            A(t) = {i <= t : i/s attended}
 *   lse      [B,H,L] float32 or NULL         out (optional): log sum_{i in A(t)} exp(scale q_t.k_i)
 *   Workspace (bf16 only): B*Hkv*L*D*2 bytes holding v in the layout the matrix-core
 *   products read, taken from a stream-ordered memory pool that the library keeps per
 *   device and returned to it on `stream` before the call returns.  The pool keeps the
 *   memory for reuse, so after the first call of a given size the allocation neither
 *   blocks the host nor synchronises the device.  If it cannot be had, the call
 *   returns SSA_ERR_LAUNCH with the HIP message and enqueues nothing else.
 */
ssa_status ssa_sparse_attn_fwd(const ssa_dims* dims, const void* q, const void* k, const void* v,
                               const int32_t* idx, int32_t topk, float scale, void* o, float* lse,
                               void* stream);

/*
 * ssa_full_attn_fwd -- dense causal attention.
 *   Paper sec. 3 (p. 3): every query attends to all preceding tokens (and itself).
 *   q        [B,H,L,D] (dtype)               in
 *   k, v     [B,Hkv,L,D] (dtype)             in (query head h attends key/value head h / G)
 *   o        [B,H,L,D] (dtype) or NULL       out: o(t) = sum_{i<=t} softmax_i(scale q_t.k_i) v_i
 *   lse      [B,H,L] float32 or NULL         out: log sum_{i<=t} exp(scale q_t.k_i)
 *   At least one of o, lse must be given; with o == NULL only the log-sum-exp is
 *   computed (the value products are skipped).
 *   Workspace (bf16 with o given): the same transient B*Hkv*L*D*2-byte copy of v as
 *   ssa_sparse_attn_fwd, from the same pool, with the same error behaviour.
 */
ssa_status ssa_full_attn_fwd(const ssa_dims* dims, const void* q, const void* k, const void* v,
                             float scale, void* o, float* lse, void* stream);

/*
 * ssa_align_stats -- per-token comparison of the full and sparse streams.
 *   Paper sec. 5 (pp. 6-7): the two streams' outputs are compared at every layer;
 *   App. B (p. 19) and sec. 4.2 (p. 6): the dropped attention mass delta(t), the
 *   full-attention probability on tokens the sparse stream does not attend.
 *   o_full, o_sparse      [B,H,L,D] (dtype), both or neither
 *   lse_full, lse_sparse  [B,H,L] float32, both or neither
 *   l2_dist   [B,H,L] float32 or NULL   out: ||o_full(t) - o_sparse(t)||_2 over D (needs the o pair)
 *   dropped   [B,H,L] float32 or NULL   out: clamp(-expm1(lse_sparse - lse_full), 0, 1)
 *                                       (needs the lse pair)
 *   At least one output must be given.
 */
ssa_status ssa_align_stats(const ssa_dims* dims, const void* o_full, const void* o_sparse,
                           const float* lse_full, const float* lse_sparse, float* l2_dist,
                           float* dropped, void* stream);

/* Text for a status code (static storage). */
const char* ssa_status_str(ssa_status status);
/* Message for the last failing call on this thread ("" if none). */
const char* ssa_last_error(void);
/* SSA_ABI_VERSION of the built library. */
int32_t ssa_abi_version(void);

/*
 * Kernel-variant control, for tests that check each code path against the CPU
 * oracle.  0 (default): choose per call (MFMA kernels for bf16 where they apply,
 * portable vector-ALU kernels otherwise).  1: always use the portable kernels.
 * Process-wide; returns the previous value.
 */
int32_t ssa_set_kernel_variant(int32_t variant);

#ifdef __cplusplus
}
#endif
#endif /* SSA_H_ */
