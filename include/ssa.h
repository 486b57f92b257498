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
 *               memory); q, k, v, o, k_mean and the caches 16-byte aligned, idx, pos,
 *               lse, sel_score, l2_dist and dropped 4-byte aligned.  The caller owns every
 *               buffer it passes.  The library keeps no pointer to them after a call
 *               returns and writes nothing outside the outputs named by a call.  These
 *               calls take a transient workspace from a per-device stream-ordered pool
 *               (sizes and error behaviour under ssa_sparse_attn_fwd and each call):
 *                 - ssa_block_topk (bf16)
 *                 - ssa_sparse_attn_fwd (bf16)
 *                 - ssa_full_attn_fwd (bf16, with o given)
 *                 - ssa_decode_sparse_fwd, ssa_decode_full_fwd
 *                 - ssa_full_attn_bwd, ssa_sparse_attn_bwd
 *                 - ssa_full_attn_fwd_stats, ssa_sparse_attn_fwd_stats
 *                 - ssa_attn_stats, ssa_align_loss
 *               ssa_decode_sparse_fwd_noalloc allocates nothing (a fixed device array);
               ssa_kv_frag, ssa_sparse_attn_fwd_frag and ssa_full_attn_fwd_frag allocate
               nothing (the copies are buffers the caller owns).
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
 *  Threads      stateless apart from a per-device properties cache, a per-device
 *               workspace pool and the per-device address of the allocation-free
 *               call's scratch array, each created once under a lock, and the
 *               process-wide kernel choice of ssa_set_kernel_variant (an atomic read
 *               by every call).  Calls from several threads are safe, except that
 *               ssa_decode_sparse_fwd_noalloc calls overlapping on one device race.
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

#define SSA_ABI_VERSION 9 /* 2: Hkv; 3: decoding; 4: backward and alignment loss; 5: attention stats;
                             6: allocation-free sparse decoding; 7: measurements fused into the full
                             forward and the stream comparison; 8: caller-owned fragment-order
                             copies of k and v shared by both forwards; 9: measurements fused
                             into the sparse forward */

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
 *   Workspace (bf16 with topk <= 65 and n <= 65536): B*Hkv*ceil(n/64)*(64*D*6 + 4)
 *   bytes holding k_mean split into three bf16 terms in the layout the matrix-core products
 *   read, from the stream-ordered pool described under ssa_sparse_attn_fwd, with the same
 *   error behaviour.
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
 *   Workspace (bf16 only): 2*B*Hkv*L*D*2 bytes holding v and k in the layouts the
 *   matrix-core products read, taken from a stream-ordered memory pool that the library keeps per
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
 * Key and value layouts shared by the two forwards (bf16).
 *   Both streams of a layer read the same keys and values (sec. 5, pp. 6-7: the full and
 *   the sparse stream run side by side on one layer's q, k, v).  On bf16 the matrix-core
 *   kernels read v, and the sparse kernel also k, in the order of their operands, so
 *   ssa_sparse_attn_fwd and ssa_full_attn_fwd each rewrite them into a transient copy.  A
 *   caller running both can write the copies once into buffers it owns with ssa_kv_frag
 *   and pass them to the _frag forms below, which take no workspace at all.  The layouts
 *   are internal to this library version: use a copy only with the k, v it was written
 *   from, and write it again after k or v change.
 *
 * ssa_kv_frag_bytes -- size of one copy.
 *   bytes    out: B*Hkv*L*D*2 for bf16, 0 for float32 (no copy exists; the _frag forms
 *            then ignore k_frag and v_frag).  dims is checked as for the forwards.
 */
ssa_status ssa_kv_frag_bytes(const ssa_dims* dims, int64_t* bytes);

/*
 * ssa_kv_frag -- write k and/or v in the operand layouts.
 *   k, v       [B,Hkv,L,D] bf16                      in (each needed only with its copy)
 *   k_frag     ssa_kv_frag_bytes bytes or NULL       out: k as the sparse kernel's score
 *              operand reads it (per 64-key chunk, 16-key tile and 32-column slice, one
 *              contiguous 1 KB fragment)
 *   v_frag     ssa_kv_frag_bytes bytes or NULL       out: v as both forwards' value-product
 *              operand reads it (per 64-key chunk, 16-column tile and key half, one 1 KB
 *              fragment)
 *   At least one copy must be asked for; buffers 16-byte aligned, not overlapping k or v.
 *   float32 dims return SSA_ERR_DTYPE.  Allocates nothing.
 */
ssa_status ssa_kv_frag(const ssa_dims* dims, const void* k, const void* v, void* k_frag, void* v_frag,
                       void* stream);

/*
 * ssa_sparse_attn_fwd_frag -- ssa_sparse_attn_fwd reading the copies ssa_kv_frag wrote
 *   from the same k and v.  Arguments and results as ssa_sparse_attn_fwd (k and v are
 *   still read: rows whose logits need the exact recompute, and the leading query chunks
 *   the dense kernel writes); k_frag and v_frag are required on bf16 and ignored (may be
 *   NULL) on float32.  Allocates nothing.
 */
ssa_status ssa_sparse_attn_fwd_frag(const ssa_dims* dims, const void* q, const void* k, const void* v,
                                    const void* k_frag, const void* v_frag, const int32_t* idx, int32_t topk,
                                    float scale, void* o, float* lse, void* stream);

/*
 * ssa_full_attn_fwd_frag -- ssa_full_attn_fwd reading the copy of v that ssa_kv_frag
 *   wrote.  Arguments and results as ssa_full_attn_fwd (bit for bit); v_frag is required
 *   on bf16 when o is given, and ignored (may be NULL) otherwise.  Allocates nothing.
 */
ssa_status ssa_full_attn_fwd_frag(const ssa_dims* dims, const void* q, const void* k, const void* v,
                                  const void* v_frag, float scale, void* o, float* lse, void* stream);

/*
 * ssa_full_attn_fwd_stats -- ssa_full_attn_fwd with the full stream's attention-pattern
 *   measurements taken from the same sweep's probabilities.
 *   The pages compare methods by attention entropy (App. H, Table A9) and by the
 *   attention mass at each distance (App. K.2, p. 31); these are the quantities
 *   ssa_attn_stats gives for idx NULL, without its second pass over q and k.
 *   q, k, v, scale, o, lse   as for ssa_full_attn_fwd, except that o and lse may both be NULL
 *   entropy    [B,H,L] float32 or NULL   out: -sum_{i<=t} p_ti ln p_ti (nats)
 *   dist_hist  [B,H,16] float32 or NULL  out: sum_t sum_{i<=t} p_ti over keys whose block
 *              distance b_t - b_i falls in bucket m (0 for the own block, 1 + floor(log2 d)
 *              for d >= 1, bucket 15 also collecting everything beyond); each head's
 *              buckets sum to L.  Summed in a fixed order (deterministic).
 *   At least one of entropy, dist_hist must be given.  On bf16 the measurements come from
 *   the forward's own sweep; on float32 (and shapes the matrix-core kernel does not take)
 *   the call runs ssa_full_attn_fwd and then the measurement pass.
 *   Workspace, from the pool: B*H*ceil(L/256)*64 bytes of histogram partials (bf16), the
 *   V copy of ssa_full_attn_fwd when o is given, and on the unfused path B*H*L*4 bytes
 *   of log-sum-exp when lse is NULL plus ssa_attn_stats' partials.
 */
ssa_status ssa_full_attn_fwd_stats(const ssa_dims* dims, const void* q, const void* k, const void* v,
                                   float scale, void* o, float* lse, float* entropy, float* dist_hist,
                                   void* stream);

/*
 * ssa_sparse_attn_fwd_stats -- ssa_sparse_attn_fwd with the sparse stream's
 *   attention-pattern measurements taken from the same sweep's probabilities.
 *   The pages compare methods by attention entropy (App. H, Table A9) and by the
 *   attention mass at each distance (App. K.2, p. 31); these are the quantities
 *   ssa_attn_stats gives for the same idx, without its second pass over q and k.
 *   q, k, v, idx, topk, scale, o, lse   as for ssa_sparse_attn_fwd
 *   entropy    [B,H,L] float32 or NULL   out: -sum_{i in A(t)} p_ti ln p_ti (nats)
 *   dist_hist  [B,H,16] float32 or NULL  out: sum_t sum_{i in A(t)} p_ti over keys whose
 *              block distance b_t - b_i falls in bucket m (buckets as for
 *              ssa_full_attn_fwd_stats); each head's buckets sum to L.  Summed in a fixed order.
 *   At least one of entropy, dist_hist must be given.  On bf16 the measurements come from
 *   the sparse kernel's own rounds (on 192-row tiles where the measurement state does not
 *   fit beside 256 rows); on float32 (and shapes the matrix-core kernel does not take) the
 *   call runs ssa_sparse_attn_fwd and then the measurement pass.  The entropies can differ
 *   in the last bits from run to run, like o.
 *   Workspace, from the pool: the transient k, v copies of ssa_sparse_attn_fwd and
 *   64 bytes of histogram partials per (b, h) and tile; on the unfused path B*H*L*4 bytes
 *   of log-sum-exp when lse is NULL plus ssa_attn_stats' workspace.
 */
ssa_status ssa_sparse_attn_fwd_stats(const ssa_dims* dims, const void* q, const void* k, const void* v,
                                     const int32_t* idx, int32_t topk, float scale, void* o, float* lse,
                                     float* entropy, float* dist_hist, void* stream);

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
 *   At least one output must be given.  The block partition is not used: block is not
 *   checked and L need not be a multiple of it (L = 1 compares one decoding step's
 *   outputs, [B,H,D] and [B,H]).
 */
ssa_status ssa_align_stats(const ssa_dims* dims, const void* o_full, const void* o_sparse,
                           const float* lse_full, const float* lse_sparse, float* l2_dist,
                           float* dropped, void* stream);

/*
 * ssa_align_stats_hist -- ssa_align_stats with the distribution of the retained mass
 *   counted in the same pass.  The pages measure attention sparsity as the attention
 *   mass the kept blocks hold (App. H, Table A9); per head this is its histogram.
 *   retained_hist  [B,H,16] float32 or NULL  out: the number of rows t whose retained mass
 *                  1 - dropped(t) lies in [m/16, (m+1)/16) (m = 15 also holding 1); each
 *                  head's counts sum to L.  Needs the lse pair and L % 64 == 0.  Whole
 *                  numbers, so the result does not depend on the order of the additions.
 *   Other arguments as for ssa_align_stats; at least one output must be given.
 */
ssa_status ssa_align_stats_hist(const ssa_dims* dims, const void* o_full, const void* o_sparse,
                                const float* lse_full, const float* lse_sparse, float* l2_dist,
                                float* dropped, float* retained_hist, void* stream);

/*
 * Decoding with a key/value cache -- one new query per sequence per step.
 *   The paper's sparse kernel has no key/value cache, which makes its decoding slow
 *   (App. E, p. 22).  These calls are the cached form of the same forward (sec. 3,
 *   pp. 3-4) for the query at position t = pos[b] of each sequence b: the same
 *   selection over the complete blocks before t's own, the same sparse attention, and
 *   dense attention over 0..t.  Their results equal row t of ssa_block_topk,
 *   ssa_sparse_attn_fwd and ssa_full_attn_fwd run over the whole sequence, up to
 *   float32 rounding (and, for the selection, score ties within rounding).
 *
 *   dims     B sequences, H query heads, Hkv key/value heads, L = cache CAPACITY in
 *            tokens (a multiple of block), D, block, dtype.  n = L / block.
 *   pos      [B] int32 DEVICE array: the position t of the new token of each sequence,
 *            read by the kernels (the host never sees it).  Sequences may be at different
 *            positions.  An entry outside [0, L) is not an error the call can report:
 *            that sequence is skipped by ssa_decode_append, gets NaN in o and lse and -1
 *            in idx from the forward calls, and nothing outside the buffers is touched.
 *   k_cache, v_cache  [B,Hkv,L,D] (dtype): token i of sequence b at row i.  Rows after
 *            pos[b] are never read by the forward calls.
 *   k_mean   [B,Hkv,n,D] float32: pooled keys of the cached blocks.  Block j < pos/block
 *            must hold the mean of its block keys (ssa_block_pool over a prompt writes it;
 *            ssa_decode_append maintains it); the entry of the open block is the mean of
 *            the tokens it holds, written by each ssa_decode_append.
 */

/*
 * ssa_decode_append -- store one new token per sequence and update its block's mean.
 *   k_new, v_new  [B,Hkv,D] (dtype)          in: key and value of the token at pos[b]
 *   k_cache, v_cache [B,Hkv,L,D] (dtype)     in/out: row pos[b] is written
 *   k_mean   [B,Hkv,n,D] float32             in/out: entry pos[b]/block is rewritten as the
 *            mean of rows block*(pos/block) .. pos (summed in float32 in the same order as
 *            ssa_block_pool, so a block completed by appends holds the same bits)
 *   Two sequences never share cache rows; calls on one stream run in order.
 */
ssa_status ssa_decode_append(const ssa_dims* dims, const int32_t* pos, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, float* k_mean, void* stream);

/*
 * ssa_decode_sparse_fwd -- selection and sparse attention for one query per sequence.
 *   q        [B,H,D] (dtype)                 in: the query at pos[b]
 *   k_cache, v_cache, k_mean                 in (as above; query head h uses key/value head h / G)
 *   topk     1 <= topk <= n                  blocks kept (own block included)
 *   scale    softmax scale (> 0, finite)
 *   o        [B,H,D] (dtype)                 out: sparse-stream output o_s(t)
 *   lse      [B,H] float32 or NULL           out (optional): log-sum-exp of the sparse stream
 *   idx      [B,H,topk] int32 or NULL        out (optional): the kept blocks, as ssa_block_topk
 *            lists them for row t
 *   Needs n <= 8192 (else SSA_ERR_UNSUPPORTED).
 *   Workspace: B*H*(ceil(topk*block/256))*(D+2)*4 bytes of split results, plus B*H*topk*4
 *   bytes for the selection when idx is NULL, from the stream-ordered pool described
 *   under ssa_sparse_attn_fwd, with the same error behaviour.
 */
ssa_status ssa_decode_sparse_fwd(const ssa_dims* dims, const int32_t* pos, const void* q, const void* k_cache,
                                 const void* v_cache, const float* k_mean, int32_t topk, float scale, void* o,
                                 float* lse, int32_t* idx, void* stream);

/*
 * ssa_decode_sparse_fwd_noalloc -- ssa_decode_sparse_fwd with no allocation.
 *   For callers that cannot allocate device memory during the call: code under HIP
 *   graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 *   checks, kernels and results as ssa_decode_sparse_fwd; its scratch (the split results,
 *   plus the kept blocks when idx is NULL) lives in a fixed 16 MiB device array that the
 *   library holds on each device it runs on until the process ends, instead of the pool.
 *   Limit: B*H*ceil(topk*block/256)*(D+2)*4 bytes, plus B*H*topk*4 when idx is NULL, at
 *   most 16 MiB (16777216); larger calls return SSA_ERR_SHAPE before any work.  Nothing
 *   in the array needs to start cleared: each call reads only what it has written.
 *   Every call on one device shares that device's array, so calls that overlap on one
 *   device (different streams, or different host threads) race and must be serialised
 *   by the caller.
 */
ssa_status ssa_decode_sparse_fwd_noalloc(const ssa_dims* dims, const int32_t* pos, const void* q,
                                         const void* k_cache, const void* v_cache, const float* k_mean, int32_t topk,
                                         float scale, void* o, float* lse, int32_t* idx, void* stream);

/*
 * ssa_decode_full_fwd -- dense attention over 0..pos[b] for one query per sequence.
 *   q        [B,H,D] (dtype)                 in
 *   k_cache, v_cache                         in (v_cache may be NULL when o is NULL)
 *   o        [B,H,D] (dtype) or NULL         out: full-stream output o_f(t)
 *   lse      [B,H] float32 or NULL           out: log-sum-exp of the full stream
 *   At least one of o, lse must be given; with o == NULL the values are not read.
 *   Workspace: B*H*ceil(L/1024)*(D+2)*4 bytes of split results, from the same pool.
 */
ssa_status ssa_decode_full_fwd(const ssa_dims* dims, const int32_t* pos, const void* q, const void* k_cache,
                               const void* v_cache, float scale, void* o, float* lse, void* stream);

/*
 * Training both streams -- backward of the attention forward, and the alignment loss.
 *   SSA trains the full and the sparse stream of every layer (sec. 5, pp. 6-7; App. C,
 *   p. 20): the sampled main stream carries the language-model gradient and both carry
 *   the gradient of the bidirectional alignment loss.  The backward calls give the
 *   gradients of one stream's forward (as computed by ssa_full_attn_fwd /
 *   ssa_sparse_attn_fwd) with respect to q, k and v, for an upstream gradient dout of
 *   that stream's output; the selection idx is held fixed (it has no gradient).
 *
 *   q, o, dout  [B,H,L,D] (dtype)     in: the forward's inputs, its output o, and dL/do
 *   k, v        [B,Hkv,L,D] (dtype)   in
 *   lse         [B,H,L] float32       in: the forward's log-sum-exp (same stream)
 *   dq          [B,H,L,D] float32     in/out: dq += dL/dq
 *   dk, dv      [B,Hkv,L,D] float32   in/out: dk += dL/dk, dv += dL/dv (all query heads of
 *               a group add into their key/value head)
 *   The gradients are ADDED to dq, dk, dv, so the two streams' calls can share them;
 *   clear them first.  The softmax term uses delta_t = sum_d dout_t,d o_t,d with the
 *   stored o.  Workspace: B*H*L*4 bytes (delta); the sparse call adds an inverted index
 *   (block -> rows that kept it) of B*H*(2n+1)*4 + B*H*L*topk*4 bytes; on bf16 the
 *   matrix-core path adds fragment-order copies of Q, dO and K for the full call
 *   (2*B*H*L*D*2 + B*Hkv*L*D*2 bytes) and of K for the sparse call (B*Hkv*L*D*2 bytes);
 *   all from the pool described under ssa_sparse_attn_fwd.  The sparse call accumulates
 *   dq, dk and dv in an order that can differ between runs (last-bit float32
 *   differences).
 */
ssa_status ssa_full_attn_bwd(const ssa_dims* dims, const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, float scale, float* dq, float* dk, float* dv,
                             void* stream);
ssa_status ssa_sparse_attn_bwd(const ssa_dims* dims, const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, const int32_t* idx, int32_t topk, float scale,
                               float* dq, float* dk, float* dv, void* stream);

/*
 * ssa_attn_stats -- attention-pattern measurements of one stream.
 *   The pages compare methods by attention sparsity and entropy (App. H, Table A9) and by
 *   histograms of attention distance (App. K.2, p. 31).  For the full stream (idx NULL)
 *   or the sparse stream (idx as given to ssa_sparse_attn_fwd) and that stream's lse:
 *   q          [B,H,L,D] (dtype)          in
 *   k          [B,Hkv,L,D] (dtype)        in
 *   lse        [B,H,L] float32            in: the stream's log-sum-exp (from its forward call)
 *   idx, topk  as for ssa_sparse_attn_fwd, or idx NULL for the full stream
 *   entropy    [B,H,L] float32 or NULL    out: -sum_i p_ti ln p_ti over the stream's keys
 *   dist_hist  [B,H,16] float32 or NULL   out: sum_t sum_i p_ti over keys whose block distance
 *              b_t - b_i falls in bucket m: 0 for the own block, 1 + floor(log2 d) for
 *              d >= 1, bucket 15 also collecting everything beyond; each head's buckets sum
 *              to L (summed in a fixed order)
 *   At least one output must be given.  The sparse stream's dropped mass and the
 *   divergence KL(p_sparse || p_full) = lse_full - lse_sparse follow from the two
 *   log-sum-exps (ssa_align_stats gives the first).  Workspace, from the pool: 64 bytes
 *   of histogram partials per (b, h) and row group -- L/128 groups for the full stream
 *   on bf16, ceil(L/512) (or ceil(L/256)) tiles for the sparse stream on bf16, L/4
 *   otherwise; when a sparse tile's block index does not fit in LDS (very large n or
 *   topk) the bf16 path scores under per-row block masks instead and adds them
 *   (B*H*L*ceil(n/32)*4 bytes).  The sparse stream's bf16 entropies are summed in an
 *   order that can differ between runs (last-bit float32 differences).
 */
ssa_status ssa_attn_stats(const ssa_dims* dims, const void* q, const void* k, const float* lse, const int32_t* idx,
                          int32_t topk, float scale, float* entropy, float* dist_hist, void* stream);

/*
 * ssa_align_loss -- the bidirectional alignment objective of sec. 5 (pp. 6-7): a
 *   sparsity term SmoothL1(o_full, held o_sparse) pulling the full output toward the
 *   sparse one, and a commitment term SmoothL1(o_sparse, held o_full), each the mean over
 *   all B*H*L*D elements, weighted by alpha.  SmoothL1(x) = 0.5 x^2 / beta for |x| < beta,
 *   |x| - beta/2 otherwise.
 *   o_full, o_sparse  [B,H,L,D] (dtype)   in
 *   loss        float32 [1]               out: alpha * (mean + mean), summed in a fixed order
 *   grad_full   [B,H,L,D] float32 or NULL out: dloss/do_full (the sparsity term only)
 *   grad_sparse [B,H,L,D] float32 or NULL out: dloss/do_sparse (the commitment term only)
 *   alpha finite, beta finite and > 0.  The block partition is not used (as for
 *   ssa_align_stats).  Workspace: 4 bytes per 256 16-byte groups of o.
 */
ssa_status ssa_align_loss(const ssa_dims* dims, const void* o_full, const void* o_sparse, float alpha, float beta,
                          float* loss, float* grad_full, float* grad_sparse, void* stream);

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
