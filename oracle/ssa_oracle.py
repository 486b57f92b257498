"""CPU oracle for the SSA per-layer attention forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this
module.  The product path (the HIP library and its Python binding) never calls it and
shares no code with it; the only thing both sides share is the seeded input generator
in `workloads.py`, which holds none of the method's arithmetic.

Everything here is plain numpy in float64, computed from the exact values of the same
bf16 / fp32 inputs the GPU receives.  Each function follows a passage of Shen et al.,
"SSA: Sparse Sparse Attention by Aligning Full and Sparse Attention Outputs in Feature
Space" (arXiv 2511.20102; the v4 summary page's section tags are cited):

  block_pool            sec. 3 (p. 4): contiguous blocks of s tokens, one mean-pooled
                        key per block.
  block_topk            sec. 3 (p. 4) and App. D (p. 21): each query scores the blocks
                        that precede its own with the pooled keys and keeps the top-k
                        blocks; its own block is always kept and counts toward k.
  attend_full           sec. 3 (p. 3): causal softmax attention over every preceding
                        token (and the token itself).
  attend_sparse         sec. 3 (p. 4): softmax attention over the tokens of the kept
                        blocks (the "reduced K and V"), causal inside the own block.
  attend_sparse_gather  the same quantity formed per query by gathering the kept
                        blocks' keys and values (a second route used as a pin).
  dropped_mass          App. B (p. 19) and sec. 4.2 (p. 6): the full-attention
                        probability mass on tokens the sparse stream does not attend.
  align_stats           sec. 5 (pp. 6-7): per-token comparison of the two streams'
                        outputs (Euclidean distance) and the dropped mass obtained from
                        the two log-sum-exps.
  open_block_mean       App. E (p. 22) names the missing key/value cache; with one new
                        token per step, the pooled key of the query's own, still open
                        block is the mean of the tokens it holds so far (sec. 3's block
                        mean over a partial block).
  decode_step           one decoding step with a key/value cache: the query at position
                        t against the cached keys and values 0..t, both streams, formed
                        from the cache alone (sec. 3, p. 3-4; App. E, p. 22).
  attend_full_bwd       gradients of the full stream's output with respect to q, k, v
  attend_sparse_bwd     and of the sparse stream's (no gradient through the selection):
                        SSA trains both streams (sec. 5, pp. 6-7; App. C, p. 20); the
                        formulas are the chain rule through softmax attention.
  attention_stats       attention-pattern measurements the pages report (App. H, Table
                        A9: sparsity; App. K.2, p. 31: entropy and distance histograms):
                        each row's attention entropy and, per head, the attention mass
                        by block distance in powers of two.
  retained_mass_hist    App. H (Table A9) measures attention sparsity as the attention
                        mass the kept blocks hold: per head, the number of rows whose
                        retained mass 1 - dropped(t) falls in each sixteenth of [0, 1].
  align_loss            the bidirectional alignment objective of sec. 5 (pp. 6-7): a
                        sparsity term pulling the full output toward the (held) sparse
                        one and a commitment term pulling the sparse output toward the
                        (held) full one, both SmoothL1, weighted by alpha; its value and
                        the gradient it sends to each stream's output.

Readings where the pages are silent (the main ones):
  * candidates are the blocks strictly before the query's block; the own block is
    always attended (causal inside) and counts toward k;
  * fewer candidates than k-1: all of them are kept;
  * the block score is the raw dot product q . mean(K_block) (no scale, no softmax);
  * ties in score go to the lower block index;
  * selected blocks are listed in ascending order, -1 pads unused slots;
  * the softmax scale is an explicit argument (1/sqrt(D) in every workload);
  * the alignment distance is the Euclidean (not squared) L2 norm over the head dim.

Every function here is pinned by the CPU tests in tests/test_oracle_pins.py (brute
force on tiny inputs, closed forms, identities, special cases); none is "parity
unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "block_pool", "block_scores", "block_topk", "attend_full", "attend_sparse",
    "attend_sparse_gather", "dropped_mass", "align_stats", "attended_blocks",
    "attended_count", "open_block_mean", "decode_step", "attend_full_bwd",
    "attend_sparse_bwd", "smooth_l1", "align_loss", "attention_stats", "distance_bucket",
    "retained_mass_hist",
]


def _rows(L: int, rows) -> np.ndarray:
    return np.arange(L, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)


# ----------------------------------------------------------------------------------
# sec. 3: block partition and mean-pooled keys
# ----------------------------------------------------------------------------------
def block_pool(k: np.ndarray, s: int) -> np.ndarray:
    """Mean of each contiguous block of s keys: [B,H,L,D] -> [B,H,L//s,D] (float64)."""
    B, H, L, D = k.shape
    if L % s:
        raise ValueError("L must be a multiple of the block size")
    return np.asarray(k, dtype=np.float64).reshape(B, H, L // s, s, D).mean(axis=3)


def block_scores(q_rows: np.ndarray, k_mean_bh: np.ndarray) -> np.ndarray:
    """Raw block scores q_t . kbar_j for the given query rows of one (b, h): [R, n]."""
    return np.asarray(q_rows, dtype=np.float64) @ np.asarray(k_mean_bh, dtype=np.float64).T


# ----------------------------------------------------------------------------------
# sec. 3 / App. D: per-query top-k over the preceding blocks
# ----------------------------------------------------------------------------------
def block_topk(q: np.ndarray, k_mean: np.ndarray, s: int, topk: int, rows=None,
               return_scores: bool = False):
    """Selected blocks per query row.

    For the query at position t (block b_t = t // s): score every block j < b_t by
    q_t . kbar_j, order the candidates by (score descending, index ascending), keep the
    first min(topk - 1, b_t), add b_t, and list them in ascending order padded with -1
    to width topk.

    Returns idx [B,H,R,topk] int32 and, if return_scores, a dict with
      "sigma_m":  the score of the last kept candidate (m-th largest, m = topk-1),
      "sigma_m1": the score of the best candidate left out ((m+1)-th largest),
    both [B,H,R] float64 (NaN where that candidate does not exist), and
      "scores":   [B,H,R,topk] float64 scores of the listed blocks (+inf for b_t,
                  -inf for padding).
    """
    q = np.asarray(q, dtype=np.float64)
    B, H, L, D = q.shape
    n = L // s
    R = _rows(L, rows)
    if not 1 <= topk <= n:
        raise ValueError("topk must be in [1, n]")
    idx = np.full((B, H, len(R), topk), -1, dtype=np.int32)
    sig_m = np.full((B, H, len(R)), np.nan)
    sig_m1 = np.full((B, H, len(R)), np.nan)
    sel_sc = np.full((B, H, len(R), topk), -np.inf)
    blocks_of_rows = R // s
    for b in range(B):
        for h in range(H):
            for qb in np.unique(blocks_of_rows):
                pos = np.nonzero(blocks_of_rows == qb)[0]
                m = min(topk - 1, int(qb))
                if qb > 0:
                    sc = block_scores(q[b, h, R[pos]], k_mean[b, h, :qb])     # [r, qb]
                    # stable sort on -score keeps equal scores in ascending block order
                    order = np.argsort(-sc, axis=1, kind="stable")
                    kept = np.sort(order[:, :m], axis=1)
                    if m > 0:
                        sig_m[b, h, pos] = np.take_along_axis(sc, order[:, m - 1:m], 1)[:, 0]
                    if m < qb:
                        sig_m1[b, h, pos] = np.take_along_axis(sc, order[:, m:m + 1], 1)[:, 0]
                    idx[b, h, pos, :m] = kept
                    sel_sc[b, h, pos, :m] = np.take_along_axis(sc, kept, 1)
                idx[b, h, pos, m] = qb
                sel_sc[b, h, pos, m] = np.inf
    if return_scores:
        return idx, {"sigma_m": sig_m, "sigma_m1": sig_m1, "scores": sel_sc}
    return idx


# ----------------------------------------------------------------------------------
# sec. 3: attended key set of the sparse stream
# ----------------------------------------------------------------------------------
def attended_blocks(idx_row: np.ndarray, t: int, s: int) -> list:
    """Blocks the sparse stream attends for the query at t: its own block b_t plus the
    listed blocks below it (-1 and out-of-range entries are not blocks)."""
    bt = t // s
    listed = {int(j) for j in np.asarray(idx_row).ravel() if 0 <= int(j) < bt}
    return sorted(listed | {bt})


def attended_count(t: int, s: int, topk: int) -> int:
    """|A(t)| for a full selection: t+1 while b_t < topk, else (topk-1)*s + t%s + 1."""
    bt = t // s
    return t + 1 if bt < topk else (topk - 1) * s + (t % s) + 1


def _sparse_key_mask(idx_rows: np.ndarray, R: np.ndarray, s: int, nkeys: int) -> np.ndarray:
    """[r, nkeys] boolean: key i attended by row R[a] (i <= t and block(i) attended)."""
    r = len(R)
    n_blk = (nkeys + s - 1) // s
    bt = R // s
    blk = np.zeros((r, n_blk + 1), dtype=bool)
    ids = np.asarray(idx_rows, dtype=np.int64)
    valid = (ids >= 0) & (ids < bt[:, None])
    rr = np.repeat(np.arange(r)[:, None], ids.shape[1], axis=1)
    blk[rr[valid], ids[valid]] = True
    blk[np.arange(r), bt] = True
    keys = np.arange(nkeys)
    mask = blk[:, keys // s] & (keys[None, :] <= R[:, None])
    return mask


def _masked_softmax_attend(logits: np.ndarray, mask: np.ndarray, v: np.ndarray):
    lg = np.where(mask, logits, -np.inf)
    m = lg.max(axis=1, keepdims=True)
    e = np.exp(lg - m)
    l = e.sum(axis=1, keepdims=True)
    o = (e @ v) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse, e / l


# ----------------------------------------------------------------------------------
# sec. 3: full causal attention
# ----------------------------------------------------------------------------------
def attend_full(q, k, v, scale: float, rows=None, want_o: bool = True):
    """o_f(t) = sum_{i<=t} softmax_i(scale q_t.k_i) v_i and lse_f(t) = log sum_{i<=t}
    exp(scale q_t.k_i), for the given rows.  Returns (o [B,H,R,D] or None, lse [B,H,R])."""
    q = np.asarray(q, dtype=np.float64)
    B, H, L, D = q.shape
    R = _rows(L, rows)
    nk = int(R.max()) + 1
    o = np.zeros((B, H, len(R), D)) if want_o else None
    lse = np.zeros((B, H, len(R)))
    keys = np.arange(nk)
    mask = keys[None, :] <= R[:, None]
    for b in range(B):
        for h in range(H):
            kk = np.asarray(k[b, h, :nk], dtype=np.float64)
            vv = np.asarray(v[b, h, :nk], dtype=np.float64)
            logits = scale * (q[b, h, R] @ kk.T)
            ob, lb, _ = _masked_softmax_attend(logits, mask, vv)
            if want_o:
                o[b, h] = ob
            lse[b, h] = lb
    return o, lse


# ----------------------------------------------------------------------------------
# sec. 3: sparse attention over the kept blocks (masked-dense route)
# ----------------------------------------------------------------------------------
def attend_sparse(q, k, v, idx, s: int, scale: float, rows=None):
    """o_s(t) = sum_{i in A(t)} softmax_i(scale q_t.k_i) v_i, lse_s(t) = log sum_{i in A(t)}
    exp(scale q_t.k_i), with A(t) = {i <= t : i // s attended}.  `idx` is [B,H,R,topk]
    for the same rows.  Returns (o [B,H,R,D], lse [B,H,R])."""
    q = np.asarray(q, dtype=np.float64)
    B, H, L, D = q.shape
    R = _rows(L, rows)
    nk = int(R.max()) + 1
    o = np.zeros((B, H, len(R), D))
    lse = np.zeros((B, H, len(R)))
    for b in range(B):
        for h in range(H):
            kk = np.asarray(k[b, h, :nk], dtype=np.float64)
            vv = np.asarray(v[b, h, :nk], dtype=np.float64)
            mask = _sparse_key_mask(idx[b, h], R, s, nk)
            logits = scale * (q[b, h, R] @ kk.T)
            o[b, h], lse[b, h], _ = _masked_softmax_attend(logits, mask, vv)
    return o, lse


def attend_sparse_gather(q, k, v, idx, s: int, scale: float, rows=None):
    """Same quantity as attend_sparse, formed per query: gather the keys and values of
    the attended blocks (keys <= t), softmax over the gathered logits."""
    q = np.asarray(q, dtype=np.float64)
    B, H, L, D = q.shape
    R = _rows(L, rows)
    o = np.zeros((B, H, len(R), D))
    lse = np.zeros((B, H, len(R)))
    for b in range(B):
        for h in range(H):
            for a, t in enumerate(R):
                blocks = attended_blocks(idx[b, h, a], int(t), s)
                keys = np.concatenate([np.arange(j * s, min(j * s + s, t + 1)) for j in blocks])
                kk = np.asarray(k[b, h, keys], dtype=np.float64)
                vv = np.asarray(v[b, h, keys], dtype=np.float64)
                lg = scale * (kk @ q[b, h, t])
                m = lg.max()
                e = np.exp(lg - m)
                o[b, h, a] = (e @ vv) / e.sum()
                lse[b, h, a] = m + np.log(e.sum())
    return o, lse


# ----------------------------------------------------------------------------------
# App. B / sec. 4.2: dropped attention mass, summed from the full probabilities
# ----------------------------------------------------------------------------------
def dropped_mass(q, k, idx, s: int, scale: float, rows=None):
    """delta(t) = sum over i <= t with i not in A(t) of the full causal attention
    probability p_f(t, i).  Summed directly (not through log-sum-exps)."""
    q = np.asarray(q, dtype=np.float64)
    B, H, L, D = q.shape
    R = _rows(L, rows)
    nk = int(R.max()) + 1
    out = np.zeros((B, H, len(R)))
    keys = np.arange(nk)
    causal = keys[None, :] <= R[:, None]
    for b in range(B):
        for h in range(H):
            kk = np.asarray(k[b, h, :nk], dtype=np.float64)
            logits = scale * (q[b, h, R] @ kk.T)
            _, _, p = _masked_softmax_attend(logits, causal, np.zeros((nk, 1)))
            keep = _sparse_key_mask(idx[b, h], R, s, nk)
            out[b, h] = np.where(causal & ~keep, p, 0.0).sum(axis=1)
    return out


# ----------------------------------------------------------------------------------
# sec. 5: per-token comparison of the two streams
# ----------------------------------------------------------------------------------
def align_stats(o_full=None, o_sparse=None, lse_full=None, lse_sparse=None):
    """dist(t) = ||o_f(t) - o_s(t)||_2 over the head dim, and
    dropped(t) = 1 - exp(lse_s(t) - lse_f(t)) = -expm1(lse_s - lse_f), clipped to [0, 1].
    Either pair may be None (then that output is None)."""
    dist = dropped = None
    if o_full is not None and o_sparse is not None:
        d = np.asarray(o_full, dtype=np.float64) - np.asarray(o_sparse, dtype=np.float64)
        dist = np.sqrt((d * d).sum(axis=-1))
    if lse_full is not None and lse_sparse is not None:
        x = np.asarray(lse_sparse, dtype=np.float64) - np.asarray(lse_full, dtype=np.float64)
        dropped = np.clip(-np.expm1(x), 0.0, 1.0)
    return dist, dropped


# ----------------------------------------------------------------------------------
# App. E: decoding with a key/value cache (one new query per step)
# ----------------------------------------------------------------------------------
def open_block_mean(k_bh: np.ndarray, t: int, s: int) -> np.ndarray:
    """Mean of the cached keys of the block holding position t, over the tokens present
    once t is appended: (1/c) sum_{i = b_t s}^{t} k_i with c = t - b_t s + 1 (float64).
    k_bh is the [L, D] cache of one (b, h); tokens after t are not read."""
    start = (t // s) * s
    rows = np.asarray(k_bh[start:t + 1], dtype=np.float64)
    return rows.sum(axis=0) / rows.shape[0]


def decode_step(q_t: np.ndarray, k_bh: np.ndarray, v_bh: np.ndarray, t: int, s: int, topk: int,
                scale: float) -> dict:
    """The query at position t of one (b, h) against its cache (keys and values 0..t;
    rows after t are ignored).

    Sparse stream: the complete blocks j < b_t are pooled from the cache (mean of their
    s keys), scored by q_t . kbar_j, ordered by (score descending, j ascending); the
    first min(topk - 1, b_t) are kept, b_t is added, and attention runs over the tokens
    of the kept blocks with i <= t.  Full stream: attention over every i <= t.
    Returns idx (topk int32, ascending, -1 padded), o_s, lse_s, o_f, lse_f (float64), and
    sigma_m / sigma_m1, the scores of the last kept and the best left-out candidate (NaN
    where that candidate does not exist)."""
    q = np.asarray(q_t, dtype=np.float64)
    K = np.asarray(k_bh[:t + 1], dtype=np.float64)
    V = np.asarray(v_bh[:t + 1], dtype=np.float64)
    bt = t // s
    m = min(topk - 1, bt)
    kept = []
    sigma_m = sigma_m1 = np.nan
    if m > 0:
        kbar = K[:bt * s].reshape(bt, s, -1).mean(axis=1)
        sc = kbar @ q
        ranked = sorted(range(bt), key=lambda j: (-sc[j], j))
        kept = sorted(ranked[:m])
        sigma_m = sc[ranked[m - 1]]
        if m < bt:
            sigma_m1 = sc[ranked[m]]
    blocks = kept + [bt]
    idx = np.full(topk, -1, dtype=np.int32)
    idx[:len(blocks)] = blocks

    def attend(keys):
        lg = scale * (K[keys] @ q)
        mx = lg.max()
        e = np.exp(lg - mx)
        return (e @ V[keys]) / e.sum(), mx + np.log(e.sum())

    sparse_keys = np.concatenate([np.arange(j * s, min(j * s + s, t + 1)) for j in blocks])
    o_s, lse_s = attend(sparse_keys)
    o_f, lse_f = attend(np.arange(t + 1))
    return {"idx": idx, "o_s": o_s, "lse_s": lse_s, "o_f": o_f, "lse_f": lse_f,
            "sigma_m": sigma_m, "sigma_m1": sigma_m1}


# ----------------------------------------------------------------------------------
# sec. 5 / App. C: training both streams -- backward of the attention forward and the
# bidirectional alignment loss
# ----------------------------------------------------------------------------------
def _attend_bwd_masked(q, k, v, do, scale, mask):
    """Gradients of o = softmax(scale q k^T, masked) v for one (b, h): with P the
    attention weights, dV = P^T dO, dP = dO V^T, dS = P * (dP - rowsum(dP * P)),
    dQ = scale dS K, dK = scale dS^T Q.  (rowsum(dP * P) equals rowsum(dO * O).)"""
    lg = np.where(mask, scale * (q @ k.T), -np.inf)
    m = lg.max(axis=1, keepdims=True)
    e = np.exp(lg - m)
    p = e / e.sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
    return scale * (ds @ k), scale * (ds.T @ q), dv


def attend_full_bwd(q, k, v, do, scale: float):
    """dq, dk, dv of the full causal stream for an upstream gradient do = dL/do_f
    ([B,H,L,D] each, float64)."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    B, H, L, D = q.shape
    mask = np.arange(L)[None, :] <= np.arange(L)[:, None]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = _attend_bwd_masked(q[b, h], k[b, h], v[b, h], do[b, h], scale, mask)
    return dq, dk, dv


def attend_sparse_bwd(q, k, v, do, idx, s: int, scale: float):
    """dq, dk, dv of the sparse stream with its kept blocks held fixed (the selection
    has no gradient): attention restricted to A(t) = {i <= t : block of i kept}."""
    q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
    B, H, L, D = q.shape
    R = np.arange(L)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            mask = _sparse_key_mask(idx[b, h], R, s, L)
            dq[b, h], dk[b, h], dv[b, h] = _attend_bwd_masked(q[b, h], k[b, h], v[b, h], do[b, h], scale, mask)
    return dq, dk, dv


def smooth_l1(x, beta: float = 1.0):
    """Elementwise SmoothL1 (Huber with threshold beta): 0.5 x^2 / beta where |x| < beta,
    |x| - 0.5 beta elsewhere."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    return np.where(ax < beta, 0.5 * x * x / beta, ax - 0.5 * beta)


def align_loss(o_full, o_sparse, alpha: float, beta: float = 1.0):
    """alpha * [mean SmoothL1(o_f - sg(o_s)) + mean SmoothL1(o_s - sg(o_f))] over every
    element.  Returns (loss, dL/do_f, dL/do_s): each term sends gradient only to its own
    first argument (the other is held), the derivative of SmoothL1 being x / beta
    clipped to [-1, 1], divided by the element count."""
    of = np.asarray(o_full, dtype=np.float64)
    os_ = np.asarray(o_sparse, dtype=np.float64)
    N = of.size
    loss = alpha * (smooth_l1(of - os_, beta).mean() + smooth_l1(os_ - of, beta).mean())
    g_f = alpha * np.clip((of - os_) / beta, -1.0, 1.0) / N
    g_s = alpha * np.clip((os_ - of) / beta, -1.0, 1.0) / N
    return loss, g_f, g_s


# ----------------------------------------------------------------------------------
# App. H / App. K.2: attention-pattern measurements
# ----------------------------------------------------------------------------------
N_DIST_BUCKETS = 16
N_RETAINED_BINS = 16


def retained_mass_hist(dropped) -> np.ndarray:
    """Per (b, h), the number of rows t whose retained mass r = 1 - dropped(t) lies in
    [m/16, (m+1)/16), for m = 0..15 (r = 1 counts in the last bin).  dropped: [B,H,L].
    Returns [B,H,16] (float64 counts)."""
    r = 1.0 - np.asarray(dropped, dtype=np.float64)
    B, H, L = r.shape
    out = np.zeros((B, H, N_RETAINED_BINS))
    for b in range(B):
        for h in range(H):
            for t in range(L):
                m = min(int(np.floor(r[b, h, t] * N_RETAINED_BINS)), N_RETAINED_BINS - 1)
                out[b, h, m] += 1.0
    return out


def distance_bucket(d: int) -> int:
    """Bucket of a block distance d = b_t - b_i >= 0: 0 for the own block, 1 + floor(log2 d)
    otherwise, the last bucket collecting everything from 2^14 on."""
    if d <= 0:
        return 0
    return min(1 + int(d).bit_length() - 1, N_DIST_BUCKETS - 1)


def attention_stats(q, k, s: int, scale: float, idx=None):
    """For each row t, the entropy -sum_i p_ti ln p_ti of its attention weights over A(t)
    (all i <= t for the full stream, the kept blocks' tokens when idx is given), and per
    (b, h) the attention mass by block distance: hist[b, h, m] = sum_t sum_{i in A(t)}
    p_ti [distance_bucket(t // s - i // s) = m].  Returns (entropy [B,H,L], hist [B,H,16])."""
    q = np.asarray(q, dtype=np.float64)
    B, H, L, D = q.shape
    R = np.arange(L)
    causal = R[None, :] <= R[:, None]
    bucket = np.array([[distance_bucket(t // s - i // s) for i in range(L)] for t in range(L)])
    ent = np.zeros((B, H, L))
    hist = np.zeros((B, H, N_DIST_BUCKETS))
    for b in range(B):
        for h in range(H):
            kk = np.asarray(k[b, h], dtype=np.float64)
            mask = causal if idx is None else _sparse_key_mask(idx[b, h], R, s, L)
            lg = np.where(mask, scale * (q[b, h] @ kk.T), -np.inf)
            m = lg.max(axis=1, keepdims=True)
            e = np.exp(lg - m)
            p = e / e.sum(axis=1, keepdims=True)
            logp = np.where(mask, lg - m - np.log(e.sum(axis=1, keepdims=True)), 0.0)
            ent[b, h] = -(p * logp).sum(axis=1)
            for m_ in range(N_DIST_BUCKETS):
                hist[b, h, m_] = p[bucket == m_].sum()
    return ent, hist
