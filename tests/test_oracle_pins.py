"""Pins for the CPU oracle, checked against things other than the oracle itself:
hand-derived worked examples (tests/golden), closed forms, brute force on tiny inputs,
identities that follow from the definitions, and special cases that reduce to a
textbook result.  CPU only.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a wrong
sign or index, an off-by-one in the causal or block mask, a transposed operand, a
wrong tie rule) fails at least one of them; test_planted_mistakes_are_caught plants
such slips in a copy of the oracle and checks that.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle.ssa_oracle as O
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {"e": math.e, "log": math.log}))


def _arr(x):
    return np.array([[_ev(v) if isinstance(v, str) else float(v) for v in row] for row in x])


def _vec(x):
    return np.array([_ev(v) if isinstance(v, str) else float(v) for v in x])


def _bhld(a):
    return np.asarray(a, dtype=np.float64)[None, None]


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ----------------------------------------------------------------------------------
# golden fixtures (hand-derived worked examples)
# ----------------------------------------------------------------------------------
def test_golden_tiny_L4_s2():
    g = json.load(open(os.path.join(GOLDEN, "tiny_L4_s2.json")))
    q, k, v = (_bhld(g[n]) for n in ("q", "k", "v"))
    s, scale = g["s"], g["scale"]
    np.testing.assert_allclose(O.block_pool(k, s)[0, 0], _arr(g["k_mean"]), atol=0)
    o_f, lse_f = O.attend_full(q, k, v, scale)
    np.testing.assert_allclose(o_f[0, 0], _arr(g["o_full"]), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse_f[0, 0], _vec(g["lse_full"]), rtol=1e-14, atol=1e-15)
    km = O.block_pool(k, s)
    for key, topk in (("topk1", 1), ("topk2", 2)):
        exp = g[key]
        idx = O.block_topk(q, km, s, topk)
        assert idx[0, 0].tolist() == exp["idx"]
        o_s, lse_s = O.attend_sparse(q, k, v, idx, s, scale)
        if "o_sparse" in exp:
            np.testing.assert_allclose(o_s[0, 0], _arr(exp["o_sparse"]), rtol=1e-14, atol=1e-15)
            np.testing.assert_allclose(lse_s[0, 0], _vec(exp["lse_sparse"]), rtol=1e-14, atol=1e-15)
        dm = O.dropped_mass(q, k, idx, s, scale)
        np.testing.assert_allclose(dm[0, 0], _vec(exp["dropped"]), rtol=1e-13, atol=1e-15)
        _, dm2 = O.align_stats(lse_full=lse_f, lse_sparse=lse_s)
        np.testing.assert_allclose(dm2[0, 0], _vec(exp["dropped"]), rtol=1e-12, atol=1e-15)


def test_golden_select_ties():
    g = json.load(open(os.path.join(GOLDEN, "select_ties_L8_s2.json")))
    q, k = _bhld(g["q"]), _bhld(g["k"])
    km = O.block_pool(k, g["s"])
    np.testing.assert_array_equal(km[0, 0], np.array(g["k_mean"], dtype=float))
    idx = O.block_topk(q, km, g["s"], g["topk"])
    assert idx[0, 0].tolist() == g["idx"]
    for var in g["block3_variants"]:
        qq = q.copy()
        qq[0, 0, 6] = var["q"]
        got = O.block_topk(qq, km, g["s"], g["topk"])[0, 0, 6].tolist()
        assert got == [var["chosen"], 3]


# ----------------------------------------------------------------------------------
# block_pool
# ----------------------------------------------------------------------------------
def test_pool_closed_forms():
    B, H, L, D, s = 2, 3, 256, 8, 16
    # K equal to its position index t in every component: block mean = j*s + (s-1)/2
    k = np.broadcast_to(np.arange(L, dtype=float)[None, None, :, None], (B, H, L, D))
    km = O.block_pool(k, s)
    expect = np.arange(L // s) * s + (s - 1) / 2.0
    np.testing.assert_array_equal(km, np.broadcast_to(expect[None, None, :, None], km.shape))
    # K constant inside each block: the mean is that constant
    c = _rand((B, H, L // s, D), 3)
    np.testing.assert_allclose(O.block_pool(np.repeat(c, s, axis=2), s), c, rtol=1e-15)
    # integer keys: exact and bounded by the block's extrema
    ki = W.integer_tensor((B, H, L, D), -8, 8, seed=4).astype(float)
    km = O.block_pool(ki, s)
    assert np.all(km * s == np.round(km * s))
    blocks = ki.reshape(B, H, L // s, s, D)
    assert np.all(km <= blocks.max(axis=3)) and np.all(km >= blocks.min(axis=3))


def test_block_scores_are_mean_token_scores():
    """By linearity a query's score against a block mean is the mean of its dot products
    with the block's keys, computed here token by token with explicit loops (no matrix
    product), on small integer inputs where both sides are exact in float64."""
    L, D, s, R = 32, 4, 8, 5
    k = W.integer_tensor((1, 1, L, D), -6, 6, seed=21).astype(float)
    q = W.integer_tensor((R, D), -5, 5, seed=22).astype(float)
    got = O.block_scores(q, O.block_pool(k, s)[0, 0])
    assert got.shape == (R, L // s)
    for r in range(R):
        for j in range(L // s):
            tot = 0.0
            for i in range(j * s, (j + 1) * s):
                tot += sum(q[r, d] * k[0, 0, i, d] for d in range(D))
            assert got[r, j] == tot / s, (r, j, got[r, j], tot / s)


def test_pool_rejects_ragged_length():
    with pytest.raises(ValueError):
        O.block_pool(np.zeros((1, 1, 10, 4)), 4)


# ----------------------------------------------------------------------------------
# block_topk
# ----------------------------------------------------------------------------------
def test_topk_q_zero_keeps_lowest_blocks():
    """q = 0: every score is exactly 0, so the tie rule keeps blocks 0..m-1."""
    B, H, L, D, s = 1, 2, 512, 16, 32
    q = np.zeros((B, H, L, D))
    km = O.block_pool(_rand((B, H, L, D), 5), s)
    for topk in (1, 2, 5, L // s):
        idx = O.block_topk(q, km, s, topk)
        for t in range(L):
            bt = t // s
            m = min(topk - 1, bt)
            expect = list(range(m)) + [bt] + [-1] * (topk - m - 1)
            assert idx[0, 1, t].tolist() == expect


def test_topk_linear_scores_closed_form():
    """kbar_j = j * e_0: score = q_0 * j.  q_0 > 0 keeps the m blocks just below b_t;
    q_0 < 0 keeps blocks 0..m-1."""
    L, D, s, topk = 256, 4, 8, 6
    n = L // s
    km = np.zeros((1, 1, n, D))
    km[0, 0, :, 0] = np.arange(n)
    for sign in (1.0, -1.0):
        q = np.zeros((1, 1, L, D))
        q[..., 0] = sign * (1.0 + np.arange(L) / L)
        idx = O.block_topk(q, km, s, topk)
        for t in range(L):
            bt = t // s
            m = min(topk - 1, bt)
            chosen = list(range(bt - m, bt)) if sign > 0 else list(range(m))
            assert idx[0, 0, t].tolist() == chosen + [bt] + [-1] * (topk - m - 1)


def _brute_force_valid_selection(sc_row, kept, m):
    """Every kept candidate beats every dropped one under (score desc, index asc)."""
    cand = range(len(sc_row))
    dropped = [j for j in cand if j not in kept]
    for a in kept:
        for d in dropped:
            assert (sc_row[a] > sc_row[d]) or (sc_row[a] == sc_row[d] and a < d)
    assert len(kept) == m


@pytest.mark.parametrize("integer", [False, True])
def test_topk_brute_force_tiny(integer):
    B, H, L, D, s = 2, 2, 96, 4, 8
    if integer:   # many exact ties
        q = W.integer_tensor((B, H, L, D), -1, 1, seed=6).astype(float)
        k = W.integer_tensor((B, H, L, D), -2, 2, seed=7).astype(float)
    else:
        q, k = _rand((B, H, L, D), 8), _rand((B, H, L, D), 9)
    km = O.block_pool(k, s)
    for topk in (1, 3, 7, L // s):
        idx, extra = O.block_topk(q, km, s, topk, return_scores=True)
        for b, h, t in itertools.product(range(B), range(H), range(L)):
            bt = t // s
            m = min(topk - 1, bt)
            row = idx[b, h, t].tolist()
            assert row[m] == bt and all(x == -1 for x in row[m + 1:])
            kept = row[:m]
            assert kept == sorted(set(kept))
            sc = [float(q[b, h, t] @ km[b, h, j]) for j in range(bt)]   # loop dot products
            _brute_force_valid_selection(sc, kept, m)
            if m > 0:
                assert extra["sigma_m"][b, h, t] == pytest.approx(min(sc[j] for j in kept), rel=1e-12, abs=1e-14)


# ----------------------------------------------------------------------------------
# attend_full
# ----------------------------------------------------------------------------------
def test_full_q_zero_is_prefix_mean():
    B, H, L, D = 1, 2, 64, 5
    v = _rand((B, H, L, D), 10)
    k = _rand((B, H, L, D), 11)
    o, lse = O.attend_full(np.zeros((B, H, L, D)), k, v, 0.3)
    pref = np.cumsum(v, axis=2) / np.arange(1, L + 1)[None, None, :, None]
    np.testing.assert_allclose(o, pref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, L + 1)), lse.shape), rtol=1e-13)


def test_full_designed_weights_closed_form():
    """Keys k_i = log(w_i) e_0 and q = e_0, scale 1: softmax weight of key i is
    w_i / sum w, so o(t) = sum_{i<=t} w_i v_i / sum_{i<=t} w_i."""
    L, D = 12, 3
    w = np.arange(1, L + 1, dtype=float) ** 1.5
    k = np.zeros((1, 1, L, D))
    k[0, 0, :, 0] = np.log(w)
    q = np.zeros((1, 1, L, D))
    q[..., 0] = 1.0
    v = _rand((1, 1, L, D), 12)
    o, lse = O.attend_full(q, k, v, 1.0)
    for t in range(L):
        ww = w[: t + 1]
        np.testing.assert_allclose(o[0, 0, t], (ww[:, None] * v[0, 0, : t + 1]).sum(0) / ww.sum(), rtol=1e-12)
        np.testing.assert_allclose(lse[0, 0, t], np.log(ww.sum()), rtol=1e-13)
    # L = 1: the output is v_0 and lse is the single logit
    o1, l1 = O.attend_full(q[:, :, :1] * 2.0, k[:, :, :1] + 1.0, v[:, :, :1], 0.5)
    np.testing.assert_allclose(o1[0, 0, 0], v[0, 0, 0])
    np.testing.assert_allclose(l1[0, 0, 0], 0.5 * 2.0 * (np.log(w[0]) + 1.0))


def test_full_is_causal_and_rows_subset_consistent():
    B, H, L, D = 1, 1, 40, 4
    q, k, v = _rand((B, H, L, D), 13), _rand((B, H, L, D), 14), _rand((B, H, L, D), 15)
    o, lse = O.attend_full(q, k, v, 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, 20:] += 7.0
    v2[:, :, 20:] -= 3.0
    o2, lse2 = O.attend_full(q, k2, v2, 0.5)
    np.testing.assert_array_equal(o[:, :, :20], o2[:, :, :20])
    rows = np.array([3, 19, 39])
    o3, lse3 = O.attend_full(q, k, v, 0.5, rows=rows)
    np.testing.assert_allclose(o3[0, 0], o[0, 0, rows], rtol=1e-13)
    np.testing.assert_allclose(lse3[0, 0], lse[0, 0, rows], rtol=1e-13)


# ----------------------------------------------------------------------------------
# attend_sparse
# ----------------------------------------------------------------------------------
def _tiny_case(seed, B=1, H=2, L=128, D=8, s=8, scale=0.7):
    q, k, v = _rand((B, H, L, D), seed), _rand((B, H, L, D), seed + 1), _rand((B, H, L, D), seed + 2)
    return q, k, v, s, scale


@pytest.mark.parametrize("topk", [1, 2, 5, 16])
def test_sparse_two_routes_agree(topk):
    q, k, v, s, scale = _tiny_case(20)
    idx = O.block_topk(q, O.block_pool(k, s), s, topk)
    o1, l1 = O.attend_sparse(q, k, v, idx, s, scale)
    o2, l2 = O.attend_sparse_gather(q, k, v, idx, s, scale)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=1e-12, atol=1e-12)


def test_sparse_all_blocks_equals_full():
    q, k, v, s, scale = _tiny_case(30)
    L = q.shape[2]
    idx = O.block_topk(q, O.block_pool(k, s), s, L // s)
    o_s, l_s = O.attend_sparse(q, k, v, idx, s, scale)
    o_f, l_f = O.attend_full(q, k, v, scale)
    np.testing.assert_allclose(o_s, o_f, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(l_s, l_f, rtol=1e-13, atol=1e-13)


def test_sparse_k1_is_block_local_causal():
    q, k, v, s, scale = _tiny_case(40)
    L = q.shape[2]
    idx = O.block_topk(q, O.block_pool(k, s), s, 1)
    o_s, l_s = O.attend_sparse(q, k, v, idx, s, scale)
    for j in range(L // s):
        sl = slice(j * s, j * s + s)
        o_b, l_b = O.attend_full(q[:, :, sl], k[:, :, sl], v[:, :, sl], scale)
        np.testing.assert_allclose(o_s[:, :, sl], o_b, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(l_s[:, :, sl], l_b, rtol=1e-13, atol=1e-13)


def test_sparse_q_zero_is_mean_over_attended_tokens():
    """q = 0: every logit is 0, so o_s(t) is the plain mean of v over A(t) and
    lse_s(t) = log |A(t)|, with |A(t)| given in closed form."""
    q, k, v, s, scale = _tiny_case(50, L=160, s=16)
    L = q.shape[2]
    q = np.zeros_like(q)
    for topk in (1, 3, 10):
        idx = O.block_topk(q, O.block_pool(k, s), s, topk)
        o_s, l_s = O.attend_sparse(q, k, v, idx, s, scale)
        for t in range(L):
            bt = t // s
            m = min(topk - 1, bt)
            keys = [i for j in list(range(m)) + [bt] for i in range(j * s, min(j * s + s, t + 1))]
            assert len(keys) == O.attended_count(t, s, topk)
            np.testing.assert_allclose(o_s[:, :, t], v[:, :, keys].mean(axis=2), rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(l_s[:, :, t], np.log(len(keys)), rtol=1e-13)


def test_sparse_s1_is_token_topk():
    """s = 1: blocks are single tokens, so the sparse stream attends token t plus the
    topk-1 earlier tokens with the largest q.k (raw scores).  Keys on a line,
    k_i = c_i e_0, make the kept set a closed form."""
    L, D, topk = 30, 3, 4
    c = np.sin(np.arange(L) * 1.7) * 3
    k = np.zeros((1, 1, L, D))
    k[0, 0, :, 0] = c
    q = np.zeros((1, 1, L, D))
    q[..., 0] = 1.0
    v = _rand((1, 1, L, D), 60)
    idx = O.block_topk(q, O.block_pool(k, 1), 1, topk)
    o_s, _ = O.attend_sparse(q, k, v, idx, 1, 0.9)
    for t in range(L):
        prev = sorted(range(t), key=lambda i: (-c[i], i))[: topk - 1]
        keys = sorted(prev) + [t]
        w = np.exp(0.9 * c[keys])
        np.testing.assert_allclose(o_s[0, 0, t], (w[:, None] * v[0, 0, keys]).sum(0) / w.sum(), rtol=1e-12)


def test_sparse_ignores_padding_and_out_of_range_entries():
    q, k, v, s, scale = _tiny_case(70)
    idx = O.block_topk(q, O.block_pool(k, s), s, 4)
    o1, l1 = O.attend_sparse(q, k, v, idx, s, scale)
    wide = np.concatenate([idx, np.full(idx.shape[:-1] + (2,), -1, np.int32)], axis=-1)
    o2, l2 = O.attend_sparse(q, k, v, wide, s, scale)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ----------------------------------------------------------------------------------
# dropped mass and alignment statistics
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("topk", [1, 3, 6])
def test_dropped_mass_identity_and_bound(topk):
    """Splitting full attention into attended and dropped keys (App. B, Theorem 1):
    o_f = (1 - delta) o_s + delta * o_drop exactly, where o_drop is the probability-
    weighted mean of v over the dropped keys; hence ||o_f - o_s|| = delta ||o_drop - o_s||
    <= 2 delta max_{j<=t} ||v_j||."""
    q, k, v, s, scale = _tiny_case(80, L=96, s=8)
    L = q.shape[2]
    idx = O.block_topk(q, O.block_pool(k, s), s, topk)
    o_f, l_f = O.attend_full(q, k, v, scale)
    o_s, l_s = O.attend_sparse(q, k, v, idx, s, scale)
    dm = O.dropped_mass(q, k, idx, s, scale)
    for b, h, t in itertools.product(range(q.shape[0]), range(q.shape[1]), range(L)):
        kept = {i for j in O.attended_blocks(idx[b, h, t], t, s) for i in range(j * s, j * s + s) if i <= t}
        drop = [i for i in range(t + 1) if i not in kept]
        d = dm[b, h, t]
        if not drop:
            assert d == 0.0
            np.testing.assert_allclose(o_f[b, h, t], o_s[b, h, t], rtol=1e-12, atol=1e-12)
            continue
        lg = scale * np.array([q[b, h, t] @ k[b, h, i] for i in drop])
        w = np.exp(lg - lg.max())
        o_drop = (w[:, None] * v[b, h, drop]).sum(0) / w.sum()
        np.testing.assert_allclose(o_f[b, h, t], (1 - d) * o_s[b, h, t] + d * o_drop, rtol=1e-11, atol=1e-12)
        vmax = np.linalg.norm(v[b, h, : t + 1], axis=1).max()
        assert np.linalg.norm(o_f[b, h, t] - o_s[b, h, t]) <= 2 * d * vmax * (1 + 1e-12)
    # the log-sum-exp route gives the same dropped mass
    _, dm2 = O.align_stats(lse_full=l_f, lse_sparse=l_s)
    np.testing.assert_allclose(dm2, dm, rtol=1e-10, atol=1e-13)


def test_dropped_mass_q_zero_closed_form():
    """q = 0: uniform full attention, so delta(t) = 1 - |A(t)| / (t + 1); and delta = 0
    whenever b_t < topk (every preceding block is kept)."""
    q, k, v, s, scale = _tiny_case(90, L=128, s=8)
    q = np.zeros_like(q)
    topk = 4
    idx = O.block_topk(q, O.block_pool(k, s), s, topk)
    dm = O.dropped_mass(q, k, idx, s, scale)
    L = q.shape[2]
    expect = np.array([1.0 - O.attended_count(t, s, topk) / (t + 1) for t in range(L)])
    np.testing.assert_allclose(dm[0, 0], expect, rtol=1e-12, atol=1e-15)
    assert np.all(dm[..., : topk * s] == 0.0)


def test_align_stats_closed_forms():
    o_f = np.zeros((1, 1, 3, 4))
    o_s = np.zeros((1, 1, 3, 4))
    o_f[0, 0, 0, :2] = [3.0, 4.0]                    # distance 5
    o_s[0, 0, 1] = [1.0, 1.0, 1.0, 1.0]              # distance 2
    o_f[0, 0, 2, 3] = -2.5                           # distance 2.5
    lse_f = np.array([[[0.0, np.log(4.0), 10.0]]])
    lse_s = np.array([[[0.0, np.log(1.0), 10.0 + 1e-9]]])   # 0, 3/4, slightly above -> clipped
    dist, dm = O.align_stats(o_f, o_s, lse_f, lse_s)
    np.testing.assert_allclose(dist[0, 0], [5.0, 2.0, 2.5], rtol=1e-15)
    np.testing.assert_allclose(dm[0, 0], [0.0, 0.75, 0.0], rtol=1e-14, atol=0)
    d1, d2 = O.align_stats(o_f, o_s, None, None)
    assert d2 is None and d1 is not None


# ----------------------------------------------------------------------------------
# the pins catch planted slips (mutation check on a copy of the oracle)
# ----------------------------------------------------------------------------------
def test_planted_mistakes_are_caught(monkeypatch):
    """Plant typical slips in the oracle on the CPU and check that at least one pin
    above then fails."""
    orig_mask = O._sparse_key_mask

    def mask_strict_causal(idx_rows, R, s, nkeys):   # i < t instead of i <= t
        m = orig_mask(idx_rows, R, s, nkeys)
        m[np.arange(len(R)), R] = False
        return m

    def mask_drop_own_block(idx_rows, R, s, nkeys):  # forget the own block
        m = orig_mask(idx_rows, R, s, nkeys)
        keys = np.arange(nkeys)
        own = (keys[None, :] // s) == (R[:, None] // s)
        return m & ~own | (m & own & (keys[None, :] == R[:, None]))

    def _ties_high(q, k_mean, s, topk, rows=None, return_scores=False):
        B, H, L, D = q.shape
        idx = np.full((B, H, L, topk), -1, np.int32)
        for b, h, t in itertools.product(range(B), range(H), range(L)):
            bt = t // s
            m = min(topk - 1, bt)
            sc = [float(q[b, h, t] @ k_mean[b, h, j]) for j in range(bt)]
            order = sorted(range(bt), key=lambda j: (-sc[j], -j))[:m]
            idx[b, h, t, : m + 1] = sorted(order) + [bt]
        return idx

    orig_full = O.attend_full

    def full_without_scale(q, k, v, scale, rows=None, want_o=True):
        return orig_full(q, k, v, 1.0, rows, want_o)

    def full_transposed_qk(q, k, v, scale, rows=None, want_o=True):   # q and k swapped
        return orig_full(k, q, v, scale, rows, want_o)

    def align_wrong_sign(o_full=None, o_sparse=None, lse_full=None, lse_sparse=None):
        dist = None if o_full is None else np.sqrt(((np.asarray(o_full) - o_sparse) ** 2).sum(-1))
        x = np.asarray(lse_full) - np.asarray(lse_sparse)
        return dist, np.clip(-np.expm1(x), 0.0, 1.0)

    checks = [test_golden_tiny_L4_s2, test_golden_select_ties, test_topk_q_zero_keeps_lowest_blocks,
              test_sparse_q_zero_is_mean_over_attended_tokens, test_dropped_mass_q_zero_closed_form,
              test_full_designed_weights_closed_form, test_full_is_causal_and_rows_subset_consistent,
              test_align_stats_closed_forms]
    for name, fake in (("_sparse_key_mask", mask_strict_causal),
                       ("_sparse_key_mask", mask_drop_own_block),
                       ("block_topk", _ties_high),
                       ("attend_full", full_without_scale),
                       ("attend_full", full_transposed_qk),
                       ("align_stats", align_wrong_sign)):
        with monkeypatch.context() as mp:
            mp.setattr(O, name, fake)
            failed = 0
            for chk in checks:
                try:
                    chk()
                except AssertionError:
                    failed += 1
            assert failed > 0, f"planted slip in {name} ({fake.__name__}) went unnoticed"


# ----------------------------------------------------------------------------------
# decoding with a key/value cache: open_block_mean, decode_step
# ----------------------------------------------------------------------------------
def test_open_block_mean_closed_forms():
    """The open block's mean over the c = t - b_t s + 1 tokens present: the token itself
    when it opens a block, block_pool's mean when it closes one, and (integer keys) an
    exact integer sum over c in between (summed here with a plain loop)."""
    s, L, D = 8, 64, 5
    ki = np.random.default_rng(7).integers(-50, 50, (L, D)).astype(np.float64)
    km = O.block_pool(ki[None, None], s)[0, 0]
    for t in range(L):
        mean = O.open_block_mean(ki, t, s)
        c = t % s + 1
        brute = np.zeros(D)
        for i in range((t // s) * s, t + 1):
            brute += ki[i]
        np.testing.assert_array_equal(np.round(mean * c), brute)
        np.testing.assert_allclose(mean * c, brute, rtol=0, atol=1e-12)
        if c == 1:
            np.testing.assert_array_equal(mean, ki[t])
        if c == s:
            np.testing.assert_array_equal(mean, km[t // s])
    # tokens after t are not read
    poisoned = ki.copy()
    poisoned[20:] = np.nan
    np.testing.assert_array_equal(O.open_block_mean(poisoned, 19, s), O.open_block_mean(ki, 19, s))


@pytest.mark.parametrize("topk", [1, 3, 10])
def test_decode_step_matches_prefill_rows(topk):
    """A decoding step at position t, formed from the cache alone (and blind to rows
    after t), equals row t of the whole-sequence forward: selection, both streams."""
    q, k, v, s, scale = _tiny_case(60, L=160, s=16)
    km = O.block_pool(k, s)
    idx = O.block_topk(q, km, s, topk)
    o_s, l_s = O.attend_sparse(q, k, v, idx, s, scale)
    o_f, l_f = O.attend_full(q, k, v, scale)
    for h in range(q.shape[1]):
        for t in range(q.shape[2]):
            kc, vc = k[0, h].copy(), v[0, h].copy()
            kc[t + 1:] = np.nan
            vc[t + 1:] = np.nan
            r = O.decode_step(q[0, h, t], kc, vc, t, s, topk, scale)
            assert r["idx"].tolist() == idx[0, h, t].tolist(), (h, t)
            np.testing.assert_allclose(r["o_s"], o_s[0, h, t], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(r["lse_s"], l_s[0, h, t], rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(r["o_f"], o_f[0, h, t], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(r["lse_f"], l_f[0, h, t], rtol=1e-13, atol=1e-14)


def test_decode_step_q_zero_closed_form():
    """q = 0: all scores tie, so blocks 0..m-1 are kept; every logit is 0, so
    lse_s = log |A(t)|, lse_f = log(t + 1) and o_f is the mean of v over 0..t."""
    _, k, v, s, scale = _tiny_case(70, H=1, L=96, s=8)
    q0 = np.zeros(k.shape[-1])
    for topk in (1, 4, 12):
        for t in range(k.shape[2]):
            r = O.decode_step(q0, k[0, 0], v[0, 0], t, s, topk, scale)
            bt = t // s
            m = min(topk - 1, bt)
            assert r["idx"].tolist() == list(range(m)) + [bt] + [-1] * (topk - m - 1)
            assert math.isclose(r["lse_s"], math.log(O.attended_count(t, s, topk)), rel_tol=1e-13)
            assert math.isclose(r["lse_f"], math.log(t + 1), rel_tol=1e-13, abs_tol=1e-15)
            np.testing.assert_allclose(r["o_f"], v[0, 0, :t + 1].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_decode_planted_mistakes_are_caught(monkeypatch):
    """Slips planted in a copy of decode_step (the open block scored as a candidate, a
    strictly causal mask, ties to the higher block) fail one of the decode pins."""
    def own_block_candidate(q_t, k_bh, v_bh, t, s, topk, scale):
        q = np.asarray(q_t, dtype=np.float64)
        K, V = np.asarray(k_bh[:t + 1], float), np.asarray(v_bh[:t + 1], float)
        bt = t // s
        cand = list(range(bt + 1))
        sc = [q @ K[j * s:min(j * s + s, t + 1)].mean(axis=0) for j in cand]
        kept = sorted(sorted(cand, key=lambda j: (-sc[j], j))[:topk])
        if bt not in kept:
            kept = sorted(kept[:topk - 1] + [bt])
        return _finish(q, K, V, t, s, topk, scale, kept)

    def strict_causal(q_t, k_bh, v_bh, t, s, topk, scale):
        r = orig(q_t, k_bh, v_bh, t, s, topk, scale)
        if t > 0:
            r2 = orig(q_t, k_bh, v_bh, t - 1, s, topk, scale)
            r["o_f"], r["lse_f"] = r2["o_f"], r2["lse_f"]
        return r

    def ties_high(q_t, k_bh, v_bh, t, s, topk, scale):
        q = np.asarray(q_t, dtype=np.float64)
        K, V = np.asarray(k_bh[:t + 1], float), np.asarray(v_bh[:t + 1], float)
        bt = t // s
        m = min(topk - 1, bt)
        sc = [q @ K[j * s:j * s + s].mean(axis=0) for j in range(bt)]
        kept = sorted(sorted(range(bt), key=lambda j: (-sc[j], -j))[:m]) + [bt]
        return _finish(q, K, V, t, s, topk, scale, kept)

    def _finish(q, K, V, t, s, topk, scale, blocks):
        idx = np.full(topk, -1, np.int32)
        idx[:len(blocks)] = blocks
        keys = np.concatenate([np.arange(j * s, min(j * s + s, t + 1)) for j in blocks])
        lg = scale * (K[keys] @ q)
        e = np.exp(lg - lg.max())
        lf = scale * (K @ q)
        ef = np.exp(lf - lf.max())
        return {"idx": idx, "o_s": e @ V[keys] / e.sum(), "lse_s": lg.max() + np.log(e.sum()),
                "o_f": ef @ V / ef.sum(), "lse_f": lf.max() + np.log(ef.sum())}

    orig = O.decode_step
    checks = [lambda: test_decode_step_matches_prefill_rows(3), test_decode_step_q_zero_closed_form]
    for fake in (own_block_candidate, strict_causal, ties_high):
        with monkeypatch.context() as mp:
            mp.setattr(O, "decode_step", fake)
            failed = 0
            for chk in checks:
                try:
                    chk()
                except AssertionError:
                    failed += 1
            assert failed > 0, f"planted slip {fake.__name__} went unnoticed"


# ----------------------------------------------------------------------------------
# training: attention backward and the alignment loss, pinned by finite differences
# ----------------------------------------------------------------------------------
def _fd_grad(f, x, h=1e-5):
    """Central finite differences of the scalar f at x (float64), element by element."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + h
        fp = f()
        x[i] = old - h
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * h)
    return g


@pytest.mark.parametrize("stream", ["full", "sparse"])
def test_attention_bwd_matches_finite_differences(stream):
    """dq, dk, dv against central differences of F = sum(do * o) through the forward
    oracle (the sparse stream with its selection held fixed)."""
    B, H, L, D, s, topk, scale = 1, 2, 24, 4, 4, 3, 0.7
    q, k, v, do = (_rand((B, H, L, D), 80 + i) for i in range(4))
    idx = O.block_topk(q, O.block_pool(k, s), s, topk)

    def F():
        if stream == "full":
            o, _ = O.attend_full(q, k, v, scale)
        else:
            o, _ = O.attend_sparse(q, k, v, idx, s, scale)
        return float((o * do).sum())

    if stream == "full":
        dq, dk, dv = O.attend_full_bwd(q, k, v, do, scale)
    else:
        dq, dk, dv = O.attend_sparse_bwd(q, k, v, do, idx, s, scale)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        np.testing.assert_allclose(g, _fd_grad(F, x), rtol=1e-6, atol=1e-8, err_msg=f"d{name}")


def test_attention_bwd_q_zero_closed_form():
    """q = 0: each row's weights are uniform over its attended keys, so
    dv_i = sum over rows t attending i of do_t / |A(t)|, and dk = 0 (every logit
    is 0 whatever k is, and stays so to first order in k)."""
    B, H, L, D, s, topk, scale = 1, 1, 40, 3, 4, 3, 0.9
    _, k, v, do = (_rand((B, H, L, D), 90 + i) for i in range(4))
    q = np.zeros((B, H, L, D))
    idx = O.block_topk(q, O.block_pool(k, s), s, topk)
    for stream in ("full", "sparse"):
        if stream == "full":
            _, dk, dv = O.attend_full_bwd(q, k, v, do, scale)
            sets = [list(range(t + 1)) for t in range(L)]
        else:
            _, dk, dv = O.attend_sparse_bwd(q, k, v, do, idx, s, scale)
            sets = [[i for j in O.attended_blocks(idx[0, 0, t], t, s) for i in range(j * s, min(j * s + s, t + 1))]
                    for t in range(L)]
        ref = np.zeros((L, D))
        for t in range(L):
            for i in sets[t]:
                ref[i] += do[0, 0, t] / len(sets[t])
        np.testing.assert_allclose(dv[0, 0], ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dk, 0.0, atol=1e-13)


def test_align_loss_closed_forms_and_gradient():
    """SmoothL1: 0.5 x^2 / beta inside the threshold, |x| - beta/2 outside; the loss is
    alpha times the two equal means; each gradient matches central differences of its
    own term with the other output held; identical outputs give zero loss and zero
    gradients."""
    beta, alpha = 0.5, 0.3
    x = np.array([-2.0, -0.5, -0.2, 0.0, 0.1, 0.49, 0.5, 3.0])
    np.testing.assert_allclose(O.smooth_l1(x, beta), [1.75, 0.25, 0.04, 0.0, 0.01, 0.2401, 0.25, 2.75], rtol=1e-14)
    of, os_ = _rand((1, 2, 5, 3), 95), _rand((1, 2, 5, 3), 96) * 0.4
    loss, gf, gs = O.align_loss(of, os_, alpha, beta)
    N = of.size
    manual = 0.0
    for a, b in zip(of.ravel(), os_.ravel()):
        d = abs(a - b)
        manual += 0.5 * d * d / beta if d < beta else d - 0.5 * beta
    assert math.isclose(loss, 2 * alpha * manual / N, rel_tol=1e-13)
    held = os_.copy()
    gf_fd = _fd_grad(lambda: alpha * float(O.smooth_l1(of - held, beta).mean()), of, h=1e-7)
    np.testing.assert_allclose(gf, gf_fd, rtol=1e-5, atol=1e-9)
    held_f = of.copy()
    gs_fd = _fd_grad(lambda: alpha * float(O.smooth_l1(os_ - held_f, beta).mean()), os_, h=1e-7)
    np.testing.assert_allclose(gs, gs_fd, rtol=1e-5, atol=1e-9)
    l0, g0f, g0s = O.align_loss(of, of, alpha, beta)
    assert l0 == 0.0 and not g0f.any() and not g0s.any()


def test_bwd_planted_mistakes_are_caught(monkeypatch):
    """Slips planted in the backward (the softmax term dropped, the scale left out of
    dq, dS used untransposed for dk) fail the finite-difference pin."""
    orig = O._attend_bwd_masked

    def no_delta(q, k, v, do, scale, mask):
        lg = np.where(mask, scale * (q @ k.T), -np.inf)
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        ds = p * (do @ v.T)
        return scale * (ds @ k), scale * (ds.T @ q), p.T @ do

    def no_scale_dq(q, k, v, do, scale, mask):
        dq, dk, dv = orig(q, k, v, do, scale, mask)
        return dq / scale, dk, dv

    def dk_untransposed(q, k, v, do, scale, mask):
        dq, dk, dv = orig(q, k, v, do, scale, mask)
        lg = np.where(mask, scale * (q @ k.T), -np.inf)
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        dp = do @ v.T
        ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
        return dq, scale * (ds @ q), dv

    for fake in (no_delta, no_scale_dq, dk_untransposed):
        with monkeypatch.context() as mp:
            mp.setattr(O, "_attend_bwd_masked", fake)
            failed = 0
            for stream in ("full", "sparse"):
                try:
                    test_attention_bwd_matches_finite_differences(stream)
                except AssertionError:
                    failed += 1
            assert failed > 0, f"planted slip {fake.__name__} went unnoticed"


# ----------------------------------------------------------------------------------
# attention-pattern measurements
# ----------------------------------------------------------------------------------
def test_distance_bucket_values():
    assert [O.distance_bucket(d) for d in (0, 1, 2, 3, 4, 7, 8, 1023, 1024)] == [0, 1, 2, 2, 3, 3, 4, 10, 11]
    assert O.distance_bucket(1 << 20) == O.N_DIST_BUCKETS - 1


def test_attention_stats_q_zero_closed_form():
    """q = 0: weights uniform over A(t), so entropy = log |A(t)| and the histogram is the
    count of attended keys per bucket divided by |A(t)|, summed over rows; every row's
    mass is 1, so each head's histogram sums to L."""
    B, H, L, D, s, topk = 1, 2, 96, 4, 8, 3
    k = _rand((B, H, L, D), 101)
    q = np.zeros((B, H, L, D))
    idx = O.block_topk(q, O.block_pool(k, s), s, topk)
    for sparse in (False, True):
        ent, hist = O.attention_stats(q, k, s, 0.5, idx if sparse else None)
        ref = np.zeros(O.N_DIST_BUCKETS)
        for t in range(L):
            blocks = O.attended_blocks(idx[0, 0, t], t, s) if sparse else list(range(t // s + 1))
            keys = [i for j in blocks for i in range(j * s, min(j * s + s, t + 1))]
            assert math.isclose(ent[0, 0, t], math.log(len(keys)), rel_tol=1e-12, abs_tol=1e-15)
            for i in keys:
                ref[O.distance_bucket(t // s - i // s)] += 1.0 / len(keys)
        np.testing.assert_allclose(hist[0, 0], ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(hist.sum(axis=-1), L, rtol=1e-12)


def test_attention_stats_brute_force():
    """Entropy and histogram against a per-row loop over the forward oracle's weights
    (recovered from o with one-hot values: v = identity picks each weight)."""
    B, H, L, s, scale = 1, 1, 20, 4, 0.3
    q, k = _rand((B, H, L, L), 111), _rand((B, H, L, L), 112)   # head dim = L for the one-hot v
    v = np.eye(L)[None, None]            # o_t = (p_t0, ..., p_t,L-1)
    o, _ = O.attend_full(q, k, v, scale)
    ent, hist = O.attention_stats(q, k, s, scale)
    ref_h = np.zeros(O.N_DIST_BUCKETS)
    for t in range(L):
        p = o[0, 0, t, :t + 1]
        assert math.isclose(ent[0, 0, t], float(-(p * np.log(p)).sum()), rel_tol=1e-12)
        for i in range(t + 1):
            ref_h[O.distance_bucket(t // s - i // s)] += p[i]
    np.testing.assert_allclose(hist[0, 0], ref_h, rtol=1e-12, atol=1e-14)


def test_topk_sigma_bounds_hand_worked():
    """block_topk's sigma_m (score of the last kept candidate) and sigma_m1 (best score
    left out), which bound the tie band the parity rule allows, worked by hand.  q = e_0
    and the pooled keys' first components are the block scores; s = 2, query row t = 10
    (block 5) so blocks 0..4 compete.
      scores [5, 3, 9, 1, 7], topk 3 (m = 2): order 9 (j2), 7 (j4), 5 (j0), 3, 1 ->
        kept {2, 4}, sigma_m = 7, sigma_m1 = 5;
      scores [5, 7, 7, 1, 0], topk 2 (m = 1): equal scores by lower index -> kept {1},
        sigma_m = 7 (j1), sigma_m1 = 7 (j2);
      topk 6 (m = 5 = b_t, every candidate kept): sigma_m = 1 (the smallest),
        sigma_m1 = NaN (nothing left out);
      a row in block 0 has no candidate: both NaN."""
    L, s, D = 12, 2, 4
    q = np.zeros((1, 1, L, D))
    q[0, 0, :, 0] = 1.0
    for scores, topk, kept, sm, sm1 in (([5, 3, 9, 1, 7], 3, [2, 4], 7.0, 5.0),
                                        ([5, 7, 7, 1, 0], 2, [1], 7.0, 7.0),
                                        ([5, 3, 9, 1, 7], 6, [0, 1, 2, 3, 4], 1.0, np.nan)):
        km = np.zeros((1, 1, L // s, D))
        km[0, 0, :5, 0] = scores
        idx, ex = O.block_topk(q, km, s, topk, rows=np.array([10, 1]), return_scores=True)
        assert idx[0, 0, 0].tolist() == kept + [5] + [-1] * (topk - len(kept) - 1)
        assert ex["sigma_m"][0, 0, 0] == sm
        if np.isnan(sm1):
            assert np.isnan(ex["sigma_m1"][0, 0, 0])
        else:
            assert ex["sigma_m1"][0, 0, 0] == sm1
        assert np.isnan(ex["sigma_m"][0, 0, 1]) and np.isnan(ex["sigma_m1"][0, 0, 1])


def test_retained_mass_hist_hand_worked():
    """Bins of r = 1 - dropped, worked by hand: r = 1 (dropped 0) and r = 15/16 go to the
    last bin, r = 1/2 to bin 8, r just below 1/2 to bin 7, r = 0.01 and r = 0 to bin 0;
    a second head with every row at r = 1/4 puts all of them in bin 4."""
    d0 = np.array([0.0, 1.0 / 16.0, 0.5, 0.5 + 1e-9, 0.99, 1.0])
    d1 = np.full(6, 0.75)
    got = O.retained_mass_hist(np.stack([d0, d1])[None])
    want = np.zeros((1, 2, 16))
    want[0, 0, 15] = 2
    want[0, 0, 8] = 1
    want[0, 0, 7] = 1
    want[0, 0, 0] = 2
    want[0, 1, 4] = 6
    np.testing.assert_array_equal(got, want)
    # each head's counts sum to L
    rng = np.random.default_rng(7)
    dd = rng.random((2, 3, 50))
    np.testing.assert_array_equal(O.retained_mass_hist(dd).sum(axis=-1), 50)
