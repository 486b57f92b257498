"""GPU parity: the HIP path (called through the C ABI via the ctypes binding) against
the CPU oracle on the same seeded inputs.  Needs an MI355X.

Rules (tests/parity.py): selections bit-exact up to score ties within 1e-5 relative;
outputs within 2e-2 (bf16) / 1e-4 (fp32) max abs error; the float32 log-sum-exps within
TOL_LSE and the dropped mass within twice that; the L2 distance per row within the
triangle-inequality bound of the two outputs' own errors; and the dropped-mass bound
||o_f - o_s|| <= 2 delta max_{j<=t} ||v_j|| on the GPU's outputs.  Every workload runs
the MFMA path (variant 0); the small ones also run the portable vector-ALU path
(variant 1).
"""
import functools
import math
import sys

import numpy as np
import pytest

import workloads as W
from parity import BOUND_SLACK, TOL, TOL_LSE, assert_close, compare_idx, max_abs, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_sparse_top_ssa_amd as ssa  # noqa: E402
import oracle.ssa_oracle as O  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(params=[0, 1], ids=["mfma", "portable"])
def variant(request):
    prev = ssa.set_kernel_variant(request.param)
    yield request.param
    ssa.set_kernel_variant(prev)


def gpu_pipeline(inp: W.Inputs, topk: int, lse_only_full=False, tag="", frag=False):
    """The whole path on the GPU.  With frag (bf16), the forwards run as bench.py times
    them: k and v written once by kv_frag, then the _frag forms; their outputs are also
    held to the default calls' on the same idx (the dense forward's bits, the sparse
    forward's within one bf16 step: its partial sums may be added in another order)."""
    w = inp.workload
    s, scale = w.s, 1.0 / math.sqrt(w.D)
    say(f"[gpu] {tag} B={w.B} H={w.H} L={w.L} D={w.D} s={s} topk={topk} dtype={w.dtype} frag={frag}")
    q, k, v = (to_device(a, w.dtype) for a in (inp.q, inp.k, inp.v))
    km = ssa.block_pool(k, s)
    idx, sel = ssa.block_topk(q, km, s, topk, want_scores=True)
    if frag:
        kf, vf = ssa.kv_frag(k, v, s)
        o_s, lse_s = ssa.sparse_attn_fwd_frag(q, k, v, kf, vf, idx, s, scale)
        o_f, lse_f = ssa.full_attn_fwd_frag(q, k, v, vf, scale, want_o=not lse_only_full, block=s)
        del kf, vf
        o_s2, lse_s2 = ssa.sparse_attn_fwd(q, k, v, idx, s, scale)
        o_f2, lse_f2 = ssa.full_attn_fwd(q, k, v, scale, want_o=not lse_only_full, block=s)
        torch.cuda.synchronize()
        assert torch.equal(lse_f, lse_f2) and (o_f is None or torch.equal(o_f.view(torch.int16),
                                                                          o_f2.view(torch.int16)))
        step = (o_s.float() - o_s2.float()).abs() <= 2.0 ** -7 * torch.maximum(o_s.float().abs(),
                                                                               o_s2.float().abs()) + 1e-6
        assert bool(step.all()), "sparse _frag form and default call differ by more than one bf16 step"
        torch.testing.assert_close(lse_s, lse_s2, rtol=1e-6, atol=1e-6)
        del o_s2, lse_s2, o_f2, lse_f2
    else:
        o_s, lse_s = ssa.sparse_attn_fwd(q, k, v, idx, s, scale)
        o_f, lse_f = ssa.full_attn_fwd(q, k, v, scale, want_o=not lse_only_full, block=s)
    if o_f is not None:
        dist, drop = ssa.align_stats(o_f, o_s, lse_f, lse_s, block=s)
    else:
        dist, drop = ssa.align_stats(None, None, lse_f, lse_s, block=s, dims_like=q)
    torch.cuda.synchronize()
    out = dict(km=km.cpu().numpy().astype(np.float64), idx=idx.cpu().numpy(), sel=sel.cpu().numpy(),
               o_s=to_f64(o_s), lse_s=to_f64(lse_s), lse_f=to_f64(lse_f), drop=to_f64(drop),
               o_f=None if o_f is None else to_f64(o_f), dist=None if dist is None else to_f64(dist))
    say(f"[gpu] {tag} done")
    return out


@functools.lru_cache(maxsize=4)
def _inputs(name):
    return W.make_workload(name)


def _oracle_checks(inp, g, topk, rows, lse_only_full=False, check_idx=True):
    """Compare one pipeline run with the oracle on `rows` (None = all)."""
    w = inp.workload
    tol = TOL[w.dtype]
    s, scale = w.s, 1.0 / math.sqrt(w.D)
    q64 = inp.as_f64("q")
    R = np.arange(w.L) if rows is None else rows
    km_kv = O.block_pool(inp.as_f64("k"), s)   # pooled keys of the key/value heads
    assert_close(g["km"], km_kv, 1e-5 * max(1.0, float(np.abs(km_kv).max())), "k_mean")
    # grouped key/value heads: each query head works with its group's k, v and kbar
    k64, v64, km = (inp.kv_per_query_head(a) for a in (inp.as_f64("k"), inp.as_f64("v"), km_kv))
    report = {}
    if check_idx:
        oidx, extra = O.block_topk(q64, km, s, topk, rows=R, return_scores=True)
        report.update(compare_idx(g["idx"][:, :, R], oidx, extra, q64, km, R, s, topk))
    gidx = g["idx"][:, :, R]
    # the sparse stream is checked on the GPU's own selection (identical up to ties)
    o_s, lse_s = O.attend_sparse(q64, k64, v64, gidx, s, scale, rows=R)
    tol_lse = TOL_LSE[w.dtype]
    report["o_s"] = assert_close(g["o_s"][:, :, R], o_s, tol, "o_sparse")
    report["lse_s"] = assert_close(g["lse_s"][:, :, R], lse_s, tol_lse, "lse_sparse")
    o_f, lse_f = O.attend_full(q64, k64, v64, scale, rows=R, want_o=not lse_only_full)
    if not lse_only_full:
        report["o_f"] = assert_close(g["o_f"][:, :, R], o_f, tol, "o_full")
    report["lse_f"] = assert_close(g["lse_f"][:, :, R], lse_f, tol_lse, "lse_full")
    dm = O.dropped_mass(q64, k64, gidx, s, scale, rows=R)
    report["dropped"] = assert_close(g["drop"][:, :, R], dm, 2 * tol_lse, "dropped mass")
    if not lse_only_full:
        dist, _ = O.align_stats(o_f, o_s)
        # |dist_gpu - dist| <= ||o_f,gpu - o_f|| + ||o_s,gpu - o_s|| row by row (triangle inequality)
        bound = (np.linalg.norm(g["o_f"][:, :, R] - o_f, axis=-1) + np.linalg.norm(g["o_s"][:, :, R] - o_s, axis=-1))
        derr = np.abs(g["dist"][:, :, R] - dist)
        assert np.all(derr <= bound + 1e-5), f"l2 distance off by {float((derr - bound).max()):.3e} beyond its bound"
        report["dist"] = float(derr.max())
        # App. B: o_f = (1 - delta) o_s + delta o_drop, so ||o_f - o_s|| <= 2 delta max_{j<=t} ||v_j||;
        # on the GPU's own outputs, with the slack rounding can add (parity.BOUND_SLACK)
        m_t = np.maximum.accumulate(np.linalg.norm(v64, axis=-1), axis=2)[:, :, R]
        lhs = g["dist"][:, :, R]
        rhs = 2 * g["drop"][:, :, R] * m_t + BOUND_SLACK[w.dtype] * m_t
        assert np.all(lhs <= rhs), f"dropped-mass bound violated by {float((lhs - rhs).max()):.3e}"
        report["bound_margin_min"] = float((rhs - lhs).min())
        # the same statistics from identical inputs (the GPU's own outputs)
        d2, dm2 = O.align_stats(g["o_f"], g["o_s"], g["lse_f"], g["lse_s"])
        assert np.allclose(g["dist"], d2, rtol=1e-5, atol=1e-6)
        assert np.allclose(g["drop"], dm2, rtol=1e-5, atol=1e-6)
    # selected scores (GPU float32) against the oracle's float64 scores of the same blocks
    sel = g["sel"][:, :, R]
    valid = (gidx >= 0) & (gidx < (R // s)[None, None, :, None])
    for b in range(w.B):
        for h in range(w.H):
            vv = valid[b, h]
            if vv.any():
                ra, ca = np.nonzero(vv)
                sc = np.einsum("rd,rd->r", q64[b, h, R[ra]], km[b, h, gidx[b, h, ra, ca]])
                assert np.allclose(sel[b, h, ra, ca], sc, rtol=1e-5, atol=1e-5 * np.abs(sc).max())
    assert np.all(np.isposinf(sel[gidx == (R // s)[None, None, :, None]]))
    assert np.all(np.isneginf(sel[gidx == -1]))
    say(f"[oracle] {report}")
    return report


# ----------------------------------------------------------------------------------
# block pool
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
@pytest.mark.parametrize("D,s", [(128, 64), (64, 128), (128, 128)])
def test_pool_integer_keys_bit_exact(variant, dtype, D, s):
    """Integer keys make every float32 block sum exact, so GPU == oracle bit for bit."""
    kk = W.integer_tensor((2, 3, 4 * s, D), -8, 8, seed=11)
    a = W.f32_to_bf16_bits(kk) if dtype == W.BF16 else kk
    say(f"[gpu] pool integer D={D} s={s} {dtype}")
    km = ssa.block_pool(to_device(a, dtype), s).cpu().numpy()
    np.testing.assert_array_equal(km, O.block_pool(kk.astype(np.float64), s).astype(np.float32))


# ----------------------------------------------------------------------------------
# selection special cases with closed forms
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("s,topk", [(64, 1), (64, 3), (64, 16), (128, 5)])
def test_topk_q_zero_closed_form(variant, s, topk):
    """q = 0: every score is exactly 0; the tie rule keeps blocks 0..m-1 plus b_t."""
    inp = W.make_qkv(1, 2, 16 * s, 128, s, W.BF16, "none", seed=12, q_zero=True)
    q, k = to_device(inp.q, W.BF16), to_device(inp.k, W.BF16)
    km = ssa.block_pool(k, s)
    idx = ssa.block_topk(q, km, s, topk).cpu().numpy()
    for t in range(16 * s):
        bt = t // s
        m = min(topk - 1, bt)
        assert idx[0, 1, t].tolist() == list(range(m)) + [bt] + [-1] * (topk - m - 1)


def test_topk_integer_ties_exact(variant):
    """Small integer q and k: block means are multiples of 1/64 and every score is exact
    in float32, with many exact ties; the selection must equal the oracle's exactly."""
    B, H, L, D, s, topk = 1, 4, 4096, 128, 64, 9
    q = W.integer_tensor((B, H, L, D), -1, 1, seed=13)
    k = W.integer_tensor((B, H, L, D), -2, 2, seed=14)
    qd, kd = to_device(W.f32_to_bf16_bits(q), W.BF16), to_device(W.f32_to_bf16_bits(k), W.BF16)
    km = ssa.block_pool(kd, s)
    idx = ssa.block_topk(qd, km, s, topk).cpu().numpy()
    oidx = O.block_topk(q.astype(np.float64), O.block_pool(k.astype(np.float64), s), s, topk)
    np.testing.assert_array_equal(idx, oidx)


def test_topk_lane_clustered_scores_exact():
    """Scores built so that the best blocks sit at few positions modulo 64 (the
    candidate's lane in a 64-wide chunk): blocks j with j % 64 < 12 score
    128 + 12 (j // 64) + j % 64, the others -(j % 64); q = e_0 and every key of block j
    equals (score_j, 0, ..., 0), so kbar and every score are exact small integers.  In
    the last query block more than 64 candidates reach the first lower bound of the
    two-pass selection, which must then tighten it and still return exactly the
    oracle's selection (ties among the negative scores go to the lower index)."""
    B, H, n, D, s, topk = 1, 1, 256, 128, 64, 32
    L = n * s
    j = np.arange(n)
    score = np.where(j % 64 < 12, 128 + 12 * (j // 64) + j % 64, -(j % 64)).astype(np.float32)
    k = np.zeros((B, H, L, D), np.float32)
    k[0, 0, :, 0] = np.repeat(score, s)
    q = np.zeros((B, H, L, D), np.float32)
    q[..., 0] = 1.0
    qd, kd = to_device(W.f32_to_bf16_bits(q), W.BF16), to_device(W.f32_to_bf16_bits(k), W.BF16)
    km = ssa.block_pool(kd, s)
    idx = ssa.block_topk(qd, km, s, topk).cpu().numpy()
    oidx = O.block_topk(q.astype(np.float64), O.block_pool(k.astype(np.float64), s), s, topk)
    np.testing.assert_array_equal(idx, oidx)
    # the last block keeps the 31 highest-scoring clustered blocks, then itself
    last = idx[0, 0, -1]
    expect = sorted(int(b) for b in j[:n - 1][np.argsort(-score[:n - 1], kind="stable")][:topk - 1])
    assert list(last[:topk - 1]) == expect and last[topk - 1] == n - 1


# ----------------------------------------------------------------------------------
# whole pipeline on the small workloads (every row)
# ----------------------------------------------------------------------------------
def test_fp32_L1024_D64_all_rows(variant):
    inp = _inputs("fp32_L1024_D64")
    g = gpu_pipeline(inp, 4, tag="fp32_L1024_D64")
    _oracle_checks(inp, g, 4, rows=None)


def test_bf16_L4096_lowrank_all_rows(variant):
    inp = _inputs("bf16_L4096_lowrank")
    g = gpu_pipeline(inp, 16, tag="bf16_L4096_lowrank")
    _oracle_checks(inp, g, 16, rows=None)


@pytest.mark.parametrize("topk", [4, 8, 16, 32, 64, 128])
def test_bf16_L8192_ksweep(topk):
    inp = _inputs("bf16_L8192_ksweep")
    w = inp.workload
    g = gpu_pipeline(inp, topk, tag=f"bf16_L8192_ksweep k={topk}", frag=True)
    rows = W.sample_rows(w.L, w.s, topk, w.sample_rows, seed=w.seed + topk)
    rep = _oracle_checks(inp, g, topk, rows=rows, check_idx=False)
    # selection on every row
    q64 = inp.as_f64("q")
    km = O.block_pool(inp.as_f64("k"), w.s)
    oidx, extra = O.block_topk(q64, km, w.s, topk, return_scores=True)
    rep.update(compare_idx(g["idx"], oidx, extra, q64, km, np.arange(w.L), w.s, topk))
    say(f"[oracle] k={topk} selection {rep}")
    if topk == w.n:
        # keeping every block is full attention
        assert max_abs(g["o_s"], g["o_f"]) <= 2e-2
        assert max_abs(g["lse_s"], g["lse_f"]) <= 1e-4
        assert np.all(g["drop"] <= 1e-4)


@pytest.mark.parametrize("H,Hkv,L,s,topk", [
    (2, 2, 16384, 64, 96),    # row lists of a 256-row tile up to 24 KB: about three batches
    (2, 2, 16384, 128, 48),   # block 128 (two 64-key chunks per block): two batches
    (4, 2, 8192, 64, 80),     # grouped K/V heads; m = 79 takes the merge selection
])
def test_sparse_row_lists_in_batches(H, Hkv, L, s, topk):
    """Long idx rows: a 256-row tile's row lists (one byte per kept block per row) do not
    fit beside its 128 KB O state, so the sparse kernel builds and consumes them in
    batches of consecutive blocks; every output must match the oracle as for short rows."""
    B, D = 1, 128
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "none", seed=21, hkv=Hkv)
    inp.workload = W.Workload("batches", B, H, L, D, s, (topk,), W.BF16, "none", 21, sample_rows=384, Hkv=Hkv)
    g = gpu_pipeline(inp, topk, tag=f"row-list batches L={L} s={s} k={topk}")
    rows = W.sample_rows(L, s, topk, 384, seed=21)
    rep = _oracle_checks(inp, g, topk, rows=rows)
    say(f"[oracle] row-list batches L={L} s={s} k={topk}: {rep}")


@pytest.mark.parametrize("B,H,Hkv,L,D,s,topk", [
    (1, 4, 2, 8192, 128, 64, 80),     # batched row lists with grouped K/V heads
    (1, 2, 2, 12288, 128, 128, 40),   # block 128, batched
    (2, 2, 1, 6144, 128, 64, 33),     # odd k, all query heads on one K/V head, two sequences
    (1, 3, 3, 5120, 64, 64, 50),      # D = 64: long rows in one batch
    (1, 2, 2, 16448, 128, 64, 120),   # ragged last 256-row tile, many batches, merge selection
    (3, 1, 1, 2304, 128, 128, 7),     # three sequences, block 128, ragged last tile
])
def test_mixed_shapes(B, H, Hkv, L, D, s, topk):
    """Shapes that combine the features the other cases take one at a time: batch size,
    grouped heads, long idx rows, ragged tiles and both block sizes, through the whole path
    against the oracle on sampled rows (the selection on every row)."""
    seed = 1000 + topk
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "none", seed=seed, hkv=Hkv)
    inp.workload = W.Workload("mixed", B, H, L, D, s, (topk,), W.BF16, "none", seed, Hkv=Hkv, sample_rows=256)
    g = gpu_pipeline(inp, topk, tag=f"mixed {B}x{H}/{Hkv}x{L}x{D} s={s} k={topk}")
    rows = W.sample_rows(L, s, topk, 256, seed=seed)
    rep = _oracle_checks(inp, g, topk, rows=rows)
    say(f"[oracle] mixed {B}x{H}/{Hkv}x{L}x{D} s={s} k={topk}: {rep}")


def test_sparse_row_lists_in_batches_d64():
    """D = 64 leaves most of the LDS to the row lists; idx rows of 400 blocks still need
    two batches per late tile.  The idx is a valid selection drawn at random (no top-k
    call): 399 earlier blocks, ascending, then the own block."""
    B, H, L, D, s, topk = 1, 1, 32768, 64, 64, 400
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "none", seed=31)
    rng = np.random.default_rng(5)
    idx = np.full((B, H, L, topk), -1, np.int32)
    for t in range(L):
        bt = t // s
        m = min(topk - 1, bt)
        idx[0, 0, t, :m] = np.sort(rng.choice(bt, size=m, replace=False)) if m < bt else np.arange(bt)
        idx[0, 0, t, m] = bt
    q, k, v = (to_device(a, W.BF16) for a in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(D)
    o, lse = ssa.sparse_attn_fwd(q, k, v, torch.from_numpy(idx).cuda(), s, scale)
    torch.cuda.synchronize()
    late = rng.choice(np.arange((topk - 1) * s, L), 96, replace=False)
    rows = np.unique(np.concatenate([late, [0, s - 1, s, (topk - 1) * s - 1, (topk - 1) * s, L - 1]]))
    o_ref, lse_ref = O.attend_sparse(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), idx[:, :, rows], s, scale,
                                     rows=rows)
    eo = assert_close(to_f64(o)[:, :, rows], o_ref, TOL[W.BF16], "o_sparse, D = 64, batched row lists")
    el = assert_close(to_f64(lse)[:, :, rows], lse_ref, TOL_LSE[W.BF16], "lse_sparse, D = 64, batched row lists")
    say(f"[oracle] D = 64 batched row lists: o {eo:.2e} lse {el:.2e}")


@pytest.mark.parametrize("s,topk", [(64, 4), (128, 3)])
def test_full_chunk_of_the_kth_block(variant, s, topk):
    """Rows of block k that list all k earlier blocks (the own block left out, which is
    always attended anyway) keep every earlier block, so their 64-row chunks are plain
    causal attention, which the sparse call hands to the dense kernel; those rows lie just
    past the k * s leading rows.  Every row must be written and match the oracle."""
    B, H, L, D = 1, 2, 1024, 128
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "none", seed=22)
    q, k, v = (to_device(a, W.BF16) for a in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(D)
    idx = ssa.block_topk(q, ssa.block_pool(k, s), s, topk).cpu().numpy().copy()
    idx[:, :, topk * s:(topk + 1) * s, :] = np.arange(topk, dtype=np.int32)
    big, o = _guarded(q.shape, torch.bfloat16)  # sentinel bits everywhere: unwritten rows show
    o_s, lse_s = ssa.sparse_attn_fwd(q, k, v, torch.from_numpy(idx.astype(np.int32)).cuda(), s, scale, out=o)
    torch.cuda.synchronize()
    assert _guards_intact(big, q.shape)
    o_ref, lse_ref = O.attend_sparse(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), idx, s, scale)
    assert_close(to_f64(o_s), o_ref, TOL[W.BF16], "o_sparse, full chunk of block k")
    assert_close(to_f64(lse_s), lse_ref, TOL_LSE[W.BF16], "lse_sparse, full chunk of block k")


# ----------------------------------------------------------------------------------
# closed forms on the GPU
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("s,topk,L", [(64, 4, 1024), (128, 3, 1024), (64, 1, 512)])
def test_q_zero_closed_forms(variant, s, topk, L):
    """q = 0: o_s(t) is the mean of v over A(t), lse_s = log|A(t)|, o_f the prefix mean,
    and the dropped mass 1 - |A(t)|/(t+1)."""
    inp = W.make_qkv(1, 2, L, 128, s, W.BF16, "none", seed=15, q_zero=True)
    g = gpu_pipeline(inp, topk, tag="q=0")
    v = inp.as_f64("v")
    cnt = np.array([O.attended_count(t, s, topk) for t in range(L)])
    pref = np.cumsum(v, axis=2) / np.arange(1, L + 1)[None, None, :, None]
    assert_close(g["o_f"], pref, 2e-2, "o_full prefix mean")
    assert_close(g["lse_f"][0, 0], np.log(np.arange(1, L + 1)), 1e-4, "lse_full")
    assert_close(g["lse_s"][0, 0], np.log(cnt), 1e-4, "lse_sparse")
    assert_close(g["drop"][0, 0], 1 - cnt / np.arange(1, L + 1), 1e-4, "dropped")
    for t in range(0, L, 37):
        bt = t // s
        m = min(topk - 1, bt)
        keys = [i for j in list(range(m)) + [bt] for i in range(j * s, min(j * s + s, t + 1))]
        assert_close(g["o_s"][:, :, t], v[:, :, keys].mean(axis=2), 2e-2, f"o_sparse row {t}")


# ----------------------------------------------------------------------------------
# edge shapes: one block, ragged tiles, odd head counts, D = 64 in bf16
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("B,H,L,D,s,topk", [
    (1, 1, 64, 128, 64, 1),      # a single block
    (1, 3, 192, 128, 64, 2),     # L not a multiple of the 256-row tile
    (2, 1, 640, 64, 64, 3),      # bf16 with D = 64
    (1, 2, 384, 128, 128, 2),    # block 128, ragged tile
    (3, 1, 1280, 128, 64, 20),   # topk = n
    (1, 2, 8192, 128, 128, 48),  # m = 47: the merge selection with one 64-key list, block 128
    (1, 2, 4096, 128, 64, 56),   # m = 55: the same with block 64
])
def test_edge_shapes(variant, B, H, L, D, s, topk):
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "none", seed=16)
    inp.workload = W.Workload("edge", B, H, L, D, s, (topk,), W.BF16, "none", 16)
    g = gpu_pipeline(inp, topk, tag=f"edge {B}x{H}x{L}x{D} s={s}")
    _oracle_checks(inp, g, topk, rows=None)


@pytest.mark.parametrize("B,H,Hkv,L,D,s,topk", [
    (2, 8, 2, 2048, 128, 64, 8),    # four query heads per key/value head
    (1, 6, 3, 1024, 64, 128, 3),    # D = 64, block 128, groups of two
    (1, 4, 1, 1280, 128, 64, 6),    # one key/value head for all, ragged 256-row tile
])
def test_grouped_kv_heads(variant, B, H, Hkv, L, D, s, topk):
    """Grouped-query attention: query head h attends key/value head h // (H // Hkv) and
    selects its own blocks from that head's pooled keys; the oracle runs on k and v
    repeated per group."""
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "lowrank", seed=18, hkv=Hkv)
    inp.workload = W.Workload("gqa", B, H, L, D, s, (topk,), W.BF16, "lowrank", 18, Hkv=Hkv)
    g = gpu_pipeline(inp, topk, tag=f"gqa {B}x{H}/{Hkv}x{L}x{D} s={s}")
    assert g["km"].shape == (B, Hkv, L // s, D)
    _oracle_checks(inp, g, topk, rows=None)


def test_huge_logit_row_recomputed(variant):
    """A key far more aligned with the query than anything in the query's own block
    (logit gap ~75) must still give the exact sparse softmax."""
    B, H, L, D, s = 1, 1, 1024, 128, 64
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "none", seed=17)
    qf, kf = W.bf16_bits_to_f32(inp.q), W.bf16_bits_to_f32(inp.k)
    qf[0, 0, 900] = 0.0
    qf[0, 0, 900, 0] = 30.0
    kf[0, 0, 130] = 0.0
    kf[0, 0, 130, 0] = 30.0
    inp.q, inp.k = W.f32_to_bf16_bits(qf), W.f32_to_bf16_bits(kf)
    inp.workload = W.Workload("huge", B, H, L, D, s, (4,), W.BF16, "none", 17)
    g = gpu_pipeline(inp, 4, tag="huge logit")
    assert 2 in g["idx"][0, 0, 900].tolist()
    _oracle_checks(inp, g, 4, rows=np.array([0, 130, 899, 900, 901, 1023]))


def test_full_stream_growing_logits(variant):
    """Logits that rise steadily along the sequence (about 170 log2 units from the first
    key to the last), so every row's later chunks outgrow the exponent reference set by
    its first chunk many times over: the dense stream's rescaling (and, on matrix cores,
    its recovery from row sums past 2^64) must still give the exact softmax."""
    B, H, L, D, s = 1, 2, 2048, 128, 64
    rng = np.random.default_rng(4501)
    a = np.linspace(0.0, 10.6, L)  # key strength along the sequence
    q = 1.0 + 0.1 * rng.standard_normal((B, H, L, D))
    k = a[None, None, :, None] * (1.0 + 0.05 * rng.standard_normal((B, H, L, D)))
    v = rng.standard_normal((B, H, L, D))
    qb, kb, vb = (W.f32_to_bf16_bits(x.astype(np.float32)) for x in (q, k, v))
    scale = 1.0 / math.sqrt(D)
    o, lse = ssa.full_attn_fwd(to_device(qb, W.BF16), to_device(kb, W.BF16), to_device(vb, W.BF16), scale, block=s)
    torch.cuda.synchronize()
    R = np.array([0, 1, 63, 64, 65, 700, 1023, 1024, 1500, 2047])
    q64, k64, v64 = (W.bf16_bits_to_f32(x).astype(np.float64) for x in (qb, kb, vb))
    ro, rl = O.attend_full(q64, k64, v64, scale, rows=R)
    eo = assert_close(to_f64(o)[:, :, R], ro, TOL[W.BF16], "o_full")
    el = assert_close(to_f64(lse)[:, :, R], rl, 1e-3 * max(1.0, float(np.abs(rl).max())), "lse_full")
    say(f"[oracle] growing logits (lse up to {float(np.abs(rl).max()):.1f}) variant={variant}: o {eo:.2e} lse {el:.2e}")


# ----------------------------------------------------------------------------------
# long-context workloads, in bench.py's launch configuration: sampled rows for outputs,
# selection on every row
# ----------------------------------------------------------------------------------
def _big(name, head_groups):
    inp = _inputs(name)
    w = inp.workload
    topk = w.ks[0]
    g = gpu_pipeline(inp, topk, lse_only_full=w.sparse_only, tag=name, frag=True)
    rows = W.sample_rows(w.L, w.s, topk, w.sample_rows, seed=w.seed)
    _oracle_checks(inp, g, topk, rows=rows, lse_only_full=w.sparse_only, check_idx=False)
    q64 = inp.as_f64("q")
    km = inp.kv_per_query_head(O.block_pool(inp.as_f64("k"), w.s))
    tot = {"rows": 0, "tolerated": 0}
    for hs in head_groups:
        sl = slice(hs[0], hs[1])
        oidx, extra = O.block_topk(q64[:, sl], km[:, sl], w.s, topk, return_scores=True)
        r = compare_idx(g["idx"][:, sl], oidx, extra, q64[:, sl], km[:, sl], np.arange(w.L), w.s, topk)
        tot = {k: tot[k] + r[k] for k in tot}
        say(f"[oracle] {name} heads {hs}: {r}")
    return tot


@pytest.mark.slow
def test_bf16_L32768_sink():
    _big("bf16_L32768_sink", [(0, 8), (8, 16), (16, 24), (24, 32)])


@pytest.mark.slow
def test_bf16_L131072_drift():
    _big("bf16_L131072_drift", [(0, 2), (2, 4), (4, 6), (6, 8)])


@pytest.mark.slow
def test_bf16_L32768_gqa2():
    _big("bf16_L32768_gqa2", [(0, 8), (8, 16), (16, 24), (24, 32)])


# ----------------------------------------------------------------------------------
# guard bands: nothing is written outside an output, on ragged and malformed inputs
# ----------------------------------------------------------------------------------
_PAD = 1024
_SENTINEL = {torch.bfloat16: (torch.int16, 0x5A5A), torch.float32: (torch.int32, 0x5A5A5A5A),
             torch.int32: (torch.int32, 0x5A5A5A5A), torch.uint8: (torch.uint8, 0x5A)}


def _guarded(shape, dtype):
    """An output of `shape` inside a larger buffer whose _PAD elements on either side
    hold a sentinel bit pattern; returns (buffer, the output view)."""
    n = int(np.prod(shape))
    big = torch.empty(n + 2 * _PAD, dtype=dtype, device="cuda")
    raw_t, pat = _SENTINEL[dtype]
    big.view(raw_t).fill_(pat)
    return big, big[_PAD:_PAD + n].view(shape)


def _guards_intact(big, shape):
    n = int(np.prod(shape))
    raw_t, pat = _SENTINEL[big.dtype]
    raw = big.view(raw_t)
    return bool((raw[:_PAD] == pat).all().item() and (raw[_PAD + n:] == pat).all().item())


@pytest.mark.parametrize("B,H,L,D,s,topk", [
    (1, 3, 192, 128, 64, 2),     # L not a multiple of the 256-row tile
    (1, 2, 384, 128, 128, 2),    # block 128, ragged tile
    (2, 1, 640, 64, 64, 3),      # D = 64
    (1, 2, 1344, 128, 64, 6),    # leading chunks left to the dense kernel, ragged last tile
    (1, 1, 4096, 128, 64, 48),   # long idx rows: the sparse kernel's row lists built in batches
])
def test_outputs_guarded(variant, B, H, L, D, s, topk):
    """Every output of the whole path written into a buffer with sentinel guard bands
    (the fragment-order copies, the forwards that read them and the forwards with
    measurements included): the bands stay intact, on the selection the path makes and on
    idx rows with a quarter of the entries replaced by -1 or by blocks past the query's own
    block or past the end; the outputs on the malformed rows match the oracle on the same
    rows."""
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "none", seed=19)
    say(f"[gpu] guarded {B}x{H}x{L}x{D} s={s} topk={topk}")
    q, k, v = (to_device(a, W.BF16) for a in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(D)
    bufs = {}

    def out(name, shape, dtype):
        bufs[name] = (*_guarded(shape, dtype), shape)
        return bufs[name][1]

    km = ssa.block_pool(k, s, out=out("km", (B, H, L // s, D), torch.float32))
    idx = ssa.block_topk(q, km, s, topk, out=out("idx", (B, H, L, topk), torch.int32))
    ssa.sparse_attn_fwd(q, k, v, idx, s, scale, out=out("o_s", q.shape, torch.bfloat16),
                        lse=out("lse_s", (B, H, L), torch.float32))
    ssa.full_attn_fwd(q, k, v, scale, block=s, out=out("o_f", q.shape, torch.bfloat16),
                      lse=out("lse_f", (B, H, L), torch.float32))
    # the fragment-order copies, the forwards that read them, the forwards with measurements
    nbytes = ssa.kv_frag_bytes(k, s)
    kf, vf = ssa.kv_frag(k, v, s, k_frag=out("k_frag", (nbytes,), torch.uint8),
                         v_frag=out("v_frag", (nbytes,), torch.uint8))
    ssa.sparse_attn_fwd_frag(q, k, v, kf, vf, idx, s, scale, out=out("o_sf", q.shape, torch.bfloat16),
                             lse=out("lse_sf", (B, H, L), torch.float32))
    ssa.full_attn_fwd_frag(q, k, v, vf, scale, block=s, out=out("o_ff", q.shape, torch.bfloat16),
                           lse=out("lse_ff", (B, H, L), torch.float32))
    ssa.sparse_attn_fwd_stats(q, k, v, idx, s, scale, out=out("o_ss", q.shape, torch.bfloat16),
                              lse=out("lse_ss", (B, H, L), torch.float32),
                              entropy=out("ent_s", (B, H, L), torch.float32),
                              hist=out("hist_s", (B, H, 16), torch.float32))
    ssa.full_attn_fwd_stats(q, k, v, scale, block=s, out=out("o_fs", q.shape, torch.bfloat16),
                            lse=out("lse_fs", (B, H, L), torch.float32),
                            entropy=out("ent_f", (B, H, L), torch.float32),
                            hist=out("hist_f", (B, H, 16), torch.float32))
    # malformed rows: a quarter of the entries become -1, a block past b_t, or past the end
    bad = idx.cpu().numpy().copy()
    rng = np.random.default_rng(20)
    hit = rng.random(bad.shape) < 0.25
    t = np.arange(L)[None, None, :, None]
    repl = rng.choice(3, size=bad.shape)
    bad[hit & (repl == 0)] = -1
    bad = np.where(hit & (repl == 1), np.broadcast_to(t // s + 1, bad.shape), bad)
    bad[hit & (repl == 2)] = L // s + 7
    bad_d = torch.from_numpy(bad.astype(np.int32)).cuda()
    o_bad, lse_bad = ssa.sparse_attn_fwd(q, k, v, bad_d, s, scale, out=out("o_bad", q.shape, torch.bfloat16),
                                         lse=out("lse_bad", (B, H, L), torch.float32))
    o_bad_f, lse_bad_f = ssa.sparse_attn_fwd_frag(q, k, v, kf, vf, bad_d, s, scale,
                                                  out=out("o_bad_f", q.shape, torch.bfloat16),
                                                  lse=out("lse_bad_f", (B, H, L), torch.float32))
    ssa.sparse_attn_fwd_stats(q, k, v, bad_d, s, scale, out=out("o_bad_s", q.shape, torch.bfloat16),
                              lse=out("lse_bad_s", (B, H, L), torch.float32),
                              entropy=out("ent_bad", (B, H, L), torch.float32),
                              hist=out("hist_bad", (B, H, 16), torch.float32))
    torch.cuda.synchronize()
    for name, (big, _, shape) in bufs.items():
        assert _guards_intact(big, shape), f"{name}: write outside the output"
    o_ref, lse_ref = O.attend_sparse(inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v"), bad, s, scale)
    assert_close(to_f64(o_bad), o_ref, TOL[W.BF16], "o_sparse on malformed idx")
    assert_close(to_f64(lse_bad), lse_ref, TOL_LSE[W.BF16], "lse_sparse on malformed idx")
    assert_close(to_f64(o_bad_f), o_ref, TOL[W.BF16], "o_sparse (frag) on malformed idx")
    assert_close(to_f64(lse_bad_f), lse_ref, TOL_LSE[W.BF16], "lse_sparse (frag) on malformed idx")
