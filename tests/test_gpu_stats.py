"""GPU parity of the attention-pattern measurements (row entropy, attention mass by block
distance) against the CPU oracle.  Needs an MI355X.

The GPU forms the weights from the stream's own float32 log-sum-exp and float32 scores
of the same inputs, the oracle from its float64 softmax: entropy within 1e-3 nats,
histogram buckets within 1e-4 of the row count L (their sum)."""
import math
import sys

import numpy as np
import pytest

import workloads as W
from parity import to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_sparse_top_ssa_amd as ssa  # noqa: E402
import oracle.ssa_oracle as O  # noqa: E402


@pytest.fixture(params=[0, 1], ids=["mfma", "portable"])
def variant(request):
    prev = ssa.set_kernel_variant(request.param)
    yield request.param
    ssa.set_kernel_variant(prev)


@pytest.mark.parametrize("dtype,D,s,Hkv", [(W.BF16, 128, 64, 2), (W.BF16, 64, 128, 2), (W.F32, 128, 64, 2),
                                           (W.BF16, 128, 64, 1)])
@pytest.mark.parametrize("stream", ["full", "sparse"])
def test_attn_stats(variant, dtype, D, s, Hkv, stream):
    B, H, L, topk = 1, 2, 1024, 4
    inp = W.make_qkv(B, H, L, D, s, dtype, "sink", seed=4100 + D + s, hkv=Hkv)
    q, k, v = (to_device(a, dtype) for a in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(D)
    if stream == "full":
        idx = None
        _, lse = ssa.full_attn_fwd(q, k, v, scale, want_o=False, block=s)
    else:
        idx = ssa.block_topk(q, ssa.block_pool(k, s), s, topk)
        _, lse = ssa.sparse_attn_fwd(q, k, v, idx, s, scale)
    ent, hist = ssa.attn_stats(q, k, lse, s, idx=idx, scale=scale)
    torch.cuda.synchronize()
    q64 = inp.as_f64("q")
    k64 = inp.kv_per_query_head(inp.as_f64("k"))
    ref_e, ref_h = O.attention_stats(q64, k64, s, scale, None if idx is None else idx.cpu().numpy())
    ge, gh = to_f64(ent), to_f64(hist)
    err_e = float(np.abs(ge - ref_e).max())
    err_h = float(np.abs(gh - ref_h).max())
    print(f"[oracle] stats {stream} {dtype} D={D} s={s} Hkv={Hkv} variant={variant}: entropy {err_e:.2e} "
          f"hist {err_h:.2e} (sum {gh.sum(-1).tolist()})", flush=True)
    sys.stdout.flush()
    assert err_e <= 1e-3, err_e
    assert err_h <= 1e-4 * L, err_h
    np.testing.assert_allclose(gh.sum(axis=-1), L, rtol=1e-4)


@pytest.mark.parametrize("B,H,Hkv,L,D,s,topk,padded", [
    (1, 2, 1, 1152, 128, 64, 8, True),   # last tile of rows ragged (128 of 512), grouped heads
    (2, 1, 1, 640, 64, 128, 3, True),    # 128-token blocks, two sequences
    (1, 1, 1, 4096, 128, 64, 32, False),  # 32 entries per row, as in the long-context workload
    (1, 2, 2, 4096, 64, 64, 48, True),    # more than 32 entries per row, D = 64
])
def test_sparse_stats_gathered_rows(B, H, Hkv, L, D, s, topk, padded):
    """The sparse stream's measurements on shapes that exercise the gathered-row kernel,
    including idx rows where a quarter of the entries are -1 or a block past the end."""
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "sink", seed=4300 + L + topk, hkv=Hkv)
    q, k, v = (to_device(a, W.BF16) for a in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(D)
    idx = ssa.block_topk(q, ssa.block_pool(k, s), s, topk)
    if padded:
        rng = np.random.default_rng(4400 + L)
        g = idx.cpu().numpy()
        hit = rng.random(g.shape) < 0.25
        g = np.where(hit, np.where(rng.random(g.shape) < 0.5, -1, L // s + 7), g).astype(np.int32)
        idx = torch.from_numpy(g).to(idx.device)
    _, lse = ssa.sparse_attn_fwd(q, k, v, idx, s, scale)
    ent, hist = ssa.attn_stats(q, k, lse, s, idx=idx, scale=scale)
    torch.cuda.synchronize()
    q64 = inp.as_f64("q")
    k64 = inp.kv_per_query_head(inp.as_f64("k"))
    ref_e, ref_h = O.attention_stats(q64, k64, s, scale, idx.cpu().numpy())
    ge, gh = to_f64(ent), to_f64(hist)
    err_e = float(np.abs(ge - ref_e).max())
    err_h = float(np.abs(gh - ref_h).max())
    print(f"[oracle] sparse stats L={L} topk={topk} padded={padded}: entropy {err_e:.2e} hist {err_h:.2e}", flush=True)
    assert err_e <= 1e-3, err_e
    assert err_h <= 1e-4 * L, err_h
    np.testing.assert_allclose(gh.sum(axis=-1), L, rtol=1e-4)


@pytest.mark.parametrize("dtype,D,s,Hkv,L", [(W.BF16, 128, 64, 2, 1024), (W.BF16, 64, 128, 1, 1152),
                                             (W.BF16, 128, 128, 1, 640), (W.F32, 128, 64, 2, 1024)])
@pytest.mark.parametrize("want_o", [True, False])
def test_full_fwd_stats_fused(dtype, D, s, Hkv, L, want_o):
    """ssa_full_attn_fwd_stats: the full stream's entropy and distance histogram from the
    forward's own sweep (bf16; float32 runs the forward and the measurement pass) against
    the oracle, its o and lse those of ssa_full_attn_fwd; ragged last tile at L = 1152."""
    B, H = 1, 2
    inp = W.make_qkv(B, H, L, D, s, dtype, "sink", seed=4500 + D + s + L, hkv=Hkv)
    q, k, v = (to_device(a, dtype) for a in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(D)
    print(f"[case] fused stats {dtype} D={D} s={s} Hkv={Hkv} L={L} want_o={want_o}", flush=True)
    o, lse, ent, hist = ssa.full_attn_fwd_stats(q, k, v, scale, want_o=want_o, block=s)
    o2, lse2 = ssa.full_attn_fwd(q, k, v, scale, want_o=want_o, block=s)
    torch.cuda.synchronize()
    # the same arithmetic for o and lse as the plain forward (checked against the oracle there)
    assert torch.equal(lse, lse2)
    if want_o:
        assert torch.equal(o, o2)
    q64 = inp.as_f64("q")
    k64 = inp.kv_per_query_head(inp.as_f64("k"))
    ref_e, ref_h = O.attention_stats(q64, k64, s, scale)
    ge, gh = to_f64(ent), to_f64(hist)
    err_e = float(np.abs(ge - ref_e).max())
    err_h = float(np.abs(gh - ref_h).max())
    print(f"[oracle] fused full stats: entropy {err_e:.2e} hist {err_h:.2e} (sum {gh.sum(-1).tolist()})", flush=True)
    assert err_e <= 1e-3, err_e
    assert err_h <= 1e-4 * L, err_h
    np.testing.assert_allclose(gh.sum(axis=-1), L, rtol=1e-4)
    # only one of the measurements
    _, _, e_only, h_none = ssa.full_attn_fwd_stats(q, k, v, scale, want_o=False, want_lse=False, want_hist=False,
                                                   block=s)
    assert h_none is None and float(np.abs(to_f64(e_only) - ref_e).max()) <= 1e-3


@pytest.mark.parametrize("dtype,D,s,topk,L,B,H", [(W.BF16, 128, 64, 4, 1024, 2, 2), (W.F32, 64, 64, 2, 512, 1, 3),
                                                   (W.BF16, 64, 128, 3, 1280, 1, 2)])
def test_align_retained_hist(dtype, D, s, topk, L, B, H):
    """ssa_align_stats_hist: per head, rows counted by retained mass 1 - dropped in
    sixteenths, against the oracle's dropped mass on the GPU's selection.  A row may land
    in the neighbouring bin only where the oracle's retained mass lies within the dropped
    mass tolerance (2 TOL_LSE) of the edge: the cumulative counts are checked edge by edge."""
    from parity import TOL_LSE
    inp = W.make_qkv(B, H, L, D, s, dtype, "sink", seed=4700 + L + D, hkv=H)
    q, k, v = (to_device(a, dtype) for a in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(D)
    print(f"[case] retained hist {dtype} D={D} s={s} topk={topk} L={L} B={B} H={H}", flush=True)
    idx = ssa.block_topk(q, ssa.block_pool(k, s), s, topk)
    _, lse_s = ssa.sparse_attn_fwd(q, k, v, idx, s, scale)
    _, lse_f = ssa.full_attn_fwd(q, k, v, scale, want_o=False, block=s)
    _, drop, rh = ssa.align_stats(None, None, lse_f, lse_s, block=s, dims_like=q, want_retained_hist=True)
    _, drop2 = ssa.align_stats(None, None, lse_f, lse_s, block=s, dims_like=q)
    torch.cuda.synchronize()
    assert torch.equal(drop, drop2)
    q64 = inp.as_f64("q")
    k64 = inp.kv_per_query_head(inp.as_f64("k"))
    ref_drop = O.dropped_mass(q64, k64, idx.cpu().numpy(), s, scale)
    got = to_f64(rh)
    assert np.array_equal(got, np.round(got)), "counts are whole numbers"
    np.testing.assert_array_equal(got.sum(axis=-1), L)
    tol = 2 * TOL_LSE[dtype]
    r = 1.0 - ref_drop
    for m in range(1, 16):
        edge = m / 16.0
        below = got[..., :m].sum(axis=-1)
        lo = (r < edge - tol).sum(axis=-1)
        hi = (r < edge + tol).sum(axis=-1)
        assert np.all((lo <= below) & (below <= hi)), (m, below, lo, hi)
    print(f"[oracle] retained hist ok: {got.reshape(-1, 16)[0].tolist()}", flush=True)


@pytest.mark.parametrize("dtype,B,H,Hkv,L,D,s,topk,padded", [
    (W.BF16, 1, 2, 2, 1024, 128, 64, 4, False),
    (W.BF16, 2, 2, 1, 1152, 64, 128, 3, False),   # ragged last tile, 128-token blocks, grouped heads
    (W.BF16, 1, 1, 1, 4096, 128, 64, 32, False),  # 32 entries per row, as in the long-context workload
    (W.BF16, 1, 2, 2, 4096, 64, 64, 48, True),    # more than 32 entries per row, malformed entries
    (W.BF16, 1, 2, 1, 1024, 128, 64, 16, False),  # k = n: every query chunk goes to the dense kernel
    (W.F32, 1, 2, 2, 1024, 128, 64, 4, False),    # float32: the forward, then the measurement pass
])
def test_sparse_fwd_stats_fused(variant, dtype, B, H, Hkv, L, D, s, topk, padded):
    """ssa_sparse_attn_fwd_stats: the sparse stream's entropy and distance histogram from
    its own forward (bf16 matrix-core kernel, or the forward then the measurement pass)
    against the oracle on the same idx; its o and lse those of ssa_sparse_attn_fwd."""
    inp = W.make_qkv(B, H, L, D, s, dtype, "sink", seed=4800 + L + topk + D, hkv=Hkv)
    q, k, v = (to_device(a, dtype) for a in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(D)
    print(f"[case] fused sparse stats {dtype} B={B} H={H}/{Hkv} L={L} D={D} s={s} k={topk} padded={padded} "
          f"variant={variant}", flush=True)
    idx = ssa.block_topk(q, ssa.block_pool(k, s), s, topk)
    if padded:
        rng = np.random.default_rng(4900 + L)
        g = idx.cpu().numpy()
        hit = rng.random(g.shape) < 0.25
        g = np.where(hit, np.where(rng.random(g.shape) < 0.5, -1, L // s + 7), g).astype(np.int32)
        idx = torch.from_numpy(g).to(idx.device)
    o, lse, ent, hist = ssa.sparse_attn_fwd_stats(q, k, v, idx, s, scale)
    o2, lse2 = ssa.sparse_attn_fwd(q, k, v, idx, s, scale)
    torch.cuda.synchronize()
    a, b = to_f64(o), to_f64(o2)
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-6)
    np.testing.assert_allclose(to_f64(lse), to_f64(lse2), rtol=1e-6, atol=1e-6)
    q64 = inp.as_f64("q")
    k64 = inp.kv_per_query_head(inp.as_f64("k"))
    ref_e, ref_h = O.attention_stats(q64, k64, s, scale, idx.cpu().numpy())
    ge, gh = to_f64(ent), to_f64(hist)
    err_e = float(np.abs(ge - ref_e).max())
    err_h = float(np.abs(gh - ref_h).max())
    print(f"[oracle] fused sparse stats: entropy {err_e:.2e} hist {err_h:.2e} (sum {gh.sum(-1).tolist()})", flush=True)
    assert err_e <= 1e-3, err_e
    assert err_h <= 1e-4 * L, err_h
    np.testing.assert_allclose(gh.sum(axis=-1), L, rtol=1e-4)
    # only one of the measurements
    _, _, e_only, h_none = ssa.sparse_attn_fwd_stats(q, k, v, idx, s, scale, want_lse=False, want_hist=False)
    assert h_none is None and float(np.abs(to_f64(e_only) - ref_e).max()) <= 1e-3


def test_sparse_fwd_stats_recomputed_row():
    """A kept key far above everything in the query's own block (logit gap ~75) sends the
    row to the exact recompute; its measurements must come out exact too."""
    B, H, L, D, s = 1, 1, 1024, 128, 64
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "none", seed=17)
    qf, kf = W.bf16_bits_to_f32(inp.q), W.bf16_bits_to_f32(inp.k)
    qf[0, 0, 900] = 0.0
    qf[0, 0, 900, 0] = 30.0
    kf[0, 0, 130] = 0.0
    kf[0, 0, 130, 0] = 30.0
    inp.q, inp.k = W.f32_to_bf16_bits(qf), W.f32_to_bf16_bits(kf)
    q, k, v = (to_device(a, W.BF16) for a in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(D)
    print("[case] fused sparse stats, recomputed row", flush=True)
    idx = ssa.block_topk(q, ssa.block_pool(k, s), s, 4)
    assert 2 in idx[0, 0, 900].tolist()
    _, _, ent, hist = ssa.sparse_attn_fwd_stats(q, k, v, idx, s, scale)
    torch.cuda.synchronize()
    ref_e, ref_h = O.attention_stats(inp.as_f64("q"), inp.as_f64("k"), s, scale, idx.cpu().numpy())
    ge, gh = to_f64(ent), to_f64(hist)
    assert abs(ge[0, 0, 900] - ref_e[0, 0, 900]) <= 1e-3
    assert float(np.abs(ge - ref_e).max()) <= 1e-3
    assert float(np.abs(gh - ref_h).max()) <= 1e-4 * L
