"""GPU parity of the training calls (backward of both streams, alignment loss) against the
CPU oracle (float64 chain rule, pinned by finite differences).  Needs an MI355X.

Tolerance: gradients are float32 from bf16 (or fp32) inputs.  The GPU forms the softmax
term with delta_t = sum_d do_t,d o_t,d from the STORED output o of its own forward, which
carries that forward's error (within its 2e-2 / 1e-4 bar: bf16 rounding of o and of the
probabilities in the value products), while the oracle uses the exact o; every other step
is float32 arithmetic on the same inputs.  The bound used is the outputs' own
bar scaled to the gradient's size: max |gpu - oracle| <= TOL[dtype] * max |oracle| per
tensor (2e-2 for bf16, 1e-4 for fp32).  The sparse stream is checked on the GPU's own
selection (the selection carries no gradient).
"""
import math
import sys

import numpy as np
import pytest

import workloads as W
from parity import TOL, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_sparse_top_ssa_amd as ssa  # noqa: E402
import oracle.ssa_oracle as O  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def close_rel(gpu, ref, tol, what):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite values"
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = float(np.abs(gpu - ref).max()) / scale
    assert err <= tol, f"{what}: max error {err:.3e} of max |ref| {scale:.3e} > {tol:.1e}"
    return err


def _kv_sum(a, H, Hkv):
    """[B, H, ...] per-query-head gradients summed into their key/value heads."""
    g = H // Hkv
    return a.reshape(a.shape[0], Hkv, g, *a.shape[2:]).sum(axis=2)


def forward_backward(inp, s, topk, do_f, do_s, tag=""):
    """GPU: both forwards, then both backwards into shared dq, dk, dv (float32)."""
    w = inp.workload
    scale = 1.0 / math.sqrt(w.D)
    q, k, v = (to_device(a, w.dtype) for a in (inp.q, inp.k, inp.v))
    km = ssa.block_pool(k, s)
    idx = ssa.block_topk(q, km, s, topk)
    o_s, lse_s = ssa.sparse_attn_fwd(q, k, v, idx, s, scale)
    o_f, lse_f = ssa.full_attn_fwd(q, k, v, scale, block=s)
    dof, dos = to_device(do_f, w.dtype), to_device(do_s, w.dtype)
    say(f"[gpu] train {tag} B={w.B} H={w.H} Hkv={w.hkv} L={w.L} D={w.D} s={s} topk={topk} {w.dtype}")
    dq, dk, dv = ssa.full_attn_bwd(q, k, v, o_f, lse_f, dof, scale=scale, block=s)
    g_full = [t.clone() for t in (dq, dk, dv)]
    ssa.sparse_attn_bwd(q, k, v, o_s, lse_s, dos, idx, s, dq, dk, dv, scale=scale)
    torch.cuda.synchronize()
    return dict(idx=idx.cpu().numpy(), full=[to_f64(t) for t in g_full], both=[to_f64(t) for t in (dq, dk, dv)])


@pytest.fixture(params=[0, 1], ids=["mfma", "portable"])
def variant(request):
    prev = ssa.set_kernel_variant(request.param)
    yield request.param
    ssa.set_kernel_variant(prev)


@pytest.mark.parametrize("dtype,D,s,Hkv", [(W.BF16, 128, 64, 4), (W.BF16, 64, 128, 2), (W.F32, 128, 64, 4),
                                           (W.F32, 64, 64, 1), (W.BF16, 128, 64, 1)])
def test_attention_bwd_both_streams(variant, dtype, D, s, Hkv):
    B, H, L, topk = 1, 4, 512, 3
    inp = W.make_qkv(B, H, L, D, s, dtype, "sink", seed=3100 + D + s + Hkv, hkv=Hkv)
    rng = np.random.default_rng(3200 + D)
    do_f = rng.standard_normal((B, H, L, D), dtype=np.float32) * np.float32(0.1)
    do_s = rng.standard_normal((B, H, L, D), dtype=np.float32) * np.float32(0.1)
    if dtype == W.BF16:
        do_f, do_s = W.f32_to_bf16_bits(do_f), W.f32_to_bf16_bits(do_s)
    g = forward_backward(inp, s, topk, do_f, do_s, tag=f"D={D}")
    scale = 1.0 / math.sqrt(D)
    q64 = inp.as_f64("q")
    k64, v64 = (inp.kv_per_query_head(inp.as_f64(n)) for n in ("k", "v"))
    dof64 = (W.bf16_bits_to_f32(do_f) if dtype == W.BF16 else do_f).astype(np.float64)
    dos64 = (W.bf16_bits_to_f32(do_s) if dtype == W.BF16 else do_s).astype(np.float64)
    rf = O.attend_full_bwd(q64, k64, v64, dof64, scale)
    rs = O.attend_sparse_bwd(q64, k64, v64, dos64, g["idx"], s, scale)
    tol = TOL[dtype]
    errs = {}
    for i, nm in enumerate(("dq", "dk", "dv")):
        ref_f = rf[i] if i == 0 else _kv_sum(rf[i], H, Hkv)
        ref_both = rf[i] + rs[i] if i == 0 else _kv_sum(rf[i] + rs[i], H, Hkv)
        errs[nm + "_full"] = close_rel(g["full"][i], ref_f, tol, nm + " (full stream)")
        errs[nm + "_both"] = close_rel(g["both"][i], ref_both, tol, nm + " (full + sparse)")
    say(f"[oracle] train D={D} s={s} Hkv={Hkv} {dtype} variant={variant}: {errs}")


def test_sparse_bwd_alone_matches_oracle():
    """The sparse stream's gradients by themselves (zeroed buffers), k = 1 (own block only)
    and k = n (every earlier block: equal to the full stream's gradients)."""
    B, H, L, D, s = 1, 2, 256, 128, 64
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "none", seed=3301)
    q, k, v = (to_device(a, W.BF16) for a in (inp.q, inp.k, inp.v))
    do = W.f32_to_bf16_bits(np.random.default_rng(3302).standard_normal((B, H, L, D), dtype=np.float32))
    dod = to_device(do, W.BF16)
    q64, k64, v64 = inp.as_f64("q"), inp.as_f64("k"), inp.as_f64("v")
    do64 = W.bf16_bits_to_f32(do).astype(np.float64)
    km = ssa.block_pool(k, s)
    for topk in (1, L // s):
        idx = ssa.block_topk(q, km, s, topk)
        o_s, lse_s = ssa.sparse_attn_fwd(q, k, v, idx, s)
        dq, dk, dv = ssa.sparse_attn_bwd(q, k, v, o_s, lse_s, dod, idx, s)
        torch.cuda.synchronize()
        ref = O.attend_sparse_bwd(q64, k64, v64, do64, idx.cpu().numpy(), s, 1.0 / math.sqrt(D))
        for got, r, nm in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
            close_rel(to_f64(got), r, TOL[W.BF16], f"{nm} k={topk}")
        if topk == L // s:
            rf = O.attend_full_bwd(q64, k64, v64, do64, 1.0 / math.sqrt(D))
            for r1, r2 in zip(ref, rf):
                np.testing.assert_allclose(r1, r2, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("D,Hkv", [(128, 2), (64, 1)])
def test_full_bwd_length_not_multiple_of_256(D, Hkv):
    """The full stream's gradients at L = 384, where the dense dq kernel takes its 128-row
    form (four waves per workgroup: L is not a multiple of 256)."""
    B, H, L, s = 1, 2, 384, 64
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "sink", seed=3800 + D, hkv=Hkv)
    q, k, v = (to_device(a, W.BF16) for a in (inp.q, inp.k, inp.v))
    do = W.f32_to_bf16_bits(np.random.default_rng(3801 + D).standard_normal((B, H, L, D), dtype=np.float32)
                            * np.float32(0.1))
    scale = 1.0 / math.sqrt(D)
    o, lse = ssa.full_attn_fwd(q, k, v, scale, block=s)
    dq, dk, dv = ssa.full_attn_bwd(q, k, v, o, lse, to_device(do, W.BF16), scale=scale, block=s)
    torch.cuda.synchronize()
    q64 = inp.as_f64("q")
    k64, v64 = (inp.kv_per_query_head(inp.as_f64(n)) for n in ("k", "v"))
    ref = O.attend_full_bwd(q64, k64, v64, W.bf16_bits_to_f32(do).astype(np.float64), scale)
    errs = {}
    for i, (got, nm) in enumerate(zip((dq, dk, dv), ("dq", "dk", "dv"))):
        r = ref[i] if i == 0 else _kv_sum(ref[i], H, Hkv)
        errs[nm] = close_rel(to_f64(got), r, TOL[W.BF16], f"{nm} L={L} D={D}")
    say(f"[oracle] full bwd L={L} D={D} Hkv={Hkv}: {errs}")


@pytest.mark.parametrize("B,H,Hkv,L,D,s,topk,padded", [
    (1, 2, 2, 384, 128, 64, 5, False),    # last tile of rows ragged (128 of 256)
    (1, 2, 1, 384, 64, 128, 2, True),     # 128-token blocks, grouped heads, padded rows
    (2, 2, 1, 2048, 128, 64, 16, True),   # several tiles, grouped heads, padded rows
    (1, 1, 1, 4096, 128, 64, 32, False),  # 32 entries per row, as in the long-context workload
    (1, 2, 2, 4096, 64, 64, 48, True),    # more than 32 entries per row (idx walked from memory), D = 64
])
def test_sparse_bwd_gathered_rows(B, H, Hkv, L, D, s, topk, padded):
    """The sparse stream's gradients alone on shapes that exercise the gathered-row dq:
    a ragged last row tile, several tiles, grouped K/V heads, 32 entries per row, and idx
    rows where some kept entries are replaced by -1 or by a block index past the end
    (skipped, like the forward skips them)."""
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "sink", seed=3600 + L + topk, hkv=Hkv)
    q, k, v = (to_device(a, W.BF16) for a in (inp.q, inp.k, inp.v))
    rng = np.random.default_rng(3700 + L)
    do = W.f32_to_bf16_bits(rng.standard_normal((B, H, L, D), dtype=np.float32) * np.float32(0.1))
    dod = to_device(do, W.BF16)
    scale = 1.0 / math.sqrt(D)
    idx = ssa.block_topk(q, ssa.block_pool(k, s), s, topk)
    if padded:
        g = idx.cpu().numpy()
        hit = rng.random(g.shape) < 0.25
        g = np.where(hit, np.where(rng.random(g.shape) < 0.5, -1, L // s + 7), g).astype(np.int32)
        idx = torch.from_numpy(g).to(idx.device)
    say(f"[gpu] sparse bwd B={B} H={H} Hkv={Hkv} L={L} D={D} s={s} topk={topk} padded={padded}")
    o_s, lse_s = ssa.sparse_attn_fwd(q, k, v, idx, s, scale)
    dq, dk, dv = ssa.sparse_attn_bwd(q, k, v, o_s, lse_s, dod, idx, s, scale=scale)
    torch.cuda.synchronize()
    q64 = inp.as_f64("q")
    k64, v64 = (inp.kv_per_query_head(inp.as_f64(n)) for n in ("k", "v"))
    ref = O.attend_sparse_bwd(q64, k64, v64, W.bf16_bits_to_f32(do).astype(np.float64), idx.cpu().numpy(), s, scale)
    errs = {}
    for i, (got, nm) in enumerate(zip((dq, dk, dv), ("dq", "dk", "dv"))):
        r = ref[i] if i == 0 else _kv_sum(ref[i], H, Hkv)
        errs[nm] = close_rel(to_f64(got), r, TOL[W.BF16], f"{nm} L={L} topk={topk}")
    say(f"[oracle] sparse bwd L={L} topk={topk} padded={padded}: {errs}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_align_loss(dtype):
    B, H, L, D = 2, 3, 256, 128
    rng = np.random.default_rng(3401)
    of = rng.standard_normal((B, H, L, D), dtype=np.float32)
    os_ = of + rng.standard_normal((B, H, L, D), dtype=np.float32) * np.float32(0.7)
    if dtype == W.BF16:
        of, os_ = W.f32_to_bf16_bits(of), W.f32_to_bf16_bits(os_)
    alpha, beta = 0.3, 0.5
    loss, gf, gs = ssa.align_loss(to_device(of, dtype), to_device(os_, dtype), alpha, beta)
    torch.cuda.synchronize()
    f64 = (lambda a: W.bf16_bits_to_f32(a).astype(np.float64)) if dtype == W.BF16 else (lambda a: a.astype(np.float64))
    rl, rgf, rgs = O.align_loss(f64(of), f64(os_), alpha, beta)
    assert math.isclose(float(loss.item()), rl, rel_tol=1e-5), (float(loss.item()), rl)
    np.testing.assert_allclose(to_f64(gf), rgf, rtol=1e-5, atol=1e-12)
    np.testing.assert_allclose(to_f64(gs), rgs, rtol=1e-5, atol=1e-12)
    say(f"[oracle] align loss {dtype}: gpu {float(loss.item()):.9g} oracle {rl:.9g}")


def test_training_step_end_to_end():
    """One layer's training step: both forwards, the alignment loss, its gradients added
    to an upstream gradient of the main (full) stream, both backwards into shared
    buffers -- against the oracle's composition of the same steps."""
    B, H, Hkv, L, D, s, topk, alpha = 1, 4, 2, 512, 128, 64, 4, 0.5
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "sink", seed=3501, hkv=Hkv)
    q, k, v = (to_device(a, W.BF16) for a in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(D)
    km = ssa.block_pool(k, s)
    idx = ssa.block_topk(q, km, s, topk)
    o_s, lse_s = ssa.sparse_attn_fwd(q, k, v, idx, s, scale)
    o_f, lse_f = ssa.full_attn_fwd(q, k, v, scale, block=s)
    loss, gf, gs = ssa.align_loss(o_f, o_s, alpha)
    up = W.f32_to_bf16_bits(np.random.default_rng(3502).standard_normal((B, H, L, D), dtype=np.float32)
                            * np.float32(1e-3))
    do_f = (to_device(up, W.BF16).float() + gf).to(torch.bfloat16)
    do_s = gs.to(torch.bfloat16)
    dq, dk, dv = ssa.full_attn_bwd(q, k, v, o_f, lse_f, do_f, scale=scale, block=s)
    ssa.sparse_attn_bwd(q, k, v, o_s, lse_s, do_s, idx, s, dq, dk, dv, scale=scale)
    torch.cuda.synchronize()
    q64 = inp.as_f64("q")
    k64, v64 = (inp.kv_per_query_head(inp.as_f64(n)) for n in ("k", "v"))
    gidx = idx.cpu().numpy()
    of64, _ = O.attend_full(q64, k64, v64, scale)
    os64, _ = O.attend_sparse(q64, k64, v64, gidx, s, scale)
    rl, rgf, rgs = O.align_loss(of64, os64, alpha)
    # the loss of the GPU's own outputs (identical inputs) and of the oracle's exact ones
    rl_same = O.align_loss(to_f64(o_f), to_f64(o_s), alpha)[0]
    assert math.isclose(float(loss.item()), rl_same, rel_tol=1e-5), (float(loss.item()), rl_same)
    assert abs(float(loss.item()) - rl) <= 5e-2 * rl, (float(loss.item()), rl)
    # the backward on the same upstream gradients the GPU used (bf16 bits)
    dof64, dos64 = to_f64(do_f), to_f64(do_s)
    rf = O.attend_full_bwd(q64, k64, v64, dof64, scale)
    rs = O.attend_sparse_bwd(q64, k64, v64, dos64, gidx, s, scale)
    close_rel(to_f64(dq), rf[0] + rs[0], TOL[W.BF16], "dq")
    close_rel(to_f64(dk), _kv_sum(rf[1] + rs[1], H, Hkv), TOL[W.BF16], "dk")
    close_rel(to_f64(dv), _kv_sum(rf[2] + rs[2], H, Hkv), TOL[W.BF16], "dv")
    say(f"[oracle] training step: loss gpu {float(loss.item()):.6g} oracle {rl:.6g}")
