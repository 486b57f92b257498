"""The caller-owned fragment-order copies of k and v (ssa_kv_frag) and the forwards that
read them (ssa_sparse_attn_fwd_frag, ssa_full_attn_fwd_frag), through the C ABI, against
the default calls (which build the same copies in pool memory) and the CPU oracle.

The dense forward is deterministic, so its _frag form must give the same bits.  The sparse
forward's partial sums can be added in an order that differs between runs, so its two forms
are compared within one bf16 step of o (and 1e-6 relative in lse), and each is held
to the oracle's bar.
"""
import math
import sys

import numpy as np
import pytest

import workloads as W
from parity import TOL, TOL_LSE, assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_sparse_top_ssa_amd as ssa  # noqa: E402
import oracle.ssa_oracle as O  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("B,H,Hkv,L,D,s,topk", [
    (1, 2, 2, 1152, 128, 64, 4),     # ragged last 256-row tile, several kept blocks
    (2, 4, 2, 2048, 64, 128, 3),     # grouped K/V heads, D = 64, 128-token blocks
    (1, 2, 1, 2048, 128, 64, 32),    # k = n: every chunk handed to the dense kernel
])
def test_frag_forms_match_default_calls(B, H, Hkv, L, D, s, topk):
    say(f"[gpu] frag B={B} H={H} Hkv={Hkv} L={L} D={D} s={s} topk={topk}")
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "lowrank", seed=31, hkv=Hkv)
    q, k, v = (to_device(a, W.BF16) for a in (inp.q, inp.k, inp.v))
    scale = 1.0 / math.sqrt(D)
    idx = ssa.block_topk(q, ssa.block_pool(k, s), s, topk)
    o_s, lse_s = ssa.sparse_attn_fwd(q, k, v, idx, s, scale)
    o_f, lse_f = ssa.full_attn_fwd(q, k, v, scale, block=s)
    nbytes = ssa.kv_frag_bytes(k, s)
    assert nbytes == B * Hkv * L * D * 2
    kf, vf = ssa.kv_frag(k, v, s)
    # sentinel bits in the outputs: every row must be written by the _frag forms
    o_s2 = torch.full_like(q, float("nan"))
    o_f2 = torch.full_like(q, float("nan"))
    o_s2, lse_s2 = ssa.sparse_attn_fwd_frag(q, k, v, kf, vf, idx, s, scale, out=o_s2)
    o_f2, lse_f2 = ssa.full_attn_fwd_frag(q, k, v, vf, scale, block=s, out=o_f2)
    # a second use of the same copies gives the same result
    o_f3, _ = ssa.full_attn_fwd_frag(q, k, v, vf, scale, block=s)
    _, lse_only = ssa.full_attn_fwd_frag(q, k, v, None, scale, want_o=False, block=s)
    torch.cuda.synchronize()
    assert torch.equal(o_f2.view(torch.int16), o_f.view(torch.int16))
    assert torch.equal(o_f3.view(torch.int16), o_f.view(torch.int16))
    assert torch.equal(lse_f2, lse_f) and torch.equal(lse_only, lse_f)
    a, b = to_f64(o_s2), to_f64(o_s)
    assert np.isfinite(a).all()
    # one bf16 step of the larger magnitude (2^-7 of it at most) covers a last-bit float32
    # difference of the unnormalised sums
    ulp = 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-6
    assert np.all(np.abs(a - b) <= ulp), f"sparse forms differ by {np.abs(a - b).max():.3e}"
    np.testing.assert_allclose(to_f64(lse_s2), to_f64(lse_s), rtol=1e-6, atol=1e-6)
    # both against the oracle (every row), on the GPU's own selection
    k64, v64 = (inp.kv_per_query_head(inp.as_f64(x)) for x in ("k", "v"))
    q64 = inp.as_f64("q")
    os_, ls_ = O.attend_sparse(q64, k64, v64, idx.cpu().numpy(), s, scale)
    of_, lf_ = O.attend_full(q64, k64, v64, scale)
    assert_close(a, os_, TOL[W.BF16], "o_sparse (frag)")
    assert_close(to_f64(lse_s2), ls_, TOL_LSE[W.BF16], "lse_sparse (frag)")
    assert_close(to_f64(o_f2), of_, TOL[W.BF16], "o_full (frag)")
    assert_close(to_f64(lse_f2), lf_, TOL_LSE[W.BF16], "lse_full (frag)")
    say(f"[gpu] frag done")


def test_frag_copies_only_where_asked():
    """ssa_kv_frag writes only the copies asked for: the other buffer keeps its bytes."""
    B, H, L, D, s = 1, 2, 512, 128, 64
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "none", seed=32)
    k, v = (to_device(a, W.BF16) for a in (inp.k, inp.v))
    nbytes = ssa.kv_frag_bytes(k, s)
    kf_ref, vf_ref = ssa.kv_frag(k, v, s)
    kf = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    vf = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device="cuda")
    ssa.kv_frag(k, v, s, want_k=False, v_frag=vf)
    torch.cuda.synchronize()
    assert torch.equal(vf, vf_ref) and bool((kf == 0xA5).all())
    ssa.kv_frag(k, v, s, want_v=False, k_frag=kf)
    torch.cuda.synchronize()
    assert torch.equal(kf, kf_ref)
    # the copies are a permutation of k's and v's 16-bit values
    for src, cp in ((k, kf), (v, vf)):
        a = np.sort(src.view(torch.int16).cpu().numpy().ravel())
        b = np.sort(cp.view(torch.int16).cpu().numpy().ravel())
        assert np.array_equal(a, b)
