"""The allocation-free sparse decoding call (ssa_decode_sparse_fwd_noalloc, scratch in a
fixed device array) against ssa_decode_sparse_fwd (scratch from the pool) on the same
seeded inputs: two calls in a row, the second with a smaller input, with and without a
caller-given idx (without it the kept blocks also live in the fixed array).  Kept blocks
must match bit for bit, o and lse within the bf16 output tolerance (the two calls run the
same kernels, so they are expected to agree exactly)."""
import math
import sys

import numpy as np
import pytest

import workloads as W
from parity import TOL, to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_sparse_top_ssa_amd as ssa  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _case(seed, B, H, Hkv, L, D, s):
    rng = np.random.default_rng(seed)
    k = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, L, D), dtype=np.float32))
    v = W.f32_to_bf16_bits(rng.standard_normal((B, Hkv, L, D), dtype=np.float32))
    q = W.f32_to_bf16_bits(rng.standard_normal((B, H, D), dtype=np.float32))
    pos = rng.integers(L // 2, L, size=B).astype(np.int32)
    pos[0] = L - 1
    kd, vd, qd = (to_device(a, W.BF16) for a in (k, v, q))
    return qd, kd, vd, ssa.block_pool(kd, s), torch.from_numpy(pos).cuda()


@pytest.mark.parametrize("give_idx", [True, False], ids=["idx", "no-idx"])
def test_noalloc_matches_pool_variant(give_idx):
    for seed, (B, H, Hkv, L, D, s, topk) in enumerate([(4, 16, 4, 8192, 128, 64, 32),   # larger first
                                                        (2, 4, 2, 1024, 64, 128, 3)]):   # then smaller
        say(f"[gpu] noalloc decode B={B} H={H} Hkv={Hkv} L={L} D={D} s={s} topk={topk} give_idx={give_idx}")
        q, k, v, km, pos = _case(100 + seed, B, H, Hkv, L, D, s)
        scale = 1.0 / math.sqrt(D)
        o_ref, lse_ref, idx_ref = ssa.decode_sparse_fwd(pos, q, k, v, km, s, topk, scale)
        o, lse, idx = ssa.decode_sparse_fwd_noalloc(pos, q, k, v, km, s, topk, scale, want_idx=give_idx)
        torch.cuda.synchronize()
        if give_idx:
            assert torch.equal(idx, idx_ref), "kept blocks differ"
        do = (o.float() - o_ref.float()).abs().max().item()
        dl = (lse - lse_ref).abs().max().item()
        say(f"[gpu] max |o - o_pool| {do:.3e}  max |lse - lse_pool| {dl:.3e}")
        assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
        assert do <= TOL[W.BF16] and dl <= TOL[W.BF16]
