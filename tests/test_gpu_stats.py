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
