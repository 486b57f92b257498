"""The Python binding checks every tensor it hands to the C ABI -- shape, dtype, device
and contiguity of inputs, caller-given outputs and pooled keys -- and raises SSAError
before anything is launched (the C ABI cannot see buffer sizes).  CPU only: each call
below fails validation before the library or a device is touched."""
import pytest
import torch

import block_sparse_top_ssa_amd as ssa
from block_sparse_top_ssa_amd import SSAError

B, H, L, D, S = 1, 2, 256, 64, 64
N = L // S


def bf(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def code_of(fn):
    with pytest.raises(SSAError) as e:
        fn()
    return e.value.code


def u8(n):
    return torch.zeros(n, dtype=torch.uint8)


QKV = dict(q=bf(B, H, L, D), k=bf(B, H, L, D), v=bf(B, H, L, D))
NFRAG = B * H * L * D * 2  # bytes of one fragment-order copy of k or v (bf16)


@pytest.mark.parametrize("fn,code", [
    # pooled keys must stay float32 (a bf16 k_mean would be read at twice its size)
    (lambda: ssa.block_topk(QKV["q"], bf(B, H, N, D), S, 2), 3),
    (lambda: ssa.block_topk(QKV["q"], f32(B, H, N + 1, D), S, 2), 2),
    (lambda: ssa.block_topk(QKV["q"], f32(B, H, N, D), S, 2, out=i32(B, H, L, 3)), 2),
    (lambda: ssa.block_pool(QKV["k"], S, out=f32(B, H, N, D + 1)), 2),
    # caller-given outputs of the forwards
    (lambda: ssa.sparse_attn_fwd(**QKV, idx=i32(B, H, L, 2), block=S, out=f32(B, H, L, D)), 3),
    (lambda: ssa.sparse_attn_fwd(**QKV, idx=i32(B, H, L, 2), block=S, lse=f32(B, H, L + 1)), 2),
    (lambda: ssa.sparse_attn_fwd(**QKV, idx=torch.zeros((B, H, L, 2), dtype=torch.int64), block=S), 2),
    (lambda: ssa.full_attn_fwd(**QKV, lse=f32(B, H, L - 1)), 2),
    (lambda: ssa.full_attn_fwd(**QKV, out=bf(B, H, L, D).t() if False else bf(B, H, L - 64, D)), 2),
    (lambda: ssa.align_stats(bf(B, H, L, D), bf(B, H, L, D), f32(B, H, L), None), 1),
    (lambda: ssa.align_stats(None, None, f32(B, H, L), bf(B, H, L), dims_like=bf(B, H, L, D)), 3),
    # decoding: pooled keys, caches, outputs, positions
    (lambda: ssa.decode_sparse_fwd(i32(B), bf(B, H, D), bf(B, H, L, D), bf(B, H, L, D), f32(B, H, N, D + 1), S, 2), 2),
    (lambda: ssa.decode_sparse_fwd(i32(B), bf(B, H, D), bf(B, H, L, D), bf(B, H, L, D), bf(B, H, N, D), S, 2), 3),
    (lambda: ssa.decode_sparse_fwd(torch.zeros(B, dtype=torch.int64), bf(B, H, D), bf(B, H, L, D), bf(B, H, L, D),
                                   f32(B, H, N, D), S, 2), 2),
    (lambda: ssa.decode_sparse_fwd_noalloc(i32(B), bf(B, H, D), bf(B, H, L, D), bf(B, H, L, D), f32(B, H, N, D), S, 2,
                                           idx=i32(B, H, 3)), 2),
    (lambda: ssa.decode_sparse_fwd_noalloc(i32(B), bf(B, H, D), bf(B, H, L, D), bf(B, H, L, D), f32(B, H, N, D), S, 2,
                                           out=f32(B, H, D)), 3),
    (lambda: ssa.decode_append(i32(B), bf(B, H, D), bf(B, H, D), bf(B, H, L, D), bf(B, H, L, D), f32(B, H, N - 1, D),
                               S), 2),
    (lambda: ssa.decode_full_fwd(i32(B), bf(B, H, D), bf(B, H, L, D), bf(B, H, L, D + 8)), 2),
    # training and measurements: lse, idx, k
    (lambda: ssa.full_attn_bwd(**QKV, o=bf(B, H, L, D), lse=bf(B, H, L), dout=bf(B, H, L, D)), 3),
    (lambda: ssa.sparse_attn_bwd(**QKV, o=bf(B, H, L, D), lse=f32(B, H, L), dout=bf(B, H, L, D),
                                 idx=i32(B, H, L, 2), block=S, dq=f32(B, H, L, D + 1)), 2),
    (lambda: ssa.attn_stats(QKV["q"], QKV["k"], f32(B, H, L - 1), S), 2),
    (lambda: ssa.attn_stats(QKV["q"], f32(B, H, L, D), f32(B, H, L), S), 3),
    (lambda: ssa.attn_stats(QKV["q"], QKV["k"], f32(B, H, L), S, idx=i32(B, H, L)), 2),
    # the fragment-order copies: sized by kv_frag_bytes, bytes (uint8), k and v alike
    (lambda: ssa.kv_frag(QKV["k"], bf(B, H, L, D + 64), S), 2),
    (lambda: ssa.kv_frag(QKV["k"], QKV["v"], S, k_frag=u8(NFRAG - 16)), 2),
    (lambda: ssa.sparse_attn_fwd_frag(**QKV, k_frag=u8(NFRAG), v_frag=u8(NFRAG // 2), idx=i32(B, H, L, 2), block=S), 2),
    (lambda: ssa.full_attn_fwd_frag(**QKV, v_frag=u8(NFRAG + 16)), 2),
    (lambda: ssa.full_attn_fwd_frag(**QKV, v_frag=torch.zeros(NFRAG, dtype=torch.int8)), 3),
    # the fused sparse measurements: the forward's own checks
    (lambda: ssa.sparse_attn_fwd_stats(**QKV, idx=i32(B, H, L, 2), block=S, lse=f32(B, H, L + 1)), 2),
    (lambda: ssa.sparse_attn_fwd_stats(**QKV, idx=i32(B, H, L), block=S), 2),
    # caller-given measurement outputs: entropy [B, H, L] and hist [B, H, 16], float32
    (lambda: ssa.sparse_attn_fwd_stats(**QKV, idx=i32(B, H, L, 2), block=S, entropy=f32(B, H, L - 1)), 2),
    (lambda: ssa.sparse_attn_fwd_stats(**QKV, idx=i32(B, H, L, 2), block=S, hist=bf(B, H, 16)), 3),
    (lambda: ssa.full_attn_fwd_stats(**QKV, block=S, hist=f32(B, H, 15)), 2),
    (lambda: ssa.full_attn_fwd_stats(**QKV, block=S, entropy=f32(B, H, L, 1)), 2),
])
def test_mismatched_tensor_raises_before_launch(fn, code):
    assert code_of(fn) == code
