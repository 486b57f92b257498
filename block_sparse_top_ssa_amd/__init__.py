"""SSA attention forward on MI355X: Python binding of libssa.

Argument marshalling only: every step of the computation runs in the HIP kernels of
libssa.so, called through its C ABI (include/ssa.h).  PyTorch provides device memory
and the stream: each call enqueues on torch's current stream and does not synchronise.

    k_mean = block_pool(k, block)
    idx = block_topk(q, k_mean, block, topk)
    o_s, lse_s = sparse_attn_fwd(q, k, v, idx, block)
    o_f, lse_f = full_attn_fwd(q, k, v)
    dist, dropped = align_stats(o_f, o_s, lse_f, lse_s)

Decoding with a key/value cache (one new query per sequence, positions in a device
int32 tensor `pos`, caches [B, Hkv, L, D] with L the capacity):

    decode_append(pos, k_new, v_new, k_cache, v_cache, k_mean, block)
    o_s, lse_s, idx = decode_sparse_fwd(pos, q, k_cache, v_cache, k_mean, block, topk)
    o_f, lse_f = decode_full_fwd(pos, q, k_cache, v_cache)

Training (gradients added into float32 buffers, the selection held fixed):

    loss, g_f, g_s = align_loss(o_f, o_s, alpha)
    full_attn_bwd(q, k, v, o_f, lse_f, do_f, dq, dk, dv)
    sparse_attn_bwd(q, k, v, o_s, lse_s, do_s, idx, block, dq, dk, dv)

q is [B, H, L, D]; k and v may have fewer heads, [B, Hkv, L, D] with Hkv dividing H
(grouped-query attention: query head h uses key/value head h // (H // Hkv)), and
k_mean then has Hkv heads too.

There is no fallback: if libssa.so is missing or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import math

import torch

from ._lib import SSA_BF16, SSA_F32, Dims, SSAError, check, load

__all__ = ["block_pool", "block_topk", "sparse_attn_fwd", "full_attn_fwd", "align_stats",
           "decode_append", "decode_sparse_fwd", "decode_full_fwd",
           "full_attn_bwd", "sparse_attn_bwd", "align_loss", "attn_stats",
           "set_kernel_variant", "SSAError", "lib", "abi_version"]


def lib():
    return load()


def abi_version() -> int:
    return int(load().ssa_abi_version())


def set_kernel_variant(variant: int) -> int:
    """0: MFMA kernels where they apply (default); 1: portable kernels only."""
    return int(load().ssa_set_kernel_variant(int(variant)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSA_BF16
    if t.dtype == torch.float32:
        return SSA_F32
    raise SSAError(3, f"unsupported tensor dtype {t.dtype}")


def _dims(x: torch.Tensor, block: int, hkv: int = 0) -> Dims:
    if x.dim() != 4:
        raise SSAError(2, "expected a [B, H, L, D] tensor")
    B, H, L, D = x.shape
    return Dims(B, H, L, D, int(block), _dtype_code(x), int(hkv))


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise SSAError(4, "tensors must be contiguous device tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _same(a: torch.Tensor, b: torch.Tensor, what: str):
    if a.shape != b.shape or a.dtype != b.dtype:
        raise SSAError(2, f"{what}: shape/dtype mismatch {tuple(a.shape)}/{a.dtype} vs {tuple(b.shape)}/{b.dtype}")


def _kv_heads(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor) -> int:
    """Key/value heads of k and v ([B, Hkv, L, D], Hkv dividing q's H)."""
    _same(k, v, "k/v")
    if (k.dim() != 4 or k.dtype != q.dtype or k.shape[0] != q.shape[0] or k.shape[2:] != q.shape[2:]
            or q.shape[1] % k.shape[1]):
        raise SSAError(2, f"k/v {tuple(k.shape)}/{k.dtype} do not fit q {tuple(q.shape)}/{q.dtype}")
    return int(k.shape[1])


def block_pool(k: torch.Tensor, block: int, out: torch.Tensor | None = None) -> torch.Tensor:
    d = _dims(k, block)
    if out is None:
        out = torch.empty((d.B, d.H, d.L // d.block, d.D), dtype=torch.float32, device=k.device)
    check(load().ssa_block_pool(ctypes.byref(d), _ptr(k), _ptr(out), _stream(k)))
    return out


def block_topk(q: torch.Tensor, k_mean: torch.Tensor, block: int, topk: int, want_scores: bool = False,
               out: torch.Tensor | None = None):
    d = _dims(q, block, k_mean.shape[1] if k_mean.dim() == 4 else 0)
    if out is None:
        out = torch.empty((d.B, d.H, d.L, topk), dtype=torch.int32, device=q.device)
    sel = torch.empty((d.B, d.H, d.L, topk), dtype=torch.float32, device=q.device) if want_scores else None
    check(load().ssa_block_topk(ctypes.byref(d), _ptr(q), _ptr(k_mean), int(topk), _ptr(out), _ptr(sel),
                                _stream(q)))
    return (out, sel) if want_scores else out


def sparse_attn_fwd(q, k, v, idx, block: int, scale: float | None = None, want_lse: bool = True,
                    out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    d = _dims(q, block, _kv_heads(q, k, v))
    if idx.dim() != 4 or tuple(idx.shape[:3]) != (d.B, d.H, d.L) or idx.dtype != torch.int32:
        raise SSAError(2, "idx must be int32 [B, H, L, topk]")
    topk = idx.shape[3]
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=q.device)
    check(load().ssa_sparse_attn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), int(topk),
                                     ctypes.c_float(scale), _ptr(out), _ptr(lse if want_lse else None),
                                     _stream(q)))
    return out, (lse if want_lse else None)


def full_attn_fwd(q, k, v, scale: float | None = None, want_o: bool = True, want_lse: bool = True,
                  block: int = 64, out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    d = _dims(q, block, _kv_heads(q, k, v))
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    if want_o and out is None:
        out = torch.empty_like(q)
    if want_lse and lse is None:
        lse = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=q.device)
    check(load().ssa_full_attn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), ctypes.c_float(scale),
                                   _ptr(out if want_o else None), _ptr(lse if want_lse else None),
                                   _stream(q)))
    return (out if want_o else None), (lse if want_lse else None)


def align_stats(o_full=None, o_sparse=None, lse_full=None, lse_sparse=None, block: int = 64,
                dims_like: torch.Tensor | None = None):
    """Per-token L2 distance (needs the o pair) and dropped mass (needs the lse pair)."""
    ref = o_full if o_full is not None else dims_like
    if ref is None:
        raise SSAError(1, "align_stats needs o_full or dims_like to know [B, H, L, D]")
    if o_full is not None:
        _same(o_full, o_sparse, "o_full/o_sparse")
    d = _dims(ref, block)
    dist = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=ref.device) if o_full is not None else None
    drop = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=ref.device) if lse_full is not None else None
    check(load().ssa_align_stats(ctypes.byref(d), _ptr(o_full), _ptr(o_sparse), _ptr(lse_full),
                                 _ptr(lse_sparse), _ptr(dist), _ptr(drop), _stream(ref)))
    return dist, drop


# ---------------------------------------------------------------- decoding
def _cache_dims(q_like: torch.Tensor, k_cache: torch.Tensor, block: int) -> Dims:
    """Dims of a decoding call: q_like is [B, H, D], k_cache [B, Hkv, L, D]."""
    if k_cache.dim() != 4 or q_like.dim() != 3:
        raise SSAError(2, "expected q [B, H, D] and a cache [B, Hkv, L, D]")
    B, Hkv, L, D = k_cache.shape
    if q_like.shape[0] != B or q_like.shape[2] != D or q_like.dtype != k_cache.dtype or q_like.shape[1] % Hkv:
        raise SSAError(2, f"q {tuple(q_like.shape)}/{q_like.dtype} does not fit the cache "
                          f"{tuple(k_cache.shape)}/{k_cache.dtype}")
    return Dims(B, q_like.shape[1], L, D, int(block), _dtype_code(k_cache), Hkv)


def _pos(pos: torch.Tensor, B: int) -> torch.Tensor:
    if pos.dtype != torch.int32 or pos.shape != (B,):
        raise SSAError(2, "pos must be an int32 [B] device tensor")
    return pos


def decode_append(pos, k_new, v_new, k_cache, v_cache, k_mean, block: int):
    """Write k_new, v_new ([B, Hkv, D]) at row pos[b] of the caches and refresh the pooled
    key of that row's block in k_mean ([B, Hkv, L // block, D] float32), in place."""
    d = _cache_dims(k_new, k_cache, block)
    _same(k_new, v_new, "k_new/v_new")
    _same(k_cache, v_cache, "k_cache/v_cache")
    check(load().ssa_decode_append(ctypes.byref(d), _ptr(_pos(pos, d.B)), _ptr(k_new), _ptr(v_new),
                                   _ptr(k_cache), _ptr(v_cache), _ptr(k_mean), _stream(k_cache)))


def decode_sparse_fwd(pos, q, k_cache, v_cache, k_mean, block: int, topk: int, scale: float | None = None,
                      want_lse: bool = True, want_idx: bool = True):
    """Selection and sparse attention for the query q[b, h] ([B, H, D]) at position pos[b].
    Returns (o [B, H, D], lse [B, H] or None, idx [B, H, topk] or None)."""
    d = _cache_dims(q, k_cache, block)
    _same(k_cache, v_cache, "k_cache/v_cache")
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    o = torch.empty_like(q)
    lse = torch.empty((d.B, d.H), dtype=torch.float32, device=q.device) if want_lse else None
    idx = torch.empty((d.B, d.H, int(topk)), dtype=torch.int32, device=q.device) if want_idx else None
    check(load().ssa_decode_sparse_fwd(ctypes.byref(d), _ptr(_pos(pos, d.B)), _ptr(q), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(k_mean), int(topk), ctypes.c_float(scale), _ptr(o),
                                       _ptr(lse), _ptr(idx), _stream(q)))
    return o, lse, idx


def decode_full_fwd(pos, q, k_cache, v_cache, scale: float | None = None, want_o: bool = True,
                    want_lse: bool = True, block: int = 64):
    """Dense attention for the query q[b, h] at position pos[b] over cache rows 0..pos[b].
    Returns (o [B, H, D] or None, lse [B, H] or None)."""
    d = _cache_dims(q, k_cache, block)
    if v_cache is not None:
        _same(k_cache, v_cache, "k_cache/v_cache")
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    o = torch.empty_like(q) if want_o else None
    lse = torch.empty((d.B, d.H), dtype=torch.float32, device=q.device) if want_lse else None
    check(load().ssa_decode_full_fwd(ctypes.byref(d), _ptr(_pos(pos, d.B)), _ptr(q), _ptr(k_cache),
                                     _ptr(v_cache), ctypes.c_float(scale), _ptr(o), _ptr(lse), _stream(q)))
    return o, lse


# ---------------------------------------------------------------- training
def _grad_bufs(q, k, dq, dk, dv):
    if dq is None:
        dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    for t, ref, what in ((dq, q, "dq"), (dk, k, "dk"), (dv, k, "dv")):
        if t.dtype != torch.float32 or t.shape != ref.shape:
            raise SSAError(2, f"{what} must be float32 of shape {tuple(ref.shape)}")
    return dq, dk, dv


def full_attn_bwd(q, k, v, o, lse, dout, dq=None, dk=None, dv=None, scale: float | None = None, block: int = 64):
    """Adds the full stream's gradients into dq, dk, dv (float32; zero-filled when not
    given) and returns them.  o, lse: the forward's outputs; dout: dL/do (q's dtype)."""
    d = _dims(q, block, _kv_heads(q, k, v))
    _same(o, q, "o/q")
    _same(dout, q, "dout/q")
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    dq, dk, dv = _grad_bufs(q, k, dq, dk, dv)
    check(load().ssa_full_attn_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                   ctypes.c_float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _stream(q)))
    return dq, dk, dv


def sparse_attn_bwd(q, k, v, o, lse, dout, idx, block: int, dq=None, dk=None, dv=None, scale: float | None = None):
    """Adds the sparse stream's gradients (kept blocks idx held fixed) into dq, dk, dv."""
    d = _dims(q, block, _kv_heads(q, k, v))
    _same(o, q, "o/q")
    _same(dout, q, "dout/q")
    if idx.dim() != 4 or tuple(idx.shape[:3]) != (d.B, d.H, d.L) or idx.dtype != torch.int32:
        raise SSAError(2, "idx must be int32 [B, H, L, topk]")
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    dq, dk, dv = _grad_bufs(q, k, dq, dk, dv)
    check(load().ssa_sparse_attn_bwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                     _ptr(idx), int(idx.shape[3]), ctypes.c_float(scale), _ptr(dq), _ptr(dk),
                                     _ptr(dv), _stream(q)))
    return dq, dk, dv


def align_loss(o_full, o_sparse, alpha: float, beta: float = 1.0, want_grads: bool = True):
    """Returns (loss [1] float32, dloss/do_full, dloss/do_sparse) of the bidirectional
    SmoothL1 alignment objective; the gradients are float32 tensors shaped like o."""
    _same(o_full, o_sparse, "o_full/o_sparse")
    d = _dims(o_full, 64)
    loss = torch.empty((1,), dtype=torch.float32, device=o_full.device)
    gf = torch.empty(o_full.shape, dtype=torch.float32, device=o_full.device) if want_grads else None
    gs = torch.empty(o_full.shape, dtype=torch.float32, device=o_full.device) if want_grads else None
    check(load().ssa_align_loss(ctypes.byref(d), _ptr(o_full), _ptr(o_sparse), ctypes.c_float(alpha),
                                ctypes.c_float(beta), _ptr(loss), _ptr(gf), _ptr(gs), _stream(o_full)))
    return loss, gf, gs


# ---------------------------------------------------------------- measurements
def attn_stats(q, k, lse, block: int, idx=None, scale: float | None = None, want_entropy: bool = True,
               want_hist: bool = True):
    """Row entropy [B, H, L] and attention mass by block distance [B, H, 16] of the full
    stream (idx None) or the sparse stream (its idx), given that stream's lse."""
    d = _dims(q, block, k.shape[1] if k.dim() == 4 else 0)
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    ent = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=q.device) if want_entropy else None
    hist = torch.empty((d.B, d.H, 16), dtype=torch.float32, device=q.device) if want_hist else None
    topk = int(idx.shape[3]) if idx is not None else 0
    check(load().ssa_attn_stats(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(lse), _ptr(idx), topk,
                                ctypes.c_float(scale), _ptr(ent), _ptr(hist), _stream(q)))
    return ent, hist
