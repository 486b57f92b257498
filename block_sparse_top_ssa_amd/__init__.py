"""SSA attention forward on MI355X: Python binding of libssa.

Argument marshalling only: every step of the computation runs in the HIP kernels of
libssa.so, called through its C ABI (include/ssa.h).  PyTorch provides device memory
and the stream: each call enqueues on torch's current stream and does not synchronise.

    k_mean = block_pool(k, block)
    idx = block_topk(q, k_mean, block, topk)
    o_s, lse_s = sparse_attn_fwd(q, k, v, idx, block)
    o_f, lse_f = full_attn_fwd(q, k, v)
    dist, dropped = align_stats(o_f, o_s, lse_f, lse_s)

With both streams over one k, v (bf16), their operand layouts can be written once into
buffers the caller owns, and the forwards then take no workspace:

    k_frag, v_frag = kv_frag(k, v, block)
    o_s, lse_s = sparse_attn_fwd_frag(q, k, v, k_frag, v_frag, idx, block)
    o_f, lse_f = full_attn_fwd_frag(q, k, v, v_frag)

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
           "kv_frag_bytes", "kv_frag", "sparse_attn_fwd_frag", "full_attn_fwd_frag",
           "full_attn_fwd_stats", "sparse_attn_fwd_stats",
           "decode_append", "decode_sparse_fwd", "decode_sparse_fwd_noalloc", "decode_full_fwd",
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


def _expect(t, shape, dtype, device, what):
    """The C ABI cannot see buffer sizes, so every tensor passed down is checked here:
    shape, dtype, device and contiguity, before any launch."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise SSAError(1, f"{what} must be a tensor")
    if t.dtype != dtype:
        raise SSAError(3, f"{what} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(int(x) for x in shape):
        raise SSAError(2, f"{what} must have shape {tuple(int(x) for x in shape)} (got {tuple(t.shape)})")
    if t.device != device:
        raise SSAError(4, f"{what} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise SSAError(4, f"{what} must be contiguous")
    return t


def _kmean_shape(d: Dims):
    return (d.B, d.Hkv or d.H, d.L // d.block, d.D)


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
    _expect(out, (d.B, d.H, d.L // d.block, d.D), torch.float32, k.device, "block_pool out")
    check(load().ssa_block_pool(ctypes.byref(d), _ptr(k), _ptr(out), _stream(k)))
    return out


def block_topk(q: torch.Tensor, k_mean: torch.Tensor, block: int, topk: int, want_scores: bool = False,
               out: torch.Tensor | None = None):
    if not isinstance(k_mean, torch.Tensor) or k_mean.dim() != 4 or k_mean.shape[1] < 1 or q.dim() != 4 \
            or q.shape[1] % k_mean.shape[1]:
        raise SSAError(2, "k_mean must be float32 [B, Hkv, L // block, D] with Hkv dividing q's heads")
    d = _dims(q, block, k_mean.shape[1])
    _expect(k_mean, _kmean_shape(d), torch.float32, q.device, "k_mean")
    if out is None:
        out = torch.empty((d.B, d.H, d.L, topk), dtype=torch.int32, device=q.device)
    _expect(out, (d.B, d.H, d.L, topk), torch.int32, q.device, "block_topk out")
    sel = torch.empty((d.B, d.H, d.L, topk), dtype=torch.float32, device=q.device) if want_scores else None
    check(load().ssa_block_topk(ctypes.byref(d), _ptr(q), _ptr(k_mean), int(topk), _ptr(out), _ptr(sel),
                                _stream(q)))
    return (out, sel) if want_scores else out


def _sparse_args(q, k, v, idx, block, scale, want_lse, out, lse):
    d = _dims(q, block, _kv_heads(q, k, v))
    if idx.dim() != 4 or tuple(idx.shape[:3]) != (d.B, d.H, d.L) or idx.dtype != torch.int32:
        raise SSAError(2, "idx must be int32 [B, H, L, topk]")
    _expect(idx, idx.shape, torch.int32, q.device, "idx")
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, q.shape, q.dtype, q.device, "sparse_attn_fwd out")
    if want_lse and lse is None:
        lse = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=q.device)
    if want_lse:
        _expect(lse, (d.B, d.H, d.L), torch.float32, q.device, "sparse_attn_fwd lse")
    return d, scale, out, (lse if want_lse else None)


def sparse_attn_fwd(q, k, v, idx, block: int, scale: float | None = None, want_lse: bool = True,
                    out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    d, scale, out, lse = _sparse_args(q, k, v, idx, block, scale, want_lse, out, lse)
    check(load().ssa_sparse_attn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), int(idx.shape[3]),
                                     ctypes.c_float(scale), _ptr(out), _ptr(lse), _stream(q)))
    return out, lse


def _full_args(q, k, v, block, scale, want_o, want_lse, out, lse, what="full_attn_fwd"):
    d = _dims(q, block, _kv_heads(q, k, v))
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    if want_o and out is None:
        out = torch.empty_like(q)
    if want_o:
        _expect(out, q.shape, q.dtype, q.device, f"{what} out")
    if want_lse and lse is None:
        lse = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=q.device)
    if want_lse:
        _expect(lse, (d.B, d.H, d.L), torch.float32, q.device, f"{what} lse")
    return d, scale, (out if want_o else None), (lse if want_lse else None)


def full_attn_fwd(q, k, v, scale: float | None = None, want_o: bool = True, want_lse: bool = True,
                  block: int = 64, out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    d, scale, out, lse = _full_args(q, k, v, block, scale, want_o, want_lse, out, lse)
    check(load().ssa_full_attn_fwd(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), ctypes.c_float(scale),
                                   _ptr(out), _ptr(lse), _stream(q)))
    return out, lse


def kv_frag_bytes(k: torch.Tensor, block: int = 64) -> int:
    """Bytes of one fragment-order copy of k or v ([B, Hkv, L, D]); 0 for float32."""
    d = _dims(k, block)
    n = ctypes.c_int64(0)
    check(load().ssa_kv_frag_bytes(ctypes.byref(d), ctypes.byref(n)))
    return int(n.value)


def _frag_buf(t, nbytes, device, what):
    if t is None:
        return None
    return _expect(t, (nbytes,), torch.uint8, device, what)


def kv_frag(k: torch.Tensor, v: torch.Tensor, block: int = 64, want_k: bool = True, want_v: bool = True,
            k_frag: torch.Tensor | None = None, v_frag: torch.Tensor | None = None):
    """k and v (bf16 [B, Hkv, L, D]) written once in the layouts the matrix-core forwards
    read, into uint8 buffers of kv_frag_bytes(k) each: (k_frag, v_frag), None where not
    asked for.  Pass them to sparse_attn_fwd_frag / full_attn_fwd_frag with the same k, v."""
    _same(k, v, "k/v")
    d = _dims(k, block)
    nbytes = kv_frag_bytes(k, block)
    if want_k and k_frag is None:
        k_frag = torch.empty(nbytes, dtype=torch.uint8, device=k.device)
    if want_v and v_frag is None:
        v_frag = torch.empty(nbytes, dtype=torch.uint8, device=k.device)
    kf = _frag_buf(k_frag if want_k else None, nbytes, k.device, "k_frag")
    vf = _frag_buf(v_frag if want_v else None, nbytes, k.device, "v_frag")
    check(load().ssa_kv_frag(ctypes.byref(d), _ptr(k), _ptr(v), _ptr(kf), _ptr(vf), _stream(k)))
    return kf, vf


def sparse_attn_fwd_frag(q, k, v, k_frag, v_frag, idx, block: int, scale: float | None = None,
                         want_lse: bool = True, out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """sparse_attn_fwd with the copies kv_frag wrote from the same k, v (no workspace)."""
    d, scale, out, lse = _sparse_args(q, k, v, idx, block, scale, want_lse, out, lse)
    nbytes = kv_frag_bytes(k, block)
    kf = _frag_buf(k_frag, nbytes, q.device, "k_frag")
    vf = _frag_buf(v_frag, nbytes, q.device, "v_frag")
    check(load().ssa_sparse_attn_fwd_frag(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(kf), _ptr(vf), _ptr(idx),
                                          int(idx.shape[3]), ctypes.c_float(scale), _ptr(out), _ptr(lse),
                                          _stream(q)))
    return out, lse


def full_attn_fwd_frag(q, k, v, v_frag, scale: float | None = None, want_o: bool = True, want_lse: bool = True,
                       block: int = 64, out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """full_attn_fwd with the copy of v kv_frag wrote (no workspace)."""
    d, scale, out, lse = _full_args(q, k, v, block, scale, want_o, want_lse, out, lse, "full_attn_fwd_frag")
    vf = _frag_buf(v_frag, kv_frag_bytes(k, block), q.device, "v_frag")
    check(load().ssa_full_attn_fwd_frag(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(vf), ctypes.c_float(scale),
                                        _ptr(out), _ptr(lse), _stream(q)))
    return out, lse


def _stats_outs(d: Dims, device, want_entropy, want_hist, entropy, hist, what):
    """The measurement outputs: entropy [B, H, L] and hist [B, H, 16] in float32, the given
    ones checked, the others allocated; None where not wanted."""
    if not want_entropy:
        entropy = None
    elif entropy is None:
        entropy = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=device)
    else:
        _expect(entropy, (d.B, d.H, d.L), torch.float32, device, what + " entropy")
    if not want_hist:
        hist = None
    elif hist is None:
        hist = torch.empty((d.B, d.H, 16), dtype=torch.float32, device=device)
    else:
        _expect(hist, (d.B, d.H, 16), torch.float32, device, what + " hist")
    return entropy, hist


def full_attn_fwd_stats(q, k, v, scale: float | None = None, want_o: bool = True, want_lse: bool = True,
                        want_entropy: bool = True, want_hist: bool = True, block: int = 64,
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                        entropy: torch.Tensor | None = None, hist: torch.Tensor | None = None):
    """full_attn_fwd with the full stream's row entropy [B, H, L] and attention mass by
    block distance [B, H, 16] from the same sweep: (o, lse, entropy, hist).  Every output
    may be given (float32 for lse, entropy and hist), else it is allocated."""
    d = _dims(q, block, _kv_heads(q, k, v))
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    if want_o and out is None:
        out = torch.empty_like(q)
    if want_o:
        _expect(out, q.shape, q.dtype, q.device, "full_attn_fwd_stats out")
    if want_lse and lse is None:
        lse = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=q.device)
    if want_lse:
        _expect(lse, (d.B, d.H, d.L), torch.float32, q.device, "full_attn_fwd_stats lse")
    ent, hist = _stats_outs(d, q.device, want_entropy, want_hist, entropy, hist, "full_attn_fwd_stats")
    check(load().ssa_full_attn_fwd_stats(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), ctypes.c_float(scale),
                                         _ptr(out if want_o else None), _ptr(lse if want_lse else None),
                                         _ptr(ent), _ptr(hist), _stream(q)))
    return (out if want_o else None), (lse if want_lse else None), ent, hist


def sparse_attn_fwd_stats(q, k, v, idx, block: int, scale: float | None = None, want_lse: bool = True,
                          want_entropy: bool = True, want_hist: bool = True, out: torch.Tensor | None = None,
                          lse: torch.Tensor | None = None, entropy: torch.Tensor | None = None,
                          hist: torch.Tensor | None = None):
    """sparse_attn_fwd with the sparse stream's row entropy [B, H, L] and attention mass by
    block distance [B, H, 16] from the same sweep: (o, lse, entropy, hist).  Every output
    may be given (float32 for lse, entropy and hist), else it is allocated."""
    d, scale, out, lse = _sparse_args(q, k, v, idx, block, scale, want_lse, out, lse)
    ent, hist = _stats_outs(d, q.device, want_entropy, want_hist, entropy, hist, "sparse_attn_fwd_stats")
    check(load().ssa_sparse_attn_fwd_stats(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(idx), int(idx.shape[3]),
                                           ctypes.c_float(scale), _ptr(out), _ptr(lse), _ptr(ent), _ptr(hist),
                                           _stream(q)))
    return out, lse, ent, hist


def align_stats(o_full=None, o_sparse=None, lse_full=None, lse_sparse=None, block: int = 64,
                dims_like: torch.Tensor | None = None, want_retained_hist: bool = False):
    """Per-token L2 distance (needs the o pair) and dropped mass (needs the lse pair); with
    want_retained_hist also the per-head histogram [B, H, 16] of the retained mass
    1 - dropped (counts of rows per sixteenth), returned third."""
    ref = o_full if o_full is not None else dims_like
    if ref is None:
        raise SSAError(1, "align_stats needs o_full or dims_like to know [B, H, L, D]")
    if o_full is not None:
        if o_sparse is None:
            raise SSAError(1, "align_stats needs both o_full and o_sparse")
        _same(o_full, o_sparse, "o_full/o_sparse")
        if o_sparse.device != o_full.device:
            raise SSAError(4, "o_full and o_sparse are on different devices")
    d = _dims(ref, block)
    if (lse_full is None) != (lse_sparse is None):
        raise SSAError(1, "align_stats needs both lse_full and lse_sparse")
    _expect(lse_full, (d.B, d.H, d.L), torch.float32, ref.device, "lse_full")
    _expect(lse_sparse, (d.B, d.H, d.L), torch.float32, ref.device, "lse_sparse")
    dist = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=ref.device) if o_full is not None else None
    drop = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=ref.device) if lse_full is not None else None
    if not want_retained_hist:
        check(load().ssa_align_stats(ctypes.byref(d), _ptr(o_full), _ptr(o_sparse), _ptr(lse_full),
                                     _ptr(lse_sparse), _ptr(dist), _ptr(drop), _stream(ref)))
        return dist, drop
    if lse_full is None:
        raise SSAError(1, "the retained-mass histogram needs lse_full and lse_sparse")
    rh = torch.empty((d.B, d.H, 16), dtype=torch.float32, device=ref.device)
    check(load().ssa_align_stats_hist(ctypes.byref(d), _ptr(o_full), _ptr(o_sparse), _ptr(lse_full),
                                      _ptr(lse_sparse), _ptr(dist), _ptr(drop), _ptr(rh), _stream(ref)))
    return dist, drop, rh


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


def _pos(pos: torch.Tensor, B: int, device) -> torch.Tensor:
    if not isinstance(pos, torch.Tensor) or pos.dtype != torch.int32 or pos.shape != (B,):
        raise SSAError(2, "pos must be an int32 [B] device tensor")
    return _expect(pos, (B,), torch.int32, device, "pos")


def _decode_operands(d: Dims, q, k_cache, v_cache, k_mean):
    """Checks the caches (same shape and dtype), k_mean ([B, Hkv, L // block, D] float32)
    and that everything sits on q's device."""
    if v_cache is not None:
        _same(k_cache, v_cache, "k_cache/v_cache")
        _expect(v_cache, k_cache.shape, k_cache.dtype, q.device, "v_cache")
    _expect(k_cache, k_cache.shape, k_cache.dtype, q.device, "k_cache")
    if k_mean is not None:
        _expect(k_mean, _kmean_shape(d), torch.float32, q.device, "k_mean")


def decode_append(pos, k_new, v_new, k_cache, v_cache, k_mean, block: int):
    """Write k_new, v_new ([B, Hkv, D]) at row pos[b] of the caches and refresh the pooled
    key of that row's block in k_mean ([B, Hkv, L // block, D] float32), in place."""
    d = _cache_dims(k_new, k_cache, block)
    _same(k_new, v_new, "k_new/v_new")
    if d.H != d.Hkv:
        raise SSAError(2, "k_new and v_new must have the cache's key/value heads [B, Hkv, D]")
    _expect(v_new, k_new.shape, k_new.dtype, k_new.device, "v_new")
    _decode_operands(d, k_new, k_cache, v_cache, k_mean)
    check(load().ssa_decode_append(ctypes.byref(d), _ptr(_pos(pos, d.B, k_new.device)), _ptr(k_new), _ptr(v_new),
                                   _ptr(k_cache), _ptr(v_cache), _ptr(k_mean), _stream(k_cache)))


def decode_sparse_fwd(pos, q, k_cache, v_cache, k_mean, block: int, topk: int, scale: float | None = None,
                      want_lse: bool = True, want_idx: bool = True):
    """Selection and sparse attention for the query q[b, h] ([B, H, D]) at position pos[b].
    Returns (o [B, H, D], lse [B, H] or None, idx [B, H, topk] or None)."""
    return _decode_sparse("ssa_decode_sparse_fwd", pos, q, k_cache, v_cache, k_mean, block, topk, scale,
                          want_lse, want_idx, None, None, None)


def decode_sparse_fwd_noalloc(pos, q, k_cache, v_cache, k_mean, block: int, topk: int, scale: float | None = None,
                              out=None, lse=None, idx=None, want_lse: bool = True, want_idx: bool = True):
    """decode_sparse_fwd through the library entry point that allocates nothing (its
    scratch is a fixed 16 MiB device array; calls overlapping on one device race).  Pass
    out ([B, H, D]), lse ([B, H] float32) and idx ([B, H, topk] int32) to allocate nothing
    here either; the ones left None are created."""
    return _decode_sparse("ssa_decode_sparse_fwd_noalloc", pos, q, k_cache, v_cache, k_mean, block, topk, scale,
                          want_lse, want_idx, out, lse, idx)


def _decode_sparse(entry, pos, q, k_cache, v_cache, k_mean, block, topk, scale, want_lse, want_idx, o, lse, idx):
    d = _cache_dims(q, k_cache, block)
    _decode_operands(d, q, k_cache, v_cache, k_mean)
    if k_mean is None or v_cache is None:
        raise SSAError(1, "decode_sparse_fwd needs v_cache and k_mean")
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    if o is None:
        o = torch.empty_like(q)
    _expect(o, q.shape, q.dtype, q.device, "o")
    if want_lse and lse is None:
        lse = torch.empty((d.B, d.H), dtype=torch.float32, device=q.device)
    if not want_lse:
        lse = None
    _expect(lse, (d.B, d.H), torch.float32, q.device, "lse")
    if want_idx and idx is None:
        idx = torch.empty((d.B, d.H, int(topk)), dtype=torch.int32, device=q.device)
    if not want_idx:
        idx = None
    _expect(idx, (d.B, d.H, int(topk)), torch.int32, q.device, "idx")
    check(getattr(load(), entry)(ctypes.byref(d), _ptr(_pos(pos, d.B, q.device)), _ptr(q), _ptr(k_cache),
                                 _ptr(v_cache), _ptr(k_mean), int(topk), ctypes.c_float(scale), _ptr(o),
                                 _ptr(lse), _ptr(idx), _stream(q)))
    return o, lse, idx


def decode_full_fwd(pos, q, k_cache, v_cache, scale: float | None = None, want_o: bool = True,
                    want_lse: bool = True, block: int = 64):
    """Dense attention for the query q[b, h] at position pos[b] over cache rows 0..pos[b].
    Returns (o [B, H, D] or None, lse [B, H] or None)."""
    d = _cache_dims(q, k_cache, block)
    _decode_operands(d, q, k_cache, v_cache, None)
    if want_o and v_cache is None:
        raise SSAError(1, "decode_full_fwd needs v_cache for o")
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    o = torch.empty_like(q) if want_o else None
    lse = torch.empty((d.B, d.H), dtype=torch.float32, device=q.device) if want_lse else None
    check(load().ssa_decode_full_fwd(ctypes.byref(d), _ptr(_pos(pos, d.B, q.device)), _ptr(q), _ptr(k_cache),
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
        _expect(t, ref.shape, torch.float32, q.device, what)
    return dq, dk, dv


def _bwd_operands(d: Dims, q, k, v, o, lse, dout):
    for t, what in ((k, "k"), (v, "v")):
        _expect(t, k.shape, q.dtype, q.device, what)
    for t, what in ((o, "o"), (dout, "dout")):
        _expect(t, q.shape, q.dtype, q.device, what)
    _expect(lse, (d.B, d.H, d.L), torch.float32, q.device, "lse")


def full_attn_bwd(q, k, v, o, lse, dout, dq=None, dk=None, dv=None, scale: float | None = None, block: int = 64):
    """Adds the full stream's gradients into dq, dk, dv (float32; zero-filled when not
    given) and returns them.  o, lse: the forward's outputs; dout: dL/do (q's dtype)."""
    d = _dims(q, block, _kv_heads(q, k, v))
    _same(o, q, "o/q")
    _same(dout, q, "dout/q")
    _bwd_operands(d, q, k, v, o, lse, dout)
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
    _expect(idx, idx.shape, torch.int32, q.device, "idx")
    _bwd_operands(d, q, k, v, o, lse, dout)
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
    _expect(o_sparse, o_full.shape, o_full.dtype, o_full.device, "o_sparse")
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
    if not isinstance(k, torch.Tensor) or k.dim() != 4 or q.dim() != 4 or k.shape[1] < 1 or q.shape[1] % k.shape[1]:
        raise SSAError(2, "k must be [B, Hkv, L, D] with Hkv dividing q's heads")
    d = _dims(q, block, k.shape[1])
    _expect(k, (d.B, k.shape[1], d.L, d.D), q.dtype, q.device, "k")
    _expect(lse, (d.B, d.H, d.L), torch.float32, q.device, "lse")
    if idx is not None:
        if idx.dim() != 4:
            raise SSAError(2, "idx must be int32 [B, H, L, topk]")
        _expect(idx, (d.B, d.H, d.L, idx.shape[3]), torch.int32, q.device, "idx")
    scale = 1.0 / math.sqrt(d.D) if scale is None else float(scale)
    ent = torch.empty((d.B, d.H, d.L), dtype=torch.float32, device=q.device) if want_entropy else None
    hist = torch.empty((d.B, d.H, 16), dtype=torch.float32, device=q.device) if want_hist else None
    topk = int(idx.shape[3]) if idx is not None else 0
    check(load().ssa_attn_stats(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(lse), _ptr(idx), topk,
                                ctypes.c_float(scale), _ptr(ent), _ptr(hist), _stream(q)))
    return ent, hist
