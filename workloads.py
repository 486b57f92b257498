"""Seeded synthetic inputs for the SSA attention forward, shared by the GPU path's
tests/bench and by the CPU oracle.

This module holds no attention arithmetic.  It only draws random numbers, adds the
structure each workload asks for to the keys (a per-head low-rank block bias, an
attention-sink key, a smooth positional drift), and rounds float32 draws to bfloat16
bit patterns (round to nearest, ties to even) so that both sides see the same bits.

Workloads (shapes follow the long-context settings of Shen et al., "SSA: Sparse Sparse
Attention by Aligning Full and Sparse Attention Outputs in Feature Space": 8k
pretraining and 32k continued training (sec. 6), receptive fields of k*s tokens
(sec. 3), sparsity-budget extrapolation (Table 1 / Fig. 3), 128k inference speed
(App. D, Table A3) and attention sinks (abstract)).  No dataset or trained weight is
used: every tensor is drawn here.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

BF16 = "bf16"
F32 = "f32"


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    L: int
    D: int
    s: int                      # block size (tokens per block)
    ks: tuple                   # blocks kept per query (one run per value)
    dtype: str                  # "bf16" or "f32" element type of q, k, v, o
    structure: str              # "scaled", "lowrank", "sink", "none", "sink_drift"
    seed: int
    sample_rows: int = 0        # rows per (b, h) the oracle checks for O / lse / stats; 0 = all
    sparse_only: bool = False   # full stream computed as LSE only (dropped mass)
    Hkv: int = 0                # key/value heads (0: as many as query heads)

    @property
    def n(self) -> int:
        return self.L // self.s

    @property
    def hkv(self) -> int:
        return self.Hkv or self.H

    @property
    def group(self) -> int:
        """Query heads per key/value head (query head h reads key/value head h // group)."""
        return self.H // self.hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


WORKLOADS = {
    w.name: w for w in [
        # fp32 correctness case: q, k, v ~ N(0,1) multiplied by 1/sqrt(64).
        Workload("fp32_L1024_D64", 1, 4, 1024, 64, 64, (4,), F32, "scaled", 1001),
        # bf16, per-head rank-4 key bias constant within each block.
        Workload("bf16_L4096_lowrank", 4, 16, 4096, 128, 64, (16,), BF16, "lowrank", 1002),
        # bf16 long context with an 8x-norm sink key at token 0 (receptive field 2048).
        Workload("bf16_L32768_sink", 1, 32, 32768, 128, 64, (32,), BF16, "sink", 1003,
                 sample_rows=512),
        # bf16 sparsity-budget sweep on one set of inputs; k = 128 = n equals full.
        Workload("bf16_L8192_ksweep", 2, 16, 8192, 128, 64, (4, 8, 16, 32, 64, 128), BF16,
                 "none", 1004, sample_rows=512),
        # bf16 extrapolation-length stress: sink plus smooth key drift; sparse stream
        # plus dropped-mass statistics (full stream as LSE only).
        Workload("bf16_L131072_drift", 1, 8, 131072, 128, 128, (64,), BF16, "sink_drift",
                 1005, sample_rows=256, sparse_only=True),
        # bf16_L32768_sink's shape with two key/value heads shared by 16 query heads each
        # (grouped-query attention, the paper's training setup).
        Workload("bf16_L32768_gqa2", 1, 32, 32768, 128, 64, (32,), BF16, "sink", 1006,
                 sample_rows=512, Hkv=2),
    ]
}

# The workload the throughput figure is quoted on (L = 32K).
BENCH_WORKLOAD = "bf16_L32768_sink"


# ----------------------------------------------------------------------------------
# bfloat16 bit patterns
# ----------------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even, returned as uint16 bit patterns.

    Inputs are finite (no NaN policy is needed for drawn normals)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------------
# generation
# ----------------------------------------------------------------------------------
@dataclass
class Inputs:
    """q, k, v in the element type the GPU path receives.

    For bf16 workloads the arrays are uint16 bit patterns; for fp32 they are float32.
    `as_f64(name)` gives the exact values the oracle works on."""
    workload: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    extras: dict = field(default_factory=dict)

    def as_f32(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        if self.workload.dtype == BF16:
            return bf16_bits_to_f32(a)
        return a

    def as_f64(self, name: str) -> np.ndarray:
        return self.as_f32(name).astype(np.float64)

    def kv_per_query_head(self, a: np.ndarray) -> np.ndarray:
        """A [B, Hkv, ...] key/value-side array repeated to one slice per query head
        (query head h reads key/value head h // group)."""
        g = self.workload.group
        return a if g == 1 else np.repeat(a, g, axis=1)


def _draw(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def make_qkv(B, H, L, D, s, dtype=BF16, structure="none", seed=0, q_zero=False,
             heads=None, hkv=0) -> Inputs:
    """Draw q of shape [B, H, L, D] and k, v of shape [B, Hkv, L, D] (Hkv = hkv or H;
    q, k, v in that order from one generator seeded with `seed`), add the key
    structure, and round to the element type.

    structure:
      "none"       q, k, v ~ N(0, 1)
      "scaled"     q, k, v ~ N(0, 1) multiplied by 1/sqrt(64)
      "lowrank"    k[b,h,t] += A_h z_{b,h,t//s}, A_h in R^{D x 4} ~ N(0, 1/4),
                   z ~ N(0, I_4) per block (drawn after v: A then z)
      "sink"       k[:, :, 0, :] *= 8
      "sink_drift" k[b,h,t,d] += 0.5 sin(2 pi t / P_d + phi_{h,d}), P_d log-spaced
                   from 1024 to 131072 over d, phi ~ U[0, 2 pi) (drawn after v);
                   then k[:, :, 0, :] *= 8
    heads: optional subset of head indices to keep (the draw is still of the whole
    tensor, so a subset has the same values as in the full draw); only with Hkv = H.
    The key structure's per-head terms are per key/value head.
    """
    rng = np.random.default_rng(seed)
    Hk = hkv or H
    if H % Hk or (heads is not None and Hk != H):
        raise ValueError("hkv must divide H, and a head subset needs hkv = H")
    q = _draw(rng, (B, H, L, D))
    k = _draw(rng, (B, Hk, L, D))
    v = _draw(rng, (B, Hk, L, D))
    if structure == "scaled":
        f = np.float32(1.0 / 8.0)
        q *= f
        k *= f
        v *= f
    elif structure == "lowrank":
        A = rng.standard_normal((Hk, D, 4), dtype=np.float32) * np.float32(0.5)
        z = rng.standard_normal((B, Hk, L // s, 4), dtype=np.float32)
        bias = np.einsum("hdr,bhjr->bhjd", A, z).astype(np.float32)   # [B,H,n,D]
        k += np.repeat(bias, s, axis=2)
    elif structure == "sink":
        k[:, :, 0, :] *= np.float32(8.0)
    elif structure == "sink_drift":
        periods = np.geomspace(1024.0, 131072.0, D)
        phi = rng.uniform(0.0, 2.0 * np.pi, size=(Hk, D))
        t = np.arange(L, dtype=np.float64)[:, None]
        for h in range(Hk):
            drift = (0.5 * np.sin(2.0 * np.pi * t / periods[None, :] + phi[h][None, :]))
            k[:, h] += drift.astype(np.float32)[None]
        k[:, :, 0, :] *= np.float32(8.0)
    elif structure != "none":
        raise ValueError(f"unknown structure {structure!r}")
    if q_zero:
        q[...] = 0.0
    if heads is not None:
        q, k, v = (np.ascontiguousarray(a[:, heads]) for a in (q, k, v))
    if dtype == BF16:
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    wl = Workload("adhoc", B, H if heads is None else len(heads), L, D, s, (), dtype,
                  structure, seed, Hkv=0 if Hk == H else Hk)
    return Inputs(wl, q, k, v)


def make_workload(name: str, heads=None) -> Inputs:
    w = WORKLOADS[name]
    inp = make_qkv(w.B, w.H, w.L, w.D, w.s, w.dtype, w.structure, w.seed, heads=heads, hkv=w.Hkv)
    inp.workload = w
    return inp


def integer_tensor(shape, lo, hi, seed, dtype=np.float32) -> np.ndarray:
    """Integer-valued tensor in [lo, hi] (exact in bf16 for |values| <= 256)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape).astype(dtype)


def sample_rows(L: int, s: int, k: int, count: int, seed: int) -> np.ndarray:
    """Seeded, sorted sample of query rows that always includes the edge rows
    0, s-1, s, k*s-1, k*s, (k+1)*s-1, (k+1)*s, L-1 and the last row of every 16th block."""
    if count <= 0 or count >= L:
        return np.arange(L)
    rng = np.random.default_rng(seed)
    must = {0, s - 1, s, k * s - 1, k * s, (k + 1) * s - 1, (k + 1) * s, L - 1}
    must |= {j * s + s - 1 for j in range(0, L // s, 16)}
    must = {r for r in must if 0 <= r < L}
    rest = rng.choice(L, size=max(0, count - len(must)), replace=False)
    return np.array(sorted(must | set(int(r) for r in rest)), dtype=np.int64)


# ----------------------------------------------------------------------------------
# decoding with a key/value cache
# ----------------------------------------------------------------------------------
@dataclass(frozen=True)
class DecodeWorkload:
    """One decoding step for B sequences at different positions of a cache of capacity L:
    the cache holds k, v for every row (rows after a sequence's position are never read
    by decoding), the queries are [B, H, D], positions are drawn in [L/2, L)."""
    name: str
    B: int
    H: int
    L: int
    D: int
    s: int
    k: int
    dtype: str
    structure: str
    seed: int
    Hkv: int = 0

    @property
    def n(self) -> int:
        return self.L // self.s

    @property
    def hkv(self) -> int:
        return self.Hkv or self.H

    @property
    def group(self) -> int:
        return self.H // self.hkv


DECODE_WORKLOADS = {
    w.name: w for w in [
        # bf16_L32768_sink's head shape, four sequences decoding at once.
        DecodeWorkload("bf16_L32768_decode", 4, 32, 32768, 128, 64, 32, BF16, "sink", 1007),
        # the same with two key/value heads (the paper's model, App. C): 16 query heads per
        # cached key/value head.
        DecodeWorkload("bf16_L32768_decode_gqa2", 4, 32, 32768, 128, 64, 32, BF16, "sink", 1008, Hkv=2),
    ]
}


@dataclass
class DecodeInputs:
    workload: DecodeWorkload
    k: np.ndarray      # [B, Hkv, L, D] cache
    v: np.ndarray      # [B, Hkv, L, D] cache
    q: np.ndarray      # [B, H, D] queries at pos
    pos: np.ndarray    # [B] int32

    def as_f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return (bf16_bits_to_f32(a) if self.workload.dtype == BF16 else a).astype(np.float64)


def make_decode(name: str) -> DecodeInputs:
    """Draw k, v (the cache), then q, then the positions, from one generator; the sink
    structure scales token 0's key by 8 as in the prefill workloads."""
    w = DECODE_WORKLOADS[name]
    rng = np.random.default_rng(w.seed)
    Hk = w.hkv
    k = _draw(rng, (w.B, Hk, w.L, w.D))
    v = _draw(rng, (w.B, Hk, w.L, w.D))
    q = _draw(rng, (w.B, w.H, w.D))
    pos = rng.integers(w.L // 2, w.L, size=w.B).astype(np.int32)
    if w.structure == "sink":
        k[:, :, 0, :] *= np.float32(8.0)
    elif w.structure != "none":
        raise ValueError(f"unknown structure {w.structure!r}")
    if w.dtype == BF16:
        k, v, q = f32_to_bf16_bits(k), f32_to_bf16_bits(v), f32_to_bf16_bits(q)
    return DecodeInputs(w, k, v, q, pos)
