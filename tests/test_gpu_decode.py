"""GPU parity of the decoding calls (key/value cache, one query per sequence) against the
CPU oracle's decode_step and open_block_mean.  Needs an MI355X.

Same rules as the whole-sequence tests (tests/parity.py): the kept blocks bit-exact
except at score ties within 1e-5 relative, outputs within 2e-2 (bf16) / 1e-4 (fp32).
The sparse output is checked against the oracle run on the GPU's own selection.
"""
import math
import sys

import numpy as np
import pytest

import workloads as W
from parity import TIE_REL, TOL, assert_close, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import block_sparse_top_ssa_amd as ssa  # noqa: E402
import oracle.ssa_oracle as O  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _f64(a, dtype):
    return (W.bf16_bits_to_f32(a) if dtype == W.BF16 else a).astype(np.float64)


def check_idx_row(g, r, q64, k64, t, s, topk, where):
    """GPU selection row g against the oracle's decode_step result r (tie-aware)."""
    bt = t // s
    m = min(topk - 1, bt)
    g = [int(x) for x in g]
    assert g[m] == bt and all(x == -1 for x in g[m + 1:]), f"{where}: malformed row {g}"
    assert g[:m] == sorted(set(g[:m])) and all(0 <= x < bt for x in g[:m]), f"{where}: bad entries {g}"
    o = r["idx"].tolist()
    if g == o:
        return 0
    sm, sm1 = r["sigma_m"], r["sigma_m1"]
    band = TIE_REL * max(abs(sm), abs(sm1))
    assert abs(sm - sm1) < band, f"{where}: selection differs outside a tie\n gpu={g}\n oracle={o}"
    kbar = k64[:bt * s].reshape(bt, s, -1).mean(axis=1)
    for j in set(g[:m]) ^ set(o[:m]):
        sj = float(kbar[j] @ q64)
        assert sm1 - band <= sj <= sm + band, f"{where}: block {j} outside the tied band"
    return 1


def run_and_check(k, v, q, pos, s, topk, dtype, Hkv, tag="", km=None):
    """k, v: [B, Hkv, L, D] caches (element type bits), q: [B, H, D], pos: [B].
    Runs pool (unless km is given), decode_sparse_fwd, decode_full_fwd and align_stats
    on the GPU and checks every (b, h) against the oracle."""
    B, H, D = q.shape
    L = k.shape[2]
    G = H // Hkv
    scale = 1.0 / math.sqrt(D)
    say(f"[gpu] decode {tag} B={B} H={H} Hkv={Hkv} L={L} D={D} s={s} topk={topk} {dtype} pos={list(pos)}")
    kd, vd, qd = to_device(k, dtype), to_device(v, dtype), to_device(q, dtype)
    posd = torch.from_numpy(np.asarray(pos, dtype=np.int32)).cuda()
    kmd = ssa.block_pool(kd, s) if km is None else km
    o_s, lse_s, idx = ssa.decode_sparse_fwd(posd, qd, kd, vd, kmd, s, topk, scale)
    o_f, lse_f = ssa.decode_full_fwd(posd, qd, kd, vd, scale, block=s)
    dist, drop = ssa.align_stats(o_f.unsqueeze(2), o_s.unsqueeze(2), lse_f.unsqueeze(2), lse_s.unsqueeze(2),
                                 block=s)
    torch.cuda.synchronize()
    g = dict(o_s=to_f64(o_s), lse_s=to_f64(lse_s), idx=idx.cpu().numpy(), o_f=to_f64(o_f),
             lse_f=to_f64(lse_f), dist=to_f64(dist)[:, :, 0], drop=to_f64(drop)[:, :, 0])
    q64 = _f64(q, dtype)
    tol = TOL[dtype]
    err = {"o_s": 0.0, "lse_s": 0.0, "o_f": 0.0, "lse_f": 0.0}
    tied = 0
    for b in range(B):
        t = int(pos[b])
        for kh in range(Hkv):
            # the cache rows 0..t of this key/value head, as the oracle's float64 values
            k64, v64 = _f64(k[b, kh, :t + 1], dtype), _f64(v[b, kh, :t + 1], dtype)
            for h in range(kh * G, kh * G + G):
                where = f"{tag} b={b} h={h} t={t}"
                r = O.decode_step(q64[b, h], k64, v64, t, s, topk, scale)
                tie = check_idx_row(g["idx"][b, h], r, q64[b, h], k64, t, s, topk, where)
                tied += tie
                os_, ls_ = r["o_s"], r["lse_s"]
                if tie:   # the sparse stream on the GPU's own selection
                    qa = np.zeros((1, 1, t + 1, D))
                    qa[0, 0, t] = q64[b, h]
                    os4, ls4 = O.attend_sparse_gather(qa, k64[None, None], v64[None, None],
                                                      g["idx"][b, h][None, None, None, :], s, scale, rows=[t])
                    os_, ls_ = os4[0, 0, 0], ls4[0, 0, 0]
                err["o_s"] = max(err["o_s"], assert_close(g["o_s"][b, h], os_, tol, where + " o_s"))
                err["lse_s"] = max(err["lse_s"], assert_close(g["lse_s"][b, h], ls_, tol, where + " lse_s"))
                err["o_f"] = max(err["o_f"], assert_close(g["o_f"][b, h], r["o_f"], tol, where + " o_f"))
                err["lse_f"] = max(err["lse_f"], assert_close(g["lse_f"][b, h], r["lse_f"], tol, where + " lse_f"))
    # per-token statistics from the GPU's own outputs
    d2, dm2 = O.align_stats(g["o_f"], g["o_s"], g["lse_f"], g["lse_s"])
    assert np.allclose(g["dist"], d2, rtol=1e-5, atol=1e-6)
    assert np.allclose(g["drop"], dm2, rtol=1e-5, atol=1e-6)
    say(f"[oracle] decode {tag}: max errors {err}, tolerated tie rows {tied}")
    return g


# ----------------------------------------------------------------------------------
# one decoding step against the oracle
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,D,s,Hkv", [(W.BF16, 128, 64, 4), (W.BF16, 64, 128, 4), (W.F32, 128, 64, 4),
                                           (W.F32, 64, 64, 2), (W.BF16, 128, 64, 1)])
@pytest.mark.parametrize("topk", [1, 4, 9])
def test_decode_step(dtype, D, s, Hkv, topk):
    B, H, L = 5, 4, 2048
    inp = W.make_qkv(B, Hkv, L, D, s, dtype, "sink", seed=2100 + D + s + topk, hkv=Hkv)
    q = W.make_qkv(B, H, 1, D, 1, dtype, "none", seed=2200 + topk).q[:, :, 0]
    n = L // s
    # first token, last of block 0, first of block 1, block topk-1/topk edges, last row
    pos = np.array([0, s - 1, s, min(topk * s, L - 1), L - 1], dtype=np.int32)[:B]
    run_and_check(inp.k, inp.v, q, pos, s, topk, dtype, Hkv, tag=f"step n={n}")


@pytest.mark.parametrize("H,Hkv", [(32, 2), (32, 1), (8, 8), (12, 4)])
def test_decode_grouped_heads(H, Hkv):
    """Many query heads per key/value head (the dense stream then runs on the matrix cores,
    16 heads per pass: G = 16, 32 (two passes), 1 and 3)."""
    B, L, D, s, topk = 2, 2048, 128, 64, 6
    inp = W.make_qkv(B, Hkv, L, D, s, W.BF16, "sink", seed=2900 + H + Hkv, hkv=Hkv)
    q = W.make_qkv(B, H, 1, D, 1, W.BF16, "none", seed=2950 + H).q[:, :, 0]
    pos = np.array([1500, 777], dtype=np.int32)
    run_and_check(inp.k, inp.v, q, pos, s, topk, W.BF16, Hkv, tag=f"G={H // Hkv}")


@pytest.mark.parametrize("dtype", [W.BF16, W.F32])
def test_decode_all_blocks_equals_full(dtype):
    """topk = n keeps every earlier block: the sparse stream equals the full stream."""
    B, H, L, D, s = 3, 2, 1024, 128, 64
    inp = W.make_qkv(B, H, L, D, s, dtype, "none", seed=2301)
    q = W.make_qkv(B, H, 1, D, 1, dtype, "none", seed=2302).q[:, :, 0]
    pos = np.array([700, 1023, 64], dtype=np.int32)
    g = run_and_check(inp.k, inp.v, q, pos, s, L // s, dtype, H, tag="k=n")
    tol = TOL[dtype]
    assert np.max(np.abs(g["o_s"] - g["o_f"])) <= tol
    assert np.max(np.abs(g["lse_s"] - g["lse_f"])) <= 1e-4
    assert np.all(g["drop"] <= 1e-4)


def test_decode_integer_ties_bit_exact():
    """Small-integer queries and keys make many block scores exactly equal (and exact in
    float32); the kept blocks must then follow the lower-index rule exactly."""
    B, H, L, D, s, topk = 4, 2, 4096, 64, 64, 12
    k = W.f32_to_bf16_bits(W.integer_tensor((B, H, L, D), -1, 1, seed=2401))
    v = W.f32_to_bf16_bits(W.integer_tensor((B, H, L, D), -3, 3, seed=2402))
    q = W.f32_to_bf16_bits(W.integer_tensor((B, H, D), -1, 1, seed=2403) * 0.125)
    pos = np.array([4095, 3000, 1500, 640], dtype=np.int32)
    g = run_and_check(k, v, q, pos, s, topk, W.BF16, H, tag="integer ties")
    # exact ties must not be tolerated: with exact scores the rows must match exactly
    q64 = _f64(q, W.BF16)
    for b in range(B):
        for h in range(H):
            k64 = _f64(k[b, h, :int(pos[b]) + 1], W.BF16)
            r = O.decode_step(q64[b, h], k64, k64, int(pos[b]), s, topk, 1.0)
            assert g["idx"][b, h].tolist() == r["idx"].tolist(), (b, h)


def test_decode_many_blocks():
    """8192 candidate blocks (the selection's largest supported n), with a sequence near
    the end of the cache."""
    B, H, L, D, s, topk = 1, 1, 8192 * 64, 64, 64, 32
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "sink", seed=2501)
    q = W.make_qkv(B, H, 1, D, 1, W.BF16, "none", seed=2502).q[:, :, 0]
    pos = np.array([L - 1], dtype=np.int32)
    run_and_check(inp.k, inp.v, q, pos, s, topk, W.BF16, H, tag="n=8192")


def test_decode_positions_outside_the_cache():
    """pos outside [0, L): the forward calls write NaN to o and lse and -1 to idx, the
    append leaves the cache and the pooled keys untouched; other sequences are normal."""
    B, H, L, D, s = 3, 2, 512, 128, 64
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "none", seed=2601)
    q = W.make_qkv(B, H, 1, D, 1, W.BF16, "none", seed=2602).q[:, :, 0]
    kd, vd, qd = to_device(inp.k, W.BF16), to_device(inp.v, W.BF16), to_device(q, W.BF16)
    pos = torch.tensor([-1, 300, L], dtype=torch.int32, device="cuda")
    km = ssa.block_pool(kd, s)
    o_s, lse_s, idx = ssa.decode_sparse_fwd(pos, qd, kd, vd, km, s, 4)
    o_f, lse_f = ssa.decode_full_fwd(pos, qd, kd, vd, block=s)
    k_before, v_before, km_before = kd.clone(), vd.clone(), km.clone()
    kn = torch.zeros((B, H, D), dtype=torch.bfloat16, device="cuda")
    ssa.decode_append(pos, kn, kn, kd, vd, km, s)
    torch.cuda.synchronize()
    for b in (0, 2):
        assert torch.isnan(o_s[b].float()).all() and torch.isnan(lse_s[b]).all()
        assert torch.isnan(o_f[b].float()).all() and torch.isnan(lse_f[b]).all()
        assert (idx[b] == -1).all()
        assert torch.equal(kd[b], k_before[b]) and torch.equal(vd[b], v_before[b])
        assert torch.equal(km[b], km_before[b])
    assert torch.isfinite(o_s[1].float()).all() and torch.isfinite(lse_f[1]).all()
    assert (kd[1, :, 300] == 0).all() and (vd[1, :, 300] == 0).all()   # sequence 1 appended


# ----------------------------------------------------------------------------------
# appends: the cache and the pooled keys
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,D,s", [(W.BF16, 128, 64), (W.F32, 64, 128)])
def test_decode_append_pooled_keys(dtype, D, s):
    """Start from a prompt pooled by ssa_block_pool (rows after it poisoned), append
    tokens one at a time at different positions per sequence.  The cache rows equal the
    tokens bit for bit; completed blocks' pooled keys equal ssa_block_pool's over the
    whole sequence bit for bit; the open block's entry is the oracle's open-block mean."""
    B, H, L = 3, 2, 1024
    inp = W.make_qkv(B, H, L, D, s, dtype, "sink", seed=2700 + D)
    kd, vd = to_device(inp.k, dtype), to_device(inp.v, dtype)
    prompt = np.array([s - 3, 2 * s + 5, 3 * s], dtype=np.int64)   # tokens already cached
    steps = s + 7
    kc, vc = kd.clone(), vd.clone()
    for b in range(B):
        kc[b, :, prompt[b]:] = 1000.0
        vc[b, :, prompt[b]:] = -1000.0
    km = ssa.block_pool(kc, s)
    km_full = ssa.block_pool(kd, s)
    for i in range(steps):
        p = torch.from_numpy((prompt + i).astype(np.int32)).cuda()
        ssa.decode_append(p, kd[torch.arange(B), :, p.long()].contiguous(),
                          vd[torch.arange(B), :, p.long()].contiguous(), kc, vc, km, s)
    torch.cuda.synchronize()
    k64 = _f64(inp.k, dtype)
    for b in range(B):
        last = int(prompt[b]) + steps - 1
        assert torch.equal(kc[b, :, :last + 1], kd[b, :, :last + 1])
        assert torch.equal(vc[b, :, :last + 1], vd[b, :, :last + 1])
        assert (kc[b, :, last + 1:].float() == 1000.0).all()
        for j in range(last // s):                    # complete blocks
            assert torch.equal(km[b, :, j], km_full[b, :, j]), (b, j)
        for h in range(H):                            # the open block
            ref = O.open_block_mean(k64[b, h], last, s)
            got = km[b, h, last // s].cpu().numpy().astype(np.float64)
            assert np.allclose(got, ref, rtol=1e-6, atol=1e-6 * max(1.0, np.abs(ref).max())), (b, h)


def test_decode_loop_gqa():
    """Prompt pooled, then a run of decoding steps (append, sparse, full, stats) with two
    key/value heads per four query heads, each step checked against the oracle."""
    B, H, Hkv, L, D, s, topk = 2, 4, 2, 512, 128, 64, 3
    inp = W.make_qkv(B, H, L, D, s, W.BF16, "sink", seed=2801, hkv=Hkv)
    kd, vd, qd = (to_device(a, W.BF16) for a in (inp.k, inp.v, inp.q))
    P = np.array([130, 60])
    kc, vc = torch.zeros_like(kd), torch.zeros_like(vd)
    for b in range(B):
        kc[b, :, :P[b]] = kd[b, :, :P[b]]
        vc[b, :, :P[b]] = vd[b, :, :P[b]]
    km = ssa.block_pool(kc, s)
    for i in range(0, 70, 7):
        pos = (P + i).astype(np.int32)
        p = torch.from_numpy(pos).cuda()
        ar = torch.arange(B)
        # append every token from the last step's position up to pos
        for j in range(max(0, i - 6), i + 1):
            pj = torch.from_numpy((P + j).astype(np.int32)).cuda()
            ssa.decode_append(pj, kd[ar, :, pj.long()].contiguous(), vd[ar, :, pj.long()].contiguous(),
                              kc, vc, km, s)
        q_now = qd[ar, :, p.long()].contiguous()
        run_and_check(kc.view(torch.int16).cpu().numpy().view(np.uint16), vc.view(torch.int16).cpu().numpy()
                      .view(np.uint16), q_now.view(torch.int16).cpu().numpy().view(np.uint16), pos, s, topk,
                      W.BF16, Hkv, tag=f"loop step {i}", km=km)


# ----------------------------------------------------------------------------------
# the decoding benchmark's configuration, sampled
# ----------------------------------------------------------------------------------
def test_decode_bench_workload_sampled():
    """bf16_L32768_decode (4 sequences, 32 heads, cache 32768) in the launch
    configuration the benchmark times; every (b, h) checked against the oracle."""
    di = W.make_decode("bf16_L32768_decode")
    w = di.workload
    run_and_check(di.k, di.v, di.q, di.pos, w.s, w.k, w.dtype, w.hkv, tag=w.name)
