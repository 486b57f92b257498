#!/usr/bin/env python3
"""Throughput of the SSA per-layer attention forward (both streams) on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input already
resident in HBM: block pool -> causal top-k selection -> k and v in the operand layouts
(ssa_kv_frag, once, into buffers owned here) -> sparse attention -> full attention (both
reading those layouts) -> alignment statistics (L2 distance and dropped mass).  Default
workload: bf16, B=1, H=32, L=32768, D=128, s=64, k=32 (token 0 an 8x-norm sink key).

Prints ONE JSON line.  `value` is the metric's quantity, the sparse-attention forward's
tokens/s: B*L / (the ssa_kv_frag time + the ssa_sparse_attn_fwd_frag time) inside the
timed steps, so the layout pass the dense forward shares is counted against the sparse
one; the whole step's rate (B*L / step time) is `step_tokens_per_s`, its time
`ms_per_step`.  The per-kernel times come from HIP events recorded on the stream the
kernels run on (torch's current stream) around each call inside the timed steps.
`roofline` is given for the sparse-attention call, the kernel the metric names, on its
useful FLOPs 4*D*sum_t |A(t)|.  `cpu_baseline` times the CPU oracle's sparse stream on a
bounded sample of the same workload (rank 0, this process).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
                    [--no-cpu-baseline] [--copy-calib] [--per-call N] [--no-peaks]

`--per-call N` also times every C-ABI call of the step alone (3 warm-ups, then N
repetitions, median), writing a 1 GiB scratch buffer between repetitions when the
workload's inputs fit in the 256 MB last-level cache (so no repetition starts warm).
After the timed region the prefill path measures the device's own peaks with the probe
library (libssa_probe.so): back-to-back bf16 MFMA from registers and a streaming read of
4 GiB; they are reported beside the published peaks (`--no-peaks` skips this).

`--path decode` measures decoding with a key/value cache instead: one step = one new
token for each of B sequences (at different positions of a 32768-token cache): append
(cache rows + open block's pooled key) -> selection + sparse attention -> full attention
-> alignment statistics; `value` is tokens/s (B / step time) and `roofline` is given
for the dominant kernel, the full-stream attention, against HBM bandwidth.

`--path train` measures one layer's training step of both streams on the same workload:
pool -> top-k -> sparse and full forward -> alignment loss -> backward of the full
stream (upstream gradient = a synthetic language-model gradient + the loss's gradient)
and of the sparse stream (the loss's gradient) into shared float32 dq, dk, dv; `value` is
tokens/s (B*L / step time) and `roofline` is for the full stream's backward against the
MFMA bf16 peak (its algorithmic FLOPs 10*D per attended (query, key) pair).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
LLC_BYTES = 256 << 20       # MI355X last-level (Infinity) cache
METRIC = "sparse-attn fwd tokens/s and TFLOP/s (% MFMA bf16 peak) at L=32K"


def attended_total(L: int, s: int, k: int) -> int:
    """sum_t |A(t)| with |A(t)| = t+1 while t//s < k, else (k-1)*s + t%s + 1."""
    t = np.arange(L, dtype=np.int64)
    a = np.where(t // s < k, t + 1, (k - 1) * s + t % s + 1)
    return int(a.sum())


def work_model(w: W.Workload, k: int) -> dict:
    e = 2 if w.dtype == W.BF16 else 4
    BH, L, D, s, n = w.B * w.H, w.L, w.D, w.s, w.n
    BHkv = w.B * w.hkv                          # key/value heads (grouped-query attention)
    t = np.arange(L, dtype=np.int64)
    cand = int((t // s).sum())                  # candidate blocks scored per (b, h)
    return {
        "pool": {"bytes": BHkv * (L * D * e + n * D * 4)},
        "topk": {"flops": 2 * D * BH * cand, "bytes": BH * (L * D * e + L * k * 4) + BHkv * n * D * 4},
        # k and v read and written once in the operand layouts (bf16 only)
        "kvfrag": {"bytes": 4 * BHkv * L * D * e if w.dtype == W.BF16 else 0},
        "sparse": {"flops": 4 * D * BH * attended_total(L, s, k)},
        "full": {"flops": 4 * D * BH * (L * (L + 1) // 2)},
        "align": {"bytes": BH * L * (2 * D * e + 4 * 4)},
    }


# The sources each call's kernels come from (the sparse call hands full 64-row chunks to
# the dense kernel; the fragment-order copies both forwards read are the kvfrag call).
KERNEL_SOURCES = {"pool": ("pool.hip",), "topk": ("topk_mfma.hip",), "kvfrag": ("vfrag.hip",),
                  "sparse": ("sparse_mfma.hip", "full_mfma.hip"),
                  "full": ("full_mfma.hip",), "align": ("align.hip",)}
SHARED_HEADERS = ("common.hpp", "mfma.hpp", "rowattn.hpp")


DECODE_SOURCES = {"append": ("decode.hip",), "sparse": ("decode.hip",), "full": ("decode.hip",),
                  "align": ("align.hip",)}


def sources_sha256(files) -> str:
    """sha256 of the named csrc files, concatenated in order."""
    import hashlib
    csrc = os.path.join(ROOT, "block_sparse_top_ssa_amd", "csrc")
    return hashlib.sha256(b"".join(open(os.path.join(csrc, f), "rb").read() for f in files)).hexdigest()


def measured_traffic(workload: str, sources: dict = KERNEL_SOURCES) -> dict:
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (profiles/hbm_traffic.json, or profiles/hbm_traffic_<workload>.json), per kernel,
    only where the kernel's source and the shared headers are unchanged since the
    counters were taken; otherwise None."""
    out = {k: None for k in sources}
    rec = None
    for fn in ("hbm_traffic.json", f"hbm_traffic_{workload}.json"):
        try:
            r = json.load(open(os.path.join(ROOT, "profiles", fn)))
        except (OSError, ValueError):
            continue
        if r.get("workload") == workload:
            rec = r
            break
    if rec is None:
        return out
    hdr = sources_sha256(SHARED_HEADERS)
    for k, files in sources.items():
        t = rec.get("kernels", {}).get(k)
        if not t:
            continue
        if t.get("source_sha256") == sources_sha256(files) and t.get("headers_sha256") == hdr:
            out[k] = int(round(t["fetch_bytes"] + t["write_bytes"]))
    return out


def cpu_baseline(inp: W.Inputs, k: int, budget_s: float = 15.0) -> dict:
    """The CPU oracle's sparse stream (pool, select, sparse attention) on the last
    2048 query rows of as many heads as fit in about `budget_s` seconds."""
    import oracle.ssa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    w = inp.workload
    s, scale = w.s, 1.0 / math.sqrt(w.D)
    rows = np.arange(max(0, w.L - 2048), w.L)
    done_rows, heads, t_total = 0, 0, 0.0
    for h in range(w.H):
        def head64(a):
            x = a[:1, h:h + 1]
            return (W.bf16_bits_to_f32(x) if w.dtype == W.BF16 else x).astype(np.float64)

        def kvhead64(a):  # the key/value head query head h reads
            x = a[:1, h // w.group:h // w.group + 1]
            return (W.bf16_bits_to_f32(x) if w.dtype == W.BF16 else x).astype(np.float64)

        q, kk, vv = head64(inp.q), kvhead64(inp.k), kvhead64(inp.v)
        t0 = time.perf_counter()
        km = O.block_pool(kk, s)
        idx = O.block_topk(q, km, s, k, rows=rows)
        O.attend_sparse(q, kk, vv, idx, s, scale, rows=rows)
        t_total += time.perf_counter() - t0
        done_rows += len(rows)
        heads += 1
        if t_total >= budget_s:
            break
    try:
        cpu = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name")), "")
    except OSError:  # pragma: no cover
        cpu = ""
    tps = done_rows / t_total
    whole = w.B * w.H * w.L / tps
    return {"value": tps, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 numpy oracle sparse stream (block pool + top-k select + masked sparse attention) "
                      f"on the last {len(rows)} query rows of {heads} of {w.B * w.H} heads (b=0), "
                      f"{t_total:.1f} s; tokens/s = timed rows / wall time; whole workload extrapolated: "
                      f"{whole:.0f} s",
            "cpu_model": cpu}


def time_calls(torch, calls: dict, reps: int, inputs_bytes: int) -> dict:
    """Each call alone on torch's current stream: 3 warm-ups, then `reps` repetitions timed
    with HIP events, median; a 1 GiB buffer is written before every repetition when the
    inputs fit in the last-level cache."""
    flush = inputs_bytes < LLC_BYTES
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if flush else None
    res = {}
    for nm, fn in calls.items():
        for _ in range(3):
            fn()
        ts = []
        for r in range(reps):
            if flush:
                scratch.fill_(float(r))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ts.append((e0, e1))
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in ts]
        res[nm] = {"median_ms": round(float(np.median(ms)), 4), "min_ms": round(float(np.min(ms)), 4), "reps": reps}
    return {"calls": res, "llc_flush_1GiB": flush, "inputs_bytes": int(inputs_bytes)}


def measure_peaks(torch) -> dict:
    """The device's reachable peaks (libssa_probe.so), best of 3, beside the published ones:
    bf16 MFMA issued back to back from registers (8 waves per SIMD, 8 independent chains
    each) and a 16-byte streaming read of 4 GiB (16x the last-level cache; 4, 8 and 16
    workgroups per CU, best taken)."""
    import ctypes
    from block_sparse_top_ssa_amd import _lib
    lib = _lib.load_probe()
    st = torch.cuda.current_stream()
    blocks, iters = 2048, 10000  # 8 waves per SIMD
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    flops = blocks * 4 * iters * 8 * 16384
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    rgrids = (256 * 4, 256 * 8, 256 * 16)  # workgroups of the read probe (4, 8, 16 per CU)
    rout = torch.empty(max(rgrids) * 256 * 4, dtype=torch.int32, device="cuda")
    best_mfma, best_rd = 0.0, 0.0
    for _ in range(3):
        e0, e1 = (torch.cuda.Event(enable_timing=True) for _ in range(2))
        e0.record()
        rc = lib.ssa_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(st.cuda_stream))
        e1.record()
        torch.cuda.synchronize()
        if rc:
            raise RuntimeError(f"MFMA peak probe launch failed ({rc})")
        best_mfma = max(best_mfma, flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        for rb in rgrids:
            e0.record()
            rc = lib.ssa_probe_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes, rb, ctypes.c_void_p(rout.data_ptr()),
                                        ctypes.c_void_p(st.cuda_stream))
            e1.record()
            torch.cuda.synchronize()
            if rc:
                raise RuntimeError(f"HBM read probe launch failed ({rc})")
            best_rd = max(best_rd, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    return {"mfma_bf16_tflops": round(best_mfma, 1), "mfma_bf16_published": PEAK_BF16_TFLOPS,
            "hbm_read_gbps": round(best_rd, 1), "hbm_published_gbps": PEAK_HBM_GBPS,
            "note": "libssa_probe.so: back-to-back v_mfma_f32_16x16x32_bf16 from registers (8 waves per SIMD); "
                    "16-byte streaming read of 4 GiB; best of 3"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=W.BENCH_WORKLOAD, choices=sorted(W.WORKLOADS))
    ap.add_argument("--topk", type=int, default=0, help="blocks per query (default: the workload's first k)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--per-call", type=int, default=0, metavar="N",
                    help="also time each call alone: 3 warm-ups, N repetitions, median")
    ap.add_argument("--no-peaks", action="store_true", help="skip the peak microbenchmarks")
    ap.add_argument("--copy-calib", action="store_true",
                    help="also run a plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--path", default="prefill", choices=["prefill", "decode", "train"],
                    help="prefill: the whole-sequence forward (default); decode: one cached decoding step; "
                         "train: forward, alignment loss and backward of both streams")
    ap.add_argument("--decode-workload", default="bf16_L32768_decode", choices=sorted(W.DECODE_WORKLOADS))
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(every kernel is independent per (b, h), so the path would shard by head with no exchange).",
              file=sys.stderr)
        sys.exit(2)
    if args.path == "decode":
        return main_decode(args)
    if args.path == "train":
        return main_train(args)

    import torch
    import block_sparse_top_ssa_amd as ssa

    w = W.WORKLOADS[args.workload]
    k = args.topk or w.ks[0]
    inp = W.make_workload(args.workload)

    def dev(a):
        if w.dtype == W.BF16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    q, kk, v = dev(inp.q), dev(inp.k), dev(inp.v)
    s, scale = w.s, 1.0 / math.sqrt(w.D)
    B, H, L, D = w.B, w.H, w.L, w.D
    km = torch.empty((B, w.hkv, w.n, D), dtype=torch.float32, device="cuda")  # pooled keys of the K/V heads
    idx = torch.empty((B, H, L, k), dtype=torch.int32, device="cuda")
    o_s = torch.empty_like(q)
    o_f = None if w.sparse_only else torch.empty_like(q)
    lse_s = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    lse_f = torch.empty_like(lse_s)

    # k and v in the matrix-core operand layouts, written once per step into buffers owned
    # here and read by both forwards (bf16; float32 takes no copies)
    frag = w.dtype == W.BF16
    nfrag = ssa.kv_frag_bytes(kk, s)
    kf = torch.empty(nfrag, dtype=torch.uint8, device="cuda") if frag else None
    vf = torch.empty(nfrag, dtype=torch.uint8, device="cuda") if frag else None
    names = ["pool", "topk", "kvfrag", "sparse", "full", "align"]

    def kv_layout():
        if frag:
            ssa.kv_frag(kk, v, s, k_frag=kf, v_frag=vf)

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        ssa.block_pool(kk, s, out=km)
        mark(1)
        ssa.block_topk(q, km, s, k, out=idx)
        mark(2)
        kv_layout()
        mark(3)
        ssa.sparse_attn_fwd_frag(q, kk, v, kf, vf, idx, s, scale, out=o_s, lse=lse_s)
        mark(4)
        ssa.full_attn_fwd_frag(q, kk, v, vf, scale, want_o=o_f is not None, block=s, out=o_f, lse=lse_f)
        mark(5)
        if o_f is not None:
            ssa.align_stats(o_f, o_s, lse_f, lse_s, block=s)
        else:
            ssa.align_stats(None, None, lse_f, lse_s, block=s, dims_like=q)
        mark(6)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    per = {nm: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, nm in enumerate(names)}

    if args.copy_calib:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    per_call = None
    if args.per_call > 0:
        calls = {
            "pool": lambda: ssa.block_pool(kk, s, out=km),
            "topk": lambda: ssa.block_topk(q, km, s, k, out=idx),
            "kvfrag": kv_layout,
            "sparse": lambda: ssa.sparse_attn_fwd_frag(q, kk, v, kf, vf, idx, s, scale, out=o_s, lse=lse_s),
            "full": lambda: ssa.full_attn_fwd_frag(q, kk, v, vf, scale, want_o=o_f is not None, block=s, out=o_f,
                                                   lse=lse_f),
            # the default calls, which write their own transient copies
            "sparse_own_copies": lambda: ssa.sparse_attn_fwd(q, kk, v, idx, s, scale, out=o_s, lse=lse_s),
            "full_own_copy": lambda: ssa.full_attn_fwd(q, kk, v, scale, want_o=o_f is not None, block=s, out=o_f,
                                                       lse=lse_f),
            "align": (lambda: ssa.align_stats(o_f, o_s, lse_f, lse_s, block=s)) if o_f is not None
            else (lambda: ssa.align_stats(None, None, lse_f, lse_s, block=s, dims_like=q)),
        }
        per_call = time_calls(torch, calls, args.per_call, inputs_bytes=q.nbytes + kk.nbytes + v.nbytes)

    model = work_model(w, k)
    traffic = measured_traffic(w.name)
    kernels = {}
    for nm in names:
        ms = per[nm]
        ent = {"ms": round(ms, 4)}
        if "flops" in model[nm]:
            tf = model[nm]["flops"] / (ms * 1e-3) / 1e12
            ent["tflops"] = round(tf, 2)
            peak = PEAK_FP32_TFLOPS if nm == "topk" else PEAK_BF16_TFLOPS
            ent["frac_peak"] = round(tf / peak, 4)
        if "bytes" in model[nm]:
            gb = model[nm]["bytes"] / (ms * 1e-3) / 1e9
            ent["gbps"] = round(gb, 1)
            if "flops" not in model[nm]:
                ent["frac_peak"] = round(gb / PEAK_HBM_GBPS, 4)
        ent["hbm_bytes_measured"] = traffic[nm]
        kernels[nm] = ent
    if o_f is None:
        kernels["full"]["note"] = "log-sum-exp only (value products skipped)"
        kernels["full"]["tflops"] = round(model["full"]["flops"] / 2 / (per["full"] * 1e-3) / 1e12, 2)

    # the sparse stream's forward: its attention call plus the operand layouts it reads
    # (both copies counted here, although the dense forward reads the v copy too)
    sp_ms = per["kvfrag"] + per["sparse"]
    sp_tflops = model["sparse"]["flops"] / (sp_ms * 1e-3) / 1e12
    attn_tflops = model["sparse"]["flops"] / (per["sparse"] * 1e-3) / 1e12
    tokens = B * L
    out = {
        "metric": METRIC,
        # the metric's quantity: sparse-attention forward tokens/s, from the HIP-event times
        # of the sparse call and the layout pass inside the timed steps; the whole step's
        # rate is step_tokens_per_s
        "value": round(tokens / (sp_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_tokens_per_s": round(tokens / (ms_step * 1e-3), 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == W.BF16 else "f32",
        "data": "synthetic (seeded N(0,1) q, k, v with the workload's key structure; no dataset, no weights)",
        "config": {"workload": w.name, "B": B, "H": H, "Hkv": w.hkv, "L": L, "D": D, "block": s, "topk": k,
                   "step": "pool+topk+kv_frag+sparse_attn+full_attn" + ("(lse only)" if o_f is None else "")
                   + "+align"},
        "sparse_attn": {"tokens_per_s": round(tokens / (sp_ms * 1e-3), 1),
                        "tflops": round(sp_tflops, 2), "pct_mfma_bf16_peak": round(100 * sp_tflops / PEAK_BF16_TFLOPS, 2),
                        "ms": round(sp_ms, 4), "ms_layout": round(per["kvfrag"], 4),
                        "ms_attention": round(per["sparse"], 4), "useful_flops": model["sparse"]["flops"]},
        # the dominant kernel: the sparse attention call (sparse_fwd_kernel and the dense
        # kernel on the 64-row chunks whose rows keep every earlier block)
        "roofline": {"kernel": "ssa_sparse_attn_fwd_frag", "bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic["sparse"], "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + "
                     "WRITE_SIZE, scaled by a 1 GiB copy; null when the kernel changed since)"},
        "kernels": kernels,
    }
    if per_call is not None:
        out["per_call"] = per_call
    if not args.no_peaks:
        out["peaks_measured"] = measure_peaks(torch)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, k)
    print(json.dumps(out), flush=True)


# ----------------------------------------------------------------------------------
# decoding with a key/value cache
# ----------------------------------------------------------------------------------
def decode_work_model(w: W.DecodeWorkload, pos: np.ndarray) -> dict:
    """Algorithmic HBM bytes per call of one decoding step (each byte read or written
    once): the full stream reads k and v rows 0..t of every key/value head; the sparse
    stream reads the pooled keys of the b_t candidate blocks and k, v of the attended
    rows of every query head, and writes the kept indices; append writes one row and
    re-reads the open block; align reads both outputs."""
    e = 2 if w.dtype == W.BF16 else 4
    D, s, k = w.D, w.s, w.k
    full = sparse = append = 0
    for t in pos.astype(np.int64):
        bt = t // s
        m = min(k - 1, bt)
        att = m * s + t % s + 1
        full += w.hkv * (t + 1) * D * e * 2 + w.H * (2 * D * e + 4)
        sparse += w.H * (bt * D * 4 + att * D * e * 2 + 2 * D * e + 4 + k * 4)
        append += w.hkv * (2 * D * e + (t % s + 1) * D * e + D * 4)
    return {"append": {"bytes": int(append)}, "sparse": {"bytes": int(sparse)}, "full": {"bytes": int(full)},
            "align": {"bytes": int(w.B * w.H * (2 * D * e + 4 * 4))}}


def cpu_baseline_decode(di: W.DecodeInputs, budget_s: float = 10.0) -> dict:
    """The CPU oracle's decode_step (both streams) on as many (sequence, head) rows as fit
    in about `budget_s` seconds; tokens/s counts a token as all H heads of a sequence."""
    import oracle.ssa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    w = di.workload
    scale = 1.0 / math.sqrt(w.D)
    rows, t_total = 0, 0.0
    for b in range(w.B):
        t = int(di.pos[b])
        for h in range(w.H):
            kh = h // w.group
            conv = (lambda a: W.bf16_bits_to_f32(a) if w.dtype == W.BF16 else a)
            kk = conv(di.k[b, kh, :t + 1]).astype(np.float64)
            vv = conv(di.v[b, kh, :t + 1]).astype(np.float64)
            qq = conv(di.q[b, h]).astype(np.float64)
            t0 = time.perf_counter()
            O.decode_step(qq, kk, vv, t, w.s, w.k, scale)
            t_total += time.perf_counter() - t0
            rows += 1
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    tps = rows / w.H / t_total
    return {"value": tps, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 numpy oracle decode_step (select, sparse and full attention) on {rows} of "
                      f"{w.B * w.H} (sequence, head) rows, {t_total:.1f} s; a token = all {w.H} heads of one "
                      f"sequence"}


def main_decode(args):
    import torch
    import block_sparse_top_ssa_amd as ssa

    di = W.make_decode(args.decode_workload)
    w = di.workload

    def dev(a):
        if w.dtype == W.BF16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    kc, vc, q = dev(di.k), dev(di.v), dev(di.q)
    pos = torch.from_numpy(di.pos).cuda()
    ar = torch.arange(w.B, device="cuda")
    k_new = kc[ar, :, pos.long()].contiguous()   # the new token's key and value (already at row pos)
    v_new = vc[ar, :, pos.long()].contiguous()
    s, scale = w.s, 1.0 / math.sqrt(w.D)
    km = ssa.block_pool(kc, s)                    # the prompt's pooled keys (outside the timed steps)
    names = ["append", "sparse", "full", "align"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        ssa.decode_append(pos, k_new, v_new, kc, vc, km, s)
        mark(1)
        o_s, lse_s, _ = ssa.decode_sparse_fwd(pos, q, kc, vc, km, s, w.k, scale, want_idx=False)
        mark(2)
        o_f, lse_f = ssa.decode_full_fwd(pos, q, kc, vc, scale, block=s)
        mark(3)
        ssa.align_stats(o_f.unsqueeze(2), o_s.unsqueeze(2), lse_f.unsqueeze(2), lse_s.unsqueeze(2), block=s)
        mark(4)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    per = {nm: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, nm in enumerate(names)}
    if args.copy_calib:
        a = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    model = decode_work_model(w, di.pos)
    traffic = measured_traffic(w.name, DECODE_SOURCES)
    kernels = {}
    for nm in names:
        gb = model[nm]["bytes"] / (per[nm] * 1e-3) / 1e9
        kernels[nm] = {"ms": round(per[nm], 4), "gbps": round(gb, 1), "frac_peak": round(gb / PEAK_HBM_GBPS, 4),
                       "algorithmic_bytes": model[nm]["bytes"], "hbm_bytes_measured": traffic[nm]}
    full_gbps = model["full"]["bytes"] / (per["full"] * 1e-3) / 1e9
    out = {
        "metric": "decode tokens/s (one new token per sequence, both streams) at a 32K cache",
        "value": round(w.B / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == W.BF16 else "f32",
        "data": "synthetic (seeded N(0,1) cache and queries, sink key at token 0; no dataset, no weights)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.hkv, "cache": w.L, "D": w.D, "block": s,
                   "topk": w.k, "positions": [int(x) for x in di.pos],
                   "step": "append+decode_sparse(select+attend)+decode_full+align"},
        "roofline": {"kernel": "ssa_decode_full_fwd", "bound": "hbm", "achieved": round(full_gbps, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(full_gbps / PEAK_HBM_GBPS, 4),
                     "traffic": traffic["full"], "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + "
                     "WRITE_SIZE, scaled by a 1 GiB copy; null when the kernel changed since)"},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(di)
    print(json.dumps(out), flush=True)


# ----------------------------------------------------------------------------------
# training step of both streams
# ----------------------------------------------------------------------------------
def cpu_baseline_train(inp: W.Inputs, k: int, Lc: int = 8192) -> dict:
    """The CPU oracle's backward of both streams on the first Lc positions of head 0 (the
    oracle forms the whole L x L weights, so the sample is a prefix, not a row subset)."""
    import oracle.ssa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    w = inp.workload
    s, scale = w.s, 1.0 / math.sqrt(w.D)
    conv = (lambda a: W.bf16_bits_to_f32(a) if w.dtype == W.BF16 else a)
    q = conv(inp.q[:1, :1, :Lc]).astype(np.float64)
    kk = conv(inp.k[:1, :1, :Lc]).astype(np.float64)
    vv = conv(inp.v[:1, :1, :Lc]).astype(np.float64)
    do = np.random.default_rng(7).standard_normal(q.shape)
    t0 = time.perf_counter()
    idx = O.block_topk(q, O.block_pool(kk, s), s, min(k, Lc // s))
    O.attend_full_bwd(q, kk, vv, do, scale)
    O.attend_sparse_bwd(q, kk, vv, do, idx, s, scale)
    dt = time.perf_counter() - t0
    return {"value": Lc / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 numpy oracle backward of both streams (plus its selection) on the first {Lc} "
                      f"positions of one head, {dt:.1f} s; tokens/s = {Lc} / wall time (one head; the oracle's "
                      f"cost grows as L^2, so this overstates its rate at L = {w.L})"}


def main_train(args):
    import torch
    import block_sparse_top_ssa_amd as ssa

    w = W.WORKLOADS[args.workload]
    k = args.topk or w.ks[0]
    inp = W.make_workload(args.workload)

    def dev(a):
        if w.dtype == W.BF16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    q, kk, v = dev(inp.q), dev(inp.k), dev(inp.v)
    s, scale, alpha = w.s, 1.0 / math.sqrt(w.D), 1.0
    B, H, L, D = w.B, w.H, w.L, w.D
    up = torch.randn(q.shape, generator=torch.Generator(device="cuda").manual_seed(11), device="cuda",
                     dtype=torch.float32).mul_(1e-3)   # stand-in for the language-model gradient
    km = torch.empty((B, w.hkv, w.n, D), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, H, L, k), dtype=torch.int32, device="cuda")
    o_s, o_f = torch.empty_like(q), torch.empty_like(q)
    lse_s = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    lse_f = torch.empty_like(lse_s)
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(kk.shape, dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    names = ["forward", "loss", "full_bwd", "sparse_bwd"]

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record()
        mark(0)
        ssa.block_pool(kk, s, out=km)
        ssa.block_topk(q, km, s, k, out=idx)
        ssa.sparse_attn_fwd(q, kk, v, idx, s, scale, out=o_s, lse=lse_s)
        ssa.full_attn_fwd(q, kk, v, scale, block=s, out=o_f, lse=lse_f)
        mark(1)
        loss, g_f, g_s = ssa.align_loss(o_f, o_s, alpha)
        do_f = (up + g_f).to(q.dtype)        # main stream: language-model gradient + alignment
        do_s = g_s.to(q.dtype)               # auxiliary stream: alignment only
        dq.zero_()
        dk.zero_()
        dv.zero_()
        mark(2)
        ssa.full_attn_bwd(q, kk, v, o_f, lse_f, do_f, dq, dk, dv, scale=scale, block=s)
        mark(3)
        ssa.sparse_attn_bwd(q, kk, v, o_s, lse_s, do_s, idx, s, dq, dk, dv, scale=scale)
        mark(4)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(evs[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    per = {nm: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, nm in enumerate(names)}
    # the attention-pattern measurements of both streams, timed apart from the step: each
    # fused into its stream's forward (the fused call's time over the plain one), and the
    # sparse stream's separate pass for comparison
    st_ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    st_ms = {"stats_full": [], "stats_sparse": [], "stats_sparse_pass": []}
    for _ in range(3):
        st_ev[0].record()
        ssa.full_attn_fwd(q, kk, v, scale, block=s, out=o_f, lse=lse_f)
        st_ev[1].record()
        ssa.full_attn_fwd_stats(q, kk, v, scale, block=s, out=o_f, lse=lse_f)
        st_ev[2].record()
        ssa.sparse_attn_fwd(q, kk, v, idx, s, scale, out=o_s, lse=lse_s)
        st_ev[3].record()
        ssa.sparse_attn_fwd_stats(q, kk, v, idx, s, scale, out=o_s, lse=lse_s)
        st_ev[4].record()
        ssa.attn_stats(q, kk, lse_s, s, idx=idx, scale=scale)
        st_ev[5].record()
        torch.cuda.synchronize()
        st_ms["stats_full"].append(st_ev[1].elapsed_time(st_ev[2]) - st_ev[0].elapsed_time(st_ev[1]))
        st_ms["stats_sparse"].append(st_ev[3].elapsed_time(st_ev[4]) - st_ev[2].elapsed_time(st_ev[3]))
        st_ms["stats_sparse_pass"].append(st_ev[4].elapsed_time(st_ev[5]))
    pairs_full = B * H * (L * (L + 1) // 2)
    pairs_sparse = B * H * attended_total(L, s, k)
    flops = {"full_bwd": 10 * D * pairs_full, "sparse_bwd": 10 * D * pairs_sparse}
    kernels = {nm: {"ms": round(per[nm], 4)} for nm in names}
    for nm, f in flops.items():
        tf = f / (per[nm] * 1e-3) / 1e12
        kernels[nm].update({"tflops": round(tf, 2), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                            "algorithmic_flops": f})
    kernels["loss"]["note"] = "alignment loss + upstream gradient composition (torch add/cast) + zeroing dq, dk, dv"
    kernels["stats_full"] = {"ms": round(float(np.median(st_ms["stats_full"])), 4),
                             "note": "entropy + distance histogram fused into the full forward "
                                     "(ssa_full_attn_fwd_stats): its time over ssa_full_attn_fwd; not part of the step"}
    kernels["stats_sparse"] = {"ms": round(float(np.median(st_ms["stats_sparse"])), 4),
                               "note": "entropy + distance histogram fused into the sparse forward "
                                       "(ssa_sparse_attn_fwd_stats): its time over ssa_sparse_attn_fwd; not part of "
                                       "the step"}
    ms = float(np.median(st_ms["stats_sparse_pass"]))
    kernels["stats_sparse_pass"] = {"ms": round(ms, 4), "tflops": round(2 * D * pairs_sparse / (ms * 1e-3) / 1e12, 2),
                                    "note": "the same measurements as a separate pass (ssa_attn_stats over the kept "
                                            "blocks), not part of the step; 2*D FLOP per attended pair"}
    tf_full = flops["full_bwd"] / (per["full_bwd"] * 1e-3) / 1e12
    out = {
        "metric": "training step tokens/s (forward, alignment loss, backward of both streams) at L=32K",
        "value": round(B * L / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == W.BF16 else "f32",
        "data": "synthetic (seeded N(0,1) q, k, v with the workload's key structure, N(0,1e-6) upstream gradient)",
        "config": {"workload": w.name, "B": B, "H": H, "Hkv": w.hkv, "L": L, "D": D, "block": s, "topk": k,
                   "alpha": alpha, "step": "pool+topk+sparse_fwd+full_fwd+align_loss+full_bwd+sparse_bwd"},
        "roofline": {"kernel": "ssa_full_attn_bwd", "bound": "mfma", "achieved": round(tf_full, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf_full / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "note": "matrix-core kernels (bf16 products, float32 accumulation)"},
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_train(inp, k)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
