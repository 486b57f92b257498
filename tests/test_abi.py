"""The C-ABI library loads, exports every symbol include/ssa.h declares, and rejects bad
arguments with the documented status codes before any GPU work (CPU-only: the pointers
below are never dereferenced, because every call fails validation first)."""
import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_top_ssa_amd import _lib
from conftest import ROOT, gpu_available

HEADER = os.path.join(ROOT, "include", "ssa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(libssa):
    names = _declared()
    assert set(names) == set(_lib.PROTOTYPES), "binding prototypes and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in names if n not in exported]
    assert not missing, f"not exported: {missing}"


def test_probe_library_exports_its_header():
    """libssa_probe.so (peak microbenchmarks, include/ssa_probe.h) exports what its header
    declares, and rejects bad arguments before launching anything."""
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "ssa_probe.h")).read(), flags=re.S)
    names = set(re.findall(r"\b(ssa_probe_[a-z_0-9]+)\s*\(", text))
    assert names == set(_lib.PROBE_PROTOTYPES), "probe prototypes and header disagree"
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.PROBE_PATH], capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert names <= exported, f"not exported: {sorted(names - exported)}"
    if gpu_available():
        return
    lib = _lib.load_probe()
    bad = 1  # hipErrorInvalidValue
    assert lib.ssa_probe_mfma_bf16(0, 10, FAKE, None) == bad
    assert lib.ssa_probe_hbm_read(FAKE, 24, 4, FAKE, None) == bad  # not a multiple of 16


def test_version_and_status_strings(libssa):
    v = int(re.search(r"#define SSA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert libssa.ssa_abi_version() == v
    for code, name in _lib.STATUS.items():
        assert libssa.ssa_status_str(code).decode() == name
    assert libssa.ssa_status_str(99).decode() == "SSA_ERR_UNKNOWN"


def test_variant_switch(libssa):
    prev = libssa.ssa_set_kernel_variant(1)
    assert libssa.ssa_set_kernel_variant(prev) == 1


FAKE = ctypes.c_void_p(1 << 20)       # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p((1 << 20) + 2)


def _dims(B=1, H=2, L=256, D=128, block=64, dtype=_lib.SSA_BF16, Hkv=0):
    return _lib.Dims(B, H, L, D, block, dtype, Hkv)


def test_dims_struct_matches_header():
    """The ctypes struct lists the header's ssa_dims fields in order (int32 each)."""
    body = re.search(r"typedef struct \{(.*?)\} ssa_dims;", open(HEADER).read(), re.S).group(1)
    names = []
    for line in body.splitlines():
        decl = line.split("/*")[0].strip().rstrip(";")
        if decl.startswith("int32_t"):
            names += [x.strip() for x in decl[len("int32_t"):].split(",")]
    assert names == [f[0] for f in _lib.Dims._fields_]
    assert ctypes.sizeof(_lib.Dims) == 4 * len(names)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), 3), (dict(D=96), 2), (dict(block=32), 2), (dict(L=200), 2), (dict(B=0), 2),
    (dict(H=-1), 2), (dict(B=1 << 10, H=1 << 10, L=1 << 10), 2),
    (dict(H=6, Hkv=4), 2), (dict(H=4, Hkv=-2), 2), (dict(H=4, Hkv=8), 2),
])
def test_bad_dims(libssa, kw, code):
    d = _dims(**kw)
    assert libssa.ssa_block_pool(ctypes.byref(d), FAKE, FAKE, None) == code
    assert libssa.ssa_last_error().decode()


def test_null_and_alignment(libssa):
    d = _dims()
    assert libssa.ssa_block_pool(None, FAKE, FAKE, None) == 1
    assert libssa.ssa_block_pool(ctypes.byref(d), None, FAKE, None) == 1
    assert libssa.ssa_block_pool(ctypes.byref(d), MISALIGNED, FAKE, None) == 4
    assert libssa.ssa_block_topk(ctypes.byref(d), FAKE, FAKE, 2, None, None, None) == 1
    assert libssa.ssa_sparse_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 2, 0.1, None, None, None) == 1
    assert libssa.ssa_full_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, 0.1, None, None, None) == 1
    assert libssa.ssa_full_attn_fwd(ctypes.byref(d), FAKE, FAKE, MISALIGNED, 0.1, FAKE, None, None) == 4
    assert libssa.ssa_align_stats(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, None) == 1
    assert libssa.ssa_align_stats(ctypes.byref(d), FAKE, None, None, None, FAKE, None, None) == 1
    assert libssa.ssa_align_stats(ctypes.byref(d), None, None, FAKE, None, None, FAKE, None) == 1


def test_decode_argument_checks(libssa):
    d = _dims()
    # append: every pointer required, 16-byte aligned tensors, 4-byte aligned pos
    assert libssa.ssa_decode_append(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert libssa.ssa_decode_append(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert libssa.ssa_decode_append(ctypes.byref(d), FAKE, MISALIGNED, FAKE, FAKE, FAKE, FAKE, None) == 4
    # sparse: o required; lse, idx optional; topk in [1, n]
    assert libssa.ssa_decode_sparse_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0.1,
                                        None, None, None, None) == 1
    assert libssa.ssa_decode_sparse_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0.1,
                                        FAKE, None, None, None) == 2
    assert libssa.ssa_decode_sparse_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 5, 0.1,
                                        FAKE, None, None, None) == 2
    assert libssa.ssa_decode_sparse_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 2, -1.0,
                                        FAKE, None, None, None) == 4
    assert libssa.ssa_decode_sparse_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0.1,
                                        FAKE, None, ctypes.c_void_p((1 << 20) + 1), None) == 4
    # full: o or lse; v_cache only needed with o
    assert libssa.ssa_decode_full_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 0.1, None, None, None) == 1
    assert libssa.ssa_decode_full_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, None, 0.1, FAKE, None, None) == 1
    assert libssa.ssa_decode_full_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, float("nan"), FAKE, None,
                                      None) == 4
    # the cache capacity follows the block rules
    bad = _dims(L=200)
    assert libssa.ssa_decode_append(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2


def test_training_argument_checks(libssa):
    d = _dims()
    F = FAKE
    # backward: every tensor required, dq/dk/dv 16-byte aligned float32, scale checked
    assert libssa.ssa_full_attn_bwd(ctypes.byref(d), F, F, F, F, F, F, 0.1, F, F, None, None) == 1
    assert libssa.ssa_full_attn_bwd(ctypes.byref(d), F, F, F, None, F, F, 0.1, F, F, F, None) == 1
    assert libssa.ssa_full_attn_bwd(ctypes.byref(d), F, F, F, F, F, F, 0.0, F, F, F, None) == 4
    assert libssa.ssa_full_attn_bwd(ctypes.byref(d), F, F, F, F, F, MISALIGNED, 0.1, F, F, F, None) == 4
    assert libssa.ssa_sparse_attn_bwd(ctypes.byref(d), F, F, F, F, F, F, None, 2, 0.1, F, F, F, None) == 1
    assert libssa.ssa_sparse_attn_bwd(ctypes.byref(d), F, F, F, F, F, F, F, 9, 0.1, F, F, F, None) == 2
    # loss: o pair and loss required, gradients optional, beta > 0
    assert libssa.ssa_align_loss(ctypes.byref(d), F, F, 1.0, 1.0, None, None, None, None) == 1
    assert libssa.ssa_align_loss(ctypes.byref(d), F, None, 1.0, 1.0, F, None, None, None) == 1
    assert libssa.ssa_align_loss(ctypes.byref(d), F, F, 1.0, 0.0, F, None, None, None) == 4
    assert libssa.ssa_align_loss(ctypes.byref(d), F, F, float("inf"), 1.0, F, None, None, None) == 4


def test_stats_argument_checks(libssa):
    d = _dims()
    F = FAKE
    assert libssa.ssa_attn_stats(ctypes.byref(d), F, F, F, None, 0, 0.1, None, None, None) == 1
    assert libssa.ssa_attn_stats(ctypes.byref(d), F, None, F, None, 0, 0.1, F, None, None) == 1
    assert libssa.ssa_attn_stats(ctypes.byref(d), F, F, F, F, 9, 0.1, F, None, None) == 2
    assert libssa.ssa_attn_stats(ctypes.byref(d), F, F, F, None, 0, -0.1, F, None, None) == 4


def test_fused_measurement_argument_checks(libssa):
    d = _dims()
    F = FAKE
    # the fused full forward needs at least one measurement output; q, k, v required, scale > 0
    assert libssa.ssa_full_attn_fwd_stats(ctypes.byref(d), F, F, F, 0.1, F, F, None, None, None) == 1
    assert libssa.ssa_full_attn_fwd_stats(ctypes.byref(d), F, None, F, 0.1, None, None, F, None, None) == 1
    assert libssa.ssa_full_attn_fwd_stats(ctypes.byref(d), F, F, MISALIGNED, 0.1, None, None, F, None, None) == 4
    assert libssa.ssa_full_attn_fwd_stats(ctypes.byref(d), F, F, F, -0.1, None, None, None, F, None) == 4
    # the retained-mass histogram needs the lse pair and whole 64-row groups
    assert libssa.ssa_align_stats_hist(ctypes.byref(d), None, None, None, None, None, None, None, None) == 1
    assert libssa.ssa_align_stats_hist(ctypes.byref(d), None, None, F, None, None, None, F, None) == 1
    d1 = _dims(L=1, block=0)
    assert libssa.ssa_align_stats_hist(ctypes.byref(d1), None, None, F, F, None, None, F, None) == 2


@pytest.mark.skipif(gpu_available(), reason="checks the no-device path; a GPU is present")
def test_align_ignores_block(libssa):
    """ssa_align_stats does not use the block partition, so L = 1 (one decoding step) and
    an unused block value pass its shape checks and fail only at the device check."""
    d = _dims(L=1, block=0)
    assert libssa.ssa_align_stats(ctypes.byref(d), FAKE, FAKE, None, None, FAKE, None, None) == 5


@pytest.mark.parametrize("topk", [0, -1, 5])
def test_topk_range(libssa, topk):
    d = _dims(L=256, block=64)   # n = 4
    assert libssa.ssa_block_topk(ctypes.byref(d), FAKE, FAKE, topk, FAKE, None, None) == 2
    assert libssa.ssa_sparse_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, topk, 0.1, FAKE, None, None) == 2


@pytest.mark.parametrize("scale", [0.0, -1.0, float("nan"), float("inf")])
def test_bad_scale(libssa, scale):
    d = _dims()
    assert libssa.ssa_full_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, scale, FAKE, None, None) == 4
    assert libssa.ssa_sparse_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 2, scale, FAKE, None, None) == 4


@pytest.mark.skipif(gpu_available(), reason="checks the no-device path; a GPU is present")
def test_valid_call_without_device_reports_device_error(libssa):
    d = _dims()
    assert libssa.ssa_block_pool(ctypes.byref(d), FAKE, FAKE, None) == 5
    assert "device" in libssa.ssa_last_error().decode().lower() or libssa.ssa_last_error()


def test_decode_noalloc_argument_checks(libssa):
    """The allocation-free sparse decoding call checks like ssa_decode_sparse_fwd and
    refuses, before any device work, a shape whose scratch would pass its 16 MiB array."""
    d = _dims()
    assert libssa.ssa_decode_sparse_fwd_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 2, 0.1,
                                                None, None, None, None) == 1
    assert libssa.ssa_decode_sparse_fwd_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 0, 0.1,
                                                FAKE, None, None, None) == 2
    assert libssa.ssa_decode_sparse_fwd_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 2, -1.0,
                                                FAKE, None, None, None) == 4
    # B*H*ceil(topk*block/256)*(D+2)*4 = 4096*8*130*4 = 17039360 bytes > 16 MiB
    big = _dims(B=32, H=128, L=2048, block=128, D=128)
    assert libssa.ssa_decode_sparse_fwd_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, 16, 0.1,
                                                FAKE, None, FAKE, None) == 2
    assert "scratch" in libssa.ssa_last_error().decode()


def test_kv_frag_argument_checks(libssa):
    """The shared fragment-order copies: size query, the copy call (bf16 only, at least one
    copy, aligned buffers) and the forwards that read them (copies required on bf16)."""
    d = _dims(B=2, H=4, L=256, D=128, Hkv=2)
    n = ctypes.c_int64(-1)
    assert libssa.ssa_kv_frag_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    assert n.value == 2 * 2 * 256 * 128 * 2
    f32 = _dims(dtype=_lib.SSA_F32)
    assert libssa.ssa_kv_frag_bytes(ctypes.byref(f32), ctypes.byref(n)) == 0 and n.value == 0
    assert libssa.ssa_kv_frag_bytes(ctypes.byref(d), None) == 1
    assert libssa.ssa_kv_frag_bytes(ctypes.byref(_dims(D=96)), ctypes.byref(n)) == 2
    F = FAKE
    assert libssa.ssa_kv_frag(ctypes.byref(d), F, F, None, None, None) == 1
    assert libssa.ssa_kv_frag(ctypes.byref(f32), F, F, F, F, None) == 3
    assert libssa.ssa_kv_frag(ctypes.byref(d), None, F, F, None, None) == 1
    assert libssa.ssa_kv_frag(ctypes.byref(d), F, F, F, MISALIGNED, None) == 4
    assert libssa.ssa_sparse_attn_fwd_frag(ctypes.byref(d), F, F, F, None, F, F, 2, 0.1, F, None, None) == 1
    assert libssa.ssa_sparse_attn_fwd_frag(ctypes.byref(d), F, F, F, F, MISALIGNED, F, 2, 0.1, F, None, None) == 4
    assert libssa.ssa_sparse_attn_fwd_frag(ctypes.byref(d), F, F, F, F, F, F, 5, 0.1, F, None, None) == 2
    assert libssa.ssa_full_attn_fwd_frag(ctypes.byref(d), F, F, F, None, 0.1, F, None, None) == 1
    assert libssa.ssa_full_attn_fwd_frag(ctypes.byref(d), F, F, F, F, 0.1, None, None, None) == 1
    assert libssa.ssa_full_attn_fwd_frag(ctypes.byref(d), F, F, F, F, -0.1, F, None, None) == 4
    if not gpu_available():
        # without o the copy of v is not needed; on float32 no copy is needed at all
        assert libssa.ssa_full_attn_fwd_frag(ctypes.byref(d), F, F, F, None, 0.1, None, F, None) == 5
        assert libssa.ssa_sparse_attn_fwd_frag(ctypes.byref(f32), F, F, F, None, None, F, 2, 0.1, F, None,
                                               None) == 5
        assert libssa.ssa_kv_frag(ctypes.byref(d), F, None, F, None, None) == 5


def test_sparse_fwd_stats_argument_checks(libssa):
    """The fused sparse measurements check like ssa_sparse_attn_fwd and need at least one
    measurement output."""
    d = _dims()
    F = FAKE
    assert libssa.ssa_sparse_attn_fwd_stats(ctypes.byref(d), F, F, F, F, 2, 0.1, F, None, None, None, None) == 1
    assert libssa.ssa_sparse_attn_fwd_stats(ctypes.byref(d), F, F, F, None, 2, 0.1, F, None, F, None, None) == 1
    assert libssa.ssa_sparse_attn_fwd_stats(ctypes.byref(d), F, F, F, F, 2, 0.1, None, None, F, None, None) == 1
    assert libssa.ssa_sparse_attn_fwd_stats(ctypes.byref(d), F, F, F, F, 9, 0.1, F, None, F, None, None) == 2
    assert libssa.ssa_sparse_attn_fwd_stats(ctypes.byref(d), F, F, F, F, 2, -0.1, F, None, None, F, None) == 4
    assert libssa.ssa_sparse_attn_fwd_stats(ctypes.byref(d), F, F, F, F, 2, 0.1, F, None, MISALIGNED, None,
                                            None) == 4
