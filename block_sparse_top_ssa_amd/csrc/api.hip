// C ABI of libssa: argument checks, device check, kernel choice, launch on the
// caller's stream.  Declared and documented in include/ssa.h.
#include <atomic>
#include <cstdarg>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/ssa.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";
std::atomic<int32_t> g_variant{0};

ssa_status fail(ssa_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ssa_status fail(ssa_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

// Per-device "is gfx950" cache, filled once per device.
constexpr int kMaxDevices = 64;
std::atomic<int8_t> g_dev_ok[kMaxDevices];  // 0 unknown, 1 ok, -1 not gfx950
std::mutex g_dev_mu;

ssa_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0) return fail(SSA_ERR_DEVICE, "no HIP device: %s", hipGetErrorString(e));
  if (dev >= kMaxDevices) return fail(SSA_ERR_DEVICE, "device index %d out of range", dev);
  int8_t st = g_dev_ok[dev].load(std::memory_order_acquire);
  if (st == 0) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    st = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (st == 0) {
      hipDeviceProp_t prop;
      e = hipGetDeviceProperties(&prop, dev);
      if (e != hipSuccess) return fail(SSA_ERR_DEVICE, "hipGetDeviceProperties: %s", hipGetErrorString(e));
      st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
      g_dev_ok[dev].store(st, std::memory_order_release);
    }
  }
  if (st != 1) return fail(SSA_ERR_DEVICE, "device %d is not gfx950 (MI355X)", dev);
  return SSA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// `blocks` = false for calls that do not use the block partition (ssa_align_stats):
// then block is not checked and L need not be a multiple of it.
ssa_status check_dims(const ssa_dims* d, ssa::Dims* out, bool blocks = true) {
  if (!d) return fail(SSA_ERR_NULL, "dims is NULL");
  if (d->dtype != SSA_F32 && d->dtype != SSA_BF16) return fail(SSA_ERR_DTYPE, "unknown dtype %d", d->dtype);
  if (d->B < 1 || d->H < 1 || d->L < 1) return fail(SSA_ERR_SHAPE, "B, H, L must be >= 1 (got %d, %d, %d)", d->B, d->H, d->L);
  if (d->D != 64 && d->D != 128) return fail(SSA_ERR_SHAPE, "head dim D must be 64 or 128 (got %d)", d->D);
  if (blocks && d->block != 64 && d->block != 128)
    return fail(SSA_ERR_SHAPE, "block size must be 64 or 128 (got %d)", d->block);
  if (blocks && d->L % d->block) return fail(SSA_ERR_SHAPE, "L=%d is not a multiple of the block size %d", d->L, d->block);
  const int hkv = d->Hkv == 0 ? d->H : d->Hkv;
  if (hkv < 1 || d->H % hkv) return fail(SSA_ERR_SHAPE, "Hkv=%d must be >= 1 and divide H=%d (0 means H)", d->Hkv, d->H);
  const int64_t tokens = (int64_t)d->B * d->H * d->L;
  if (tokens > (int64_t(1) << 24)) return fail(SSA_ERR_SHAPE, "B*H*L=%lld exceeds 2^24", (long long)tokens);
  *out = ssa::Dims{d->B, d->H, d->L, d->D, blocks ? d->block : 64, d->dtype, hkv};
  return SSA_OK;
}

ssa_status check_ptr(const void* p, const char* name, size_t align) {
  if (!p) return fail(SSA_ERR_NULL, "%s is NULL", name);
  if (!aligned(p, align)) return fail(SSA_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", name, align);
  return SSA_OK;
}

ssa_status check_opt_ptr(const void* p, const char* name, size_t align) {
  if (p && !aligned(p, align)) return fail(SSA_ERR_UNSUPPORTED, "%s is not %zu-byte aligned", name, align);
  return SSA_OK;
}

ssa_status check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(SSA_ERR_UNSUPPORTED, "scale must be finite and > 0");
  return SSA_OK;
}

ssa_status finish(const ssa::LaunchResult& r, const char* what) {
  if (r.unsupported) return fail(SSA_ERR_UNSUPPORTED, "%s: %s", what, r.unsupported);
  if (r.err != hipSuccess) return fail(SSA_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(r.err));
  g_last_error[0] = '\0';
  return SSA_OK;
}

#define SSA_TRY(expr)              \
  do {                             \
    ssa_status _s = (expr);        \
    if (_s != SSA_OK) return _s;   \
  } while (0)

bool use_mfma() { return g_variant.load(std::memory_order_relaxed) == 0; }

}  // namespace

extern "C" {

ssa_status ssa_block_pool(const ssa_dims* dims, const void* k, float* k_mean, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(k, "k", 16));
  SSA_TRY(check_ptr(k_mean, "k_mean", 16));
  SSA_TRY(check_device());
  return finish(ssa::launch_pool(d.kv(), k, k_mean, (hipStream_t)stream), "ssa_block_pool");  // over K/V heads
}

ssa_status ssa_block_topk(const ssa_dims* dims, const void* q, const float* k_mean, int32_t topk, int32_t* idx,
                          float* sel_score, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(q, "q", 16));
  SSA_TRY(check_ptr(k_mean, "k_mean", 16));
  SSA_TRY(check_ptr(idx, "idx", 4));
  SSA_TRY(check_opt_ptr(sel_score, "sel_score", 4));
  if (topk < 1 || topk > d.n()) return fail(SSA_ERR_SHAPE, "topk=%d outside [1, n=%d]", topk, d.n());
  SSA_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  if (d.dtype == SSA_BF16 && use_mfma() && ssa::topk_mfma_supported(d, topk))
    return finish(ssa::launch_topk_mfma(d, q, k_mean, topk, idx, sel_score, st), "ssa_block_topk");
  return finish(ssa::launch_topk_generic(d, q, k_mean, topk, idx, sel_score, st), "ssa_block_topk");
}

}  // extern "C"

namespace {

// ssa_sparse_attn_fwd with (frag) or without the caller's fragment-order copies of k, v.
ssa_status sparse_fwd(const char* what, bool frag, const ssa_dims* dims, const void* q, const void* k, const void* v,
                      const void* k_frag, const void* v_frag, const int32_t* idx, int32_t topk, float scale, void* o,
                      float* lse, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(q, "q", 16));
  SSA_TRY(check_ptr(k, "k", 16));
  SSA_TRY(check_ptr(v, "v", 16));
  if (frag && d.dtype == SSA_BF16) {
    SSA_TRY(check_ptr(k_frag, "k_frag", 16));
    SSA_TRY(check_ptr(v_frag, "v_frag", 16));
  }
  SSA_TRY(check_ptr(idx, "idx", 4));
  SSA_TRY(check_ptr(o, "o", 16));
  SSA_TRY(check_opt_ptr(lse, "lse", 4));
  if (topk < 1 || topk > d.n()) return fail(SSA_ERR_SHAPE, "topk=%d outside [1, n=%d]", topk, d.n());
  SSA_TRY(check_scale(scale));
  SSA_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  if (d.dtype == SSA_BF16 && use_mfma() && ssa::sparse_mfma_supported(d, topk)) {
    if (frag)
      return finish(ssa::launch_sparse_mfma_frag(d, q, k, v, static_cast<const ssa::u32x4*>(k_frag),
                                                 static_cast<const ssa::u32x4*>(v_frag), idx, topk, scale, o, lse, st),
                    what);
    return finish(ssa::launch_sparse_mfma(d, q, k, v, idx, topk, scale, o, lse, st), what);
  }
  return finish(ssa::launch_sparse_generic(d, q, k, v, idx, topk, scale, o, lse, st), what);
}

// ssa_full_attn_fwd with (frag) or without the caller's fragment-order copy of v.
ssa_status full_fwd(const char* what, bool frag, const ssa_dims* dims, const void* q, const void* k, const void* v,
                    const void* v_frag, float scale, void* o, float* lse, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(q, "q", 16));
  SSA_TRY(check_ptr(k, "k", 16));
  SSA_TRY(check_ptr(v, "v", 16));
  if (!o && !lse) return fail(SSA_ERR_NULL, "%s needs o or lse", what);
  if (frag && d.dtype == SSA_BF16 && o) SSA_TRY(check_ptr(v_frag, "v_frag", 16));
  SSA_TRY(check_opt_ptr(o, "o", 16));
  SSA_TRY(check_opt_ptr(lse, "lse", 4));
  SSA_TRY(check_scale(scale));
  SSA_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  if (d.dtype == SSA_BF16 && use_mfma() && ssa::full_mfma_supported(d)) {
    if (frag)
      return finish(ssa::launch_full_mfma_frag(d, q, k, o ? static_cast<const ssa::u32x4*>(v_frag) : nullptr, scale, o,
                                               lse, st),
                    what);
    return finish(ssa::launch_full_mfma(d, q, k, v, scale, o, lse, st), what);
  }
  return finish(ssa::launch_full_generic(d, q, k, v, scale, o, lse, st), what);
}

}  // namespace

extern "C" {

ssa_status ssa_sparse_attn_fwd(const ssa_dims* dims, const void* q, const void* k, const void* v, const int32_t* idx,
                               int32_t topk, float scale, void* o, float* lse, void* stream) {
  return sparse_fwd("ssa_sparse_attn_fwd", false, dims, q, k, v, nullptr, nullptr, idx, topk, scale, o, lse, stream);
}

ssa_status ssa_full_attn_fwd(const ssa_dims* dims, const void* q, const void* k, const void* v, float scale, void* o,
                             float* lse, void* stream) {
  return full_fwd("ssa_full_attn_fwd", false, dims, q, k, v, nullptr, scale, o, lse, stream);
}

ssa_status ssa_sparse_attn_fwd_stats(const ssa_dims* dims, const void* q, const void* k, const void* v,
                                    const int32_t* idx, int32_t topk, float scale, void* o, float* lse,
                                    float* entropy, float* dist_hist, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(q, "q", 16));
  SSA_TRY(check_ptr(k, "k", 16));
  SSA_TRY(check_ptr(v, "v", 16));
  SSA_TRY(check_ptr(idx, "idx", 4));
  SSA_TRY(check_ptr(o, "o", 16));
  SSA_TRY(check_opt_ptr(lse, "lse", 4));
  if (!entropy && !dist_hist) return fail(SSA_ERR_NULL, "ssa_sparse_attn_fwd_stats needs entropy or dist_hist");
  SSA_TRY(check_opt_ptr(entropy, "entropy", 4));
  SSA_TRY(check_opt_ptr(dist_hist, "dist_hist", 4));
  if (topk < 1 || topk > d.n()) return fail(SSA_ERR_SHAPE, "topk=%d outside [1, n=%d]", topk, d.n());
  SSA_TRY(check_scale(scale));
  SSA_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  const bool mfma = d.dtype == SSA_BF16 && use_mfma();
  if (mfma && ssa::sparse_mfma_stats_supported(d, topk))
    return finish(ssa::launch_sparse_mfma_stats(d, q, k, v, idx, topk, scale, o, lse, entropy, dist_hist, st),
                  "ssa_sparse_attn_fwd_stats");
  return finish(ssa::launch_sparse_stats_unfused(d, mfma, q, k, v, idx, topk, scale, o, lse, entropy, dist_hist, st),
                "ssa_sparse_attn_fwd_stats");
}

ssa_status ssa_kv_frag_bytes(const ssa_dims* dims, int64_t* bytes) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  if (!bytes) return fail(SSA_ERR_NULL, "bytes is NULL");
  *bytes = d.dtype == SSA_BF16 ? (int64_t)d.B * d.Hkv * d.L * d.D * 2 : 0;
  g_last_error[0] = '\0';
  return SSA_OK;
}

ssa_status ssa_kv_frag(const ssa_dims* dims, const void* k, const void* v, void* k_frag, void* v_frag, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  if (d.dtype != SSA_BF16) return fail(SSA_ERR_DTYPE, "ssa_kv_frag: the fragment-order copies exist for bf16 only");
  if (!k_frag && !v_frag) return fail(SSA_ERR_NULL, "ssa_kv_frag needs k_frag or v_frag");
  if (k_frag) {
    SSA_TRY(check_ptr(k, "k", 16));
    SSA_TRY(check_ptr(k_frag, "k_frag", 16));
  }
  if (v_frag) {
    SSA_TRY(check_ptr(v, "v", 16));
    SSA_TRY(check_ptr(v_frag, "v_frag", 16));
  }
  SSA_TRY(check_device());
  ssa::LaunchResult r;
  r.err = ssa::kv_frag_into(d.kv(), k, v, k_frag, v_frag, (hipStream_t)stream);
  return finish(r, "ssa_kv_frag");
}

ssa_status ssa_sparse_attn_fwd_frag(const ssa_dims* dims, const void* q, const void* k, const void* v,
                                    const void* k_frag, const void* v_frag, const int32_t* idx, int32_t topk,
                                    float scale, void* o, float* lse, void* stream) {
  return sparse_fwd("ssa_sparse_attn_fwd_frag", true, dims, q, k, v, k_frag, v_frag, idx, topk, scale, o, lse, stream);
}

ssa_status ssa_full_attn_fwd_frag(const ssa_dims* dims, const void* q, const void* k, const void* v,
                                  const void* v_frag, float scale, void* o, float* lse, void* stream) {
  return full_fwd("ssa_full_attn_fwd_frag", true, dims, q, k, v, v_frag, scale, o, lse, stream);
}

ssa_status ssa_full_attn_fwd_stats(const ssa_dims* dims, const void* q, const void* k, const void* v, float scale,
                                   void* o, float* lse, float* entropy, float* dist_hist, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(q, "q", 16));
  SSA_TRY(check_ptr(k, "k", 16));
  SSA_TRY(check_ptr(v, "v", 16));
  if (!entropy && !dist_hist) return fail(SSA_ERR_NULL, "ssa_full_attn_fwd_stats needs entropy or dist_hist");
  SSA_TRY(check_opt_ptr(o, "o", 16));
  SSA_TRY(check_opt_ptr(lse, "lse", 4));
  SSA_TRY(check_opt_ptr(entropy, "entropy", 4));
  SSA_TRY(check_opt_ptr(dist_hist, "dist_hist", 4));
  SSA_TRY(check_scale(scale));
  SSA_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  if (d.dtype == SSA_BF16 && use_mfma() && ssa::full_mfma_supported(d))
    return finish(ssa::launch_full_mfma_stats(d, q, k, v, scale, o, lse, entropy, dist_hist, st),
                  "ssa_full_attn_fwd_stats");
  return finish(ssa::launch_full_stats_unfused(d, q, k, v, scale, o, lse, entropy, dist_hist, st),
                "ssa_full_attn_fwd_stats");
}

ssa_status ssa_align_stats(const ssa_dims* dims, const void* o_full, const void* o_sparse, const float* lse_full,
                           const float* lse_sparse, float* l2_dist, float* dropped, void* stream) {
  return ssa_align_stats_hist(dims, o_full, o_sparse, lse_full, lse_sparse, l2_dist, dropped, nullptr, stream);
}

ssa_status ssa_align_stats_hist(const ssa_dims* dims, const void* o_full, const void* o_sparse,
                                const float* lse_full, const float* lse_sparse, float* l2_dist, float* dropped,
                                float* retained_hist, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d, false));
  if (!l2_dist && !dropped && !retained_hist)
    return fail(SSA_ERR_NULL, "ssa_align_stats needs l2_dist, dropped or retained_hist");
  if (retained_hist) {
    SSA_TRY(check_ptr(lse_full, "lse_full", 4));
    SSA_TRY(check_ptr(lse_sparse, "lse_sparse", 4));
    SSA_TRY(check_ptr(retained_hist, "retained_hist", 4));
    if (d.L % 64) return fail(SSA_ERR_SHAPE, "retained_hist needs L %% 64 == 0 (got L=%d)", d.L);
  }
  if (l2_dist) {
    SSA_TRY(check_ptr(o_full, "o_full", 16));
    SSA_TRY(check_ptr(o_sparse, "o_sparse", 16));
    SSA_TRY(check_ptr(l2_dist, "l2_dist", 4));
  }
  if (dropped) {
    SSA_TRY(check_ptr(lse_full, "lse_full", 4));
    SSA_TRY(check_ptr(lse_sparse, "lse_sparse", 4));
    SSA_TRY(check_ptr(dropped, "dropped", 4));
  }
  SSA_TRY(check_device());
  return finish(ssa::launch_align(d, o_full, o_sparse, lse_full, lse_sparse, l2_dist, dropped, (hipStream_t)stream,
                                  retained_hist),
                "ssa_align_stats");
}

ssa_status ssa_decode_append(const ssa_dims* dims, const int32_t* pos, const void* k_new, const void* v_new,
                             void* k_cache, void* v_cache, float* k_mean, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(pos, "pos", 4));
  SSA_TRY(check_ptr(k_new, "k_new", 16));
  SSA_TRY(check_ptr(v_new, "v_new", 16));
  SSA_TRY(check_ptr(k_cache, "k_cache", 16));
  SSA_TRY(check_ptr(v_cache, "v_cache", 16));
  SSA_TRY(check_ptr(k_mean, "k_mean", 16));
  SSA_TRY(check_device());
  return finish(ssa::launch_decode_append(d, pos, k_new, v_new, k_cache, v_cache, k_mean, (hipStream_t)stream),
                "ssa_decode_append");
}

ssa_status ssa_decode_sparse_fwd(const ssa_dims* dims, const int32_t* pos, const void* q, const void* k_cache,
                                 const void* v_cache, const float* k_mean, int32_t topk, float scale, void* o,
                                 float* lse, int32_t* idx, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(pos, "pos", 4));
  SSA_TRY(check_ptr(q, "q", 16));
  SSA_TRY(check_ptr(k_cache, "k_cache", 16));
  SSA_TRY(check_ptr(v_cache, "v_cache", 16));
  SSA_TRY(check_ptr(k_mean, "k_mean", 16));
  SSA_TRY(check_ptr(o, "o", 16));
  SSA_TRY(check_opt_ptr(lse, "lse", 4));
  SSA_TRY(check_opt_ptr(idx, "idx", 4));
  if (topk < 1 || topk > d.n()) return fail(SSA_ERR_SHAPE, "topk=%d outside [1, n=%d]", topk, d.n());
  SSA_TRY(check_scale(scale));
  SSA_TRY(check_device());
  return finish(ssa::launch_decode_sparse(d, pos, q, k_cache, v_cache, k_mean, topk, scale, o, lse, idx,
                                          (hipStream_t)stream),
                "ssa_decode_sparse_fwd");
}

ssa_status ssa_decode_sparse_fwd_noalloc(const ssa_dims* dims, const int32_t* pos, const void* q,
                                         const void* k_cache, const void* v_cache, const float* k_mean, int32_t topk,
                                         float scale, void* o, float* lse, int32_t* idx, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(pos, "pos", 4));
  SSA_TRY(check_ptr(q, "q", 16));
  SSA_TRY(check_ptr(k_cache, "k_cache", 16));
  SSA_TRY(check_ptr(v_cache, "v_cache", 16));
  SSA_TRY(check_ptr(k_mean, "k_mean", 16));
  SSA_TRY(check_ptr(o, "o", 16));
  SSA_TRY(check_opt_ptr(lse, "lse", 4));
  SSA_TRY(check_opt_ptr(idx, "idx", 4));
  if (topk < 1 || topk > d.n()) return fail(SSA_ERR_SHAPE, "topk=%d outside [1, n=%d]", topk, d.n());
  SSA_TRY(check_scale(scale));
  const size_t need = ssa::decode_sparse_scratch_bytes(d, topk, idx != nullptr);
  if (need > ssa::kDecodeScratchMax)
    return fail(SSA_ERR_SHAPE, "ssa_decode_sparse_fwd_noalloc: needs %zu bytes of scratch, above its %zu-byte limit",
                need, ssa::kDecodeScratchMax);
  SSA_TRY(check_device());
  return finish(ssa::launch_decode_sparse_noalloc(d, pos, q, k_cache, v_cache, k_mean, topk, scale, o, lse, idx,
                                                  (hipStream_t)stream),
                "ssa_decode_sparse_fwd_noalloc");
}

ssa_status ssa_decode_full_fwd(const ssa_dims* dims, const int32_t* pos, const void* q, const void* k_cache,
                               const void* v_cache, float scale, void* o, float* lse, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(pos, "pos", 4));
  SSA_TRY(check_ptr(q, "q", 16));
  SSA_TRY(check_ptr(k_cache, "k_cache", 16));
  if (!o && !lse) return fail(SSA_ERR_NULL, "ssa_decode_full_fwd needs o or lse");
  if (o) SSA_TRY(check_ptr(v_cache, "v_cache", 16));
  SSA_TRY(check_opt_ptr(o, "o", 16));
  SSA_TRY(check_opt_ptr(lse, "lse", 4));
  SSA_TRY(check_scale(scale));
  SSA_TRY(check_device());
  return finish(ssa::launch_decode_full(d, pos, q, k_cache, v_cache, scale, o, lse, (hipStream_t)stream),
                "ssa_decode_full_fwd");
}

static ssa_status attn_bwd(const char* what, bool sparse, const ssa_dims* dims, const void* q, const void* k,
                           const void* v, const void* o, const float* lse, const void* dout, const int32_t* idx,
                           int32_t topk, float scale, float* dq, float* dk, float* dv, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(q, "q", 16));
  SSA_TRY(check_ptr(k, "k", 16));
  SSA_TRY(check_ptr(v, "v", 16));
  SSA_TRY(check_ptr(o, "o", 16));
  SSA_TRY(check_ptr(lse, "lse", 4));
  SSA_TRY(check_ptr(dout, "dout", 16));
  SSA_TRY(check_ptr(dq, "dq", 16));
  SSA_TRY(check_ptr(dk, "dk", 16));
  SSA_TRY(check_ptr(dv, "dv", 16));
  if (sparse) {
    SSA_TRY(check_ptr(idx, "idx", 4));
    if (topk < 1 || topk > d.n()) return fail(SSA_ERR_SHAPE, "topk=%d outside [1, n=%d]", topk, d.n());
  }
  SSA_TRY(check_scale(scale));
  SSA_TRY(check_device());
  return finish(ssa::launch_attn_bwd(d, sparse, use_mfma(), q, k, v, o, lse, dout, idx, sparse ? topk : 1, scale,
                                     dq, dk, dv, (hipStream_t)stream),
                what);
}

ssa_status ssa_full_attn_bwd(const ssa_dims* dims, const void* q, const void* k, const void* v, const void* o,
                             const float* lse, const void* dout, float scale, float* dq, float* dk, float* dv,
                             void* stream) {
  return attn_bwd("ssa_full_attn_bwd", false, dims, q, k, v, o, lse, dout, nullptr, 1, scale, dq, dk, dv, stream);
}

ssa_status ssa_sparse_attn_bwd(const ssa_dims* dims, const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, const int32_t* idx, int32_t topk, float scale,
                               float* dq, float* dk, float* dv, void* stream) {
  return attn_bwd("ssa_sparse_attn_bwd", true, dims, q, k, v, o, lse, dout, idx, topk, scale, dq, dk, dv, stream);
}

ssa_status ssa_attn_stats(const ssa_dims* dims, const void* q, const void* k, const float* lse, const int32_t* idx,
                          int32_t topk, float scale, float* entropy, float* dist_hist, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d));
  SSA_TRY(check_ptr(q, "q", 16));
  SSA_TRY(check_ptr(k, "k", 16));
  SSA_TRY(check_ptr(lse, "lse", 4));
  if (!entropy && !dist_hist) return fail(SSA_ERR_NULL, "ssa_attn_stats needs entropy or dist_hist");
  SSA_TRY(check_opt_ptr(entropy, "entropy", 4));
  SSA_TRY(check_opt_ptr(dist_hist, "dist_hist", 4));
  SSA_TRY(check_opt_ptr(idx, "idx", 4));
  if (idx && (topk < 1 || topk > d.n())) return fail(SSA_ERR_SHAPE, "topk=%d outside [1, n=%d]", topk, d.n());
  SSA_TRY(check_scale(scale));
  SSA_TRY(check_device());
  return finish(ssa::launch_attn_stats(d, use_mfma(), q, k, lse, idx, idx ? topk : 1, scale, entropy, dist_hist,
                                       (hipStream_t)stream),
                "ssa_attn_stats");
}

ssa_status ssa_align_loss(const ssa_dims* dims, const void* o_full, const void* o_sparse, float alpha, float beta,
                          float* loss, float* grad_full, float* grad_sparse, void* stream) {
  ssa::Dims d;
  SSA_TRY(check_dims(dims, &d, false));
  SSA_TRY(check_ptr(o_full, "o_full", 16));
  SSA_TRY(check_ptr(o_sparse, "o_sparse", 16));
  SSA_TRY(check_ptr(loss, "loss", 4));
  SSA_TRY(check_opt_ptr(grad_full, "grad_full", 16));
  SSA_TRY(check_opt_ptr(grad_sparse, "grad_sparse", 16));
  if (!std::isfinite(alpha) || !std::isfinite(beta) || !(beta > 0.f))
    return fail(SSA_ERR_UNSUPPORTED, "alpha must be finite and beta finite and > 0");
  SSA_TRY(check_device());
  return finish(ssa::launch_align_loss(d, o_full, o_sparse, alpha, beta, loss, grad_full, grad_sparse,
                                       (hipStream_t)stream),
                "ssa_align_loss");
}

const char* ssa_status_str(ssa_status s) {
  switch (s) {
    case SSA_OK: return "SSA_OK";
    case SSA_ERR_NULL: return "SSA_ERR_NULL";
    case SSA_ERR_SHAPE: return "SSA_ERR_SHAPE";
    case SSA_ERR_DTYPE: return "SSA_ERR_DTYPE";
    case SSA_ERR_UNSUPPORTED: return "SSA_ERR_UNSUPPORTED";
    case SSA_ERR_DEVICE: return "SSA_ERR_DEVICE";
    case SSA_ERR_LAUNCH: return "SSA_ERR_LAUNCH";
    default: return "SSA_ERR_UNKNOWN";
  }
}

const char* ssa_last_error(void) { return g_last_error; }

int32_t ssa_abi_version(void) { return SSA_ABI_VERSION; }

int32_t ssa_set_kernel_variant(int32_t variant) { return g_variant.exchange(variant == 1 ? 1 : 0); }

}  // extern "C"
