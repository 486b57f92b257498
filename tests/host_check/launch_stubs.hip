// Stand-ins for the kernel launchers of libssa, linked with csrc/api.hip alone into the
// host-sanitizer build of the C ABI's argument checks.  On a host without a GPU every call
// stops at an argument check or at the device check, so no launcher runs; if one ever
// does, it refuses the shape instead of launching anything.  The decoding scratch size is
// reported as unbounded, so the allocation-free decoding call refuses every shape at its
// scratch check (which comes after its argument checks).
#include "../../block_sparse_top_ssa_amd/csrc/launch.hpp"

namespace ssa {
namespace {
LaunchResult refused() {
  LaunchResult r;
  r.unsupported = "host-check build: no kernels linked";
  return r;
}
}  // namespace

LaunchResult launch_pool(const Dims&, const void*, float*, hipStream_t) { return refused(); }
LaunchResult launch_align(const Dims&, const void*, const void*, const float*, const float*, float*, float*,
                          hipStream_t, float*) {
  return refused();
}
LaunchResult launch_topk_generic(const Dims&, const void*, const float*, int, int32_t*, float*, hipStream_t) {
  return refused();
}
LaunchResult launch_sparse_generic(const Dims&, const void*, const void*, const void*, const int32_t*, int, float,
                                   void*, float*, hipStream_t) {
  return refused();
}
LaunchResult launch_full_generic(const Dims&, const void*, const void*, const void*, float, void*, float*,
                                 hipStream_t) {
  return refused();
}
LaunchResult launch_decode_append(const Dims&, const int32_t*, const void*, const void*, void*, void*, float*,
                                  hipStream_t) {
  return refused();
}
LaunchResult launch_decode_sparse(const Dims&, const int32_t*, const void*, const void*, const void*, const float*,
                                  int, float, void*, float*, int32_t*, hipStream_t) {
  return refused();
}
size_t decode_sparse_scratch_bytes(const Dims&, int, bool) { return SIZE_MAX; }
LaunchResult launch_decode_sparse_noalloc(const Dims&, const int32_t*, const void*, const void*, const void*,
                                          const float*, int, float, void*, float*, int32_t*, hipStream_t) {
  return refused();
}
LaunchResult launch_decode_full(const Dims&, const int32_t*, const void*, const void*, const void*, float, void*,
                                float*, hipStream_t) {
  return refused();
}
LaunchResult launch_attn_bwd(const Dims&, bool, bool, const void*, const void*, const void*, const void*,
                             const float*, const void*, const int32_t*, int, float, float*, float*, float*,
                             hipStream_t) {
  return refused();
}
LaunchResult launch_attn_stats(const Dims&, bool, const void*, const void*, const float*, const int32_t*, int,
                               float, float*, float*, hipStream_t) {
  return refused();
}
LaunchResult launch_align_loss(const Dims&, const void*, const void*, float, float, float*, float*, float*,
                               hipStream_t) {
  return refused();
}
bool topk_mfma_supported(const Dims&, int) { return false; }
LaunchResult launch_topk_mfma(const Dims&, const void*, const float*, int, int32_t*, float*, hipStream_t) {
  return refused();
}
bool full_mfma_supported(const Dims&) { return false; }
LaunchResult launch_full_mfma(const Dims&, const void*, const void*, const void*, float, void*, float*,
                              hipStream_t) {
  return refused();
}
LaunchResult launch_full_mfma_stats(const Dims&, const void*, const void*, const void*, float, void*, float*, float*,
                                    float*, hipStream_t) {
  return refused();
}
LaunchResult launch_full_stats_unfused(const Dims&, const void*, const void*, const void*, float, void*, float*,
                                       float*, float*, hipStream_t) {
  return refused();
}
bool sparse_mfma_supported(const Dims&, int) { return false; }
LaunchResult launch_sparse_mfma(const Dims&, const void*, const void*, const void*, const int32_t*, int, float,
                                void*, float*, hipStream_t) {
  return refused();
}
LaunchResult launch_sparse_mfma_frag(const Dims&, const void*, const void*, const void*, const u32x4*,
                                     const u32x4*, const int32_t*, int, float, void*, float*, hipStream_t) {
  return refused();
}
LaunchResult launch_full_mfma_frag(const Dims&, const void*, const void*, const u32x4*, float, void*, float*,
                                   hipStream_t) {
  return refused();
}
bool sparse_mfma_stats_supported(const Dims&, int) { return false; }
LaunchResult launch_sparse_mfma_stats(const Dims&, const void*, const void*, const void*, const int32_t*, int, float,
                                      void*, float*, float*, float*, hipStream_t) {
  return refused();
}
LaunchResult launch_sparse_stats_unfused(const Dims&, bool, const void*, const void*, const void*, const int32_t*, int,
                                         float, void*, float*, float*, float*, hipStream_t) {
  return refused();
}
hipError_t kv_frag_into(const Dims&, const void*, const void*, void*, void*, hipStream_t) {
  return hipErrorInvalidValue;
}

}  // namespace ssa
