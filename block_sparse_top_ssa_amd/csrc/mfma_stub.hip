#include "launch.hpp"
namespace ssa {
bool topk_mfma_supported(const Dims&, int) { return false; }
LaunchResult launch_topk_mfma(const Dims&, const void*, const float*, int, int32_t*, float*, hipStream_t) { return {}; }
}
