// Segmentation kernel: one workgroup of 16 waves groups the (token, slot)
// pairs by adapter (the segments of the segmented gather matrix multiply,
// AdaFuse technical summary §2.B).  The algorithm is segment_block in
// route_common.h, shared with the fused route-and-project launch.
#include "route_common.h"

namespace rp {
namespace {

constexpr int kWaves = 16;

__global__ __launch_bounds__(kWaves * 64) void segment_kernel(SegmentArgs a) {
  __shared__ int hist[kWaves * kMaxE];
  __shared__ int wave_tot[kWaves];
  __shared__ int bad;
  segment_block<kWaves>(a, hist, wave_tot, &bad);
}

}  // namespace

hipError_t launch_segment(const SegmentArgs& a, hipStream_t s) {
  segment_kernel<<<1, kWaves * 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace rp
