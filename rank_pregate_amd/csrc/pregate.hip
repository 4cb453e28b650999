// Token-level pre-gating kernel (AdaFuse, technical summary §2.A; §2.B decoding
// steps 1-2): one workgroup per tile of TT tokens; the arithmetic lives in
// route_common.h and is shared with the fused route-and-project launch.  bf16
// routers with more than 64 columns (a multiple of 8) run on the matrix cores
// instead (route_mfma.hip).
#include <algorithm>

#include "route_common.h"

namespace rp {
namespace {

template <typename Tin, int TT, int NT>
__global__ __launch_bounds__(NT) void pregate_kernel(PregateArgs a, RoutePlan p) {
  extern __shared__ float smem[];
  route_tile<Tin, TT, NT>(a, blockIdx.x * TT, p, smem);
}

// Fewer tokens per tile while that still leaves tiles for every CU: a tile
// reads the whole router weight, so small batches are spread wide.  The
// summation order of a logit does not depend on the tile size.
constexpr int kRouteFillTiles = 256;

template <typename Tin, int NT>
void launch_nt(const PregateArgs& a, const RoutePlan& p, hipStream_t s) {
  constexpr int kMaxTT = NT <= 512 ? 4 : 2;  // wider tiles hold at most two tokens
  const int TT = std::min(kMaxTT, a.T <= kRouteFillTiles ? 1 : a.T <= 2 * kRouteFillTiles ? 2 : p.TT);
  const size_t lds = sizeof(float) * route_lds_floats(p, a.E, TT);
  if (TT == 1)
    pregate_kernel<Tin, 1, NT><<<a.T, NT, lds, s>>>(a, p);
  else if (TT == 2 || kMaxTT == 2)
    pregate_kernel<Tin, 2, NT><<<(a.T + 1) / 2, NT, lds, s>>>(a, p);
  else
    pregate_kernel<Tin, kMaxTT, NT><<<(a.T + 3) / 4, NT, lds, s>>>(a, p);
}

template <typename Tin>
hipError_t launch_t(const PregateArgs& a, hipStream_t s) {
  const RoutePlan p = route_plan(a.E, a.d_in, (int)sizeof(Tin));
  if (p.NT == kRouteThreads)
    launch_nt<Tin, kRouteThreads>(a, p, s);
  else
    launch_nt<Tin, kRouteThreadsWide>(a, p, s);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pregate(const PregateArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (mfma_router_supported(a.dt, a.E)) return launch_route_mfma(a, s);
  return a.dt == kBF16 ? launch_t<bf16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace rp
