// Token-level pre-gating kernel (AdaFuse, technical summary §2.A; §2.B decoding
// steps 1-2): one workgroup per tile of TT tokens; the arithmetic lives in
// route_common.h and is shared with the fused route-and-project launch.
#include "route_common.h"

namespace rp {
namespace {

template <typename Tin, int TT, int NT>
__global__ __launch_bounds__(NT) void pregate_kernel(PregateArgs a, RoutePlan p) {
  extern __shared__ float smem[];
  route_tile<Tin, TT, NT>(a, blockIdx.x * TT, p, smem);
}

template <typename Tin>
hipError_t launch_t(const PregateArgs& a, hipStream_t s) {
  const RoutePlan p = route_plan(a.E, a.d_in, (int)sizeof(Tin));
  const size_t lds = sizeof(float) * route_lds_floats(p, a.E, p.TT);
  if (p.NT == kRouteThreads) {
    if (p.TT == 4)
      pregate_kernel<Tin, 4, kRouteThreads><<<(a.T + 3) / 4, kRouteThreads, lds, s>>>(a, p);
    else
      pregate_kernel<Tin, 2, kRouteThreads><<<(a.T + 1) / 2, kRouteThreads, lds, s>>>(a, p);
  } else {
    if (p.TT == 4)
      pregate_kernel<Tin, 4, kRouteThreadsWide><<<(a.T + 3) / 4, kRouteThreadsWide, lds, s>>>(a, p);
    else
      pregate_kernel<Tin, 2, kRouteThreadsWide><<<(a.T + 1) / 2, kRouteThreadsWide, lds, s>>>(a, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pregate(const PregateArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return a.dt == kBF16 ? launch_t<bf16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace rp
