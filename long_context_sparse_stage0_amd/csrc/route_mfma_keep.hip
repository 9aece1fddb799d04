// Stage 1 routing on bf16 MFMA, the instances that also keep each head's entmax threshold
// and normaliser for the backward pass (kernel templates in route_mfma.h).
#include "route_mfma.h"

namespace dash {

hipError_t launch_route_mfma_keep(const RouteArgs& a, const void* summ_split, hipStream_t s) {
  if (a.D == 128) launch_d<128, true>(a, (const bf16*)summ_split, s);
  else launch_d<64, true>(a, (const bf16*)summ_split, s);
  return hipGetLastError();
}

}  // namespace dash
