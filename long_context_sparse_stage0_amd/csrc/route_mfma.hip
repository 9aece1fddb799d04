// Stage 1 routing on bf16 MFMA: the launches of the forward (kernel templates and the
// launch-shape table in route_mfma.h).  When the caller asks for each head's threshold
// and normaliser (the backward pass's recompute), the instances that keep them are
// launched instead; they live in route_mfma_keep.hip so both compile in parallel.
#include "route_mfma.h"

namespace dash {

hipError_t launch_route_mfma_keep(const RouteArgs& a, const void* summ_split, hipStream_t s);

hipError_t launch_route_mfma(const RouteArgs& a, const void* summ_split, hipStream_t s) {
  if (a.tau_out != nullptr && a.topk == 0) return launch_route_mfma_keep(a, summ_split, s);
  if (a.D == 128) launch_d<128, false>(a, (const bf16*)summ_split, s);
  else launch_d<64, false>(a, (const bf16*)summ_split, s);
  return hipGetLastError();
}

}  // namespace dash
