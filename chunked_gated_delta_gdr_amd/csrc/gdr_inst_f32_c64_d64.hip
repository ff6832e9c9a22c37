// Explicit instantiation: io dtype float, chunk 64, K = V = 64, both gate forms, both passes.
#include "gdr_launch.hpp"
namespace gdr {
template hipError_t launch_bwd<float, 64, 64, false>(const Params&, hipStream_t, hipEvent_t const*);
template hipError_t launch_fwd<float, 64, 64, false>(const Params&, hipStream_t, hipEvent_t const*);
template hipError_t launch_bwd<float, 64, 64, true>(const Params&, hipStream_t, hipEvent_t const*);
template hipError_t launch_fwd<float, 64, 64, true>(const Params&, hipStream_t, hipEvent_t const*);
}  // namespace gdr
