// Explicit instantiation: io dtype __bf16, chunk 32, K = V = 128, both gate forms, both passes and the fused reverse backward.
#include "gdr_launch.hpp"
namespace gdr {
template hipError_t launch_bwd<__bf16, 32, 128, false>(const Params&, hipStream_t, hipEvent_t const*);
template hipError_t launch_fwd<__bf16, 32, 128, false>(const Params&, hipStream_t, hipEvent_t const*);
template hipError_t launch_bwd<__bf16, 32, 128, true>(const Params&, hipStream_t, hipEvent_t const*);
template hipError_t launch_fwd<__bf16, 32, 128, true>(const Params&, hipStream_t, hipEvent_t const*);
template hipError_t launch_fused<__bf16, 32, 128, false>(const Params&, hipStream_t, hipEvent_t const*);
template hipError_t launch_fused<__bf16, 32, 128, true>(const Params&, hipStream_t, hipEvent_t const*);
}  // namespace gdr
