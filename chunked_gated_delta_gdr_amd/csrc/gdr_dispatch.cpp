// gdr_dispatch.cpp -- maps (io dtype, chunk, K = V, gate form) to the launcher
// instantiated for it in gdr_inst_*.hip.
#include "gdr_launch.hpp"

namespace gdr {

#define GDR_DECL(T, C, D)                                                         \
    extern template hipError_t launch_bwd<T, C, D, false>(const Params&, hipStream_t, hipEvent_t const*); \
    extern template hipError_t launch_bwd<T, C, D, true>(const Params&, hipStream_t, hipEvent_t const*);  \
    extern template hipError_t launch_fwd<T, C, D, false>(const Params&, hipStream_t, hipEvent_t const*); \
    extern template hipError_t launch_fwd<T, C, D, true>(const Params&, hipStream_t, hipEvent_t const*);
#define GDR_DECL_F(T, D)                                                         \
    extern template hipError_t launch_fused<T, 32, D, false>(const Params&, hipStream_t, hipEvent_t const*); \
    extern template hipError_t launch_fused<T, 32, D, true>(const Params&, hipStream_t, hipEvent_t const*);
#define GDR_DECL_T(T) GDR_DECL(T, 32, 64) GDR_DECL(T, 32, 128) GDR_DECL(T, 64, 64) GDR_DECL(T, 64, 128)
GDR_DECL(float, 32, 64)
GDR_DECL(float, 64, 64)
GDR_DECL_T(__bf16)
GDR_DECL_T(_Float16)
GDR_DECL_F(float, 64)
GDR_DECL_F(__bf16, 64)
GDR_DECL_F(__bf16, 128)
GDR_DECL_F(_Float16, 64)
GDR_DECL_F(_Float16, 128)

#define GDR_CASE(T, C, D)                                                                         \
    if (chunk == C && dim == D && pass < 2)                                                       \
        return pass ? (scalar ? &launch_fwd<T, C, D, true> : &launch_fwd<T, C, D, false>)         \
                    : (scalar ? &launch_bwd<T, C, D, true> : &launch_bwd<T, C, D, false>);
// the fused reverse backward is built for chunk 32 only
#define GDR_CASE_F(T, D)                                                                          \
    if (chunk == 32 && dim == D && pass == 2)                                                     \
        return scalar ? &launch_fused<T, 32, D, true> : &launch_fused<T, 32, D, false>;

template <typename T>
static LaunchFn pick(int chunk, int dim, int scalar, int pass) {
    GDR_CASE(T, 32, 64) GDR_CASE(T, 32, 128) GDR_CASE(T, 64, 64) GDR_CASE(T, 64, 128)
    GDR_CASE_F(T, 64) GDR_CASE_F(T, 128)
    return nullptr;
}

// fp32 io (full-precision operands) is built for K = V = 64 only: its LDS
// tiles are twice as large and K = 128 does not fit the 160 KB of a CU.
template <>
LaunchFn pick<float>(int chunk, int dim, int scalar, int pass) {
    GDR_CASE(float, 32, 64) GDR_CASE(float, 64, 64)
    GDR_CASE_F(float, 64)
    return nullptr;
}
#undef GDR_CASE
#undef GDR_CASE_F

LaunchFn find_launcher(int io_dtype, int chunk, int dim, int scalar, int pass) {
    switch (io_dtype) {
        case 0: return pick<float>(chunk, dim, scalar, pass);
        case 1: return pick<__bf16>(chunk, dim, scalar, pass);
        case 2: return pick<_Float16>(chunk, dim, scalar, pass);
        default: return nullptr;
    }
}

}  // namespace gdr
