// gdr_launch.hpp -- enqueues the four kernels of one backward pass on a stream.
#pragma once
#include "gdr_chunk_bwd.hpp"
#include "gdr_fwd_out.hpp"
#include "gdr_prep.hpp"
#include "gdr_states.hpp"
#include "gdr_sweep.hpp"
#include "gdr_sweep_ws.hpp"

namespace gdr {

// ev: NULL, or GDR_STAGE_EVENTS hipEvent_t recorded on `stream` before the
// first kernel and after each of the four kernels.
using LaunchFn = hipError_t (*)(const Params&, hipStream_t, hipEvent_t const* ev);

// V columns of the state per sweep workgroup (chosen per launch, below): 32;
// 16 for one direction at C = 64, so that a single sweep still has a workgroup
// on every CU (each one moving fewer bytes per step); 64 when there are enough
// (sequence, head) pairs to fill the CUs twice over with 32-column tiles
constexpr int kSweepBV = 32, kSweepBV1 = 16, kSweepBVW = 64;


// Compute units of the current device (queried once per device).
inline int compute_units() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Chunk table, per-chunk preparation and the state sweep(s) (p.dirs of them,
// from direction p.dir0): the start of both passes. A backward after the
// forward pass (p.dir0 == 1) finds the factors, h and X in the workspace and
// runs the reverse sweep only; it rebuilds the chunk table all the same, so
// that every index the kernels use comes from cu_seqlens and the shapes, not
// from workspace contents. A backward from caller-supplied per-chunk states
// (p.hsrc, p.dir0 == 1) runs the preparation, then the chunk-parallel states
// kernel in place of the forward sweep, then the reverse sweep. ev as above
// (entries 0..3).
template <typename T, int C, int D, bool SCALAR>
hipError_t launch_front(const Params& p, hipStream_t stream, hipEvent_t const* ev) {
    auto mark = [&](int i) -> hipError_t { return ev ? hipEventRecord(ev[i], stream) : hipSuccess; };
    hipError_t e = mark(0);
    // chunk table (device-side, so varlen needs no host sync)
    gdr_chunk_table<C><<<dim3(1), dim3(256), 0, stream>>>(p);
    if (e == hipSuccess) e = mark(1);
    // V tile of the sweep: 64 columns when 32-column tiles would need two or
    // more rounds of the CUs (each workgroup then loads the chunk operands once
    // for twice the columns); else 16 for a single direction at C = 64 (one
    // round either way, fewer bytes per workgroup); else 32. The preparation
    // stores k~^T and w^T when the sweeps do not form them themselves (which
    // depends on the operand type and K only, so a backward after a forward
    // pass finds what its sweep needs).
    const int tiles32 = p.dirs * p.N * p.H * (D / kSweepBV);
    const bool wide = tiles32 >= 2 * compute_units();
    constexpr bool store_a2t = !sweep_transposes_a2<T, C, D, kSweepBV>();
    static_assert(sweep_transposes_a2<T, C, D, kSweepBV>() == sweep_transposes_a2<T, C, D, kSweepBV1>() &&
                      sweep_transposes_a2<T, C, D, kSweepBV>() == sweep_transposes_a2<T, C, D, kSweepBVW>(),
                  "sweeps of every tile width take the same operands");
    if ((p.dir0 == 0 || p.hsrc) && p.nc_max > 0) {
        // persistent: as many workgroups as the CUs hold at once
        const int items = p.nc_max * p.H, slots = compute_units() * resident_per_cu<T, C>();
        const dim3 grid(items < slots ? items : slots), block(128 * (C / 16));
        gdr_prep<T, C, D, SCALAR, store_a2t><<<grid, block, 0, stream>>>(p);
    }
    if (e == hipSuccess) e = mark(2);
    if (p.hsrc && p.nc_max > 0) {   // X and the tiled h from the caller's states
        const dim3 grid(p.nc_max, p.H, D / kTileV);
        if (p.vfirst) gdr_states_in<T, C, D, true><<<grid, dim3(256), 0, stream>>>(p);
        else gdr_states_in<T, C, D, false><<<grid, dim3(256), 0, stream>>>(p);
    }
    if (wide) {
        // refills spread over the step (measured: C = 64 with one set of
        // operands in flight 400 -> 363 us varlen; C = 32 878 -> 866 us GDN GQA)
        if constexpr (sizeof(T) == 2 && D == 128)   // loader waves (GDN GQA sweep 889 -> 876 us, varlen 363 -> 350 us)
            gdr_sweep_ws<T, C, D, kSweepBVW><<<dim3(p.dirs * p.N * p.H * (D / kSweepBVW)), dim3(512), 0, stream>>>(p);
        else
            gdr_sweep<T, C, D, kSweepBVW, true><<<dim3(p.dirs * p.N * p.H * (D / kSweepBVW)), dim3(256), 0, stream>>>(p);
    } else {
        bool narrow = false;
        if constexpr (C == 64) {
            narrow = p.dirs == 1;
            // refills spread over the step (forward pass 0.215 -> 0.213 ms headline)
            if (narrow) gdr_sweep<T, C, D, kSweepBV1, true><<<dim3(p.N * p.H * (D / kSweepBV1)), dim3(256), 0, stream>>>(p);
        }
        if (!narrow) {
            if constexpr (sizeof(T) == 2 && C == 64 && D == 128) {
                // loader waves (headline sweep 121.1 -> 117.7 us, 1024 chunks
                // per sequence 1739 -> 1704 us)
                gdr_sweep_ws<T, C, D, kSweepBV><<<dim3(tiles32), dim3(512), 0, stream>>>(p);
            } else {
                // C = 64, 32-column tiles: more than 128 chunks per sequence (on
                // average; nc_max bounds the total) take the refills spread over
                // the step (measured with two sets in flight: 1.74 vs 1.80 ms at
                // 1024 chunks; 190.1 vs 189.0 us at 128 chunks; at 64 chunks
                // 127 vs 121 us)
                if (C == 64 && p.nc_max > 128 * p.N) gdr_sweep<T, C, D, kSweepBV, C == 64><<<dim3(tiles32), dim3(256), 0, stream>>>(p);
                else gdr_sweep<T, C, D, kSweepBV><<<dim3(tiles32), dim3(256), 0, stream>>>(p);
            }
        }
    }
    if (e == hipSuccess) e = mark(3);
    return e;
}

// The backward pass: four kernels (p.dirs == 2), or the reverse sweep and the
// gradient kernel after the forward pass (p.dir0 == 1, p.dirs == 1).
template <typename T, int C, int D, bool SCALAR>
hipError_t launch_bwd(const Params& p, hipStream_t stream, hipEvent_t const* ev) {
    hipError_t e = launch_front<T, C, D, SCALAR>(p, stream, ev);
    if (p.nc_max > 0) {
        const dim3 block(128 * (C / 16));
        if (p.G > 1) {
            gdr_chunk_bwd<T, C, D, SCALAR, true><<<dim3(p.nc_max, p.Hg), block, 0, stream>>>(p);
        } else {   // persistent over (chunk, head) items, as many workgroups as the CUs hold
            const int items = p.nc_max * p.Hg, slots = compute_units() * resident_per_cu<T, C>();
            gdr_chunk_bwd<T, C, D, SCALAR, false><<<dim3(items < slots ? items : slots), block, 0, stream>>>(p);
        }
    }
    if (e == hipSuccess && ev) e = hipEventRecord(ev[4], stream);
    const hipError_t le = hipGetLastError();
    return le != hipSuccess ? le : e;
}

// The fused reverse backward (chunk 32): chunk table, preparation and the
// forward sweep alone (p.dirs == 1, p.dir0 == 0: h and X), then one gradient
// workgroup per (sequence, value head) that runs the reverse sweep itself with
// the state gradient on chip, then, with GQA, the fp32 group sums of dq, dk.
template <typename T, int C, int D, bool SCALAR>
hipError_t launch_fused(const Params& p, hipStream_t stream, hipEvent_t const* ev) {
    hipError_t e = launch_front<T, C, D, SCALAR>(p, stream, ev);
    if constexpr (C == 32) {
        // always launched: with no chunks it still writes dh0 = dht
        gdr_chunk_bwd<T, C, D, SCALAR, false, true><<<dim3(p.N * p.H), dim3(128 * (C / 16)), 0, stream>>>(p);
        if (p.G > 1 && p.B * p.T > 0) {
            const size_t n = (size_t)(p.B * p.T) * p.Hg * (D / 4);
            gdr_group_sum<T, D><<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream>>>(p);
        }
    } else {
        return hipErrorInvalidValue;   // not built: its LDS plan needs chunk 32
    }
    if (e == hipSuccess && ev) e = hipEventRecord(ev[4], stream);
    const hipError_t le = hipGetLastError();
    return le != hipSuccess ? le : e;
}

// The forward pass (p.dirs == 1): the same front, then the output kernel.
template <typename T, int C, int D, bool SCALAR>
hipError_t launch_fwd(const Params& p, hipStream_t stream, hipEvent_t const* ev) {
    hipError_t e = launch_front<T, C, D, SCALAR>(p, stream, ev);
    if (p.nc_max > 0) gdr_fwd_out<T, C, D><<<dim3(p.nc_max, p.H), dim3(64 * (C / 16)), 0, stream>>>(p);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[4], stream);
    const hipError_t le = hipGetLastError();
    return le != hipSuccess ? le : e;
}

// Instantiated in gdr_inst_*.hip; looked up by the C ABI.
// pass: 0 = backward, 1 = forward, 2 = fused reverse backward (chunk 32 only).
LaunchFn find_launcher(int io_dtype, int chunk, int dim, int scalar, int pass);

}  // namespace gdr
