// gdr_states.hpp -- the backward's per-chunk states taken from the caller.
//
// The backward of the FlashQLA issue #30 page (fused_bwd.py, and its wrapper
// fused_gdr_bwd) takes the per-chunk states h_c that the forward pass saved,
// [chunks][H][K][V] or, with state_v_first, [chunks][H][V][K], instead of
// recomputing them. gdr_states_in replaces the forward state sweep for such a
// call: it is chunk-parallel (no recurrence left to run), one workgroup per
// (chunk, value head, tile of 32 state columns), and writes what the sweep
// would have written for the tile:
//     h_c tile -> the workspace's state region (its tiled layout),
//     X_c = u_c - w_c h_c -> the workspace's X region,
// with u_c, w_c from the preparation kernel. The reverse sweep and the
// gradient kernel then run as in the full backward.
#pragma once
#include "gdr_common.hpp"

namespace gdr {

template <typename T, int C, int D, bool VFIRST>
__global__ __launch_bounds__(256) void gdr_states_in(Params p) {
    constexpr int BV = kTileV;                 // state columns per workgroup: one stored tile
    constexpr int V8 = 16 / sizeof(T);         // elements per 16-byte piece
    constexpr int KS = kstep<T>();
    constexpr int LB = BV + pad<T>();          // h tile rows [D][LB] (key-first) / X rows [C][LB]
    constexpr int LD = D + pad<T>();           // h tile rows [BV][LD] (value-first)
    constexpr int RT = C / 16, CT = BV / 16;   // row / column tiles of X
    constexpr int TPW = RT * CT / 4;           // tiles per wave (4 waves)
    static_assert(TPW * 4 == RT * CT && BV % V8 == 0 && D % V8 == 0, "states_in tiling");
    using Q = typename Mfma<T>::quad;
    __shared__ __attribute__((aligned(16))) T hS[VFIRST ? BV * LD : D * LB];
    __shared__ __attribute__((aligned(16))) T xS[C * LB];

    const int j = blockIdx.x, h = blockIdx.y, vt = blockIdx.z, v0 = vt * BV;
    // chunks past the table's count, or past what the caller's buffer holds: nothing to do
    if (j >= p.seq_off[p.N] || j >= p.nh_src) return;
    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const size_t jh = (size_t)j * p.H + h;
    const T* hc = static_cast<const T*>(p.hsrc) + jh * D * D;
    T* hb = static_cast<T*>(p.hbuf) + jh * D * D + (size_t)vt * D * BV;   // tile [D][BV]

    // 1. the caller's h_c columns v0 .. v0 + BV to LDS (and, key-first, straight
    //    to the workspace tile: its rows are the caller's row pieces)
    if constexpr (!VFIRST) {
        for (int e = tid; e < D * (BV / V8); e += 256) {
            const int d = e / (BV / V8), c = (e % (BV / V8)) * V8;
            const Vec16 x = ld16(hc + (size_t)d * D + v0 + c);
            st16(hS + d * LB + c, x);
            st16(hb + d * BV + c, x);
        }
    } else {
        for (int e = tid; e < BV * (D / V8); e += 256) {
            const int c = e / (D / V8), d = (e % (D / V8)) * V8;
            st16(hS + c * LD + d, ld16(hc + (size_t)(v0 + c) * D + d));
        }
    }
    __syncthreads();
    if constexpr (VFIRST) {   // the workspace tile, key-first, read back across the LDS rows
        for (int e = tid; e < D * (BV / V8); e += 256) {
            const int d = e / (BV / V8), c = (e % (BV / V8)) * V8;
            Vec16 x;
            T* xp = reinterpret_cast<T*>(&x);
#pragma unroll
            for (int q = 0; q < V8; ++q) xp[q] = hS[(c + q) * LD + d];
            st16(hb + d * BV + c, x);
        }
    }

    // 2. X = u - w h for the wave's tiles (w rows as stored, in fragment order;
    //    h columns from LDS; u at the accumulator elements, in accumulator order)
    const T* wg = static_cast<const T*>(p.w) + jh * C * D;
    const T* uT = static_cast<const T*>(p.uT) + jh * D * C;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int tl = w * TPW + i, rt = tl / CT, ct = tl % CT;
        f32x4 acc = zero4();
#pragma unroll
        for (int k0 = 0; k0 < D; k0 += KS) {
            const auto a = frag_fo<T, D>(wg, 16 * rt, k0, l);
            const auto b = VFIRST ? frag_kc(hS, LD, 16 * ct, k0, l) : frag_ks(hS, LB, 16 * ct, k0, l);
            acc = Mfma<T>::mma(a, b, acc);
        }
        const int r = 16 * rt + acc_row(0, l), c = 16 * ct + acc_col(l);
        const Q uq = *reinterpret_cast<const Q*>(uT + ao_index<C>(v0 + c, r));
#pragma unroll
        for (int e = 0; e < 4; ++e) xS[(r + e) * LB + c] = from_f32<T>(to_f32(uq[e]) - acc[e]);
    }
    __syncthreads();

    // 3. the X tile [C][BV] to the workspace, 16 bytes per access
    T* xb = static_cast<T*>(p.xbuf) + jh * C * D + (size_t)vt * C * BV;
    for (int e = tid; e < C * (BV / V8); e += 256) {
        const int r = e / (BV / V8), c = (e % (BV / V8)) * V8;
        st16(xb + r * BV + c, ld16(xS + r * LB + c));
    }
}

}  // namespace gdr
