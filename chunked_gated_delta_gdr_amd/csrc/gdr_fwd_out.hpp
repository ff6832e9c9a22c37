// gdr_fwd_out.hpp -- chunk-parallel output kernel of the forward pass.
//
// With h_c the state before chunk c (from the forward state sweep) and the
// chunk factors of the preparation kernel, the chunk form of the output
//     o_c = scale [(q 2^G) h_c + Aqk X_c],   X_c = u - w h_c
// (the WY recompute of the FlashQLA page's fused_bwd.py) is, with
// q~ = q 2^G - Aqk w,
//     o_c = (scale q~) h_c + (scale Aqk) u,
// two products on the stored scale q~^T, scale Aqk^T, u^T and h_c. One
// workgroup per (chunk, value head); wave w owns rows 16 w .. +16 and every
// column. Operands are staged in LDS as stored; the ones kept with the
// reduction index as the row are read as strided fragments.
#pragma once
#include "gdr_common.hpp"

namespace gdr {

template <typename T, int C, int D>
struct FwdOutLds {
    // h rows unpadded: its strided B-fragment reads (rows 8 apart) meet the same
    // banks with or without a pad, and without it the kernel fits 80 KB of LDS,
    // so that two workgroups share a CU
    static constexpr int LC = C + pad<T>(), LH = D;
    static constexpr size_t QS = 0;                                  // T [D][LC] scale q~^T
    static constexpr size_t SA = QS + size_t(D) * LC * sizeof(T);    // T [C][LC] scale Aqk^T
    static constexpr size_t UT = SA + size_t(C) * LC * sizeof(T);    // T [D][LC] u^T
    static constexpr size_t HL = UT + size_t(D) * LC * sizeof(T);    // T [D][LH] h_c, row-major
    static constexpr size_t TOTAL = HL + size_t(D) * LH * sizeof(T);
    static constexpr size_t OS = 0;                                  // T [C][LH] o, over the dead operands
    static_assert(size_t(C) * LH * sizeof(T) <= HL, "o staging clear of h");
    static_assert(TOTAL <= 163840, "LDS budget of gdr_fwd_out");
    static_assert(sizeof(T) != 2 || TOTAL <= 81920, "two workgroups per CU (16-bit io)");
};

template <typename T, int C, int D>
__global__ __launch_bounds__(64 * (C / 16)) void gdr_fwd_out(Params p) {
    using L = FwdOutLds<T, C, D>;
    constexpr int NB = C / 16, NT = 64 * NB, LC = L::LC, LH = L::LH, NTD = D / 16;
    constexpr int V8 = 16 / sizeof(T), KS = kstep<T>(), PT = kTileV / V8;
    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    T* qsL = reinterpret_cast<T*>(smem + L::QS);
    T* saL = reinterpret_cast<T*>(smem + L::SA);
    T* uL = reinterpret_cast<T*>(smem + L::UT);
    T* hL = reinterpret_cast<T*>(smem + L::HL);
    T* oS = reinterpret_cast<T*>(smem + L::OS);

    const int j = blockIdx.x, h = blockIdx.y;
    if (j >= p.seq_off[p.N]) return;
    const ChunkEntry ce = p.ctab[j];
    const int tid = threadIdx.x, w = wave_id(), l = lane_id();
    const size_t jh = (size_t)j * p.H + h;
    const T* gq = static_cast<const T*>(p.qsT) + jh * D * C;
    const T* ga = static_cast<const T*>(p.sAqkT) + jh * C * C;
    const T* gu = static_cast<const T*>(p.uT) + jh * D * C;
    const T* gh = static_cast<const T*>(p.hbuf) + jh * D * D;   // [D/kTileV][D][kTileV]

    // every global load of the thread's pieces goes out before the first LDS
    // write (constant trip counts, unrolled), so the loads overlap
    constexpr int NQ = D * (C / V8) / NT, NA = C * (C / V8) / NT, NH = D * (D / V8) / NT;
    static_assert(NQ * NT == D * (C / V8) && NA * NT == C * (C / V8) && NH * NT == D * (D / V8), "piece split");
    Vec16 qv[NQ], uv[NQ], av[NA], hv[NH];
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
        const int e = tid + it * NT, d = e / (C / V8), c = (e % (C / V8)) * V8;
        qv[it] = ld16(gq + fo_index<T, C>(d, c));   // fragment order
        // u^T in accumulator order: a 16-byte row piece is 4-element quads
        if constexpr (sizeof(T) == 2) {
            uv[it].w[0] = reinterpret_cast<const unsigned*>(gu + ao_index<C>(d, c))[0];
            uv[it].w[1] = reinterpret_cast<const unsigned*>(gu + ao_index<C>(d, c))[1];
            uv[it].w[2] = reinterpret_cast<const unsigned*>(gu + ao_index<C>(d, c + 4))[0];
            uv[it].w[3] = reinterpret_cast<const unsigned*>(gu + ao_index<C>(d, c + 4))[1];
        } else {
            uv[it] = ld16(gu + ao_index<C>(d, c));
        }
    }
#pragma unroll
    for (int it = 0; it < NA; ++it) {
        const int e = tid + it * NT, r = e / (C / V8), c = (e % (C / V8)) * V8;
        av[it] = ld16(ga + fo_index<T, C>(r, c));   // fragment order
    }
#pragma unroll
    for (int it = 0; it < NH; ++it) {   // contiguous in the tiled layout
        const int e = tid + it * NT, vt = e / (D * PT), rem = e % (D * PT), d = rem / PT, c = (rem % PT) * V8;
        hv[it] = ld16(gh + (size_t)vt * D * kTileV + d * kTileV + c);
    }
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
        const int e = tid + it * NT, d = e / (C / V8), c = (e % (C / V8)) * V8;
        st16(qsL + d * LC + c, qv[it]);
        st16(uL + d * LC + c, uv[it]);
    }
#pragma unroll
    for (int it = 0; it < NA; ++it) {
        const int e = tid + it * NT, r = e / (C / V8), c = (e % (C / V8)) * V8;
        st16(saL + r * LC + c, av[it]);
    }
#pragma unroll
    for (int it = 0; it < NH; ++it) {
        const int e = tid + it * NT, vt = e / (D * PT), rem = e % (D * PT), d = rem / PT, c = (rem % PT) * V8;
        st16(hL + d * LH + vt * kTileV + c, hv[it]);
    }
    __syncthreads();

    const int r0 = 16 * w;
    f32x4 acc[NTD];
#pragma unroll
    for (int t = 0; t < NTD; ++t) acc[t] = zero4();
    // (scale q~) h: A(r, d) = qsT[d][r], B(d, v) = h[d][v]
    for (int k0 = 0; k0 < D; k0 += KS) {
        const auto a = frag_ks(qsL, LC, r0, k0, l);
#pragma unroll
        for (int t = 0; t < NTD; ++t) acc[t] = Mfma<T>::mma(a, frag_ks(hL, LH, 16 * t, k0, l), acc[t]);
    }
    // (scale Aqk) u: A(r, s) = sAqkT[s][r], B(s, v) = u[s][v] = uT[v][s]
#pragma unroll
    for (int k0 = 0; k0 < C; k0 += KS) {
        const auto a = frag_ks(saL, LC, r0, k0, l);
#pragma unroll
        for (int t = 0; t < NTD; ++t) acc[t] = Mfma<T>::mma(a, frag_kc(uL, LC, 16 * t, k0, l), acc[t]);
    }
    __syncthreads();  // operands read: the staging of o overwrites them
#pragma unroll
    for (int t = 0; t < NTD; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) oS[(r0 + acc_row(i, l)) * LH + 16 * t + acc_col(l)] = from_f32<T>(acc[t][i]);
    __syncthreads();
    T* go = static_cast<T*>(p.o) + ((size_t)ce.tok0 * p.H + h) * D;
    constexpr int NO = C * (D / V8) / NT;
    static_assert(NO * NT == C * (D / V8), "piece split");
#pragma unroll
    for (int it = 0; it < NO; ++it) {
        const int e = tid + it * NT, r = e / (D / V8), c = (e % (D / V8)) * V8;
        if (r < ce.len) st16(go + (size_t)r * p.H * D + c, ld16(oS + r * LH + c));
    }
}

}  // namespace gdr
