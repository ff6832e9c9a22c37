// gdr_sweep.hpp -- the two sequential state sweeps over chunks, one launch.
//
// Forward (dir 0), per (sequence, value head, V tile), state h (K x BV, fp32
// in MFMA accumulators), h = h0 at the first chunk:
//     store h_c;  X_c = u_c - w_c h_c;  store X_c;
//     h_{c+1} = Diag(2^G_last) h_c + k~_c^T X_c
// Reverse (dir 1), state dh = dht at the end:
//     store dh_{c+1};  T_c = k~_c dh_{c+1};  store T_c;
//     dh_c = Diag(2^G_last) dh_{c+1} - w_c^T T_c + (scale q~_c)^T do_c
// with q~ = q 2^G - Aqk w, so that scale (q 2^G)^T do - w^T (scale Aqk^T do)
// collapses into one term (the state-gradient recurrence of the CONSUMER_S
// role of fused_bwd.py on the FlashQLA issue #30 page: decay by the chunk's
// last gate, plus the key-side and query-side products). Columns of the state never mix (Diag acts on K, every product keeps
// the column), so a V tile per workgroup is exact. dh0 = dh_0 is written in
// fp32. The two directions are independent and share one grid (a pass that
// needs one direction launches only that one).
//
// The per-chunk operands (w, k~, u, q~, 2^G_last) are read straight from
// global memory as MFMA fragments of the rows each wave owns (stored in
// fragment / accumulator order, so each is one contiguous wave load), NPF
// chunks ahead into NPF fixed register sets (the chunk loop is unrolled NPF
// times so that no register copy forces an early wait on a load in flight).
// Only the state and X / T (and do for the reverse direction) pass through
// LDS, double-buffered, two barriers per chunk; the stores of h_c and X_c
// (T_c) to the workspace read those LDS tiles back as 16-byte row pieces.
#pragma once
#include "gdr_common.hpp"

namespace gdr {

template <typename T, int C, int D, int BV>
struct SweepTiles {
    static constexpr int KS = kstep<T>();
    static constexpr int SCT = BV / 16;                       // column tiles of the state / X
    // state [D][BV]: SRW row tiles per wave, all SCT column tiles
    static constexpr int SRW = (D / 16) / 4;
    // X / T [C][BV]: XRT row tiles x XCT column tiles per wave
    static constexpr int XR = C / 16;
    static constexpr int XRT = XR >= 4 ? XR / 4 : 1;
    static constexpr int XCT = XR >= 4 ? SCT : SCT * XR / 4;
    static_assert(SRW >= 1 && XCT >= 1 && XRT * XCT * 4 == XR * SCT, "sweep tiling");
    static __device__ __forceinline__ int xrow(int w, int i) { return XR >= 4 ? w * XRT + i : w / (4 / XR); }
    static __device__ __forceinline__ int xcol(int w, int j) { return XR >= 4 ? j : (w % (4 / XR)) * XCT + j; }
};

// Operands of one chunk, as the MFMA fragments / raw values this lane needs
// (kept in the operand type: a conversion at load time would wait for the load).
template <typename T, int C, int D, int BV, int DIR>
struct SweepOps {
    using S = SweepTiles<T, C, D, BV>;
    using F = typename Mfma<T>::frag;
    using Q = typename Mfma<T>::quad;
    static constexpr int NDO = (C * (BV / (16 / sizeof(T))) + 255) / 256;
    // the state update's A operand k~^T (fwd) or w^T (rev): read as such, or
    // (TRA2) as the wave's 32-column block of k~ or w in fragment order, one
    // 1 KB tile per 16 rows, transposed in LDS at use
    static constexpr bool TRA2 = sweep_transposes_a2<T, C, D, BV>();
    static_assert(!TRA2 || S::SRW == 2, "a wave's state rows: one 32-column block");
    F a1[S::XRT][D / S::KS];                  // chunk-row product A operand: w (fwd) or k~ (rev)
    F a2[TRA2 ? 1 : S::SRW][TRA2 ? 1 : C / S::KS];
    Vec16 a2r[TRA2 ? C / 16 : 1];
    F a3[DIR == 1 ? S::SRW : 1][C / S::KS];   // reverse: (scale q~)^T
    Q u[DIR == 0 ? S::XRT : 1][S::XCT];       // forward: u at this lane's X elements
    f32x4 gl[S::SRW];                         // 2^G_last at this lane's state rows
    Vec16 dov[DIR == 1 ? NDO : 1];            // reverse: this thread's 16-byte pieces of do
};

// Loads the operands of global chunk j (first token tok0, len real rows).
// PART selects which operands: 0 all; 1 those the step has used by its first
// barrier (the staged k~ / w tiles, do); 2 those of the chunk-row product
// (w / k~ fragments, u); 3 those of the state update (k~^T / w^T fragments,
// (scale q~)^T, 2^G_last).
template <typename T, int C, int D, int BV, int DIR, int PART = 0>
__device__ __forceinline__ void sweep_load(SweepOps<T, C, D, BV, DIR>& o, const Params& p, int j, int tok0,
                                           int len, int h, int v0, int w) {
    using S = SweepTiles<T, C, D, BV>;
    using Q = typename Mfma<T>::quad;
    const size_t jh = (size_t)j * p.H + h;
    const T* A1 = static_cast<const T*>(DIR == 0 ? p.w : p.kt) + jh * C * D;
    const T* A2 = static_cast<const T*>(DIR == 0 ? p.ktT : p.wT) + jh * D * C;
    constexpr bool P1 = PART == 0 || PART == 1, P2 = PART == 0 || PART == 2, P3 = PART == 0 || PART == 3;
    if constexpr (P2) {
#pragma unroll
        for (int i = 0; i < S::XRT; ++i)
#pragma unroll
            for (int k = 0; k < D / S::KS; ++k) o.a1[i][k] = frag_fo<T, D>(A1, 16 * S::xrow(w, i), k * S::KS);
    }
    if constexpr (SweepOps<T, C, D, BV, DIR>::TRA2) {
        if constexpr (P1) {
            const T* A2r = static_cast<const T*>(DIR == 0 ? p.kt : p.w) + jh * C * D;
            const int l = lane_id();
#pragma unroll
            for (int ct = 0; ct < C / 16; ++ct)
                o.a2r[ct] = ld16(A2r + fo_index<T, D>(16 * ct + (l & 15), 32 * w + 8 * (l >> 4)));
        }
    } else if constexpr (P3) {
#pragma unroll
        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
            for (int k = 0; k < C / S::KS; ++k) o.a2[i][k] = frag_fo<T, C>(A2, 16 * (w * S::SRW + i), k * S::KS);
    }
    if constexpr (P3) {
        const float* gl = p.glast + jh * D;
#pragma unroll
        for (int i = 0; i < S::SRW; ++i) o.gl[i] = *reinterpret_cast<const f32x4*>(gl + 16 * (w * S::SRW + i) + acc_row(0));
    }
    if constexpr (DIR == 0 && P2) {
        const T* uT = static_cast<const T*>(p.uT) + jh * D * C;
#pragma unroll
        for (int i = 0; i < S::XRT; ++i)
#pragma unroll
            for (int jj = 0; jj < S::XCT; ++jj) {
                const int r = 16 * S::xrow(w, i) + acc_row(0);
                const int c = v0 + 16 * S::xcol(w, jj) + acc_col();
                o.u[i][jj] = *reinterpret_cast<const Q*>(uT + ao_index<C>(c, r));   // accumulator order
            }
    }
    if constexpr (DIR == 1 && P3) {
        const T* qsT = static_cast<const T*>(p.qsT) + jh * D * C;
#pragma unroll
        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
            for (int k = 0; k < C / S::KS; ++k) o.a3[i][k] = frag_fo<T, C>(qsT, 16 * (w * S::SRW + i), k * S::KS);
    }
    if constexpr (DIR == 1 && P1) {
        // do rows of the chunk, this thread's 16-byte piece; rows past the
        // sequence end read its last row (always valid) and are zeroed at use
        constexpr int V8 = 16 / sizeof(T);
#pragma unroll
        for (int pi = 0; pi < o.NDO; ++pi) {
            const int e = min((int)threadIdx.x + 256 * pi, C * (BV / V8) - 1);  // spare threads: a valid duplicate
            const int r = e / (BV / V8), cc = (e % (BV / V8)) * V8;
            const int rr = min(r, len - 1);
            o.dov[pi] = ld16(static_cast<const T*>(p.dout) + ((size_t)(tok0 + rr) * p.H + h) * D + v0 + cc);
        }
    }
}

// Offset of (row r, column v0 + c) in a matrix of R rows stored as tiles of
// kTileV columns ([D / kTileV][R][kTileV]); a 16-byte piece never straddles
// two tiles. A V tile of BV <= kTileV columns lies in one stored tile, whose
// offset is then uniform over the workgroup.
template <int R, int BV>
__device__ __forceinline__ size_t tiled_index(int r, int v0, int c) {
    if constexpr (BV <= kTileV) return (size_t)(v0 / kTileV) * kTileV * R + v0 % kTileV + (size_t)r * kTileV + c;
    const int cc = v0 + c;
    return (size_t)(cc / kTileV) * kTileV * R + (size_t)r * kTileV + cc % kTileV;
}

// A fragment (rows i0 .. +15, reduction k0 + 8 (l / 16) + 0..7) of M^T, where
// a 32-column block of the C x D matrix M sits in LDS as 16 x 32 tiles in
// fragment order (tile t: rows 16 t .. +15, 512 elements, lane slot
// s = row % 16 + 16 (column / 8) at 8 s): the 4-element pieces the transposed
// loads take are halves of those slots (as in frag_ks, with that addressing).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag_fo_tr(const T* tiles, int i0, int k0, int l) {
    static_assert(sizeof(T) == 2, "16-bit transposed loads");
    auto piece = [&](int kk) {   // lane: row kk + (l % 16) / 4, columns i0 + 4 (l % 4) .. + 3
        const int c = kk + ((l & 15) >> 2), d = i0 + 4 * (l & 3);
        const T* q = tiles + (c >> 4) * 512 + ((c & 15) + 16 * (d >> 3)) * 8 + (d & 7);
        return __builtin_bit_cast(
            uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(q)));
    };
    // the two loads' 64-bit values, not their elements (see ks_tr4_bits)
    const uint64_t v[2] = {piece(k0 + 8 * (l >> 4)), piece(k0 + 8 * (l >> 4) + 4)};
    typename Mfma<T>::frag f;
    __builtin_memcpy(&f, v, sizeof(f));
    return f;
}

// Row pitch (elements) of the do rows in LDS: 16-byte aligned rows whose
// transposed loads (four rows by four 8-byte column pieces per 16 lanes) fall
// in distinct banks.
template <typename T, int BV>
constexpr int do_pitch() { return BV + (sizeof(T) == 2 ? 16 : 4); }
// Whether the reverse direction keeps do rows as loaded (one 16-byte LDS write
// per piece, do^T fragments through transposed loads) instead of writing do^T
// element by element: measured faster at C = 32 (GDN GQA sweep 1.20 -> 1.17
// ms) and for 32-column tiles at C = 64 (headline sweep 121.9 -> 120.9 us),
// slower for 64-column tiles at C = 64 (varlen sweep 364 -> 368 us).
template <typename T, int C, int BV>
constexpr bool do_rows() { return sizeof(T) == 2 && (C == 32 || BV <= 32); }

// 64-column tiles with 16-bit operands copy the state and X / T out with
// 16-bit reads, 8 rows per thread piece, rows 8 apart: at the padded row
// pitches those rows share one LDS bank (and the C = 64 reverse direction
// writes do^T the same way). So these buffers hold element (row c, index k)
// at c * pitch + (k ^ swz(c)), an XOR of k's 8-element groups by c / 8
// (limited to the K / 8 groups of the index range K): the 8-element MFMA
// fragment reads and 4-element writes stay contiguous, and the eight rows of
// a copy-out read fall in distinct banks (at most two share one for X / T at
// C = 32, whose 32-element rows have four groups). Measured: varlen workload
// sweep (C = 64) 675 -> 600 us, GDN GQA sweep (C = 32) 1102 -> 879 us.
template <typename T, int C, int BV, int K>
__device__ __forceinline__ int sweep_swz(int c) {
    if constexpr (sizeof(T) == 2 && BV == 64) return 8 * ((c >> 3) & ((K / 8 < 8 ? K / 8 : 8) - 1));
    else return 0;
}
// frag_kc on a buffer laid out as above
template <typename T, int C, int BV, int K>
__device__ __forceinline__ typename Mfma<T>::frag frag_kc_swz(const T* p, int ld, int i0, int k0, int l = lane_id()) {
    const int i = i0 + (l & 15), k = k0 + (l >> 4) * Mfma<T>::KL;
    return *reinterpret_cast<const typename Mfma<T>::frag*>(p + (long)i * ld + (k ^ sweep_swz<T, C, BV, K>(i)));
}

// One direction of the sweep for (sequence n, value head h, V tile at v0).
template <typename T, int C, int D, int BV, int DIR, int NPF, bool SPREAD>
__device__ __forceinline__ void sweep_run(const Params& p, int n, int h, int v0, T* sS0, T* sS1, T* sX0, T* sX1, T* sDo0,
                                          T* sDo1, T* sA2) {
    using S = SweepTiles<T, C, D, BV>;
    using Ops = SweepOps<T, C, D, BV, DIR>;
    constexpr int SCT = S::SCT, KS = S::KS;
    constexpr int LS = D + pad<T>();                 // state^T rows [BV][LS]
    constexpr int LX = C + pad<T>();                 // X^T / -T^T / do^T rows [BV][LX]
    constexpr int LDO = do_pitch<T, BV>();           // do rows as loaded [C][LDO] (do_rows)
    constexpr int V8 = 16 / sizeof(T);
    const int w = wave_id();
    const int c0 = p.seq_off[n], c1 = p.seq_off[n + 1];
    const int nch = c1 - c0;
    // chunk geometry of the sequence (the chunk table's, computed here so that
    // no load of it sits between a prefetch and its use)
    int stok0, slen;
    seq_span(p, n, stok0, slen);
    const size_t sh = ((size_t)n * p.H + h) * D * D;

    f32x4 st[S::SRW][SCT];
    {   // initial state: h0 (forward) or dht (reverse), zero when absent
        const float* init = DIR == 0 ? p.h0 : p.dht;
#pragma unroll
        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
            for (int ct = 0; ct < SCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int d = 16 * (w * S::SRW + i) + acc_row(e), c = v0 + 16 * ct + acc_col();
                    st[i][ct][e] = init ? init[sh + state_index<D>(p, d, c)] : 0.f;
                }
    }
    // step k of this direction works on chunk `it` of the sequence
    auto chunk_it = [&](int k) { return DIR == 0 ? k : nch - 1 - k; };
    // part 0: all operands; 1-3: the groups a step has finished with at its
    // three refill points (see sweep_load)
    auto load = [&](auto part_c, Ops& o, int k) __attribute__((always_inline)) {
        const int it = chunk_it(k < nch ? k : nch - 1);   // past the end: a redundant valid load
        sweep_load<T, C, D, BV, DIR, decltype(part_c)::value>(o, p, c0 + it, stok0 + it * C, min(C, slen - it * C), h,
                                                             v0, w);
    };
    // refill(part): request the next use of this register set, part by part,
    // as soon as the step no longer reads that part (spreading the requests
    // over the step instead of issuing them all behind its stores)
    auto step = [&](const Ops& cur, const int k, auto&& refill) __attribute__((always_inline)) {
        const int it = chunk_it(k);
        const size_t jh = (size_t)(c0 + it) * p.H + h;
        T* sS = (k & 1) ? sS1 : sS0;
        T* sX = (k & 1) ? sX1 : sX0;
        T* sDo = (k & 1) ? sDo1 : sDo0;

        // 1. publish the incoming state to LDS (transposed: B operand with K
        //    contiguous); do^T of this chunk's V tile for the reverse direction
#pragma unroll
        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
            for (int ct = 0; ct < SCT; ++ct) {
                const int d = 16 * (w * S::SRW + i) + acc_row(0), c = 16 * ct + acc_col();
                store4<T>(sS + c * LS + (d ^ sweep_swz<T, C, BV, D>(c)), st[i][ct][0], st[i][ct][1], st[i][ct][2],
                          st[i][ct][3]);
            }
        if constexpr (DIR == 1) {
            const int len = min(C, slen - it * C);
#pragma unroll
            for (int pi = 0; pi < Ops::NDO; ++pi) {
                const int e = threadIdx.x + 256 * pi;
                if (e < C * (BV / V8)) {
                    const int r = e / (BV / V8), cc = (e % (BV / V8)) * V8;
                    if constexpr (do_rows<T, C, BV>()) {
                        // rows as loaded (the product reads them through transposed loads)
                        st16(sDo + r * LDO + cc, r < len ? cur.dov[pi] : Vec16{});
                    } else {
                        // opaque here: keeps the element extraction (and the wait
                        // for the load) from being hoisted to the previous chunk
                        Vec16 dv = cur.dov[pi];
                        asm volatile("" : "+v"(dv.w[0]), "+v"(dv.w[1]), "+v"(dv.w[2]), "+v"(dv.w[3]));
                        const T* xp = reinterpret_cast<const T*>(&dv);
#pragma unroll
                        for (int q = 0; q < V8; ++q)
                            sDo[(cc + q) * LX + (r ^ sweep_swz<T, C, BV, C>(cc + q))] = r < len ? xp[q] : T(0.f);
                    }
                }
            }
        }
        if constexpr (Ops::TRA2) {   // the wave's k~ / w tiles to its own LDS block
            const int l = lane_id();
#pragma unroll
            for (int ct = 0; ct < C / 16; ++ct) st16(sA2 + (w * (C / 16) + ct) * 512 + 8 * l, cur.a2r[ct]);
        }
        __syncthreads();
        refill(std::integral_constant<int, 1>{});

        // 2. chunk-row product: X = u - w h (fwd) or T = k~ dh (rev); forward
        //    keeps +X, reverse keeps -T so the state update is a pure sum. All
        //    B fragments are read before the first product (the scheduling
        //    barrier keeps the compiler from sinking each read to its use, which
        //    would expose one LDS round trip per MFMA).
        // (TRA2: the update's A fragments, transposed from the staged tiles, are
        // read here too, ahead of both products)
        typename Mfma<T>::frag a2f[Ops::TRA2 ? S::SRW : 1][Ops::TRA2 ? C / KS : 1];
        {
            typename Mfma<T>::frag bx[S::XCT][D / KS];
#pragma unroll
            for (int jj = 0; jj < S::XCT; ++jj)
#pragma unroll
                for (int k2 = 0; k2 < D / KS; ++k2) bx[jj][k2] = frag_kc_swz<T, C, BV, D>(sS, LS, 16 * S::xcol(w, jj), k2 * KS);
            if constexpr (Ops::TRA2) {
                const int l = lane_id();
#pragma unroll
                for (int i = 0; i < S::SRW; ++i)
#pragma unroll
                    for (int k2 = 0; k2 < C / KS; ++k2)
                        a2f[i][k2] = frag_fo_tr(sA2 + w * (C / 16) * 512, 16 * i, k2 * KS, l);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < S::XRT; ++i) {
                f32x4 acc[S::XCT];
#pragma unroll
                for (int jj = 0; jj < S::XCT; ++jj) acc[jj] = zero4();
#pragma unroll
                for (int k2 = 0; k2 < D / KS; ++k2)
#pragma unroll
                    for (int jj = 0; jj < S::XCT; ++jj) acc[jj] = Mfma<T>::mma(cur.a1[i][k2], bx[jj][k2], acc[jj]);
#pragma unroll
                for (int jj = 0; jj < S::XCT; ++jj) {
                    const int r = 16 * S::xrow(w, i) + acc_row(0), c = 16 * S::xcol(w, jj) + acc_col();
                    float o[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = DIR == 0 ? to_f32(cur.u[i][jj][e]) - acc[jj][e] : -acc[jj][e];
                    store4<T>(sX + c * LX + (r ^ sweep_swz<T, C, BV, C>(c)), o[0], o[1], o[2], o[3]);
                }
            }
        }
        refill(std::integral_constant<int, 2>{});
        __syncthreads();

        // 3. state update: st = Diag(2^G_last) st + A2 X (+ (scale q~)^T do for reverse).
        //    State, X / T and do^T are double-buffered: the next chunk writes the
        //    other buffers, and this chunk's buffers are rewritten only after
        //    the next chunk's barriers, which every wave reaches after its
        //    copy-outs below, so no third barrier is needed.
        {   // B fragments first (as in 2), then the SRW x SCT chains interleaved
            typename Mfma<T>::frag bxs[SCT][C / KS], bdo[DIR == 1 ? SCT : 1][C / KS];
#pragma unroll
            for (int ct = 0; ct < SCT; ++ct)
#pragma unroll
                for (int k2 = 0; k2 < C / KS; ++k2) {
                    bxs[ct][k2] = frag_kc_swz<T, C, BV, C>(sX, LX, 16 * ct, k2 * KS);
                    if constexpr (DIR == 1)
                        bdo[ct][k2] = do_rows<T, C, BV>() ? frag_ks(sDo, LDO, 16 * ct, k2 * KS)    // do^T from do rows
                                                      : frag_kc_swz<T, C, BV, C>(sDo, LX, 16 * ct, k2 * KS);
                }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < S::SRW; ++i)
#pragma unroll
                for (int ct = 0; ct < SCT; ++ct)
#pragma unroll
                    for (int e = 0; e < 4; ++e) st[i][ct][e] *= cur.gl[i][e];
#pragma unroll
            for (int k2 = 0; k2 < C / KS; ++k2)
#pragma unroll
                for (int i = 0; i < S::SRW; ++i)
#pragma unroll
                    for (int ct = 0; ct < SCT; ++ct)
                        st[i][ct] = Mfma<T>::mma(Ops::TRA2 ? a2f[i][k2] : cur.a2[i][k2], bxs[ct][k2], st[i][ct]);
            if constexpr (DIR == 1) {
#pragma unroll
                for (int k2 = 0; k2 < C / KS; ++k2)
#pragma unroll
                    for (int i = 0; i < S::SRW; ++i)
#pragma unroll
                        for (int ct = 0; ct < SCT; ++ct)
                            st[i][ct] = Mfma<T>::mma(cur.a3[i][k2], bdo[ct][k2], st[i][ct]);
            }
        }
        refill(std::integral_constant<int, 3>{});
        {   // the incoming state to the workspace, row-major: 8 columns per piece,
            // read back from its LDS buffer while the update's MFMAs run.
            // Stores are never behind a branch (spare threads repeat a piece with
            // the same data): a store on one path only would make the compiler's
            // memory-counter waits for the prefetched loads also wait for it.
            T* gS = static_cast<T*>(DIR == 0 ? p.hbuf : p.dhbuf) + jh * D * D;
            if constexpr (sizeof(T) == 2 && BV == 32) {
                // 16 rows x 32 columns per wave and tile: two transposed loads
                // give lane l row 16 dt + l % 16 at columns 32 ct + 8 (l / 16) + 0..7
                // (with 64-column tiles, at C = 32, the 16-bit reads below
                // measured faster)
                constexpr int NTL = (D / 16) * (BV / 32);
                static_assert(NTL % 4 == 0, "tiles per wave");
                const int l = lane_id();
#pragma unroll
                for (int it = 0; it < NTL / 4; ++it) {
                    const int tl = w + 4 * it, dt = tl % (D / 16), ct = tl / (D / 16);
                    const uint64_t a = ks_tr4_bits(sS, LS, 16 * dt, 32 * ct, 8, l);
                    const uint64_t b = ks_tr4_bits(sS, LS, 16 * dt, 32 * ct + 4, 8, l);
                    const Vec16 v = {{uint32_t(a), uint32_t(a >> 32), uint32_t(b), uint32_t(b >> 32)}};
                    st16(gS + tiled_index<D, BV>(16 * dt + (l & 15), v0, 32 * ct + 8 * (l >> 4)), v);
                }
            } else {
                constexpr int NP = D * BV / V8;
#pragma unroll
                for (int pi = 0; pi < (NP + 255) / 256; ++pi) {
                    const int e = (int)(threadIdx.x + 256 * pi) % NP;
                    const int d = e / (BV / V8), c = (e % (BV / V8)) * V8;
                    Vec16 v;
                    T* vp = reinterpret_cast<T*>(&v);
#pragma unroll
                    for (int q = 0; q < V8; ++q) vp[q] = sS[(c + q) * LS + (d ^ sweep_swz<T, C, BV, D>(c + q))];
                    st16(gS + tiled_index<D, BV>(d, v0, c), v);
                }
            }
        }
        {   // X (T) of this chunk to the workspace, row-major pieces of 8 columns
            // (unconditional stores, as above)
            T* gX = static_cast<T*>(DIR == 0 ? p.xbuf : p.tbuf) + jh * C * D;
            constexpr int NTL = (C / 16) * (BV / 32);
            if constexpr (sizeof(T) == 2 && BV == 32 && NTL % 4 == 0) {
                // as for the state; the reverse direction stores -T (sign flips)
                const int l = lane_id();
                constexpr uint64_t kNeg = DIR == 0 ? 0 : 0x8000800080008000ull;
#pragma unroll
                for (int it = 0; it < NTL / 4; ++it) {
                    const int tl = w + 4 * it, rt = tl % (C / 16), ct = tl / (C / 16);
                    const uint64_t a = ks_tr4_bits(sX, LX, 16 * rt, 32 * ct, 8, l) ^ kNeg;
                    const uint64_t b = ks_tr4_bits(sX, LX, 16 * rt, 32 * ct + 4, 8, l) ^ kNeg;
                    const Vec16 v = {{uint32_t(a), uint32_t(a >> 32), uint32_t(b), uint32_t(b >> 32)}};
                    st16(gX + tiled_index<C, BV>(16 * rt + (l & 15), v0, 32 * ct + 8 * (l >> 4)), v);
                }
            } else {
                constexpr int NP = C * BV / V8;
#pragma unroll
                for (int pi = 0; pi < (NP + 255) / 256; ++pi) {
                    const int e = (int)(threadIdx.x + 256 * pi) % NP;
                    const int r = e / (BV / V8), c = (e % (BV / V8)) * V8;
                    Vec16 v;
                    T* vp = reinterpret_cast<T*>(&v);
#pragma unroll
                    for (int q = 0; q < V8; ++q) {
                        const T x = sX[(c + q) * LX + (r ^ sweep_swz<T, C, BV, C>(c + q))];
                        vp[q] = DIR == 0 ? x : from_f32<T>(-to_f32(x));
                    }
                    st16(gX + tiled_index<C, BV>(r, v0, c), v);
                }
            }
        }
    };

    if (nch > 0) {
        // NPF register sets, each refilled right after its chunk is done; the
        // loop is unrolled NPF times so that the sets never move
        Ops ops[NPF];
#pragma unroll
        for (int s2 = 0; s2 < NPF; ++s2) load(std::integral_constant<int, 0>{}, ops[s2], s2);
        int k0 = 0;
        for (; k0 + NPF <= nch; k0 += NPF) {
#pragma unroll
            for (int s2 = 0; s2 < NPF; ++s2) {
                if constexpr (SPREAD) {
                    step(ops[s2], k0 + s2, [&](auto part_c) __attribute__((always_inline)) {
                        load(part_c, ops[s2], k0 + s2 + NPF);
                    });
                } else {
                    step(ops[s2], k0 + s2, [](auto) {});
                    load(std::integral_constant<int, 0>{}, ops[s2], k0 + s2 + NPF);
                }
            }
        }
#pragma unroll
        for (int s2 = 0; s2 < NPF - 1; ++s2)
            if (k0 + s2 < nch) step(ops[s2], k0 + s2, [](auto) {});
    }
    // the final state: dh0 (reverse), or ht for the forward pass when asked
    float* fin = DIR == 1 ? p.dh0 : p.ht;
    if (fin) {
#pragma unroll
        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
            for (int ct = 0; ct < SCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int d = 16 * (w * S::SRW + i) + acc_row(e), c = v0 + 16 * ct + acc_col();
                    fin[sh + state_index<D>(p, d, c)] = st[i][ct][e];
                }
    }
}

// SPREAD: the next use of a register set is requested part by part, as the
// step finishes with each part (see sweep_load), instead of all at once after
// the step.
template <typename T, int C, int D, int BV, bool SPREAD = false>
__global__ __launch_bounds__(256) void gdr_sweep(Params p) {
    constexpr int LS = D + pad<T>();
    constexpr int LX = C + pad<T>();
    // chunks of operands in flight: at C = 64 with 64-column tiles one, its
    // refills spread over the step (two sets measured slower there: their
    // registers spilled); else two (three measured slower at 32-column tiles:
    // headline sweep 128 vs 120 us)
    constexpr int NPF = C == 64 && BV == 64 ? 1 : 2;
    static_assert(kTileV % BV == 0 || BV % kTileV == 0, "sweep V tiles and stored tiles nest");
    static_assert(kTileV % (16 / sizeof(T)) == 0, "a 16-byte piece lies within one stored tile");
    __shared__ __attribute__((aligned(16))) T sS[2][BV * LS];
    __shared__ __attribute__((aligned(16))) T sX[2][BV * LX];
    __shared__ __attribute__((aligned(16))) T sDo[2][do_rows<T, C, BV>() ? C * do_pitch<T, BV>() : BV * LX];
    // per wave: its 32-column block of k~ / w (C / 16 fragment-order tiles)
    __shared__ __attribute__((aligned(16))) T sA2[sweep_transposes_a2<T, C, D, BV>() ? 4 * (C / 16) * 512 : 8];

    // Block order: the longer jobs start first, which matters when the grid
    // takes several rounds of the CUs. All reverse workgroups come first (with
    // both directions in the grid: a reverse step costs more than a forward
    // one), and varlen sequences are taken longest first (the chunk table's
    // order), so shorter jobs fill in behind. Within a direction, workgroups are
    // dispatched to the 8 XCDs round-robin by block id: with N H a multiple of
    // 8, the D/BV tiles of one (sequence, head) get block ids 8 apart (same
    // XCD, dispatched together), so they share the chunk operands (w, k~, q~,
    // do) through that XCD's L2 while they run; otherwise the V tile varies
    // slowest.
    constexpr int NV = D / BV;
    const int nh = p.N * p.H, per_dir = NV * nh;
    const int rd = blockIdx.x / per_dir;      // dirs = 1: the direction dir0 only
    const int dir = p.dirs == 2 ? 1 - rd : p.dir0;
    const int i = blockIdx.x % per_dir;
    int vt, hh;
    if (nh % 8 == 0) {
        vt = (i / 8) % NV;
        hh = (i / (8 * NV)) * 8 + i % 8;
    } else {
        vt = i / nh;
        hh = i % nh;
    }
    // varlen: sequences longest first (the chunk table's order)
    const int h = hh % p.H, n = p.varlen ? p.seq_ord[hh / p.H] : hh / p.H;
    if (dir == 0) sweep_run<T, C, D, BV, 0, NPF, SPREAD>(p, n, h, vt * BV, sS[0], sS[1], sX[0], sX[1], sDo[0], sDo[1], sA2);
    else sweep_run<T, C, D, BV, 1, NPF, SPREAD>(p, n, h, vt * BV, sS[0], sS[1], sX[0], sX[1], sDo[0], sDo[1], sA2);
}

}  // namespace gdr
