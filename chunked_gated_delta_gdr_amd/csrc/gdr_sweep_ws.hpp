// gdr_sweep_ws.hpp -- the two state sweeps with loader waves, for 16-bit
// operands at D = 128: C = 64 with 32- or 64-column V tiles, C = 32 with
// 64-column tiles.
//
// Same recurrences, block order and workspace layouts as gdr_sweep (forward:
// X_c = u_c - w_c h_c, h_{c+1} = Diag(2^G_last) h_c + k~_c^T X_c; reverse:
// T_c = k~_c dh_{c+1}, dh_c = Diag(2^G_last) dh_{c+1} - w_c^T T_c +
// (scale q~_c)^T do_c), split over two kinds of waves in a 512-thread
// workgroup, as the producer and consumer roles of fused_bwd.py on the
// FlashQLA issue #30 page split theirs:
// - four compute waves hold the state in MFMA accumulators, run the two
//   products of each chunk step reading every operand from LDS, and store h
//   and X / T of the step;
// - four loader waves move the chunk operands from global memory straight
//   into LDS with 16-byte direct-to-LDS loads (no registers on the way) and
//   do nothing else, so their memory counter holds only those loads.
// Measured against gdr_sweep's register sets: headline sweep 121.1 -> 117.7
// us, 1024 chunks per sequence 1739 -> 1704 us; GDN GQA workload (C = 32,
// 64-column tiles) 889 -> 876 us; varlen workload (C = 64, 64-column tiles)
// 363 -> 350 us. (Loader waves that also stored h and X / T
// were no faster than the register sets: their waits for the next chunk's
// operands then also waited for those stores. A third buffer for the
// update's operands, two steps ahead, gained nothing more.)
//
// Two operand buffers, each split by when a step has finished with its part:
//   early: the chunk-row product's operands (w / k~ fragments, the update's
//          k~ / w tiles, forward u), free after that product;
//   late:  the update's operands ((scale q~)^T, do, 2^G_last), free at the
//          next step.
// Loader work in step k: after the step's first barrier (chunk k-1 done) the
// late part of chunk k+1; after the second (chunk k's product done) the early
// part of chunk k+2; then a wait for the late part of chunk k+1, and with it
// everything issued before, ahead of the next step's first barrier.
#pragma once
#include "gdr_sweep.hpp"

namespace gdr {

template <typename T, int C, int D, int BV>
struct SweepWs {
    static_assert(sizeof(T) == 2 && D == 128 && ((C == 64 && (BV == 32 || BV == 64)) || (C == 32 && BV == 64)),
                  "loader-wave sweep: 16-bit, D 128, C 64 with 32 or 64 columns, C 32 with 64");
    using S = SweepTiles<T, C, D, BV>;
    static constexpr int LS = D + pad<T>();   // state^T rows [BV][LS]
    static constexpr int LX = C + pad<T>();   // X^T / -T^T rows [BV][LX]
    // one operand buffer (bytes; forward u and reverse (scale q~)^T share a slot)
    static constexpr int A1 = 0;                       // fo C x D: w (fwd) / k~ (rev)
    static constexpr int A2 = A1 + C * D * 2;          // fo C x D: k~ (fwd) / w (rev), the update's A^T tiles
    static constexpr int U = A2 + C * D * 2;           // fwd: u^T of the tile, accumulator order (BV x C)
    static constexpr int A3 = A2 + C * D * 2;          // rev: fo D x C (scale q~)^T
    static constexpr int DO = A3 + D * C * 2;          // rev: do rows [C][BV], 16-byte pieces swizzled
    static constexpr int GL = DO + C * BV * 2;         // 2^G_last [D] fp32
    static constexpr int BUF = GL + D * 4;
    // 1 KB blocks of a C x D operand per loader wave; loads per loader wave in
    // the early part (forward, reverse)
    static constexpr int NBW = C * D / 2048;
    static constexpr int NUW = BV * C / 2048;     // 1 KB blocks of the u^T tile per loader wave
    static constexpr int NDW = C * BV / 8 / 256;  // do pieces per loader-wave lane
    static_assert(NUW * 2048 == BV * C && NDW * 2048 == C * BV, "whole blocks per loader wave");
    static constexpr int N_EARLY_F = 2 * NBW + NUW, N_EARLY_R = 2 * NBW;
    static constexpr int PPR = BV / 8;   // 16-byte pieces per do row
    // X / T single-buffered at C = 64 with 64 columns (to fit the LDS): every
    // read of step k's X is done before any wave passes step k+1's first
    // barrier, after which the next X is written
    static constexpr bool SX1 = C == 64 && BV == 64;
    static constexpr int TOTAL = 2 * BUF + (2 * BV * LS + (SX1 ? 1 : 2) * BV * LX) * 2;
};

// 16 bytes per lane from global memory to LDS (lane l writes lds + 16 l; the
// LDS address must be the same for the whole wave)
__device__ __forceinline__ void dma16(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 encoding; the other counters left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// do rows [C][BV] in LDS as 16-byte pieces, XOR-swizzled by row so that the
// transposed reads of four consecutive rows (two pieces each) cover all 32
// banks once: 32 columns (64-byte rows, two rows per bank window) piece pc of
// row r at 4 r + (pc ^ 2 ((r >> 1) & 1)); 64 columns (128-byte rows) at
// 8 r + (pc ^ 2 (r & 3))
template <int BV>
__device__ __forceinline__ int do_slot(int r, int pc) {
    if constexpr (BV == 32) return 4 * r + (pc ^ (((r >> 1) & 1) << 1));
    else return 8 * r + (pc ^ ((r & 3) << 1));
}

// do^T fragment (v columns i0 + (l & 15), rows k0 + 8 (l >> 4) + 0..7) from
// those swizzled rows: two transposed loads, as frag_ks
template <typename T, int BV>
__device__ __forceinline__ typename Mfma<T>::frag frag_do_ws(const T* rows, int i0, int k0, int l) {
    auto piece = [&](int kk) {
        const int r = kk + ((l & 15) >> 2), c = i0 + 4 * (l & 3);
        const T* q = rows + do_slot<BV>(r, c >> 3) * 8 + (c & 7);
        return __builtin_bit_cast(
            uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(q)));
    };
    const uint64_t v[2] = {piece(k0 + 8 * (l >> 4)), piece(k0 + 8 * (l >> 4) + 4)};
    typename Mfma<T>::frag f;
    __builtin_memcpy(&f, v, sizeof(f));
    return f;
}

// frag_fo_tr on fragment-order tiles TS elements apart
template <typename T, int TS>
__device__ __forceinline__ typename Mfma<T>::frag frag_fo_tr_s(const T* tiles, int i0, int k0, int l) {
    auto piece = [&](int kk) {
        const int c = kk + ((l & 15) >> 2), d = i0 + 4 * (l & 3);
        const T* q = tiles + (c >> 4) * TS + ((c & 15) + 16 * (d >> 3)) * 8 + (d & 7);
        return __builtin_bit_cast(
            uint64_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(q)));
    };
    const uint64_t v[2] = {piece(k0 + 8 * (l >> 4)), piece(k0 + 8 * (l >> 4) + 4)};
    typename Mfma<T>::frag f;
    __builtin_memcpy(&f, v, sizeof(f));
    return f;
}

template <typename T, int C, int D, int BV, int DIR>
__device__ __forceinline__ void sweep_run_ws(const Params& p, int n, int h, int v0, char* lds) {
    using W = SweepWs<T, C, D, BV>;
    using S = typename W::S;
    using F = typename Mfma<T>::frag;
    using Q = typename Mfma<T>::quad;
    constexpr int SCT = S::SCT, KS = S::KS, LS = W::LS, LX = W::LX;
    T* const sS0 = reinterpret_cast<T*>(lds + 2 * W::BUF);
    T* const sS1 = sS0 + BV * LS;
    T* const sX0 = sS1 + BV * LS;
    T* const sX1 = W::SX1 ? sX0 : sX0 + BV * LX;
    char* const ob0 = lds;
    char* const ob1 = lds + W::BUF;
    // the wave's role must be a uniform branch: both roles hold barriers
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int c0 = p.seq_off[n], c1 = p.seq_off[n + 1];
    const int nch = c1 - c0;
    int stok0, slen;
    seq_span(p, n, stok0, slen);
    auto chunk_it = [&](int k) { return DIR == 0 ? k : nch - 1 - k; };

    if (w < 4) {
        // ---------------- compute waves ----------------
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
        if (nch > 0) {
            __syncthreads();   // chunk 0's operands in LDS
            const int l = lane_id();
            for (int k = 0; k < nch; ++k) {
                const char* ob = (k & 1) ? ob1 : ob0;
                T* sS = (k & 1) ? sS1 : sS0;
                T* sX = (k & 1) ? sX1 : sX0;
                // 1. the incoming state to LDS, transposed (B operand, K contiguous)
#pragma unroll
                for (int i = 0; i < S::SRW; ++i)
#pragma unroll
                    for (int ct = 0; ct < SCT; ++ct) {
                        const int d = 16 * (w * S::SRW + i) + acc_row(0), c = 16 * ct + acc_col();
                        store4<T>(sS + c * LS + (d ^ sweep_swz<T, C, BV, D>(c)), st[i][ct][0], st[i][ct][1], st[i][ct][2],
                                  st[i][ct][3]);
                    }
                __syncthreads();
                // 2. chunk-row product X = u - w h (fwd) / -T = -k~ dh (rev); all
                //    fragments read ahead of the products
                {
                    const T* A1 = reinterpret_cast<const T*>(ob + W::A1);
                    const T* A2 = reinterpret_cast<const T*>(ob + W::A2);
                    F bx[S::XCT][D / KS], a1f[S::XRT][D / KS];
                    Q uq[DIR == 0 ? S::XRT : 1][S::XCT];
#pragma unroll
                    for (int jj = 0; jj < S::XCT; ++jj)
#pragma unroll
                        for (int k2 = 0; k2 < D / KS; ++k2) bx[jj][k2] = frag_kc_swz<T, C, BV, D>(sS, LS, 16 * S::xcol(w, jj), k2 * KS, l);
#pragma unroll
                    for (int i = 0; i < S::XRT; ++i)
#pragma unroll
                        for (int k2 = 0; k2 < D / KS; ++k2)
                            a1f[i][k2] = *reinterpret_cast<const F*>(A1 + (S::xrow(w, i) * (D / 32) + k2) * 512 + l * 8);
                    if constexpr (DIR == 0) {
                        const T* Ul = reinterpret_cast<const T*>(ob + W::U);
#pragma unroll
                        for (int i = 0; i < S::XRT; ++i)
#pragma unroll
                            for (int jj = 0; jj < S::XCT; ++jj)
                                uq[i][jj] = *reinterpret_cast<const Q*>(
                                    Ul + ao_index<C>(16 * S::xcol(w, jj) + acc_col(l), 16 * S::xrow(w, i) + acc_row(0, l)));
                    }
                    F a2f[S::SRW][C / KS];
#pragma unroll
                    for (int i = 0; i < S::SRW; ++i)
#pragma unroll
                        for (int k2 = 0; k2 < C / KS; ++k2)
                            a2f[i][k2] = frag_fo_tr_s<T, (D / 32) * 512>(A2 + w * 512, 16 * i, k2 * KS, l);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < S::XRT; ++i) {
                        f32x4 acc[S::XCT];
#pragma unroll
                        for (int jj = 0; jj < S::XCT; ++jj) acc[jj] = zero4();
#pragma unroll
                        for (int k2 = 0; k2 < D / KS; ++k2)
#pragma unroll
                            for (int jj = 0; jj < S::XCT; ++jj) acc[jj] = Mfma<T>::mma(a1f[i][k2], bx[jj][k2], acc[jj]);
#pragma unroll
                        for (int jj = 0; jj < S::XCT; ++jj) {
                            const int r = 16 * S::xrow(w, i) + acc_row(0, l), c = 16 * S::xcol(w, jj) + acc_col(l);
                            float o[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) o[e] = DIR == 0 ? to_f32(uq[i][jj][e]) - acc[jj][e] : -acc[jj][e];
                            store4<T>(sX + c * LX + (r ^ sweep_swz<T, C, BV, C>(c)), o[0], o[1], o[2], o[3]);
                        }
                    }
                    __syncthreads();
                    // 3. state update: st = Diag(2^G_last) st + A2 X (+ (scale q~)^T do)
                    F bxs[SCT][C / KS], bdo[DIR == 1 ? SCT : 1][C / KS], a3f[DIR == 1 ? S::SRW : 1][C / KS];
                    f32x4 gl[S::SRW];
                    const float* G = reinterpret_cast<const float*>(ob + W::GL);
#pragma unroll
                    for (int ct = 0; ct < SCT; ++ct)
#pragma unroll
                        for (int k2 = 0; k2 < C / KS; ++k2) {
                            bxs[ct][k2] = frag_kc_swz<T, C, BV, C>(sX, LX, 16 * ct, k2 * KS, l);
                            if constexpr (DIR == 1)
                                bdo[ct][k2] = frag_do_ws<T, BV>(reinterpret_cast<const T*>(ob + W::DO), 16 * ct, k2 * KS, l);
                        }
                    if constexpr (DIR == 1) {
                        const T* A3 = reinterpret_cast<const T*>(ob + W::A3);
#pragma unroll
                        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
                            for (int k2 = 0; k2 < C / KS; ++k2)
                                a3f[i][k2] = *reinterpret_cast<const F*>(A3 + ((w * S::SRW + i) * (C / 32) + k2) * 512 + l * 8);
                    }
#pragma unroll
                    for (int i = 0; i < S::SRW; ++i)
                        gl[i] = *reinterpret_cast<const f32x4*>(G + 16 * (w * S::SRW + i) + acc_row(0, l));
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int i = 0; i < S::SRW; ++i)
#pragma unroll
                        for (int ct = 0; ct < SCT; ++ct)
#pragma unroll
                            for (int e = 0; e < 4; ++e) st[i][ct][e] *= gl[i][e];
#pragma unroll
                    for (int k2 = 0; k2 < C / KS; ++k2)
#pragma unroll
                        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
                            for (int ct = 0; ct < SCT; ++ct) st[i][ct] = Mfma<T>::mma(a2f[i][k2], bxs[ct][k2], st[i][ct]);
                    if constexpr (DIR == 1) {
#pragma unroll
                        for (int k2 = 0; k2 < C / KS; ++k2)
#pragma unroll
                            for (int i = 0; i < S::SRW; ++i)
#pragma unroll
                                for (int ct = 0; ct < SCT; ++ct) st[i][ct] = Mfma<T>::mma(a3f[i][k2], bdo[ct][k2], st[i][ct]);
                    }
                }
                {   // the incoming state and X (T) of this chunk to the workspace,
                    // read back from LDS while the update's MFMAs run, row-major
                    // pieces of 8 columns: through transposed loads at 32 columns,
                    // through 16-bit reads of the swizzled buffers at 64 (as gdr_sweep)
                    const int it = chunk_it(k);
                    const size_t jh = (size_t)(c0 + it) * p.H + h;
                    T* gS = static_cast<T*>(DIR == 0 ? p.hbuf : p.dhbuf) + jh * D * D;
                    T* gX = static_cast<T*>(DIR == 0 ? p.xbuf : p.tbuf) + jh * C * D;
                    if constexpr (BV == 32) {
#pragma unroll
                        for (int t2 = 0; t2 < 2; ++t2) {
                            const int dt = w + 4 * t2;
                            const uint64_t a = ks_tr4_bits(sS, LS, 16 * dt, 0, 8, l);
                            const uint64_t b = ks_tr4_bits(sS, LS, 16 * dt, 4, 8, l);
                            const Vec16 v = {{uint32_t(a), uint32_t(a >> 32), uint32_t(b), uint32_t(b >> 32)}};
                            st16(gS + tiled_index<D, BV>(16 * dt + (l & 15), v0, 8 * (l >> 4)), v);
                        }
                        constexpr uint64_t kNeg = DIR == 0 ? 0 : 0x8000800080008000ull;
                        const uint64_t a = ks_tr4_bits(sX, LX, 16 * w, 0, 8, l) ^ kNeg;
                        const uint64_t b = ks_tr4_bits(sX, LX, 16 * w, 4, 8, l) ^ kNeg;
                        const Vec16 v = {{uint32_t(a), uint32_t(a >> 32), uint32_t(b), uint32_t(b >> 32)}};
                        st16(gX + tiled_index<C, BV>(16 * w + (l & 15), v0, 8 * (l >> 4)), v);
                    } else {
                        constexpr int V8 = 16 / sizeof(T), NPS = D * BV / V8, NPX = C * BV / V8;
                        static_assert(NPS % 256 == 0 && NPX % 256 == 0, "whole rounds of the compute threads");
#pragma unroll
                        for (int pi = 0; pi < NPS / 256; ++pi) {
                            const int e = (int)threadIdx.x + 256 * pi;
                            const int d = e / (BV / V8), c = (e % (BV / V8)) * V8;
                            Vec16 v;
                            T* vp = reinterpret_cast<T*>(&v);
#pragma unroll
                            for (int q = 0; q < V8; ++q) vp[q] = sS[(c + q) * LS + (d ^ sweep_swz<T, C, BV, D>(c + q))];
                            st16(gS + tiled_index<D, BV>(d, v0, c), v);
                        }
#pragma unroll
                        for (int pi = 0; pi < NPX / 256; ++pi) {
                            const int e = (int)threadIdx.x + 256 * pi;
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
            }
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
        return;
    }

    // ---------------- loader waves ----------------
    // (no compiler-visible LDS read here: one would be made to wait for the
    // direct-to-LDS loads in flight)
    if (nch == 0) return;
    const int lw = w - 4, l = lane_id();
    // operands of step k's chunk (past the end: the last chunk again, a
    // redundant valid load into a buffer no step reads any more)
    auto early = [&](int k, char* ob) __attribute__((always_inline)) {
        const int it = chunk_it(k < nch ? k : nch - 1);
        const size_t jh = (size_t)(c0 + it) * p.H + h;
        const T* A1g = static_cast<const T*>(DIR == 0 ? p.w : p.kt) + jh * C * D;
        const T* A2g = static_cast<const T*>(DIR == 0 ? p.kt : p.w) + jh * C * D;
#pragma unroll
        for (int b = 0; b < W::NBW; ++b) dma16(A1g + (lw * W::NBW + b) * 512 + l * 8, ob + W::A1 + (lw * W::NBW + b) * 1024);
#pragma unroll
        for (int b = 0; b < W::NBW; ++b) dma16(A2g + (lw * W::NBW + b) * 512 + l * 8, ob + W::A2 + (lw * W::NBW + b) * 1024);
        if constexpr (DIR == 0) {
            const T* Ug = static_cast<const T*>(p.uT) + jh * D * C + (v0 / 16) * (C / 16) * 256;
#pragma unroll
            for (int b = 0; b < W::NUW; ++b) dma16(Ug + (lw * W::NUW + b) * 512 + l * 8, ob + W::U + (lw * W::NUW + b) * 1024);
        }
    };
    auto late = [&](int k, char* ob) __attribute__((always_inline)) {
        const int it = chunk_it(k < nch ? k : nch - 1);
        const size_t jh = (size_t)(c0 + it) * p.H + h;
        if constexpr (DIR == 1) {
            const T* A3g = static_cast<const T*>(p.qsT) + jh * D * C;
#pragma unroll
            for (int b = 0; b < W::NBW; ++b) dma16(A3g + (lw * W::NBW + b) * 512 + l * 8, ob + W::A3 + (lw * W::NBW + b) * 1024);
            // do: this lane's LDS slot s holds piece pc of row r; rows past the
            // sequence end read its last row and are zeroed once landed
            const int len = min(C, slen - it * C);
#pragma unroll
            for (int b = 0; b < W::NDW; ++b) {
                const int s = (lw * W::NDW + b) * 64 + l, r = s / W::PPR, pc0 = s % W::PPR;
                const int pc = do_slot<BV>(r, pc0) - W::PPR * r;   // the slot map is an involution within a row
                const int rr = min(r, len - 1);
                dma16(static_cast<const T*>(p.dout) + ((size_t)(stok0 + it * C + rr) * p.H + h) * D + v0 + 8 * pc,
                      ob + W::DO + (lw * W::NDW + b) * 1024);
            }
        }
        const float* Gg = p.glast + jh * D;
        if (l < 8) dma16(Gg + (lw * 8 + l) * 4, ob + W::GL + lw * 128);
    };
    // after the late part of step k's chunk has landed: its do rows past the
    // sequence end to zero (each wave its own slots)
    auto zero_tail = [&](int k, char* ob) __attribute__((always_inline)) {
        if constexpr (DIR == 1) {
            if (k < nch) {
                const int it = chunk_it(k);
                const int len = min(C, slen - it * C);
#pragma unroll
                for (int b = 0; b < W::NDW; ++b) {
                    const int s = (lw * W::NDW + b) * 64 + l, r = s / W::PPR;
                    if (r >= len) st16(ob + W::DO + s * 16, Vec16{});
                }
            }
        }
    };
    constexpr int NE = DIR == 0 ? W::N_EARLY_F : W::N_EARLY_R;
    early(0, ob0);
    late(0, ob0);
    early(1, ob1);
    wait_vm<NE>();     // chunk 0 in LDS (the early part of chunk 1 may be in flight)
    zero_tail(0, ob0);
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    for (int k = 0; k < nch; ++k) {
        char* obn = (k & 1) ? ob0 : ob1;   // chunk k+1's buffer
        char* obc = (k & 1) ? ob1 : ob0;   // chunk k's (and k+2's)
        __builtin_amdgcn_s_barrier();      // state published
        late(k + 1, obn);
        __builtin_amdgcn_s_barrier();      // X / T written
        early(k + 2, obc);
        // the late part of chunk k+1 (and everything before it) has landed
        wait_vm<NE>();
        zero_tail(k + 1, obn);
        wait_lgkm0();
    }
}

// One workgroup of 512 threads per (direction, sequence, head, V tile), in
// the block order of gdr_sweep.
template <typename T, int C, int D, int BV>
__global__ __launch_bounds__(512) void gdr_sweep_ws(Params p) {
    static_assert(kTileV % BV == 0 || BV % kTileV == 0, "sweep V tiles and stored tiles nest");
    using W = SweepWs<T, C, D, BV>;
    __shared__ __attribute__((aligned(16))) char lds[W::TOTAL];
    constexpr int NV = D / BV;
    const int nh = p.N * p.H, per_dir = NV * nh;
    const int rd = blockIdx.x / per_dir;
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
    const int h = hh % p.H, n = p.varlen ? p.seq_ord[hh / p.H] : hh / p.H;
    if (dir == 0) sweep_run_ws<T, C, D, BV, 0>(p, n, h, vt * BV, lds);
    else sweep_run_ws<T, C, D, BV, 1>(p, n, h, vt * BV, lds);
}

}  // namespace gdr
