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
// collapses into one term; the FlashQLA page's CONSUMER_S role carries the
// same recurrence ("dS0 = g_last * dSt", "dS0 += K^T @ dVg", "dS0 += Q^T @
// dOg"). Columns of the state never mix (Diag acts on K, every product keeps
// the column), so a V tile per workgroup is exact. dh0 = dh_0 is written in
// fp32. The two directions are independent and share one grid.
//
// The per-chunk operands (w, k~, u, q~, 2^G_last) are read straight from
// global memory as MFMA fragments of the rows each wave owns, one chunk ahead
// (software pipelining: the loads for chunk c+1 are in flight while chunk c
// computes). Only the state and X / T (and do for the reverse direction)
// pass through LDS, double-buffered, two barriers per chunk.
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

// Operands of one chunk, as the MFMA fragments / values this lane needs.
template <typename T, int C, int D, int BV>
struct SweepOps {
    using S = SweepTiles<T, C, D, BV>;
    using F = typename Mfma<T>::frag;
    F a1[S::XRT][D / S::KS];      // chunk-row product A operand: w (fwd) or k~ (rev)
    F a2[S::SRW][C / S::KS];      // state update A operand: k~^T (fwd) or w^T (rev)
    F a3[S::SRW][C / S::KS];      // reverse only: (scale q~)^T
    float u[S::XRT][S::XCT][4];   // forward only: u at this lane's X elements
    float gl[S::SRW][4];          // 2^G_last at this lane's state rows
    static constexpr int NDO = (C * (BV / (16 / sizeof(T))) + 255) / 256;
    Vec16 dov[NDO];               // reverse only: this thread's 16-byte pieces of do
};

template <typename T, int C, int D, int BV>
__device__ __forceinline__ void sweep_load(SweepOps<T, C, D, BV>& o, const Params& p, int dir, int j,
                                           int h, int v0, int w) {
    using S = SweepTiles<T, C, D, BV>;
    const size_t jh = (size_t)j * p.H + h;
    const T* A1 = static_cast<const T*>(dir == 0 ? p.w : p.kt) + jh * C * D;
    const T* A2 = static_cast<const T*>(dir == 0 ? p.ktT : p.wT) + jh * D * C;
#pragma unroll
    for (int i = 0; i < S::XRT; ++i)
#pragma unroll
        for (int k = 0; k < D / S::KS; ++k) o.a1[i][k] = frag_kc(A1, D, 16 * S::xrow(w, i), k * S::KS);
#pragma unroll
    for (int i = 0; i < S::SRW; ++i)
#pragma unroll
        for (int k = 0; k < C / S::KS; ++k) o.a2[i][k] = frag_kc(A2, C, 16 * (w * S::SRW + i), k * S::KS);
    const float* gl = p.glast + jh * D;
#pragma unroll
    for (int i = 0; i < S::SRW; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) o.gl[i][e] = gl[16 * (w * S::SRW + i) + acc_row(e)];
    if (dir == 0) {
        const T* uT = static_cast<const T*>(p.uT) + jh * D * C;
#pragma unroll
        for (int i = 0; i < S::XRT; ++i)
#pragma unroll
            for (int jj = 0; jj < S::XCT; ++jj) {
                const int r = 16 * S::xrow(w, i) + acc_row(0);
                const int c = v0 + 16 * S::xcol(w, jj) + acc_col();
#pragma unroll
                for (int e = 0; e < 4; ++e) o.u[i][jj][e] = to_f32(uT[(size_t)c * C + r + e]);
            }
    } else {
        const T* qsT = static_cast<const T*>(p.qsT) + jh * D * C;
#pragma unroll
        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
            for (int k = 0; k < C / S::KS; ++k) o.a3[i][k] = frag_kc(qsT, C, 16 * (w * S::SRW + i), k * S::KS);
        // do rows of the chunk, this thread's 16-byte piece (zero past the sequence end)
        constexpr int V8 = 16 / sizeof(T);
        const ChunkEntry ce = p.ctab[j];
#pragma unroll
        for (int pi = 0; pi < o.NDO; ++pi) {
            const int e = threadIdx.x + 256 * pi;
            o.dov[pi] = Vec16{};
            if (e < C * (BV / V8)) {
                const int r = e / (BV / V8), cc = (e % (BV / V8)) * V8;
                if (r < ce.len)
                    o.dov[pi] = ld16(static_cast<const T*>(p.dout) + ((size_t)(ce.tok0 + r) * p.H + h) * D + v0 + cc);
            }
        }
    }
}

template <typename T, int C, int D, int BV>
__global__ __launch_bounds__(256) void gdr_sweep(Params p) {
    using S = SweepTiles<T, C, D, BV>;
    constexpr int NVT = D / BV, SCT = S::SCT, KS = S::KS;
    constexpr int LS = D + pad<T>();                 // state^T rows [BV][LS]
    constexpr int LX = C + pad<T>();                 // X^T / -T^T / do^T rows [BV][LX]
    constexpr int V8 = 16 / sizeof(T);
    __shared__ __attribute__((aligned(16))) T sS[BV * LS];
    __shared__ __attribute__((aligned(16))) T sX[2][BV * LX];
    __shared__ __attribute__((aligned(16))) T sDo[2][BV * LX];

    // Block order: the V tile varies slowest. Workgroups are dispatched to the
    // 8 XCDs round-robin by block id, so with 2 N H a multiple of 8 the NVT
    // tiles of one (direction, sequence, head) land on the same XCD and share
    // the chunk operands (w, k~, q~, do) through its L2.
    const int ngroups = 2 * p.N * p.H;
    const int vt = blockIdx.x / ngroups;
    int bid = blockIdx.x % ngroups;
    const int h = bid % p.H; bid /= p.H;
    const int n = bid % p.N;
    const int dir = bid / p.N;
    const int v0 = vt * BV;
    const int w = wave_id();
    const int c0 = p.seq_off[n], c1 = p.seq_off[n + 1];
    const int nch = c1 - c0;
    const size_t sh = ((size_t)n * p.H + h) * D * D;

    f32x4 st[S::SRW][SCT];
    {   // initial state: h0 (forward) or dht (reverse), zero when absent
        const float* init = dir == 0 ? p.h0 : p.dht;
#pragma unroll
        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
            for (int ct = 0; ct < SCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int d = 16 * (w * S::SRW + i) + acc_row(e), c = v0 + 16 * ct + acc_col();
                    st[i][ct][e] = init ? init[sh + (size_t)d * D + c] : 0.f;
                }
    }

    SweepOps<T, C, D, BV> cur, nxt;
    auto chunk_of = [&](int it) { return dir == 0 ? c0 + it : c1 - 1 - it; };
    if (nch > 0) sweep_load(cur, p, dir, chunk_of(0), h, v0, w);

    for (int it = 0; it < nch; ++it) {
        const int j = chunk_of(it);
        const int buf = it & 1;
        const size_t jh = (size_t)j * p.H + h;
        if (it + 1 < nch) sweep_load(nxt, p, dir, chunk_of(it + 1), h, v0, w);

        // 1. publish the incoming state: workspace (row-major, for the gradient
        //    kernel) and LDS (transposed: B operand with K contiguous)
        T* gS = static_cast<T*>(dir == 0 ? p.hbuf : p.dhbuf) + jh * D * D;
#pragma unroll
        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
            for (int ct = 0; ct < SCT; ++ct) {
                const int d = 16 * (w * S::SRW + i) + acc_row(0), c = 16 * ct + acc_col();
#pragma unroll
                for (int e = 0; e < 4; ++e) gS[(size_t)(d + e) * D + v0 + c] = from_f32<T>(st[i][ct][e]);
                store4<T>(sS + c * LS + d, st[i][ct][0], st[i][ct][1], st[i][ct][2], st[i][ct][3]);
            }
        if (dir == 1) {  // do^T of this chunk's V tile
#pragma unroll
            for (int pi = 0; pi < cur.NDO; ++pi) {
                const int e = threadIdx.x + 256 * pi;
                if (e < C * (BV / V8)) {
                    const int r = e / (BV / V8), cc = (e % (BV / V8)) * V8;
                    const T* xp = reinterpret_cast<const T*>(&cur.dov[pi]);
#pragma unroll
                    for (int q = 0; q < V8; ++q) sDo[buf][(cc + q) * LX + r] = xp[q];
                }
            }
        }
        __syncthreads();

        // 2. chunk-row product: X = u - w h (fwd) or T = k~ dh (rev)
        T* gX = static_cast<T*>(dir == 0 ? p.xbuf : p.tbuf) + jh * C * D;
#pragma unroll
        for (int i = 0; i < S::XRT; ++i)
#pragma unroll
            for (int jj = 0; jj < S::XCT; ++jj) {
                const int ct = S::xcol(w, jj);
                f32x4 acc = zero4();
#pragma unroll
                for (int k = 0; k < D / KS; ++k)
                    acc = Mfma<T>::mma(cur.a1[i][k], frag_kc(sS, LS, 16 * ct, k * KS), acc);
                const int r = 16 * S::xrow(w, i) + acc_row(0), c = 16 * ct + acc_col();
                float o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = dir == 0 ? cur.u[i][jj][e] - acc[e] : acc[e];
#pragma unroll
                for (int e = 0; e < 4; ++e) gX[(size_t)(r + e) * D + v0 + c] = from_f32<T>(o[e]);
                // forward keeps +X; reverse keeps -T so the state update is a pure sum
                const float sg = dir == 0 ? 1.f : -1.f;
                store4<T>(sX[buf] + c * LX + r, sg * o[0], sg * o[1], sg * o[2], sg * o[3]);
            }
        __syncthreads();

        // 3. state update: st = Diag(2^G_last) st + A2 X (+ (scale q~)^T do for reverse).
        //    The next chunk's step 1 rewrites sS (read only before the last barrier)
        //    and the other buffer of sX / sDo, so no third barrier is needed.
#pragma unroll
        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
            for (int ct = 0; ct < SCT; ++ct) {
#pragma unroll
                for (int e = 0; e < 4; ++e) st[i][ct][e] *= cur.gl[i][e];
#pragma unroll
                for (int k = 0; k < C / KS; ++k)
                    st[i][ct] = Mfma<T>::mma(cur.a2[i][k], frag_kc(sX[buf], LX, 16 * ct, k * KS), st[i][ct]);
                if (dir == 1) {
#pragma unroll
                    for (int k = 0; k < C / KS; ++k)
                        st[i][ct] = Mfma<T>::mma(cur.a3[i][k], frag_kc(sDo[buf], LX, 16 * ct, k * KS), st[i][ct]);
                }
            }
        cur = nxt;
    }
    if (dir == 1) {
#pragma unroll
        for (int i = 0; i < S::SRW; ++i)
#pragma unroll
            for (int ct = 0; ct < SCT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int d = 16 * (w * S::SRW + i) + acc_row(e), c = v0 + 16 * ct + acc_col();
                    p.dh0[sh + (size_t)d * D + c] = st[i][ct][e];
                }
    }
}

}  // namespace gdr
