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
// Per-chunk operands (w, k~, u, q~) are read straight from global memory as
// MFMA fragments of the rows each wave owns; only the state and X / T pass
// through LDS, where every wave needs all of them.
#pragma once
#include "gdr_common.hpp"

namespace gdr {

template <typename T, int C, int D, int BV>
__global__ __launch_bounds__(256) void gdr_sweep(Params p) {
    constexpr int NVT = D / BV;
    constexpr int SRT = D / 16, SCT = BV / 16;       // state tiles
    constexpr int SPW = SRT * SCT / 4;               // state tiles per wave
    constexpr int XPW = (C / 16) * SCT / 4;          // X / T tiles per wave
    static_assert(SPW >= 1 && XPW >= 1 && (SRT * SCT) % 4 == 0 && ((C / 16) * SCT) % 4 == 0, "tiling");
    constexpr int LS = D + pad<T>();                 // state^T rows [BV][LS]
    constexpr int LX = C + pad<T>();                 // X^T / T^T / do^T rows [BV][LX]
    __shared__ __attribute__((aligned(16))) T sS[BV * LS];
    __shared__ __attribute__((aligned(16))) T sX[BV * LX];
    __shared__ __attribute__((aligned(16))) T sDo[BV * LX];

    int bid = blockIdx.x;
    const int vt = bid % NVT; bid /= NVT;
    const int h = bid % p.H; bid /= p.H;
    const int n = bid % p.N;
    const int dir = bid / p.N;
    const int v0 = vt * BV;
    const int w = wave_id();
    const int c0 = p.seq_off[n], c1 = p.seq_off[n + 1];
    const size_t sh = ((size_t)n * p.H + h) * D * D;

    f32x4 st[SPW];
    // initial state: h0 (forward) or dht (reverse), zero when absent
    {
        const float* init = dir == 0 ? p.h0 : p.dht;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int t = w * SPW + i, rt = t / SCT, ct = t % SCT;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = 16 * rt + acc_row(e), c = v0 + 16 * ct + acc_col();
                st[i][e] = init ? init[sh + (size_t)d * D + c] : 0.f;
            }
        }
    }

    const T* dout = static_cast<const T*>(p.dout);
    for (int it = 0; it < c1 - c0; ++it) {
        const int j = dir == 0 ? c0 + it : c1 - 1 - it;
        const size_t jh = (size_t)j * p.H + h;
        const float* gl = p.glast + jh * D;
        // 1. publish the incoming state: workspace (row-major, for the gradient
        //    kernel) and LDS (transposed, B operand with K contiguous)
        T* gS = static_cast<T*>(dir == 0 ? p.hbuf : p.dhbuf) + jh * D * D;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int t = w * SPW + i, rt = t / SCT, ct = t % SCT;
            const int d = 16 * rt + acc_row(0), c = 16 * ct + acc_col();
#pragma unroll
            for (int e = 0; e < 4; ++e) gS[(size_t)(d + e) * D + v0 + c] = from_f32<T>(st[i][e]);
            store4<T>(sS + c * LS + d, st[i][0], st[i][1], st[i][2], st[i][3]);
        }
        if (dir == 1) {  // do^T of this chunk's V tile (zero past the sequence end)
            const ChunkEntry ce = p.ctab[j];
            constexpr int V8 = 16 / sizeof(T);
            for (int e = threadIdx.x; e < C * (BV / V8); e += 256) {
                const int r = e / (BV / V8), cc = (e % (BV / V8)) * V8;
                Vec16 x{};
                if (r < ce.len) x = ld16(dout + ((size_t)(ce.tok0 + r) * p.H + h) * D + v0 + cc);
                const T* xp = reinterpret_cast<const T*>(&x);
#pragma unroll
                for (int q = 0; q < V8; ++q) sDo[(cc + q) * LX + r] = xp[q];
            }
        }
        __syncthreads();
        // 2. chunk-row product: X = u - w h (fwd) or T = k~ dh (rev)
        const T* Arow = static_cast<const T*>(dir == 0 ? p.w : p.kt) + jh * C * D;
        T* gX = static_cast<T*>(dir == 0 ? p.xbuf : p.tbuf) + jh * C * D;
        const T* uT = static_cast<const T*>(p.uT) + jh * D * C;
#pragma unroll
        for (int i = 0; i < XPW; ++i) {
            const int t = w * XPW + i, rt = t / SCT, ct = t % SCT;
            f32x4 acc = zero4();
#pragma unroll
            for (int k0 = 0; k0 < D; k0 += kstep<T>())
                acc = Mfma<T>::mma(frag_kc(Arow, D, 16 * rt, k0), frag_kc(sS, LS, 16 * ct, k0), acc);
            const int r = 16 * rt + acc_row(0), c = 16 * ct + acc_col();
            float o[4];
            if (dir == 0) {
                const T* up = uT + (size_t)(v0 + c) * C + r;
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = to_f32(up[e]) - acc[e];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = acc[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) gX[(size_t)(r + e) * D + v0 + c] = from_f32<T>(o[e]);
            // forward keeps +X; reverse keeps -T so the state update is a pure sum
            const float sg = dir == 0 ? 1.f : -1.f;
            store4<T>(sX + c * LX + r, sg * o[0], sg * o[1], sg * o[2], sg * o[3]);
        }
        __syncthreads();
        // 3. state update: st = Diag(2^G_last) st + A2 * sX (+ qs^T do^T for reverse)
        const T* A2 = static_cast<const T*>(dir == 0 ? p.ktT : p.wT) + jh * D * C;
        const T* qsT = static_cast<const T*>(p.qsT) + jh * D * C;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int t = w * SPW + i, rt = t / SCT, ct = t % SCT;
#pragma unroll
            for (int e = 0; e < 4; ++e) st[i][e] *= gl[16 * rt + acc_row(e)];
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += kstep<T>())
                st[i] = Mfma<T>::mma(frag_kc(A2, C, 16 * rt, k0), frag_kc(sX, LX, 16 * ct, k0), st[i]);
            if (dir == 1) {
#pragma unroll
                for (int k0 = 0; k0 < C; k0 += kstep<T>())
                    st[i] = Mfma<T>::mma(frag_kc(qsT, C, 16 * rt, k0), frag_kc(sDo, LX, 16 * ct, k0), st[i]);
            }
        }
        // the next iteration's first barrier orders these LDS reads before the
        // next writes of sX / sDo; sS is only rewritten after this point
        __syncthreads();
    }
    if (dir == 1) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int t = w * SPW + i, rt = t / SCT, ct = t % SCT;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = 16 * rt + acc_row(e), c = v0 + 16 * ct + acc_col();
                p.dh0[sh + (size_t)d * D + c] = st[i][e];
            }
        }
    }
}

}  // namespace gdr
