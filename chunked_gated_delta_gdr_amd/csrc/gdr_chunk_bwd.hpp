// gdr_chunk_bwd.hpp -- chunk-parallel gradient kernel.
//
// One workgroup per (chunk, q/k head); it loops over the value heads of the
// GQA group and sums dq / dk over them in fp32. Wave w owns rows 16w..16w+15
// (diagonal block w) of every [C][*] product. With h = h_c, dh' = dh_{c+1},
// X = u - w h (forward sweep) and T = k~ dh' (reverse sweep):
//   dX  = scale Aqk^T do + T
//   dAqk = scale Lower_incl(do X^T)          (the FlashQLA page's dP step)
//   dq^  = scale do h^T  -> dq += dq^ 2^G
//   dk~  = X dh'^T       -> dk += dk~ 2^(G_last - G)
//   dw   = -dX h^T;  dv^ = A^T dX -> dv = beta dv^
//   dk^  = A^T dw       -> dk += beta 2^G dk^
//   dA   = (dX v^T + dw (k 2^G)^T) Diag(beta)
//   dAkk = -StrictLower(A^T dA A^T)          (the page's "dA = -Ar^T @ dAr @ Ar^T")
// then the intra-chunk gradient of Aqk / Akk (the bwd_intra page):
//   accq_r = sum_{s<=r} dAqk[r,s] k_s 2^(G_r-G_s),  acck_r = sum_{s<r} dAkk[r,s] k_s 2^(G_r-G_s)
//   dkt_s  = sum_{r>=s} (dAqk[r,s] q_r + dAkk[r,s] beta_r k_r) 2^(G_r-G_s)
//   dq += accq, dk += beta acck + dkt, db += k . acck,
//   dG += ln2 [q accq + k (beta acck - dkt)],
// cross-block terms on MFMA through the block boundary rho (q/k prescaled by
// 2^(G - G_rho) or 2^(G_rho - G), post-factors 2^(G_r - G_rho) and
// 2^(G_rho - G_s), every exponent <= 0), the diagonal 16x16 blocks on VALU
// with one running decay per (r, s, d). Finally dg = reverse cumsum of dG in
// the chunk (the page's fold_dg), dG_last collecting
//   ln2 [2^G_last rowsum_v(h dh') + sum_r k_r dk~_r 2^(G_last - G_r)].
#pragma once
#include "gdr_common.hpp"

namespace gdr {

template <typename T, int C, int D>
struct BwdLds {
    static constexpr int NB = C / 16;
    static constexpr int BVS = sizeof(T) == 4 ? 16 : 32;  // V slice of the state products
    static constexpr int LT = D + pad<T>();
    static constexpr int LC = C + pad<T>();
    static constexpr int LB = BVS + pad<T>();
    static constexpr int LF = D + 4;
    static constexpr int KSTEP = 4 * Mfma<T>::KL;
    static constexpr int rup(int x) { return (x + KSTEP - 1) / KSTEP * KSTEP; }
    static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
    static constexpr size_t sz(int rows, int ld, int bytes) { return size_t(rows) * ld * bytes; }
    // persistent
    static constexpr size_t Q_OFF = 0;
    static constexpr size_t K_OFF = Q_OFF + sz(C, LT, sizeof(T));
    static constexpr size_t BETA_OFF = K_OFF + sz(C, LT, sizeof(T));        // f32 [C]
    static constexpr size_t DB_OFF = BETA_OFF + C * 4;                       // f32 [C]
    static constexpr size_t GL_OFF = DB_OFF + C * 4;                         // f32 [D] dG_last
    static constexpr size_t GLW_OFF = GL_OFF + D * 4;                        // f32 [NB][D] per-wave dG_last
    static constexpr size_t BT_OFF = GLW_OFF + size_t(NB) * D * 4;           // f32 [NB][D] block totals
    static constexpr size_t DIAG_OFF = BT_OFF + size_t(NB) * D * 4;          // f32 [2][NB][16][16]
    static constexpr size_t U_OFF = DIAG_OFF + size_t(2) * NB * 256 * 4;     // union region
    // phase 1 (state products, one V slice)
    static constexpr size_t P1_DOT = 0;                                      // T [BVS][LC]
    static constexpr size_t P1_XL = P1_DOT + sz(BVS, LC, sizeof(T));         // T [C][LB]
    static constexpr size_t P1_HL = P1_XL + sz(C, LB, sizeof(T));            // T [D][LB]
    static constexpr size_t P1_DHL = P1_HL + sz(D, LB, sizeof(T));           // T [D][LB]
    static constexpr size_t P1_DXL = P1_DHL + sz(D, LB, sizeof(T));          // T [C][LB]
    static constexpr size_t P1_DXT = P1_DXL + sz(C, LB, sizeof(T));          // T [BVS][LC]
    static constexpr size_t P1_VL = P1_DXT + sz(BVS, LC, sizeof(T));         // T [C][LB]
    static constexpr size_t P1_END = P1_VL + sz(C, LB, sizeof(T));
    // phase 2: Gs lives from 2a to the end of the cross terms
    static constexpr size_t P2_GS = 0;                                       // f32 [C][LF]
    static constexpr size_t P2_A = P2_GS + sz(C, LF, 4);
    //   2b-2e
    static constexpr size_t P2_DWT = P2_A;                                   // T [D][LC]
    static constexpr size_t P2_DWL = P2_DWT + sz(D, LC, sizeof(T));          // T [C][LT]
    static constexpr size_t P2_KG = P2_DWL + sz(C, LT, sizeof(T));           // T [C][LT]
    static constexpr size_t P2_DAL = P2_KG + sz(C, LT, sizeof(T));           // T [C][LC]
    static constexpr size_t P2_T1T = P2_DAL + sz(C, LC, sizeof(T));          // T [C][LC]
    static constexpr size_t P2_B_END = P2_T1T + sz(C, LC, sizeof(T));
    //   2e-2f: dAqk / dAkk operands (row-major and transposed) over the dead
    //   dw / k 2^G / dA buffers; they must stay clear of T1T, still read in 2e
    static constexpr size_t P2_DAQ = P2_A;                                   // T [C][LC] x4
    static constexpr size_t P2_DA_END = P2_DAQ + 4 * sz(C, LC, sizeof(T));
    //   2f: prescaled cross operands for one boundary and one D chunk of DH
    //   columns: k^T [DH][rup(rho)], q^T and (beta k)^T [DH][rup(C-rho)]
    static constexpr int DH = sizeof(T) == 4 ? 32 : 64;
    static constexpr int cross_cols(int rho) { return rup(rho) + 2 * rup(C - rho) + 3 * pad<T>(); }
    static constexpr int max_cross_cols() {
        int m = 0;
        for (int rho = 16; rho < C; rho += 16) m = cross_cols(rho) > m ? cross_cols(rho) : m;
        return m;
    }
    static constexpr size_t P2_X = P2_DA_END;
    static constexpr size_t P2_X_END = P2_X + sz(DH, max_cross_cols(), sizeof(T));
    // phase 3: three fp32 exchange buffers [C][LF] for the diagonal pass
    static constexpr size_t P3_EX = 0;
    static constexpr size_t P3_END = 3 * sz(C, LF, 4);
    static constexpr size_t U_BYTES = cmax(cmax(P1_END, cmax(P2_B_END, P2_X_END)), P3_END);
    static constexpr size_t TOTAL = U_OFF + U_BYTES;
    static_assert(P2_DA_END <= P2_T1T, "dAqk/dAkk operands must not overlap T1T");
    static_assert(TOTAL <= 163840, "LDS budget of gdr_chunk_bwd");
};

// Fragment of rows [i0, i0+16) of a global token-major matrix: element
// (i, kk) at p[i*ld + kk]; rows >= nrows (past the sequence end) read as zero.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag_rows(const T* p, long ld, int i0, int k0, int nrows) {
    const int l = lane_id();
    const int i = i0 + (l & 15);
    typename Mfma<T>::frag f;
    if (i < nrows) {
        f = *reinterpret_cast<const typename Mfma<T>::frag*>(p + (long)i * ld + k0 + (l >> 4) * Mfma<T>::KL);
    } else {
        if constexpr (Mfma<T>::KL == 1) f = 0.f;
        else {
#pragma unroll
            for (int q = 0; q < Mfma<T>::KL; ++q) f[q] = (T)0.f;
        }
    }
    return f;
}

template <typename T, int C, int D, bool SCALAR>
__global__ __launch_bounds__(64 * (C / 16)) void gdr_chunk_bwd(Params p) {
    using L = BwdLds<T, C, D>;
    constexpr int NB = L::NB, NT = 64 * NB, BVS = L::BVS;
    constexpr int LT = L::LT, LC = L::LC, LB = L::LB, LF = L::LF;
    constexpr int NTD = D / 16, NTC = C / 16, NTV = BVS / 16;
    constexpr int V8 = 16 / sizeof(T);
    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    T* qL = reinterpret_cast<T*>(smem + L::Q_OFF);
    T* kL = reinterpret_cast<T*>(smem + L::K_OFF);
    float* bs = reinterpret_cast<float*>(smem + L::BETA_OFF);
    float* dbS = reinterpret_cast<float*>(smem + L::DB_OFF);
    float* dGl = reinterpret_cast<float*>(smem + L::GL_OFF);
    float* dGlw = reinterpret_cast<float*>(smem + L::GLW_OFF);
    float* btot = reinterpret_cast<float*>(smem + L::BT_OFF);
    float* dqD = reinterpret_cast<float*>(smem + L::DIAG_OFF);   // [NB][16 s][16 r] dAqk
    float* dkD = dqD + NB * 256;                                   // [NB][16 s][16 r] dAkk
    char* U = smem + L::U_OFF;

    const int j = blockIdx.x, hk = blockIdx.y;
    if (j >= p.seq_off[p.N]) return;
    const ChunkEntry ce = p.ctab[j];
    const int tok0 = ce.tok0, len = ce.len;
    const int tid = threadIdx.x, w = wave_id(), l = lane_id();
    const int r0 = 16 * w;  // this wave's rows
    const T* q = static_cast<const T*>(p.q);
    const T* k = static_cast<const T*>(p.k);
    const T* v = static_cast<const T*>(p.v);
    const T* dout = static_cast<const T*>(p.dout);
    const T* beta = static_cast<const T*>(p.beta);

    // q, k rows of this chunk (zero past the sequence end)
    for (int e = tid; e < C * (D / V8); e += NT) {
        const int r = e / (D / V8), d0 = (e % (D / V8)) * V8;
        Vec16 qv{}, kv{};
        if (r < len) {
            qv = ld16(q + ((size_t)(tok0 + r) * p.Hg + hk) * D + d0);
            kv = ld16(k + ((size_t)(tok0 + r) * p.Hg + hk) * D + d0);
        }
        st16(qL + r * LT + d0, qv);
        st16(kL + r * LT + d0, kv);
    }

    // fp32 group sums of dq, dk in the diagonal pass layout: lane owns
    // columns d = l + 64 cc, all 16 rows of block w
    constexpr int NCOL = D / 64;
    float dq_tot[NCOL][16], dk_tot[NCOL][16];
#pragma unroll
    for (int cc = 0; cc < NCOL; ++cc)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dq_tot[cc][r] = 0.f; dk_tot[cc][r] = 0.f; }

    for (int gi = 0; gi < p.G; ++gi) {
        const int h = hk * p.G + gi;
        const size_t jh = (size_t)j * p.H + h;
        const T* AT = static_cast<const T*>(p.AT) + jh * C * C;
        const T* Am = static_cast<const T*>(p.Am) + jh * C * C;
        const T* sAqkT = static_cast<const T*>(p.sAqkT) + jh * C * C;
        const T* xb = static_cast<const T*>(p.xbuf) + jh * C * D;
        const T* tb = static_cast<const T*>(p.tbuf) + jh * C * D;
        const T* hb = static_cast<const T*>(p.hbuf) + jh * D * D;
        const T* dhb = static_cast<const T*>(p.dhbuf) + jh * D * D;
        const T* dorow = dout + ((size_t)tok0 * p.H + h) * D;   // row r at dorow + r*H*D
        const long ldo = (long)p.H * D;

        __syncthreads();  // previous head's LDS use is over
        for (int r = tid; r < C; r += NT) {
            bs[r] = r < len ? to_f32(beta[(size_t)(tok0 + r) * p.H + h]) : 0.f;
            dbS[r] = 0.f;
        }
        for (int d = tid; d < D; d += NT) dGl[d] = 0.f;

        // ================= phase 1: state products over V slices =================
        f32x4 dqh[NTD], dkt_[NTD], dwP[NTD], dAq[NTC], dAp[NTC];
#pragma unroll
        for (int t = 0; t < NTD; ++t) { dqh[t] = zero4(); dkt_[t] = zero4(); dwP[t] = zero4(); }
#pragma unroll
        for (int t = 0; t < NTC; ++t) { dAq[t] = zero4(); dAp[t] = zero4(); }
        float dbp[4] = {0.f, 0.f, 0.f, 0.f};   // partial db of rows r0 + acc_row(i)
        float hdh = 0.f;                        // partial rowsum(h dh') of column tid % D

        T* doT = reinterpret_cast<T*>(U + L::P1_DOT);
        T* XL = reinterpret_cast<T*>(U + L::P1_XL);
        T* hL = reinterpret_cast<T*>(U + L::P1_HL);
        T* dhL = reinterpret_cast<T*>(U + L::P1_DHL);
        T* dXL = reinterpret_cast<T*>(U + L::P1_DXL);
        T* dXT = reinterpret_cast<T*>(U + L::P1_DXT);
        T* vL = reinterpret_cast<T*>(U + L::P1_VL);
        T* dvout = static_cast<T*>(p.dv) + ((size_t)tok0 * p.H + h) * D;

        for (int v0 = 0; v0 < D; v0 += BVS) {
            __syncthreads();
            for (int e = tid; e < C * (BVS / V8); e += NT) {
                const int r = e / (BVS / V8), c = (e % (BVS / V8)) * V8;
                Vec16 dv{}, vv{};
                if (r < len) {
                    dv = ld16(dorow + (long)r * ldo + v0 + c);
                    vv = ld16(v + ((size_t)(tok0 + r) * p.H + h) * D + v0 + c);
                }
                const T* dp = reinterpret_cast<const T*>(&dv);
#pragma unroll
                for (int i = 0; i < V8; ++i) doT[(c + i) * LC + r] = dp[i];
                st16(vL + r * LB + c, vv);
                st16(XL + r * LB + c, ld16(xb + (size_t)r * D + v0 + c));
            }
            for (int e = tid; e < D * (BVS / V8); e += NT) {
                const int d = e / (BVS / V8), c = (e % (BVS / V8)) * V8;
                st16(hL + d * LB + c, ld16(hb + (size_t)d * D + v0 + c));
                st16(dhL + d * LB + c, ld16(dhb + (size_t)d * D + v0 + c));
            }
            __syncthreads();
            // dX = T + sAqkT do  (own rows, [16][BVS])
            f32x4 dX[NTV];
#pragma unroll
            for (int t = 0; t < NTV; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dX[t][i] = to_f32(tb[(size_t)(r0 + acc_row(i)) * D + v0 + 16 * t + acc_col()]);
            }
            panel_mma<T, NTV, C>(dX, sAqkT, C, r0, doT, LC, 0);
#pragma unroll
            for (int t = 0; t < NTV; ++t) {
                const int c = 16 * t + acc_col(), rb = r0 + acc_row(0);
#pragma unroll
                for (int i = 0; i < 4; ++i) dXL[(rb + i) * LB + c] = from_f32<T>(dX[t][i]);
                store4<T>(dXT + c * LC + rb, dX[t][0], dX[t][1], dX[t][2], dX[t][3]);
            }
            // rowsum(h dh') over this slice, column d = tid % D
            for (int d = tid; d < D; d += NT) {
                float s = 0.f;
#pragma unroll 8
                for (int c = 0; c < BVS; ++c) s += to_f32(hL[d * LB + c]) * to_f32(dhL[d * LB + c]);
                hdh += s;
            }
            __syncthreads();
#pragma unroll
            for (int k0 = 0; k0 < BVS; k0 += kstep<T>()) {
                const auto a_do = frag_rows(dorow, ldo, r0, v0 + k0, len);
                const auto a_x = frag_kc(xb + v0, D, r0, k0);
                const auto a_dx = frag_kc(dXL, LB, r0, k0);
#pragma unroll
                for (int t = 0; t < NTC; ++t) {
                    dAq[t] = Mfma<T>::mma(a_do, frag_kc(XL, LB, 16 * t, k0), dAq[t]);
                    dAp[t] = Mfma<T>::mma(a_dx, frag_kc(vL, LB, 16 * t, k0), dAp[t]);
                }
#pragma unroll
                for (int t = 0; t < NTD; ++t) {
                    const auto bh = frag_kc(hL, LB, 16 * t, k0);
                    dqh[t] = Mfma<T>::mma(a_do, bh, dqh[t]);
                    dwP[t] = Mfma<T>::mma(a_dx, bh, dwP[t]);
                    dkt_[t] = Mfma<T>::mma(a_x, frag_kc(dhL, LB, 16 * t, k0), dkt_[t]);
                }
            }
            // dv^ = A^T dX; dv = beta dv^; db += rowsum(dv^ v)
            f32x4 dvh[NTV];
#pragma unroll
            for (int t = 0; t < NTV; ++t) dvh[t] = zero4();
            panel_mma<T, NTV, C>(dvh, AT, C, r0, dXT, LC, 0);
#pragma unroll
            for (int t = 0; t < NTV; ++t) {
                const int c = 16 * t + acc_col();
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = r0 + acc_row(i);
                    dbp[i] += dvh[t][i] * to_f32(vL[r * LB + c]);
                    if (r < len) dvout[(size_t)r * ldo + v0 + c] = from_f32<T>(bs[r] * dvh[t][i]);
                }
            }
        }
        // dG_last, part 1: ln2 2^G_last rowsum_v(h dh')  (glast of this chunk)
        {
            const float* gl = p.glast + jh * D;
            for (int d = tid; d < D; d += NT) dGl[d] = kLn2 * gl[d] * hdh;
        }
        __syncthreads();  // phase-1 LDS is dead from here

        // ================= phase 2 =================
        float* Gs = reinterpret_cast<float*>(U + L::P2_GS);
        for (int e = tid; e < C * (D / 4); e += NT) {
            const int r = e / (D / 4), d0 = (e % (D / 4)) * 4;
            f32x4 gv = zero4();
            if (r < len) {
                if constexpr (SCALAR) {
                    const float s = p.g[(size_t)(tok0 + r) * p.H + h];
                    gv = f32x4{s, s, s, s};
                } else {
                    gv = *reinterpret_cast<const f32x4*>(p.g + ((size_t)(tok0 + r) * p.H + h) * D + d0);
                }
            }
            *reinterpret_cast<f32x4*>(Gs + r * LF + d0) = gv;
        }
        __syncthreads();
        for (int d = tid; d < D; d += NT) {
            float s = 0.f;
            for (int r = 0; r < C; ++r) { s += Gs[r * LF + d]; Gs[r * LF + d] = s; }
        }
        __syncthreads();

        // 2b: post-factors, dw -> LDS, k 2^G -> LDS
        T* dwT = reinterpret_cast<T*>(U + L::P2_DWT);
        T* dwL = reinterpret_cast<T*>(U + L::P2_DWL);
        T* kgL = reinterpret_cast<T*>(U + L::P2_KG);
        f32x4 Pq[NTD], Pk[NTD], PG[NTD];
#pragma unroll
        for (int t = 0; t < NTD; ++t) {
            const int c = 16 * t + acc_col();
            const float gls = Gs[(C - 1) * LF + c];
            float colk = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + acc_row(i);
                const float G = Gs[r * LF + c];
                const float dqi = p.scale * dqh[t][i] * fast_exp2(G);
                const float dki = dkt_[t][i] * fast_exp2(gls - G);
                const float qv = to_f32(qL[r * LT + c]), kv = to_f32(kL[r * LT + c]);
                Pq[t][i] = dqi;
                Pk[t][i] = dki;
                PG[t][i] = kLn2 * (qv * dqi - kv * dki);
                colk += kv * dki;
            }
            // sum over the 16 rows of this wave (4 in-lane, 4 lane groups)
            colk += __shfl_xor(colk, 16);
            colk += __shfl_xor(colk, 32);
            if (l < 16) dGlw[w * D + c] = kLn2 * colk;  // summed in wave order later
            const int rb = r0 + acc_row(0);
            store4<T>(dwT + c * LC + rb, -dwP[t][0], -dwP[t][1], -dwP[t][2], -dwP[t][3]);
#pragma unroll
            for (int i = 0; i < 4; ++i) dwL[(rb + i) * LT + c] = from_f32<T>(-dwP[t][i]);
        }
        for (int e = tid; e < C * D; e += NT) {
            const int r = e / D, d = e % D;
            kgL[r * LT + d] = from_f32<T>(to_f32(kL[r * LT + d]) * fast_exp2(Gs[r * LF + d]));
        }
        __syncthreads();
        // 2c: dk^ = A^T dw ; dA' += dw (k 2^G)^T
        {
            f32x4 dkh[NTD];
#pragma unroll
            for (int t = 0; t < NTD; ++t) dkh[t] = zero4();
            panel_mma<T, NTD, C>(dkh, AT, C, r0, dwT, LC, 0);
#pragma unroll
            for (int t = 0; t < NTD; ++t) {
                const int c = 16 * t + acc_col();
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = r0 + acc_row(i);
                    const float kgv = to_f32(kL[r * LT + c]) * fast_exp2(Gs[r * LF + c]);
                    Pk[t][i] += bs[r] * fast_exp2(Gs[r * LF + c]) * dkh[t][i];
                    PG[t][i] += kLn2 * bs[r] * kgv * dkh[t][i];
                    dbp[i] += dkh[t][i] * kgv;
                }
            }
        }
        panel_mma<T, NTC, D>(dAp, dwL, LT, r0, kgL, LT, 0);
        // dA = dA' Diag(beta); T1 = dA A^T
        T* dAL = reinterpret_cast<T*>(U + L::P2_DAL);
        T* T1T = reinterpret_cast<T*>(U + L::P2_T1T);
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
            const int c = 16 * t + acc_col();
#pragma unroll
            for (int i = 0; i < 4; ++i) dAL[(r0 + acc_row(i)) * LC + c] = from_f32<T>(dAp[t][i] * bs[c]);
        }
        __syncthreads();
        {
            f32x4 t1[NTC];
#pragma unroll
            for (int t = 0; t < NTC; ++t) t1[t] = zero4();
            panel_mma<T, NTC, C>(t1, dAL, LC, r0, Am, C, 0);
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                const int c = 16 * t + acc_col(), rb = r0 + acc_row(0);
                store4<T>(T1T + c * LC + rb, t1[t][0], t1[t][1], t1[t][2], t1[t][3]);
            }
        }
        __syncthreads();
        // 2e: dAkk = -StrictLower(A^T T1); dAqk = scale Lower_incl(...)
        T* dAqL = reinterpret_cast<T*>(U + L::P2_DAQ);
        T* dAqT = dAqL + C * LC;
        T* dAkL = dAqT + C * LC;
        T* dAkT = dAkL + C * LC;
        {
            f32x4 dAk[NTC];
#pragma unroll
            for (int t = 0; t < NTC; ++t) dAk[t] = zero4();
            panel_mma<T, NTC, C>(dAk, AT, C, r0, T1T, LC, 0);
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                const int s = 16 * t + acc_col(), rb = r0 + acc_row(0);
                float aq[4], ak[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rb + i;
                    aq[i] = s <= r ? p.scale * dAq[t][i] : 0.f;
                    ak[i] = s < r ? -dAk[t][i] : 0.f;
                    dAqL[r * LC + s] = from_f32<T>(aq[i]);
                    dAkL[r * LC + s] = from_f32<T>(ak[i]);
                    if (t == w) {  // diagonal block, fp32 for the VALU pass: [s][r]
                        dqD[w * 256 + (s - r0) * 16 + (r - r0)] = aq[i];
                        dkD[w * 256 + (s - r0) * 16 + (r - r0)] = ak[i];
                    }
                }
                store4<T>(dAqT + s * LC + rb, aq[0], aq[1], aq[2], aq[3]);
                store4<T>(dAkT + s * LC + rb, ak[0], ak[1], ak[2], ak[3]);
            }
        }
        __syncthreads();

        // 2f: cross-block terms through each boundary rho = 16 ib, DH columns at a time
        constexpr int NTH = L::DH / 16;
        for (int ib = 1; ib < NB; ++ib) {
            const int rho = 16 * ib;
            const int kbn = L::rup(rho);                  // row-side reduction length
            const int kcn = L::rup(C - rho);              // col-side reduction length
            const int kcb = C - kcn;                      // col-side reduction start
            const int lkb = kbn + pad<T>(), lkc = kcn + pad<T>();
            T* kbT = reinterpret_cast<T*>(U + L::P2_X);   // [DH][lkb]  k_s 2^(G_rho - G_s), s < rho
            T* qbT = kbT + L::DH * lkb;                   // [DH][lkc]  q_r 2^(G_r - G_rho), r >= rho
            T* kbbT = qbT + L::DH * lkc;                  // [DH][lkc]  beta_r k_r 2^(G_r - G_rho)
            for (int dh0 = 0; dh0 < D; dh0 += L::DH) {
                for (int e = tid; e < L::DH * kbn; e += NT) {
                    const int dd = e / kbn, s = e % kbn, d = dh0 + dd;
                    float x = 0.f;
                    if (s < rho) x = to_f32(kL[s * LT + d]) * fast_exp2(Gs[rho * LF + d] - Gs[s * LF + d]);
                    kbT[dd * lkb + s] = from_f32<T>(x);
                }
                for (int e = tid; e < L::DH * kcn; e += NT) {
                    const int dd = e / kcn, rr = e % kcn, r = kcb + rr, d = dh0 + dd;
                    float xq = 0.f, xk = 0.f;
                    if (r >= rho) {
                        const float f = fast_exp2(Gs[r * LF + d] - Gs[rho * LF + d]);
                        xq = to_f32(qL[r * LT + d]) * f;
                        xk = bs[r] * to_f32(kL[r * LT + d]) * f;
                    }
                    qbT[dd * lkc + rr] = from_f32<T>(xq);
                    kbbT[dd * lkc + rr] = from_f32<T>(xk);
                }
                __syncthreads();
                const int tb0 = dh0 / 16;   // first accumulator tile of this D chunk
                if (w == ib) {  // row side of target block ib
                    f32x4 aq[NTH], ak[NTH];
#pragma unroll
                    for (int t = 0; t < NTH; ++t) { aq[t] = zero4(); ak[t] = zero4(); }
                    for (int k0 = 0; k0 < kbn; k0 += kstep<T>()) {
                        const auto fq = frag_kc(dAqL, LC, r0, k0);
                        const auto fk = frag_kc(dAkL, LC, r0, k0);
#pragma unroll
                        for (int t = 0; t < NTH; ++t) {
                            const auto b = frag_kc(kbT, lkb, 16 * t, k0);
                            aq[t] = Mfma<T>::mma(fq, b, aq[t]);
                            ak[t] = Mfma<T>::mma(fk, b, ak[t]);
                        }
                    }
#pragma unroll
                    for (int t = 0; t < NTH; ++t) {
                        const int c = dh0 + 16 * t + acc_col();
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = r0 + acc_row(i);
                            const float f = fast_exp2(Gs[r * LF + c] - Gs[rho * LF + c]);
                            const float xq = f * aq[t][i], xk = f * ak[t][i];
                            const float qv = to_f32(qL[r * LT + c]), kv = to_f32(kL[r * LT + c]);
                            Pq[tb0 + t][i] += xq;
                            Pk[tb0 + t][i] += bs[r] * xk;
                            PG[tb0 + t][i] += kLn2 * (qv * xq + bs[r] * kv * xk);
                            dbp[i] += kv * xk;
                        }
                    }
                }
                if (w == ib - 1) {  // column side of source block ib-1
                    f32x4 dk[NTH];
#pragma unroll
                    for (int t = 0; t < NTH; ++t) dk[t] = zero4();
                    for (int k0 = 0; k0 < kcn; k0 += kstep<T>()) {
                        const auto fq = frag_kc(dAqT, LC, r0, kcb + k0);
                        const auto fk = frag_kc(dAkT, LC, r0, kcb + k0);
#pragma unroll
                        for (int t = 0; t < NTH; ++t) {
                            dk[t] = Mfma<T>::mma(fq, frag_kc(qbT, lkc, 16 * t, k0), dk[t]);
                            dk[t] = Mfma<T>::mma(fk, frag_kc(kbbT, lkc, 16 * t, k0), dk[t]);
                        }
                    }
#pragma unroll
                    for (int t = 0; t < NTH; ++t) {
                        const int c = dh0 + 16 * t + acc_col();
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int s = r0 + acc_row(i);
                            const float x = fast_exp2(Gs[rho * LF + c] - Gs[s * LF + c]) * dk[t][i];
                            Pk[tb0 + t][i] += x;
                            PG[tb0 + t][i] -= kLn2 * to_f32(kL[s * LT + c]) * x;
                        }
                    }
                }
                __syncthreads();
            }
        }
        // row sums of db over the 16 lanes of each row group
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x = dbp[i];
            x += __shfl_xor(x, 1); x += __shfl_xor(x, 2);
            x += __shfl_xor(x, 4); x += __shfl_xor(x, 8);
            if ((l & 15) == 0) dbS[r0 + acc_row(i)] += x;
        }
        __syncthreads();  // Gs and the cross operands are dead from here

        // ================= phase 3: diagonal blocks (VALU) and epilogue =================
        float* exq = reinterpret_cast<float*>(U + L::P3_EX);
        float* exk = exq + C * LF;
        float* exg = exk + C * LF;
#pragma unroll
        for (int t = 0; t < NTD; ++t) {
            const int c = 16 * t + acc_col();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + acc_row(i);
                exq[r * LF + c] = Pq[t][i];
                exk[r * LF + c] = Pk[t][i];
                exg[r * LF + c] = PG[t][i];
            }
        }
        __syncthreads();
        const float* gsrc = p.g;
        float dGc[NCOL][16];
        float dbd[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) dbd[r] = 0.f;
#pragma unroll
        for (int cc = 0; cc < NCOL; ++cc) {
            const int d = l + 64 * cc;
            float qr[16], kr[16], ar[16], br[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = r0 + r;
                qr[r] = to_f32(qL[rr * LT + d]);
                kr[r] = to_f32(kL[rr * LT + d]);
                br[r] = bs[rr];
                float gv = 0.f;
                if (rr < len) {
                    if constexpr (SCALAR) gv = gsrc[(size_t)(tok0 + rr) * p.H + h];
                    else gv = gsrc[((size_t)(tok0 + rr) * p.H + h) * D + d];
                }
                ar[r] = fast_exp2(gv);
            }
            float accq[16], acck[16], dkt[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) { accq[r] = 0.f; acck[r] = 0.f; }
            const float* aqD = dqD + w * 256;
            const float* akD = dkD + w * 256;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                float E = 1.f, acc = 0.f;
                const float ks = kr[s];
#pragma unroll
                for (int r = s; r < 16; ++r) {
                    if (r > s) E *= ar[r];          // E = 2^(G_r - G_s)
                    const float aq = aqD[s * 16 + r], ak = akD[s * 16 + r];
                    const float t = ks * E;
                    accq[r] += aq * t;
                    acck[r] += ak * t;
                    acc += (aq * qr[r] + ak * br[r] * kr[r]) * E;
                }
                dkt[s] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = r0 + r;
                dq_tot[cc][r] += exq[rr * LF + d] + accq[r];
                dk_tot[cc][r] += exk[rr * LF + d] + br[r] * acck[r] + dkt[r];
                dGc[cc][r] = exg[rr * LF + d] +
                             kLn2 * (qr[r] * accq[r] + kr[r] * (br[r] * acck[r] - dkt[r]));
                dbd[r] += kr[r] * acck[r];
            }
        }
        // dG_last joins the last row of the chunk; local suffix sums per block
#pragma unroll
        for (int cc = 0; cc < NCOL; ++cc) {
            const int d = l + 64 * cc;
            if (w == NB - 1) {
                float s = dGl[d];
                for (int b2 = 0; b2 < NB; ++b2) s += dGlw[b2 * D + d];
                dGc[cc][15] += s;
            }
            float s = 0.f;
#pragma unroll
            for (int r = 15; r >= 0; --r) { s += dGc[cc][r]; dGc[cc][r] = s; }
            btot[w * D + d] = s;
        }
        // db: diagonal part summed over the wave's columns
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = dbd[r];
            x += __shfl_xor(x, 1); x += __shfl_xor(x, 2); x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8); x += __shfl_xor(x, 16); x += __shfl_xor(x, 32);
            dbd[r] = x;
        }
        __syncthreads();
        {
            T* dbo = static_cast<T*>(p.db);
            if (l < 16) {
                const int r = r0 + l;
                float x = 0.f;
#pragma unroll
                for (int i = 0; i < 16; ++i) x = (i == l) ? dbd[i] : x;
                if (r < len) dbo[(size_t)(tok0 + r) * p.H + h] = from_f32<T>(dbS[r] + x);
            }
        }
#pragma unroll
        for (int cc = 0; cc < NCOL; ++cc) {
            const int d = l + 64 * cc;
            float later = 0.f;
            for (int b2 = w + 1; b2 < NB; ++b2) later += btot[b2 * D + d];
            if constexpr (SCALAR) {
                // scalar gate: dg is the sum over channels of the per-channel gradient
#pragma unroll
                for (int r = 0; r < 16; ++r) dGc[cc][r] += later;
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rr = r0 + r;
                    if (rr < len) p.dg[((size_t)(tok0 + rr) * p.H + h) * D + d] = dGc[cc][r] + later;
                }
            }
        }
        if constexpr (SCALAR) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float x = 0.f;
#pragma unroll
                for (int cc = 0; cc < NCOL; ++cc) x += dGc[cc][r];
                x += __shfl_xor(x, 1); x += __shfl_xor(x, 2); x += __shfl_xor(x, 4);
                x += __shfl_xor(x, 8); x += __shfl_xor(x, 16); x += __shfl_xor(x, 32);
                const int rr = r0 + r;
                if (l == 0 && rr < len) p.dg[(size_t)(tok0 + rr) * p.H + h] = x;
            }
        }
    }
    // dq, dk (group sums) in the io dtype
    T* dqo = static_cast<T*>(p.dq);
    T* dko = static_cast<T*>(p.dk);
#pragma unroll
    for (int cc = 0; cc < NCOL; ++cc) {
        const int d = l + 64 * cc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int rr = r0 + r;
            if (rr < len) {
                const size_t o = ((size_t)(tok0 + rr) * p.Hg + hk) * D + d;
                dqo[o] = from_f32<T>(dq_tot[cc][r]);
                dko[o] = from_f32<T>(dk_tot[cc][r]);
            }
        }
    }
}

}  // namespace gdr
