// gdr_chunk_bwd.hpp -- chunk-parallel gradient kernel.
//
// One workgroup per (chunk, q/k head); it loops over the value heads of the
// GQA group and sums dq / dk over them in fp32. 2 C/16 waves: wave w owns
// rows 16 (w % NB) .. +16 (diagonal block w % NB) and the column half w / NB
// of every [C][*] product, which keeps each wave's accumulators small enough
// for two waves per SIMD. With h = h_c, dh' = dh_{c+1},
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
    static constexpr int BVS = 32;  // V slice of the state products
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
    static constexpr size_t DB_OFF = BETA_OFF + C * 4;                       // f32 [4][C] db partials
    static constexpr size_t GL_OFF = DB_OFF + 4 * C * 4;                     // f32 [D] dG_last
    static constexpr size_t GLW_OFF = GL_OFF + D * 4;                        // f32 [NB][D] per-wave dG_last
    static constexpr size_t BT_OFF = GLW_OFF + size_t(NB) * D * 4;           // f32 [NB][D] block totals + [2][C]
    static constexpr size_t DIAG_OFF = BT_OFF + (size_t(NB) * D + 2 * C) * 4; // f32 [2][NB][16][16]
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
__device__ __forceinline__ typename Mfma<T>::frag frag_rows(const T* p, long ld, int i0, int k0, int nrows,
                                                            int l = lane_id()) {
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

template <typename T, int C, int D, bool SCALAR, bool GROUPED>
__global__ __launch_bounds__(128 * (C / 16)) void gdr_chunk_bwd(Params p) {
    using L = BwdLds<T, C, D>;
    constexpr int NB = L::NB, NW = 2 * NB, NT = 64 * NW, BVS = L::BVS;
    constexpr int LT = L::LT, LC = L::LC, LB = L::LB, LF = L::LF;
    constexpr int DH2 = D / 2, CH2 = C / 2, VH2 = BVS / 2;    // column halves
    constexpr int NTD = DH2 / 16, NTC = CH2 / 16, NTV = VH2 / 16;
    constexpr int V8 = 16 / sizeof(T);
    static_assert(NTD >= 1 && NTC >= 1 && NTV >= 1 && D <= NT, "tiling");
    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    T* const qL0 = reinterpret_cast<T*>(smem + L::Q_OFF);
    T* const kL0 = reinterpret_cast<T*>(smem + L::K_OFF);
    float* bs = reinterpret_cast<float*>(smem + L::BETA_OFF);
    float* dbS = reinterpret_cast<float*>(smem + L::DB_OFF);     // [4][C]: MFMA halves, diagonal halves
    float* dGl = reinterpret_cast<float*>(smem + L::GL_OFF);
    float* dGlw = reinterpret_cast<float*>(smem + L::GLW_OFF);
    float* btot = reinterpret_cast<float*>(smem + L::BT_OFF);
    float* dqD = reinterpret_cast<float*>(smem + L::DIAG_OFF);   // [NB][16 s][16 r] dAqk
    float* dkD = dqD + NB * 256;                                   // [NB][16 s][16 r] dAkk
    char* const U0 = smem + L::U_OFF;

    const int j = blockIdx.x, hk = blockIdx.y;
    if (j >= p.seq_off[p.N]) return;
    const ChunkEntry ce = p.ctab[j];
    const int tok0 = ce.tok0, len = ce.len;
    const int tid = threadIdx.x, w = wave_id(), l = lane_id();
    const int rb = w % NB, ch = w / NB;
    const int r0 = 16 * rb;                   // this wave's rows
    const int cd0 = ch * DH2, cc0 = ch * CH2, cv0 = ch * VH2;  // its column halves
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
        st16(qL0 + r * LT + d0, qv);
        st16(kL0 + r * LT + d0, kv);
    }

    // diagonal-pass layout: lane owns column dcol (when lane < D/2) and the
    // 16 rows of block rb; GROUPED keeps fp32 group sums of dq, dk there
    const bool colact = l < DH2;
    const int dcol = cd0 + (colact ? l : 0);
    float dq_tot[GROUPED ? 16 : 1], dk_tot[GROUPED ? 16 : 1];
    if constexpr (GROUPED) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { dq_tot[r] = 0.f; dk_tot[r] = 0.f; }
    }

    // One value head per call of `head`. With G == 1 there is no loop at all:
    // a loop around this body lets the compiler hoist the (lane-dependent)
    // address arithmetic of every unrolled LDS access out of it and keep it
    // live across iterations, which costs hundreds of registers.
    auto head = [&](const int gi) __attribute__((always_inline)) {
        const int l = opaque_lane_id();  // fresh per head: see above
        char* U = U0;
        T* qL = qL0;
        T* kL = kL0;
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
        for (int r = tid; r < C; r += NT) bs[r] = r < len ? to_f32(beta[(size_t)(tok0 + r) * p.H + h]) : 0.f;

        // ================= phase 1: state products over V slices =================
        f32x4 dqh[NTD], dkt_[NTD], dwP[NTD], dAq[NTC], dAp[NTC];
#pragma unroll
        for (int t = 0; t < NTD; ++t) { dqh[t] = zero4(); dkt_[t] = zero4(); dwP[t] = zero4(); }
#pragma unroll
        for (int t = 0; t < NTC; ++t) { dAq[t] = zero4(); dAp[t] = zero4(); }
        float dbp[4] = {0.f, 0.f, 0.f, 0.f};   // partial db of rows r0 + acc_row(i, l)
        float hdh = 0.f;                        // partial rowsum(h dh') of column tid

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
            // dX = T + sAqkT do  (own rows, own half of the slice)
            f32x4 dX[NTV];
#pragma unroll
            for (int t = 0; t < NTV; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dX[t][i] = to_f32(tb[(size_t)(r0 + acc_row(i, l)) * D + v0 + cv0 + 16 * t + acc_col(l)]);
            }
            panel_mma<T, NTV, C>(dX, sAqkT, C, r0, doT, LC, cv0, l);
#pragma unroll
            for (int t = 0; t < NTV; ++t) {
                const int c = cv0 + 16 * t + acc_col(l), rr = r0 + acc_row(0, l);
#pragma unroll
                for (int i = 0; i < 4; ++i) dXL[(rr + i) * LB + c] = from_f32<T>(dX[t][i]);
                store4<T>(dXT + c * LC + rr, dX[t][0], dX[t][1], dX[t][2], dX[t][3]);
            }
            // rowsum(h dh') over this slice, column d = tid
            if (tid < D) {
                float s2 = 0.f;
#pragma unroll 8
                for (int c = 0; c < BVS; ++c) s2 += to_f32(hL[tid * LB + c]) * to_f32(dhL[tid * LB + c]);
                hdh += s2;
            }
            __syncthreads();
#pragma unroll
            for (int k0 = 0; k0 < BVS; k0 += kstep<T>()) {
                const auto a_do = frag_rows(dorow, ldo, r0, v0 + k0, len, l);
                const auto a_x = frag_kc(xb + v0, D, r0, k0, l);
                const auto a_dx = frag_kc(dXL, LB, r0, k0, l);
#pragma unroll
                for (int t = 0; t < NTC; ++t) {
                    dAq[t] = Mfma<T>::mma(a_do, frag_kc(XL, LB, cc0 + 16 * t, k0, l), dAq[t]);
                    dAp[t] = Mfma<T>::mma(a_dx, frag_kc(vL, LB, cc0 + 16 * t, k0, l), dAp[t]);
                }
#pragma unroll
                for (int t = 0; t < NTD; ++t) {
                    const auto bh = frag_kc(hL, LB, cd0 + 16 * t, k0, l);
                    dqh[t] = Mfma<T>::mma(a_do, bh, dqh[t]);
                    dwP[t] = Mfma<T>::mma(a_dx, bh, dwP[t]);
                    dkt_[t] = Mfma<T>::mma(a_x, frag_kc(dhL, LB, cd0 + 16 * t, k0, l), dkt_[t]);
                }
            }
            // dv^ = A^T dX; dv = beta dv^; db += rowsum(dv^ v)
            f32x4 dvh[NTV];
#pragma unroll
            for (int t = 0; t < NTV; ++t) dvh[t] = zero4();
            panel_mma<T, NTV, C>(dvh, AT, C, r0, dXT, LC, cv0, l);
#pragma unroll
            for (int t = 0; t < NTV; ++t) {
                const int c = cv0 + 16 * t + acc_col(l);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = r0 + acc_row(i, l);
                    dbp[i] += dvh[t][i] * to_f32(vL[r * LB + c]);
                    if (r < len) dvout[(size_t)r * ldo + v0 + c] = from_f32<T>(bs[r] * dvh[t][i]);
                }
            }
        }
        // dG_last, part 1: ln2 2^G_last rowsum_v(h dh')  (glast of this chunk)
        if (tid < D) dGl[tid] = kLn2 * p.glast[jh * D + tid] * hdh;
        __syncthreads();  // phase-1 LDS is dead from here

        // ================= phase 2 =================
        float* Gs = reinterpret_cast<float*>(U + L::P2_GS);
        for (int e = tid; e < C * (D / 4); e += NT) {
            const int r = e / (D / 4), d0 = (e % (D / 4)) * 4;
            f32x4 gv = zero4();
            if (r < len) {
                if constexpr (SCALAR) {
                    const float s2 = p.g[(size_t)(tok0 + r) * p.H + h];
                    gv = f32x4{s2, s2, s2, s2};
                } else {
                    gv = *reinterpret_cast<const f32x4*>(p.g + ((size_t)(tok0 + r) * p.H + h) * D + d0);
                }
            }
            *reinterpret_cast<f32x4*>(Gs + r * LF + d0) = gv;
        }
        __syncthreads();
        if (tid < D) {
            float s2 = 0.f;
            for (int r = 0; r < C; ++r) { s2 += Gs[r * LF + tid]; Gs[r * LF + tid] = s2; }
        }
        __syncthreads();

        // 2b: post-factors, dw -> LDS, k 2^G -> LDS
        T* dwT = reinterpret_cast<T*>(U + L::P2_DWT);
        T* dwL = reinterpret_cast<T*>(U + L::P2_DWL);
        T* kgL = reinterpret_cast<T*>(U + L::P2_KG);
        f32x4 Pq[NTD], Pk[NTD], PG[NTD];
#pragma unroll
        for (int t = 0; t < NTD; ++t) {
            const int c = cd0 + 16 * t + acc_col(l);
            const float gls = Gs[(C - 1) * LF + c];
            float colk = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + acc_row(i, l);
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
            if (l < 16) dGlw[rb * D + c] = kLn2 * colk;  // summed in block order later
            const int rr = r0 + acc_row(0, l);
            store4<T>(dwT + c * LC + rr, -dwP[t][0], -dwP[t][1], -dwP[t][2], -dwP[t][3]);
#pragma unroll
            for (int i = 0; i < 4; ++i) dwL[(rr + i) * LT + c] = from_f32<T>(-dwP[t][i]);
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
            panel_mma<T, NTD, C>(dkh, AT, C, r0, dwT, LC, cd0, l);
#pragma unroll
            for (int t = 0; t < NTD; ++t) {
                const int c = cd0 + 16 * t + acc_col(l);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = r0 + acc_row(i, l);
                    const float gam = fast_exp2(Gs[r * LF + c]);
                    const float kgv = to_f32(kL[r * LT + c]) * gam;
                    Pk[t][i] += bs[r] * gam * dkh[t][i];
                    PG[t][i] += kLn2 * bs[r] * kgv * dkh[t][i];
                    dbp[i] += dkh[t][i] * kgv;
                }
            }
        }
        panel_mma<T, NTC, D>(dAp, dwL, LT, r0, kgL, LT, cc0, l);
        // dA = dA' Diag(beta); T1 = dA A^T
        T* dAL = reinterpret_cast<T*>(U + L::P2_DAL);
        T* T1T = reinterpret_cast<T*>(U + L::P2_T1T);
#pragma unroll
        for (int t = 0; t < NTC; ++t) {
            const int c = cc0 + 16 * t + acc_col(l);
#pragma unroll
            for (int i = 0; i < 4; ++i) dAL[(r0 + acc_row(i, l)) * LC + c] = from_f32<T>(dAp[t][i] * bs[c]);
        }
        __syncthreads();
        {
            f32x4 t1[NTC];
#pragma unroll
            for (int t = 0; t < NTC; ++t) t1[t] = zero4();
            panel_mma<T, NTC, C>(t1, dAL, LC, r0, Am, C, cc0, l);
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                const int c = cc0 + 16 * t + acc_col(l), rr = r0 + acc_row(0, l);
                store4<T>(T1T + c * LC + rr, t1[t][0], t1[t][1], t1[t][2], t1[t][3]);
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
            panel_mma<T, NTC, C>(dAk, AT, C, r0, T1T, LC, cc0, l);
            __syncthreads();  // T1T reads done before the dA operands overwrite dead buffers
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                const int s = cc0 + 16 * t + acc_col(l), rr = r0 + acc_row(0, l);
                float aq[4], ak[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rr + i;
                    aq[i] = s <= r ? p.scale * dAq[t][i] : 0.f;
                    ak[i] = s < r ? -dAk[t][i] : 0.f;
                    dAqL[r * LC + s] = from_f32<T>(aq[i]);
                    dAkL[r * LC + s] = from_f32<T>(ak[i]);
                    if (s >= r0 && s < r0 + 16) {  // diagonal block, fp32 for the VALU pass: [s][r]
                        dqD[rb * 256 + (s - r0) * 16 + (r - r0)] = aq[i];
                        dkD[rb * 256 + (s - r0) * 16 + (r - r0)] = ak[i];
                    }
                }
                store4<T>(dAqT + s * LC + rr, aq[0], aq[1], aq[2], aq[3]);
                store4<T>(dAkT + s * LC + rr, ak[0], ak[1], ak[2], ak[3]);
            }
        }
        __syncthreads();

        // 2f: cross-block terms through each boundary rho = 16 ib, DH columns
        // at a time (the waves of the matching column half do the MFMA work)
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
                    const int dd = e / kbn, s2 = e % kbn, d = dh0 + dd;
                    float x = 0.f;
                    if (s2 < rho) x = to_f32(kL[s2 * LT + d]) * fast_exp2(Gs[rho * LF + d] - Gs[s2 * LF + d]);
                    kbT[dd * lkb + s2] = from_f32<T>(x);
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
                // a wave's column half lies entirely inside or outside the D chunk
                static_assert(L::DH % DH2 == 0, "column halves must tile the D chunks");
                if (cd0 >= dh0 && cd0 < dh0 + L::DH) {
                    const int bt0 = cd0 - dh0;   // operand row of this wave's first tile
                    if (rb == ib) {  // row side of target block ib
                        f32x4 aq[NTD], ak[NTD];
#pragma unroll
                        for (int t = 0; t < NTD; ++t) { aq[t] = zero4(); ak[t] = zero4(); }
                        for (int k0 = 0; k0 < kbn; k0 += kstep<T>()) {
                            const auto fq = frag_kc(dAqL, LC, r0, k0, l);
                            const auto fk = frag_kc(dAkL, LC, r0, k0, l);
#pragma unroll
                            for (int t = 0; t < NTD; ++t) {
                                const auto b = frag_kc(kbT, lkb, bt0 + 16 * t, k0, l);
                                aq[t] = Mfma<T>::mma(fq, b, aq[t]);
                                ak[t] = Mfma<T>::mma(fk, b, ak[t]);
                            }
                        }
#pragma unroll
                        for (int t = 0; t < NTD; ++t) {
                            const int c = cd0 + 16 * t + acc_col(l);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int r = r0 + acc_row(i, l);
                                const float f = fast_exp2(Gs[r * LF + c] - Gs[rho * LF + c]);
                                const float xq = f * aq[t][i], xk = f * ak[t][i];
                                const float qv = to_f32(qL[r * LT + c]), kv = to_f32(kL[r * LT + c]);
                                Pq[t][i] += xq;
                                Pk[t][i] += bs[r] * xk;
                                PG[t][i] += kLn2 * (qv * xq + bs[r] * kv * xk);
                                dbp[i] += kv * xk;
                            }
                        }
                    }
                    if (rb == ib - 1) {  // column side of source block ib-1
                        f32x4 dk[NTD];
#pragma unroll
                        for (int t = 0; t < NTD; ++t) dk[t] = zero4();
                        for (int k0 = 0; k0 < kcn; k0 += kstep<T>()) {
                            const auto fq = frag_kc(dAqT, LC, r0, kcb + k0, l);
                            const auto fk = frag_kc(dAkT, LC, r0, kcb + k0, l);
#pragma unroll
                            for (int t = 0; t < NTD; ++t) {
                                dk[t] = Mfma<T>::mma(fq, frag_kc(qbT, lkc, bt0 + 16 * t, k0, l), dk[t]);
                                dk[t] = Mfma<T>::mma(fk, frag_kc(kbbT, lkc, bt0 + 16 * t, k0, l), dk[t]);
                            }
                        }
#pragma unroll
                        for (int t = 0; t < NTD; ++t) {
                            const int c = cd0 + 16 * t + acc_col(l);
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const int s2 = r0 + acc_row(i, l);
                                const float x = fast_exp2(Gs[rho * LF + c] - Gs[s2 * LF + c]) * dk[t][i];
                                Pk[t][i] += x;
                                PG[t][i] -= kLn2 * to_f32(kL[s2 * LT + c]) * x;
                            }
                        }
                    }
                }
                __syncthreads();
            }
        }
        // row sums of db over the 16 lanes of each row group (this column half)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x = dbp[i];
            x += __shfl_xor(x, 1); x += __shfl_xor(x, 2);
            x += __shfl_xor(x, 4); x += __shfl_xor(x, 8);
            if ((l & 15) == 0) dbS[ch * C + r0 + acc_row(i, l)] = x;
        }
        __syncthreads();  // Gs and the cross operands are dead from here

        // ================= phase 3: diagonal blocks (VALU) and epilogue =================
        float* exq = reinterpret_cast<float*>(U + L::P3_EX);
        float* exk = exq + C * LF;
        float* exg = exk + C * LF;
#pragma unroll
        for (int t = 0; t < NTD; ++t) {
            const int c = cd0 + 16 * t + acc_col(l);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + acc_row(i, l);
                exq[r * LF + c] = Pq[t][i];
                exk[r * LF + c] = Pk[t][i];
                exg[r * LF + c] = PG[t][i];
            }
        }
        __syncthreads();
        {
            const int d = dcol;
            float qr[16], kr[16], ar[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = r0 + r;
                qr[r] = to_f32(qL[rr * LT + d]);
                kr[r] = to_f32(kL[rr * LT + d]);
                float gv = 0.f;
                if (rr < len) {
                    if constexpr (SCALAR) gv = p.g[(size_t)(tok0 + rr) * p.H + h];
                    else gv = p.g[((size_t)(tok0 + rr) * p.H + h) * D + d];
                }
                ar[r] = fast_exp2(gv);
            }
            float accq[16], acck[16], dkt[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) { accq[r] = 0.f; acck[r] = 0.f; }
            // the fp32 16x16 blocks of dAqk / dAkk, spread over the wave: lane L
            // holds entries 4L..4L+3 of [s][r]; each (r, s) value is fetched with
            // v_readlane into a scalar register (wave-uniform operand)
            const f32x4 aqv = *reinterpret_cast<const f32x4*>(dqD + rb * 256 + 4 * l);
            const f32x4 akv = *reinterpret_cast<const f32x4*>(dkD + rb * 256 + 4 * l);
#pragma unroll
            for (int s2 = 0; s2 < 16; ++s2) {
                // keep each source row's loads and math together (no hoisting of
                // the whole 16x16 block's loads into registers)
                float E = 1.f, acc = 0.f;
                const float ks = kr[s2];
#pragma unroll
                for (int r = s2; r < 16; ++r) {
                    if (r > s2) E *= ar[r];          // E = 2^(G_r - G_s)
                    const float aq = lane_value(aqv, s2 * 16 + r), ak = lane_value(akv, s2 * 16 + r);
                    const float tq = ks * E;
                    accq[r] += aq * tq;
                    acck[r] += ak * tq;
                    acc += (aq * qr[r] + ak * bs[r0 + r] * kr[r]) * E;
                }
                dkt[s2] = acc;
            }
            // combine with the MFMA partials; dG in place in exg; the diagonal
            // db terms k_r . acck_r in place in exq (summed per row below)
            float gsum = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = r0 + r;
                const float br = bs[rr];
                const float dqv = exq[rr * LF + d] + accq[r];
                const float dkv = exk[rr * LF + d] + br * acck[r] + dkt[r];
                float dG = exg[rr * LF + d] + kLn2 * (qr[r] * accq[r] + kr[r] * (br * acck[r] - dkt[r]));
                if (rb == NB - 1 && r == 15) {  // dG_last joins the last row of the chunk
                    float sl = dGl[d];
                    for (int b2 = 0; b2 < NB; ++b2) sl += dGlw[b2 * D + d];
                    dG += sl;
                }
                if constexpr (GROUPED) {
                    dq_tot[r] += dqv;
                    dk_tot[r] += dkv;
                } else if (colact && rr < len) {
                    const size_t o = ((size_t)(tok0 + rr) * p.Hg + hk) * D + d;
                    static_cast<T*>(p.dq)[o] = from_f32<T>(dqv);
                    static_cast<T*>(p.dk)[o] = from_f32<T>(dkv);
                }
                gsum += dG;
                if (colact) {
                    exg[rr * LF + d] = dG;
                    exq[rr * LF + d] = kr[r] * acck[r];
                }
            }
            if (colact) btot[rb * D + d] = gsum;
        }
        __syncthreads();
        // reverse cumsum of dG over the chunk, per column: in place in exg
        if (colact) {
            const int d = dcol;
            float suf = 0.f;
            for (int b2 = rb + 1; b2 < NB; ++b2) suf += btot[b2 * D + d];
            for (int r = 15; r >= 0; --r) {
                const int rr = r0 + r;
                suf += exg[rr * LF + d];
                if constexpr (SCALAR) exg[rr * LF + d] = suf;
                else if (rr < len) p.dg[((size_t)(tok0 + rr) * p.H + h) * D + d] = suf;
            }
        }
        if constexpr (SCALAR) __syncthreads();
        // per-row sums: db = MFMA partials + sum_d k . acck (diagonal);
        // scalar gate: dg = sum over channels of the per-channel suffix sums
        if (tid < C && tid < len) {
            float x = dbS[tid] + dbS[C + tid];
            for (int d = 0; d < D; ++d) x += exq[tid * LF + d];
            static_cast<T*>(p.db)[(size_t)(tok0 + tid) * p.H + h] = from_f32<T>(x);
            if constexpr (SCALAR) {
                float gsum2 = 0.f;
                for (int d = 0; d < D; ++d) gsum2 += exg[tid * LF + d];
                p.dg[(size_t)(tok0 + tid) * p.H + h] = gsum2;
            }
        }
    };
    if constexpr (GROUPED) {
        for (int gi = 0; gi < p.G; ++gi) head(gi);
    } else {
        head(0);
    }
    if constexpr (GROUPED) {
        if (colact) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = r0 + r;
                if (rr < len) {
                    const size_t o = ((size_t)(tok0 + rr) * p.Hg + hk) * D + dcol;
                    static_cast<T*>(p.dq)[o] = from_f32<T>(dq_tot[r]);
                    static_cast<T*>(p.dk)[o] = from_f32<T>(dk_tot[r]);
                }
            }
        }
    }
}

}  // namespace gdr
