// gdr_chunk_bwd.hpp -- chunk-parallel gradient kernel.
//
// Work item: one (chunk, q/k head). Without GQA the kernel is persistent (at
// most one workgroup per CU walks the items and requests the next item's
// first inputs during the current item's epilogue); with GQA one workgroup per
// item loops over the value heads of the group and sums dq / dk over them in
// fp32. 2 C/16 waves: wave w owns
// rows 16 (w % NB) .. +16 (diagonal block w % NB) and the column half w / NB
// of every [C][*] product, which keeps each wave's accumulators small enough
// for two waves per SIMD. With h = h_c, dh' = dh_{c+1},
// X = u - w h (forward sweep) and T = k~ dh' (reverse sweep):
//   dX  = scale Aqk^T do + T
//   dAqk = scale Lower_incl(do X^T)
//   dq^  = scale do h^T  -> dq += dq^ 2^G
//   dk~  = X dh'^T       -> dk += dk~ 2^(G_last - G)
//   dw   = -dX h^T;  dv^ = A^T dX -> dv = beta dv^
//   dk^  = A^T dw       -> dk += beta 2^G dk^
//   dA   = (dX v^T + dw (k 2^G)^T) Diag(beta)
//   dAkk = -StrictLower(A^T dA A^T)          (gradient through the inverse,
//                                             CONSUMER_A of fused_bwd.py)
// then the intra-chunk gradient of Aqk / Akk (the bwd_intra page):
//   accq_r = sum_{s<=r} dAqk[r,s] k_s 2^(G_r-G_s),  acck_r = sum_{s<r} dAkk[r,s] k_s 2^(G_r-G_s)
//   dkt_s  = sum_{r>=s} (dAqk[r,s] q_r + dAkk[r,s] beta_r k_r) 2^(G_r-G_s)
//   dq += accq, dk += beta acck + dkt, db += k . acck,
//   dG += ln2 [q accq + k (beta acck - dkt)],
// all on MFMA, one 16x16x16 product per pair of 16-row blocks. With block b =
// rows 16b..16b+15, Ein_r = 2^(G_r - G_16b(r)) and Eout_s = 2^(G_16(b(s)+1) - G_s)
// (both <= 1) and phi_j = 2^(G_16(j+1) - G_16j), the decay between a row r of
// block b and a source s of an earlier block b' factors as
//   2^(G_r - G_s) = Ein_r * phi_{b'+1} ... phi_{b-1} * Eout_s,
// so the operands k Eout, q Ein, beta k Ein are scaled once per chunk and the
// phi are applied to the accumulators between blocks (Horner); every exponent
// of these cross-block terms is <= 0. Inside a diagonal block the source side
// needs 2^(G_16b - G_s) >= 1, taken as the k Eout operand times
// 2^(G_16b - G_16(b+1)) on the accumulator (the last block references its own
// last row): exp2 of a positive argument, up to the guard. The MFMA form is
// used there when the block's gate range, its next block's first row
// included, stays within 64 (8 for fp16 operands) for every column of the
// wave, else an exact VALU pass with one exp2 per (r, s, d) of arguments <= 0
// (the only form the bwd_intra page uses for diagonal blocks). Finally
// dg = reverse cumsum of dG in the chunk (the page's fold_dg), dG_last collecting
//   ln2 [2^G_last rowsum_v(h dh') + sum_r k_r dk~_r 2^(G_last - G_r)].
#pragma once
#include "gdr_common.hpp"

namespace gdr {

template <typename T, int C, int D>
struct BwdLds {
    static constexpr int NB = C / 16;
    // V slice of the state products: two stored tiles at C = 64 with 16-bit
    // operands (half as many slice loads, each twice as large, so that fewer
    // round trips to memory sit between the slices), else one
    static constexpr int BVS = C == 64 && sizeof(T) == 2 ? 2 * kTileV : kTileV;
    static_assert(BVS % kTileV == 0 && D % BVS == 0, "slices of whole stored tiles");
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
    static constexpr size_t DB_OFF = BETA_OFF + C * 4;                       // f32 [2][C] db row partials
    static constexpr size_t DGR_OFF = DB_OFF + 2 * C * 4;                    // f32 [2][C] scalar-gate dg rows
    static constexpr size_t GL_OFF = DGR_OFF + 2 * C * 4;                    // f32 [D] dG_last
    static constexpr size_t GLW_OFF = GL_OFF + D * 4;                        // f32 [NB][D] per-wave dG_last
    static constexpr size_t BT_OFF = GLW_OFF + size_t(NB) * D * 4;           // f32 [NB][D] block totals
    static constexpr size_t AM_OFF = BT_OFF + size_t(NB) * D * 4;            // T [C][LC] A of the head
    static constexpr size_t U_OFF = AM_OFF + sz(C, LC, sizeof(T));           // union region
    // phase 1 (state products, one V slice)
    static constexpr size_t P1_XL = 0;                                       // T [C][LB]
    static constexpr size_t P1_HL = P1_XL + sz(C, LB, sizeof(T));            // T [D][LB]
    static constexpr size_t P1_DHL = P1_HL + sz(D, LB, sizeof(T));           // T [D][LB]
    static constexpr size_t P1_DXT = P1_DHL + sz(D, LB, sizeof(T));          // T [BVS][LC] dX^T
    static constexpr size_t P1_VL = P1_DXT + sz(BVS, LC, sizeof(T));         // T [C][LB]
    static constexpr size_t P1_DOL = P1_VL + sz(C, LB, sizeof(T));          // T [C][LB] do rows
    static constexpr size_t P1_TL = P1_DOL + sz(C, LB, sizeof(T));           // T [C][LB] T = k~ dh'
    static constexpr size_t P1_END = P1_TL + sz(C, LB, sizeof(T));
    // phase 2: Gs lives from 2a to the end of 2f
    static constexpr size_t P2_GS = 0;                                       // f32 [C][LF]
    static constexpr size_t P2_A = P2_GS + sz(C, LF, 4);
    //   2a-2e
    static constexpr size_t P2_DWT = P2_A;                                   // T [D][LC]
    static constexpr size_t P2_KG = P2_DWT + sz(D, LC, sizeof(T));           // T [C][LT]
    static constexpr size_t P2_DAL = P2_KG + sz(C, LT, sizeof(T));           // T [C][LC]
    static constexpr size_t P2_T1T = P2_DAL + sz(C, LC, sizeof(T));          // T [C][LC]
    static constexpr size_t P2_B_END = P2_T1T + sz(C, LC, sizeof(T));
    //   2a: cumsum segment totals f32 [NT/D][D] in the dw region (written in 2b)
    static constexpr size_t P2_SEG = P2_DWT;
    //   2e-2f: dAqk / dAkk [C][LC] each, over the dead dw / k 2^G / dA buffers;
    //   they must stay clear of T1T, still read in 2e
    static constexpr size_t P2_DAQ = P2_A;
    static constexpr size_t P2_DA_END = P2_DAQ + 2 * sz(C, LC, sizeof(T));
    //   2f: scaled operands of both column halves, transposed: k Eout, q Ein,
    //   beta k Ein, each [2][D/2][LC]
    static constexpr size_t P2_X = P2_DA_END;
    static constexpr size_t P2_X_END = P2_X + 6 * sz(D / 2, LC, sizeof(T));
    // epilogue: dq, dk [C][LT] and dg f32 [C][LF] staged for row-contiguous stores
    static constexpr size_t E_DQ = 0;
    static constexpr size_t E_DK = E_DQ + sz(C, LT, sizeof(T));
    static constexpr size_t E_DG = E_DK + sz(C, LT, sizeof(T));
    static constexpr size_t E_END = E_DG + sz(C, LF, 4);
    // dv [C][LT], staged in phase 1 and stored in 2a: clear of the phase-1
    // buffers and of what 2a writes (Gs, segment totals, k 2^G)
    static constexpr size_t DVS = cmax(P1_END, P2_KG + sz(C, LT, sizeof(T)));
    static constexpr size_t DVS_END = DVS + sz(C, LT, sizeof(T));
    static constexpr size_t U_BYTES = cmax(cmax(cmax(P1_END, P2_B_END), cmax(P2_X_END, E_END)), DVS_END);
    static constexpr size_t TOTAL = U_OFF + U_BYTES;
    // the fused reverse kernel (state gradient on chip) adds: w rows [C][LT]
    // (read as w^T through transposed loads), -T^T of the slice [BVS][LC],
    // 2^G_last f32 [D]
    static constexpr size_t F_W = TOTAL;
    static constexpr size_t F_TT = F_W + sz(C, LT, sizeof(T));
    static constexpr size_t F_GAM = F_TT + sz(BVS, LC, sizeof(T));
    static constexpr size_t F_TOTAL = F_GAM + size_t(D) * 4;
    static_assert(P2_DA_END <= P2_T1T, "dAqk/dAkk operands must not overlap T1T");
    static_assert(size_t(4) * C * 16 <= sz(D, LC, sizeof(T)), "cumsum segment totals fit the dw region");
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

// Rows 0..len-1 of the staged dq, dk tiles ([C][D + pad] in LDS) to the
// token-major outputs, 16 bytes per access.
template <typename T, int C, int D, int NT>
__device__ __forceinline__ void store_rows(const Params& p, const T* dqS, const T* dkS, int tok0, int len,
                                           int hk, int tid) {
    constexpr int V8 = 16 / sizeof(T), LT = D + pad<T>();
    constexpr int NS = C * (D / V8) / NT;   // pieces per thread: all read first, one LDS wait
    static_assert(NS * NT == C * (D / V8), "row piece split");
    Vec16 a[NS], b[NS];
#pragma unroll
    for (int it = 0; it < NS; ++it) {
        const int e = tid + it * NT, r = e / (D / V8), c = (e % (D / V8)) * V8;
        a[it] = ld16(dqS + r * LT + c);
        b[it] = ld16(dkS + r * LT + c);
    }
#pragma unroll
    for (int it = 0; it < NS; ++it) {
        const int e = tid + it * NT, r = e / (D / V8), c = (e % (D / V8)) * V8;
        if (r < len) {
            const size_t o = ((size_t)(tok0 + r) * p.Hg + hk) * D + c;
            st16(static_cast<T*>(p.dq) + o, a[it]);
            st16(static_cast<T*>(p.dk) + o, b[it]);
        }
    }
}

// Diagonal blocks use the MFMA form while |G_r - G_16b| <= this bound (log2):
// the operand k 2^range must stay finite and q 2^-range normal in T, so
// 2^8 for fp16 (5 exponent bits), 2^64 for bf16 and fp32 (8 exponent bits).
template <typename T>
constexpr float diag_guard() { return __is_same(T, _Float16) ? 8.f : 64.f; }

// Workgroups of the preparation and gradient kernels one CU holds at once: at
// C = 64 their LDS (about 157 KB) allows one; at C = 32 with 16-bit operands
// (under 80 KB each) two, when the gradient kernel's four waves keep to 256
// registers; fp32 operands at C = 32 need over 80 KB, so one.
template <typename T, int C>
constexpr int resident_per_cu() { return C == 32 && sizeof(T) == 2 ? 2 : 1; }

// Waves per SIMD of the gradient kernel (caps its registers): its C / 8 waves
// times the workgroups a CU holds, over 4 SIMDs (the fused reverse kernel: one
// workgroup per CU).
//
// FUSED: the reverse state sweep runs inside the gradient kernel. One
// workgroup per (sequence, value head) walks the sequence's chunks from the
// last to the first, holding the state gradient dh (fp32, K x V) in the
// accumulators of its waves: each chunk's body takes dh' = dh_{c+1} from them
// (a bf16 copy per V slice in LDS), forms T = k~ dh' itself, and ends each
// slice with the sweep's update dh_c = Diag(2^G_last) dh' - w^T T +
// (scale q~)^T do on those accumulators, so neither dh nor T goes through
// memory (the FlashQLA issue #30 page's fused design: the CONSUMER_S state
// stays resident for the whole loop). The next chunk's inputs are requested in
// the current chunk's epilogue. With GQA the value heads of a group are in
// different workgroups: dq, dk go out as fp32 partials per value head and
// gdr_group_sum adds them in group order.
template <typename T, int C, int D, bool SCALAR, bool GROUPED, bool FUSED = false>
__global__ __launch_bounds__(128 * (C / 16)) __attribute__((amdgpu_waves_per_eu(
    C / 32 * (FUSED ? 1 : resident_per_cu<T, C>()), C / 32 * (FUSED ? 1 : resident_per_cu<T, C>())))) void
gdr_chunk_bwd(Params p) {
    using L = BwdLds<T, C, D>;
    static_assert(!FUSED || (!GROUPED && L::F_TOTAL <= 163840), "fused reverse kernel: per value head, LDS budget");
    constexpr int NB = L::NB, NW = 2 * NB, NT = 64 * NW, BVS = L::BVS;
    constexpr int LT = L::LT, LC = L::LC, LB = L::LB, LF = L::LF;
    constexpr int DH2 = D / 2, CH2 = C / 2, VH2 = BVS / 2;    // column halves
    constexpr int NTD = DH2 / 16, NTC = CH2 / 16, NTV = VH2 / 16;
    constexpr int V8 = 16 / sizeof(T);
    static_assert(NTD >= 1 && NTC >= 1 && NTV >= 1 && D <= NT, "tiling");
    __shared__ __attribute__((aligned(16))) char smem[FUSED ? L::F_TOTAL : L::TOTAL];
    T* const qL0 = reinterpret_cast<T*>(smem + L::Q_OFF);
    T* const kL0 = reinterpret_cast<T*>(smem + L::K_OFF);
    float* bs = reinterpret_cast<float*>(smem + L::BETA_OFF);
    float* dbS = reinterpret_cast<float*>(smem + L::DB_OFF);     // [2][C] per column half
    float* dgR = reinterpret_cast<float*>(smem + L::DGR_OFF);    // [2][C] per column half
    float* dGl = reinterpret_cast<float*>(smem + L::GL_OFF);
    float* dGlw = reinterpret_cast<float*>(smem + L::GLW_OFF);
    float* btot = reinterpret_cast<float*>(smem + L::BT_OFF);
    char* const U0 = smem + L::U_OFF;

    const int w = __builtin_amdgcn_readfirstlane(wave_id());   // uniform: a scalar register
    const int wave_k = w;
    const int rb = w % NB, ch = w / NB;
    const int r0 = 16 * rb;                   // this wave's rows
    const int cd0 = ch * DH2, cc0 = ch * CH2, cv0 = ch * VH2;  // its column halves
    const T* q = static_cast<const T*>(p.q);
    const T* k = static_cast<const T*>(p.k);
    const T* v = static_cast<const T*>(p.v);
    const T* dout = static_cast<const T*>(p.dout);
    const T* beta = static_cast<const T*>(p.beta);

    // What a head needs before its first slice: the chunk's q, k rows (first
    // head only), the first slice's pieces, the row fragments of scale Aqk^T,
    // A (staged in LDS: the B operand of dA A^T, and through transposed loads
    // the A operand of every A^T product), beta and 2^G_last. They are requested
    // together, so that one wait covers them all; the persistent (non-grouped)
    // kernel requests them for its next item during the current item's epilogue.
    using Frag = typename Mfma<T>::frag;
    constexpr int KS = kstep<T>(), NKC = C / KS;
    constexpr int NQP = C * (D / V8) / NT;
    static_assert(NQP * NT == C * (D / V8), "piece split");
    constexpr int PR = BVS / V8;                              // 16-byte pieces per slice row
    constexpr int NPC = (C * PR + NT - 1) / NT, NPD = (D * PR + NT - 1) / NT;
    constexpr int NAM = (C * (C / V8) + NT - 1) / NT;
    Vec16 qv[NQP], kv[NQP];
    Vec16 pdo[NPC], pv[NPC], px[NPC], pt[NPC], ph[NPD], pdh[NPD];
    Frag fAq[NKC];             // rows r0.. of scale Aqk^T
    Vec16 pam[NAM];
    float pbeta, pgl[NPD];
    // rows past the sequence end read its last row (zeroed at use)
    auto request_qk = [&](const ChunkEntry& e2, const int hk2, const int tid) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NQP; ++i) {
            const int e = tid + i * NT, r = min(e / (D / V8), e2.len - 1), d0 = (e % (D / V8)) * V8;
            qv[i] = ld16(q + ((size_t)(e2.tok0 + r) * p.Hg + hk2) * D + d0);
            kv[i] = ld16(k + ((size_t)(e2.tok0 + r) * p.Hg + hk2) * D + d0);
        }
    };
    // slice pieces of value columns v0 .. v0 + BVS: unconditional loads (spare
    // threads and rows past the sequence end read valid duplicates, zeroed at
    // use), so no load waits on a branch
    auto request_slice = [&](const ChunkEntry& e2, const size_t jh2, const int h2, const int v0,
                             const int tid) __attribute__((always_inline)) {
        const T* xb = static_cast<const T*>(p.xbuf) + jh2 * C * D;
        const T* tb = static_cast<const T*>(p.tbuf) + jh2 * C * D;
        const T* hb = static_cast<const T*>(p.hbuf) + jh2 * D * D;
        const T* dhb = static_cast<const T*>(p.dhbuf) + jh2 * D * D;
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int e = min(tid + NT * i, C * PR - 1);
            const int r = e / PR, c = (e % PR) * V8, rt = min(r, e2.len - 1);
            const size_t row = ((size_t)(e2.tok0 + rt) * p.H + h2) * D + v0 + c;
            pdo[i] = ld16(dout + row);
            pv[i] = ld16(v + row);
            const int col = v0 + c;   // V-tiled: tile col / kTileV, column col % kTileV
            px[i] = ld16(xb + (size_t)(col / kTileV) * kTileV * C + r * kTileV + col % kTileV);
            if constexpr (!FUSED) pt[i] = ld16(tb + (size_t)(col / kTileV) * kTileV * C + r * kTileV + col % kTileV);
        }
#pragma unroll
        for (int i = 0; i < NPD; ++i) {
            const int e = min(tid + NT * i, D * PR - 1);
            const int d = e / PR, c = (e % PR) * V8;
            const int col = v0 + c;   // V-tiled, as above
            ph[i] = ld16(hb + (size_t)(col / kTileV) * kTileV * D + d * kTileV + col % kTileV);
            if constexpr (!FUSED) pdh[i] = ld16(dhb + (size_t)(col / kTileV) * kTileV * D + d * kTileV + col % kTileV);
        }
    };
    // (tid, l, rows: the caller's thread, lane and first row of the wave; the
    // persistent kernel passes its per-item opaque ones, see `head`)
    auto request_head = [&](const ChunkEntry& e2, const int j2, const int h2, const int tid, const int l,
                            const int rows) __attribute__((always_inline)) {
        const size_t jh2 = (size_t)j2 * p.H + h2;
        const T* Am = static_cast<const T*>(p.Am) + jh2 * C * C;
        const T* sAqkT = static_cast<const T*>(p.sAqkT) + jh2 * C * C;
        pbeta = to_f32(beta[(size_t)(e2.tok0 + min(tid, e2.len - 1)) * p.H + h2]);
#pragma unroll
        for (int i = 0; i < NAM; ++i) {
            const int e = min(tid + NT * i, C * (C / V8) - 1);
            pam[i] = ld16(Am + (size_t)e * V8);
        }
#pragma unroll
        for (int k2 = 0; k2 < NKC; ++k2) fAq[k2] = frag_fo<T, C>(sAqkT, rows, k2 * KS, l);   // fragment order
        request_slice(e2, jh2, h2, 0, tid);
#pragma unroll
        for (int i = 0; i < NPD; ++i) pgl[i] = p.glast[jh2 * D + min((tid + NT * i) / PR, D - 1)];
    };

    // FUSED: the chunk operands of the state update and of T, requested with
    // the rest of a head's inputs: rows r0.. of k~ and the wave's state rows of
    // scale q~^T as MFMA fragments, and w (for w^T) as 16-byte pieces; the
    // state gradient itself, the wave's RW row tiles x all column tiles
    constexpr int NKD = D / KS;
    constexpr int RW = FUSED ? (D / 16) / NW : 1, CWT = FUSED ? D / 16 : 1;
    static_assert(!FUSED || RW * NW == D / 16, "state row tiles per wave");
    Frag fKt[FUSED ? NKD : 1];
    Frag fQs[RW][FUSED ? NKC : 1];
    Vec16 pw[FUSED ? NQP : 1];
    f32x4 dst[RW][CWT];
    auto request_fused = [&](const size_t jh2, const int tid, const int l, const int rows,
                             const int srows) __attribute__((always_inline)) {
        if constexpr (FUSED) {
            const T* ktp = static_cast<const T*>(p.kt) + jh2 * C * D;
            const T* qsp = static_cast<const T*>(p.qsT) + jh2 * D * C;
            const T* wp = static_cast<const T*>(p.w) + jh2 * C * D;
#pragma unroll
            for (int k2 = 0; k2 < NKD; ++k2) fKt[k2] = frag_fo<T, D>(ktp, rows, k2 * KS, l);
#pragma unroll
            for (int i = 0; i < RW; ++i)
#pragma unroll
                for (int k2 = 0; k2 < NKC; ++k2) fQs[i][k2] = frag_fo<T, C>(qsp, srows + 16 * i, k2 * KS, l);
#pragma unroll
            for (int i = 0; i < NQP; ++i) pw[i] = ld16(wp + (size_t)(tid + i * NT) * V8);   // fragment order
        }
    };

    // GROUPED: fp32 group sums of dq, dk in this wave's accumulator tiles
    f32x4 dq_tot[GROUPED ? NTD : 1], dk_tot[GROUPED ? NTD : 1];
    if constexpr (GROUPED) {
#pragma unroll
        for (int t = 0; t < NTD; ++t) { dq_tot[t] = zero4(); dk_tot[t] = zero4(); }
    }

    // One value head per call of `head`. Around a loop (the item loop, or the
    // GQA group's heads) the compiler would hoist the lane- and wave-dependent
    // address arithmetic of every unrolled LDS access out of the body and keep
    // it live across iterations, which costs hundreds of registers: the body
    // derives its thread, lane and wave indices from opaque values instead.
    auto head = [&](const int j, const int hk, const int gi, const ChunkEntry ce, const bool first,
                    auto&& at_epilogue) __attribute__((always_inline)) {
        const int l = opaque_lane_id();  // fresh per head: see above
        const int tid = fresh_tid(w);
        // the wave's rows and column halves, also fresh per head (shadowing the
        // kernel-scope ones), so that no address derived from them is kept
        // live across the items of the persistent kernel
        const int w = [wk = wave_k] {
            int t = wk;
            asm volatile("" : "+s"(t));
            return t;
        }();
        const int rb = w % NB, ch = w / NB;
        const int r0 = 16 * rb;
        const int cd0 = ch * DH2, cc0 = ch * CH2, cv0 = ch * VH2;
        const int tok0 = ce.tok0, len = ce.len;
        char* U = U0;
        T* qL = qL0;
        T* kL = kL0;
        const int h = hk * p.G + gi;
        const size_t jh = (size_t)j * p.H + h;
        const long ldo = (long)p.H * D;

        __syncthreads();  // previous head's LDS use is over

        // ================= phase 1: state products over V slices =================
        // The slice pieces (rows of do, v, X, T and of h, dh') are loaded one
        // slice ahead into registers; every MFMA operand then comes from LDS or
        // from the row fragments of scale Aqk^T held in registers.
        f32x4 dqh[NTD], dkt_[NTD], dwP[NTD], dAq[NTC], dAp[NTC];
#pragma unroll
        for (int t = 0; t < NTD; ++t) { dqh[t] = zero4(); dkt_[t] = zero4(); dwP[t] = zero4(); }
#pragma unroll
        for (int t = 0; t < NTC; ++t) { dAq[t] = zero4(); dAp[t] = zero4(); }
        float dbp[4] = {0.f, 0.f, 0.f, 0.f};   // partial db of rows r0 + acc_row(i, l)

        T* XL = reinterpret_cast<T*>(U + L::P1_XL);
        T* hL = reinterpret_cast<T*>(U + L::P1_HL);
        T* dhL = reinterpret_cast<T*>(U + L::P1_DHL);
        T* dXT = reinterpret_cast<T*>(U + L::P1_DXT);
        T* vL = reinterpret_cast<T*>(U + L::P1_VL);
        T* doL = reinterpret_cast<T*>(U + L::P1_DOL);
        T* TL = reinterpret_cast<T*>(U + L::P1_TL);
        T* dvS = reinterpret_cast<T*>(U + L::DVS);
        const T* AmL = reinterpret_cast<const T*>(smem + L::AM_OFF);   // A [C][LC]; A^T through transposed loads

        float hdh[NPD];                                           // partial rowsum(h dh') per piece row
#pragma unroll
        for (int i = 0; i < NPD; ++i) hdh[i] = 0.f;
        if (first) {
#pragma unroll
            for (int i = 0; i < NQP; ++i) {
                const int e = tid + i * NT, r = e / (D / V8), d0 = (e % (D / V8)) * V8;
                st16(qL0 + r * LT + d0, r < len ? qv[i] : Vec16{});
                st16(kL0 + r * LT + d0, r < len ? kv[i] : Vec16{});
            }
        }
        // gate rows of the cumsum in 2a (one column, SR rows per thread), requested
        // in the last slice in place of a slice load; rows past the end zeroed at use
        constexpr int NSEG = NT / D, SR = C / NSEG;
        static_assert(NT % D == 0 && C % NSEG == 0, "cumsum segments");
        const int gd = tid % D, gsg = tid / D, grs0 = gsg * SR;
        float gpre[SR];

#pragma unroll
        for (int v0 = 0; v0 < D; v0 += BVS) {
            // GQA (whose group sums hold more registers): fresh opaque thread and
            // lane indices per slice, so that the slice's LDS and global
            // addresses are recomputed here instead of being kept live from the
            // head's start (29 -> 3 spilled registers at C = 32). Without GQA
            // the kept addresses measured faster.
            const int tid_h = tid, l_h = l;
            const int tid = GROUPED ? fresh_tid(w)
                                    : tid_h;
            const int l = GROUPED ? opaque_lane_id() : l_h;
            __syncthreads();  // the previous slice's LDS reads are over
            if (v0 == 0) {
                if (tid < C) bs[tid] = tid < len ? pbeta : 0.f;
                T* AmW = reinterpret_cast<T*>(smem + L::AM_OFF);
#pragma unroll
                for (int i = 0; i < NAM; ++i) {
                    const int e = min(tid + NT * i, C * (C / V8) - 1);
                    int ar, ac;   // A is stored in fragment order
                    fo_piece<T, C>(e, ar, ac);
                    st16(AmW + ar * LC + ac, pam[i]);
                }
                if constexpr (FUSED) {   // w rows (stored in fragment order) and 2^G_last
                    T* wW = reinterpret_cast<T*>(smem + L::F_W);
                    float* gam = reinterpret_cast<float*>(smem + L::F_GAM);
#pragma unroll
                    for (int i = 0; i < NQP; ++i) {
                        int wr, wc;
                        fo_piece<T, D>(tid + i * NT, wr, wc);
                        st16(wW + wr * LT + wc, pw[i]);
                    }
#pragma unroll
                    for (int i = 0; i < NPD; ++i) {
                        const int e = tid + NT * i;
                        if (e < D * PR && e % PR == 0) gam[e / PR] = pgl[i];
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < NPC; ++i) {
                const int e = tid + NT * i;
                if (e < C * PR) {
                    const int r = e / PR, c = (e % PR) * V8;
                    const bool real = r < len;
                    const Vec16 dv = real ? pdo[i] : Vec16{}, vv = real ? pv[i] : Vec16{};
                    st16(doL + r * LB + c, dv);
                    st16(vL + r * LB + c, vv);
                    st16(XL + r * LB + c, px[i]);
                    if constexpr (!FUSED) st16(TL + r * LB + c, pt[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < NPD; ++i) {
                const int e = tid + NT * i;
                if (e < D * PR) {
                    const int d = e / PR, c = (e % PR) * V8;
                    st16(hL + d * LB + c, ph[i]);
                    if constexpr (!FUSED) {
                        st16(dhL + d * LB + c, pdh[i]);
                        const T* ha = reinterpret_cast<const T*>(&ph[i]);
                        const T* hb2 = reinterpret_cast<const T*>(&pdh[i]);
                        float s2 = 0.f;
#pragma unroll
                        for (int q2 = 0; q2 < V8; ++q2) s2 += to_f32(ha[q2]) * to_f32(hb2[q2]);
                        hdh[i] += s2;
                    }
                }
            }
            if constexpr (FUSED) {   // dh' of the slice: the bf16 copy of the wave's state tiles
#pragma unroll
                for (int rt = 0; rt < RW; ++rt)
#pragma unroll
                    for (int ct = 0; ct < BVS / 16; ++ct)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            dhL[(16 * (RW * w + rt) + acc_row(e, l)) * LB + 16 * ct + acc_col(l)] =
                                from_f32<T>(dst[rt][v0 / 16 + ct][e]);
            }
            if (v0 + BVS < D) {
                request_slice(ce, jh, h, v0 + BVS, tid);   // next slice
            } else {
#pragma unroll
                for (int jj = 0; jj < SR; ++jj) {
                    const int rt = min(grs0 + jj, len - 1);
                    if constexpr (SCALAR) gpre[jj] = p.g[(size_t)(tok0 + rt) * p.H + h];
                    else gpre[jj] = p.g[((size_t)(tok0 + rt) * p.H + h) * D + gd];
                }
            }
            __syncthreads();
            // dX = T + scale Aqk^T do  (own rows, own half of the slice)
            f32x4 dX[NTV];
            if constexpr (FUSED) {
                // T = k~ dh' on chip (dh' rows as B through transposed loads),
                // kept as -T^T for the state update; rowsum(h dh') from LDS
                T* TTw = reinterpret_cast<T*>(smem + L::F_TT);
#pragma unroll
                for (int t = 0; t < NTV; ++t) dX[t] = zero4();
                panel_mma_ra<T, NTV, NKD, true>(dX, fKt, dhL, LB, cv0, l);
#pragma unroll
                for (int t = 0; t < NTV; ++t) {
                    const int c = cv0 + 16 * t + acc_col(l), rr = r0 + acc_row(0, l);
                    store4<T>(TTw + c * LC + rr, -dX[t][0], -dX[t][1], -dX[t][2], -dX[t][3]);
                }
#pragma unroll
                for (int i = 0; i < NPD; ++i) {
                    const int e = tid + NT * i;
                    if (e < D * PR) {
                        const int d = e / PR, c = (e % PR) * V8;
                        // both from LDS: the registers of h already hold the next slice
                        const Vec16 hv = ld16(hL + d * LB + c), dhv = ld16(dhL + d * LB + c);
                        const T* ha = reinterpret_cast<const T*>(&hv);
                        const T* hb2 = reinterpret_cast<const T*>(&dhv);
                        float s2 = 0.f;
#pragma unroll
                        for (int q2 = 0; q2 < V8; ++q2) s2 += to_f32(ha[q2]) * to_f32(hb2[q2]);
                        hdh[i] += s2;
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < NTV; ++t) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        dX[t][i] = to_f32(TL[(r0 + acc_row(i, l)) * LB + cv0 + 16 * t + acc_col(l)]);
                }
            }
            panel_mma_ra<T, NTV, NKC, true>(dX, fAq, doL, LB, cv0, l);   // do rows as B (transposed loads)
#pragma unroll
            for (int t = 0; t < NTV; ++t) {
                const int c = cv0 + 16 * t + acc_col(l), rr = r0 + acc_row(0, l);
                store4<T>(dXT + c * LC + rr, dX[t][0], dX[t][1], dX[t][2], dX[t][3]);
            }
            __syncthreads();
#pragma unroll
            for (int k0 = 0; k0 < BVS; k0 += KS) {
                const auto a_do = frag_kc(doL, LB, r0, k0, l);
                const auto a_x = frag_kc(XL, LB, r0, k0, l);
                const auto a_dx = frag_ks(dXT, LC, r0, k0, l);   // dX rows from dX^T (transposed loads)
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
            // dv^ = A^T dX; dv = beta dv^ (staged for row stores); db += rowsum(dv^ v)
            f32x4 dvh[NTV];
#pragma unroll
            for (int t = 0; t < NTV; ++t) dvh[t] = zero4();
            panel_mma<T, NTV, C, true>(dvh, AmL, LC, r0, dXT, LC, cv0, l);
#pragma unroll
            for (int t = 0; t < NTV; ++t) {
                const int c = cv0 + 16 * t + acc_col(l);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = r0 + acc_row(i, l);
                    dbp[i] += dvh[t][i] * to_f32(vL[r * LB + c]);
                    dvS[r * LT + v0 + c] = from_f32<T>(bs[r] * dvh[t][i]);
                }
            }
            if constexpr (FUSED) {
                // the reverse sweep's update of the slice's state columns:
                // dh = Diag(2^G_last) dh' + (scale q~)^T do + w^T (-T)
                const T* wL = reinterpret_cast<const T*>(smem + L::F_W);
                const T* TTr = reinterpret_cast<const T*>(smem + L::F_TT);
                const float* gam = reinterpret_cast<const float*>(smem + L::F_GAM);
#pragma unroll
                for (int rt = 0; rt < RW; ++rt) {
                    const int d0 = 16 * (RW * w + rt);
                    float gm[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) gm[e] = gam[d0 + acc_row(e, l)];
#pragma unroll
                    for (int ct = 0; ct < BVS / 16; ++ct) {
                        f32x4& sv = dst[rt][v0 / 16 + ct];
#pragma unroll
                        for (int e = 0; e < 4; ++e) sv[e] *= gm[e];
#pragma unroll
                        for (int k2 = 0; k2 < NKC; ++k2) {
                            sv = Mfma<T>::mma(fQs[rt][k2], frag_ks(doL, LB, 16 * ct, k2 * KS, l), sv);
                            sv = Mfma<T>::mma(frag_ks(wL, LT, d0, k2 * KS, l), frag_kc(TTr, LC, 16 * ct, k2 * KS, l), sv);
                        }
                    }
                }
            }
        }
        // dG_last, part 1: ln2 2^G_last rowsum_v(h dh') (the PR pieces of a row
        // sit in PR consecutive lanes)
#pragma unroll
        for (int i = 0; i < NPD; ++i) {
            static_assert(PR == 4 || PR == 8, "piece rows of 4 or 8 lanes");
            const float x = PR == 4 ? quad_sum(hdh[i]) : row8_sum(hdh[i]);
            const int e = tid + NT * i;
            if (e < D * PR && e % PR == 0) dGl[e / PR] = kLn2 * pgl[i] * x;
        }
        __syncthreads();  // phase-1 LDS is dead from here; dv is staged

        // ================= phase 2 =================
        // dv rows to the output, 16 bytes per access
        {
            T* dvout = static_cast<T*>(p.dv) + ((size_t)tok0 * p.H + h) * D;
            constexpr int NS = C * (D / V8) / NT;   // pieces per thread, read first
            static_assert(NS * NT == C * (D / V8), "row piece split");
            Vec16 a[NS];
#pragma unroll
            for (int it = 0; it < NS; ++it) {
                const int e = tid + it * NT, r = e / (D / V8), c = (e % (D / V8)) * V8;
                a[it] = ld16(dvS + r * LT + c);
            }
#pragma unroll
            for (int it = 0; it < NS; ++it) {
                const int e = tid + it * NT, r = e / (D / V8), c = (e % (D / V8)) * V8;
                if (r < len) st16(dvout + (size_t)r * ldo + c, a[it]);
            }
        }
        // 2a: G = chunk-local inclusive cumsum of g, one column and NT/D row
        // segments per thread, and k 2^G
        float* Gs = reinterpret_cast<float*>(U + L::P2_GS);
        T* kgL = reinterpret_cast<T*>(U + L::P2_KG);
        {
            float* segt = reinterpret_cast<float*>(U + L::P2_SEG);
            const int d = gd, sg = gsg, rs0 = grs0;
            float gl[SR];
            float run = 0.f;
#pragma unroll
            for (int jj = 0; jj < SR; ++jj) {
                run += rs0 + jj < len ? gpre[jj] : 0.f;
                gl[jj] = run;
            }
            segt[sg * D + d] = run;
            T kr[SR];   // the segment's k column, read before any write below
#pragma unroll
            for (int jj = 0; jj < SR; ++jj) kr[jj] = kL[(rs0 + jj) * LT + d];
            __syncthreads();
            float off = 0.f;   // all segment totals read (one wait), the earlier ones summed
#pragma unroll
            for (int s2 = 0; s2 < NSEG - 1; ++s2) {
                const float x = segt[s2 * D + d];
                off += s2 < sg ? x : 0.f;
            }
#pragma unroll
            for (int jj = 0; jj < SR; ++jj) {
                const int r = rs0 + jj;
                const float G = gl[jj] + off;
                Gs[r * LF + d] = G;
                kgL[r * LT + d] = from_f32<T>(to_f32(kr[jj]) * fast_exp2(G));
            }
        }
        __syncthreads();

        // 2b: post-factors, dw -> LDS. The LDS reads of the wave's rows (G, q,
        // k, beta) come first, in one batch; 2^G and k are kept for 2c.
        T* dwT = reinterpret_cast<T*>(U + L::P2_DWT);
        f32x4 Pq[NTD], Pk[NTD], PG[NTD];
        float eG[NTD][4], kvr[NTD][4], bsr[4];
        {
            float Gv[NTD][4], gls[NTD], qvr[NTD][4];
#pragma unroll
            for (int t = 0; t < NTD; ++t) {
                const int c = cd0 + 16 * t + acc_col(l);
                gls[t] = Gs[(C - 1) * LF + c];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = r0 + acc_row(i, l);
                    Gv[t][i] = Gs[r * LF + c];
                    qvr[t][i] = to_f32(qL[r * LT + c]);
                    kvr[t][i] = to_f32(kL[r * LT + c]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) bsr[i] = bs[r0 + acc_row(i, l)];
#pragma unroll
            for (int t = 0; t < NTD; ++t) {
                const int c = cd0 + 16 * t + acc_col(l);
                float colk = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    eG[t][i] = fast_exp2(Gv[t][i]);
                    const float dqi = p.scale * dqh[t][i] * eG[t][i];
                    const float dki = dkt_[t][i] * fast_exp2(gls[t] - Gv[t][i]);
                    Pq[t][i] = dqi;
                    Pk[t][i] = dki;
                    PG[t][i] = kLn2 * (qvr[t][i] * dqi - kvr[t][i] * dki);
                    colk += kvr[t][i] * dki;
                }
                // sum over the 16 rows of this wave (4 in-lane, 4 lane groups)
                colk = cross_row_sum(colk);
                if (l < 16) dGlw[rb * D + c] = kLn2 * colk;  // summed in block order later
                const int rr = r0 + acc_row(0, l);
                store4<T>(dwT + c * LC + rr, -dwP[t][0], -dwP[t][1], -dwP[t][2], -dwP[t][3]);
            }
        }
        __syncthreads();
        // 2c: dk^ = A^T dw ; dA' += dw (k 2^G)^T
        {
            f32x4 dkh[NTD];
#pragma unroll
            for (int t = 0; t < NTD; ++t) dkh[t] = zero4();
            panel_mma<T, NTD, C, true>(dkh, AmL, LC, r0, dwT, LC, cd0, l);
#pragma unroll
            for (int t = 0; t < NTD; ++t) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float gam = eG[t][i];
                    const float kgv = kvr[t][i] * gam;
                    Pk[t][i] += bsr[i] * gam * dkh[t][i];
                    PG[t][i] += kLn2 * bsr[i] * kgv * dkh[t][i];
                    dbp[i] += dkh[t][i] * kgv;
                }
            }
        }
        panel_mma<T, NTC, D, true>(dAp, dwT, LC, r0, kgL, LT, cc0, l);   // dw rows from dw^T (transposed loads)
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
            panel_mma<T, NTC, C>(t1, dAL, LC, r0, AmL, LC, cc0, l);
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                const int c = cc0 + 16 * t + acc_col(l), rr = r0 + acc_row(0, l);
                store4<T>(T1T + c * LC + rr, t1[t][0], t1[t][1], t1[t][2], t1[t][3]);
            }
        }
        __syncthreads();
        // 2e: dAkk = -StrictLower(A^T T1); dAqk = scale Lower_incl(do X^T), both
        // row-major [r][s] for the intra-chunk products
        T* dAqL = reinterpret_cast<T*>(U + L::P2_DAQ);
        T* dAkL = dAqL + C * LC;
        {
            f32x4 dAk[NTC];
#pragma unroll
            for (int t = 0; t < NTC; ++t) dAk[t] = zero4();
            panel_mma<T, NTC, C, true>(dAk, AmL, LC, r0, T1T, LC, cc0, l);
            __syncthreads();  // T1T reads done before the dA operands overwrite dead buffers
#pragma unroll
            for (int t = 0; t < NTC; ++t) {
                const int s = cc0 + 16 * t + acc_col(l), rr = r0 + acc_row(0, l);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rr + i;
                    dAqL[r * LC + s] = from_f32<T>(s <= r ? p.scale * dAq[t][i] : 0.f);
                    dAkL[r * LC + s] = from_f32<T>(s < r ? -dAk[t][i] : 0.f);
                }
            }
        }

        // 2f: intra-chunk gradient on MFMA: all threads scale the operands of
        // both column halves, then every wave multiplies in its own half
        T* const kE0 = reinterpret_cast<T*>(U + L::P2_X);   // [2][DH2][LC] k_s Eout_s
        T* const qE0 = kE0 + 2 * DH2 * LC;                    // [2][DH2][LC] q_r Ein_r
        T* const bkE0 = qE0 + 2 * DH2 * LC;                   // [2][DH2][LC] beta_r k_r Ein_r
        __syncthreads();  // dA written
        {   // all LDS reads of the thread's pieces first (one wait), then the
            // products and the transposed writes
            constexpr int NF = D * (C / 4) / NT;
            static_assert(NF * NT == D * (C / 4), "fill split");
            float Gv[NF][4], Gb[NF], Gn[NF], kv[NF][4], qv2[NF][4], bv[NF][4];
#pragma unroll
            for (int it = 0; it < NF; ++it) {
                const int e = tid + it * NT, d = e % D, s0 = (e / D) * 4;
                const int b0 = s0 & ~15;
                const int nb = b0 + 16 < C ? b0 + 16 : C - 1;  // Eout reference (last block: its last row)
                Gb[it] = Gs[b0 * LF + d];
                Gn[it] = Gs[nb * LF + d];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int s = s0 + jj;
                    Gv[it][jj] = Gs[s * LF + d];
                    kv[it][jj] = to_f32(kL[s * LT + d]);
                    qv2[it][jj] = to_f32(qL[s * LT + d]);
                    bv[it][jj] = bs[s];
                }
            }
#pragma unroll
            for (int it = 0; it < NF; ++it) {
                const int e = tid + it * NT, d = e % D, s0 = (e / D) * 4;
                float ke[4], qe[4], bke[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float ein = fast_exp2(Gv[it][jj] - Gb[it]);
                    ke[jj] = kv[it][jj] * fast_exp2(Gn[it] - Gv[it][jj]);
                    qe[jj] = qv2[it][jj] * ein;
                    bke[jj] = bv[it][jj] * kv[it][jj] * ein;
                }
                const int o = ((d / DH2) * DH2 + d % DH2) * LC + s0;
                store4<T>(kE0 + o, ke[0], ke[1], ke[2], ke[3]);
                store4<T>(qE0 + o, qe[0], qe[1], qe[2], qe[3]);
                store4<T>(bkE0 + o, bke[0], bke[1], bke[2], bke[3]);
            }
        }
        __syncthreads();
        // each wave runs its half once, at hf == ch (the loop keeps the compiler
        // from moving the half's address arithmetic ahead of the fill)
#pragma unroll 1
        for (int hf = 0; hf < 2; ++hf) {
            if (ch != hf) continue;
            T* const kET = kE0 + ch * DH2 * LC;
            T* const qET = qE0 + ch * DH2 * LC;
            T* const bkET = bkE0 + ch * DH2 * LC;
            const int l = opaque_lane_id();  // see the head body
            using F16 = typename Mfma16<T>::frag;
            constexpr int ST = Mfma16<T>::STEPS;
            // G of this wave's rows and of its block's first row; the guard
            // also covers the next block's first row (the diagonal's Eout reference)
            float gr[NTD][4], grho[NTD];
            float rmax = 0.f;
#pragma unroll
            for (int t = 0; t < NTD; ++t) {
                const int c = cd0 + 16 * t + acc_col(l);
                grho[t] = Gs[r0 * LF + c];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    gr[t][i] = Gs[(r0 + acc_row(i, l)) * LF + c];
                    rmax = fmaxf(rmax, fabsf(gr[t][i] - grho[t]));
                }
                if (rb < NB - 1) rmax = fmaxf(rmax, fabsf(Gs[(r0 + 16) * LF + c] - grho[t]));
            }
            const bool diag_mfma = wave_max(rmax) <= diag_guard<T>();

            // row side: accq, acck of rows r in block rb
            {
                const int l = opaque_lane_id();
                f32x4 aq[NTD], ak[NTD];
#pragma unroll
                for (int t = 0; t < NTD; ++t) { aq[t] = zero4(); ak[t] = zero4(); }
                // the operands of block b1 (the two G rows of its decay factor,
                // the dAqk / dAkk fragments, the k Eout fragments) are read one
                // block ahead, so each step waits only on reads issued a step
                // earlier (the last read is a redundant valid one); with GQA,
                // whose group sums hold more registers, at the top of the step
                struct RowOps {
                    float g1[NTD], g0[NTD];
                    F16 fq[ST], fk[ST], fb[ST][NTD];
                };
                auto read_row = [&](RowOps& o, const int b1) __attribute__((always_inline)) {
#pragma unroll
                    for (int t = 0; t < NTD; ++t) {
                        const int c = cd0 + 16 * t + acc_col(l);
                        o.g1[t] = Gs[16 * (b1 + 1) * LF + c];
                        o.g0[t] = Gs[16 * b1 * LF + c];
                    }
#pragma unroll
                    for (int st = 0; st < ST; ++st) {
                        o.fq[st] = frag16_kc(dAqL, LC, r0, 16 * b1, st, l);
                        o.fk[st] = frag16_kc(dAkL, LC, r0, 16 * b1, st, l);
#pragma unroll
                        for (int t = 0; t < NTD; ++t) o.fb[st][t] = frag16_kc(kET, LC, 16 * t, 16 * b1, st, l);
                    }
                };
                RowOps cur, nxt;
                if constexpr (!GROUPED) {
                    if (rb > 0) read_row(cur, 0);
                }
                for (int b1 = 0; b1 < rb; ++b1) {
                    if constexpr (GROUPED) read_row(cur, b1);
                    else read_row(nxt, b1 + 1 < rb ? b1 + 1 : b1);
#pragma unroll
                    for (int t = 0; t < NTD; ++t) {
                        const float ph = fast_exp2(b1 > 0 ? cur.g1[t] - cur.g0[t] : 0.f);
                        aq[t] *= ph;
                        ak[t] *= ph;
                    }
#pragma unroll
                    for (int t = 0; t < NTD; ++t)
#pragma unroll
                        for (int st = 0; st < ST; ++st) {
                            aq[t] = Mfma16<T>::mma(cur.fq[st], cur.fb[st][t], aq[t]);
                            ak[t] = Mfma16<T>::mma(cur.fk[st], cur.fb[st][t], ak[t]);
                        }
                    if constexpr (!GROUPED) cur = nxt;
                }
                // reference of the sum: G_16rb for the cross part alone; with the
                // diagonal on MFMA (sources k Eout, reference G_nb) the cross part
                // is moved to G_nb first (a factor <= 1, >= 2^-guard)
                const int nbr = rb < NB - 1 ? r0 + 16 : C - 1;
                float gref[NTD];
#pragma unroll
                for (int t = 0; t < NTD; ++t) gref[t] = diag_mfma ? Gs[nbr * LF + cd0 + 16 * t + acc_col(l)] : grho[t];
                if (diag_mfma) {
#pragma unroll
                    for (int t = 0; t < NTD; ++t) {
                        const float ph = fast_exp2(gref[t] - grho[t]);
                        aq[t] *= ph;
                        ak[t] *= ph;
                        aq[t] = mma16<T, false>(aq[t], dAqL, LC, r0, r0, kET, LC, 16 * t, r0, l);
                        ak[t] = mma16<T, false>(ak[t], dAkL, LC, r0, r0, kET, LC, 16 * t, r0, l);
                    }
                }
#pragma unroll
                for (int t = 0; t < NTD; ++t) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float f = fast_exp2(gr[t][i] - gref[t]);   // Ein, or 2^(G_r - G_nb) <= 2^guard
                        aq[t][i] *= f;
                        ak[t][i] *= f;
                    }
                }
                if (!diag_mfma) {  // exact diagonal block, one exp2 per (r, s, d)
                    for (int j2 = 0; j2 < 16; ++j2) {
                        const int s = r0 + j2;
                        float aqs[4], aks[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int r = r0 + acc_row(i, l);
                            aqs[i] = to_f32(dAqL[r * LC + s]);
                            aks[i] = to_f32(dAkL[r * LC + s]);
                        }
#pragma unroll
                        for (int t = 0; t < NTD; ++t) {
                            const int c = cd0 + 16 * t + acc_col(l);
                            const float ks = to_f32(kL[s * LT + c]), gsv = Gs[s * LF + c];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                if (j2 <= acc_row(i, l)) {
                                    const float e = ks * fast_exp2(gr[t][i] - gsv);
                                    aq[t][i] += aqs[i] * e;
                                    ak[t][i] += aks[i] * e;
                                }
                            }
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < NTD; ++t) {
                    const int c = cd0 + 16 * t + acc_col(l);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = r0 + acc_row(i, l);
                        const float qv = to_f32(qL[r * LT + c]), kv = to_f32(kL[r * LT + c]), br = bs[r];
                        Pq[t][i] += aq[t][i];
                        Pk[t][i] += br * ak[t][i];
                        PG[t][i] += kLn2 * (qv * aq[t][i] + br * kv * ak[t][i]);
                        dbp[i] += kv * ak[t][i];
                    }
                }
            }
            // column side: dkt of sources s in block rb, later blocks first (Horner)
            {
                const int l = opaque_lane_id();
                f32x4 dk[NTD];
#pragma unroll
                for (int t = 0; t < NTD; ++t) dk[t] = zero4();
                // operands one block ahead, as on the row side
                struct ColOps {
                    float g1[NTD], g0[NTD];
                    F16 fq[ST], fk[ST], fbq[ST][NTD], fbk[ST][NTD];
                };
                auto read_col = [&](ColOps& o, const int b2) __attribute__((always_inline)) {
#pragma unroll
                    for (int t = 0; t < NTD; ++t) {
                        const int c = cd0 + 16 * t + acc_col(l);
                        o.g1[t] = Gs[(16 * (b2 + 1) < C ? 16 * (b2 + 1) : C - 1) * LF + c];
                        o.g0[t] = Gs[16 * b2 * LF + c];
                    }
#pragma unroll
                    for (int st = 0; st < ST; ++st) {
                        o.fq[st] = frag16_ks(dAqL, LC, r0, 16 * b2, st, l);
                        o.fk[st] = frag16_ks(dAkL, LC, r0, 16 * b2, st, l);
#pragma unroll
                        for (int t = 0; t < NTD; ++t) {
                            o.fbq[st][t] = frag16_kc(qET, LC, 16 * t, 16 * b2, st, l);
                            o.fbk[st][t] = frag16_kc(bkET, LC, 16 * t, 16 * b2, st, l);
                        }
                    }
                };
                ColOps cur, nxt;
                if constexpr (!GROUPED) {
                    if (rb < NB - 1) read_col(cur, NB - 1);
                }
                for (int b2 = NB - 1; b2 > rb; --b2) {
                    if constexpr (GROUPED) read_col(cur, b2);
                    else read_col(nxt, b2 - 1 > rb ? b2 - 1 : b2);
#pragma unroll
                    for (int t = 0; t < NTD; ++t) dk[t] *= fast_exp2(b2 < NB - 1 ? cur.g1[t] - cur.g0[t] : 0.f);
#pragma unroll
                    for (int t = 0; t < NTD; ++t) {
#pragma unroll
                        for (int st = 0; st < ST; ++st) dk[t] = Mfma16<T>::mma(cur.fq[st], cur.fbq[st][t], dk[t]);
#pragma unroll
                        for (int st = 0; st < ST; ++st) dk[t] = Mfma16<T>::mma(cur.fk[st], cur.fbk[st][t], dk[t]);
                    }
                    if constexpr (!GROUPED) cur = nxt;
                }
                if (diag_mfma) {
                    if (rb < NB - 1) {
#pragma unroll
                        for (int t = 0; t < NTD; ++t) {
                            const int c = cd0 + 16 * t + acc_col(l);
                            dk[t] *= fast_exp2(Gs[(r0 + 16) * LF + c] - grho[t]);
                        }
                    }
#pragma unroll
                    for (int t = 0; t < NTD; ++t) {
                        dk[t] = mma16<T, true>(dk[t], dAqL, LC, r0, r0, qET, LC, 16 * t, r0, l);
                        dk[t] = mma16<T, true>(dk[t], dAkL, LC, r0, r0, bkET, LC, 16 * t, r0, l);
#pragma unroll
                        for (int i = 0; i < 4; ++i) dk[t][i] *= fast_exp2(grho[t] - gr[t][i]);
                    }
                } else {
                    if (rb < NB - 1) {
#pragma unroll
                        for (int t = 0; t < NTD; ++t) {
                            const int c = cd0 + 16 * t + acc_col(l);
                            const float gn = Gs[(r0 + 16) * LF + c];
#pragma unroll
                            for (int i = 0; i < 4; ++i) dk[t][i] *= fast_exp2(gn - gr[t][i]);
                        }
                    }
                    for (int j2 = 0; j2 < 16; ++j2) {  // exact diagonal block
                        const int r = r0 + j2;
                        float aqs[4], aks[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const int s = r0 + acc_row(i, l);
                            aqs[i] = to_f32(dAqL[r * LC + s]);
                            aks[i] = to_f32(dAkL[r * LC + s]);
                        }
                        const float br = bs[r];
#pragma unroll
                        for (int t = 0; t < NTD; ++t) {
                            const int c = cd0 + 16 * t + acc_col(l);
                            const float qv = to_f32(qL[r * LT + c]), bkv = br * to_f32(kL[r * LT + c]);
                            const float gv = Gs[r * LF + c];
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                if (j2 >= acc_row(i, l)) {
                                    const float e = fast_exp2(gv - gr[t][i]);
                                    dk[t][i] += (aqs[i] * qv + aks[i] * bkv) * e;
                                }
                            }
                        }
                    }
                }
#pragma unroll
                for (int t = 0; t < NTD; ++t) {
                    const int c = cd0 + 16 * t + acc_col(l);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int s = r0 + acc_row(i, l);
                        Pk[t][i] += dk[t][i];
                        PG[t][i] -= kLn2 * to_f32(kL[s * LT + c]) * dk[t][i];
                    }
                }
            }
        }

        // ================= epilogue (accumulator layout) =================
        {   // the next item's first requests (persistent kernel), addressed from
            // fresh opaque thread and lane indices, so that no address part is
            // shared with this item's own requests and kept live until here
            const int t2 = fresh_tid(w);
            at_epilogue(t2, opaque_lane_id(), r0);
        }
        {
            const int l = opaque_lane_id();
            // db: row sums of the partials over this wave's column half
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = row16_sum(dbp[i]);
                if ((l & 15) == 0) dbS[ch * C + r0 + acc_row(i, l)] = x;
            }
            // dG_last joins the last row of the chunk
            const int lg = l >> 4;
            if (rb == NB - 1 && lg == 3) {
#pragma unroll
                for (int t = 0; t < NTD; ++t) {
                    const int c = cd0 + 16 * t + acc_col(l);
                    float sl = dGl[c];
                    for (int b2 = 0; b2 < NB; ++b2) sl += dGlw[b2 * D + c];
                    PG[t][3] += sl;
                }
            }
            // reverse cumsum of dG over the chunk, per column: the lane's 4 rows,
            // then the later lane groups, then the later row blocks
#pragma unroll
            for (int t = 0; t < NTD; ++t) {
                const int c = cd0 + 16 * t + acc_col(l);
                PG[t][2] += PG[t][3];
                PG[t][1] += PG[t][2];
                PG[t][0] += PG[t][1];
                const float tot = PG[t][0];
                // totals of the later lane groups (rows lg ^ 1, lg ^ 2, lg ^ 3)
                const float u = xor16(tot, l), v = xor32(tot, l), uv = xor32(u, l);
                const float ex = lg == 0 ? u + v + uv : lg == 1 ? v + uv : lg == 2 ? u : 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) PG[t][i] += ex;
                if (lg == 0) btot[rb * D + c] = PG[t][0];
            }
            __syncthreads();  // block totals, db partials; 2f LDS is dead
#pragma unroll
            for (int t = 0; t < NTD; ++t) {
                const int c = cd0 + 16 * t + acc_col(l);
                float suf = 0.f;   // all NB totals read (one wait), the later blocks' summed
#pragma unroll
                for (int b2 = 1; b2 < NB; ++b2) {
                    const float x = btot[b2 * D + c];
                    suf += b2 > rb ? x : 0.f;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) PG[t][i] += suf;
            }
            // stage dq, dk, dg for row-contiguous stores
            T* dqS = reinterpret_cast<T*>(U + L::E_DQ);
            T* dkS = reinterpret_cast<T*>(U + L::E_DK);
            float* dgS = reinterpret_cast<float*>(U + L::E_DG);
#pragma unroll
            for (int t = 0; t < NTD; ++t) {
                const int c = cd0 + 16 * t + acc_col(l);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = r0 + acc_row(i, l);
                    if constexpr (!SCALAR) dgS[r * LF + c] = PG[t][i];
                    if constexpr (GROUPED) {
                        dq_tot[t][i] += Pq[t][i];
                        dk_tot[t][i] += Pk[t][i];
                    } else if (FUSED && p.G > 1) {   // fp32 partials of this value head
                        if (r < len) {
                            const size_t o = ((size_t)(tok0 + r) * p.H + h) * D + c;
                            p.dqp[o] = Pq[t][i];
                            p.dkp[o] = Pk[t][i];
                        }
                    } else {
                        dqS[r * LT + c] = from_f32<T>(Pq[t][i]);
                        dkS[r * LT + c] = from_f32<T>(Pk[t][i]);
                    }
                }
            }
            if constexpr (SCALAR) {  // dg_r = sum over channels of the suffix sums
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = 0.f;
#pragma unroll
                    for (int t = 0; t < NTD; ++t) x += PG[t][i];
                    x = row16_sum(x);
                    if ((l & 15) == 0) dgR[ch * C + r0 + acc_row(i, l)] = x;
                }
            }
            __syncthreads();
            if constexpr (!GROUPED) {
                if (!FUSED || p.G == 1) store_rows<T, C, D, NT>(p, dqS, dkS, tok0, len, hk, tid);
            }
            if constexpr (!SCALAR) {
                constexpr int NS = C * (D / 4) / NT;   // pieces per thread, read first
                static_assert(NS * NT == C * (D / 4), "row piece split");
                f32x4 a[NS];
#pragma unroll
                for (int it = 0; it < NS; ++it) {
                    const int e = tid + it * NT, r = e / (D / 4), c = (e % (D / 4)) * 4;
                    a[it] = *reinterpret_cast<const f32x4*>(dgS + r * LF + c);
                }
#pragma unroll
                for (int it = 0; it < NS; ++it) {
                    const int e = tid + it * NT, r = e / (D / 4), c = (e % (D / 4)) * 4;
                    if (r < len) *reinterpret_cast<f32x4*>(p.dg + ((size_t)(tok0 + r) * p.H + h) * D + c) = a[it];
                }
            }
        }
        if (tid < C && tid < len) {
            static_cast<T*>(p.db)[(size_t)(tok0 + tid) * p.H + h] = from_f32<T>(dbS[tid] + dbS[C + tid]);
            if constexpr (SCALAR) p.dg[(size_t)(tok0 + tid) * p.H + h] = dgR[tid] + dgR[C + tid];
        }
    };
    if constexpr (GROUPED) {
        // one workgroup per (chunk, q/k head); its value heads in turn, dq and
        // dk summed over them in fp32
        const int j = blockIdx.x, hk = blockIdx.y;
        if (j >= p.seq_off[p.N]) return;
        const ChunkEntry ce = p.ctab[j];
        const int tok0 = ce.tok0, len = ce.len, tid = threadIdx.x, l = lane_id();
        auto none = [](int, int, int) {};
        request_qk(ce, hk, tid);
        request_head(ce, j, hk * p.G, tid, l, r0);
        head(j, hk, 0, ce, true, none);
        for (int gi = 1; gi < p.G; ++gi) {
            request_head(ce, j, hk * p.G + gi, tid, l, r0);
            head(j, hk, gi, ce, false, none);
        }
        // dq, dk group sums: staged in LDS, stored row-contiguous
        __syncthreads();
        T* dqS = reinterpret_cast<T*>(U0 + L::E_DQ);
        T* dkS = reinterpret_cast<T*>(U0 + L::E_DK);
#pragma unroll
        for (int t = 0; t < NTD; ++t) {
            const int c = cd0 + 16 * t + acc_col(l);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + acc_row(i, l);
                dqS[r * LT + c] = from_f32<T>(dq_tot[t][i]);
                dkS[r * LT + c] = from_f32<T>(dk_tot[t][i]);
            }
        }
        __syncthreads();
        store_rows<T, C, D, NT>(p, dqS, dkS, tok0, len, hk, tid);
    } else if constexpr (FUSED) {
        // one workgroup per (sequence n, value head h), chunks from the last to
        // the first; dh starts as dht and ends as dh0
        // varlen: sequences longest first (the chunk table's order), so the
        // longest walks start first
        const int ns = blockIdx.x / p.H, h = blockIdx.x % p.H, hk = h / p.G, gi = h % p.G;
        const int n = p.varlen ? p.seq_ord[ns] : ns;
        const int c0 = p.seq_off[n], c1 = p.seq_off[n + 1];
        const size_t sh = ((size_t)n * p.H + h) * D * D;
        const int l = lane_id();
#pragma unroll
        for (int rt = 0; rt < RW; ++rt)
#pragma unroll
            for (int ct = 0; ct < CWT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int d = 16 * (RW * w + rt) + acc_row(e, l), c = 16 * ct + acc_col(l);
                    dst[rt][ct][e] = p.dht ? p.dht[sh + state_index<D>(p, d, c)] : 0.f;
                }
        if (c1 > c0) {
            ChunkEntry ce = p.ctab[c1 - 1];
            request_qk(ce, hk, threadIdx.x);
            request_head(ce, c1 - 1, h, threadIdx.x, l, r0);
            request_fused((size_t)(c1 - 1) * p.H + h, threadIdx.x, l, r0, 16 * RW * w);
#pragma unroll 1
            for (int j = c1 - 1; j >= c0; --j) {
                const int jn = j > c0 ? j - 1 : j;   // past the first chunk: a redundant valid request
                const ChunkEntry ce_n = p.ctab[jn];
                head(j, hk, gi, ce, true, [&](const int tid, const int l2, const int rows) __attribute__((always_inline)) {
                    request_qk(ce_n, hk, tid);
                    request_head(ce_n, jn, h, tid, l2, rows);
                    request_fused((size_t)jn * p.H + h, tid, l2, rows, 16 * RW * (tid >> 6));
                });
                ce = ce_n;
            }
        }
#pragma unroll
        for (int rt = 0; rt < RW; ++rt)
#pragma unroll
            for (int ct = 0; ct < CWT; ++ct)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int d = 16 * (RW * w + rt) + acc_row(e, l), c = 16 * ct + acc_col(l);
                    p.dh0[sh + state_index<D>(p, d, c)] = dst[rt][ct][e];
                }
    } else {
        // persistent: at most one workgroup per CU walks the (chunk, head)
        // items blockIdx.x, + gridDim.x, ...; the next item's first requests go
        // out in the current item's epilogue (past the end: a redundant valid one)
        const int nit = p.seq_off[p.N] * p.Hg;
        int item = blockIdx.x;
        if (item >= nit) return;
        ChunkEntry ce = p.ctab[item / p.Hg];
        request_qk(ce, item % p.Hg, threadIdx.x);
        request_head(ce, item / p.Hg, item % p.Hg, threadIdx.x, lane_id(), r0);
#pragma unroll 1
        for (; item < nit; item += gridDim.x) {
            const int nxt = min(item + (int)gridDim.x, nit - 1);
            const ChunkEntry ce_n = p.ctab[nxt / p.Hg];
            head(item / p.Hg, item % p.Hg, 0, ce, true, [&](const int tid, const int l, const int rows) __attribute__((always_inline)) {
                request_qk(ce_n, nxt % p.Hg, tid);
                request_head(ce_n, nxt / p.Hg, nxt % p.Hg, tid, l, rows);
            });
            ce = ce_n;
        }
    }
}

// dq, dk of the fused reverse kernel with GQA: the fp32 partials of the value
// heads of each group added in group order (deterministic), rounded once to
// the io type. One thread per 4 consecutive columns of a (token, q/k head);
// varlen tokens outside [cu_seqlens[0], cu_seqlens[n]) are not written.
template <typename T, int D>
__global__ __launch_bounds__(256) void gdr_group_sum(Params p) {
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (size_t)(p.B * p.T) * p.Hg * (D / 4)) return;
    const int c = (int)(e % (D / 4)) * 4;
    const size_t th = e / (D / 4);
    const int hk = (int)(th % p.Hg);
    const int tok = (int)(th / p.Hg);
    if (p.varlen) {
        const int nt = (int)p.T, a = min(max(p.cu[0], 0), nt), b = min(max(p.cu[p.N], a), nt);
        if (tok < a || tok >= b) return;
    }
    f32x4 sq = zero4(), sk = zero4();
    for (int gi = 0; gi < p.G; ++gi) {
        const size_t o = ((size_t)tok * p.H + hk * p.G + gi) * D + c;
        sq += *reinterpret_cast<const f32x4*>(p.dqp + o);
        sk += *reinterpret_cast<const f32x4*>(p.dkp + o);
    }
    const size_t oo = ((size_t)tok * p.Hg + hk) * D + c;
    store4<T>(static_cast<T*>(p.dq) + oo, sq[0], sq[1], sq[2], sq[3]);
    store4<T>(static_cast<T*>(p.dk) + oo, sk[0], sk[1], sk[2], sk[3]);
}

}  // namespace gdr
