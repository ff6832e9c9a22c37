// gdr_prep.hpp -- chunk table and the chunk-parallel preparation kernel.
//
// gdr_prep computes, for one (chunk, value head), the WY factors of the chunk
// form of the gated delta rule and the quantities the two state sweeps need:
//   G     chunk-local inclusive cumsum of the raw log2 gate (fp32, in LDS only;
//         the bwd_intra page takes this cumsum as its g input),
//   Aqk   [r,s] = sum_d q_rd k_sd 2^(G_rd - G_sd),          s <= r,
//   Akk   [r,s] = beta_r sum_d k_rd k_sd 2^(G_rd - G_sd),    s <  r,
//   A     = (I + Akk)^-1 (unit lower triangular; the "Ar"/"Ag" factor of the
//           FlashQLA page's CONSUMER_A steps),
//   w     = A (beta k 2^G),  u = A (beta v),
//   k~    = k 2^(G_last - G),  q~ = q 2^G - Aqk w,  2^G_last.
// Diagonal 16x16 blocks of Aqk/Akk use MFMA on operands scaled through the
// block's first row b0: q_r 2^(G_r - G_b0) <= 1 against k_s 2^(G_b0 - G_s),
// whose exponent G_b0 - G_s is >= 0: a positive exponent, allowed only while
// the block's gate range |G_r - G_b0| stays within a bound that keeps that
// operand finite in the operand type (64, i.e. 2^64, for bf16 / fp32; 8 for
// fp16). This departs from the bwd_intra page, which forms every diagonal
// block per element with exponents <= 0 only; beyond the bound the block is
// formed that way here too, one decay per (r, s, d), as a running product of
// per-token factors 2^g <= 1 along s.
// Off-diagonal blocks use MFMA on operands prescaled through the block
// boundary rho = 16 i of the target row block: q 2^(G_r - G_rho) and
// k 2^(G_rho - G_s), both exponents <= 0 (the per-block-boundary form of the
// bwd_intra page).
// A chunk (C = 64 or 32) whose every |G_r - G_last / 2| is within that same bound
// takes a shorter route instead: all of Aqk and Akk as two masked C x C
// products over D, on operands scaled once through the one reference
// G_last / 2 per column (exponents of either sign, bounded as above). The
// bound is checked per chunk from its cumsum; a chunk beyond it takes the
// per-boundary route.
// With a scalar gate (one G per row) the decay 2^(G_r - G_s) is the same for
// every channel, so Aqk and Akk are the plain products q k^T and k k^T over D
// (operands as loaded), each element then times its decay (exponent <= 0
// below the diagonal) in fp32: one route for every chunk at C = 64 or 32, no
// operand scaling and no bound (GDN GQA workload prep 475 -> 418 us).
#pragma once
#include "gdr_common.hpp"

namespace gdr {

// ---------------------------------------------------------------------------
// Chunk table: one workgroup. seq_off[n] = first global chunk of sequence n,
// ctab[j] = {first token, length, sequence, chunk index in the sequence}.
// Varlen: seq_ord = the sequences by chunk count, longest first.
// Fixed length: B sequences of T. Sequences are taken 256 at a time: a scan
// of their chunk counts gives their first chunks, then every thread writes
// entries of the block's chunks, finding each chunk's sequence by binary
// search over the scan (so a long sequence is not written by one thread).
// ---------------------------------------------------------------------------
template <int C>
__global__ __launch_bounds__(256) void gdr_chunk_table(Params p) {
    __shared__ int s_scan[256], s_tok[256], s_len[256];
    __shared__ int s_base;
    const int tid = threadIdx.x;
    if (tid == 0) s_base = 0;
    __syncthreads();
    for (int n0 = 0; n0 < p.N; n0 += 256) {
        const int n = n0 + tid;
        int len = 0, tok0 = 0;
        if (n < p.N) seq_span(p, n, tok0, len);
        const int nch = (len + C - 1) / C;
        s_scan[tid] = nch;
        s_tok[tid] = tok0;
        s_len[tid] = len;
        __syncthreads();
        for (int off = 1; off < 256; off <<= 1) {  // inclusive Hillis-Steele scan
            int v = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += v;
            __syncthreads();
        }
        const int base = s_base, tot = s_scan[255];
        if (n < p.N) p.seq_off[n] = min(base + s_scan[tid] - nch, p.nc_max);
        for (int c = tid; c < tot && base + c < p.nc_max; c += 256) {
            int lo = 0, hi = 255;   // first i with s_scan[i] > c
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (s_scan[mid] > c) hi = mid;
                else lo = mid + 1;
            }
            const int cc = c - (lo ? s_scan[lo - 1] : 0);   // chunk index within sequence n0 + lo
            ChunkEntry e;
            e.tok0 = s_tok[lo] + cc * C;
            e.len = min(C, s_len[lo] - cc * C);
            e.seq = n0 + lo;
            e.pad_ = cc;
            p.ctab[base + c] = e;
        }
        __syncthreads();
        if (tid == 0) s_base = base + tot;
        __syncthreads();
    }
    if (tid == 0) p.seq_off[p.N] = min(s_base, p.nc_max);
    if (!p.varlen) return;
    // Varlen: the sequences ordered by chunk count, longest first, for the
    // state sweeps' block order (the longest jobs start first). A counting
    // sort over kBuckets counts (longer sequences share the top bucket):
    // histogram, exclusive scan from the top bucket down, then each sequence
    // takes the next slot of its bucket (ties land in any order; only the
    // order of the workgroups depends on it, not any result).
    constexpr int kBuckets = 1024, BPT = kBuckets / 256;
    __shared__ int s_hist[kBuckets];
    auto bucket = [&](int n) {
        int len, tok0;
        seq_span(p, n, tok0, len);
        return kBuckets - 1 - min((len + C - 1) / C, kBuckets - 1);   // 0 = longest
    };
    for (int b = tid; b < kBuckets; b += 256) s_hist[b] = 0;
    __syncthreads();
    for (int n = tid; n < p.N; n += 256) atomicAdd(&s_hist[bucket(n)], 1);
    __syncthreads();
    int cnt[BPT], sum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) sum += (cnt[i] = s_hist[BPT * tid + i]);
    s_scan[tid] = sum;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive scan of the per-thread sums
        int v = tid >= off ? s_scan[tid - off] : 0;
        __syncthreads();
        s_scan[tid] += v;
        __syncthreads();
    }
    int start = s_scan[tid] - sum;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        s_hist[BPT * tid + i] = start;
        start += cnt[i];
    }
    __syncthreads();
    for (int n = tid; n < p.N; n += 256) p.seq_ord[atomicAdd(&s_hist[bucket(n)], 1)] = n;
}

// ---------------------------------------------------------------------------
// LDS plan of gdr_prep (byte offsets), see the phase comments in the kernel.
// ---------------------------------------------------------------------------
template <typename T, int C, int D>
struct PrepLds {
    static constexpr int NB = C / 16;
    static constexpr int NW = 2 * NB;         // waves: two per 16-row block
    static constexpr int NT = 64 * NW;
    static constexpr int LT = D + pad<T>();   // T  [*][D]
    static constexpr int LC = C + pad<T>();   // T  [*][C]
    static constexpr int LF = D + 4;          // f32 [*][D]
    static constexpr int LCF = C + 4;         // f32 [*][C]
    static constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }
    static constexpr size_t G_OFF = 0;
    static constexpr size_t Q_OFF = G_OFF + size_t(C) * LF * 4;
    static constexpr size_t K_OFF = Q_OFF + size_t(C) * LT * sizeof(T);
    static constexpr size_t X_OFF = K_OFF + size_t(C) * LT * sizeof(T);
    static constexpr size_t X_BYTES = cmax(cmax(size_t(C) * LF * 4, size_t(C + 16) * LT * sizeof(T)),
                                           size_t(D) * LC * sizeof(T));
    static constexpr size_t AQK_OFF = X_OFF + X_BYTES;
    static constexpr size_t AKK_OFF = AQK_OFF + size_t(C) * LCF * 4;
    static constexpr size_t AF_OFF = AKK_OFF + size_t(C) * LCF * 4;
    static constexpr size_t SCR_OFF = AF_OFF + size_t(C) * LCF * 4;
    static constexpr size_t FLAG_OFF = SCR_OFF + size_t(NB) * 16 * 20 * 4;     // f32 [NW]: per wave, max |G_r - G_last / 2|
    static constexpr size_t BETA_OFF = FLAG_OFF + size_t(NW) * 4;
    static constexpr size_t TOTAL = BETA_OFF + size_t(C) * 4;
    // the one-reference form of Aqk / Akk (phases 2-3) keeps its three [C][LT]
    // operands in the X region and the Aqk / Akk regions that follow it (the
    // products land there after a barrier); A's region stays untouched
    // (both chunk sizes: at C = 32 the three operands fill that span exactly)
    static constexpr bool FAST = (C == 64 || C == 32) && 3 * size_t(C) * LT * sizeof(T) <= AF_OFF - X_OFF;
    // after the inverse, A and Aqk are converted in place to MFMA operands
    static_assert(size_t(C) * LC * sizeof(T) <= size_t(C) * LCF * 4, "A/Aqk in place");
    static_assert(size_t(NB) * 16 * 20 >= size_t(NT > D ? NT : D) * 1, "cumsum scratch");
    static_assert(TOTAL <= 163840, "LDS budget of gdr_prep");
};

// Eight consecutive elements of a T row at p (16 bytes for 16-bit T, 32 for fp32).
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&x)[8]) {
    if constexpr (sizeof(T) == 2) {
        const Vec16 v = ld16(p);
        const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = to_f32(e[i]);
    } else {
        const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[i + 4] = b[i]; }
    }
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&x)[8]) {
    if constexpr (sizeof(T) == 2) {
        Vec16 v;
        T* e = reinterpret_cast<T*>(&v);
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = from_f32<T>(x[i]);
        st16(p, v);
    } else {
        *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
    }
}
__device__ __forceinline__ void load8f(const float* p, float (&x)[8]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[i + 4] = b[i]; }
}

// STORE_A2T: also store w^T and k~^T (for a sweep that does not form them).
// Diagonal block m of A = (I + Akk)^-1 by forward substitution: column jj
// (one per lane) from the strictly lower part of Akk's block m (row pitch LCF).
template <int LCF>
__device__ __forceinline__ void diag_block_inverse(const float* akk, float* a, const int m, const int jj) {
    const int b0 = 16 * m;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        float acc = (r == jj) ? 1.f : 0.f;
#pragma unroll
        for (int s2 = 0; s2 < r; ++s2) acc -= akk[(b0 + r) * LCF + b0 + s2] * x[s2];
        x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) a[(b0 + r) * LCF + b0 + jj] = x[r];
}

// Two waves per SIMD: at C = 64 the one 8-wave workgroup a CU holds; at
// C = 32 two 4-wave workgroups per CU, which needs VGPRs + AGPRs <= 256.
template <typename T, int C, int D, bool SCALAR, bool STORE_A2T>
__global__ __launch_bounds__(128 * (C / 16)) __attribute__((amdgpu_waves_per_eu(2, 2))) void gdr_prep(Params p) {
    using L = PrepLds<T, C, D>;
    constexpr int NB = L::NB, NT = L::NT, LT = L::LT, LC = L::LC, LF = L::LF, LCF = L::LCF;
    constexpr int NTD = D / 16;  // column tiles of a [C][D] product
    constexpr int NTH = NTD / 2; // per wave: one column half
    __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
    float* Gs = reinterpret_cast<float*>(smem + L::G_OFF);
    float* At = reinterpret_cast<float*>(smem + L::X_OFF);    // phase 1-2: 2^g per token
    T* Xb = reinterpret_cast<T*>(smem + L::X_OFF);            // later phases
    T* qL = reinterpret_cast<T*>(smem + L::Q_OFF);
    T* kL = reinterpret_cast<T*>(smem + L::K_OFF);
    float* AqkF = reinterpret_cast<float*>(smem + L::AQK_OFF);
    float* AkkF = reinterpret_cast<float*>(smem + L::AKK_OFF);
    float* AF = reinterpret_cast<float*>(smem + L::AF_OFF);
    float* scr = reinterpret_cast<float*>(smem + L::SCR_OFF);
    float* flags = reinterpret_cast<float*>(smem + L::FLAG_OFF);
    float* bs = reinterpret_cast<float*>(smem + L::BETA_OFF);

    // Persistent: at most one workgroup per CU walks the (chunk, value head)
    // items blockIdx.x, + gridDim.x, ...; the next item's g, q, k, beta are
    // requested right after the current ones reach LDS, its v after the
    // current v is used (v stays in registers until its product).
    const int nit = p.seq_off[p.N] * p.H;
    int item = blockIdx.x;
    if (item >= nit) return;
    const int tid = threadIdx.x, w = wave_id();
    const T* q = static_cast<const T*>(p.q);
    const T* k = static_cast<const T*>(p.k);
    const T* v = static_cast<const T*>(p.v);
    const T* beta = static_cast<const T*>(p.beta);
    constexpr int V8 = 16 / sizeof(T);  // elements per 16-byte vector
    constexpr int NGP = C * (D / 4) / NT;    // 4-float gate pieces per thread
    constexpr int NQP = C * (D / V8) / NT;   // 16-byte q / k / v pieces per thread
    static_assert(NGP * NT == C * (D / 4) && NQP * NT == C * (D / V8), "piece split");
    f32x4 gpre[SCALAR ? 1 : NGP];   // per-channel gate pieces
    float gsc;                       // scalar gate: the gate of row (lane id)
    Vec16 qpre[NQP], kpre[NQP], vpre[NQP];
    float bpre;
    // rows past the sequence end read the last row (zeroed at use)
    auto load_in = [&](const int it, const ChunkEntry& e2) __attribute__((always_inline)) {
        const int hh = it % p.H, hkk = hh / p.G;
        if constexpr (SCALAR) {
            gsc = p.g[(size_t)(e2.tok0 + min(tid & 63, e2.len - 1)) * p.H + hh];
        } else {
#pragma unroll
            for (int i = 0; i < NGP; ++i) {
                const int e = tid + i * NT, r = e / (D / 4), d0 = (e % (D / 4)) * 4, rt = min(r, e2.len - 1);
                gpre[i] = *reinterpret_cast<const f32x4*>(p.g + ((size_t)(e2.tok0 + rt) * p.H + hh) * D + d0);
            }
        }
#pragma unroll
        for (int i = 0; i < NQP; ++i) {
            const int e = tid + i * NT, r = e / (D / V8), d0 = (e % (D / V8)) * V8, rt = min(r, e2.len - 1);
            qpre[i] = ld16(q + ((size_t)(e2.tok0 + rt) * p.Hg + hkk) * D + d0);
            kpre[i] = ld16(k + ((size_t)(e2.tok0 + rt) * p.Hg + hkk) * D + d0);
        }
        bpre = to_f32(beta[(size_t)(e2.tok0 + min(tid, e2.len - 1)) * p.H + hh]);
    };
    // v pieces as q and k: whole rows (16 lanes cover a 256-byte row)
    auto load_v = [&](const int it, const ChunkEntry& e2) __attribute__((always_inline)) {
        const int hh = it % p.H;
#pragma unroll
        for (int i = 0; i < NQP; ++i) {
            const int e = tid + i * NT, r = e / (D / V8), d0 = (e % (D / V8)) * V8, rt = min(r, e2.len - 1);
            vpre[i] = ld16(v + ((size_t)(e2.tok0 + rt) * p.H + hh) * D + d0);
        }
    };
    // The chunk entries are requested an item ahead of their use: a vector
    // load of the next item's entry at the top of an item would make its wait
    // (memory counters retire in order) also wait for all of the previous
    // item's output stores.
    ChunkEntry ce = p.ctab[item / p.H];
    ChunkEntry ce_n = p.ctab[min(item + (int)gridDim.x, nit - 1) / p.H];
    load_in(item, ce);
    load_v(item, ce);

    for (; item < nit; item += gridDim.x) {
    const int j = item / p.H, h = item % p.H;
    const int tok0 = ce.tok0, len = ce.len;
    const size_t jh = size_t(j) * p.H + h;
    const int nxt = min(item + (int)gridDim.x, nit - 1);   // past the end: a redundant valid load
    const ChunkEntry ce_nn = p.ctab[min(item + 2 * (int)gridDim.x, nit - 1) / p.H];
    // a fresh opaque thread index per item: thread-dependent address arithmetic
    // is recomputed in every item instead of being kept live across items
    const int tid = [] { int t = static_cast<int>(threadIdx.x); asm volatile("" : "+v"(t)); return t; }();
    const int l = tid & 63;
    __syncthreads();  // the previous item's LDS use is over

    // ---- phase 1: this item's inputs (already in registers) to LDS ----
    // A above its diagonal blocks stays zero; so does Aqk above its diagonal,
    // which the one-reference form writes itself (its operands overlay Aqk)
    for (int e = tid; e < C * LCF / 4; e += NT) {
        reinterpret_cast<f32x4*>(AF)[e] = zero4();
        if constexpr (!L::FAST) reinterpret_cast<f32x4*>(AqkF)[e] = zero4();
    }
    if constexpr (SCALAR) {
        // one gate per row: every wave scans the chunk's C gates across its
        // lanes (lane = row; rows past the end add 0, so they take G_last) and
        // writes its pieces of the cumsum G (and, for the per-block route, of
        // 2^g) broadcast over the columns
        static_assert(C <= 64, "one row per lane");
        const int ll = tid & 63;
        const float gr = ll < len ? gsc : 0.f;
        float G = gr;
#pragma unroll
        for (int off = 1; off < C; off <<= 1) {
            const float y = __shfl_up(G, off);
            G += ll >= off ? y : 0.f;
        }
#pragma unroll
        for (int i = 0; i < NGP; ++i) {
            const int e = tid + i * NT, r = e / (D / 4), d0 = (e % (D / 4)) * 4;
            const float Gv = __shfl(G, r);
            *reinterpret_cast<f32x4*>(Gs + r * LF + d0) = f32x4{Gv, Gv, Gv, Gv};
            if constexpr (!L::FAST) {   // only the per-block route reads 2^g
                const float ex = fast_exp2(__shfl(gr, r));
                *reinterpret_cast<f32x4*>(At + r * LF + d0) = f32x4{ex, ex, ex, ex};
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NGP; ++i) {
            const int e = tid + i * NT, r = e / (D / 4), d0 = (e % (D / 4)) * 4;
            const f32x4 gv = r < len ? gpre[i] : zero4();
            *reinterpret_cast<f32x4*>(Gs + r * LF + d0) = gv;
            *reinterpret_cast<f32x4*>(At + r * LF + d0) =
                f32x4{fast_exp2(gv[0]), fast_exp2(gv[1]), fast_exp2(gv[2]), fast_exp2(gv[3])};
        }
    }
#pragma unroll
    for (int i = 0; i < NQP; ++i) {
        const int e = tid + i * NT, r = e / (D / V8), d0 = (e % (D / V8)) * V8;
        st16(qL + r * LT + d0, r < len ? qpre[i] : Vec16{});
        st16(kL + r * LT + d0, r < len ? kpre[i] : Vec16{});
    }
    if (tid < C) bs[tid] = tid < len ? bpre : 0.f;
    if constexpr (!L::FAST) load_in(nxt, ce_n);  // the next item's g, q, k, beta
    __syncthreads();
    if constexpr (!SCALAR) {   // column cumsum in NSEG segments of SR rows: local scans, then segment offsets
        constexpr int NSEG = NT / D > 0 ? NT / D : 1, SR = C / NSEG;
        static_assert(NT % D == 0 || NT < D, "cumsum split");
        float* segtot = scr;  // [NSEG][D]
        const int d = tid % D, sg = tid / D;
        // the segment's SR values read at once and scanned in registers, kept
        // there for the offset pass
        float gv[SR];
        if (sg < NSEG) {
#pragma unroll
            for (int i = 0; i < SR; ++i) gv[i] = Gs[(sg * SR + i) * LF + d];
#pragma unroll
            for (int i = 1; i < SR; ++i) gv[i] += gv[i - 1];
            segtot[sg * D + d] = gv[SR - 1];
        }
        __syncthreads();
        float dev = 0.f;   // the largest |G_r - G_last / 2| of the thread's rows
        if (sg < NSEG) {
            float off = 0.f, tot = 0.f;   // all segment totals read (one wait), the earlier ones summed
#pragma unroll
            for (int s2 = 0; s2 < NSEG; ++s2) {
                const float x = segtot[s2 * D + d];
                off += s2 < sg ? x : 0.f;
                tot += x;
            }
#pragma unroll
            for (int i = 0; i < SR; ++i) {
                const float G = gv[i] + off;
                Gs[(sg * SR + i) * LF + d] = G;
                if constexpr (L::FAST) dev = fmaxf(dev, fabsf(G - 0.5f * tot));
            }
        }
        if constexpr (L::FAST) {
            dev = wave_max(dev);
            if ((tid & 63) == 0) flags[w] = dev;
        }
        __syncthreads();
    }
    // Whether every |G_r - G_last / 2| of the chunk is within the guard of the
    // MFMA form (a decaying column qualifies when its range -G_last is at most
    // twice the guard): then all of Aqk and Akk are formed through that one
    // reference per column; else through the block boundaries and the
    // diagonal blocks' own rows, as below.
    bool fast = false;
    if constexpr (L::FAST && SCALAR) {
        fast = true;   // plain q k^T and k k^T times the decay: no operand scaling, no guard
    } else if constexpr (L::FAST) {
        constexpr float guard = __is_same(T, _Float16) ? 8.f : 64.f;
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < L::NW; ++i) m = fmaxf(m, flags[i]);
        fast = m <= guard;
    }

    // 4a (of the inverse below): the diagonal blocks of A = (I + Akk)^-1. The
    // per-boundary path runs them for all blocks in the last wave (lanes
    // 0..C-1) during its first product round, where that wave has no tile;
    // the one-reference path in the waves that form Akk's diagonal blocks.
    // (written out here rather than through diag_block_inverse: at C = 32 the
    // call form raised the kernel's registers past two waves per SIMD)
    auto diag_inverse = [&](const int lane) __attribute__((always_inline)) {
        if (lane < C) {
            const int m = lane >> 4, jj = lane & 15, b0 = 16 * m;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = (r == jj) ? 1.f : 0.f;
#pragma unroll
                for (int s2 = 0; s2 < r; ++s2) acc -= AkkF[(b0 + r) * LCF + b0 + s2] * x[s2];
                x[r] = acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) AF[(b0 + r) * LCF + b0 + jj] = x[r];
        }
    };

    if (fast) {
        // ---- phases 2-3, one reference per column: every element of Aqk and
        //      Akk on MFMA from q 2^(G - G_m), k 2^(G - G_m) and k 2^(G_m - G)
        //      with G_m = G_last / 2 (the reference cancels in each channel's
        //      term q_r,d k_s,d 2^(G_r,d - G_s,d)). The exponents G_r - G_m
        //      take either sign; the check above bounds them by the guard, so
        //      the scaled operands stay finite and normal in T, as in the
        //      diagonal-block form below, here for the whole chunk at once.
        //      Each term is still one product of two rounded operands.
        //      Scalar gate: the products take q and k as loaded, and the
        //      decay multiplies each element as it is written. ----
        T* xq = reinterpret_cast<T*>(smem + L::X_OFF);   // [C][LT] each
        T* xkq = xq + C * LT;
        T* xk = xkq + C * LT;
        if constexpr (!SCALAR) {   // all LDS reads of the thread's pieces first (one wait), then the writes
            constexpr int NP = C * (D / 8) / NT;
            static_assert(NP * NT == C * (D / 8), "piece split");
            static_assert(NT % (D / 8) == 0, "a thread's pieces share their columns");
            struct Raw8 { T v[8]; };   // 8 elements as stored
            float gv[NP][8], gl[8];
            Raw8 qr[NP], kr[NP];
            load8f(Gs + (C - 1) * LF + (tid % (D / 8)) * 8, gl);
#pragma unroll
            for (int it = 0; it < NP; ++it) {
                const int e = tid + it * NT, r = e / (D / 8), d0 = (e % (D / 8)) * 8;
                load8f(Gs + r * LF + d0, gv[it]);
                qr[it] = *reinterpret_cast<const Raw8*>(qL + r * LT + d0);
                kr[it] = *reinterpret_cast<const Raw8*>(kL + r * LT + d0);
            }
#pragma unroll
            for (int it = 0; it < NP; ++it) {
                const int e = tid + it * NT, r = e / (D / 8), d0 = (e % (D / 8)) * 8;
                float a[8], b[8], c[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float x = gv[it][i] - 0.5f * gl[i];
                    const float ex = fast_exp2(x), exi = fast_exp2(-x);
                    const float qv = to_f32(qr[it].v[i]), kv = to_f32(kr[it].v[i]);
                    a[i] = qv * ex;
                    b[i] = kv * ex;
                    c[i] = kv * exi;
                }
                store8<T>(xq + r * LT + d0, a);
                store8<T>(xkq + r * LT + d0, b);
                store8<T>(xk + r * LT + d0, c);
            }
            __syncthreads();
        }
        // the lower 16 x 16 tiles of Aqk (t < NLT) and Akk (t >= NLT), tile t
        // on wave t % NW; the tile loops are unrolled, so that each copy's
        // block indices and masks are constants and only the wave's own copies run
        constexpr int NLT = NB * (NB + 1) / 2, NTI = 2 * NLT, TPW = (NTI + L::NW - 1) / L::NW;
        auto tile_ij = [](int tt, int& bi, int& bj) {   // row-major order of the lower triangle
            bi = 0;
            while ((bi + 1) * (bi + 2) / 2 <= tt) ++bi;
            bj = tt - bi * (bi + 1) / 2;
        };
        f32x4 accT[TPW];
#pragma unroll
        for (int i = 0; i < TPW; ++i) accT[i] = zero4();
#pragma unroll
        for (int t = 0; t < NTI; ++t) {
            if (t % L::NW != w) continue;
            int bi, bj;
            tile_ij(t % NLT, bi, bj);
            f32x4 a1[1] = {zero4()};
            if constexpr (SCALAR) panel_mma<T, 1, D>(a1, t >= NLT ? kL : qL, LT, 16 * bi, kL, LT, 16 * bj, l);
            else panel_mma<T, 1, D>(a1, t >= NLT ? xkq : xq, LT, 16 * bi, xk, LT, 16 * bj, l);
            accT[t / L::NW] = a1[0];
        }
        __syncthreads();   // the operand reads are done: Aqk and Akk overlay them
        int mydiag = -1;   // the Akk diagonal block this wave formed, if any
#pragma unroll
        for (int t = 0; t < NTI; ++t) {
            if (t % L::NW != w) continue;
            const bool kk = t >= NLT;
            int bi, bj;
            tile_ij(t % NLT, bi, bj);
            float bsv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) bsv[e] = kk ? bs[16 * bi + acc_row(e, l)] : 1.f;
            float dec[4] = {1.f, 1.f, 1.f, 1.f};
            if constexpr (SCALAR) {   // G is stored broadcast over the columns
                const float gs = Gs[(16 * bj + acc_col(l)) * LF];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * bi + acc_row(e, l), s2 = 16 * bj + acc_col(l);
                    dec[e] = s2 <= r ? fast_exp2(Gs[r * LF] - gs) : 0.f;
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * bi + acc_row(e, l), s2 = 16 * bj + acc_col(l);
                const float v = accT[t / L::NW][e] * dec[e];
                if (kk) AkkF[r * LCF + s2] = s2 < r ? bsv[e] * v : 0.f;
                else AqkF[r * LCF + s2] = s2 <= r ? v : 0.f;
            }
            if (kk && bi == bj) mydiag = bi;
        }
        if (mydiag >= 0) {   // its inverse, from the wave's own writes
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
            __builtin_amdgcn_wave_barrier();
            if (l < 16) diag_block_inverse<LCF>(AkkF, AF, mydiag, l);
        }
        // the next item's g, q, k, beta: with the one-reference form compiled
        // in, requested here (after its operand and product registers are
        // free, before the inverse, while the memory pipeline is idle) rather
        // than in phase 1, where they would spill at C = 64; or at the
        // matching point of the per-boundary path
        if constexpr (L::FAST) load_in(nxt, ce_n);
        // the tiles of Aqk above the diagonal are zero
        for (int t = w; t < NB * (NB - 1) / 2; t += L::NW) {
            int bi, bj;
            tile_ij(t, bi, bj);   // (bi, bj) of the strict lower triangle, shifted: (bj, bi + 1)
            const int ti = bj, tj = bi + 1;
#pragma unroll
            for (int e = 0; e < 4; ++e) AqkF[(16 * ti + acc_row(e, l)) * LCF + 16 * tj + acc_col(l)] = 0.f;
        }
        __syncthreads();
    } else {
    // Aqk above its diagonal is zero (no thread of phases 2-3 writes there;
    // below it and on it they write every element, as they do in Akk's
    // strictly lower part, the only part of Akk that is read)
    if constexpr (L::FAST) {
        for (int e = tid; e < C * C; e += NT) {
            const int r = e / C, s2 = e % C;
            if (s2 > r) AqkF[r * LCF + s2] = 0.f;
        }
    }
    // ---- phase 2: diagonal 16x16 blocks; wave w -> block w % NB, Aqk (w < NB) or Akk ----
    const bool is_kk = w >= NB;
    bool diag_mfma;
    {
        // MFMA form: lane l builds the fragments of its own row b0 + l%16 and
        // d-range (the A and B operands share the lane -> (row, d) map)
        using F = typename Mfma<T>::frag;
        constexpr int KL = Mfma<T>::KL, KS = 4 * KL;
        constexpr float guard = __is_same(T, _Float16) ? 8.f : 64.f;
        const int b0 = 16 * (w % NB), r = b0 + (l & 15);
        f32x4 acc = zero4();
        float rmax = 0.f;
#pragma unroll 2
        for (int k0 = 0; k0 < D; k0 += KS) {
            const int d0 = k0 + (l >> 4) * KL;
            F fa, fi;
            const T* arow = (is_kk ? kL : qL) + r * LT;
            // the lane's KL consecutive elements of each row, one vector read per row
            float gq[KL], gb[KL];
            T ar[KL], kr[KL];
            if constexpr (KL == 4) {
                const f32x4 g4 = *reinterpret_cast<const f32x4*>(Gs + r * LF + d0);
                const f32x4 b4 = *reinterpret_cast<const f32x4*>(Gs + b0 * LF + d0);
                const uint2 a2 = *reinterpret_cast<const uint2*>(arow + d0);
                const uint2 k2 = *reinterpret_cast<const uint2*>(kL + r * LT + d0);
#pragma unroll
                for (int i = 0; i < 4; ++i) { gq[i] = g4[i]; gb[i] = b4[i]; }
                __builtin_memcpy(ar, &a2, sizeof(a2));
                __builtin_memcpy(kr, &k2, sizeof(k2));
            } else {
#pragma unroll
                for (int i = 0; i < KL; ++i) {
                    gq[i] = Gs[r * LF + d0 + i]; gb[i] = Gs[b0 * LF + d0 + i];
                    ar[i] = arow[d0 + i]; kr[i] = kL[r * LT + d0 + i];
                }
            }
#pragma unroll
            for (int i = 0; i < KL; ++i) {
                const float x = gq[i] - gb[i];
                rmax = fmaxf(rmax, fabsf(x));
                const float e = fast_exp2(x), ei = fast_exp2(fminf(-x, guard));
                const float av = to_f32(ar[i]), kv = to_f32(kr[i]);
                if constexpr (KL == 1) {
                    fa = av * e; fi = kv * ei;
                } else {
                    fa[i] = from_f32<T>(av * e); fi[i] = from_f32<T>(kv * ei);
                }
            }
            acc = Mfma<T>::mma(fa, fi, acc);
        }
        diag_mfma = wave_max(rmax) <= guard;
        if (diag_mfma) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = b0 + acc_row(i, l), s2 = b0 + acc_col(l);
                if (!is_kk && s2 <= rr) AqkF[rr * LCF + s2] = acc[i];
                if (is_kk && s2 < rr) AkkF[rr * LCF + s2] = bs[rr] * acc[i];
            }
        }
    }
    // per-element form (gate range beyond the bound; both waves of the block
    // compute, each keeps its matrix): lane -> (mirror row pair pr, d-part
    // e8) of the wave's block; the pair (16m+pr, 16m+15-pr)
    // gives every lane 17 (r, s) steps. Partial dot products over the d-part
    // are summed across the 8 parts with xor shuffles.
    if (!diag_mfma) {
        constexpr int PW = D / 8;
        static_assert(PW % 8 == 0, "d-part of whole 8-element vectors");
        const int m = w % NB, pr = (tid & 63) >> 3, e8 = tid & 7, d0 = e8 * PW;
        float qr[PW], kr[PW], E[PW];
        int r = 16 * m + pr, s = r;
        auto load_row = [&](int rr) {
#pragma unroll
            for (int i0 = 0; i0 < PW; i0 += 8) {
                float x[8], y[8];
                load8<T>(qL + rr * LT + d0 + i0, x);
                load8<T>(kL + rr * LT + d0 + i0, y);
#pragma unroll
                for (int i = 0; i < 8; ++i) { qr[i0 + i] = x[i]; kr[i0 + i] = y[i]; E[i0 + i] = 1.f; }
            }
        };
        load_row(r);
        for (int it = 0; it < 17; ++it) {
            if (it == pr + 1) {  // switch to the mirror row
                r = 16 * m + 15 - pr;
                s = r;
                load_row(r);
            }
            float pq = 0.f, pk = 0.f;
#pragma unroll
            for (int i0 = 0; i0 < PW; i0 += 8) {
                float ks[8], as[8];
                load8<T>(kL + s * LT + d0 + i0, ks);
                load8f(At + s * LF + d0 + i0, as);
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float t = ks[i] * E[i0 + i];
                    pq += qr[i0 + i] * t;
                    pk += kr[i0 + i] * t;
                    E[i0 + i] *= as[i];   // E(r, s-1) = E(r, s) * 2^g_s
                }
            }
            pq = row8_sum(pq);   // the 8 d-parts are 8 consecutive lanes
            pk = row8_sum(pk);
            if (e8 == 0) {
                if (!is_kk) AqkF[r * LCF + s] = pq;
                else if (s < r) AkkF[r * LCF + s] = bs[r] * pk;
            }
            --s;
        }
    }
    __syncthreads();

    // ---- phase 3: off-diagonal blocks through the boundary rho = 16 i (MFMA) ----
    // For boundary i: q_r 2^(G_r - G_rho) and k_r 2^(G_r - G_rho) of block i,
    // k_s 2^(G_rho - G_s) of the rows s < rho, then the block products. Two
    // boundaries share a pass (one fill, one product round, two barriers) when
    // their rows fit the X region together.
    {
        constexpr int XROWS = int(L::X_BYTES / (size_t(LT) * sizeof(T)));
        constexpr bool PAIR = NB == 4 && (32 + 16) + (32 + 32) <= XROWS;
        auto pass = [&](auto nib_c, const int ib0, const bool first) __attribute__((always_inline)) {
            constexpr int NIB = decltype(nib_c)::value;
            // rows of boundary ib0 + j start at base(j) in the X region
            auto base = [&](int j) { return j == 0 ? 0 : 32 + 16 * ib0; };
            const int rows = base(NIB - 1) + 32 + 16 * (ib0 + NIB - 1);
            const int np = rows * (D / 8);
            constexpr int MAXROWS = NIB == 2 ? (32 + 16) + (32 + 32) : 32 + 16 * (NB - 1);
            constexpr int NFP = (MAXROWS * (D / 8) + NT - 1) / NT;
            struct Raw8 { T v[8]; };   // 8 elements as stored (16 or 32 bytes)
            float grv[NFP][8], gx[NFP][8];
            Raw8 xr[NFP];
            // every LDS read of the thread's pieces first (one wait); spare
            // pieces read a valid duplicate and store nothing
#pragma unroll
            for (int it = 0; it < NFP; ++it) {
                const int e = min(tid + it * NT, np - 1), g = e / (D / 8), d0 = (e % (D / 8)) * 8;
                const int j = NIB == 2 && g >= base(1) ? 1 : 0, rr = g - base(j), rho = 16 * (ib0 + j);
                const int r = rr < 32 ? rho + (rr & 15) : rr - 32;
                load8f(Gs + rho * LF + d0, grv[it]);
                load8f(Gs + r * LF + d0, gx[it]);
                xr[it] = *reinterpret_cast<const Raw8*>((rr < 16 ? qL : kL) + r * LT + d0);
            }
#pragma unroll
            for (int it = 0; it < NFP; ++it) {
                const int e = tid + it * NT, g = e / (D / 8), d0 = (e % (D / 8)) * 8;
                const int j = NIB == 2 && g >= base(1) ? 1 : 0, rr = g - base(j);
                if (e < np) {
                    float x[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i)   // exponents <= 0 on both sides of the boundary
                        x[i] = to_f32(xr[it].v[i]) *
                               fast_exp2(rr < 32 ? gx[it][i] - grv[it][i] : grv[it][i] - gx[it][i]);
                    store8<T>(Xb + g * LT + d0, x);
                }
            }
            __syncthreads();
            // tiles: per boundary ib, (which in {Aqk, Akk}) x (ib column tiles)
            const int ntile = NIB == 2 ? 2 * ib0 + 2 * (ib0 + 1) : 2 * ib0;
            for (int t = w; t < ntile; t += L::NW) {
                const int j = NIB == 2 && t >= 2 * ib0 ? 1 : 0, tt = t - (j ? 2 * ib0 : 0), ib = ib0 + j;
                const int which = tt / ib, ct = tt % ib, rho = 16 * ib;
                const T* qb = Xb + base(j) * LT;   // [16][LT]  q_r 2^(G_r - G_rho), r in block ib
                const T* kqb = qb + 16 * LT;       // [16][LT]  k_r 2^(G_r - G_rho)
                const T* kb = qb + 32 * LT;        // [rho][LT] k_s 2^(G_rho - G_s), s < rho
                f32x4 acc[1] = {zero4()};
                panel_mma<T, 1, D>(acc, which ? kqb : qb, LT, 0, kb, LT, 16 * ct, l);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = rho + acc_row(i, l), s2 = 16 * ct + acc_col(l);
                    if (which) AkkF[r * LCF + s2] = bs[r] * acc[0][i];
                    else AqkF[r * LCF + s2] = acc[0][i];
                }
            }
            if (first && w == L::NW - 1) diag_inverse(tid - (NT - 64));
            __syncthreads();
        };
        // the last wave has no tile in the first product round (at most
        // 2 + 4 tiles there), which is where it inverts the diagonal blocks
        static_assert(L::NW - 1 >= (PAIR ? 6 : 2), "a free wave in the first product round");
        if constexpr (PAIR) {
            pass(std::integral_constant<int, 2>{}, 1, true);
            pass(std::integral_constant<int, 1>{}, 3, false);
        } else {
            for (int ib = 1; ib < NB; ++ib) pass(std::integral_constant<int, 1>{}, ib, ib == 1);
        }
    }
    if constexpr (L::FAST) load_in(nxt, ce_n);
    }   // per-boundary path

    // k~ = k 2^(G_last - G) in fragment order, by NTK threads from t0 (16-bit:
    // row fastest, so the fragment-order stores are contiguous); ktS: also the
    // k~ rows staged in LDS (for k~^T), or null
    auto kt_out = [&](auto ntk_c, const int t0, T* ktS) __attribute__((always_inline)) {
        constexpr int NTK = decltype(ntk_c)::value;
        T* gkt = static_cast<T*>(p.kt) + jh * C * D;
        static_assert(C * (D / 8) % NTK == 0, "piece split");
#pragma unroll
        for (int it = 0; it < C * (D / 8) / NTK; ++it) {
            const int e = t0 + it * NTK;
            const int r = sizeof(T) == 2 ? e % C : e / (D / 8);
            const int d0 = sizeof(T) == 2 ? (e / C) * 8 : (e % (D / 8)) * 8;
            float x[8], gl[8], g[8];
            load8<T>(kL + r * LT + d0, x);
            load8f(Gs + (C - 1) * LF + d0, gl);
            load8f(Gs + r * LF + d0, g);
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] *= fast_exp2(gl[i] - g[i]);
            store8<T>(gkt + fo_index<T, D>(r, d0), x);
            if (ktS) store8<T>(ktS + r * LT + d0, x);
        }
    };
    // At C = 64 without the k~^T store, waves 4..7 write k~ while waves 0..3
    // form the lower-left blocks of the inverse (phase 4b, level 2)
    constexpr bool EARLY_KT = NB == 4 && !STORE_A2T;

    // ---- phase 4: A = (I + Akk)^-1 (4a, the diagonal blocks, ran in phases 2-3) ----
    // 4b: the blocks below the diagonal (fp32 MFMA), A_ij = -A_ii P_ij with
    // P_ij = sum_{kb=j}^{i-1} L_i,kb A_kb,j. At C = 64 in two levels (below);
    // at C = 32 one block, by wave 0. Each wave orders only its own LDS writes
    // (a wave-level fence) until a workgroup barrier.
    auto wave_fence = [] {
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
    };
    if constexpr (NB == 4) {
        // Two levels instead of one walk per block column (whose first column
        // chains three dependent steps): with P = L A (a 16 x 16 block product
        // through the scratch tile) and A_ij = -A_ii P,
        //   level 1: A10 = -A11 L10 A00 (wave 0), A32 = -A33 L32 A22 (wave 1);
        //   level 2: the lower left 32 x 32 block, -A_bot (L_bl A_top):
        //     A20 = -A22 (L20 A00 + L21 A10), A21 = -A22 L21 A11,
        //     A30 = -(A32 (L20 A00 + L21 A10) + A33 (L30 A00 + L31 A10)),
        //     A31 = -(A32 L21 A11 + A33 L31 A11), waves 0..3, each forming
        //     the products it needs itself (waves 2, 3 keep their second
        //     tile in Akk's diagonal blocks 0, 1, which 4a has finished with).
        auto prod = [&](const int ai, const int aj, const int kd, const float* B, const int ldb, const int bk0,
                        const int bj0) __attribute__((always_inline)) {
            f32x4 acc = zero4();
            return tile_f32(acc, AkkF, LCF, ai, aj, B, ldb, bk0, bj0, kd, l);
        };
        auto put = [&](float* dst, const int ld, const f32x4 acc) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[acc_row(i, l) * ld + acc_col(l)] = acc[i];
        };
        float* sc = scr + w * 16 * 20;
        if (w < 2) {   // level 1
            const int b = 2 * w;   // A_{b+1,b}
            put(sc, 20, prod(16 * (b + 1), 16 * b, 16, AF, LCF, 16 * b, 16 * b));
            wave_fence();
            f32x4 acc = zero4();
            acc = tile_f32(acc, AF, LCF, 16 * (b + 1), 16 * (b + 1), sc, 20, 0, 0, 16, l);
#pragma unroll
            for (int i = 0; i < 4; ++i) AF[(16 * (b + 1) + acc_row(i, l)) * LCF + 16 * b + acc_col(l)] = -acc[i];
        }
        __syncthreads();
        if (w < 4) {   // level 2: wave w forms A_{2 + w / 2, w % 2}
            const int jc = w & 1, ir = 2 + (w >> 1);
            // Y_{2, jc} = L_{2, jc..1} A_{jc..1, jc} (K = 32 - 16 jc)
            put(sc, 20, prod(32, 16 * jc, 32 - 16 * jc, AF, LCF, 16 * jc, 16 * jc));
            float* sc2 = AkkF + (16 * jc) * LCF + 16 * jc;   // Akk's diagonal block jc
            if (ir == 3) put(sc2, LCF, prod(48, 16 * jc, 32 - 16 * jc, AF, LCF, 16 * jc, 16 * jc));   // Y_{3, jc}
            wave_fence();
            f32x4 acc = zero4();
            // A_{2, jc} = -A22 Y_2jc; A_{3, jc} = -(A32 Y_2jc + A33 Y_3jc)
            acc = tile_f32(acc, AF, LCF, 16 * ir, 32, sc, 20, 0, 0, 16, l);
            if (ir == 3) acc = tile_f32(acc, AF, LCF, 48, 48, sc2, LCF, 0, 0, 16, l);
#pragma unroll
            for (int i = 0; i < 4; ++i) AF[(16 * ir + acc_row(i, l)) * LCF + 16 * jc + acc_col(l)] = -acc[i];
        } else if constexpr (EARLY_KT) {
            kt_out(std::integral_constant<int, NT / 2>{}, tid - NT / 2, nullptr);
        }
    } else {
    if (w < NB - 1) {
        const int bj = w;
        float* sc = scr + w * 16 * 20;
        for (int bi = bj + 1; bi < NB; ++bi) {
            f32x4 acc = zero4();
            acc = tile_f32(acc, AkkF, LCF, 16 * bi, 16 * bj, AF, LCF, 16 * bj, 16 * bj, 16 * (bi - bj), l);
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[acc_row(i, l) * 20 + acc_col(l)] = acc[i];
            wave_fence();   // sc written by all lanes before any lane reads it
            acc = zero4();
            acc = tile_f32(acc, AF, LCF, 16 * bi, 16 * bi, sc, 20, 0, 0, 16, l);
#pragma unroll
            for (int i = 0; i < 4; ++i) AF[(16 * bi + acc_row(i, l)) * LCF + 16 * bj + acc_col(l)] = -acc[i];
            wave_fence();   // A_ij and the sc reads done before the next row reuses them
        }
    }
    }
    __syncthreads();

    // ---- phase 5: A and scale Aqk^T to the workspace in 8-element row
    //      pieces (the gradient kernel takes A^T from its LDS copy of A through
    //      transposed loads); A and Aqk in place as MFMA operands in LDS ----
    float av[8], qv[8];   // this thread's piece of A and Aqk (at most one: C <= 64)
    static_assert(C * (C / 8) <= NT, "one piece of a C x C matrix per thread");
    const bool has_piece = tid < C * (C / 8);
    const int pr5 = tid % C, ps5 = (tid / C) * 8;   // row fastest: transposed reads conflict-free
    if (has_piece) {
        T* gA = static_cast<T*>(p.Am) + jh * C * C;
        T* gSq = static_cast<T*>(p.sAqkT) + jh * C * C;
        float sq[8];
        load8f(AF + pr5 * LCF + ps5, av);
        load8f(AqkF + pr5 * LCF + ps5, qv);
#pragma unroll
        for (int i = 0; i < 8; ++i) sq[i] = p.scale * AqkF[(ps5 + i) * LCF + pr5];
        store8<T>(gA + fo_index<T, C>(pr5, ps5), av);
        store8<T>(gSq + fo_index<T, C>(pr5, ps5), sq);
    }
    __syncthreads();
    T* AtL = reinterpret_cast<T*>(smem + L::AF_OFF);    // A   [C][LC], over the dead fp32 A
    T* AqkL = reinterpret_cast<T*>(smem + L::AQK_OFF);  // Aqk [C][LC], over the dead fp32 Aqk
    if (has_piece) {
        store8<T>(AtL + pr5 * LC + ps5, av);
        store8<T>(AqkL + pr5 * LC + ps5, qv);
    }
    // k^[s][d] = beta_s k_sd 2^G_sd, row-major (the B operand of w = A k^,
    // read through transposed loads): 16-byte row pieces
    T* kh = Xb;  // [C][LT]
    {   // all LDS reads of the thread's pieces first (one wait), then the writes
        constexpr int NP = C * (D / 8) / NT;
        static_assert(NP * NT == C * (D / 8), "piece split");
        float x[NP][8];
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int e = tid + it * NT, s0 = e / (D / 8), d0 = (e % (D / 8)) * 8;
            float kv[8], gv[8];
            load8<T>(kL + s0 * LT + d0, kv);
            load8f(Gs + s0 * LF + d0, gv);
            const float b = bs[s0];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[it][i] = b * kv[i] * fast_exp2(gv[i]);
        }
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int e = tid + it * NT, s0 = e / (D / 8), d0 = (e % (D / 8)) * 8;
            store8<T>(kh + s0 * LT + d0, x[it]);
        }
    }
    __syncthreads();

    // ---- phase 6: w = A k^ (wave w owns rows 16 (w % NB) .. +16 and the
    //      column half w / NB of every [C][D] product) ----
    const int r0 = 16 * (w % NB), ch0 = (w / NB) * (D / 2);
    f32x4 acc[NTH];
#pragma unroll
    for (int t = 0; t < NTH; ++t) acc[t] = zero4();
    panel_mma<T, NTH, C, false, true>(acc, AtL, LC, r0, kh, LT, ch0, l);
    __syncthreads();  // k^ is about to be overwritten by w^T
    T* wTL = Xb;  // [D][LC]
#pragma unroll
    for (int t = 0; t < NTH; ++t) {
        const int c = ch0 + 16 * t + acc_col(l), rb = r0 + acc_row(0, l);
        store4<T>(wTL + c * LC + rb, acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    }
    __syncthreads();
    {   // w^T rows out (16-byte pieces; not needed where the sweep transposes
        // w itself), w out through transposing LDS reads
        T* gw = static_cast<T*>(p.w) + jh * C * D;
        T* gwT = static_cast<T*>(p.wT) + jh * D * C;
        // constant trip counts: unrolled, the LDS reads go out ahead of the stores
        static_assert(D * (C / 8) % NT == 0, "piece split");
        if constexpr (STORE_A2T) {
#pragma unroll
            for (int it = 0; it < D * (C / 8) / NT; ++it) {
                const int e = tid + it * NT, d = e / (C / 8), s0 = (e % (C / 8)) * 8;
                float x[8];
                load8<T>(wTL + d * LC + s0, x);
                store8<T>(gwT + fo_index<T, C>(d, s0), x);
            }
        }
        if constexpr (sizeof(T) == 2) {
            // w in 16 x 32 fragment-order tiles: per tile two transposed loads
            // give lane l row 16 rt + l % 16 at columns 32 dt + 8 (l / 16) + 0..7,
            // exactly its 16-byte piece of the tile's contiguous 1 KB
            constexpr int NTL = (C / 16) * (D / 32) / L::NW;
            static_assert(NTL * L::NW == (C / 16) * (D / 32), "tiles per wave");
#pragma unroll
            for (int it = 0; it < NTL; ++it) {
                const int tl = w + L::NW * it, rt = tl / (D / 32), dt = tl % (D / 32);
                const uint64_t a = ks_tr4_bits(wTL, LC, 16 * rt, 32 * dt, 8, l), b = ks_tr4_bits(wTL, LC, 16 * rt, 32 * dt + 4, 8, l);
                const Vec16 v = {{uint32_t(a), uint32_t(a >> 32), uint32_t(b), uint32_t(b >> 32)}};
                st16(gw + fo_index<T, D>(16 * rt + (l & 15), 32 * dt + 8 * (l >> 4)), v);
            }
        } else {
#pragma unroll
            for (int it = 0; it < C * (D / 8) / NT; ++it) {
                const int e = tid + it * NT, r = e % C, d0 = (e / C) * 8;   // r fastest: the transposed reads conflict-free
                float x[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = to_f32(wTL[(d0 + i) * LC + r]);
                store8<T>(gw + fo_index<T, D>(r, d0), x);
            }
        }
    }

    // ---- phase 7: q~ = q 2^G - Aqk w, stored as scale * q~^T ----
#pragma unroll
    for (int t = 0; t < NTH; ++t) acc[t] = zero4();
    panel_mma<T, NTH, C>(acc, AqkL, LC, r0, wTL, LC, ch0, l);
    {
        T* gq = static_cast<T*>(p.qsT) + jh * D * C;
#pragma unroll
        for (int t = 0; t < NTH; ++t) {
            const int c = ch0 + 16 * t + acc_col(l), rb = r0 + acc_row(0, l);
            float qv4[4], o[4];
            if constexpr (sizeof(T) == 2) {   // the lane's 4 rows of column c: one transposed load
                const uint64_t u = ks_tr4_bits(qL, LT, ch0 + 16 * t, r0, 4, l);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    qv4[i] = to_f32(__builtin_bit_cast(T, static_cast<unsigned short>(u >> (16 * i))));
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) qv4[i] = to_f32(qL[(rb + i) * LT + c]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = rb + i;
                o[i] = p.scale * (qv4[i] * fast_exp2(Gs[r * LF + c]) - acc[t][i]);
            }
            store4<T>(gq + fo_index<T, C>(c, rb), o[0], o[1], o[2], o[3]);
        }
    }
    __syncthreads();  // Xb (w^T) -> v^T

    // ---- phase 8: u = A (beta v) ----
    T* vh = Xb;  // [C][LT] beta v, rows as loaded (the product reads them through transposed loads)
#pragma unroll
    for (int i5 = 0; i5 < NQP; ++i5) {
        const int e = tid + i5 * NT, s2 = e / (D / V8), d0 = (e % (D / V8)) * V8;   // as loaded
        const Vec16 vv = s2 < len ? vpre[i5] : Vec16{};
        const T* vp = reinterpret_cast<const T*>(&vv);
        Vec16 o;
        T* op = reinterpret_cast<T*>(&o);
#pragma unroll
        for (int i = 0; i < V8; ++i) op[i] = from_f32<T>(bs[s2] * to_f32(vp[i]));
        st16(vh + s2 * LT + d0, o);
    }
    load_v(nxt, ce_n);  // the next item's v
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NTH; ++t) acc[t] = zero4();
    panel_mma<T, NTH, C, false, true>(acc, AtL, LC, r0, vh, LT, ch0, l);
    {
        T* gu = static_cast<T*>(p.uT) + jh * D * C;
#pragma unroll
        for (int t = 0; t < NTH; ++t) {
            const int c = ch0 + 16 * t + acc_col(l), rb = r0 + acc_row(0, l);
            store4<T>(gu + ao_index<C>(c, rb), acc[t][0], acc[t][1], acc[t][2], acc[t][3]);   // accumulator order
        }
    }

    // ---- phase 9: k~ = k 2^(G_last - G) (fragment order, and transposed where
    //      the sweep does not transpose it itself; written in phase 4b instead
    //      where EARLY_KT), 2^G_last ----
    {
        T* gktT = static_cast<T*>(p.ktT) + jh * D * C;
        // 16-bit: k~ rows also staged over the dead Aqk / Akk (for k~^T below)
        T* ktS = reinterpret_cast<T*>(smem + L::AQK_OFF);
        static_assert(size_t(C) * LT * sizeof(T) <= 2 * size_t(C) * LCF * 4, "k~ staging fits over Aqk, Akk");
        if constexpr (!EARLY_KT)
            kt_out(std::integral_constant<int, NT>{}, tid, sizeof(T) == 2 && STORE_A2T ? ktS : nullptr);
        if constexpr (!STORE_A2T) {
            // k~^T is formed by the sweep
        } else if constexpr (sizeof(T) == 2) {
            // k~^T in 16 x 32 fragment-order tiles from the staged k~ rows: two
            // transposed loads give lane l row d = 16 dt + l % 16 at columns
            // 32 rt + 8 (l / 16) + 0..7, its 16-byte piece of the tile
            __syncthreads();
            constexpr int NTL = (D / 16) * (C / 32) / L::NW;
            static_assert(NTL * L::NW == (D / 16) * (C / 32), "tiles per wave");
#pragma unroll
            for (int it = 0; it < NTL; ++it) {
                const int tl = w + L::NW * it, dt = tl / (C / 32), rt = tl % (C / 32);
                const uint64_t a = ks_tr4_bits(ktS, LT, 16 * dt, 32 * rt, 8, l), b = ks_tr4_bits(ktS, LT, 16 * dt, 32 * rt + 4, 8, l);
                const Vec16 v = {{uint32_t(a), uint32_t(a >> 32), uint32_t(b), uint32_t(b >> 32)}};
                st16(gktT + fo_index<T, C>(16 * dt + (l & 15), 32 * rt + 8 * (l >> 4)), v);
            }
        } else {
#pragma unroll
            for (int it = 0; it < D * (C / 8) / NT; ++it) {
                const int e = tid + it * NT, d = e % D, r0b = (e / D) * 8;   // d fastest (bank-conflict free)
                const float gl = Gs[(C - 1) * LF + d];
                float x[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    x[i] = to_f32(kL[(r0b + i) * LT + d]) * fast_exp2(gl - Gs[(r0b + i) * LF + d]);
                store8<T>(gktT + fo_index<T, C>(d, r0b), x);
            }
        }
        for (int d = tid; d < D; d += NT) p.glast[jh * D + d] = fast_exp2(Gs[(C - 1) * LF + d]);
    }
    ce = ce_n;
    ce_n = ce_nn;
    }
}

}  // namespace gdr
