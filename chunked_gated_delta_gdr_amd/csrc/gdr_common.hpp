// gdr_common.hpp -- device building blocks shared by the gfx950 kernels of the
// chunkwise gated delta-rule backward: MFMA traits for the three operand types,
// fragment loads from LDS/global, fp32 <-> io conversions and the kernel
// parameter block.
//
// MFMA lane layouts (gfx950, wave64), checked on the device:
//   v_mfma_f32_16x16x32_{bf16,f16}: lane l holds A[l%16][8*(l/16) + 0..7] and
//     B[8*(l/16) + 0..7][l%16]; the f32x4 result holds D[4*(l/16) + 0..3][l%16].
//   v_mfma_f32_16x16x4_f32: A[l%16][l/16], B[l/16][l%16]; D as above.
// Both are "16 rows x 16 cols, reduction in steps of 4*KL" with KL = 8 or 1.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;

template <typename T> struct Mfma;

template <> struct Mfma<__bf16> {
    static constexpr int KL = 8;
    using frag = bf16x8;
    using quad = bf16x4;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<_Float16> {
    static constexpr int KL = 8;
    using frag = f16x8;
    using quad = f16x4;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<float> {
    static constexpr int KL = 1;
    using frag = float;
    using quad = f32x4;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

template <typename T> constexpr int kstep() { return 4 * Mfma<T>::KL; }
// Row padding (elements) that keeps 16-row fragment reads bank-conflict free.
template <typename T> constexpr int pad() { return sizeof(T) == 4 ? 4 : 8; }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(_Float16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return (T)x; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Fragment of a matrix stored with the reduction index contiguous: element
// (i, kk) at p[i*ld + kk]; lane l gets i = i0 + l%16, kk = k0 + KL*(l/16) + [0,KL).
// Works for LDS and global pointers; needs 16-byte alignment for 16-bit types.
// Every lane-dependent helper takes the lane index as its last argument
// (default: the hardware lane id) so that a kernel can pass an opaque copy.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag_kc(const T* p, int ld, int i0, int k0,
                                                          int l = lane_id()) {
    const T* q = p + (long)(i0 + (l & 15)) * ld + k0 + (l >> 4) * Mfma<T>::KL;
    return *reinterpret_cast<const typename Mfma<T>::frag*>(q);
}

// MFMA fragment order of a [R][K] operand matrix with 16-bit elements (the
// 16x16x32 MFMAs): the 16 x 32 tile (row tile r / 16, k step k / 32) is one
// contiguous 1 KB block in which lane l's 8 elements (row 16 (r / 16) + l % 16,
// columns 32 (k / 32) + 8 (l / 16) ..+7) sit at 16 l bytes, so that a wave
// loads a whole A fragment as one contiguous 1 KB access (whole cache lines).
// fp32 operands (16x16x4 MFMAs) stay row-major. Element index of (r, k):
template <typename T, int K>
__device__ __forceinline__ size_t fo_index(int r, int k) {
    if constexpr (sizeof(T) == 2) {
        static_assert(K % 32 == 0, "k steps of 32");
        return ((size_t)(r >> 4) * (K / 32) + (k >> 5)) * 512 + ((r & 15) + 16 * ((k & 31) >> 3)) * 8 + (k & 7);
    } else {
        return (size_t)r * K + k;
    }
}
// Accumulator order of a [R][K] matrix: the 16 x 16 tile (r / 16, k / 16) is one
// contiguous block of 256 elements in which lane l's 4 elements (row
// 16 (r / 16) + l % 16, columns 16 (k / 16) + 4 (l / 16) ..+3) sit at 4 l: the
// order in which an MFMA accumulator tile of the transposed product holds
// them, so that such a tile is stored, and read back as quads, contiguously.
template <int K>
__device__ __forceinline__ size_t ao_index(int r, int k) {
    static_assert(K % 16 == 0, "k tiles of 16");
    return ((size_t)(r >> 4) * (K / 16) + (k >> 4)) * 256 + ((r & 15) + 16 * ((k & 15) >> 2)) * 4 + (k & 3);
}
// Row and first column of the e-th 16-byte piece of such a matrix (the inverse
// of fo_index at piece granularity: a lane slot of a tile for 16-bit elements).
template <typename T, int K>
__device__ __forceinline__ void fo_piece(int e, int& r, int& c) {
    if constexpr (sizeof(T) == 2) {
        const int b = e >> 6, ln = e & 63;
        r = 16 * (b / (K / 32)) + (ln & 15);
        c = 32 * (b % (K / 32)) + 8 * (ln >> 4);
    } else {
        constexpr int V = 16 / sizeof(T);
        r = e / (K / V);
        c = (e % (K / V)) * V;
    }
}
// Whether the sweep with V tiles of BV columns forms its k~^T and w^T
// fragments from k~ and w itself (staged in LDS, read through transposed
// loads): 16-bit operands at K = 128. The preparation stores k~^T and w^T
// only for a sweep that does not.
template <typename T, int C, int D, int BV>
constexpr bool sweep_transposes_a2() { return sizeof(T) == 2 && D == 128; }
// The A fragment (rows i0 .. +15, k0 .. +KS) of such a matrix.
template <typename T, int K>
__device__ __forceinline__ typename Mfma<T>::frag frag_fo(const T* p, int i0, int k0, int l = lane_id()) {
    if constexpr (sizeof(T) == 2) {
        return *reinterpret_cast<const typename Mfma<T>::frag*>(
            p + ((size_t)(i0 >> 4) * (K / 32) + (k0 >> 5)) * 512 + l * 8);
    } else {
        return frag_kc(p, K, i0, k0, l);
    }
}

// Four 16-bit elements (i0 + (l & 15), kk0 + gs (l >> 4) + q), q = 0..3, of
// a matrix stored with the reduction index as the row (element (i, kk) at
// p[kk*ld + i], p in LDS), in one gfx950 transpose load (ds_read_b64_tr_b16).
// Within each 16-lane group the load hands lane j element j % 4 of the 64-bit
// chunks that lanes 4q + j / 4 of the group address (q = 0..3; measured on
// the device), so lane l addresses row kk0 + gs (l >> 4) + (l & 15) / 4 at
// columns i0 + 4 (l % 4) .. + 3.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i16x4 ks_tr4(const void* p, int ld, int i0, int kk0, int gs, int l) {
    const short* q = static_cast<const short*>(p) + (kk0 + gs * (l >> 4) + ((l & 15) >> 2)) * ld + i0 + 4 * (l & 3);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(q));
}
// The same four elements as one 64-bit value, for callers that take them apart
// one by one: reading single elements of the builtin's vector result lets the
// compiler confuse them (it has used element 0 for all four).
__device__ __forceinline__ uint64_t ks_tr4_bits(const void* p, int ld, int i0, int kk0, int gs, int l) {
    return __builtin_bit_cast(uint64_t, ks_tr4(p, ld, i0, kk0, gs, l));
}

// Same fragment of a matrix stored with the reduction index as the row:
// element (i, kk) at p[kk*ld + i], p in LDS (16-bit: two transpose loads, for
// kk = k0 + 8 (l >> 4) + 0..3 and + 4..7).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag_ks(const T* p, int ld, int i0, int k0,
                                                          int l = lane_id()) {
    typename Mfma<T>::frag f;
    if constexpr (sizeof(T) == 2) {
        // the two loads' 64-bit values, not their elements (see ks_tr4_bits)
        const uint64_t v[2] = {ks_tr4_bits(p, ld, i0, k0, 8, l), ks_tr4_bits(p, ld, i0, k0 + 4, 8, l)};
        __builtin_memcpy(&f, v, sizeof(f));
    } else if constexpr (Mfma<T>::KL == 1) {
        f = p[(long)(k0 + (l >> 4)) * ld + i0 + (l & 15)];
    } else {
#pragma unroll
        for (int j = 0; j < Mfma<T>::KL; ++j)
            f[j] = p[(long)(k0 + (l >> 4) * Mfma<T>::KL + j) * ld + i0 + (l & 15)];
    }
    return f;
}

// Row-panel product: acc[t] += A[i0..i0+16, 0..KD) * Bt[j0+16t .. +16, 0..KD)^T
// with both operands stored reduction-contiguous (A[i*lda+kk], Bt[j*ldb+kk]).
// AKS: A stored with the reduction index as the row (A[kk*lda + i], in LDS);
// BKS: B likewise (B[kk*ldb + j], in LDS) instead of transposed (Bt[j*ldb + kk]).
template <typename T, int NT, int KD, bool AKS = false, bool BKS = false>
__device__ __forceinline__ void panel_mma(f32x4 (&acc)[NT], const T* A, int lda, int i0,
                                          const T* Bt, int ldb, int j0, int l = lane_id()) {
#pragma unroll
    for (int k0 = 0; k0 < KD; k0 += kstep<T>()) {
        const auto a = AKS ? frag_ks(A, lda, i0, k0, l) : frag_kc(A, lda, i0, k0, l);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = Mfma<T>::mma(a, BKS ? frag_ks(Bt, ldb, j0 + 16 * t, k0, l) : frag_kc(Bt, ldb, j0 + 16 * t, k0, l),
                                  acc[t]);
    }
}

// Row-panel product with the A operand already in registers (fragments of a
// C-long reduction): A rows (a[k] for reduction step k) against Bt in memory.
// BKS: B stored with the reduction index as the row (B[kk*ldb + j], in LDS)
// instead of transposed (Bt[j*ldb + kk]).
template <typename T, int NT, int NK, bool BKS = false>
__device__ __forceinline__ void panel_mma_ra(f32x4 (&acc)[NT], const typename Mfma<T>::frag (&a)[NK],
                                             const T* Bt, int ldb, int j0, int l) {
#pragma unroll
    for (int k = 0; k < NK; ++k)
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = Mfma<T>::mma(a[k], BKS ? frag_ks(Bt, ldb, j0 + 16 * t, k * kstep<T>(), l)
                                            : frag_kc(Bt, ldb, j0 + 16 * t, k * kstep<T>(), l), acc[t]);
}
// fp32 16x16 tile product on fp32 arrays, reduction length kd (multiple of 16):
// acc += A[(ai0+i)*lda + ak0 + kk] * B[(bk0+kk)*ldb + bj0 + j].
__device__ __forceinline__ f32x4 tile_f32(f32x4 acc, const float* A, int lda, int ai0, int ak0,
                                          const float* B, int ldb, int bk0, int bj0, int kd,
                                          int l = lane_id()) {
    // kd is a multiple of 16: the 8 LDS reads of four steps go out together
    for (int k0 = 0; k0 < kd; k0 += 16) {
        float a[4], b[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = k0 + 4 * j;
            a[j] = A[(ai0 + (l & 15)) * lda + ak0 + k + (l >> 4)];
            b[j] = B[(bk0 + k + (l >> 4)) * ldb + bj0 + (l & 15)];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
    }
    return acc;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// 16x16 products with a reduction of exactly 16 (one 16-row block):
// v_mfma_f32_16x16x16_{bf16,f16} (lane l holds A[l%16][4*(l/16) + 0..3],
// B[4*(l/16) + 0..3][l%16]), or four 16x16x4 fp32 steps for fp32 operands.
// ---------------------------------------------------------------------------
template <typename T> struct Mfma16;
template <> struct Mfma16<__bf16> {
    static constexpr int KL = 4, STEPS = 1;
    using frag = bf16x4;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma16<_Float16> {
    static constexpr int KL = 4, STEPS = 1;
    using frag = f16x4;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma16<float> {
    static constexpr int KL = 1, STEPS = 4;
    using frag = float;
    static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// Step `st` fragment of a 16-long reduction, operand stored reduction-contiguous
// (element (i, kk) at p[i*ld + kk]).
template <typename T>
__device__ __forceinline__ typename Mfma16<T>::frag frag16_kc(const T* p, int ld, int i0, int k0, int st, int l) {
    using M = Mfma16<T>;
    const T* q = p + (i0 + (l & 15)) * ld + k0 + 4 * st + (l >> 4) * M::KL;
    return *reinterpret_cast<const typename M::frag*>(q);
}
// Same, operand stored with the reduction index as the row (element (i, kk) at p[kk*ld + i]).
template <typename T>
__device__ __forceinline__ typename Mfma16<T>::frag frag16_ks(const T* p, int ld, int i0, int k0, int st, int l) {
    using M = Mfma16<T>;
    typename M::frag f;
    if constexpr (M::KL == 1) {
        f = p[(k0 + 4 * st + (l >> 4)) * ld + i0 + (l & 15)];
    } else {   // 16-bit, p in LDS: one transpose load
        const uint64_t a = ks_tr4_bits(p, ld, i0, k0, 4, l);
        __builtin_memcpy(&f, &a, sizeof(f));
    }
    return f;
}
// acc += A[i0.., k0..k0+16) * B[k0..k0+16, j0..), A reduction-contiguous (AT = false)
// or stored transposed (AT = true: A(i, kk) at A[kk*lda + i]); B given as Bt[j][kk].
template <typename T, bool AT>
__device__ __forceinline__ f32x4 mma16(f32x4 acc, const T* A, int lda, int i0, int ak0,
                                       const T* Bt, int ldb, int j0, int bk0, int l) {
#pragma unroll
    for (int st = 0; st < Mfma16<T>::STEPS; ++st) {
        const auto a = AT ? frag16_ks(A, lda, i0, ak0, st, l) : frag16_kc(A, lda, i0, ak0, st, l);
        acc = Mfma16<T>::mma(a, frag16_kc(Bt, ldb, j0, bk0, st, l), acc);
    }
    return acc;
}

// Cross-lane reductions without LDS: DPP moves within the 16-lane rows of the
// wave (quad_perm xor 1 / xor 2, half-row mirror, row mirror) and gfx950's
// permlane swaps across rows. Every lane of the group receives the result;
// all 64 lanes must be active.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
// sum over the 4 lanes of a quad, the 8 lanes of a half row, the 16 lanes of a row
__device__ __forceinline__ float quad_sum(float x) {
    x += dpp_mov<kDppXor1>(x);
    return x + dpp_mov<kDppXor2>(x);
}
__device__ __forceinline__ float row8_sum(float x) {
    x = quad_sum(x);                       // quads q0, q1 of the half row
    return x + dpp_mov<kDppHalfMirror>(x); // lane i <- lane 7 - i: the other quad
}
__device__ __forceinline__ float row16_sum(float x) {
    x = row8_sum(x);
    return x + dpp_mov<kDppMirror>(x);     // lane i <- lane 15 - i: the other half
}
// v_permlane16_swap on two copies of a leaves (rows 0,0,2,2 of a) in the first
// register and (rows 1,1,3,3) in the second; v_permlane32_swap leaves (rows
// 0,1,0,1) and (rows 2,3,2,3) (checked on the device): the two halves of each
// lane's exchange with row r ^ 1 (r ^ 2). Written as asm with both registers
// read-write: this toolchain's builtins lose track of the second result. The
// s_nop gives the two wait states the compiler itself puts before the
// instruction after a VALU write of its operands.
__device__ __forceinline__ void swap16(float x, float& lo, float& hi) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    lo = __builtin_bit_cast(float, a);
    hi = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ void swap32(float x, float& lo, float& hi) {
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    lo = __builtin_bit_cast(float, a);
    hi = __builtin_bit_cast(float, b);
}
// The value of row r ^ 1 (xor16) / r ^ 2 (xor32) at the same lane of the row.
__device__ __forceinline__ float xor16(float x, int l) {
    float lo, hi;
    swap16(x, lo, hi);
    return (l & 16) ? lo : hi;
}
__device__ __forceinline__ float xor32(float x, int l) {
    float lo, hi;
    swap32(x, lo, hi);
    return (l & 32) ? lo : hi;
}
// sum over the 4 rows at the same lane of the row
__device__ __forceinline__ float cross_row_sum(float x) {
    float lo, hi;
    swap16(x, lo, hi);
    x = lo + hi;
    swap32(x, lo, hi);
    return lo + hi;
}

// Maximum over the wave, returned as a wave-uniform (scalar) value.
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp_mov<kDppXor1>(x));
    x = fmaxf(x, dpp_mov<kDppXor2>(x));
    x = fmaxf(x, dpp_mov<kDppHalfMirror>(x));
    x = fmaxf(x, dpp_mov<kDppMirror>(x));
    float lo, hi;
    swap16(x, lo, hi);
    x = fmaxf(lo, hi);
    swap32(x, lo, hi);
    x = fmaxf(lo, hi);
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// Row / column of element i (0..3) of an f32x4 accumulator tile held by this lane.
__device__ __forceinline__ int acc_row(int i, int l = lane_id()) { return 4 * (l >> 4) + i; }
__device__ __forceinline__ int acc_col(int l = lane_id()) { return l & 15; }

// The lane id from the count of lower lanes in the full mask (v_mbcnt), which
// needs no register kept from the kernel's start. The mask goes through an
// empty asm: with a visible all-ones mask the compiler folds the count back
// into the thread id register.
__device__ __forceinline__ int mbcnt_lane() {
    unsigned m = ~0u;
    asm volatile("" : "+s"(m));
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(m, __builtin_amdgcn_mbcnt_lo(m, 0u)));
}

// The hardware lane id behind an empty asm: each call yields a value the
// compiler cannot prove equal to any other, so lane-dependent arithmetic
// derived from it is neither hoisted out of loops nor merged across copies.
__device__ __forceinline__ int opaque_lane_id() {
    int l = mbcnt_lane();
    asm volatile("" : "+v"(l));
    return l;
}
// The thread index as wave * 64 + lane, behind an empty asm like the lane id
// above; wv is the wave index held in a scalar register. Neither part reads
// the thread id register, so a persistent kernel need not keep that register
// (or a spilled copy of it) alive across its items.
__device__ __forceinline__ int fresh_tid(int wv) {
    int t = wv * 64 + mbcnt_lane();
    asm volatile("" : "+v"(t));
    return t;
}

// Store 4 consecutive values (accumulator rows r..r+3 of one column) to
// p[0..3] (contiguous), converting to T.
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
    } else {
        typename Mfma<T>::quad v;
        v[0] = (T)a; v[1] = (T)b; v[2] = (T)c; v[3] = (T)d;
        *reinterpret_cast<typename Mfma<T>::quad*>(p) = v;
    }
}

// 16-byte vector load / store helpers (8 x 16-bit or 4 x fp32).
struct alignas(16) Vec16 { uint32_t w[4]; };
__device__ __forceinline__ Vec16 ld16(const void* p) { return *reinterpret_cast<const Vec16*>(p); }
__device__ __forceinline__ void st16(void* p, Vec16 v) { *reinterpret_cast<Vec16*>(p) = v; }

// ---------------------------------------------------------------------------
// Kernel parameters (one struct passed by value to every kernel).
// ---------------------------------------------------------------------------
// Column tile of the stored per-chunk states and X / T (the state sweep's
// V tile and the gradient kernel's V slice).
constexpr int kTileV = 32;

struct ChunkEntry {
    int tok0;   // flattened token index (b*T + t) of the chunk's first token
    int len;    // real tokens in the chunk (1..C)
    int seq;    // sequence index n
    int pad_;
};

struct Params {
    // problem
    int64_t B, T;
    int H, Hg, G;        // G = H / Hg
    int N;               // sequences
    int nc_max;          // chunk-table capacity (grid size of chunk-parallel kernels)
    int varlen;
    int dirs;            // state sweeps run: 1 = one direction, 2 = both
    int dir0;            // first direction: 0 = forward (forward pass, or both for the
                         // backward); 1 = reverse only (a backward after the forward
                         // pass, whose table, factors, h and X are in the workspace,
                         // or a backward from caller-supplied per-chunk states)
    int vfirst;          // h0, dht, dh0, ht (and hsrc) stored [V][K] instead of [K][V]
    float scale;
    // per-chunk states supplied by the caller (backward from states), or NULL:
    // [nh_src][H][K][V] ([..][V][K] with vfirst) in the io type
    const void* hsrc;
    int nh_src;          // chunk states the caller's buffer holds
    // fused reverse backward with GQA: fp32 dq, dk per value head [B*T][H][K]
    float* dqp; float* dkp;
    // inputs
    const void* q; const void* k; const void* v; const float* g; const void* beta;
    const float* h0; const void* dout; const float* dht; const int* cu;
    // outputs
    void* dq; void* dk; void* dv; float* dg; void* db; float* dh0;
    void* o; float* ht;  // forward pass: outputs and final states (ht may be NULL)
    // workspace
    ChunkEntry* ctab;    // [nc_max]
    int* seq_off;        // [N+1] first chunk of each sequence; seq_off[N] = chunk count
    int* seq_ord;        // [N] varlen: sequences by chunk count, longest first (ties in any order)
    void* sAqkT;         // [nc][H][C][C]  scale * Aqk^T
    void* Am;            // [nc][H][C][C]  A = (I + Akk)^-1
    // scale Aqk^T, A, w, w^T, k~, k~^T and scale q~^T in MFMA fragment order (fo_index)
    void* w;             // [nc][H][C][D]  w = A (beta k 2^G)
    void* wT;            // [nc][H][D][C]
    void* kt;            // [nc][H][C][D]  k 2^(G_last - G)
    void* ktT;           // [nc][H][D][C]
    void* uT;            // [nc][H][D][C]  u = A (beta v), transposed, in accumulator order (ao_index)
    void* qsT;           // [nc][H][D][C]  scale * (q 2^G - Aqk w), transposed
    float* glast;        // [nc][H][D]     2^G_last
    // V-tiled ([..][D / kTileV][rows][kTileV]): one contiguous block per
    // (chunk, head, tile of kTileV state columns)
    void* hbuf;          // [nc][H][D/kTileV][D][kTileV]  state before the chunk
    void* xbuf;          // [nc][H][D/kTileV][C][kTileV]  X = u - w h
    void* dhbuf;         // [nc][H][D/kTileV][D][kTileV]  dL/dS at the chunk end
    void* tbuf;          // [nc][H][D/kTileV][C][kTileV]  k~ dh
};

// Offset of state element (key row d, value column c) within one K x V state:
// row-major [K][V], or [V][K] when the caller stores states value-first.
template <int D>
__device__ __forceinline__ size_t state_index(const Params& p, int d, int c) {
    return p.vfirst ? (size_t)c * D + d : (size_t)d * D + c;
}

// First token (flattened b*T + t) and length of sequence n. Varlen offsets
// are clamped to [0, T], each end to at least its start, so that no
// cu_seqlens content can address a token outside the buffers; the chunk table
// and the sweeps both take a sequence's span from here.
__device__ __forceinline__ void seq_span(const Params& p, int n, int& tok0, int& len) {
    if (p.varlen) {
        const int T = (int)p.T;
        const int a = min(max(p.cu[n], 0), T);
        const int b = min(max(p.cu[n + 1], a), T);
        tok0 = a;
        len = b - a;
    } else {
        tok0 = (int)(n * p.T);
        len = (int)p.T;
    }
}

}  // namespace gdr
