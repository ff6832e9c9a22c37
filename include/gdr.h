/*
 * gdr.h -- C ABI of the MI355X (gfx950) chunkwise backward pass of gated
 * delta-rule linear attention.
 *
 * The operation. Per sequence n and value head h, tokens t = 1..T_n, the
 * forward recurrence (the one the "kernel_fun kda bwd_intra" page and the
 * FlashQLA issue #30 page both take apart chunk by chunk) is
 *     S_t = (I - beta_t k_t k_t^T) Diag(2^{g_t}) S_{t-1} + beta_t k_t v_t^T,
 *     o_t = scale * S_t^T q_t,          S_0 = h0,
 * with the gate g_t either per channel (g_t in R^K, the KDA form of the
 * bwd_intra page) or one scalar per token and head (the GDN form of the
 * FlashQLA page's fused_bwd.py). Given do = dL/do and dht = dL/dS_T, gdr_bwd
 * returns dq, dk, dv, dg, db (= dL/dbeta) and dh0 = dL/dS_0. g is the raw
 * per-token log2 gate (the kernels form its chunk-local cumulative sum
 * themselves, as the bwd_intra page's inputs assume), and dg is the gradient
 * with respect to that raw g. Value head h reads q/k head h / (H / Hg) (GQA,
 * as in fused_bwd.py's head map); dq and dk are summed over each group.
 *
 * Conventions shared by every call:
 *  - All pointers other than the descriptor are DEVICE pointers (HBM),
 *    contiguous row-major, owned by the caller. The library allocates nothing,
 *    frees nothing, keeps no pointer after returning, and only enqueues work
 *    on `stream` (a hipStream_t passed as void*; NULL = the null stream).
 *    Calls return without synchronising the host.
 *  - Return value: GDR_OK (0) or a negative gdr_status_t. Nothing is printed
 *    and no C++ exception crosses the ABI. gdr_strerror() describes a code;
 *    for GDR_EHIP it also holds the HIP error text of the failing call
 *    (thread-local, until the next failing call on the same host thread).
 *  - Preconditions that are documented but not checked: g <= 0 elementwise
 *    (the gate decays; the off-diagonal exp2 arguments the kernels form are
 *    then <= 0, the diagonal-block MFMA form uses arguments up to its guard,
 *    see gdr_chunk_bwd.hpp), finite inputs, non-overlapping output buffers,
 *    and on the device cu_seqlens[0] >= 0, cu_seqlens non-decreasing,
 *    cu_seqlens[n_seqs] <= T. cu_seqlens values are clamped to [0, T] (each
 *    end to at least its start) before any use, so a violation gives
 *    meaningless results for the sequences concerned but never an access
 *    outside the given buffers.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDR_OK = 0,
    GDR_EINVAL = -1,        /* bad shape, null required pointer, misaligned buffer */
    GDR_EUNSUPPORTED = -2,  /* valid but not built: K, V not in {64,128}, K != V, fp32 with K != 64, chunk not in {32,64} */
    GDR_EWORKSPACE = -3,    /* workspace NULL or smaller than gdr_bwd_workspace_bytes() */
    GDR_EHIP = -4,          /* a HIP launch or query failed */
    GDR_ESCRATCH = -5       /* gdr_bwd_static: the problem needs more workspace than
                               GDR_STATIC_SCRATCH_BYTES */
} gdr_status_t;

typedef enum {
    GDR_GATE_PER_CHANNEL = 0, /* KDA: g [B,T,H,K] fp32 */
    GDR_GATE_SCALAR = 1       /* GDN: g [B,T,H]   fp32 */
} gdr_gate_t;

typedef enum {
    GDR_DTYPE_F32 = 0,
    GDR_DTYPE_BF16 = 1,
    GDR_DTYPE_F16 = 2
} gdr_dtype_t;

/*
 * Problem descriptor (host memory; read during the call only).
 *   B, T      batch and tokens per sequence; varlen: B == 1 and T = packed total
 *   H, Hg     value heads and q/k heads, H % Hg == 0
 *   K, V      key and value head dims; supported: K == V in {64, 128} (64 only for fp32 io)
 *   chunk     chunk length C in {32, 64} (the chunk of the chunkwise form)
 *   sub_chunk diagonal sub-block of the intra-chunk gradient; must be 16
 *   n_seqs    0 = fixed length (B sequences of T tokens);
 *             > 0 = varlen: cu_seqlens holds n_seqs + 1 offsets, B must be 1
 *   gate      gdr_gate_t
 *   io_dtype  gdr_dtype_t of q, k, v, beta, do and of dq, dk, dv, db
 *   scale     readout scale; <= 0 means K^-0.5
 *   state_v_first  0: every state buffer (h0, dht, dh0, ht, and the per-chunk
 *             states of gdr_bwd_from_states) is [..][K][V], row k holding the
 *             value columns; 1: [..][V][K] (the transposed layout the FlashQLA
 *             page's state_v_first option selects). Shapes are unchanged
 *             (K == V); only the order of the two state axes differs.
 */
typedef struct {
    int64_t B, T;
    int32_t H, Hg, K, V;
    int32_t chunk, sub_chunk;
    int32_t n_seqs;
    int32_t gate;
    int32_t io_dtype;
    float scale;
    int32_t state_v_first;
} gdr_bwd_desc_t;

/*
 * Checks a descriptor without touching the GPU.
 * Returns GDR_OK, GDR_EINVAL or GDR_EUNSUPPORTED.
 */
int gdr_bwd_check(const gdr_bwd_desc_t* d);

/*
 * Bytes of device workspace gdr_bwd needs for descriptor d (0 if d is invalid).
 * The workspace holds the per-chunk intermediates of the chunkwise form (the
 * WY factors, the per-chunk states h_c and state gradients dh_c) and, for
 * varlen, the chunk table built on the device. Touches no GPU state.
 */
size_t gdr_bwd_workspace_bytes(const gdr_bwd_desc_t* d);

/*
 * The backward pass: the argument list of the FlashQLA issue #30 page's
 * fused_gdr_bwd wrapper (q, k, v, g, b, do, dht, scale, cu_seqlens,
 * chunk_size) minus the forward-saved states it also takes (see
 * gdr_bwd_from_states for that form), plus h0, which this call needs to
 * recompute them; the outputs of the kernel_fun page's host wrapper
 * chunk_kda_bwd_intra_cutedsl (dq, dk, db, dg, with the fold of dg into the
 * raw-gate gradient) completed by dv and dh0. Inputs (device, read only):
 *   q, k        [B,T,Hg,K] io_dtype
 *   v, do_      [B,T,H,V]  io_dtype
 *   g           [B,T,H,K] (per channel) or [B,T,H] (scalar) fp32, raw log2 gate
 *   beta        [B,T,H]    io_dtype
 *   h0          [N,H,K,V]  fp32 initial states, N = n_seqs or B; NULL = zero
 *               ([N,H,V,K] when d->state_v_first, as for dht and dh0)
 *   dht         [N,H,K,V]  fp32 gradient of the final states; NULL = zero
 *   cu_seqlens  int32 [n_seqs+1] (varlen) or NULL (fixed length)
 * Outputs (device, fully overwritten, never accumulated into):
 *   dq, dk      [B,T,Hg,K] io_dtype (fp32 group sum, then one rounding)
 *   dv          [B,T,H,V]  io_dtype
 *   dg          same shape as g, fp32 (w.r.t. the raw per-token gate)
 *   db          [B,T,H]    io_dtype
 *   dh0         [N,H,K,V]  fp32, always written (zero-state gradient included)
 * workspace:    device buffer of at least gdr_bwd_workspace_bytes(d) bytes,
 *               256-byte aligned; contents on entry are ignored.
 * Every buffer must be 16-byte aligned. Varlen tokens outside
 * [cu_seqlens[0], cu_seqlens[n_seqs]) are not written. With T == 0 (no tokens;
 * varlen: every sequence empty) the token buffers may be NULL; dh0 is still
 * written (= dht, or zero).
 */
int gdr_bwd(const gdr_bwd_desc_t* d,
            const void* q, const void* k, const void* v, const float* g,
            const void* beta, const float* h0, const void* do_, const float* dht,
            const int32_t* cu_seqlens,
            void* dq, void* dk, void* dv, float* dg, void* db, float* dh0,
            void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdr_bwd plus a measurement hook: stage_events is NULL or an array of
 * GDR_STAGE_EVENTS hipEvent_t (created by the caller, passed as void*) that
 * are recorded on `stream` before the first kernel and after each of the four
 * kernels (chunk table, per-chunk preparation, state sweeps, chunk gradients),
 * so that a caller can time every kernel on the stream it runs on. The events
 * add no synchronisation. Same arguments, ownership and errors as gdr_bwd.
 */
#define GDR_STAGE_EVENTS 5
int gdr_bwd_with_events(const gdr_bwd_desc_t* d,
                        const void* q, const void* k, const void* v, const float* g,
                        const void* beta, const float* h0, const void* do_, const float* dht,
                        const int32_t* cu_seqlens,
                        void* dq, void* dk, void* dv, float* dg, void* db, float* dh0,
                        void* workspace, size_t workspace_bytes, void* stream,
                        void* const* stage_events);

/*
 * The forward pass of the same recurrence: o_t = scale S_t^T q_t for every
 * token and the final state S_T of every sequence, in the chunk form
 *   o_c = scale [(q 2^G) h_c + Aqk X_c],   X_c = u_c - w_c h_c,
 * h_{c+1} = Diag(2^G_last) h_c + (k 2^(G_last - G))^T X_c
 * (the WY recompute on the FlashQLA page's fused_bwd.py; the kda chain of the
 * kernel-fun page opens with its forward stage). Inputs q, k, v, g, beta, h0,
 * cu_seqlens: as for gdr_bwd. Outputs (device, fully overwritten):
 *   o           [B,T,H,V]  io_dtype
 *   ht          [N,H,K,V]  fp32 final states; NULL = not written
 * With T == 0 the token buffers (q, k, v, g, beta, o) may be NULL.
 * workspace:    as for gdr_bwd (gdr_bwd_workspace_bytes(d) bytes); the pass
 *               leaves the per-chunk states h_c in it (region 12).
 * Same descriptor, alignment, ownership and error codes as gdr_bwd.
 */
int gdr_fwd(const gdr_bwd_desc_t* d,
            const void* q, const void* k, const void* v, const float* g,
            const void* beta, const float* h0, const int32_t* cu_seqlens,
            void* o, float* ht,
            void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward pass after gdr_fwd, from the per-chunk states the forward pass
 * saved (the FlashQLA page's backward takes the forward's per-chunk states and
 * its A factor as inputs instead of recomputing them). `workspace` must be the
 * buffer of a gdr_fwd call with the same descriptor and the same q, k, v, g,
 * beta, h0 and cu_seqlens, unchanged since: it holds that call's chunk table,
 * WY factors and per-chunk h and X, so this call runs only the chunk table,
 * the reverse state sweep and the gradient kernel (no preparation or forward
 * sweep; h0 is not needed again). The results equal gdr_bwd's on the same
 * inputs. Arguments, outputs, alignment and error codes: as for gdr_bwd
 * (without h0). A workspace that does not hold such a forward state is not
 * detected: the outputs are then meaningless, but every access stays within
 * the given buffers (the chunk table is rebuilt from cu_seqlens and the shapes).
 */
int gdr_bwd_after_fwd(const gdr_bwd_desc_t* d,
                      const void* q, const void* k, const void* v, const float* g,
                      const void* beta, const void* do_, const float* dht,
                      const int32_t* cu_seqlens,
                      void* dq, void* dk, void* dv, float* dg, void* db, float* dh0,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward from per-chunk states the caller already holds: the interface
 * of the FlashQLA issue #30 page's backward (fused_bwd.py's kernel signature
 * and its fused_gdr_bwd wrapper take the forward's per-chunk states h as an
 * input, with state_v_first choosing their layout). h_c is the state before
 * chunk c (h_0 = h0 of each sequence):
 *   h           io_dtype [n_h_chunks][H][K][V], or [n_h_chunks][H][V][K] when
 *               d->state_v_first is 1; chunk c of sequence n is entry
 *               sum_{m<n} ceil(len_m / chunk) + c (fixed length: n ceil(T /
 *               chunk) + c, i.e. the [B][ceil(T/chunk)] order of a 5-d
 *               [B, chunks, H, K, V] tensor).
 *   n_h_chunks  entries in h: must be B ceil(T / chunk) for fixed length
 *               (GDR_EINVAL otherwise); for varlen, the sum above (not
 *               checkable without reading cu_seqlens: chunks at or past
 *               n_h_chunks are never read, their gradients are then meaningless).
 * The forward state sweep is not run: a chunk-parallel kernel forms X_c =
 * u_c - w_c h_c from the given states, then the reverse sweep and the gradient
 * kernel run as in gdr_bwd. h0 is not needed. Everything else (arguments,
 * outputs, workspace size, alignment, error codes) as for gdr_bwd; dht and dh0
 * follow d->state_v_first too.
 */
int gdr_bwd_from_states(const gdr_bwd_desc_t* d,
                        const void* q, const void* k, const void* v, const float* g,
                        const void* beta, const void* do_, const float* dht,
                        const int32_t* cu_seqlens, const void* h, int64_t n_h_chunks,
                        void* dq, void* dk, void* dv, float* dg, void* db, float* dh0,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The backward as one fused reverse kernel per (sequence, value head) with the
 * state gradient resident on chip (the FlashQLA issue #30 page's single fused
 * backward kernel, whose state-gradient role keeps dh in registers for the
 * whole loop over chunks): the chunk table, the preparation and the forward
 * state sweep run as in gdr_bwd, then each workgroup walks its sequence's
 * chunks from the last to the first, computing that chunk's gradients and the
 * reverse sweep's update of dh without writing dh (or T = k~ dh) to memory.
 * With GQA, dq and dk of the value heads of a group are added in fp32 by a
 * second small kernel, in group order. Built for chunk == 32 only (its LDS
 * plan): other chunks return GDR_EUNSUPPORTED. Same arguments, outputs and
 * error codes as gdr_bwd; the workspace must hold
 * gdr_bwd_fused_workspace_bytes(d) bytes (gdr_bwd's regions plus, with GQA,
 * the fp32 partials of dq and dk). The results match gdr_bwd's within the
 * rounding of the io type (the reductions are ordered differently).
 */
size_t gdr_bwd_fused_workspace_bytes(const gdr_bwd_desc_t* d);
int gdr_bwd_fused(const gdr_bwd_desc_t* d,
                  const void* q, const void* k, const void* v, const float* g,
                  const void* beta, const float* h0, const void* do_, const float* dht,
                  const int32_t* cu_seqlens,
                  void* dq, void* dk, void* dv, float* dg, void* db, float* dh0,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Byte offsets of the workspace regions for descriptor d, in this order:
 *   0 chunk table, 1 per-sequence chunk offsets (n + 1 int32, then, for
 *   varlen, the n sequences by chunk count, longest first), 2 scale*Aqk^T, 3 A,
 *   4 (empty: A^T is taken from A; kept so that the numbering holds),
 *   5 w, 6 w^T, 7 k~, 8 k~^T (6 and 8 are written only where the state
 *   sweep does not form them from w and k~ itself: fp32 io or K = 64),
 *   9 u^T, 10 scale*q~^T, 11 2^G_last,
 *   12 h (state before each chunk), 13 X, 14 dh (state gradient at each
 *   chunk end), 15 T = k~ dh, 16 = total bytes.
 * Per-chunk regions are [chunks][H][..] in io_dtype (2^G_last in fp32);
 * h, X, dh and T are stored in tiles of 32 state columns, [D/32][rows][32];
 * with 16-bit io, scale*Aqk^T, A, w, w^T, k~, k~^T and scale*q~^T are
 * stored in MFMA fragment order (each 16 x 32 tile one contiguous 1 KB block)
 * and u^T in accumulator order (each 16 x 16 tile one contiguous block).
 * For inspecting intermediates in tests; n must be >= 17.
 * Returns GDR_OK, GDR_EINVAL or GDR_EUNSUPPORTED. Touches no GPU state.
 */
int gdr_bwd_workspace_offsets(const gdr_bwd_desc_t* d, size_t* offsets, int n);

/*
 * gdr_bwd without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. The same backward as gdr_bwd (same arguments,
 * outputs, alignment and error codes, minus the workspace), with the
 * workspace taken from a fixed device array inside this library:
 * GDR_STATIC_SCRATCH_BYTES on each GPU the call runs on, held from the first
 * such call on that GPU until the process ends. The call allocates and frees
 * nothing. A descriptor whose gdr_bwd_workspace_bytes() exceeds
 * GDR_STATIC_SCRATCH_BYTES is rejected with GDR_ESCRATCH before anything is
 * enqueued. Every call on one GPU shares that GPU's array, which keeps the
 * last call's contents (no call reads them: every region is written before it
 * is read). Calls that can overlap on one GPU (on different streams, or from
 * host threads without an order between them) race on the array and give
 * meaningless results; calls on one stream are ordered and safe. The current
 * device must be the device of the buffers and of the stream.
 */
#define GDR_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int gdr_bwd_static(const gdr_bwd_desc_t* d,
                   const void* q, const void* k, const void* v, const float* g,
                   const void* beta, const float* h0, const void* do_, const float* dht,
                   const int32_t* cu_seqlens,
                   void* dq, void* dk, void* dv, float* dg, void* db, float* dh0,
                   void* stream);

/* Static description of a status code (plus the HIP message for GDR_EHIP). */
const char* gdr_strerror(int status);

/* Library version as "major.minor.patch". */
const char* gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
